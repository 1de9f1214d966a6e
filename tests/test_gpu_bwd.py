"""GPU parity of the backward against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, np64, ratio, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")
KINDS = ("tok", "tok", "tok", "tok", "tok", "state")


def gpu_fwd_bwd(d, svf=False, cp=0, vt=0):
    import gated_delta_rule_66_amd as gdr
    dd = to_dev(d)
    h0, dht = dd["h0"], dd["dht"]
    if svf:
        h0 = None if h0 is None else h0.transpose(-1, -2).contiguous()
        dht = None if dht is None else dht.transpose(-1, -2).contiguous()
    cu_cpu = d["cu_seqlens"]
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"], initial_state=h0,
        output_final_state=True, cu_seqlens=dd["cu_seqlens"], state_v_first=svf, cp_segments=cp,
        cu_seqlens_cpu=cu_cpu, wave_tiles=vt)
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dht, scale=dd["scale"],
        initial_state=h0, cu_seqlens=dd["cu_seqlens"], state_v_first=svf, dg_dtype=dd["g"].dtype,
        cp_segments=cp, cu_seqlens_cpu=cu_cpu, wave_tiles=vt)
    torch.cuda.synchronize()
    return o, ht, grads


def oracle_grads(d):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    return oracle.bwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]),
                      d["scale"], np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                      cu_seqlens=cu)


def P(name, **kw):
    kw.setdefault("backward", True)
    return gdr_synth.Problem(name, **kw)


CASES = {
    "dense_state_dht": P("dense", B=2, T=200, Hq=2, Hv=2, init_state=True, dht=True),
    "no_state": P("nostate", B=1, T=130, Hq=2, Hv=2),
    "fp16_gva": P("fp16_gva", B=1, T=333, Hq=1, Hv=2, dtype="fp16", init_state=True, dht=True),
    # groups of three and four value heads per q/k head (odd group size; two
    # q/k heads of four value heads each)
    "gva_group3": P("gva3", B=2, T=150, Hq=1, Hv=3, init_state=True, dht=True),
    "gva_group4": P("gva4", B=1, T=200, Hq=2, Hv=8, init_state=True, dht=True),
    "varlen": P("varlen", B=1, T=0, Hq=2, Hv=2, init_state=True, dht=True,
                lens=[70, 1, 64, 129, 250]),
    "varlen_empty_seq": P("varlen_empty", B=1, T=0, Hq=1, Hv=1, init_state=True, dht=True,
                          lens=[70, 0, 65]),
    "one_token": P("one", B=1, T=1, Hq=1, Hv=1, init_state=True, dht=True),
    "long_slow_decay": P("long", B=1, T=1500, Hq=2, Hv=2, init_state=True, dht=True, g_shift=2.0),
    # dense, few heads, 16+ chunks: the states-path backward runs in one
    # launch scheduled by data (the gradient workgroups of a chunk start once
    # the scan has stored its state gradient; with q / k normalised, in
    # slices); ragged last chunk
    "pipe": P("pipe", B=2, T=1100, Hq=2, Hv=2, init_state=True, dht=True),
    "pipe_no_state": P("pipe0", B=1, T=1030, Hq=3, Hv=3),
    # the same launch with grouped heads (groups of three value heads): it
    # runs heads 0 .. G-2 of every group, the gradient kernel the last
    "pipe_gva": P("pipe_gva", B=2, T=1030, Hq=2, Hv=6, init_state=True, dht=True),
    # packed sequences, the longest with 16+ chunks, an empty and a one-token
    # one: the gradient workgroups in the item table's order
    "pipe_varlen": P("pipe_varlen", B=1, T=0, Hq=2, Hv=2, init_state=True, dht=True,
                     lens=[1100, 0, 70, 2000, 1, 640]),
    # (sequence, head) units a multiple of 8: rank-ordered scan blocks
    "varlen_ranked": P("varlen_ranked", B=1, T=0, Hq=2, Hv=2, init_state=True, dht=True,
                       lens=[300, 1000, 64, 700]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    d = gdr_synth.make(CASES[name])
    print("case", name, CASES[name], flush=True)
    o, ht, g = gpu_fwd_bwd(d, cp=1)
    ref = oracle_grads(d)
    for nm, kind, x, r in zip(NAMES, KINDS, g, ref):
        check(nm, x, r, kind, d["cu_seqlens"])


CP_CASES = [("long_slow_decay", 2), ("long_slow_decay", 4), ("long_slow_decay", 7),
            ("varlen", 2), ("varlen", 3), ("fp16_gva", 4)]


@pytest.mark.parametrize("name,cp", CP_CASES)
def test_context_parallel_backward_matches_oracle(name, cp):
    d = gdr_synth.make(CASES[name])
    print("case", name, "cp", cp, flush=True)
    o, ht, g = gpu_fwd_bwd(d, cp=cp)
    ref = oracle_grads(d)
    for nm, kind, x, r in zip(NAMES, KINDS, g, ref):
        check(nm, x, r, kind, d["cu_seqlens"])


@pytest.mark.parametrize("cp", [1, 3])
def test_backward_state_v_first_is_bit_exact(cp):
    d = gdr_synth.make(CASES["varlen"])
    _, _, a = gpu_fwd_bwd(d, svf=False, cp=cp)
    _, _, b = gpu_fwd_bwd(d, svf=True, cp=cp)
    for x, y in zip(a[:5], b[:5]):
        assert torch.equal(x, y)
    assert torch.equal(a[5].transpose(-1, -2), b[5])


def test_backward_is_deterministic():
    d = gdr_synth.make(CASES["fp16_gva"])
    _, _, a = gpu_fwd_bwd(d)
    _, _, b = gpu_fwd_bwd(d)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_end_to_end():
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(CASES["dense_state_dht"])
    dd = to_dev(d)
    leaves = {k: dd[k].clone().requires_grad_(True) for k in ("q", "k", "v", "g", "beta", "h0")}
    o, ht = gdr.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"],
                                       leaves["beta"], scale=dd["scale"],
                                       initial_state=leaves["h0"], output_final_state=True)
    loss = (o.float() * dd["do"].float()).sum() + (ht * dd["dht"]).sum()
    loss.backward()
    ref = oracle_grads(d)
    for nm, kind, key in zip(NAMES, KINDS, ("q", "k", "v", "beta", "g", "h0")):
        check(nm, leaves[key].grad, ref[NAMES.index(nm)], kind)


@pytest.mark.parametrize("name", ["dense_state_dht", "fp16_gva", "varlen_empty_seq",
                                  "varlen_ranked"])
@pytest.mark.parametrize("vt,cp", [(1, 1), (2, 1), (1, 3), (2, 3)])
def test_backward_scan_variants(name, vt, cp):
    """One and two 16-column tiles per wave, unsplit and in three segments."""
    d = gdr_synth.make(CASES[name])
    print("case", name, "wave_tiles", vt, "cp", cp, flush=True)
    o, ht, g = gpu_fwd_bwd(d, cp=cp, vt=vt)
    ref = oracle_grads(d)
    for n, kind, x, r in zip(NAMES, KINDS, g, ref):
        check(n, x, r, kind, d["cu_seqlens"])


def gpu_fwd_bwd_states(d, cp=0, use_trans=True, vt=0):
    """The autograd path: the forward keeps its chunk-start states (packed)
    and, for a split plan, its segment transitions; the backward takes them
    instead of recomputing (use_trans=False: it forms its own transitions)."""
    import gated_delta_rule_66_amd as gdr
    dd = to_dev(d)
    cu_cpu = d["cu_seqlens"]
    g_cum, A, o, h, trans, ht = gdr.chunk_gated_delta_rule_fwd_states(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], output_final_state=True, cu_seqlens=dd["cu_seqlens"],
        cp_segments=cp, cu_seqlens_cpu=cu_cpu, wave_tiles=vt)
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
        scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
        dg_dtype=dd["g"].dtype, cp_segments=cp, cu_seqlens_cpu=cu_cpu, h=h,
        trans=trans if use_trans else None, wave_tiles=vt)
    torch.cuda.synchronize()
    return h, grads


@pytest.mark.parametrize("name,cp,use_trans,vt", [
    ("dense_state_dht", 1, True, 0), ("varlen", 1, True, 0), ("fp16_gva", 1, True, 0),
    ("varlen_empty_seq", 1, True, 0), ("gva_group3", 1, True, 0),
    ("long_slow_decay", 4, True, 1), ("long_slow_decay", 4, True, 2),
    ("long_slow_decay", 4, False, 1), ("varlen", 3, True, 0), ("varlen", 3, False, 0),
    ("dense_state_dht", 2, True, 2), ("fp16_gva", 3, True, 1), ("gva_group4", 2, True, 0),
    ("varlen_empty_seq", 2, True, 0), ("pipe", 1, True, 1), ("pipe_no_state", 1, True, 1),
    ("pipe_gva", 1, True, 1), ("pipe_varlen", 1, True, 1),
    ("varlen_ranked", 1, True, 0), ("varlen_ranked", 3, True, 1),
    ("fp16_gva", 1, True, 2), ("varlen_ranked", 1, True, 2), ("varlen", 3, True, 2)])
def test_backward_from_the_forward_states(name, cp, use_trans, vt):
    d = gdr_synth.make(CASES[name])
    print("case", name, "cp", cp, "trans", use_trans, "wave_tiles", vt, flush=True)
    h, g = gpu_fwd_bwd_states(d, cp=cp, use_trans=use_trans, vt=vt)
    ref = oracle_grads(d)
    for nm, kind, x, r in zip(NAMES, KINDS, g, ref):
        check(nm, x, r, kind, d["cu_seqlens"])
    # the same scans produce the same states: with one plan for both passes
    # the gradients are those of the recomputing backward, bit for bit
    if cp == 1:
        _, _, g2 = gpu_fwd_bwd(d, cp=1)
        for nm, x, y in zip(NAMES, g, g2):
            assert (x is None and y is None) or torch.equal(x, y), nm


def test_packed_h_holds_the_default_states():
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(CASES["varlen"])
    dd = to_dev(d)
    kw = dict(scale=dd["scale"], initial_state=dd["h0"], output_final_state=True,
              cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=d["cu_seqlens"], output_h=True)
    a = gdr.chunk_gated_delta_rule_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **kw)
    b = gdr.chunk_gated_delta_rule_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"],
                                       h_packed=True, **kw)
    torch.cuda.synchronize()
    # the same states, rounded the same way, in another order
    assert torch.equal(gdr.unpack_states(b[3]), a[3])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    check("o", b[2], np64(a[2]), "tok", d["cu_seqlens"])
    assert torch.equal(a[4], b[4])


def test_kept_transitions_are_the_segment_maps():
    """Each kept T_seg is the linear part of the segment's state map: for any
    start state S0, the oracle's end state from S0 minus its end state from
    zero is T_seg S0 (the recurrence is affine in the state)."""
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(P("trans", B=2, T=700, Hq=1, Hv=2, init_state=True))
    dd = to_dev(d)
    P_ = 4   # 11 chunks per sequence: segments of chunks [0,3) [3,6) [6,9) [9,11)
    out = gdr.chunk_gated_delta_rule_fwd_states(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], cp_segments=P_)
    torch.cuda.synchronize()
    trans = out[4].cpu().double().view(2 * 2, P_, 128, 128)
    rng = np.random.default_rng(11)
    for n in range(2):
        for p in (1, 2):   # the segments that are neither first nor last
            t0, t1 = 64 * 3 * p, 64 * 3 * (p + 1)
            sl = lambda x: np64(x[n:n + 1, t0:t1])
            args = (sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), d["scale"])
            s0 = rng.standard_normal((1, 2, 128, 128)) * 0.1
            _, e1 = oracle.fwd(*args, initial_state=s0)
            _, e0 = oracle.fwd(*args, initial_state=np.zeros_like(s0))
            for h in range(2):
                want = e1[0, h] - e0[0, h]
                got = trans[n * 2 + h, p].numpy() @ s0[0, h]
                r = ratio(got, want)
                print("sequence", n, "segment", p, "head", h, "ratio", r, flush=True)
                assert r <= TOL, (n, p, h, r)


PIPE_OPTS = {"plain": {}, "qk_norm": dict(use_qk_l2norm_in_kernel=True),
             "beta_logit_neg": dict(use_beta_sigmoid_in_kernel=True, allow_neg_eigval=True),
             "qk_norm_beta_logit": dict(use_qk_l2norm_in_kernel=True,
                                        use_beta_sigmoid_in_kernel=True),
             "gate": "gate"}


@pytest.mark.parametrize("name", list(PIPE_OPTS))
def test_pipelined_backward_equals_the_one_pass_backward(name):
    """The pipelined backward hands the fp32 state gradient from slice to
    slice unrounded and runs the same per-chunk work, so its results are the
    one-pass (recomputing) backward's, bit for bit, under every option."""
    import gated_delta_rule_66_amd as gdr
    opts = PIPE_OPTS[name]
    d = gdr_synth.make(CASES["pipe"])
    dd = to_dev(d)
    print("case pipe", name, flush=True)
    kw = dict(scale=dd["scale"], initial_state=dd["h0"], cp_segments=1, wave_tiles=1)
    g = dd["g"]
    if opts == "gate":
        gen = torch.Generator().manual_seed(3)
        A_log = (torch.rand(2, generator=gen) * 2 - 1).to(g.device)
        dt_bias = (torch.rand(2, generator=gen) - 0.5).to(g.device)
        opts = dict(use_gate_in_kernel=True, A_log=A_log, dt_bias=dt_bias)
    g_cum, A, o, h, trans, ht = gdr.chunk_gated_delta_rule_fwd_states(
        dd["q"], dd["k"], dd["v"], g, dd["beta"], **kw, **opts)
    # nothing is split; with q / k normalised the forward keeps the unit rows
    qkn = bool(opts.get("use_qk_l2norm_in_kernel"))
    assert (trans is not None) == qkn
    bkw = dict(kw, dht=dd["dht"], dg_dtype=g.dtype, **opts)
    if "A_log" in opts:
        bkw["g_input"] = g
    piped = gdr.chunk_gated_delta_rule_bwd(dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A,
                                           dd["do"], h=h, trans=trans, **bkw)
    plain = gdr.chunk_gated_delta_rule_bwd(dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A,
                                           dd["do"], **bkw)
    runs = [piped]
    if qkn:  # the states without the unit rows: the backward normalises q, k itself
        runs.append(gdr.chunk_gated_delta_rule_bwd(dd["q"], dd["k"], dd["v"], g_cum,
                                                   dd["beta"], A, dd["do"], h=h, **bkw))
    torch.cuda.synchronize()
    for run in runs:
        for i, (x, y) in enumerate(zip(run, plain)):
            assert (x is None and y is None) or torch.equal(x, y), i


def test_pipelined_backward_in_both_state_layouts():
    """The pipelined backward hands its fp32 gradient between slices in the
    key-major layout whatever the caller's state layout: value-first states
    give the same results, bit for bit, with dh0 transposed."""
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(CASES["pipe"])
    dd = to_dev(d)
    out = []
    for svf in (False, True):
        h0, dht = dd["h0"], dd["dht"]
        if svf:
            h0, dht = h0.transpose(-1, -2).contiguous(), dht.transpose(-1, -2).contiguous()
        kw = dict(scale=dd["scale"], initial_state=h0, state_v_first=svf, cp_segments=1)
        g_cum, A, o, h, trans, ht = gdr.chunk_gated_delta_rule_fwd_states(
            dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **kw)
        out.append(gdr.chunk_gated_delta_rule_bwd(
            dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dht,
            dg_dtype=dd["g"].dtype, h=h, **kw))
    torch.cuda.synchronize()
    for x, y in zip(out[0][:5], out[1][:5]):
        assert torch.equal(x, y)
    assert torch.equal(out[0][5].transpose(-1, -2), out[1][5])
