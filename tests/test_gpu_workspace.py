"""The workspace needs no initialisation: every kernel reads only workspace
memory that an earlier kernel of the same call wrote (needs an MI355X).

Each case runs the forward and the backward on a caller workspace filled with
0xFF bytes (NaN as fp32 and bf16, -1 as int32), so any read of memory the call
did not write shows up as NaN or a wrong value.  The plans include context
parallelism with one-chunk segments, where the transition pass of an inner
segment must start its value columns from zero rather than from the (not yet
chained) segment start state."""
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, np64, ratio, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")
WS_BYTES = 256 << 20


def P(name, **kw):
    kw.setdefault("init_state", True)
    kw.setdefault("backward", True)
    kw.setdefault("dht", True)
    return gdr_synth.Problem(name, **kw)


# (problem, cp_segments, wave_tiles)
CASES = {
    "one_chunk_segments_3": (P("s3", B=1, T=0, Hq=2, Hv=2, lens=[129]), 3, 1),
    "one_chunk_segments_4": (P("s4", B=1, T=0, Hq=2, Hv=2, lens=[250]), 4, 1),
    "mixed_varlen_cp3": (P("mix", B=1, T=0, Hq=2, Hv=2, lens=[70, 1, 64, 129, 250]), 3, 1),
    "dense_cp4_vt2": (P("d4", B=2, T=600, Hq=2, Hv=2, g_shift=2.0), 4, 2),
    "gva_fp16_cp2": (P("gva", B=1, T=333, Hq=1, Hv=4, dtype="fp16"), 2, 1),
    "gate_gva_cp3": (P("gate", B=1, T=0, Hq=1, Hv=2, lens=[129, 200], gate=True), 3, 1),
    "no_cp": (P("plain", B=2, T=200, Hq=2, Hv=4), 1, 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_poisoned_workspace(name):
    import gated_delta_rule_66_amd as gdr
    prob, cp, vt = CASES[name]
    d = gdr_synth.make(prob)
    print("case", name, "cp", cp, "vt", vt, flush=True)
    dd = to_dev(d)
    cu_cpu = d["cu_seqlens"]
    gate = d["A_log"] is not None
    kw = dict(use_gate_in_kernel=True, A_log=dd["A_log"], dt_bias=dd["dt_bias"]) if gate else {}
    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(2):  # the second call finds the first call's leftovers
        if rep == 0:
            ws.fill_(0xFF)
        g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
            dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
            initial_state=dd["h0"], output_final_state=True, cu_seqlens=dd["cu_seqlens"],
            cp_segments=cp, wave_tiles=vt, cu_seqlens_cpu=cu_cpu, workspace=ws, **kw)
        if rep == 0:
            ws.fill_(0xFF)
        bkw = dict(kw, g_input=dd["g"]) if gate else {}
        grads = gdr.chunk_gated_delta_rule_bwd(
            dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
            scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
            cp_segments=cp, wave_tiles=vt, cu_seqlens_cpu=cu_cpu, workspace=ws, **bkw)
        torch.cuda.synchronize()
        outs.append((o, ht) + tuple(grads))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)  # and deterministic
    cu = None if cu_cpu is None else cu_cpu.numpy()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    okw = dict(gate=(np64(d["A_log"]), np64(d["dt_bias"]))) if gate else {}
    o_r, ht_r = oracle.fwd(*args, initial_state=np64(d["h0"]), cu_seqlens=cu, **okw)
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                     cu_seqlens=cu, **okw)
    o, ht = outs[0][:2]
    grads = outs[0][2:]
    res = {"o": check("o", o, o_r, "tok", d["cu_seqlens"]), "final_state": check("final_state", ht, ht_r, "state")}
    for nm, x, r in zip(NAMES, grads, ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok", d["cu_seqlens"])
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for t in outs[0]:
        assert bool(torch.isfinite(t).all())
    for k, v in res.items():
        assert v <= TOL, (k, v)


_SWEEP = {}


def _sweep_reference():
    """Inputs and fp64 results for the plan sweep, computed once."""
    if not _SWEEP:
        d = gdr_synth.make(P("sweep", B=1, T=0, Hq=1, Hv=2,
                             lens=[1, 63, 64, 65, 129, 200, 400, 0, 130]))
        cu = d["cu_seqlens"].numpy()
        args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]),
                d["scale"])
        o_r, ht_r = oracle.fwd(*args, initial_state=np64(d["h0"]), cu_seqlens=cu)
        ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                         cu_seqlens=cu)
        _SWEEP.update(d=d, ref=(o_r, ht_r) + tuple(ref))
    return _SWEEP["d"], _SWEEP["ref"]


@pytest.mark.parametrize("vt", [1, 2])
@pytest.mark.parametrize("cp", [1, 2, 3, 4, 5, 7, 8])
def test_every_plan_on_a_poisoned_workspace(cp, vt):
    """Every segment count and tile width on one packed batch whose sequences
    split into empty, one-chunk and ragged segments: each plan matches the
    oracle on a workspace filled with NaN bytes."""
    import gated_delta_rule_66_amd as gdr
    d, ref = _sweep_reference()
    print("sweep cp", cp, "vt", vt, flush=True)
    dd = to_dev(d)
    cu_cpu = d["cu_seqlens"]
    for bwd in (False, True):  # the plan asked for is the plan that runs (7 chunks at most)
        assert gdr.plan_info(dd["q"], dd["v"], cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=cu_cpu,
                             cp_segments=cp, wave_tiles=vt, backward=bwd) == (min(cp, 7), vt)
    ws = torch.full((WS_BYTES // 4,), 0xFF, dtype=torch.uint8, device="cuda")
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], output_final_state=True, cu_seqlens=dd["cu_seqlens"],
        cp_segments=cp, wave_tiles=vt, cu_seqlens_cpu=cu_cpu, workspace=ws)
    ws.fill_(0xFF)
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
        scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"], cp_segments=cp,
        wave_tiles=vt, cu_seqlens_cpu=cu_cpu, workspace=ws)
    torch.cuda.synchronize()
    res = {}
    for nm, x, r in zip(("o", "final_state") + NAMES, (o, ht) + tuple(grads), ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok", d["cu_seqlens"])
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)
    # the empty sequence keeps its state; its state gradient passes through
    assert torch.equal(ht[7].cpu(), d["h0"][7])
    assert torch.equal(grads[5][7].cpu(), d["dht"][7])
