"""GPU parity with the beta options (use_beta_sigmoid_in_kernel: beta is a
logit; allow_neg_eigval: the recurrence uses 2 beta) against the fp64 oracle
run with the same options, forward, backward and token-by-token (needs an
MI355X)."""
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, np64, ratio, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")
OPTS = [(True, False), (False, True), (True, True)]


def P(name, sig, **kw):
    return gdr_synth.Problem(name, beta_logit=sig, **kw)


def shapes(sig):
    return {
        "dense_state_dht": P("dense", sig, B=2, T=200, Hq=2, Hv=2, init_state=True,
                             backward=True, dht=True),
        "fp16_gva_varlen": P("gva", sig, B=1, T=0, Hq=1, Hv=2, dtype="fp16", init_state=True,
                             backward=True, dht=True, lens=[70, 1, 129]),
        "long_cp": P("long", sig, B=1, T=1100, Hq=2, Hv=2, init_state=True, backward=True,
                     dht=True, g_shift=2.0),
    }


def opts_kw(sig, neg):
    return dict(use_beta_sigmoid_in_kernel=sig, allow_neg_eigval=neg)


@pytest.mark.parametrize("sig,neg", OPTS)
@pytest.mark.parametrize("name", ["dense_state_dht", "fp16_gva_varlen", "long_cp"])
def test_beta_options_fwd_bwd(name, sig, neg):
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(shapes(sig)[name])
    dd = to_dev(d)
    cp = 3 if name == "long_cp" else 1
    print("case", name, "sigmoid", sig, "neg_eigval", neg, "cp", cp, flush=True)
    cu_cpu = d["cu_seqlens"]
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"], initial_state=dd["h0"],
        output_final_state=True, cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=cu_cpu,
        cp_segments=cp, **opts_kw(sig, neg))
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
        scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
        dg_dtype=dd["g"].dtype, cu_seqlens_cpu=cu_cpu, cp_segments=cp, **opts_kw(sig, neg))
    torch.cuda.synchronize()
    cu = None if cu_cpu is None else cu_cpu.numpy()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    kw = dict(beta_sigmoid=sig, neg_eigval=neg)
    _, A_r, o_r, _, ht_r = oracle.chunked_fwd(*args, chunk=64, initial_state=np64(d["h0"]),
                                              cu_seqlens=cu, **kw)
    res = {"o": check("o", o, o_r, "tok", d["cu_seqlens"]), "final_state": check("final_state", ht, ht_r, "state"), "A": check("A", A, A_r, "tok", d["cu_seqlens"])}
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                     cu_seqlens=cu, **kw)
    for nm, x, r in zip(NAMES, grads, ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok", d["cu_seqlens"])
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("sig,neg", OPTS)
def test_beta_options_recurrent(sig, neg):
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(P("rec", sig, B=3, T=6, Hq=2, Hv=4, init_state=True))
    dd = to_dev(d)
    o, ht = gdr.fused_recurrent_gated_delta_rule(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], **opts_kw(sig, neg))
    torch.cuda.synchronize()
    o_r, ht_r = oracle.fwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]),
                           d["scale"], initial_state=np64(d["h0"]), beta_sigmoid=sig, neg_eigval=neg)
    check("o", o, o_r, "tok", d["cu_seqlens"])
    check("final_state", ht, ht_r, "state")


def test_autograd_passes_the_options():
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(P("ag", True, B=1, T=130, Hq=2, Hv=2, init_state=True, backward=True,
                         qk_l2norm=True))
    dd = to_dev(d)
    leaves = {n: dd[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta")}
    o, _ = gdr.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"],
                                      leaves["beta"], scale=dd["scale"], initial_state=dd["h0"],
                                      use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True,
                                      allow_neg_eigval=True)
    (o.float() * dd["do"].float()).sum().backward()
    torch.cuda.synchronize()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), use_qk_l2norm=True,
                     beta_sigmoid=True, neg_eigval=True)
    for n, i in (("q", 0), ("k", 1), ("v", 2), ("beta", 3), ("g", 4)):
        check(n, leaves[n].grad, ref[i], "tok", d["cu_seqlens"])


@pytest.mark.parametrize("vt", [1, 2])
def test_beta_options_states_path_split(vt):
    """The forward keeping its states and segment transitions, the backward
    taking them, in three segments, with both beta options."""
    import gated_delta_rule_66_amd as gdr
    sig, neg = True, True
    d = gdr_synth.make(shapes(sig)["long_cp"])
    dd = to_dev(d)
    print("case long_cp states path cp 3 wave_tiles", vt, flush=True)
    g_cum, A, o, h, trans, ht = gdr.chunk_gated_delta_rule_fwd_states(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], output_final_state=True, cp_segments=3, wave_tiles=vt,
        **opts_kw(sig, neg))
    assert trans is not None
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
        scale=dd["scale"], initial_state=dd["h0"], dg_dtype=dd["g"].dtype, cp_segments=3,
        wave_tiles=vt, h=h, trans=trans, **opts_kw(sig, neg))
    torch.cuda.synchronize()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    kw = dict(beta_sigmoid=sig, neg_eigval=neg)
    o_r, ht_r = oracle.fwd(*args, initial_state=np64(d["h0"]), **kw)
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]), **kw)
    res = {"o": check("o", o, o_r, "tok"), "final_state": check("final_state", ht, ht_r, "state")}
    for nm, x, r in zip(NAMES, grads, ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok")
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)
