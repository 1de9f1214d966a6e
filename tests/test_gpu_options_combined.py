"""Every kernel option at once (needs an MI355X): the in-kernel gate, q / k
normalisation, the beta sigmoid and negative eigenvalues, together with
grouped value heads, packed sequences, context parallelism and both state
layouts, against the fp64 oracle run with the same options (gate, then the
q / k normalisation, then the beta map, each chained in its backward)."""
import numpy as np
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, np64, ratio, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def P(name, **kw):
    return gdr_synth.Problem(name, init_state=True, backward=True, dht=True, qk_l2norm=True,
                             beta_logit=True, gate=True, **kw)


# (problem, cp_segments, wave_tiles, state_v_first)
CASES = {
    "varlen_gva_cp3": (P("a", B=1, T=0, Hq=1, Hv=2, lens=[129, 7, 300]), 3, 1, False),
    "fp16_svf_vt2": (P("b", B=2, T=150, Hq=2, Hv=4, dtype="fp16"), 1, 2, True),
    "dense_cp2_svf": (P("c", B=1, T=500, Hq=2, Hv=2), 2, 1, True),
}


def opts(d):
    return dict(use_qk_l2norm=True, beta_sigmoid=True, neg_eigval=True,
                gate=(np64(d["A_log"]), np64(d["dt_bias"])))


@pytest.mark.parametrize("name", list(CASES))
def test_all_options_chunked(name):
    import gated_delta_rule_66_amd as gdr
    prob, cp, vt, svf = CASES[name]
    d = gdr_synth.make(prob)
    print("case", name, flush=True)
    dd = to_dev(d)
    cu_cpu = d["cu_seqlens"]
    tr = (lambda t: t.transpose(-1, -2).contiguous()) if svf else (lambda t: t)
    kw = dict(use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True,
              allow_neg_eigval=True, use_gate_in_kernel=True, A_log=dd["A_log"],
              dt_bias=dd["dt_bias"])
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=tr(dd["h0"]), output_final_state=True, cu_seqlens=dd["cu_seqlens"],
        state_v_first=svf, cp_segments=cp, wave_tiles=vt, cu_seqlens_cpu=cu_cpu, **kw)
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=tr(dd["dht"]),
        scale=dd["scale"], initial_state=tr(dd["h0"]), cu_seqlens=dd["cu_seqlens"],
        state_v_first=svf, cp_segments=cp, wave_tiles=vt, cu_seqlens_cpu=cu_cpu,
        g_input=dd["g"], **kw)
    torch.cuda.synchronize()
    cu = None if cu_cpu is None else cu_cpu.numpy()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    o_r, ht_r = oracle.fwd(*args, initial_state=np64(d["h0"]), cu_seqlens=cu, **opts(d))
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                     cu_seqlens=cu, **opts(d))
    back = (lambda t: t.transpose(-1, -2)) if svf else (lambda t: t)
    res = {"o": check("o", o, o_r, "tok", d["cu_seqlens"]), "final_state": check("final_state", back(ht), ht_r, "state")}
    got = list(grads[:5]) + [back(grads[5])]
    for nm, x, r in zip(NAMES, got, ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok", d["cu_seqlens"])
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)


def test_all_options_token_by_token():
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(P("rec", B=1, T=0, Hq=1, Hv=4, lens=[1, 5, 0, 70]))
    dd = to_dev(d)
    o, ht = gdr.fused_recurrent_gated_delta_rule(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
        initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=d["cu_seqlens"],
        use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True, allow_neg_eigval=True,
        use_gate_in_kernel=True, A_log=dd["A_log"], dt_bias=dd["dt_bias"])
    torch.cuda.synchronize()
    o_r, ht_r = oracle.fwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]),
                           np64(d["beta"]), d["scale"], initial_state=np64(d["h0"]),
                           cu_seqlens=d["cu_seqlens"].numpy(), **opts(d))
    check("o", o, o_r, "tok", d["cu_seqlens"])
    check("final_state", ht, ht_r, "state")
