"""Full-size parity: the four large workloads at their real shapes, run with
the library's own launch plan (the one bench.py times), checked against the
fp64 oracle on sampled value heads (whole q/k groups; the (sequence, head)
chains are independent, so a head's outputs depend only on its own inputs)."""
import numpy as np
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, ratio

pytestmark = pytest.mark.gpu


def f64(t):
    return None if t is None else t.float().numpy().astype(np.float64)


def run_full(i, heads, svf_check=False, states=False):
    """states: the launch configuration bench.py times (the autograd op's):
    the forward keeps its chunk-start states and segment transitions and the
    backward takes them."""
    import gated_delta_rule_66_amd as gdr
    if i == "headline":
        prob = gdr_synth.Problem("fwd_bwd_B2_T4096_H32", B=2, T=4096, Hq=32, Hv=32,
                                 init_state=True, backward=True, dht=True)
        d = gdr_synth.make(prob)
    else:
        prob, d = gdr_synth.make_workload(i)
    print("workload", i, prob.name, "T", prob.T, "heads", heads, "states", states, flush=True)
    dev = torch.device("cuda", 0)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu_cpu = d["cu_seqlens"]
    for bwd in (False, True):
        cp, vt = gdr.plan_info(dd["q"], dd["v"], cu_seqlens=dd["cu_seqlens"],
                               cu_seqlens_cpu=cu_cpu, backward=bwd, h_packed=states)
        print("plan", "bwd" if bwd else "fwd", "cp", cp, "wave_tiles", vt, flush=True)

    def fwd_bwd(svf):
        h0 = dd["h0"]
        dht = dd["dht"]
        if svf:
            h0 = None if h0 is None else h0.transpose(-1, -2).contiguous()
            dht = None if dht is None else dht.transpose(-1, -2).contiguous()
        fkw = dict(scale=dd["scale"], initial_state=h0, output_final_state=True,
                   cu_seqlens=dd["cu_seqlens"], state_v_first=svf, cu_seqlens_cpu=cu_cpu)
        h = trans = None
        if states:
            g_cum, A, o, h, trans, ht = gdr.chunk_gated_delta_rule_fwd_states(
                dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **fkw)
        else:
            g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
                dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **fkw)
        grads = None
        if prob.backward:
            grads = gdr.chunk_gated_delta_rule_bwd(
                dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dht,
                scale=dd["scale"], initial_state=h0, cu_seqlens=dd["cu_seqlens"],
                state_v_first=svf, dg_dtype=dd["g"].dtype, cu_seqlens_cpu=cu_cpu, h=h,
                trans=trans)
        torch.cuda.synchronize()
        return o, ht, grads

    o, ht, grads = fwd_bwd(False)
    if svf_check:
        o2, ht2, grads2 = fwd_bwd(True)
        assert torch.equal(o, o2)
        assert torch.equal(ht.transpose(-1, -2), ht2)
        for x, y in zip(grads[:5], grads2[:5]):
            assert torch.equal(x, y)
        if grads[5] is not None:
            assert torch.equal(grads[5].transpose(-1, -2), grads2[5])
        del o2, ht2, grads2

    G = prob.Hv // prob.Hq
    qh = sorted({h // G for h in heads})
    vh = [hq * G + r for hq in qh for r in range(G)]
    sel = lambda t, hs, dim=2: None if t is None else t.index_select(dim, torch.tensor(hs))
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy().astype(np.int64)
    args = (f64(sel(d["q"], qh)), f64(sel(d["k"], qh)), f64(sel(d["v"], vh)), f64(sel(d["g"], vh)),
            f64(sel(d["beta"], vh)), d["scale"])
    h0s = f64(sel(d["h0"], vh, 1))
    o_ref, ht_ref = oracle.fwd(*args, initial_state=h0s, cu_seqlens=cu, nthreads=16)
    res = {"o": check("o", f64(sel(o.cpu(), vh)), o_ref, "tok", cu),
           "final_state": check("final_state", f64(sel(ht.cpu(), vh, 1)), ht_ref, "state")}
    if prob.backward:
        g_ref = oracle.bwd(*args[:5], d["scale"], f64(sel(d["do"], vh)), initial_state=h0s,
                           dht=f64(sel(d["dht"], vh, 1)), cu_seqlens=cu, nthreads=16)
        got = [sel(grads[0].cpu(), qh), sel(grads[1].cpu(), qh), sel(grads[2].cpu(), vh),
               sel(grads[3].cpu(), vh), sel(grads[4].cpu(), vh),
               None if grads[5] is None else sel(grads[5].cpu(), vh, 1)]
        for name, x, r in zip(("dq", "dk", "dv", "dbeta", "dg", "dh0"), got, g_ref):
            res[name] = check(name, None if x is None else f64(x), r,
                              "state" if name == "dh0" else "tok", cu)
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)


def test_full_forward_B2_T4096_H32_with_state():
    run_full(1, heads=[0, 17, 31])


def test_full_varlen8_H32_fwd_bwd():
    run_full(2, heads=[0, 31])


def test_full_gva_B4_T8192_fp16_fwd_bwd_both_state_layouts():
    run_full(3, heads=[2, 3], svf_check=True)


def test_full_long_T65536_H32_fwd_bwd_context_parallel():
    run_full(4, heads=[5])


# the launch configuration bench.py times: the states path


def test_full_headline_fwd_bwd_B2_T4096_H32_states():
    run_full("headline", heads=[0, 13, 31], states=True)


def test_full_varlen8_H32_fwd_bwd_states():
    run_full(2, heads=[7], states=True)


def test_full_gva_B4_T8192_fp16_fwd_bwd_states_both_layouts():
    run_full(3, heads=[5], svf_check=True, states=True)


def test_full_long_T65536_H32_fwd_bwd_states_context_parallel():
    run_full(4, heads=[21], states=True)
