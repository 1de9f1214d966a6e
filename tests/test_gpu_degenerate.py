"""GPU parity on the degenerate ends of the method (needs an MI355X): decay so
strong that e^gamma underflows inside a chunk, no decay at all, beta = 0 (no
writes), beta = 1 on unit keys (exact overwrites), and many tiny packed
sequences (mostly shorter than one chunk, one empty)."""
import numpy as np
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, check, np64, ratio, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def base(**kw):
    kw.setdefault("B", 2)
    kw.setdefault("T", 150)
    return gdr_synth.Problem("degenerate", Hq=2, Hv=2, init_state=True, backward=True, dht=True,
                             **kw)


def strong_decay():
    return gdr_synth.make(base(g_shift=-6.0))     # g about -6 per token: e^gamma -> 0 in a chunk


def no_decay():
    d = gdr_synth.make(base())
    d["g"] = torch.zeros_like(d["g"], dtype=torch.float32)
    return d


def beta_zero():
    # slow decay: with nothing written the state only decays, and over 150
    # tokens of the default gates it would fall below fp32's range
    d = gdr_synth.make(base(g_shift=4.0))
    d["beta"] = torch.zeros_like(d["beta"])
    return d


def beta_one():
    d = gdr_synth.make(base())
    d["beta"] = torch.ones_like(d["beta"])
    return d


def tiny_sequences():
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 11, size=100)]
    lens[37] = 0
    lens[80] = 64
    lens[81] = 65
    return gdr_synth.make(gdr_synth.Problem("tiny", B=1, T=0, Hq=2, Hv=4, init_state=True,
                                            backward=True, dht=True, lens=lens))


CASES = {"strong_decay": strong_decay, "no_decay": no_decay, "beta_zero": beta_zero,
         "beta_one_unit_keys": beta_one, "tiny_sequences": tiny_sequences}


@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_fwd_bwd(name):
    import gated_delta_rule_66_amd as gdr
    d = CASES[name]()
    print("case", name, flush=True)
    dd = to_dev(d)
    cu_cpu = d["cu_seqlens"]
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"], initial_state=dd["h0"],
        output_final_state=True, cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=cu_cpu)
    grads = gdr.chunk_gated_delta_rule_bwd(
        dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
        scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
        dg_dtype=dd["g"].dtype, cu_seqlens_cpu=cu_cpu)
    torch.cuda.synchronize()
    for t in (o, ht) + tuple(grads):
        assert torch.isfinite(t).all()
    cu = None if cu_cpu is None else cu_cpu.numpy()
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]), d["scale"])
    o_r, ht_r = oracle.fwd(*args, initial_state=np64(d["h0"]), cu_seqlens=cu)
    ref = oracle.bwd(*args, np64(d["do"]), initial_state=np64(d["h0"]), dht=np64(d["dht"]),
                     cu_seqlens=cu)
    res = {"o": check("o", o, o_r, "tok", d["cu_seqlens"]), "final_state": check("final_state", ht, ht_r, "state")}
    for nm, x, r in zip(NAMES, grads, ref):
        res[nm] = check(nm, x, r, "state" if nm in ("dh0", "final_state") else "tok", d["cu_seqlens"])
    print({k: round(v, 5) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)
    if name == "beta_zero":
        # nothing is written: dk and dv vanish exactly, the state only decays
        assert float(grads[1].abs().max()) == 0.0 and float(grads[2].abs().max()) == 0.0


def test_tiny_sequences_token_by_token():
    import gated_delta_rule_66_amd as gdr
    d = tiny_sequences()
    dd = to_dev(d)
    o, ht = gdr.fused_recurrent_gated_delta_rule(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"], initial_state=dd["h0"],
        cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=d["cu_seqlens"])
    torch.cuda.synchronize()
    o_r, ht_r = oracle.fwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]),
                           d["scale"], initial_state=np64(d["h0"]),
                           cu_seqlens=d["cu_seqlens"].numpy())
    check("o", o, o_r, "tok", d["cu_seqlens"])
    check("final_state", ht, ht_r, "state")
    assert torch.equal(ht[37].cpu(), d["h0"][37])  # the empty sequence keeps its state
