"""GPU parity of the token-by-token forward (gdr_recurrent_fwd: decode steps,
short inputs, continuation from a cached state) against the fp64 token
recurrence of the oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import gdr_synth
import oracle
from _util import TOL, np64, ratio, to_dev

pytestmark = pytest.mark.gpu


def P(name, **kw):
    return gdr_synth.Problem(name, **kw)


CASES = {
    "decode_B16_H4": P("decode", B=16, T=1, Hq=4, Hv=4, init_state=True),
    "T7_state": P("t7", B=2, T=7, Hq=2, Hv=2, init_state=True),
    "T7_no_state": P("t7n", B=2, T=7, Hq=2, Hv=2),
    "varlen_empty": P("varlen", B=1, T=0, Hq=2, Hv=2, init_state=True, lens=[1, 0, 5, 33]),
    "gva_fp16": P("gva", B=3, T=4, Hq=1, Hv=4, dtype="fp16", init_state=True),
    "qk_l2norm": P("l2", B=2, T=9, Hq=2, Hv=2, init_state=True, qk_l2norm=True),
    "long_T300": P("long", B=1, T=300, Hq=1, Hv=2, init_state=True, g_shift=2.0),
}


def run(d, svf=False, inplace=False):
    import gated_delta_rule_66_amd as gdr
    dd = to_dev(d)
    h0 = dd["h0"]
    if h0 is not None and svf:
        h0 = h0.transpose(-1, -2).contiguous()
    if h0 is not None and inplace:
        h0 = h0.clone()
    o, ht = gdr.fused_recurrent_gated_delta_rule(
        dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"], initial_state=h0,
        output_final_state=True, cu_seqlens=dd["cu_seqlens"], state_v_first=svf,
        use_qk_l2norm_in_kernel=d["qk_l2norm"], inplace_final_state=inplace,
        cu_seqlens_cpu=d["cu_seqlens"])
    torch.cuda.synchronize()
    if inplace:
        assert ht.data_ptr() == h0.data_ptr()
    return o, ht


def reference(d):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    return oracle.fwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]), np64(d["beta"]),
                      d["scale"], initial_state=np64(d["h0"]), cu_seqlens=cu,
                      use_qk_l2norm=d["qk_l2norm"])


@pytest.mark.parametrize("svf", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_recurrent_matches_oracle(name, svf):
    d = gdr_synth.make(CASES[name])
    print("case", name, "svf", svf, flush=True)
    o, ht = run(d, svf=svf)
    o_r, ht_r = reference(d)
    if svf:
        ht = ht.transpose(-1, -2)
    res = {"o": ratio(np64(o), o_r), "final_state": ratio(np64(ht), ht_r)}
    print({k: round(v, 6) for k, v in res.items()}, flush=True)
    for k, v in res.items():
        assert v <= TOL, (k, v)


def test_in_place_state_is_bitwise_the_out_of_place_result():
    d = gdr_synth.make(CASES["varlen_empty"])
    o1, ht1 = run(d)
    o2, ht2 = run(d, inplace=True)
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    # the empty sequence keeps its initial state
    assert torch.equal(ht1[1].cpu(), d["h0"][1])


def test_decode_continues_a_chunked_prefill():
    """Prefill 200 tokens with the chunked forward, then decode 5 tokens one
    step at a time, updating the state in place: outputs and state follow the
    recurrence over all 205 tokens."""
    import gated_delta_rule_66_amd as gdr
    d = gdr_synth.make(P("cont", B=2, T=205, Hq=2, Hv=4, init_state=True))
    dd = to_dev(d)
    sl = lambda t, a, b: t[:, a:b].contiguous()
    _, _, o_pre, _, state = gdr.chunk_gated_delta_rule_fwd(
        sl(dd["q"], 0, 200), sl(dd["k"], 0, 200), sl(dd["v"], 0, 200), sl(dd["g"], 0, 200),
        sl(dd["beta"], 0, 200), scale=dd["scale"], initial_state=dd["h0"],
        output_final_state=True)
    outs = [o_pre]
    for t in range(200, 205):
        o_t, state2 = gdr.fused_recurrent_gated_delta_rule(
            sl(dd["q"], t, t + 1), sl(dd["k"], t, t + 1), sl(dd["v"], t, t + 1),
            sl(dd["g"], t, t + 1), sl(dd["beta"], t, t + 1), scale=dd["scale"],
            initial_state=state, inplace_final_state=True)
        assert state2.data_ptr() == state.data_ptr()
        outs.append(o_t)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    o_r, ht_r = reference(d)
    assert ratio(np64(o), o_r) <= TOL
    assert ratio(np64(o[:, 200:]), o_r[:, 200:]) <= TOL
    assert ratio(np64(state), ht_r) <= TOL


def test_decode_full_B256_H32():
    """One decode step at serving size (256 sequences x 32 heads), sampled
    (sequence, head) units against the oracle."""
    prob = P("decode_full", B=256, T=1, Hq=32, Hv=32, init_state=True)
    d = gdr_synth.make(prob)
    o, ht = run(d)
    seqs, heads = [0, 77, 255], [0, 19, 31]
    pick = lambda t, hd=2: t[seqs][:, :, heads] if hd == 2 else t[seqs][:, heads]
    f = lambda t: t.float().numpy().astype(np.float64)
    o_r, ht_r = oracle.fwd(f(pick(d["q"])), f(pick(d["k"])), f(pick(d["v"])), f(pick(d["g"])),
                           f(pick(d["beta"])), d["scale"], initial_state=f(pick(d["h0"], 1)))
    assert ratio(f(pick(o.cpu())), o_r) <= TOL
    assert ratio(f(pick(ht.cpu(), 1)), ht_r) <= TOL
