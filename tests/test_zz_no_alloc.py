"""The forward without allocation (gdr_chunk_fwd_noalloc) against the forward
with a caller's workspace (gdr_chunk_fwd), through the C ABI (needs an
MI355X).  Two calls in a row, the second on a smaller problem, so the second
runs on the static scratch the first left behind."""
import pytest
import torch

import gdr_synth
import oracle
from _util import check, np64, to_dev

pytestmark = pytest.mark.gpu


def fwd(d, cp, no_alloc):
    import gated_delta_rule_66_amd as gdr
    dd = to_dev(d)
    out = gdr.chunk_gated_delta_rule_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"],
                                         scale=dd["scale"], initial_state=dd["h0"],
                                         output_final_state=True, cu_seqlens=dd["cu_seqlens"],
                                         cu_seqlens_cpu=d["cu_seqlens"], output_h=True,
                                         cp_segments=cp, no_alloc=no_alloc)
    torch.cuda.synchronize()
    return out


# (lengths, Hq, Hv, forced context-parallel segments): packed sequences split
# in segments, so the scratch holds chunk offsets and segment buffers
CALLS = [([700, 1300, 90], 2, 4, 4), ([100, 260], 1, 2, 3)]


def test_no_alloc_forward_matches_the_workspace_forward_twice():
    for lens, hq, hv, cp in CALLS:
        prob = gdr_synth.Problem("noalloc", B=1, T=0, Hq=hq, Hv=hv, init_state=True, lens=lens)
        d = gdr_synth.make(prob)
        print("no-alloc forward: lengths", lens, "Hq", hq, "Hv", hv, "cp", cp, flush=True)
        got = fwd(d, cp, True)
        ref = fwd(d, cp, False)
        for name, x, y in zip(("g_cum", "A", "o", "h", "final_state"), got, ref):
            assert torch.equal(x, y), name    # same plan, same kernels: identical bits
        cu = d["cu_seqlens"]
        o_r, ht_r = oracle.fwd(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["g"]),
                               np64(d["beta"]), d["scale"], initial_state=np64(d["h0"]),
                               cu_seqlens=cu.numpy())
        check("o", got[2], o_r, "tok", cu)
        check("final_state", got[4], ht_r, "state")
