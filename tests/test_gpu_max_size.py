"""Past 2^31 elements (needs an MI355X with about 80 GB free): 4,200 packed
sequences of 130 tokens at 32 heads, so q, k, v, o, do and their gradients
each hold 2.24e9 elements (4.5 GB), and the last sequences sit beyond every
32-bit element and byte offset.  The first, a middle and the last sequence
are checked against the fp64 oracle, forward and backward.

The inputs are drawn on the device with a seeded torch generator (the same
distributions as the other problems: unit q / k rows, logsigmoid gates,
sigmoid betas); only the sampled sequences are copied to the host."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from _util import TOL, ratio

pytestmark = pytest.mark.gpu

NSEQ, L, H = 4200, 130, 32
SAMPLE = (0, 2100, NSEQ - 1)


def draw(gen, *shape, unit=False):
    x = torch.randn(*shape, device="cuda", generator=gen)
    if unit:
        x = F.normalize(x, p=2.0, dim=-1)
    return x.to(torch.bfloat16)


def test_beyond_32bit_offsets():
    import gated_delta_rule_66_amd as gdr
    free, _ = torch.cuda.mem_get_info()
    if free < (90 << 30):
        pytest.skip("needs about 90 GB of free device memory")
    T = NSEQ * L
    assert T * H * 128 > 2**31
    gen = torch.Generator(device="cuda").manual_seed(0)
    q = draw(gen, 1, T, H, 128, unit=True)
    k = draw(gen, 1, T, H, 128, unit=True)
    v = draw(gen, 1, T, H, 128)
    g = F.logsigmoid(torch.randn(1, T, H, device="cuda", generator=gen)).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn(1, T, H, device="cuda", generator=gen)).to(torch.bfloat16)
    do = draw(gen, 1, T, H, 128)
    cu_cpu = torch.arange(NSEQ + 1, dtype=torch.int32) * L
    cu = cu_cpu.cuda()
    scale = 128 ** -0.5
    print("max size: T", T, "elements per tensor", T * H * 128, flush=True)
    g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
        q, k, v, g, beta, scale=scale, output_final_state=True, cu_seqlens=cu,
        cu_seqlens_cpu=cu_cpu)
    dq, dk, dv, db, dg, _ = gdr.chunk_gated_delta_rule_bwd(
        q, k, v, g_cum, beta, A, do, scale=scale, cu_seqlens=cu, cu_seqlens_cpu=cu_cpu)
    torch.cuda.synchronize()
    del A, g_cum
    for n in SAMPLE:
        sl = slice(n * L, (n + 1) * L)
        f = lambda t: t[:, sl].float().cpu().numpy().astype(np.float64)
        args = (f(q), f(k), f(v), f(g), f(beta), scale)
        o_r, ht_r = oracle.fwd(*args)
        ref = oracle.bwd(*args, f(do))
        res = {"o": ratio(f(o), o_r),
               "final_state": ratio(ht[n:n + 1].double().cpu().numpy(), ht_r)}
        for nm, x, r in zip(("dq", "dk", "dv", "dbeta", "dg"), (dq, dk, dv, db, dg), ref):
            res[nm] = ratio(f(x), r)
        print("sequence", n, {kk: round(vv, 5) for kk, vv in res.items()}, flush=True)
        for kk, vv in res.items():
            assert vv <= TOL, (n, kk, vv)
    del q, k, v, g, beta, do, o, ht, dq, dk, dv, db, dg
    torch.cuda.empty_cache()
