"""Seeded synthetic inputs for the chunked gated delta rule.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the fp64 oracle side and the HIP side of the tests
and the benchmark can use it.

Recipe (one CPU ``torch.Generator`` per problem, drawn in this fixed order):
packed lengths (variable-length problems only) -> q -> k -> v -> g -> beta ->
initial state -> do -> dht.

* q, k ~ N(0, 1) in fp32, L2-normalised over the head dimension per
  (token, head), then rounded to the input dtype.  Problems that ask the
  kernel to normalise (``qk_l2norm``) keep the raw N(0, 1) rows instead.
* v ~ N(0, 1); g = logsigmoid(N(shift, 1)) (a natural-log decay <= 0;
  ``shift = 2`` gives the slow-decay long-context workload);
  beta = sigmoid(N(0, 1)) (the logit N(0, 1) itself for problems whose kernel
  takes the sigmoid); all rounded to the input dtype (round to nearest
  even), the way bf16 / fp16 inputs reach a kernel.
* initial state and dht = 0.1 * N(0, 1), kept in fp32 (std 0.1).
* do ~ N(0, 1) in the input dtype.
* packed lengths: uniform integers in [lo, hi], redrawn while a multiple of 64,
  so that every sequence ends in a ragged chunk.
* problems with the in-kernel gate (``gate``) keep g as the raw gate input
  N(shift, 1) (no logsigmoid) and draw, after everything else, the per-head
  parameters A_log = log U(1, 16) and dt_bias ~ U(-6.9, -2.3) in fp32 (the
  ranges of a Mamba-2 style initialisation: decay rates 1..16 and step sizes
  of about 0.001..0.1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch
import torch.nn.functional as F

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@dataclass
class Problem:
    name: str
    B: int
    T: int
    Hq: int
    Hv: int
    K: int = 128
    V: int = 128
    dtype: str = "bf16"
    lens: Optional[List[int]] = None     # packed variable-length input if set
    init_state: bool = False
    backward: bool = False
    dht: bool = False
    g_shift: float = 0.0
    qk_l2norm: bool = False              # raw q, k rows; the kernel normalises them
    beta_logit: bool = False             # beta drawn as the logit N(0, 1) (sigmoid in-kernel)
    gate: bool = False                   # g is the raw gate input; A_log, dt_bias drawn
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return len(self.lens) if self.lens is not None else self.B

    @property
    def tokens(self) -> int:
        return self.B * self.T


def draw_lengths(n: int, lo: int, hi: int, gen: torch.Generator, avoid_multiple: int = 64):
    out = []
    for _ in range(n):
        while True:
            L = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
            if avoid_multiple is None or L % avoid_multiple != 0:
                break
        out.append(L)
    return out


def make(prob: Problem, lengths_from=None) -> dict:
    """Draw every tensor of ``prob`` on the CPU.

    Returns a dict with q, k, v, g, beta (input dtype), h0, dht (fp32 or None),
    do (input dtype or None), cu_seqlens (int32 or None) and scale.
    """
    gen = torch.Generator().manual_seed(prob.seed)
    dt = DTYPES[prob.dtype]
    cu = None
    if lengths_from is not None:
        # (n, lo, hi): draw the packed lengths first, from the same generator
        n, lo, hi = lengths_from
        prob.lens = draw_lengths(n, lo, hi, gen)
    if prob.lens is not None:
        prob.B = 1
        prob.T = int(sum(prob.lens))
        cu = torch.zeros(len(prob.lens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(prob.lens, dtype=torch.int64), 0).to(torch.int32)
    B, T, Hq, Hv, K, V = prob.B, prob.T, prob.Hq, prob.Hv, prob.K, prob.V
    q = torch.randn(B, T, Hq, K, generator=gen)
    if not prob.qk_l2norm:
        q = F.normalize(q, p=2.0, dim=-1)
    q = q.to(dt)
    k = torch.randn(B, T, Hq, K, generator=gen)
    if not prob.qk_l2norm:
        k = F.normalize(k, p=2.0, dim=-1)
    k = k.to(dt)
    v = torch.randn(B, T, Hv, V, generator=gen).to(dt)
    g = torch.randn(B, T, Hv, generator=gen) + prob.g_shift
    g = (g if prob.gate else F.logsigmoid(g)).to(dt)
    beta = torch.randn(B, T, Hv, generator=gen)
    beta = (beta if prob.beta_logit else torch.sigmoid(beta)).to(dt)
    N = prob.N
    h0 = (0.1 * torch.randn(N, Hv, K, V, generator=gen)) if prob.init_state else None
    do = torch.randn(B, T, Hv, V, generator=gen).to(dt) if prob.backward else None
    dht = (0.1 * torch.randn(N, Hv, K, V, generator=gen)) if (prob.backward and prob.dht) else None
    A_log = dt_bias = None
    if prob.gate:
        A_log = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=gen))
        dt_bias = -6.9 + 4.6 * torch.rand(Hv, generator=gen)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, do=do, dht=dht, cu_seqlens=cu,
                scale=K ** -0.5, qk_l2norm=prob.qk_l2norm, A_log=A_log, dt_bias=dt_bias)


# The five workloads.  Sizes are those of the pages' API example
# (B=2, T=4096, H=32, K=V=128) and of the dense / varlen / GVA / long-context
# cases their test plan names.
def workload(i: int) -> Problem:
    if i == 0:
        return Problem("fwd_B1_T256_H2", B=1, T=256, Hq=2, Hv=2)
    if i == 1:
        return Problem("fwd_B2_T4096_H32_state", B=2, T=4096, Hq=32, Hv=32, init_state=True)
    if i == 2:
        return Problem("varlen8_H32_fwdbwd", B=1, T=0, Hq=32, Hv=32, init_state=True,
                       backward=True, dht=True, extra=dict(varlen=(8, 128, 4096)))
    if i == 3:
        return Problem("gva_B4_T8192_Hq16_Hv32_fp16", B=4, T=8192, Hq=16, Hv=32, dtype="fp16",
                       backward=True)
    if i == 4:
        return Problem("long_B1_T65536_H32_fwdbwd", B=1, T=65536, Hq=32, Hv=32, init_state=True,
                       backward=True, dht=True, g_shift=2.0)
    raise ValueError(i)


def make_workload(i: int) -> tuple:
    p = workload(i)
    data = make(p, lengths_from=p.extra.get("varlen"))
    return p, data
