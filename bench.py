#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule (forward + backward) on one MI355X.

One step = one pass of the whole hot path over one batch: forward (gate cumsum,
WY inverse, state scan with output, intra-GPU context parallelism when the plan
uses it; the chunk-start states are kept) and backward (reverse
state-gradient scan and per-chunk gradients from the forward's states; with
``--recompute-states`` the backward recomputes them instead).  The default workload is B=2, T=4096, Hq=Hv=32, K=V=128, bf16 with
an initial state and a final-state gradient (the shape of the FlashQLA API
example), synthetic seeded inputs resident in HBM before timing starts.

Prints one JSON line.  ``value`` / ``ms_per_step`` time exactly ``--steps``
back-to-back steps with two events and nothing else inside.  Separate passes
then time the forward and backward alone, cold runs (a 512 MiB buffer write
before each run, so no input is served from the 256 MiB Infinity Cache), and
every library kernel with HIP events on its own stream (the dominant kernel
gives the ``roofline`` entry).  Fractions of peak use the minimum bytes of each
pass (every input read once, every output written once, nothing intermediate
in HBM) and its algorithmic flops.  A ``configs`` block times every workload
the path is specified on the same way.  The CPU baseline times the fp64 oracle
on a bounded sample of the default workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
FWD_FLOP = 140629               # algorithmic flop per (token, value head), forward
BWD_FLOP = 393216               # backward, counted with the state recompute

# The workloads the path is specified on, each timed in the same run (the
# "configs" block of the JSON line).  The B=1 T=256 H=2 forward is a parity case
# only.  name: (direction, B, T, Hq, Hv, dtype, g_shift, varlen, h0, dht, svf)
CONFIGS = {
    "1_fwd_B2_T4096_H32_bf16": ("fwd", 2, 4096, 32, 32, "bf16", 0.0, None, True, False, False),
    "2_fwd_bwd_varlen8_H32_bf16": ("fwd+bwd", 1, 0, 32, 32, "bf16", 0.0, (8, 128, 4096), True,
                                   True, False),
    "3_fwd_bwd_B4_T8192_Hq16_Hv32_fp16": ("fwd+bwd", 4, 8192, 16, 32, "fp16", 0.0, None, False,
                                          False, False),
    "3_fwd_bwd_B4_T8192_Hq16_Hv32_fp16_svf": ("fwd+bwd", 4, 8192, 16, 32, "fp16", 0.0, None,
                                              False, False, True),
    "4_fwd_bwd_B1_T65536_H32_bf16": ("fwd+bwd", 1, 65536, 32, 32, "bf16", 2.0, None, True, True,
                                     False),
}
STATE_BYTES = 128 * 128 * 4     # one fp32 state, per (sequence, value head)
FLUSH_BYTES = 512 << 20         # written before each cold run: more than the 256 MiB MALL
FWD_KERNELS = ("fwd_prep", "scan_out", "scan_aug", "scan_state", "cp_combine_fwd")
BWD_KERNELS = ("bwd_scans", "bwd_scan_aug", "cp_combine_bwd", "bwd_pipe", "bwd_dyn",
               "bwd_flags", "grad", "gate_param_grad")


def alg_bytes_per_unit(direction, r, isz=2, gsz=2):
    """Minimum HBM bytes per (token, value head) of one pass, with nothing
    intermediate in HBM (each input read once, each output written once);
    r = Hq / Hv, isz the input dtype's size, gsz that of g (and dg).
    Forward: q, k (2 x 128 isz r), v, o (128 isz each), g, beta, A (64 isz),
    g_cum (4): 1160 B at r = 1 and 904 B at r = 1/2 for 16-bit inputs.
    Backward: q, k, dq, dk (4 x 128 isz r), v, do, dv (128 isz each), g_cum (4),
    beta, dbeta, A (64 isz), dg: 1930 B and 1418 B."""
    if direction == "fwd":
        return 2 * 128 * isz * r + 128 * isz + gsz + isz + 128 * isz + 64 * isz + 4
    if direction == "bwd":
        return 4 * 128 * isz * r + 3 * 128 * isz + 4 + 2 * isz + 64 * isz + gsz
    raise ValueError(direction)


def pass_bytes(direction, tokens, Hq, Hv, N, n_states, isz=2, gsz=2):
    """Minimum bytes of a whole pass: the per-(token, value head) figure times
    tokens x Hv, plus 64 KiB per (sequence, value head) for each fp32 state
    tensor the pass reads or writes (forward: initial and final state;
    backward: initial state, dht and dh0)."""
    return (tokens * Hv * alg_bytes_per_unit(direction, Hq / Hv, isz, gsz)
            + N * Hv * n_states * STATE_BYTES)


def fractions(t_s, flop, nbytes):
    """HBM, MFMA and roofline fractions of a time t_s for `flop` and `nbytes`
    of algorithmic work: each is the time its bound alone allows divided by
    t_s; the roofline fraction takes the larger of the two bounds."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flop / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {"hbm": round(t_hbm / t_s, 4), "mfma": round(t_mfma / t_s, 4),
            "roofline": round(max(t_hbm, t_mfma) / t_s, 4),
            "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "GBs": round(nbytes / t_s / 1e9, 1), "tflops": round(flop / t_s / 1e12, 2)}



WORKLOADS = {
    # name: (B, T, Hq, Hv, dtype, g_shift, varlen, initial state, dht), the
    # states as in the configs block
    "fwd_bwd_B2_T4096_H32_bf16": (2, 4096, 32, 32, "bf16", 0.0, None, True, True),
    "fwd_bwd_varlen8_H32_bf16": (1, 0, 32, 32, "bf16", 0.0, (8, 128, 4096), True, True),
    "fwd_bwd_B4_T8192_Hq16_Hv32_fp16": (4, 8192, 16, 32, "fp16", 0.0, None, False, False),
    "fwd_bwd_B1_T65536_H32_bf16": (1, 65536, 32, 32, "bf16", 2.0, None, True, True),
}
DEFAULT = "fwd_bwd_B2_T4096_H32_bf16"
# token-by-token forward: (B sequences, Hv = Hq heads, tokens per step, dtype)
DECODE_WORKLOADS = {"decode_B256_H32_bf16": (256, 32, 1, "bf16")}


def kernel_bytes(name, B, T, Hq, Hv, nchunks, N, cp, isz=2, gsz=2, with_h0=True, with_dht=True,
                 qk_norm=False, states=True):
    """Operand bytes of one launch of a library kernel: every operand it
    touches read once and every result it writes written once, workspace
    intermediates (the chunk states and state gradients) included.  With
    ``states`` the forward scan writes the chunk-start states and the
    backward's scan launch runs the state-gradient scan alone.  A per-kernel diagnostic: the roofline fractions use
    the pass minimum of pass_bytes instead.  Per (token, value head) terms with r = Hq / Hv:
    q, k 256 r each, v / o / do / dv 256, A 128, g_cum 4, beta 2, g 2;
    chunk states 32 KiB (bf16) per (chunk, head); fp32 states 64 KiB per
    (sequence, head)."""
    TH = B * T * Hv
    r = Hq / Hv
    NCH = nchunks * Hv
    U = N * Hv
    st = 128 * 128 * 4
    ch = 128 * 128 * isz
    frac = (cp - 1) / cp if cp > 1 else 0.0
    if name == "fwd_prep":
        return TH * (256 * r + gsz + isz + 4 + 128)
    if name == "scan_out":
        return (TH * (512 * r + 256 + 128 + 4 + isz + 256) + U * st * (int(with_h0) + 1) +
                NCH * ch * int(states))
    if name == "scan_state":
        return TH * (256 * r + 256 + 128 + 4 + isz) + NCH * ch + U * st * int(with_h0)
    if name == "scan_aug":
        return frac * TH * (256 * r + 256 + 128 + 4 + isz) + U * (cp - 1) * 2 * st
    if name == "dh_scan_out":
        return TH * (512 * r + 256 + 128 + 4 + isz) + NCH * ch + U * st * (int(with_dht) + int(with_h0))
    if name == "dh_scan_aug":
        return frac * TH * (512 * r + 256 + 128 + 4 + isz) + U * (cp - 1) * 2 * st
    if name == "bwd_scans":  # the state scan (unless given) and the state-gradient scan
        return (kernel_bytes("scan_state", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht)
                * int(not states) +
                kernel_bytes("dh_scan_out", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht))
    if name == "bwd_scan_aug":
        return (kernel_bytes("scan_aug", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht) +
                kernel_bytes("dh_scan_aug", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht))
    if name in ("cp_combine_fwd", "cp_combine_bwd"):
        return U * max(cp - 1, 0) * 3 * st
    if name == "grad":
        dqk = 512 * r if Hq == Hv else 1024
        return TH * (512 * r + 256 + 256 + 128 + 4 + isz + dqk + 256 + isz + gsz) + NCH * 2 * ch
    if name == "bwd_dyn":  # the state-gradient scan and every chunk's gradients, one launch
        return (kernel_bytes("dh_scan_out", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht) +
                kernel_bytes("grad", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht))
    if name == "chunk_offsets":
        return 8 * (N + 1)
    return None


def code_text(src):
    """C/C++ source without its comments and blank space, so that an edit of
    comments alone leaves the kernels' digest unchanged."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(" ".join(ln.split()) for ln in src.splitlines() if ln.strip())


def source_digest(csrc=None):
    """Digest of the kernel sources' code, which the committed counter
    summaries carry: their figures apply only while it matches."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "gated_delta_rule_66_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), encoding="utf-8") as f:
            h.update(fn.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel, workload, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy calibration), or
    None when absent or taken from different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest() or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return (k["fetch_kib"] * t["fetch_factor"] + k["write_kib"] * t["write_factor"]) * 1024.0


def measured_mfma(kernel, workload):
    """The kernel's MFMA-busy fraction from the committed rocprofv3 counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over the active cycles of all SIMDs),
    or None when absent or taken from different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest() or t.get("workload") != workload:
        return None
    k = t.get("mfma", {}).get(kernel)
    return None if not k else k.get("busy_frac")


def cpu_baseline(d, prob, nthreads_cap=16, max_units=32, qk_norm=False, gate=False):
    """The fp64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    import oracle
    B, T, Hq, Hv = prob
    G = Hv // Hq
    cu = d["cu_seqlens"]
    nseq = 1 if cu is None else int(cu.numel()) - 1
    # sample: value heads 0 .. nh-1 (whole q/k groups) of the first sequence,
    # or of every sequence of a packed batch
    nh = max(G, min(Hv, max_units // nseq))
    nh -= nh % G
    nq = nh // G

    def f(t, heads, dim):
        if t is None:
            return None
        x = t if cu is not None else t[0:1]  # packed: every sequence; dense: sequence 0
        sl = [slice(None)] * x.dim()
        sl[dim] = slice(0, heads)
        return x[tuple(sl)].float().numpy().astype(np.float64)

    q, k = f(d["q"], nq, 2), f(d["k"], nq, 2)
    v, g, beta, do = (f(d[n], nh, 2) for n in ("v", "g", "beta", "do"))
    h0, dht = f(d["h0"], nh, 1), f(d["dht"], nh, 1)
    cun = None if cu is None else cu.numpy().astype(np.int64)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    units = nh * nseq
    threads = max(1, min(nthreads_cap, avail, units))
    t0 = time.perf_counter()
    gkw = {}
    if gate:
        gkw["gate"] = (d["A_log"][:nh].double().numpy(), d["dt_bias"][:nh].double().numpy())
    oracle.fwd(q, k, v, g, beta, d["scale"], initial_state=h0, cu_seqlens=cun, nthreads=threads,
               use_qk_l2norm=qk_norm, **gkw)
    oracle.bwd(q, k, v, g, beta, d["scale"], do, initial_state=h0, dht=dht, cu_seqlens=cun,
               nthreads=threads, use_qk_l2norm=qk_norm, **gkw)
    dt = time.perf_counter() - t0
    total_units = (B if cu is None else nseq) * Hv
    frac = units / float(total_units)
    tokens = B * T
    where = "sequence 0" if cu is None else "all %d packed sequences" % nseq
    return {"value": round(tokens * frac / dt / 1e6, 6), "unit": "Mtokens/s", "cores": threads,
            "nproc": os.cpu_count(), "affinity": avail, "kind": "oracle",
            "sample": "fp64 token recurrence fwd+bwd on %s, value heads 0..%d (%d of %d "
                      "(sequence, head) units); %.1f s wall on %d threads (about %.0f "
                      "thread-seconds); value scaled to the whole workload"
                      % (where, nh - 1, units, total_units, dt, threads, dt * threads)}


class Case:
    """One workload on the device: seeded inputs resident in HBM and closures
    for its forward, its backward (on the forward's g_cum and A) and a step."""

    def __init__(self, gdr, torch, gdr_synth, B, T, Hq, Hv, dt, g_shift, varlen, h0, dht, svf,
                 cp=0, vt=0, qk_norm=False, gate=False, name="case", recompute=False,
                 fwd_only=False):
        prob = gdr_synth.Problem(name, B=B, T=T, Hq=Hq, Hv=Hv, dtype=dt, init_state=h0,
                                 backward=True, dht=dht, g_shift=g_shift, qk_l2norm=qk_norm,
                                 gate=gate)
        d = gdr_synth.make(prob, lengths_from=varlen)
        self.prob, self.host = prob, d
        self.B, self.T, self.Hq, self.Hv = prob.B, prob.T, Hq, Hv
        self.N = len(prob.lens) if prob.lens else prob.B
        self.tokens = prob.B * prob.T
        self.nchunks = (sum((L + 63) // 64 for L in prob.lens) if prob.lens
                        else prob.B * ((prob.T + 63) // 64))
        self.isz = 2
        self.h0, self.dht = h0, dht
        dev = torch.device("cuda", 0)
        dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        if svf:
            for key in ("h0", "dht"):
                if dd[key] is not None:
                    dd[key] = dd[key].transpose(-1, -2).contiguous()
        self.dd = dd
        cu_cpu = d["cu_seqlens"]
        gkw = dict(use_gate_in_kernel=True, A_log=dd["A_log"], dt_bias=dd["dt_bias"]) if gate else {}
        # a forward run for a backward keeps what that backward takes; an
        # inference forward keeps nothing
        keep = not (recompute or fwd_only)
        self.plans = {d_: gdr.plan_info(dd["q"], dd["v"], cu_seqlens=dd["cu_seqlens"],
                                        cu_seqlens_cpu=cu_cpu, cp_segments=cp, wave_tiles=vt,
                                        backward=(d_ == "bwd"), h_packed=keep)
                      for d_ in ("fwd", "bwd")}
        # the backward's pipeline on the states path: (slices, chunk bounds)
        self.pipe = (gdr.pipeline_info(dd["q"], dd["v"], cu_seqlens=dd["cu_seqlens"],
                                       cu_seqlens_cpu=cu_cpu, cp_segments=cp, wave_tiles=vt)
                     if keep else (0, []))

        # the autograd op's calls: the forward keeps its chunk-start states
        # (packed) and the segment transitions of a split plan, and the
        # backward takes them instead of recomputing
        fkw = dict(scale=dd["scale"], initial_state=dd["h0"], output_final_state=True,
                   cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=cu_cpu, state_v_first=svf,
                   cp_segments=cp, wave_tiles=vt, use_qk_l2norm_in_kernel=qk_norm, **gkw)

        def fwd():
            if not keep:
                g_cum, A, o, _, ht = gdr.chunk_gated_delta_rule_fwd(
                    dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **fkw)
                return g_cum, A, o, None, None, ht
            return gdr.chunk_gated_delta_rule_fwd_states(
                dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], **fkw)

        def bwd(g_cum, A, h, trans):
            return gdr.chunk_gated_delta_rule_bwd(
                dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A, dd["do"], dht=dd["dht"],
                scale=dd["scale"], initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
                state_v_first=svf, dg_dtype=dd["g"].dtype, cu_seqlens_cpu=cu_cpu,
                cp_segments=cp, wave_tiles=vt, use_qk_l2norm_in_kernel=qk_norm, h=h,
                trans=trans, **(dict(gkw, g_input=dd["g"]) if gate else {}))

        def step():
            g_cum, A, o, h, trans, ht = fwd()
            return bwd(g_cum, A, h, trans)

        self.fwd, self.bwd, self.step = fwd, bwd, step

    def alg(self, direction):
        """(flop, bytes) of the pass's algorithmic work."""
        flop = self.tokens * self.Hv * (FWD_FLOP if direction == "fwd" else BWD_FLOP)
        n_states = (int(self.h0) + 1) if direction == "fwd" else (2 * int(self.h0) + int(self.dht))
        nbytes = pass_bytes(direction, self.tokens, self.Hq, self.Hv, self.N, n_states, self.isz)
        return flop, nbytes


class Timer:
    """Back-to-back and cold timing with events on torch's current stream,
    which is the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.flush = None

    def mean_ms(self, fn, n):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def cold_ms(self, fn, n):
        """Median of n runs, each after a 512 MiB buffer write (outside the
        events) that evicts the inputs from the Infinity Cache."""
        torch = self.torch
        if self.flush is None:
            self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        out = []
        for i in range(n):
            self.flush.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        out.sort()
        return out[len(out) // 2]


def kernel_times(gdr, torch, fn, n):
    """{name: (total_ms, launches)} of the library's kernels over n runs of fn,
    from HIP events the library records around each launch."""
    torch.cuda.synchronize()
    with gdr.KernelTimer() as timer:
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return timer.read()


def kernel_direction(name):
    return "bwd" if name in BWD_KERNELS else "fwd"


def measure_case(gdr, torch, timer, case, direction, steps, warmup, n_cold, warm_ms=50.0):
    """Times one workload; returns the configs-block record.  The warm-up
    runs at least `warmup` times and at least `warm_ms` of wall time: after
    the host has prepared a workload the GPU has idled, and its first
    milliseconds of work run slower."""
    fwd_flop, fwd_bytes = case.alg("fwd")
    bwd_flop, bwd_bytes = case.alg("bwd")
    fn = case.step if direction == "fwd+bwd" else case.fwd
    t0, n = time.perf_counter(), 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    rec = {"direction": direction, "tokens": case.tokens,
           "plan": {k: {"cp_segments": v[0], "wave_tiles": v[1]} for k, v in case.plans.items()}}
    fwd_ms = timer.mean_ms(case.fwd, steps)
    fwd_cold = timer.cold_ms(case.fwd, n_cold)
    rec["fwd_ms"], rec["fwd_cold_ms"] = round(fwd_ms, 4), round(fwd_cold, 4)
    rec["fwd_frac"] = fractions(fwd_ms * 1e-3, fwd_flop, fwd_bytes)
    if direction == "fwd":
        ms, cold = fwd_ms, fwd_cold
        flop, nbytes = fwd_flop, fwd_bytes
        kt = kernel_times(gdr, torch, case.fwd, steps)
    else:
        g_cum, A, _, h, trans, _ = case.fwd()
        bwd_ms = timer.mean_ms(lambda: case.bwd(g_cum, A, h, trans), steps)
        bwd_cold = timer.cold_ms(lambda: case.bwd(g_cum, A, h, trans), n_cold)
        rec["bwd_ms"], rec["bwd_cold_ms"] = round(bwd_ms, 4), round(bwd_cold, 4)
        rec["bwd_frac"] = fractions(bwd_ms * 1e-3, bwd_flop, bwd_bytes)
        ms = timer.mean_ms(case.step, steps)
        cold = timer.cold_ms(case.step, n_cold)
        flop, nbytes = fwd_flop + bwd_flop, fwd_bytes + bwd_bytes
        kt = kernel_times(gdr, torch, case.step, steps)
    rec["ms"], rec["cold_ms"] = round(ms, 4), round(cold, 4)
    rec["Mtokens_s"] = round(case.tokens / (ms * 1e-3) / 1e6, 4)
    rec["cold_Mtokens_s"] = round(case.tokens / (cold * 1e-3) / 1e6, 4)
    rec["frac"] = fractions(ms * 1e-3, flop, nbytes)
    rec["algorithmic_bytes"] = int(nbytes)
    rec["kernels_us"] = {k: round(t / c * 1e3, 2) for k, (t, c) in kt.items()}
    return rec, kt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the first few steps of a process run slower")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS) + sorted(DECODE_WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the selected workload, not the configs block")
    ap.add_argument("--cold", type=int, default=5, help="cold runs per measurement (median)")
    ap.add_argument("--cp", type=int, default=0,
                    help="context-parallel segments per sequence (0 = the library's plan)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (counter calibration)")
    ap.add_argument("--vt", type=int, default=0,
                    help="16-column state tiles per wave in the scans (0 = the library's plan)")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="raw q / k rows, normalised inside the kernels (use_qk_l2norm_in_kernel)")
    ap.add_argument("--gate", action="store_true",
                    help="g is the raw gate input, activated inside the kernels "
                         "(use_gate_in_kernel: -exp(A_log) softplus(g + dt_bias))")
    ap.add_argument("--recompute-states", action="store_true",
                    help="the backward recomputes the chunk-start states instead of taking the "
                         "forward's (autograd's recompute_states=True)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path runs on a single MI355X and the library "
              "has no multi-GPU mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gdr_synth
    import gated_delta_rule_66_amd as gdr

    if args.workload in DECODE_WORKLOADS:
        return bench_decode(args)
    B, T, Hq, Hv, dt, g_shift, varlen, w_h0, w_dht = WORKLOADS[args.workload]
    qkn = args.qk_l2norm
    case = Case(gdr, torch, gdr_synth, B, T, Hq, Hv, dt, g_shift, varlen, w_h0, w_dht, False,
                cp=args.cp, vt=args.vt, qk_norm=qkn, gate=args.gate, name=args.workload,
                recompute=args.recompute_states)
    B, T = case.B, case.T
    dev = torch.device("cuda", 0)
    timer = Timer(torch)

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        flush = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(2.0)  # 1 GiB
        torch.cuda.synchronize()
        del flush
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        case.step()
    # the headline: exactly --steps back-to-back steps between two events
    ms = timer.mean_ms(case.step, args.steps)

    # the forward and the backward alone, cold runs, then per-kernel times
    g_cum, A, o, h, trans, ht = case.fwd()
    n_sub = max(3, args.steps // 2)
    fwd_ms = timer.mean_ms(case.fwd, n_sub)
    bwd_ms = timer.mean_ms(lambda: case.bwd(g_cum, A, h, trans), n_sub)
    cold_ms = timer.cold_ms(case.step, args.cold)
    fwd_cold = timer.cold_ms(case.fwd, args.cold)
    bwd_cold = timer.cold_ms(lambda: case.bwd(g_cum, A, h, trans), args.cold)
    kernels = kernel_times(gdr, torch, case.step, args.steps)

    tokens = case.tokens
    value = tokens / (ms * 1e-3) / 1e6
    fwd_flop, fwd_bytes = case.alg("fwd")
    bwd_flop, bwd_bytes = case.alg("bwd")
    tflops = (fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12
    frac = {"step": fractions(ms * 1e-3, fwd_flop + bwd_flop, fwd_bytes + bwd_bytes),
            "step_cold": fractions(cold_ms * 1e-3, fwd_flop + bwd_flop, fwd_bytes + bwd_bytes),
            "fwd": fractions(fwd_ms * 1e-3, fwd_flop, fwd_bytes),
            "bwd": fractions(bwd_ms * 1e-3, bwd_flop, bwd_bytes)}

    # dominant kernel and its roofline: the minimum bytes of the pass it
    # belongs to over its mean launch time (the fraction of peak that pass
    # would reach in this kernel's time alone)
    per_kernel = {}
    tot_all = max(sum(v[0] for v in kernels.values()), 1e-9)
    for name, (tot, cnt) in kernels.items():
        per_kernel[name] = {"avg_us": round(tot / cnt * 1e3, 2), "launches": cnt,
                            "share": round(tot / tot_all, 4)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    avg_s = kernels[dom][0] / kernels[dom][1] * 1e-3
    ddir = kernel_direction(dom)
    alg = fwd_bytes if ddir == "fwd" else bwd_bytes
    alg_desc = ("minimum bytes of the %s pass (%s B per (token, value head) + fp32 states)"
                % (ddir, round(alg_bytes_per_unit(ddir, Hq / Hv), 1)))
    dom_cp = case.plans[ddir][0]
    wl_key = args.workload + ("+qk_l2norm" if qkn else "") + ("+gate" if args.gate else "")
    operand = kernel_bytes(dom, B, T, Hq, Hv, case.nchunks, case.N, dom_cp, qk_norm=qkn,
                           states=not args.recompute_states)
    if dom == "grad" and case.pipe[0] > 0:
        # pipelined: the gradient launch covers chunks bounds[0] .. bounds[1]
        # of every sequence (the other chunks' gradients run beside the scan)
        covered = case.N * min(64 * case.pipe[1][1], T)
        alg = pass_bytes("bwd", covered, Hq, Hv, case.N, 0)
        alg_desc = ("minimum bytes of the backward for the tokens the launch covers (%d of %d; "
                    "%s B per (token, value head))"
                    % (covered, case.tokens, round(alg_bytes_per_unit("bwd", Hq / Hv), 1)))
        operand = None if operand is None else operand * covered / case.tokens
    traffic = measured_traffic(dom, wl_key, operand)
    achieved = alg / avg_s / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "traffic_over_alg": None if traffic is None else round(traffic / alg, 3),
                "algorithmic_bytes_per_launch": int(alg),
                "algorithmic_bytes": alg_desc,
                "avg_launch_us": round(avg_s * 1e6, 2),
                "operand_bytes_per_launch": None if operand is None else int(operand),
                "operand_frac": None if operand is None else
                round(operand / avg_s / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_busy_frac": measured_mfma(dom, wl_key)}
    # counter traffic of whole passes over their minimum, where every kernel
    # of the pass has a committed counter figure
    for d_, kset, nb in (("fwd", FWD_KERNELS, fwd_bytes), ("bwd", BWD_KERNELS, bwd_bytes)):
        # per step: each kernel's bytes per launch times its launches per step
        tr = [None if measured_traffic(k_, wl_key, 0) is None else
              measured_traffic(k_, wl_key, 0) * kernels[k_][1] / args.steps
              for k_ in kernels if k_ in kset]
        roofline["%s_traffic_over_alg" % d_] = (round(sum(tr) / nb, 3)
                                                 if tr and all(x is not None for x in tr) else None)

    out = {
        "metric": "GDN chunk fwd+bwd Mtokens/s at H=32,K=V=128 bf16 (and % of bf16 MFMA peak)",
        "value": round(value, 4),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded; %s, %s, beta=sigmoid)" % (
            "raw N(0,1) q,k normalised in-kernel" if qkn else "q,k L2-normalised",
            "g = raw gate input N(0,1), activated in-kernel" if args.gate else "g=logsigmoid"),
        "config": {"workload": args.workload, "B": B, "T": T, "Hq": Hq, "Hv": Hv, "K": 128,
                   "V": 128, "chunk": 64, "tokens": tokens, "initial_state": w_h0, "dht": w_dht,
                   "cp_segments": {k_: v_[0] for k_, v_ in case.plans.items()},
                   "wave_tiles": {k_: v_[1] for k_, v_ in case.plans.items()},
                   "qk_l2norm_in_kernel": qkn, "gate_in_kernel": bool(args.gate),
                   "backward_states": "recomputed" if args.recompute_states else
                   "kept by the forward (autograd default)",
                   "parallelism": "single GPU"},
        "cold_ms_per_step": round(cold_ms, 4),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "fwd_cold_ms": round(fwd_cold, 4),
        "bwd_cold_ms": round(bwd_cold, 4),
        "tflops": round(tflops, 3),
        "pct_bf16_mfma_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 3),
        "fractions": frac,
        "algorithmic_bytes": {"fwd": int(fwd_bytes), "bwd": int(bwd_bytes)},
        "kernels": per_kernel,
        "roofline": roofline,
        "configs": None,
        "cpu_baseline": None,
    }
    del g_cum, A, o, h, trans, ht
    host = case.host
    if not args.no_configs and args.workload == DEFAULT and not qkn and not args.gate:
        del case
        torch.cuda.empty_cache()
        cfgs = {}
        for name, (direc, cB, cT, cHq, cHv, cdt, gsh, vl, ch0, cdht, svf) in CONFIGS.items():
            c = Case(gdr, torch, gdr_synth, cB, cT, cHq, cHv, cdt, gsh, vl, ch0, cdht, svf,
                     name=name, fwd_only=(direc == "fwd"))
            cfgs[name], _ = measure_case(gdr, torch, timer, c, direc, steps=10, warmup=3,
                                         n_cold=args.cold)
            cfgs[name].update({"B": c.B, "T": c.T, "Hq": cHq, "Hv": cHv, "dtype": cdt,
                               "state_v_first": svf, "initial_state": ch0, "dht": cdht})
            del c
            torch.cuda.empty_cache()
        out["configs"] = cfgs
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(host, (B, T, Hq, Hv), qk_norm=qkn, gate=args.gate)
    print(json.dumps(out), flush=True)


def bench_decode(args):
    """Decode steps of the token-by-token forward: every sequence advances by
    one token per step, its fp32 state updated in place.  The kernel moves
    each state in and out once (2 x 64 KiB per (sequence, head)) plus the
    token's q, k, v, g, beta and o, so it is HBM-bound."""
    import torch
    import gdr_synth
    import gated_delta_rule_66_amd as gdr

    B, H, T, dt = DECODE_WORKLOADS[args.workload]
    prob = gdr_synth.Problem(args.workload, B=B, T=T, Hq=H, Hv=H, dtype=dt, init_state=True,
                             qk_l2norm=args.qk_l2norm)
    d = gdr_synth.make(prob)
    dev = torch.device("cuda", 0)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    state = dd["h0"].clone()

    def step():
        return gdr.fused_recurrent_gated_delta_rule(
            dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], scale=dd["scale"],
            initial_state=state, inplace_final_state=True,
            use_qk_l2norm_in_kernel=args.qk_l2norm)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    ms = timer.mean_ms(step, args.steps)
    kernels = kernel_times(gdr, torch, step, args.steps)
    tot, cnt = kernels["recurrent"]
    avg_s = tot / cnt * 1e-3
    isz = 2
    units = B * H
    nbytes = units * (2 * 128 * 128 * 4 + T * (3 * 128 * isz + 2 * isz + 128 * isz))
    achieved = nbytes / avg_s / 1e9
    out = {
        "metric": "GDN decode (token-by-token forward) Mtokens/s at H=32,K=V=128 bf16",
        "value": round(B * T / (ms * 1e-3) / 1e6, 4),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded; fp32 states updated in place)",
        "config": {"workload": args.workload, "B": B, "T_per_step": T, "Hq": H, "Hv": H,
                   "K": 128, "V": 128, "qk_l2norm_in_kernel": args.qk_l2norm,
                   "parallelism": "single GPU"},
        "kernels": {"recurrent": {"avg_us": round(avg_s * 1e6, 2), "launches": cnt}},
        "roofline": {"bound": "hbm", "kernel": "recurrent", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_us": round(avg_s * 1e6, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
