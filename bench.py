#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule (forward + backward) on one MI355X.

One step = one pass of the whole hot path over one batch: forward (gate cumsum,
WY inverse, state scan with output, intra-GPU context parallelism when the plan
uses it) and backward (state recompute, reverse state-gradient scan, per-chunk
gradients).  The default workload is B=2, T=4096, Hq=Hv=32, K=V=128, bf16 with
an initial state and a final-state gradient (the shape of the FlashQLA API
example), synthetic seeded inputs resident in HBM before timing starts.

Prints one JSON line.  Per-kernel durations come from HIP events the library
records around each of its launches during the timed steps; the dominant
kernel's algorithmic bytes per launch divided by its mean duration gives the
roofline entry.  The CPU baseline times the fp64 oracle on a bounded sample of
the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
FWD_FLOP = 140629               # algorithmic flop per (token, value head), forward
BWD_FLOP = 393216               # backward incl. the state recompute

WORKLOADS = {
    # name: (B, T, Hq, Hv, dtype, g_shift, varlen)
    "fwd_bwd_B2_T4096_H32_bf16": (2, 4096, 32, 32, "bf16", 0.0, None),
    "fwd_bwd_varlen8_H32_bf16": (1, 0, 32, 32, "bf16", 0.0, (8, 128, 4096)),
    "fwd_bwd_B4_T8192_Hq16_Hv32_fp16": (4, 8192, 16, 32, "fp16", 0.0, None),
    "fwd_bwd_B1_T65536_H32_bf16": (1, 65536, 32, 32, "bf16", 2.0, None),
}
DEFAULT = "fwd_bwd_B2_T4096_H32_bf16"
# token-by-token forward: (B sequences, Hv = Hq heads, tokens per step, dtype)
DECODE_WORKLOADS = {"decode_B256_H32_bf16": (256, 32, 1, "bf16")}


def kernel_bytes(name, B, T, Hq, Hv, nchunks, N, cp, isz=2, gsz=2, with_h0=True, with_dht=True,
                 qk_norm=False):
    """Algorithmic HBM bytes of one launch of a library kernel: every operand
    read once and every result written once (the minimum any schedule of that
    kernel must move).  Per (token, value head) terms with r = Hq / Hv:
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
        return TH * (512 * r + 256 + 128 + 4 + isz + 256) + U * st * (int(with_h0) + 1)
    if name == "scan_state":
        return TH * (256 * r + 256 + 128 + 4 + isz) + NCH * ch + U * st * int(with_h0)
    if name == "scan_aug":
        return frac * TH * (256 * r + 256 + 128 + 4 + isz) + U * (cp - 1) * 2 * st
    if name == "dh_scan_out":
        return TH * (512 * r + 256 + 128 + 4 + isz) + NCH * ch + U * st * (int(with_dht) + int(with_h0))
    if name == "dh_scan_aug":
        return frac * TH * (512 * r + 256 + 128 + 4 + isz) + U * (cp - 1) * 2 * st
    if name == "bwd_scans":  # the state scan and the state-gradient scan in one launch
        return (kernel_bytes("scan_state", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht) +
                kernel_bytes("dh_scan_out", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht))
    if name == "bwd_scan_aug":
        return (kernel_bytes("scan_aug", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht) +
                kernel_bytes("dh_scan_aug", B, T, Hq, Hv, nchunks, N, cp, isz, gsz, with_h0, with_dht))
    if name == "cp_combine":
        return U * max(cp - 1, 0) * 3 * st
    if name == "grad":
        dqk = 512 * r if Hq == Hv else 1024
        return TH * (512 * r + 256 + 256 + 128 + 4 + isz + dqk + 256 + isz + gsz) + NCH * 2 * ch
    if name == "gva_reduce":
        G = Hv // Hq
        # fp32 partials in, dq / dk out; with q / k normalisation the raw rows too
        return B * T * Hq * 128 * (2 * 4 * G + 2 * isz + (2 * isz if qk_norm else 0))
    if name == "chunk_offsets":
        return 8 * (N + 1)
    return None


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_66_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode())
            h.update(f.read())
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
            "kind": "oracle",
            "sample": "fp64 token recurrence fwd+bwd on %s, value heads 0..%d (%d of %d "
                      "(sequence, head) units); %.1f s wall on %d threads (about %.0f "
                      "thread-seconds); value scaled to the whole workload"
                      % (where, nh - 1, units, total_units, dt, threads, dt * threads)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS) + sorted(DECODE_WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
    B, T, Hq, Hv, dt, g_shift, varlen = WORKLOADS[args.workload]
    prob = gdr_synth.Problem(args.workload, B=B, T=T, Hq=Hq, Hv=Hv, dtype=dt, init_state=True,
                             backward=True, dht=True, g_shift=g_shift, qk_l2norm=args.qk_l2norm,
                             gate=args.gate)
    qkn = args.qk_l2norm
    d = gdr_synth.make(prob, lengths_from=varlen)
    B, T = prob.B, prob.T
    dev = torch.device("cuda", 0)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cu_cpu = d["cu_seqlens"]
    gkw = dict(use_gate_in_kernel=True, A_log=dd["A_log"], dt_bias=dd["dt_bias"]) \
        if args.gate else {}
    plans = {d_: gdr.plan_info(dd["q"], dd["v"], cu_seqlens=dd["cu_seqlens"],
                               cu_seqlens_cpu=cu_cpu, cp_segments=args.cp, wave_tiles=args.vt,
                               backward=(d_ == "bwd"))
             for d_ in ("fwd", "bwd")}

    def fwd():
        return gdr.chunk_gated_delta_rule_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"],
                                              scale=dd["scale"], initial_state=dd["h0"],
                                              output_final_state=True,
                                              cu_seqlens=dd["cu_seqlens"], cu_seqlens_cpu=cu_cpu,
                                              cp_segments=args.cp, wave_tiles=args.vt,
                                              use_qk_l2norm_in_kernel=qkn, **gkw)

    def bwd(g_cum, A):
        return gdr.chunk_gated_delta_rule_bwd(dd["q"], dd["k"], dd["v"], g_cum, dd["beta"], A,
                                              dd["do"], dht=dd["dht"], scale=dd["scale"],
                                              initial_state=dd["h0"], cu_seqlens=dd["cu_seqlens"],
                                              dg_dtype=dd["g"].dtype, cu_seqlens_cpu=cu_cpu,
                                              cp_segments=args.cp, wave_tiles=args.vt,
                                              use_qk_l2norm_in_kernel=qkn,
                                              **(dict(gkw, g_input=dd["g"]) if args.gate else {}))

    def step():
        g_cum, A, o, _, ht = fwd()
        return bwd(g_cum, A)

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
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with gdr.KernelTimer() as timer:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        kernels = timer.read()
    ms = e0.elapsed_time(e1) / args.steps

    # forward-only and backward-only step times (separately, after)
    g_cum, A, o, _, ht = fwd()
    torch.cuda.synchronize()
    n_sub = max(3, args.steps // 2)
    e0.record()
    for _ in range(n_sub):
        fwd()
    e1.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / n_sub
    e0.record()
    for _ in range(n_sub):
        bwd(g_cum, A)
    e1.record()
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / n_sub

    tokens = B * T
    value = tokens / (ms * 1e-3) / 1e6
    tflops = tokens * Hv * (FWD_FLOP + BWD_FLOP) / (ms * 1e-3) / 1e12
    N = len(prob.lens) if prob.lens else B
    nchunks = sum((L + 63) // 64 for L in prob.lens) if prob.lens else B * ((T + 63) // 64)

    # dominant kernel and its roofline
    per_kernel = {}
    for name, (tot, cnt) in kernels.items():
        per_kernel[name] = {"avg_us": round(tot / cnt * 1e3, 2), "launches": cnt,
                            "share": round(tot / max(sum(v[0] for v in kernels.values()), 1e-9), 4)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    avg_s = kernels[dom][0] / kernels[dom][1] * 1e-3
    dom_cp = plans["bwd" if dom.startswith(("bwd", "grad", "gva")) else "fwd"][0]
    nbytes = kernel_bytes(dom, B, T, Hq, Hv, nchunks, N, dom_cp, qk_norm=qkn)
    achieved = nbytes / avg_s / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, args.workload + ("+qk_l2norm" if qkn else "")
                                            + ("+gate" if args.gate else ""), nbytes),
                "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_us": round(avg_s * 1e6, 2),
                "mfma_busy_frac": measured_mfma(dom, args.workload + ("+qk_l2norm" if qkn else "")
                                                + ("+gate" if args.gate else ""))}

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
                   "V": 128, "chunk": 64, "tokens": tokens,
                   "cp_segments": {k_: v_[0] for k_, v_ in plans.items()},
                   "wave_tiles": {k_: v_[1] for k_, v_ in plans.items()},
                   "qk_l2norm_in_kernel": qkn, "gate_in_kernel": bool(args.gate),
                   "parallelism": "single GPU"},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "tflops": round(tflops, 3),
        "pct_bf16_mfma_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 3),
        "kernels": per_kernel,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(d, (B, T, Hq, Hv), qk_norm=qkn, gate=args.gate)
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
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with gdr.KernelTimer() as timer:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        kernels = timer.read()
    ms = e0.elapsed_time(e1) / args.steps
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
