"""bench.py's host-side reporting logic (no GPU): the one-GPU contract, the
counter look-ups guarded by the kernel-source hash, the algorithmic bytes of
a launch, and the CPU baseline record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import gdr_synth  # noqa: E402

WORKLOAD = "fwd_bwd_B2_T4096_H32_bf16"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _write_summary(tmp_path, digest, workload=WORKLOAD):
    prof = tmp_path / "profiles"
    prof.mkdir()
    summary = {
        "workload": workload, "source_sha256": digest, "fetch_factor": 2.0, "write_factor": 1.0,
        "kernels": {"grad": {"fetch_kib": 100.0, "write_kib": 50.0}},
        "mfma": {"grad": {"busy_frac": 0.125}},
    }
    (prof / "traffic.json").write_text(json.dumps(summary))


def test_counter_lookups_follow_the_source_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    _write_summary(tmp_path, "abc")
    # FETCH_SIZE and WRITE_SIZE are KiB per dispatch, each scaled by its factor
    assert bench.measured_traffic("grad", WORKLOAD, 0) == (100.0 * 2.0 + 50.0) * 1024.0
    assert bench.measured_mfma("grad", WORKLOAD) == 0.125
    # another workload, another kernel, or other kernel sources: no figure
    assert bench.measured_traffic("grad", "fwd_bwd_varlen8_H32_bf16", 0) is None
    assert bench.measured_traffic("scan_out", WORKLOAD, 0) is None
    assert bench.measured_mfma("scan_out", WORKLOAD) is None
    monkeypatch.setattr(bench, "source_digest", lambda: "changed")
    assert bench.measured_traffic("grad", WORKLOAD, 0) is None
    assert bench.measured_mfma("grad", WORKLOAD) is None


def test_counter_lookups_without_a_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("grad", WORKLOAD, 0) is None
    assert bench.measured_mfma("grad", WORKLOAD) is None


def test_algorithmic_bytes_of_fwd_prep_by_hand():
    # B=1, T=128 (2 chunks), Hq=Hv=1, bf16 g: per (token, value head) the k
    # row 256 B, g 2 B, beta 2 B, g_cum 4 B and the A row 128 B
    assert bench.kernel_bytes("fwd_prep", 1, 128, 1, 1, 2, 1, 1) == 128 * (256 + 2 + 2 + 4 + 128)
    # grouped heads halve the k bytes per value head
    assert bench.kernel_bytes("fwd_prep", 1, 128, 1, 2, 2, 1, 1) == 2 * 128 * (128 + 2 + 2 + 4 + 128)


def test_fused_scan_bytes_are_the_sum_of_both_scans():
    args = (2, 4096, 32, 32, 128, 2, 1)
    kb = bench.kernel_bytes
    assert kb("bwd_scans", *args, states=False) == (kb("scan_state", *args) +
                                                    kb("dh_scan_out", *args))
    # given the forward's chunk states the launch runs the state-gradient scan
    # alone, and the forward scan writes those states (one bf16 128 x 128
    # tile per chunk and head)
    assert kb("bwd_scans", *args) == kb("dh_scan_out", *args)
    assert kb("scan_out", *args) - kb("scan_out", *args, states=False) == 128 * 32 * 128 * 128 * 2


def test_cpu_baseline_record():
    prob = gdr_synth.Problem("tiny", B=1, T=70, Hq=1, Hv=2, init_state=True, backward=True,
                             dht=True)
    d = gdr_synth.make(prob)
    out = bench.cpu_baseline(d, (1, 70, 1, 2), nthreads_cap=2)
    assert out["kind"] == "oracle"
    assert out["unit"] == "Mtokens/s"
    assert out["value"] > 0
    assert 1 <= out["cores"] <= 2
    assert "thread-seconds" in out["sample"]


def test_pass_minimum_bytes_per_token_and_head():
    # 16-bit inputs: 1160 / 904 B forward and 1930 / 1418 B backward per
    # (token, value head) at Hq = Hv and Hq = Hv / 2
    assert bench.alg_bytes_per_unit("fwd", 1.0) == 1160
    assert bench.alg_bytes_per_unit("fwd", 0.5) == 904
    assert bench.alg_bytes_per_unit("bwd", 1.0) == 1930
    assert bench.alg_bytes_per_unit("bwd", 0.5) == 1418
    # an fp32 g adds two bytes on each side (g read forward, dg written backward)
    assert bench.alg_bytes_per_unit("fwd", 1.0, gsz=4) == 1162
    assert bench.alg_bytes_per_unit("bwd", 1.0, gsz=4) == 1932


def test_pass_bytes_add_the_fp32_states():
    # B=2 T=4096 H=32: 262144 (token, head) units and 64 (sequence, head) units
    fwd = bench.pass_bytes("fwd", 8192, 32, 32, 2, n_states=2)
    assert fwd == 262144 * 1160 + 64 * 2 * 65536
    bwd = bench.pass_bytes("bwd", 8192, 32, 32, 2, n_states=3)
    assert bwd == 262144 * 1930 + 64 * 3 * 65536


def test_fractions_take_the_larger_bound():
    # 8 GB in 2 ms is 0.5 of 8 TB/s; 1 TFLOP in 2 ms is 500 TFLOP/s, 0.199 of
    # the bf16 MFMA peak
    f = bench.fractions(2e-3, 1e12, 8e9)
    assert f["hbm"] == 0.5 and f["bound"] == "hbm" and f["roofline"] == 0.5
    assert abs(f["mfma"] - 500.0 / bench.MFMA_BF16_PEAK_TFLOPS) < 1e-4
    g = bench.fractions(2e-3, 4e12, 1e9)
    assert g["bound"] == "mfma" and g["roofline"] == g["mfma"]


def test_every_library_kernel_has_a_direction():
    for k in ("fwd_prep", "scan_out", "scan_aug", "cp_combine_fwd"):
        assert bench.kernel_direction(k) == "fwd"
    for k in ("bwd_scans", "bwd_scan_aug", "cp_combine_bwd", "bwd_pipe", "bwd_dyn", "bwd_flags",
              "grad"):
        assert bench.kernel_direction(k) == "bwd"


def test_source_digest_ignores_comments_only():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */\n}\n"
    b = "int f(int x) {\n\n  return 2 * x;\n}  // edited comment\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
