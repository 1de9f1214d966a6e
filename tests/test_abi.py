"""The C ABI on the host: exports, argument validation, workspace queries.

Validation finishes before the first HIP call, so every rejection branch runs
on a machine without a GPU (the analogue of the verifier rejection tests in
the FLA backend pull request's test plan)."""
import ctypes
import os
import re

import pytest
import torch

from gated_delta_rule_66_amd import _lib
from gated_delta_rule_66_amd._lib import GDR_BF16, GDR_FP16, GDR_FP32, Problem, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "gdr.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 17
    assert sorted(_lib.EXPORTS) == names
    cdll = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(cdll, n), n


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert lib.gdr_status_string(code).decode() == name


FAKE_DEV = 0x1000  # never dereferenced: validation happens on the host copy


def good(**kw):
    base = dict(B=2, T=200, Hq=2, Hv=4, K=128, V=128, N=2, cu_seqlens_dev=None,
                cu_seqlens_host=None, in_dtype=GDR_BF16, g_dtype=GDR_BF16, scale=0.088,
                state_v_first=0, cp_segments=0, wave_tiles=0, use_qk_l2norm=0,
                beta_sigmoid=0, neg_eigval=0)
    base.update(kw)
    return Problem(**base)


def check(p):
    reason = ctypes.create_string_buffer(256)
    st = lib.gdr_check_supported(ctypes.byref(p), reason, 256)
    return _lib.STATUS[st], reason.value.decode()


def test_acceptance_path():
    assert check(good()) == ("GDR_OK", "")
    assert check(good(in_dtype=GDR_FP16, g_dtype=GDR_FP32))[0] == "GDR_OK"
    assert check(good(use_qk_l2norm=1))[0] == "GDR_OK"
    assert check(good(use_gate=1, gate_A_log=FAKE_DEV))[0] == "GDR_OK"
    assert check(good(use_gate=1, gate_A_log=FAKE_DEV, gate_dt_bias=FAKE_DEV))[0] == "GDR_OK"


HOST_CU = (ctypes.c_int32 * 4)(0, 70, 70, 200)
HOST_CU_BAD0 = (ctypes.c_int32 * 4)(1, 70, 70, 200)
HOST_CU_DEC = (ctypes.c_int32 * 4)(0, 70, 60, 200)
HOST_CU_END = (ctypes.c_int32 * 4)(0, 70, 70, 199)


def varlen(cu, **kw):
    return good(B=1, N=3, cu_seqlens_dev=FAKE_DEV,
                cu_seqlens_host=ctypes.cast(cu, ctypes.c_void_p).value, **kw)


REJECT = [
    ("K=64", good(K=64), "GDR_ERR_HEAD_DIM", "requires K=128, got 64"),
    ("V=64", good(V=64), "GDR_ERR_HEAD_DIM", "requires V=128, got 64"),
    ("fp32 inputs", good(in_dtype=GDR_FP32, g_dtype=GDR_FP32), "GDR_ERR_DTYPE", "bf16 or fp16"),
    ("g dtype", good(g_dtype=GDR_FP16), "GDR_ERR_DTYPE", "g must"),
    ("Hq>Hv", good(Hq=8, Hv=4), "GDR_ERR_HEADS", "multiple"),
    ("Hv%Hq", good(Hq=3, Hv=4), "GDR_ERR_HEADS", "multiple"),
    ("T=0", good(T=0), "GDR_ERR_SHAPE", "positive"),
    ("N!=B", good(N=3), "GDR_ERR_SHAPE", "N == B"),
    ("scale", good(scale=float("inf")), "GDR_ERR_ARG", "scale"),
    ("svf", good(state_v_first=2), "GDR_ERR_ARG", "state_v_first"),
    ("cp", good(cp_segments=-1), "GDR_ERR_ARG", "cp_segments"),
    ("wave_tiles", good(wave_tiles=3), "GDR_ERR_ARG", "wave_tiles"),
    ("qk_l2norm", good(use_qk_l2norm=2), "GDR_ERR_ARG", "use_qk_l2norm"),
    ("beta_sigmoid", good(beta_sigmoid=2), "GDR_ERR_ARG", "beta_sigmoid"),
    ("neg_eigval", good(neg_eigval=-1), "GDR_ERR_ARG", "neg_eigval"),
    ("use_gate", good(use_gate=2, gate_A_log=FAKE_DEV), "GDR_ERR_ARG", "use_gate"),
    ("gate without A_log", good(use_gate=1, gate_dt_bias=FAKE_DEV), "GDR_ERR_NULL", "gate_A_log"),
    ("gate params, gate off", good(gate_dt_bias=FAKE_DEV), "GDR_ERR_ARG", "use_gate is 0"),
]


@pytest.mark.parametrize("name,p,status,msg", REJECT, ids=[r[0] for r in REJECT])
def test_rejections(name, p, status, msg):
    st, reason = check(p)
    assert st == status
    assert msg in reason
    assert msg in lib.gdr_last_error().decode()


def test_varlen_rejections():
    assert check(varlen(HOST_CU, T=200))[0] == "GDR_OK"
    p = varlen(HOST_CU, T=200)
    p.B = 2
    assert check(p)[0] == "GDR_ERR_VARLEN"
    assert check(varlen(HOST_CU_BAD0, T=200))[0] == "GDR_ERR_VARLEN"
    assert check(varlen(HOST_CU_DEC, T=200))[0] == "GDR_ERR_VARLEN"
    assert check(varlen(HOST_CU_END, T=200))[0] == "GDR_ERR_VARLEN"
    p = varlen(HOST_CU, T=200)
    p.cu_seqlens_host = None
    assert check(p)[0] == "GDR_ERR_VARLEN"
    assert lib.gdr_check_supported(None, None, 0) == 1  # GDR_ERR_NULL


def test_workspace_queries():
    p = good()
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(p)) == 0
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(p)) > 0
    pv = varlen(HOST_CU, T=200)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(pv)) > 0
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(good(K=64))) == 0
    long = good(B=1, N=1, T=65536, Hq=32, Hv=32)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(long)) > 0  # context-parallel buffers
    # the gate adds the per-(chunk, head) parameter-gradient shares: 2 floats each
    pg = good(use_gate=1, gate_A_log=FAKE_DEV)
    extra = lib.gdr_chunk_bwd_workspace_size(ctypes.byref(pg)) - \
        lib.gdr_chunk_bwd_workspace_size(ctypes.byref(p))
    assert 2 * 4 * 4 * 8 <= extra < 2 * 4 * 4 * 8 + 256   # B=2 x 4 chunks, Hv=4


def plan(p, backward):
    cp = ctypes.c_int32()
    vt = ctypes.c_int32()
    assert lib.gdr_plan_info(ctypes.byref(p), backward, ctypes.byref(cp), ctypes.byref(vt)) == 0
    return cp.value, vt.value


def test_plan_depends_only_on_shapes():
    for bwd in (0, 1):
        plans = [plan(good(B=1, N=1, T=65536, Hq=32, Hv=32, state_v_first=svf), bwd)
                 for svf in (0, 1)]
        assert plans[0] == plans[1]
        assert plans[0][1] in (1, 2)
    assert plan(good(B=1, N=1, T=65536, Hq=32, Hv=32), 0)[0] > 1  # one long sequence split along T
    for bwd in (0, 1):
        assert plan(good(B=1, N=1, T=65536, Hq=32, Hv=32, cp_segments=1), bwd)[0] == 1
        assert plan(good(B=1, N=1, T=65536, Hq=32, Hv=32, cp_segments=4, wave_tiles=2), bwd) == (4, 2)
    # short sequences are never split
    assert plan(good(B=2, N=2, T=256, Hq=32, Hv=32), 0)[0] == 1


def test_states_path_plans_both_directions_together():
    # a forward that keeps packed states and the backward that takes them
    # split sequences the same way, so that the backward can apply the
    # forward's segment transitions
    shapes = [dict(B=1, N=1, T=65536, Hq=32, Hv=32), dict(B=1, N=1, T=16384, Hq=16, Hv=32),
              dict(B=4, N=4, T=8192, Hq=16, Hv=32), dict(B=2, N=2, T=4096, Hq=32, Hv=32),
              dict(B=1, N=1, T=32768, Hq=4, Hv=8)]
    for kw in shapes:
        f = plan(good(h_packed=1, **kw), 0)
        b = plan(good(h_packed=1, **kw), 1)
        assert f[0] == b[0], (kw, f, b)
    assert plan(good(h_packed=1, B=1, N=1, T=65536, Hq=32, Hv=32), 0)[0] > 1
    for cp in (2, 3, 5):
        kw = dict(B=1, N=1, T=4096, Hq=2, Hv=4, cp_segments=cp)
        assert plan(good(h_packed=1, **kw), 0)[0] == plan(good(h_packed=1, **kw), 1)[0] == cp


def test_backward_pipeline_plan():
    n = ctypes.c_int32()
    b = (ctypes.c_int32 * 9)()

    def info(p):
        assert lib.gdr_bwd_pipeline_info(ctypes.byref(p), ctypes.byref(n), b, 9) == 0
        return n.value, (list(b[:n.value + 1]) if n.value else [])
    # B=2 T=4096 H=32: one launch scheduled by data (the scan and every
    # chunk's gradient workgroups)
    assert info(good(B=2, N=2, T=4096, Hq=32, Hv=32)) == (1, [0, 64])
    # with q / k normalised in the kernel, two slices; the last launch's
    # gradients cover 48 of the 64 chunks, 3072 workgroups, twelve whole
    # rounds of the 256 CUs
    assert info(good(B=2, N=2, T=4096, Hq=32, Hv=32, use_qk_l2norm=1)) == (2, [0, 48, 64])
    # grouped heads and up to 128 units (the scan on at most half the CUs)
    # keep the data-scheduled launch
    assert info(good(B=2, N=2, T=4096, Hq=16, Hv=32)) == (1, [0, 64])
    assert info(good(B=4, N=4, T=8192, Hq=16, Hv=32)) == (1, [0, 128])
    assert info(good(B=4, N=4, T=4096, Hq=32, Hv=32)) == (1, [0, 64])
    # the slices keep two 64-column scan workgroups per unit: no grouped
    # heads, at most 64 units
    assert info(good(B=2, N=2, T=4096, Hq=16, Hv=32, use_qk_l2norm=1))[0] == 0
    assert info(good(B=4, N=4, T=4096, Hq=32, Hv=32, use_qk_l2norm=1))[0] == 0
    # packed sequences whose longest has 16+ chunks: the data-scheduled
    # launch (bounds up to the longest sequence's chunks), not with grouped
    # heads
    long_cu = (ctypes.c_int32 * 4)(0, 70, 1100, 3100)
    assert info(varlen(long_cu, T=3100, Hq=8, Hv=8)) == (1, [0, 32])
    assert info(varlen(long_cu, T=3100, Hq=4, Hv=8))[0] == 0
    assert info(varlen(long_cu, T=3100, Hq=8, Hv=8, use_qk_l2norm=1))[0] == 0
    # one pass: short packed sequences, a scan that fills the chip, short
    # sequences, a split along T
    assert info(varlen(HOST_CU, T=200))[0] == 0
    assert info(good(B=8, N=8, T=4096, Hq=32, Hv=32))[0] == 0
    assert info(good(B=2, N=2, T=512, Hq=32, Hv=32))[0] == 0
    assert info(good(B=1, N=1, T=65536, Hq=32, Hv=32))[0] == 0
    # fewer units leave more CUs idle beside the scan, which then hide the
    # gradients of a longer first slice: the slice walked first grows
    assert info(good(B=1, N=1, T=1024, Hq=8, Hv=8)) == (1, [0, 16])
    s, bnd = info(good(B=1, N=1, T=1024, Hq=8, Hv=8, use_qk_l2norm=1))
    assert s == 2 and bnd[0] == 0 and bnd[2] == 16 and 0 < bnd[1] < 8


def test_transition_buffer_size():
    P = lambda **kw: ctypes.byref(good(**kw))
    # one fp32 K x K matrix per (sequence, value head, segment) of a split plan
    assert lib.gdr_chunk_trans_size(P(h_packed=1, B=1, N=1, T=4096, Hq=2, Hv=4,
                                      cp_segments=3)) == 1 * 4 * 3 * 128 * 128 * 4
    assert lib.gdr_chunk_trans_size(P(h_packed=1, B=1, N=1, T=4096, Hq=2, Hv=4,
                                      cp_segments=1)) == 0
    # nothing is kept without the states path
    assert lib.gdr_chunk_trans_size(P(h_packed=0, B=1, N=1, T=4096, Hq=2, Hv=4,
                                      cp_segments=3)) == 0
    cp, _ = plan(good(h_packed=1, B=1, N=1, T=65536, Hq=32, Hv=32), 0)
    assert lib.gdr_chunk_trans_size(P(h_packed=1, B=1, N=1, T=65536, Hq=32, Hv=32)) == \
        32 * cp * 128 * 128 * 4
    # q / k normalised in the kernel: the unit q and k rows (bf16) and their
    # fp32 norms follow the transitions, 256-byte aligned, whatever the plan
    a256 = lambda n: (n + 255) // 256 * 256
    rows = 2 * 4096 * 16
    assert lib.gdr_chunk_trans_size(P(h_packed=1, B=2, N=2, T=4096, Hq=16, Hv=32,
                                      use_qk_l2norm=1)) == \
        2 * a256(rows * 128 * 2) + a256(rows * 4) + rows * 4
    rows = 4096 * 2
    assert lib.gdr_chunk_trans_size(P(h_packed=1, B=1, N=1, T=4096, Hq=2, Hv=4, cp_segments=3,
                                      use_qk_l2norm=1)) == \
        a256(4 * 3 * 128 * 128 * 4) + 2 * a256(rows * 128 * 2) + a256(rows * 4) + rows * 4
    assert lib.gdr_chunk_trans_size(P(h_packed=0, B=1, N=1, T=4096, Hq=2, Hv=4,
                                      use_qk_l2norm=1)) == 0


def test_null_and_workspace_errors_before_any_device_work():
    p = good()
    P = ctypes.c_void_p
    # missing required outputs
    st = lib.gdr_chunk_fwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), None, None, P(16),
                           P(16), None, None, None, 0, None)
    assert _lib.STATUS[st] == "GDR_ERR_NULL"
    st = lib.gdr_chunk_bwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), P(16), P(16), None,
                           P(16), P(16), P(16), P(16), P(16), P(16), None, P(16), 1 << 40, None)
    assert _lib.STATUS[st] == "GDR_ERR_NULL"  # initial_state without dh0
    pv = varlen(HOST_CU, T=200)
    st = lib.gdr_chunk_fwd(ctypes.byref(pv), P(16), P(16), P(16), P(16), P(16), None, P(16),
                           P(16), P(16), None, None, P(16), 1, None)
    assert _lib.STATUS[st] == "GDR_ERR_WORKSPACE"
    # the token-by-token forward: o is required, the states are optional
    st = lib.gdr_recurrent_fwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), None, None,
                               None, None)
    assert _lib.STATUS[st] == "GDR_ERR_NULL"
    st = lib.gdr_recurrent_fwd(ctypes.byref(good(K=64)), P(16), P(16), P(16), P(16), P(16), None,
                               P(16), None, None)
    assert _lib.STATUS[st] == "GDR_ERR_HEAD_DIM"
    # the gate: the plain backward refuses it, the gated backward needs it and g
    pg = good(use_gate=1, gate_A_log=FAKE_DEV)
    args = [P(16)] * 16
    st = lib.gdr_chunk_bwd(ctypes.byref(pg), *args[:7], None, *args[7:14], P(16), 1 << 40, None)
    assert _lib.STATUS[st] == "GDR_ERR_ARG" and "gdr_chunk_bwd_gate" in lib.gdr_last_error().decode()
    gate_args = [P(16)] * 19  # q .. ddt_bias, workspace
    st = lib.gdr_chunk_bwd_gate(ctypes.byref(p), *gate_args, 1 << 40, None)
    assert _lib.STATUS[st] == "GDR_ERR_ARG" and "use_gate" in lib.gdr_last_error().decode()
    gate_args[4] = None  # the gate input g
    st = lib.gdr_chunk_bwd_gate(ctypes.byref(pg), *gate_args, 1 << 40, None)
    assert _lib.STATUS[st] == "GDR_ERR_NULL"
    gate_args[4] = P(16)
    gate_args[16] = gate_args[17] = None  # the parameter gradients are optional
    st = lib.gdr_chunk_bwd_gate(ctypes.byref(pg), *gate_args, 1, None)
    assert _lib.STATUS[st] == "GDR_ERR_WORKSPACE"


def test_states_forward_rejections():
    P = ctypes.c_void_p
    req = [P(16)] * 10   # q, k, v, g, beta, initial_state, g_cum, A, o, h

    def call(p, h=P(16), trans=None, trans_bytes=0):
        a = list(req)
        a[9] = h
        return _lib.STATUS[lib.gdr_chunk_fwd_states(ctypes.byref(p), *a, trans, trans_bytes,
                                                    None, None, 0, None)]
    assert call(good()) == "GDR_ERR_ARG"                   # h_packed = 0
    assert call(good(h_packed=1), h=None) == "GDR_ERR_NULL"
    split = good(h_packed=1, B=1, N=1, T=4096, cp_segments=3)
    assert call(split) == "GDR_ERR_NULL"                   # a split plan needs trans
    assert "gdr_chunk_trans_size" in lib.gdr_last_error().decode()
    need = lib.gdr_chunk_trans_size(ctypes.byref(split))
    assert call(split, trans=P(16), trans_bytes=need - 4) == "GDR_ERR_WORKSPACE"
    # the backward checks the size of the transitions it is handed too
    args = [P(16)] * 10 + [P(16), P(16)]  # q .. initial_state, h, trans
    st = lib.gdr_chunk_bwd_states(ctypes.byref(split), *args, need - 4, *([P(16)] * 9),
                                  1 << 40, None)
    assert _lib.STATUS[st] == "GDR_ERR_WORKSPACE" and "trans" in lib.gdr_last_error().decode()


@pytest.mark.skipif(torch.cuda.is_available(), reason="exercises the no-device path")
def test_no_device_is_reported():
    assert _lib.STATUS[lib.gdr_check_device()] == "GDR_ERR_DEVICE"
    p = good()
    P = ctypes.c_void_p
    st = lib.gdr_chunk_fwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), None, P(16), P(16),
                           P(16), None, None, None, 0, None)
    assert _lib.STATUS[st] == "GDR_ERR_DEVICE"
    st = lib.gdr_recurrent_fwd(ctypes.byref(p), P(16), P(16), P(16), P(16), P(16), None, P(16),
                               None, None)
    assert _lib.STATUS[st] == "GDR_ERR_DEVICE"


def test_python_rejects_verifier_options():
    import gated_delta_rule_66_amd as gdr
    x = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 1, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        gdr.chunk_gated_delta_rule(x, x, x, g, g, transpose_state_layout=True)
    # the gate is supported, but needs its decay parameters
    with pytest.raises(gdr.GdrError):
        gdr.chunk_gated_delta_rule(x, x, x, g, g, use_gate_in_kernel=True)


def _inputs(B=1, T=100, Hq=2, Hv=4, dt=torch.bfloat16):
    q = torch.zeros(B, T, Hq, 128, dtype=dt)
    return dict(q=q, k=q.clone(), v=torch.zeros(B, T, Hv, 128, dtype=dt),
                g=torch.zeros(B, T, Hv, dtype=dt), beta=torch.zeros(B, T, Hv, dtype=dt))


BINDING_REJECT = [
    # (name, fwd or bwd, override, error name, message part)
    ("short k", "fwd", dict(k=torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)), "GDR_ERR_SHAPE",
     "k must have shape"),
    ("fp16 k", "fwd", dict(k=torch.zeros(1, 100, 2, 128, dtype=torch.float16)), "GDR_ERR_DTYPE",
     "k must be"),
    ("fp32 beta", "fwd", dict(beta=torch.zeros(1, 100, 4)), "GDR_ERR_DTYPE", "beta must be"),
    ("beta per q head", "fwd", dict(beta=torch.zeros(1, 100, 2, dtype=torch.bfloat16)),
     "GDR_ERR_SHAPE", "beta must have shape"),
    ("v of another length", "fwd", dict(v=torch.zeros(1, 99, 4, 128, dtype=torch.bfloat16)),
     "GDR_ERR_SHAPE", "v must have shape"),
    ("one-row h0 for two sequences", "fwd",
     dict(initial_state=torch.zeros(1, 4, 128, 128), cu_seqlens=torch.tensor([0, 40, 100])),
     "GDR_ERR_SHAPE", "initial_state must have shape"),
    ("transposed h0 without state_v_first", "fwd",
     dict(initial_state=torch.zeros(1, 4, 128, 64)), "GDR_ERR_SHAPE", "initial_state"),
    ("A with 32 columns", "bwd", dict(A=torch.zeros(1, 100, 4, 32, dtype=torch.bfloat16)),
     "GDR_ERR_SHAPE", "A must have shape"),
    ("bf16 g_cum", "bwd", dict(g=torch.zeros(1, 100, 4, dtype=torch.bfloat16)),
     "GDR_ERR_DTYPE", "fp32 g_cum"),
    ("do per q head", "bwd", dict(do=torch.zeros(1, 100, 2, 128, dtype=torch.bfloat16)),
     "GDR_ERR_SHAPE", "do must have shape"),
    ("dht with three rows", "bwd", dict(dht=torch.zeros(3, 4, 128, 128)), "GDR_ERR_SHAPE",
     "dht must have shape"),
]


@pytest.mark.parametrize("name,which,over,status,msg", BINDING_REJECT,
                         ids=[r[0] for r in BINDING_REJECT])
def test_binding_checks_every_tensor_before_the_call(name, which, over, status, msg):
    """A tensor whose shape, dtype or device disagrees with the problem would
    be read out of bounds (or reinterpreted) by the kernels through its raw
    pointer: the binding rejects it on the host first."""
    import gated_delta_rule_66_amd as gdr
    x = _inputs()
    if which == "fwd":
        x.update(over)
        with pytest.raises(gdr.GdrError) as e:
            gdr.chunk_gated_delta_rule_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                           initial_state=x.get("initial_state"),
                                           cu_seqlens=x.get("cu_seqlens"))
    else:
        b = dict(g=torch.zeros(1, 100, 4), A=torch.zeros(1, 100, 4, 64, dtype=torch.bfloat16),
                 do=torch.zeros(1, 100, 4, 128, dtype=torch.bfloat16), dht=None)
        b.update(over)
        with pytest.raises(gdr.GdrError) as e:
            gdr.chunk_gated_delta_rule_bwd(x["q"], x["k"], x["v"], b["g"], x["beta"], b["A"],
                                           b["do"], dht=b["dht"])
    assert e.value.name == status
    assert msg in str(e.value)


def test_binding_rejects_a_tensor_on_another_device():
    import gated_delta_rule_66_amd as gdr
    x = _inputs()
    meta_v = torch.empty(1, 100, 4, 128, dtype=torch.bfloat16, device="meta")
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_gated_delta_rule_fwd(x["q"], x["k"], meta_v, x["g"], x["beta"])
    assert e.value.name == "GDR_ERR_DEVICE"


def test_no_alloc_forward_rejects_problems_past_its_scratch_before_device_work():
    P = ctypes.c_void_p
    assert _lib.lib.gdr_chunk_fwd_noalloc is not None
    # four 65,536-token sequences of 32 heads split in segments need 192 MiB
    # of context-parallel buffers: more than the 64 MiB static array
    big = good(B=4, N=4, T=65536, Hq=32, Hv=32, cp_segments=8)
    need = lib.gdr_chunk_fwd_workspace_size(ctypes.byref(big))
    assert need > (64 << 20)
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(big), *[P(16)] * 5, None, P(16), P(16), P(16),
                                   None, None, None)
    assert _lib.STATUS[st] == "GDR_ERR_WORKSPACE"
    assert "no-allocation forward holds at most 67108864" in lib.gdr_last_error().decode()
    # the same validation as gdr_chunk_fwd comes first
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(good(K=64)), *[P(16)] * 5, None, P(16), P(16),
                                   P(16), None, None, None)
    assert _lib.STATUS[st] == "GDR_ERR_HEAD_DIM"
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(good()), *[P(16)] * 5, None, None, P(16), P(16),
                                   None, None, None)
    assert _lib.STATUS[st] == "GDR_ERR_NULL"
    # one long sequence fits (48 MiB of segment buffers)
    one = good(B=1, N=1, T=65536, Hq=32, Hv=32, cp_segments=8)
    assert 0 < lib.gdr_chunk_fwd_workspace_size(ctypes.byref(one)) <= (64 << 20)


def test_unpack_states_follows_the_packed_layout():
    """unpack_states against the packed layout the header states, element by
    element: ((vb * 4 + kb) * 64 + 16 g + c) * 8 + e holds value 16 vb + c at
    key 32 kb + 4 g + e (e < 4) or 32 kb + 16 + 4 g + e - 4 (e >= 4)."""
    import gated_delta_rule_66_amd as gdr
    kv = torch.arange(128 * 128, dtype=torch.float64).reshape(128, 128)  # [key][value]
    packed = torch.empty(128 * 128, dtype=torch.float64)
    for vb in range(8):
        for kb in range(4):
            for g in range(4):
                for c in range(16):
                    for e in range(8):
                        key = 32 * kb + 4 * g + e if e < 4 else 32 * kb + 16 + 4 * g + e - 4
                        packed[((vb * 4 + kb) * 64 + 16 * g + c) * 8 + e] = kv[key, 16 * vb + c]
    out = gdr.unpack_states(packed.reshape(1, 1, -1).repeat(2, 3, 1))
    assert out.shape == (2, 3, 128, 128)
    assert torch.equal(out[1, 2], kv)
