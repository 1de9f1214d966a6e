"""Chunked gated delta rule (GDN chunked prefill) for AMD MI355X.

A thin binding over libgdr.so (``include/gdr.h``).  PyTorch provides device
memory and the current stream; every step of the computation runs in the HIP
kernels of the library.  Names and arguments follow the FlashQLA pages
("flashqla-linear-attention", Core API and Low-Level API; "FlashQLA
Documentation", forward / backward and the utilities prepare_lens,
prepare_chunk_indices, prepare_chunk_offsets).

Shapes: q, k ``[B, T, Hq, K]``; v ``[B, T, Hv, V]``; g, beta ``[B, T, Hv]``;
states ``[N, Hv, K, V]`` (``[N, Hv, V, K]`` with ``state_v_first``), fp32.
K = V = 128; bf16 or fp16 inputs; Hv a multiple of Hq.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (GDR_BF16, GDR_FP16, GDR_FP32, GdrError, Problem, check, lib)

__all__ = [
    "chunk_gated_delta_rule", "chunk_gated_delta_rule_fwd", "chunk_gated_delta_rule_fwd_states",
    "chunk_gated_delta_rule_bwd",
    "fused_recurrent_gated_delta_rule", "prepare_lens", "prepare_chunk_indices",
    "prepare_chunk_offsets", "unpack_states", "GdrError",
]

CHUNK = 64
_DT = {torch.bfloat16: GDR_BF16, torch.float16: GDR_FP16, torch.float32: GDR_FP32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _code(dtype):
    if dtype not in _DT:
        raise GdrError(4, "unsupported dtype %s" % dtype)
    return _DT[dtype]


class _Call:
    """Problem descriptor plus the host copy of cu_seqlens it points to."""

    def __init__(self, q, v, g_dtype, scale, cu_seqlens, cu_seqlens_cpu, state_v_first,
                 cp_segments, wave_tiles=0, use_qk_l2norm=False, beta_sigmoid=False,
                 neg_eigval=False, gate=None, h_packed=False):
        if q.dim() != 4 or v.dim() != 4:
            raise GdrError(2, "q and v must be 4-D ([B, T, H, dim]), got %s and %s"
                           % (tuple(q.shape), tuple(v.shape)))
        B, T, Hq, K = q.shape
        Hv, V = v.shape[2], v.shape[3]
        # gate = (A_log, dt_bias or None): fp32 [Hv] device copies the problem points to
        self.gate = None
        if gate is not None:
            A_log, dt_bias = gate
            if A_log is None:
                raise GdrError(1, "use_gate_in_kernel needs A_log")
            self.gate = tuple(None if t is None else
                              t.detach().to(device=q.device, dtype=torch.float32).reshape(-1)
                              .contiguous() for t in (A_log, dt_bias))
            for t in self.gate:
                if t is not None and t.numel() != Hv:
                    raise GdrError(2, "A_log and dt_bias need Hv=%d entries" % Hv)
        self.cu_host = None
        self.cu_dev = None
        if cu_seqlens is not None:
            self.cu_dev = cu_seqlens.to(device=q.device, dtype=torch.int32).contiguous()
            if cu_seqlens_cpu is None:
                # launch planning needs the lengths on the host: one blocking
                # device-to-host copy (pass cu_seqlens_cpu to avoid it)
                cu_seqlens_cpu = cu_seqlens.detach().to("cpu")
            self.cu_host = cu_seqlens_cpu.to(torch.int32).contiguous()
            N = self.cu_host.numel() - 1
        else:
            N = B
        if scale is None:
            scale = K ** -0.5
        self.p = Problem(B=B, T=T, Hq=Hq, Hv=Hv, K=K, V=V, N=N,
                         cu_seqlens_dev=None if self.cu_dev is None else self.cu_dev.data_ptr(),
                         cu_seqlens_host=None if self.cu_host is None else self.cu_host.data_ptr(),
                         in_dtype=_code(q.dtype), g_dtype=_code(g_dtype), scale=float(scale),
                         state_v_first=1 if state_v_first else 0, cp_segments=int(cp_segments),
                         wave_tiles=int(wave_tiles), use_qk_l2norm=1 if use_qk_l2norm else 0,
                         beta_sigmoid=1 if beta_sigmoid else 0,
                         neg_eigval=1 if neg_eigval else 0,
                         use_gate=0 if self.gate is None else 1,
                         gate_A_log=None if self.gate is None else self.gate[0].data_ptr(),
                         gate_dt_bias=None if self.gate is None or self.gate[1] is None
                         else self.gate[1].data_ptr(),
                         h_packed=1 if h_packed else 0)
        self.N, self.Hv, self.K, self.V = N, Hv, K, V
        self.ref = ctypes.byref(self.p)
        reason = ctypes.create_string_buffer(256)
        check(lib.gdr_check_supported(self.ref, reason, 256))

    def state_shape(self, state_v_first):
        return (self.N, self.Hv, self.V, self.K) if state_v_first else (self.N, self.Hv, self.K, self.V)

    def h_shape(self, state_v_first, h_packed=False):
        """Shape of the chunk-start states h: [NC, Hv, K, V] ([NC, Hv, V, K]
        with state_v_first), or [NC, Hv, 128 * 128] packed (h_packed)."""
        if h_packed:
            return (self.num_chunks(), self.Hv, self.K * self.V)
        return (self.num_chunks(), self.Hv) + self.state_shape(state_v_first)[2:]

    def num_chunks(self):
        if self.cu_host is None:
            return self.p.B * ((self.p.T + CHUNK - 1) // CHUNK)
        n = ctypes.c_int64(0)
        offs = torch.empty(self.cu_host.numel(), dtype=torch.int32)
        check(lib.gdr_prepare_chunk_offsets_i32(_ptr(self.cu_host), self.cu_host.numel(), CHUNK,
                                                _ptr(offs), ctypes.byref(n)))
        return int(n.value)


def _contig(*ts):
    return [None if t is None else t.contiguous() for t in ts]


def _expect(name, t, shape, dtypes, device):
    """Rejects a tensor whose shape, dtype or device does not match what the
    kernels read through its pointer (None passes: optional arguments)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise GdrError(2, "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if dtypes is not None and t.dtype not in dtypes:
        raise GdrError(4, "%s must be %s, got %s"
                       % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if t.device != device:
        raise GdrError(8, "%s is on %s but q is on %s" % (name, t.device, device))


_FLOATS = (torch.float32, torch.bfloat16, torch.float16)


def _check_inputs(c, q, k, v, g, beta, state_v_first, initial_state=None, A=None, do=None,
                  dht=None, g_cum=None, g_input=None):
    """Every tensor the C call receives as a raw pointer against the problem
    the descriptor states: token tensors [B, T, heads, ..] in q's dtype,
    g_cum fp32, states [N, Hv, K, V] (or [N, Hv, V, K]) with one row per
    sequence, all on q's device."""
    B, T, Hq, K = q.shape
    dev, dt = q.device, (q.dtype,)
    Hv, V = c.Hv, c.V
    _expect("k", k, (B, T, Hq, K), dt, dev)
    _expect("v", v, (B, T, Hv, V), dt, dev)
    _expect("g", g, (B, T, Hv), (q.dtype, torch.float32), dev)
    _expect("beta", beta, (B, T, Hv), dt, dev)
    _expect("A", A, (B, T, Hv, CHUNK), dt, dev)
    _expect("do", do, (B, T, Hv, V), dt, dev)
    _expect("g_cum", g_cum, (B, T, Hv), (torch.float32,), dev)
    _expect("g_input", g_input, (B, T, Hv), (q.dtype, torch.float32), dev)
    st = c.state_shape(state_v_first)
    _expect("initial_state", initial_state, st, _FLOATS, dev)
    _expect("dht", dht, st, _FLOATS, dev)


def _workspace(nbytes, dev, workspace):
    """The caller's workspace (a device uint8 tensor of at least nbytes), or a
    new one."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if (workspace.device != dev or workspace.dtype != torch.uint8
            or not workspace.is_contiguous() or workspace.numel() < nbytes):
        raise GdrError(7, "workspace must be a contiguous uint8 tensor of at least %d bytes on %s"
                       % (nbytes, dev))
    return workspace


def chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale=None, initial_state=None,
                               output_final_state=True, cu_seqlens=None, state_v_first=False,
                               output_h=False, cp_segments=0, cu_seqlens_cpu=None,
                               wave_tiles=0, use_qk_l2norm_in_kernel=False,
                               use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                               use_gate_in_kernel=False, A_log=None, dt_bias=None,
                               workspace=None, no_alloc=False, h_packed=False):
    """Forward.  Returns ``(g_cum, A, o, h, final_state)``: the chunk-local
    cumsum of g (fp32), the per-chunk inverse A ``[B,T,Hv,64]``, the output,
    the chunk-start states (``None`` unless ``output_h``) and the fp32 final
    state (``None`` unless ``output_final_state``).  With
    ``use_qk_l2norm_in_kernel`` the kernels scale q and k per (token, head)
    to unit length, ``x / sqrt(sum x^2 + 1e-6)``, before use.  With
    ``use_beta_sigmoid_in_kernel`` beta is a logit and the recurrence uses
    ``sigmoid(beta)``; with ``allow_neg_eigval`` it uses twice that.  With
    ``use_gate_in_kernel`` g is the gate's raw input x and the log decay is
    ``-exp(A_log[h]) * softplus(x + dt_bias[h])`` (A_log, dt_bias: ``[Hv]``;
    dt_bias may be None); g_cum is the cumsum of that log decay.  ``workspace``
    (optional): a device uint8 tensor of at least
    ``gdr_chunk_fwd_workspace_size`` bytes to use instead of a new one; its
    contents need no initialisation.  ``no_alloc``: call
    ``gdr_chunk_fwd_noalloc``, which takes no workspace (the library's static
    64 MiB device array instead; larger problems raise).  The outputs are
    still new tensors unless the caller hands them in through the C ABI.
    ``h_packed``: with ``output_h``, h is ``[NC, Hv, 16384]`` in the packed
    layout ``chunk_gated_delta_rule_bwd`` takes as its ``h`` (the states are
    then not recomputed): element ``((vb*4 + kb)*64 + 16*g + c)*8 + e`` is the
    state at value ``16*vb + c`` and key ``32*kb + 16*(e >= 4) + 4*g + e % 4``
    (:func:`unpack_states` gives ``[NC, Hv, K, V]``)."""
    return _fwd(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                state_v_first, output_h, cp_segments, cu_seqlens_cpu, wave_tiles,
                use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, allow_neg_eigval,
                use_gate_in_kernel, A_log, dt_bias, workspace, no_alloc, h_packed, False)


def chunk_gated_delta_rule_fwd_states(q, k, v, g, beta, scale=None, initial_state=None,
                                      output_final_state=True, cu_seqlens=None,
                                      state_v_first=False, cp_segments=0, cu_seqlens_cpu=None,
                                      wave_tiles=0, use_qk_l2norm_in_kernel=False,
                                      use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                                      use_gate_in_kernel=False, A_log=None, dt_bias=None,
                                      workspace=None):
    """The forward the autograd op runs (``gdr_chunk_fwd_states``):
    :func:`chunk_gated_delta_rule_fwd` with ``output_h=True, h_packed=True``
    that also keeps, when the plan splits sequences into T-segments, each
    segment's fp32 state transition for the backward.  Returns ``(g_cum, A,
    o, h, trans, final_state)``; ``trans`` also keeps, with
    ``use_qk_l2norm_in_kernel``, the unit q and k rows and their norms, and is
    ``None`` when nothing is split and q, k are not normalised.
    Hand ``h`` and ``trans`` to :func:`chunk_gated_delta_rule_bwd`."""
    return _fwd(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                state_v_first, True, cp_segments, cu_seqlens_cpu, wave_tiles,
                use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, allow_neg_eigval,
                use_gate_in_kernel, A_log, dt_bias, workspace, False, True, True)


def _fwd(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens, state_v_first,
         output_h, cp_segments, cu_seqlens_cpu, wave_tiles, use_qk_l2norm_in_kernel,
         use_beta_sigmoid_in_kernel, allow_neg_eigval, use_gate_in_kernel, A_log, dt_bias,
         workspace, no_alloc, h_packed, keep):
    q, k, v, g, beta, initial_state = _contig(q, k, v, g, beta, initial_state)
    c = _Call(q, v, g.dtype, scale, cu_seqlens, cu_seqlens_cpu, state_v_first, cp_segments,
              wave_tiles, use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, allow_neg_eigval,
              (A_log, dt_bias) if use_gate_in_kernel else None, h_packed=h_packed)
    _check_inputs(c, q, k, v, g, beta, state_v_first, initial_state=initial_state)
    dev = q.device
    B, T = q.shape[0], q.shape[1]
    g_cum = torch.empty(B, T, c.Hv, dtype=torch.float32, device=dev)
    A = torch.empty(B, T, c.Hv, CHUNK, dtype=q.dtype, device=dev)
    o = torch.empty(B, T, c.Hv, c.V, dtype=q.dtype, device=dev)
    h = None
    if output_h:
        h = torch.empty(c.h_shape(state_v_first, h_packed), dtype=q.dtype, device=dev)
    ht = torch.empty(c.state_shape(state_v_first), dtype=torch.float32, device=dev) \
        if output_final_state else None
    if initial_state is not None:
        initial_state = initial_state.to(torch.float32).contiguous()
    if no_alloc:
        if workspace is not None:
            raise GdrError(10, "no_alloc takes no workspace")
        check(lib.gdr_chunk_fwd_noalloc(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(initial_state), _ptr(g_cum), _ptr(A), _ptr(o),
                                        _ptr(h), _ptr(ht), _stream(dev)))
        return g_cum, A, o, h, ht
    ws_bytes = lib.gdr_chunk_fwd_workspace_size(c.ref)
    ws = _workspace(ws_bytes, dev, workspace)
    if keep:
        tr_bytes = lib.gdr_chunk_trans_size(c.ref)
        trans = (torch.empty(tr_bytes // 4, dtype=torch.float32, device=dev)
                 if tr_bytes else None)
        check(lib.gdr_chunk_fwd_states(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(initial_state), _ptr(g_cum), _ptr(A), _ptr(o),
                                       _ptr(h), _ptr(trans), tr_bytes, _ptr(ht), _ptr(ws),
                                       ws_bytes, _stream(dev)))
        return g_cum, A, o, h, trans, ht
    check(lib.gdr_chunk_fwd(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(initial_state), _ptr(g_cum), _ptr(A), _ptr(o), _ptr(h), _ptr(ht),
                            _ptr(ws), ws_bytes, _stream(dev)))
    return g_cum, A, o, h, ht


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht=None, scale=None, initial_state=None,
                               cu_seqlens=None, state_v_first=False, dg_dtype=None,
                               cp_segments=0, cu_seqlens_cpu=None, wave_tiles=0,
                               use_qk_l2norm_in_kernel=False, use_beta_sigmoid_in_kernel=False,
                               allow_neg_eigval=False, use_gate_in_kernel=False, A_log=None,
                               dt_bias=None, g_input=None, workspace=None, h=None,
                               trans=None):
    """Backward.  ``g`` is the forward's fp32 ``g_cum`` output.  Returns
    ``(dq, dk, dv, dbeta, dg, dh0)``; ``dg`` is the gradient with respect to
    the raw log-decay g (dtype ``dg_dtype``, default the input dtype) and
    ``dh0`` is ``None`` without an initial state.  With
    ``use_qk_l2norm_in_kernel`` (as in the forward that produced ``A``), q and
    k are the raw rows and dq, dk are with respect to them; with the beta
    options dbeta is with respect to the beta input.  With
    ``use_gate_in_kernel`` ``g_input`` is the gate input the forward took,
    ``dg`` is with respect to it (dtype ``dg_dtype``, default g_input's) and
    two more entries follow: the fp32 gradients of ``A_log`` and ``dt_bias``
    (``[Hv]``).  ``workspace`` as in the forward, of at least
    ``gdr_chunk_bwd_workspace_size`` bytes (``..._states_workspace_size`` with
    ``h``).  ``h``: the packed chunk-start states the forward returned for the
    same inputs with ``output_h=True, h_packed=True``; the backward then
    skips recomputing them (``gdr_chunk_bwd_states``).  ``trans`` (with
    ``h``): the segment transitions :func:`chunk_gated_delta_rule_fwd_states`
    returned for the same inputs; a split backward then applies them instead
    of forming its own."""
    q, k, v, g, beta, A, do, dht, initial_state, g_input, h, trans = _contig(
        q, k, v, g, beta, A, do, dht, initial_state, g_input, h, trans)
    if trans is not None and h is None:
        raise GdrError(1, "trans comes with the forward's states h")
    if g.dtype != torch.float32:
        raise GdrError(4, "the backward takes the forward's fp32 g_cum as g")
    if use_gate_in_kernel and g_input is None:
        raise GdrError(1, "use_gate_in_kernel needs the gate input (g_input)")
    if dg_dtype is None:
        dg_dtype = g_input.dtype if use_gate_in_kernel else q.dtype
    if use_gate_in_kernel and g_input.dtype != dg_dtype:
        g_input = g_input.to(dg_dtype).contiguous()
    c = _Call(q, v, dg_dtype, scale, cu_seqlens, cu_seqlens_cpu, state_v_first, cp_segments,
              wave_tiles, use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, allow_neg_eigval,
              (A_log, dt_bias) if use_gate_in_kernel else None, h_packed=h is not None)
    _check_inputs(c, q, k, v, None, beta, state_v_first, initial_state=initial_state, A=A,
                  do=do, dht=dht, g_cum=g, g_input=g_input)
    _expect("h", h, c.h_shape(state_v_first, True), (q.dtype,), q.device)
    if trans is not None:
        n_tr = lib.gdr_chunk_trans_size(c.ref) // 4
        _expect("trans", trans, (n_tr,), (torch.float32,), q.device)
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    db = torch.empty_like(beta)
    dg = torch.empty(g.shape, dtype=dg_dtype, device=dev)
    dh0 = None
    if initial_state is not None:
        initial_state = initial_state.to(torch.float32).contiguous()
        dh0 = torch.empty(c.state_shape(state_v_first), dtype=torch.float32, device=dev)
    if dht is not None:
        dht = dht.to(torch.float32).contiguous()
    if h is not None:
        ws_bytes = lib.gdr_chunk_bwd_states_workspace_size(c.ref)
        ws = _workspace(ws_bytes, dev, workspace)
        dA_log = ddt_bias = None
        if use_gate_in_kernel:
            dA_log = torch.empty(c.Hv, dtype=torch.float32, device=dev)
            ddt_bias = torch.empty(c.Hv, dtype=torch.float32, device=dev)
        check(lib.gdr_chunk_bwd_states(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(g_input if use_gate_in_kernel else None), _ptr(beta),
                                       _ptr(A), _ptr(do), _ptr(dht), _ptr(initial_state), _ptr(h),
                                       _ptr(trans),
                                       0 if trans is None else trans.numel() * 4,
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(dg), _ptr(dh0),
                                       _ptr(dA_log), _ptr(ddt_bias), _ptr(ws), ws_bytes,
                                       _stream(dev)))
        if use_gate_in_kernel:
            return dq, dk, dv, db, dg, dh0, dA_log, ddt_bias
        return dq, dk, dv, db, dg, dh0
    ws_bytes = lib.gdr_chunk_bwd_workspace_size(c.ref)
    ws = _workspace(ws_bytes, dev, workspace)
    if use_gate_in_kernel:
        dA_log = torch.empty(c.Hv, dtype=torch.float32, device=dev)
        ddt_bias = torch.empty(c.Hv, dtype=torch.float32, device=dev)
        check(lib.gdr_chunk_bwd_gate(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_input),
                                     _ptr(beta), _ptr(A), _ptr(do), _ptr(dht),
                                     _ptr(initial_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db),
                                     _ptr(dg), _ptr(dh0), _ptr(dA_log), _ptr(ddt_bias), _ptr(ws),
                                     ws_bytes, _stream(dev)))
        return dq, dk, dv, db, dg, dh0, dA_log, ddt_bias
    check(lib.gdr_chunk_bwd(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                            _ptr(do), _ptr(dht), _ptr(initial_state), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(db), _ptr(dg), _ptr(dh0), _ptr(ws), ws_bytes, _stream(dev)))
    return dq, dk, dv, db, dg, dh0


class _GatedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                state_v_first, cp_segments, cu_seqlens_cpu, use_qk_l2norm, beta_sigmoid,
                neg_eigval, use_gate, A_log, dt_bias, recompute_states):
        if cu_seqlens is not None and cu_seqlens_cpu is None:
            # the one device-to-host copy of the lengths, shared by the backward
            cu_seqlens_cpu = cu_seqlens.detach().to("cpu")
        kw = dict(use_qk_l2norm_in_kernel=use_qk_l2norm, use_beta_sigmoid_in_kernel=beta_sigmoid,
                  allow_neg_eigval=neg_eigval, use_gate_in_kernel=use_gate, A_log=A_log,
                  dt_bias=dt_bias)
        h = trans = None
        if recompute_states:
            g_cum, A, o, _, ht = chunk_gated_delta_rule_fwd(
                q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                state_v_first, False, cp_segments, cu_seqlens_cpu, **kw)
        else:
            g_cum, A, o, h, trans, ht = chunk_gated_delta_rule_fwd_states(
                q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                state_v_first, cp_segments, cu_seqlens_cpu, **kw)
        ctx.save_for_backward(q, k, v, g_cum, beta, A, initial_state, cu_seqlens, cu_seqlens_cpu,
                              g if use_gate else None, A_log, dt_bias, h, trans)
        ctx.scale, ctx.svf, ctx.cp, ctx.g_dtype = scale, state_v_first, cp_segments, g.dtype
        ctx.qk_norm, ctx.beta_sigmoid, ctx.neg_eigval = use_qk_l2norm, beta_sigmoid, neg_eigval
        ctx.use_gate = use_gate
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g_cum, beta, A, h0, cu, cu_cpu, g_in, A_log, dt_bias, h, trans = ctx.saved_tensors
        grads = chunk_gated_delta_rule_bwd(
            q, k, v, g_cum, beta, A, do, dht, ctx.scale, h0, cu, ctx.svf, ctx.g_dtype, ctx.cp,
            cu_cpu, use_qk_l2norm_in_kernel=ctx.qk_norm,
            use_beta_sigmoid_in_kernel=ctx.beta_sigmoid, allow_neg_eigval=ctx.neg_eigval,
            use_gate_in_kernel=ctx.use_gate, A_log=A_log, dt_bias=dt_bias, g_input=g_in, h=h,
            trans=trans)
        dq, dk, dv, db, dg, dh0 = grads[:6]
        dA = ddt = None
        if ctx.use_gate:
            dA = grads[6].to(A_log.dtype)
            ddt = None if dt_bias is None else grads[7].to(dt_bias.dtype)
        return (dq, dk, dv, dg, db, None, dh0, None, None, None, None, None, None, None, None,
                None, dA, ddt, None)


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=False, use_qk_l2norm_in_kernel=False,
                           state_v_first=False, cu_seqlens=None, cp_segments=0,
                           cu_seqlens_cpu=None, use_beta_sigmoid_in_kernel=False,
                           allow_neg_eigval=False, use_gate_in_kernel=False, A_log=None,
                           dt_bias=None, recompute_states=False, **unsupported):
    """High-level op with autograd: returns ``(o, final_state)``.

    The forward keeps its chunk-start states (packed, in the input dtype, 32
    KiB per chunk and value head) and, when its plan splits sequences into
    T-segments, each segment's fp32 state transition (64 KiB per segment and
    value head) for the backward, which then neither recomputes the states
    nor forms its own transitions; ``recompute_states=True`` keeps only the
    inputs and recomputes the states in the backward instead.

    ``use_qk_l2norm_in_kernel`` scales q and k per (token, head) to unit
    length inside the kernels (and carries the gradient back to the raw q, k);
    ``use_beta_sigmoid_in_kernel`` takes beta as a logit (sigmoid in the
    kernels) and ``allow_neg_eigval`` doubles beta.  ``use_gate_in_kernel``
    takes g as the gate's raw input, with the log decay
    ``-exp(A_log) * softplus(g + dt_bias)`` per value head (gradients flow to
    g, A_log and dt_bias).  Inter-card context parallelism and
    transpose_state_layout raise NotImplementedError."""
    for key, val in unsupported.items():
        if val:
            raise NotImplementedError("%s is not supported" % key)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _GatedDeltaRule.apply(q, k, v, g, beta, scale, initial_state, output_final_state,
                                 cu_seqlens, state_v_first, cp_segments, cu_seqlens_cpu,
                                 bool(use_qk_l2norm_in_kernel), bool(use_beta_sigmoid_in_kernel),
                                 bool(allow_neg_eigval), bool(use_gate_in_kernel),
                                 A_log if use_gate_in_kernel else None,
                                 dt_bias if use_gate_in_kernel else None, bool(recompute_states))


def fused_recurrent_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                                     output_final_state=True, cu_seqlens=None,
                                     state_v_first=False, use_qk_l2norm_in_kernel=False,
                                     inplace_final_state=False, cu_seqlens_cpu=None,
                                     use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                                     use_gate_in_kernel=False, A_log=None, dt_bias=None):
    """Forward one token at a time (decode steps, a few speculative tokens,
    a prefill continued from a cached state).  Same inputs and outputs as
    :func:`chunk_gated_delta_rule` without autograd: returns ``(o,
    final_state)``; ``g`` is the raw log decay (the gate input with
    ``use_gate_in_kernel``).  With ``inplace_final_state`` the fp32
    ``initial_state`` tensor is updated in place and returned as the final
    state."""
    q, k, v, g, beta = _contig(q, k, v, g, beta)
    c = _Call(q, v, g.dtype, scale, cu_seqlens, cu_seqlens_cpu, state_v_first, 1, 0,
              use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, allow_neg_eigval,
              (A_log, dt_bias) if use_gate_in_kernel else None)
    _check_inputs(c, q, k, v, g, beta, state_v_first, initial_state=initial_state)
    dev = q.device
    B, T = q.shape[0], q.shape[1]
    o = torch.empty(B, T, c.Hv, c.V, dtype=q.dtype, device=dev)
    if inplace_final_state:
        if (initial_state is None or initial_state.dtype != torch.float32
                or not initial_state.is_contiguous()
                or tuple(initial_state.shape) != c.state_shape(state_v_first)):
            raise GdrError(10, "inplace_final_state needs a contiguous fp32 initial_state of "
                               "shape %s" % (c.state_shape(state_v_first),))
        ht = initial_state
    else:
        if initial_state is not None:
            initial_state = initial_state.to(torch.float32).contiguous()
        ht = torch.empty(c.state_shape(state_v_first), dtype=torch.float32, device=dev) \
            if output_final_state else None
    check(lib.gdr_recurrent_fwd(c.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(initial_state), _ptr(o), _ptr(ht), _stream(dev)))
    return o, ht


def unpack_states(h):
    """``[NC, Hv, K, V]`` from packed chunk-start states ``[NC, Hv, 16384]``
    (``h_packed``): a view change and a permutation, no arithmetic."""
    nc, hv = h.shape[0], h.shape[1]
    x = h.reshape(nc, hv, 8, 4, 4, 16, 2, 4)   # vb, kb, g, c, half, e
    return x.permute(0, 1, 3, 6, 4, 7, 2, 5).reshape(nc, hv, 128, 128)


# ---- variable-length helpers ------------------------------------------------

def _cu_host(cu_seqlens):
    cu = cu_seqlens.detach().to("cpu")
    if cu.dtype == torch.int32:
        return cu.contiguous(), "i32"
    return cu.to(torch.int64).contiguous(), "i64"


def prepare_lens(cu_seqlens: torch.Tensor) -> torch.Tensor:
    """Sequence lengths ``cu[i+1] - cu[i]`` (same dtype and device)."""
    cu, sfx = _cu_host(cu_seqlens)
    out = torch.empty(max(cu.numel() - 1, 0), dtype=cu.dtype)
    check(getattr(lib, "gdr_prepare_lens_" + sfx)(_ptr(cu), cu.numel(), _ptr(out)))
    return out.to(cu_seqlens.device)


def prepare_chunk_indices(cu_seqlens: torch.Tensor, chunk_size: int) -> torch.Tensor:
    """``[num_chunks, 2]``: per chunk, its sequence index and its chunk index
    inside that sequence."""
    cu, sfx = _cu_host(cu_seqlens)
    n = ctypes.c_int64(0)
    f = getattr(lib, "gdr_prepare_chunk_indices_" + sfx)
    check(f(_ptr(cu), cu.numel(), int(chunk_size), None, ctypes.byref(n)))
    out = torch.empty(int(n.value), 2, dtype=cu.dtype)
    check(f(_ptr(cu), cu.numel(), int(chunk_size), _ptr(out), ctypes.byref(n)))
    return out.to(cu_seqlens.device)


def prepare_chunk_offsets(cu_seqlens: torch.Tensor, chunk_size: int):
    """``(chunk_offsets, total_chunks)``: offsets has the shape of cu_seqlens;
    chunk c of sequence n sits at row ``chunk_offsets[n] + c`` of a global
    per-chunk buffer."""
    cu, sfx = _cu_host(cu_seqlens)
    out = torch.empty(cu.numel(), dtype=cu.dtype)
    total = ctypes.c_int64(0)
    check(getattr(lib, "gdr_prepare_chunk_offsets_" + sfx)(_ptr(cu), cu.numel(), int(chunk_size),
                                                           _ptr(out), ctypes.byref(total)))
    return out.to(cu_seqlens.device), int(total.value)


# ---- diagnostics --------------------------------------------------------------

def plan_info(q, v, g_dtype=None, cu_seqlens=None, cu_seqlens_cpu=None, cp_segments=0,
              wave_tiles=0, backward=False, h_packed=False):
    """``(cp_segments, wave_tiles)`` the library plans for these shapes, for the
    forward pass or (``backward=True``) the backward pass; ``h_packed``: the
    states path (a forward that keeps packed states, and the backward that
    takes them), which plans one tile per wave for the forward and one
    segment count for both directions."""
    c = _Call(q, v, q.dtype if g_dtype is None else g_dtype, None, cu_seqlens, cu_seqlens_cpu,
              False, cp_segments, wave_tiles, h_packed=h_packed)
    cp = ctypes.c_int32(0)
    vt = ctypes.c_int32(0)
    check(lib.gdr_plan_info(c.ref, 1 if backward else 0, ctypes.byref(cp), ctypes.byref(vt)))
    return int(cp.value), int(vt.value)


def pipeline_info(q, v, cu_seqlens=None, cu_seqlens_cpu=None, cp_segments=0, wave_tiles=0):
    """The backward's pipeline for these shapes on the states path (the
    autograd op's backward): ``(slices, bounds)``.  ``slices == 1``: one
    launch runs the state-gradient scan and every chunk's gradient
    workgroups, each starting once its chunk's state gradient is stored
    (``bounds == [0, chunks]``).  ``slices >= 2`` (q / k normalised in the
    kernel): the scan runs in ranges of chunks ``bounds[i] .. bounds[i+1]``
    and the last launch runs the gradients of chunks ``bounds[0] ..
    bounds[1]`` alone.  ``(0, [])``: one scan launch, then one gradient
    launch."""
    c = _Call(q, v, q.dtype, None, cu_seqlens, cu_seqlens_cpu, False, cp_segments, wave_tiles,
              h_packed=True)
    n = ctypes.c_int32(0)
    b = (ctypes.c_int32 * 9)()
    check(lib.gdr_bwd_pipeline_info(c.ref, ctypes.byref(n), b, 9))
    return int(n.value), [int(x) for x in b[:n.value + 1]] if n.value else []


class KernelTimer:
    """Brackets every kernel the library launches with HIP events while
    active; ``read()`` returns ``{name: (total_ms, launches)}``."""

    def __enter__(self):
        check(lib.gdr_profile_enable(1))
        return self

    def __exit__(self, *exc):
        lib.gdr_profile_enable(0)
        return False

    @staticmethod
    def read(max_entries=32):
        stride = 64
        names = ctypes.create_string_buffer(stride * max_entries)
        tot = (ctypes.c_double * max_entries)()
        cnt = (ctypes.c_int * max_entries)()
        n = lib.gdr_profile_read(names, stride, ctypes.cast(tot, ctypes.c_void_p),
                                 ctypes.cast(cnt, ctypes.c_void_p), max_entries)
        out = {}
        for i in range(n):
            nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
            out[nm] = (float(tot[i]), int(cnt[i]))
        return out
