"""Kimi Delta Attention (KDA) token mixer on MI355X (gfx950).

Thin Python binding over the C ABI in include/kda.h.  Every step of the
computation runs in the HIP kernels of ``libkda.so``; this module only checks
tensor metadata, allocates outputs and workspace with torch, and passes raw
device pointers plus the current HIP stream.  There is no fallback: if the
library is missing or a tensor is not on a GPU, the call raises.

    y, final_state = chunk_fwd(q, k, v, log_alpha, beta, gate,
                               initial_state=None, output_final_state=False, chunk=0)
    y = decode_step(q, k, v, log_alpha, beta, gate, state)   # state updated in place
    M, b = chunk_summary(k, v, log_alpha, beta)                # segment summary
    seg_states, final = combine_states(M_stack, b_stack, initial_state)

Outputs are fp32 by default (``out_dtype``); bf16 outputs are available but
their rounding alone exceeds a 2e-2 max-error-to-RMS budget on typical data.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi

__all__ = ["chunk_fwd", "chunk_bwd", "chunk_bwd_varlen", "chunk_fwd_varlen", "snapshot_slot", "chunk_summary",
           "combine_states", "decode_step", "workspace_bytes", "library_path", "KDAError"]


class KDAError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_abi.status_str(code)} (status {code})")
        self.code = code


def library_path() -> str:
    return _abi.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.KDA_BF16
    if t.dtype == torch.float32:
        return _abi.KDA_F32
    raise TypeError(f"KDA tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(ts, device):
    for name, t in ts.items():
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _out_code(dt) -> int:
    if dt == torch.float32:
        return _abi.KDA_F32
    if dt == torch.bfloat16:
        return _abi.KDA_BF16
    raise TypeError(f"out_dtype must be float32 or bfloat16, got {dt}")


def _prep_flags(clamp, qk_norm, gate_logits) -> int:
    f = 0 if clamp else _abi.KDA_FLAG_NO_CLAMP
    if qk_norm:
        f |= _abi.KDA_FLAG_QK_L2NORM
    if gate_logits:
        f |= _abi.KDA_FLAG_GATE_LOGITS
    return f


def _fwd_args(q, k, v, log_alpha, beta, gate, chunk, clamp, out_dtype):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape:
        raise ValueError("q, k, log_alpha must share the shape [B, T, H, Dk]")
    if v.shape != (B, T, H, Dv) or gate.shape != (B, T, H, Dv) or beta.shape != (B, T, H):
        raise ValueError("v, gate must be [B, T, H, Dv] and beta [B, T, H]")
    code = _dtype_code(q)
    for t in (k, v, log_alpha, beta, gate):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, log_alpha, beta and gate must share one dtype")
    a = _abi.FwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, Dk, Dv
    a.dtype, a.out_dtype, a.chunk = code, _out_code(out_dtype), int(chunk)
    a.flags = 0 if clamp else _abi.KDA_FLAG_NO_CLAMP
    return a


def workspace_bytes(B, T, H, D, dtype=torch.bfloat16, chunk=0) -> int:
    a = _abi.FwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, D, D
    a.dtype = _abi.KDA_BF16 if dtype == torch.bfloat16 else _abi.KDA_F32
    a.chunk = chunk
    n = ctypes.c_size_t(0)
    rc = _abi.load().kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_workspace_size")
    return int(n.value)


def chunk_fwd(q, k, v, log_alpha, beta, gate, initial_state=None, output_final_state=False,
              chunk=0, clamp=True, out_dtype=torch.float32, out=None, final_state=None,
              workspace=None, segment_scan=True, qk_norm=False, gate_logits=False, cards_ready=False,
              no_alloc=False):
    """Chunkwise-parallel KDA forward on the current HIP stream.

    q, k, log_alpha: [B, T, H, Dk]; v, gate: [B, T, H, Dv]; beta: [B, T, H];
    all bf16 or all fp32, contiguous, on one GPU.  initial_state: fp32
    [B, H, Dk, Dv] or None.  Returns (y, final_state or None); y has
    ``out_dtype`` (fp32 by default).  ``segment_scan=False`` keeps one sequential
    pass per (b, h) where the library would otherwise cut few, long sequences
    into segments (the same result up to rounding).  ``qk_norm``: q and k are raw
    projections, L2-normalised per token inside (q also scaled by 1/sqrt(Dk)).
    ``gate_logits``: ``log_alpha`` holds forget-gate logits x and the kernel uses
    max(logsigmoid(x), ln 0.0067).  ``cards_ready``: ``workspace`` already holds the
    cards of these inputs (from ``chunk_summary(..., q=q, workspace=workspace)``), so
    the card builder is skipped.  ``no_alloc``: call ``kda_chunk_fwd_noalloc``, which
    keeps the cards in the library's fixed per-device scratch instead of a workspace
    (``workspace`` must then be None; pass ``out`` and ``final_state`` too for a call
    that allocates nothing at all).
    """
    lib = _abi.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd needs GPU tensors (the HIP kernels are the only implementation)")
    a = _fwd_args(q, k, v, log_alpha, beta, gate, chunk, clamp, out_dtype)
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    if not segment_scan:
        a.flags |= _abi.KDA_FLAG_NO_SEGMENT_SCAN
    if cards_ready:
        if workspace is None:
            raise ValueError("cards_ready needs the workspace that holds the cards")
        a.flags |= _abi.KDA_FLAG_CARDS_READY
    B, T, H, Dk, Dv = a.B, a.T, a.H, a.Dk, a.Dv
    if initial_state is not None and (initial_state.dtype != torch.float32 or
                                      tuple(initial_state.shape) != (B, H, Dk, Dv)):
        raise ValueError("initial_state must be fp32 [B, H, Dk, Dv]")
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=out_dtype, device=dev)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, T, H, Dv):
        raise ValueError("out must be [B, T, H, Dv] of out_dtype")
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    if no_alloc:
        if workspace is not None or cards_ready:
            raise ValueError("no_alloc takes no workspace (the cards go to the library's scratch)")
    else:
        n = ctypes.c_size_t(0)
        rc = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
        if rc != _abi.KDA_OK:
            raise KDAError(rc, "kda_chunk_fwd_workspace_size")
        if workspace is None or workspace.numel() < n.value:
            workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    _check_dev(dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, gate=gate, out=out,
                    initial_state=initial_state, final_state=final_state), dev)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.log_alpha, a.beta, a.gate, a.out = _ptr(log_alpha), _ptr(beta), _ptr(gate), _ptr(out)
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state) if output_final_state else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    if no_alloc:
        rc = lib.kda_chunk_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(stream))
        if rc != _abi.KDA_OK:
            raise KDAError(rc, "kda_chunk_fwd_noalloc")
        return out, (final_state if output_final_state else None)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    rc = lib.kda_chunk_fwd(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd")
    return out, (final_state if output_final_state else None)


def snapshot_slot(cu_seqlens, i: int, k: int, snapshot_every: int) -> int:
    """Slot of the k-th snapshot of sequence i in ``chunk_fwd_varlen``'s snapshot tensor
    (host arithmetic on well-formed offsets): start_i // P + i + k."""
    return int(cu_seqlens[i]) // snapshot_every + i + k


def chunk_fwd_varlen(q, k, v, log_alpha, beta, gate, cu_seqlens, initial_state=None,
                     output_final_state=False, snapshot_every=0, clamp=True, out_dtype=torch.float32,
                     qk_norm=False, gate_logits=False, out=None, workspace=None, chunk=0):
    """Variable-length batch on the current HIP stream: N sequences packed along the
    rows of q, k, log_alpha [rows, H, Dk], v, gate [rows, H, Dv], beta [rows, H]
    (fp32 or bf16), sequence i being rows cu_seqlens[i] .. cu_seqlens[i+1] - 1 (int64
    device tensor [N + 1]); ``chunk`` as for ``chunk_fwd`` (0: the default).
    initial_state: fp32 [N, H, Dk, Dv] or None.  With ``snapshot_every`` P > 0 (a multiple of 64) the state after every P tokens of
    each sequence is returned in an fp32 [rows // P + N, H, Dk, Dv] tensor, the k-th
    of sequence i in slot ``snapshot_slot(cu_seqlens, i, k, P)``.  Returns
    (y [rows, H, Dv], final_state or None, snapshots or None); rows outside the
    sequences are left as they are in ``out``.
    """
    lib = _abi.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_varlen needs GPU tensors (the HIP kernels are the only implementation)")
    rows, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (rows, H, Dv) or \
            gate.shape != (rows, H, Dv) or beta.shape != (rows, H):
        raise ValueError("q, k, log_alpha must be [rows, H, Dk], v, gate [rows, H, Dv], beta [rows, H]")
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be an int64 vector [N + 1] on the same GPU")
    N = cu_seqlens.numel() - 1
    code = _dtype_code(q)
    for t in (k, v, log_alpha, beta, gate):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, log_alpha, beta and gate must share one dtype")
    if initial_state is not None and (initial_state.dtype != torch.float32 or
                                      tuple(initial_state.shape) != (N, H, Dk, Dv)):
        raise ValueError("initial_state must be fp32 [N, H, Dk, Dv]")
    if out is None:
        out = torch.empty((rows, H, Dv), dtype=out_dtype, device=dev)
    final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if output_final_state else None
    snaps = None
    if snapshot_every:
        snaps = torch.empty((rows // snapshot_every + N, H, Dk, Dv), dtype=torch.float32, device=dev)
    a = _abi.VarlenArgs()
    a.N, a.rows, a.H, a.Dk, a.Dv = N, rows, H, Dk, Dv
    a.dtype, a.out_dtype, a.chunk = code, _out_code(out_dtype), int(chunk)
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    a.snapshot_every = int(snapshot_every)
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_fwd_varlen_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_varlen_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    _check_dev(dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, gate=gate, out=out,
                    initial_state=initial_state, final_state=final, snapshots=snaps,
                    cu_seqlens=cu_seqlens), dev)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.log_alpha, a.beta, a.gate, a.out = _ptr(log_alpha), _ptr(beta), _ptr(gate), _ptr(out)
    a.initial_state, a.final_state, a.snapshots = _ptr(initial_state), _ptr(final), _ptr(snaps)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_fwd_varlen(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_varlen")
    return out, final, snaps


def chunk_summary(k, v, log_alpha, beta, clamp=True, transition=None, offset=None, workspace=None,
                  qk_norm=False, gate_logits=False, q=None, chunk=0):
    """Segment summary of every (b, h) sequence on the current HIP stream.

    The T tokens map an incoming state S to ``M @ S + b`` (``M`` the product of the
    per-token transitions, ``b`` the state reached from zero).  k, log_alpha:
    [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H] (fp32 or bf16, one dtype);
    ``chunk`` as for ``chunk_fwd``.  Returns ``(M, b)``: fp32 [B, H, Dk, Dk] and
    [B, H, Dk, Dv].  Given ``q`` (and a ``workspace``), with bf16 inputs and chunk 64
    the cards left in the workspace also serve a following
    ``chunk_fwd(..., workspace=workspace, cards_ready=True)`` over the same inputs.
    """
    lib = _abi.load()
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("chunk_summary needs GPU tensors (the HIP kernels are the only implementation)")
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    if log_alpha.shape != k.shape or v.shape != (B, T, H, Dv) or beta.shape != (B, T, H):
        raise ValueError("k, log_alpha must be [B, T, H, Dk], v [B, T, H, Dv] and beta [B, T, H]")
    code = _dtype_code(k)
    for t in (v, log_alpha, beta):
        if t.dtype != k.dtype:
            raise TypeError("k, v, log_alpha and beta must share one dtype")
    a = _abi.FwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv, a.dtype, a.chunk = B, T, H, Dk, Dv, code, int(chunk)
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    if transition is None:
        transition = torch.empty((B, H, Dk, Dk), dtype=torch.float32, device=dev)
    if offset is None:
        offset = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    if transition.dtype != torch.float32 or tuple(transition.shape) != (B, H, Dk, Dk):
        raise ValueError("transition must be fp32 [B, H, Dk, Dk]")
    if offset.dtype != torch.float32 or tuple(offset.shape) != (B, H, Dk, Dv):
        raise ValueError("offset must be fp32 [B, H, Dk, Dv]")
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    _check_dev(dict(k=k, v=v, log_alpha=log_alpha, beta=beta, transition=transition, offset=offset), dev)
    a.k, a.v, a.log_alpha, a.beta = _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta)
    if q is not None:
        if q.shape != k.shape or q.dtype != k.dtype or q.device != dev or not q.is_contiguous():
            raise ValueError("q must match k (shape, dtype, device) and be contiguous")
        a.q = _ptr(q)
    a.final_state = _ptr(offset)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_summary(ctypes.byref(a), _ptr(transition), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_summary")
    return transition, offset


def chunk_bwd(q, k, v, log_alpha, beta, gate, d_out, initial_state=None, d_final_state=None,
              clamp=True, workspace=None, need_initial_state_grad=True, qk_norm=False,
              gate_logits=False):
    """Gradients of ``sum(d_out * y) + sum(d_final_state * S_T)`` through ``chunk_fwd``
    (fp32 output, the same ``clamp``, ``qk_norm`` and ``gate_logits``), on the current
    HIP stream: with ``qk_norm`` those of the raw q and k, with ``gate_logits`` that of
    the logits.

    Inputs as for ``chunk_fwd``; ``d_out`` has their shape [B, T, H, Dv] and dtype.
    Returns a dict of fp32 tensors: dq, dk, dlog_alpha [B, T, H, Dk]; dv, dgate
    [B, T, H, Dv]; dbeta [B, T, H]; dinitial_state [B, H, Dk, Dv] (or None).
    """
    lib = _abi.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_bwd needs GPU tensors (the HIP kernels are the only implementation)")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (B, T, H, Dv) or \
            gate.shape != v.shape or d_out.shape != v.shape or beta.shape != (B, T, H):
        raise ValueError("q, k, log_alpha must be [B, T, H, Dk], v, gate, d_out [B, T, H, Dv], beta [B, T, H]")
    code = _dtype_code(q)
    for t in (k, v, log_alpha, beta, gate, d_out):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, log_alpha, beta, gate and d_out must share one dtype")
    st_shape = (B, H, Dk, Dv)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != st_shape):
            raise ValueError(f"{name} must be fp32 [B, H, Dk, Dv]")
    a = _abi.BwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv, a.dtype = B, T, H, Dk, Dv, code
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dq=torch.empty((B, T, H, Dk), **f32), dk=torch.empty((B, T, H, Dk), **f32),
             dv=torch.empty((B, T, H, Dv), **f32), dlog_alpha=torch.empty((B, T, H, Dk), **f32),
             dbeta=torch.empty((B, T, H), **f32), dgate=torch.empty((B, T, H, Dv), **f32),
             dinitial_state=torch.empty(st_shape, **f32) if need_initial_state_grad else None)
    _check_dev(dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, gate=gate, d_out=d_out,
                    initial_state=initial_state, d_final_state=d_final_state), dev)
    a.q, a.k, a.v, a.log_alpha, a.beta, a.gate = (_ptr(t) for t in (q, k, v, log_alpha, beta, gate))
    a.d_out, a.initial_state, a.d_final_state = _ptr(d_out), _ptr(initial_state), _ptr(d_final_state)
    a.dq, a.dk, a.dv, a.dlog_alpha = _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"])
    a.dbeta, a.dgate, a.d_initial_state = _ptr(g["dbeta"]), _ptr(g["dgate"]), _ptr(g["dinitial_state"])
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_bwd(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd")
    return g


def chunk_bwd_varlen(q, k, v, log_alpha, beta, gate, d_out, cu_seqlens, initial_state=None,
                     d_final_state=None, clamp=True, workspace=None, need_initial_state_grad=True,
                     qk_norm=False, gate_logits=False):
    """Gradients of ``sum(d_out * y) + sum(d_final_state * S_T)`` through
    ``chunk_fwd_varlen`` (fp32 output, the same ``clamp``, ``qk_norm`` and
    ``gate_logits``) on the current HIP stream, for N sequences packed along the rows:
    q, k, log_alpha [rows, H, Dk], v, gate, d_out [rows, H, Dv], beta [rows, H] (fp32
    or bf16, one dtype), sequence i being rows cu_seqlens[i] .. cu_seqlens[i+1] - 1
    (int64 device tensor [N + 1]).  initial_state, d_final_state: fp32 [N, H, Dk, Dv]
    or None.  Returns a dict of fp32 tensors: dq, dk, dlog_alpha [rows, H, Dk]; dv,
    dgate [rows, H, Dv]; dbeta [rows, H] (zero on rows outside the sequences);
    dinitial_state [N, H, Dk, Dv] (or None).
    """
    lib = _abi.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_bwd_varlen needs GPU tensors (the HIP kernels are the only implementation)")
    rows, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (rows, H, Dv) or \
            gate.shape != v.shape or d_out.shape != v.shape or beta.shape != (rows, H):
        raise ValueError("q, k, log_alpha must be [rows, H, Dk], v, gate, d_out [rows, H, Dv], beta [rows, H]")
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
        raise ValueError("cu_seqlens must be an int64 vector [N + 1] on the same GPU")
    N = cu_seqlens.numel() - 1
    code = _dtype_code(q)
    for t in (k, v, log_alpha, beta, gate, d_out):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, log_alpha, beta, gate and d_out must share one dtype")
    st_shape = (N, H, Dk, Dv)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != st_shape):
            raise ValueError(f"{name} must be fp32 [N, H, Dk, Dv]")
    a = _abi.BwdVarlenArgs()
    a.N, a.rows, a.H, a.Dk, a.Dv, a.dtype = N, rows, H, Dk, Dv, code
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_bwd_varlen_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd_varlen_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    # zeros: rows outside the sequences are not written
    g = dict(dq=torch.zeros((rows, H, Dk), **f32), dk=torch.zeros((rows, H, Dk), **f32),
             dv=torch.zeros((rows, H, Dv), **f32), dlog_alpha=torch.zeros((rows, H, Dk), **f32),
             dbeta=torch.zeros((rows, H), **f32), dgate=torch.zeros((rows, H, Dv), **f32),
             dinitial_state=torch.empty(st_shape, **f32) if need_initial_state_grad else None)
    _check_dev(dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, gate=gate, d_out=d_out,
                    initial_state=initial_state, d_final_state=d_final_state, cu_seqlens=cu_seqlens), dev)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.q, a.k, a.v, a.log_alpha, a.beta, a.gate = (_ptr(t) for t in (q, k, v, log_alpha, beta, gate))
    a.d_out, a.initial_state, a.d_final_state = _ptr(d_out), _ptr(initial_state), _ptr(d_final_state)
    a.dq, a.dk, a.dv, a.dlog_alpha = _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"])
    a.dbeta, a.dgate, a.d_initial_state = _ptr(g["dbeta"]), _ptr(g["dgate"]), _ptr(g["dinitial_state"])
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_bwd_varlen(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_chunk_bwd_varlen")
    return g


def combine_states(transition, offset, initial_state=None, segment_states=True, final_state=None):
    """Ordered combination of P segment summaries on the current HIP stream:
    S_{p+1} = M_p S_p + b_p from S_0 = ``initial_state`` (zeros when None).

    transition: fp32 [P, B, H, Dk, Dk]; offset: fp32 [P, B, H, Dk, Dv].  Returns
    ``(segment_states or None, final_state)``: the state entering each segment,
    [P, B, H, Dk, Dv], and the state after the last, [B, H, Dk, Dv].
    """
    lib = _abi.load()
    dev = transition.device
    if dev.type != "cuda":
        raise ValueError("combine_states needs GPU tensors (the HIP kernels are the only implementation)")
    P, B, H, Dk, _ = transition.shape
    Dv = offset.shape[-1]
    for name, t, shape in (("transition", transition, (P, B, H, Dk, Dk)), ("offset", offset, (P, B, H, Dk, Dv)),
                           ("initial_state", initial_state, (B, H, Dk, Dv)),
                           ("final_state", final_state, (B, H, Dk, Dv))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape):
            raise ValueError(f"{name} must be fp32 {list(shape)}")
    seg = torch.empty((P, B, H, Dk, Dv), dtype=torch.float32, device=dev) if segment_states else None
    if final_state is None:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    _check_dev(dict(transition=transition, offset=offset, initial_state=initial_state,
                    segment_states=seg, final_state=final_state), dev)
    a = _abi.CombineArgs()
    a.P, a.B, a.H, a.Dk, a.Dv = P, B, H, Dk, Dv
    a.transition, a.offset = _ptr(transition), _ptr(offset)
    a.initial_state, a.segment_states, a.final_state = _ptr(initial_state), _ptr(seg), _ptr(final_state)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_combine_states(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_combine_states")
    return seg, final_state


def decode_step(q, k, v, log_alpha, beta, gate, state, clamp=True, out_dtype=torch.float32,
                out=None, qk_norm=False, gate_logits=False):
    """One recurrent KDA token per (b, h) on the current HIP stream.

    q, k, log_alpha: [B, H, Dk]; v, gate: [B, H, Dv]; beta: [B, H]; state: fp32
    [B, H, Dk, Dv], updated in place.  Returns y [B, H, Dv].
    """
    lib = _abi.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step needs GPU tensors (the HIP kernels are the only implementation)")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, Dk, Dv):
        raise ValueError("state must be fp32 [B, H, Dk, Dv]")
    code = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=out_dtype, device=dev)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, H, Dv):
        raise ValueError("out must be [B, H, Dv] of out_dtype")
    _check_dev(dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, gate=gate, state=state, out=out), dev)
    a = _abi.DecodeArgs()
    a.B, a.H, a.Dk, a.Dv, a.dtype, a.out_dtype = B, H, Dk, Dv, code, _out_code(out_dtype)
    a.flags = _prep_flags(clamp, qk_norm, gate_logits)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.log_alpha, a.beta, a.gate = _ptr(log_alpha), _ptr(beta), _ptr(gate)
    a.out, a.state = _ptr(out), _ptr(state)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_decode_step(ctypes.byref(a), ctypes.c_void_p(stream))
    if rc != _abi.KDA_OK:
        raise KDAError(rc, "kda_decode_step")
    return out
