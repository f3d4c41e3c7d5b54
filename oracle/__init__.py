"""fp64 CPU oracle for the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library under
``gated_delta_rule_106_amd`` and its binding) never imports it, and the two
share no code.

The arithmetic lives in ``kda_oracle.c``: the plain token-by-token recurrence
of Kimi Delta Attention in double precision (page "3T models are no longer
magic", section "Gate 1: KDA makes it computable": forget per channel, delta
rule corrective write, read the new state with the query, sigmoid output
gate), and the segment summary of a run of tokens (same page, section "KDA
context parallelism").  This module builds that file with gcc and marshals
arguments; the one computation done here is ``combine``, the ordered
composition of segment summaries, written as a plain fp64 matrix product per
segment.

Every input is passed as the exact bit pattern the GPU receives (float32 or
bfloat16) and is widened exactly inside the C code; nothing here rounds,
normalises or rescales.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

ORC_F32 = 0
ORC_BF16 = 1
LOG_ALPHA_MIN = -5.005647752585217  # ln 0.0067, the per-step retention floor


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP)."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _open(path):
    lib = ctypes.CDLL(path)
    i64, vp, dp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp,
                                   dp, dp, dp, ci, ci]
    lib.kda_oracle_fwd.restype = ci
    lib.kda_oracle_fwd_ex.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp,
                                      dp, dp, dp, ci, ci, ci, ci]
    lib.kda_oracle_fwd_ex.restype = ci
    lib.kda_oracle_decode.argtypes = [i64, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp,
                                      dp, dp, ci, ci, ci, ci]
    lib.kda_oracle_decode.restype = ci
    lib.kda_oracle_summary.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, vp, dp, dp, ci, ci, ci, ci]
    lib.kda_oracle_summary.restype = ci
    lib.kda_oracle_bwd.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp, dp, dp, dp,
                                   dp, dp, dp, dp, dp, dp, dp, ci, ci]
    lib.kda_oracle_bwd.restype = ci
    lib.kda_oracle_bwd_ex.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, vp, vp, vp, dp, dp, dp,
                                      dp, dp, dp, dp, dp, dp, dp, ci, ci, ci, ci]
    lib.kda_oracle_bwd_ex.restype = ci
    lib.kda_oracle_default_threads.argtypes = []
    lib.kda_oracle_default_threads.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _open(_LIB_PATH)
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile a (modified) copy of the oracle source to ``out_path`` and return a
    handle whose ``fwd``/``decode`` behave like this module's.  Used by the tests
    that plant mistakes in the oracle and check that the pins catch them."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-shared", "-fPIC", src, "-o", out_path, "-lm"], check=True)
    lib = _open(out_path)

    class _Handle:
        def fwd(self, *a, **kw):
            return fwd(*a, _lib_handle=lib, **kw)

        def decode(self, *a, **kw):
            return decode(*a, _lib_handle=lib, **kw)

        def summary(self, *a, **kw):
            return summary(*a, _lib_handle=lib, **kw)

        def bwd(self, *a, **kw):
            return bwd(*a, _lib_handle=lib, **kw)
    return _Handle()


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def default_threads() -> int:
    return int(_load().kda_oracle_default_threads())


def _raw(x):
    """Return (contiguous numpy array of raw bits, dtype code) for a CPU tensor/array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), ORC_BF16
            if x.dtype == torch.float32:
                return np.ascontiguousarray(x.numpy()), ORC_F32
            raise TypeError(f"oracle accepts float32 or bfloat16 tensors, got {x.dtype}")
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    x = np.asarray(x)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), ORC_F32
    if x.dtype == np.uint16:  # raw bfloat16 bits
        return np.ascontiguousarray(x), ORC_BF16
    raise TypeError(f"oracle accepts float32 arrays or uint16 bfloat16 bits, got {x.dtype}")


def _state64(s, shape):
    if s is None:
        return None
    try:
        import torch
        if isinstance(s, torch.Tensor):
            s = s.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
    if s.shape != tuple(shape):
        raise ValueError(f"state shape {s.shape} != {tuple(shape)}")
    return s


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, log_alpha, beta, gate, initial_state=None, clamp=True, threads=0,
        return_seconds=False, qk_norm=False, gate_logits=False, _lib_handle=None):
    """Sequential fp64 recurrence over [B, T, H].

    ``qk_norm``: q and k are raw; each token's k is divided by its L2 norm and q
    by its L2 norm times sqrt(d_k).  ``gate_logits``: log_alpha holds forget-gate
    logits x and log alpha = logsigmoid(x) (then the floor clamp as usual).

    Returns ``(y, final_state)`` as float64 numpy arrays of shapes [B, T, H, Dv]
    and [B, H, Dk, Dv] (and the wall time of the C call when
    ``return_seconds``).
    """
    qa, dt = _raw(q)
    ka, dt_k = _raw(k)
    va, dt_v = _raw(v)
    la, dt_l = _raw(log_alpha)
    ba, dt_b = _raw(beta)
    ga, dt_g = _raw(gate)
    if len({dt, dt_k, dt_v, dt_l, dt_b, dt_g}) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    B, T, H, Dk = qa.shape
    Dv = va.shape[-1]
    if ka.shape != (B, T, H, Dk) or la.shape != (B, T, H, Dk):
        raise ValueError("q, k, log_alpha must be [B, T, H, Dk]")
    if va.shape != (B, T, H, Dv) or ga.shape != (B, T, H, Dv) or ba.shape != (B, T, H):
        raise ValueError("v, gate must be [B, T, H, Dv] and beta [B, T, H]")
    s0 = _state64(initial_state, (B, H, Dk, Dv))
    y = np.zeros((B, T, H, Dv), dtype=np.float64)
    sT = np.zeros((B, H, Dk, Dv), dtype=np.float64)
    t0 = time.perf_counter()
    lib = _lib_handle if _lib_handle is not None else _load()
    rc = lib.kda_oracle_fwd_ex(B, T, H, Dk, Dv, dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(la),
                               _ptr(ba), _ptr(ga), _ptr(s0), _ptr(y), _ptr(sT),
                               1 if clamp else 0, 1 if qk_norm else 0, 1 if gate_logits else 0,
                               int(threads))
    secs = time.perf_counter() - t0
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    return (y, sT, secs) if return_seconds else (y, sT)


def decode(q, k, v, log_alpha, beta, gate, state, clamp=True, threads=0, qk_norm=False,
           gate_logits=False, _lib_handle=None):
    """One recurrent step for every (b, h): inputs [B, H, D], beta [B, H].

    ``state`` is [B, H, Dk, Dv] (any float type); returns ``(y, new_state)`` in
    float64 without modifying the argument.
    """
    qa, dt = _raw(q)
    ka, _ = _raw(k)
    va, _ = _raw(v)
    la, _ = _raw(log_alpha)
    ba, _ = _raw(beta)
    ga, _ = _raw(gate)
    B, H, Dk = qa.shape
    Dv = va.shape[-1]
    s = _state64(state, (B, H, Dk, Dv)).copy()
    y = np.zeros((B, H, Dv), dtype=np.float64)
    lib = _lib_handle if _lib_handle is not None else _load()
    rc = lib.kda_oracle_decode(B, H, Dk, Dv, dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(la),
                               _ptr(ba), _ptr(ga), _ptr(s), _ptr(y), 1 if clamp else 0,
                               1 if qk_norm else 0, 1 if gate_logits else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode failed with code {rc}")
    return y, s


def summary(k, v, log_alpha, beta, clamp=True, threads=0, qk_norm=False, gate_logits=False,
            _lib_handle=None):
    """Segment summary of every (b, h) run over [B, T, H] (page "3T models are no
    longer magic", section "KDA context parallelism"): the run maps an incoming
    state S to ``M @ S + b``, with ``M`` the product of the per-token transitions
    (I - beta k k^T) Diag(alpha), latest on the left, and ``b`` the state reached
    from zero.  Returns ``(M, b)`` as float64 arrays [B, H, Dk, Dk], [B, H, Dk, Dv].
    """
    ka, dt = _raw(k)
    va, dt_v = _raw(v)
    la, dt_l = _raw(log_alpha)
    ba, dt_b = _raw(beta)
    if len({dt, dt_v, dt_l, dt_b}) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    B, T, H, Dk = ka.shape
    Dv = va.shape[-1]
    if la.shape != (B, T, H, Dk) or va.shape != (B, T, H, Dv) or ba.shape != (B, T, H):
        raise ValueError("k, log_alpha must be [B, T, H, Dk], v [B, T, H, Dv], beta [B, T, H]")
    M = np.zeros((B, H, Dk, Dk), dtype=np.float64)
    b = np.zeros((B, H, Dk, Dv), dtype=np.float64)
    lib = _lib_handle if _lib_handle is not None else _load()
    rc = lib.kda_oracle_summary(B, T, H, Dk, Dv, dt, _ptr(ka), _ptr(va), _ptr(la), _ptr(ba),
                                _ptr(M), _ptr(b), 1 if clamp else 0, 1 if qk_norm else 0,
                                1 if gate_logits else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_summary failed with code {rc}")
    return M, b


def combine(M, b, initial_state=None):
    """Ordered composition of P consecutive segment summaries (page "Kimi K3
    report walk-through", section "KDA Context Parallelism": the state handed to
    segment p + 1 is what segment p makes of the state it received).

    ``M`` is [P, B, H, Dk, Dk] and ``b`` [P, B, H, Dk, Dv]; the state entering
    segment 0 is ``initial_state`` (zeros when None).  Returns
    ``(segment_states, final_state)``: the state entering each segment,
    [P, B, H, Dk, Dv], and the state after the last one, [B, H, Dk, Dv], all
    float64.  S_{p+1} = M_p S_p + b_p, one matrix product per segment.
    """
    M = np.asarray(M, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    P, B, H, Dk, _ = M.shape
    Dv = b.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if initial_state is None else _state64(initial_state, (B, H, Dk, Dv)).copy()
    seg = np.zeros((P, B, H, Dk, Dv))
    for p in range(P):
        seg[p] = S
        S = np.matmul(M[p], S) + b[p]
    return seg, S


def bwd(q, k, v, log_alpha, beta, gate, dy, initial_state=None, d_final_state=None, clamp=True,
        threads=0, qk_norm=False, gate_logits=False, _lib_handle=None):
    """Gradients of L = sum(dy * y) + sum(d_final_state * S_T) for the forward above
    (reverse mode through the token steps; page "3T models are no longer magic",
    section "Gate 1: KDA makes it computable", taken backwards).

    Returns a dict of float64 arrays: dq, dk, dlog_alpha [B, T, H, Dk]; dv, dgate
    [B, T, H, Dv]; dbeta [B, T, H]; dinitial_state [B, H, Dk, Dv].  Keeps every
    state of a sequence: small cases only.  ``qk_norm`` / ``gate_logits``: the inputs
    are raw (as in ``fwd``) and dq, dk, dlog_alpha are the gradients with respect to
    the raw q, k and forget logits.
    """
    qa, dt = _raw(q)
    ka, _ = _raw(k)
    va, _ = _raw(v)
    la, _ = _raw(log_alpha)
    ba, _ = _raw(beta)
    ga, _ = _raw(gate)
    B, T, H, Dk = qa.shape
    Dv = va.shape[-1]
    s0 = _state64(initial_state, (B, H, Dk, Dv))
    dST = _state64(d_final_state, (B, H, Dk, Dv))
    dya = np.ascontiguousarray(np.asarray(dy, dtype=np.float64))
    if dya.shape != (B, T, H, Dv):
        raise ValueError("dy must be [B, T, H, Dv]")
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
               dlog_alpha=np.zeros((B, T, H, Dk)), dbeta=np.zeros((B, T, H)),
               dgate=np.zeros((B, T, H, Dv)), dinitial_state=np.zeros((B, H, Dk, Dv)))
    lib = _lib_handle if _lib_handle is not None else _load()
    rc = lib.kda_oracle_bwd_ex(B, T, H, Dk, Dv, dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(la), _ptr(ba),
                               _ptr(ga), _ptr(s0), _ptr(dya), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]),
                               _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                               _ptr(out["dgate"]), _ptr(out["dinitial_state"]), 1 if clamp else 0,
                               1 if qk_norm else 0, 1 if gate_logits else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed with code {rc}")
    return out
