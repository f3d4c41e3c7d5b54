"""The C-ABI library: it loads, exports every symbol include/kda.h declares, its
structs match the header byte for byte, and host-side validation rejects bad
arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_106_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(kda_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_abi.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings(lib):
    assert lib.kda_version() == 5
    for code in range(-7, 1):
        assert lib.kda_status_str(code).decode()
    assert lib.kda_status_str(12345).decode() == "unknown status"


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "kda.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu ", sizeof(kda_fwd_args), offsetof(kda_fwd_args, q),
         offsetof(kda_fwd_args, workspace_bytes), sizeof(kda_decode_args),
         offsetof(kda_decode_args, q), offsetof(kda_decode_args, state),
         sizeof(kda_combine_args), offsetof(kda_combine_args, transition),
         offsetof(kda_combine_args, final_state));
  printf("%zu %zu %zu %zu ", sizeof(kda_varlen_args), offsetof(kda_varlen_args, cu_seqlens),
         offsetof(kda_varlen_args, snapshot_every), offsetof(kda_varlen_args, workspace_bytes));
  printf("%zu %zu %zu %zu %zu ", sizeof(kda_bwd_args), offsetof(kda_bwd_args, q),
         offsetof(kda_bwd_args, d_final_state), offsetof(kda_bwd_args, d_initial_state),
         offsetof(kda_bwd_args, workspace_bytes));
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(kda_bwd_varlen_args), offsetof(kda_bwd_varlen_args, cu_seqlens),
         offsetof(kda_bwd_varlen_args, q), offsetof(kda_bwd_varlen_args, d_final_state),
         offsetof(kda_bwd_varlen_args, d_initial_state), offsetof(kda_bwd_varlen_args, workspace_bytes));
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                    "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(_abi.FwdArgs), _abi.FwdArgs.q.offset, _abi.FwdArgs.workspace_bytes.offset,
            ctypes.sizeof(_abi.DecodeArgs), _abi.DecodeArgs.q.offset, _abi.DecodeArgs.state.offset,
            ctypes.sizeof(_abi.CombineArgs), _abi.CombineArgs.transition.offset,
            _abi.CombineArgs.final_state.offset,
            ctypes.sizeof(_abi.VarlenArgs), _abi.VarlenArgs.cu_seqlens.offset,
            _abi.VarlenArgs.snapshot_every.offset, _abi.VarlenArgs.workspace_bytes.offset,
            ctypes.sizeof(_abi.BwdArgs), _abi.BwdArgs.q.offset, _abi.BwdArgs.d_final_state.offset,
            _abi.BwdArgs.d_initial_state.offset, _abi.BwdArgs.workspace_bytes.offset,
            ctypes.sizeof(_abi.BwdVarlenArgs), _abi.BwdVarlenArgs.cu_seqlens.offset, _abi.BwdVarlenArgs.q.offset,
            _abi.BwdVarlenArgs.d_final_state.offset, _abi.BwdVarlenArgs.d_initial_state.offset,
            _abi.BwdVarlenArgs.workspace_bytes.offset]
    assert got == want


def _good_fwd(B=1, T=64, H=2, D=128, dtype=_abi.KDA_BF16, chunk=0):
    a = _abi.FwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv, a.dtype, a.chunk = B, T, H, D, D, dtype, chunk
    fake = 0x10000  # aligned, never dereferenced: every case below fails validation first
    for f in ("q", "k", "v", "log_alpha", "beta", "gate", "out"):
        setattr(a, f, fake)
    return a


def _ws(lib, a):
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return rc, n.value


def test_workspace_size_query(lib):
    a = _good_fwd(B=1, T=4096, H=8)
    rc, n = _ws(lib, a)
    assert rc == 0
    # one card per (b, h, chunk): 5 fp16 C x D tiles + fp32 Gamma
    assert n == 8 * 64 * (5 * 64 * 128 * 2 + 128 * 4)
    a.T = 4095
    assert _ws(lib, a) == (0, n)  # ragged tail still needs 64 chunks
    a.T = 0
    assert _ws(lib, a) == (0, 0)
    a32 = _good_fwd(B=1, T=256, H=2, D=64, dtype=_abi.KDA_F32, chunk=16)
    assert _ws(lib, a32) == (0, 2 * 16 * (5 * 16 * 64 * 4 + 64 * 4))
    assert lib.kda_chunk_fwd_workspace_size(None, None) == _abi.KDA_ERR_NULL


def test_workspace_size_includes_segment_summaries(lib):
    """A single long sequence takes the segment scan: the workspace adds, per summarised
    segment, the zero-start end state and the transition (fp32 Dk x Dv each); shapes
    with enough (b, h) sequences or short ones add nothing."""
    card = 5 * 64 * 128 * 2 + 128 * 4
    a = _good_fwd(B=1, T=8192, H=1, D=128)
    assert _ws(lib, a)[1] == 128 * card + 3 * 2 * 128 * 128 * 4  # 4 segments of 32 chunks
    a = _good_fwd(B=1, T=32768, H=2, D=128)
    assert _ws(lib, a)[1] == 2 * 512 * card + 2 * 7 * 2 * 128 * 128 * 4  # 8 segments
    a = _good_fwd(B=2, T=65536, H=32, D=128)
    assert _ws(lib, a)[1] == 64 * 1024 * card
    a = _good_fwd(B=1, T=4096, H=8, D=128)
    assert _ws(lib, a)[1] == 8 * 64 * card


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "B", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "T", -5), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "Dk", 0), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "Dk", 96), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: (setattr(a, "Dk", 64)), _abi.KDA_ERR_UNSUPPORTED),  # Dk != Dv
    (lambda a: setattr(a, "dtype", 7), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "chunk", 48), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "chunk", 128), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 32), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 31), _abi.KDA_ERR_WORKSPACE),  # every known flag: accepted
    (lambda a: (setattr(a, "flags", 16), setattr(a, "chunk", 32)), _abi.KDA_ERR_UNSUPPORTED),  # cards: chunk 64
    (lambda a: (setattr(a, "flags", 16), setattr(a, "dtype", _abi.KDA_F32), setattr(a, "chunk", 16)),
     _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "out_dtype", 2), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "T", 2 ** 62), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "q", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "gate", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "out", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "v", 0x10008), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "initial_state", 0x10004), _abi.KDA_ERR_ALIGN),
    (lambda a: None, _abi.KDA_ERR_WORKSPACE),  # no workspace given
    (lambda a: (setattr(a, "workspace", 0x20000), setattr(a, "workspace_bytes", 100)),
     _abi.KDA_ERR_WORKSPACE),
])
def test_fwd_validation_rejects_before_any_hip_call(lib, mutate, code):
    a = _good_fwd()
    mutate(a)
    assert lib.kda_chunk_fwd(ctypes.byref(a), None) == code


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "B", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "Dk", 96), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "chunk", 128), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 16), _abi.KDA_ERR_UNSUPPORTED),  # the shared scratch holds no known cards
    (lambda a: setattr(a, "q", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "v", 0x10008), _abi.KDA_ERR_ALIGN),
    # B1 H16 T65536: 16384 cards of 82 432 B, far beyond the fixed buffer
    (lambda a: (setattr(a, "H", 16), setattr(a, "T", 65536)), _abi.KDA_ERR_TOO_LARGE),
    # 815 cards of five chunks (too short for segments): one more than the buffer holds
    (lambda a: (setattr(a, "H", 163), setattr(a, "T", 5 * 64)), _abi.KDA_ERR_TOO_LARGE),
])
def test_noalloc_validation_rejects_before_any_hip_call(lib, mutate, code):
    a = _good_fwd()
    mutate(a)
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(a), None) == code


def test_noalloc_limit_and_empty_calls(lib):
    """The fixed buffer holds 814 chunk-64 cards at d = 128 (one card is 82 432 B); the
    workspace query of the ordinary call is what is compared against it.  Empty calls
    return before any HIP call."""
    card = 5 * 64 * 128 * 2 + 128 * 4
    assert _abi.KDA_NOALLOC_SCRATCH_BYTES // card == 814
    assert _ws(lib, _good_fwd(B=1, T=4096, H=8, D=128))[1] <= _abi.KDA_NOALLOC_SCRATCH_BYTES
    assert _ws(lib, _good_fwd(B=1, T=5 * 64, H=162, D=128))[1] == 810 * card
    assert _ws(lib, _good_fwd(B=1, T=5 * 64, H=163, D=128))[1] > _abi.KDA_NOALLOC_SCRATCH_BYTES
    f = _good_fwd(B=0)
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(f), None) == 0
    f = _good_fwd(T=0)  # no final state requested: nothing to do
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(f), None) == 0
    assert lib.kda_chunk_fwd_noalloc(None, None) == _abi.KDA_ERR_NULL


def test_fp32_chunk64_d128_is_unsupported(lib):
    a = _good_fwd(dtype=_abi.KDA_F32, chunk=64)
    assert _ws(lib, a)[0] == _abi.KDA_ERR_UNSUPPORTED
    assert lib.kda_chunk_fwd(None, None) == _abi.KDA_ERR_NULL


def _good_dec():
    a = _abi.DecodeArgs()
    a.B, a.H, a.Dk, a.Dv, a.dtype = 4, 2, 128, 128, _abi.KDA_BF16
    for f in ("q", "k", "v", "log_alpha", "beta", "gate", "out", "state"):
        setattr(a, f, 0x10000)
    return a


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "H", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "Dv", 64), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dtype", 3), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 16), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 2), _abi.KDA_ERR_UNSUPPORTED),  # no segments in a decode step
    (lambda a: (setattr(a, "flags", 13), setattr(a, "state", None)), _abi.KDA_ERR_NULL),  # flags accepted
    (lambda a: setattr(a, "reserved", 1), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "out_dtype", -1), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "state", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "beta", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "k", 0x10002), _abi.KDA_ERR_ALIGN),
])
def test_decode_validation(lib, mutate, code):
    a = _good_dec()
    mutate(a)
    assert lib.kda_decode_step(ctypes.byref(a), None) == code


def test_empty_problems_are_no_ops(lib):
    a = _good_dec()
    a.B = 0
    assert lib.kda_decode_step(ctypes.byref(a), None) == 0
    f = _good_fwd(B=0)
    assert lib.kda_chunk_fwd(ctypes.byref(f), None) == 0
    f = _good_fwd(T=0)  # no final state requested: nothing to do
    assert lib.kda_chunk_fwd(ctypes.byref(f), None) == 0


def _good_sum():
    a = _good_fwd(T=300, H=2)
    a.final_state = 0x30000
    return a


@pytest.mark.parametrize("mutate,code", [
    # every path kda_chunk_fwd takes: fp32 inputs and chunks of 16 / 32 are accepted
    (lambda a: setattr(a, "dtype", _abi.KDA_F32), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "chunk", 32), _abi.KDA_ERR_WORKSPACE),
    (lambda a: (setattr(a, "dtype", _abi.KDA_F32), setattr(a, "chunk", 64)), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "chunk", 128), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_NO_SEGMENT_SCAN), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_CARDS_READY), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 16), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 13), _abi.KDA_ERR_WORKSPACE),  # clamp off, q/k norm, logits: accepted
    (lambda a: setattr(a, "Dk", 96), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "T", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "final_state", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "final_state", 0x30008), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "k", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "beta", 0x10002), _abi.KDA_ERR_ALIGN),
    (lambda a: None, _abi.KDA_ERR_WORKSPACE),  # no workspace given
    (lambda a: (setattr(a, "workspace", 0x20000), setattr(a, "workspace_bytes", 4096)),
     _abi.KDA_ERR_WORKSPACE),
])
def test_summary_validation(lib, mutate, code):
    a = _good_sum()
    a.q = a.gate = a.out = None  # not read by the summary
    mutate(a)
    assert lib.kda_chunk_summary(ctypes.byref(a), ctypes.c_void_p(0x40000), None) == code


def test_summary_needs_transition_and_empty_batch_is_a_no_op(lib):
    a = _good_sum()
    assert lib.kda_chunk_summary(ctypes.byref(a), None, None) == _abi.KDA_ERR_NULL
    assert lib.kda_chunk_summary(ctypes.byref(a), ctypes.c_void_p(0x40004), None) == _abi.KDA_ERR_ALIGN
    assert lib.kda_chunk_summary(None, None, None) == _abi.KDA_ERR_NULL
    a.H = 0
    assert lib.kda_chunk_summary(ctypes.byref(a), None, None) == 0


def _good_comb():
    a = _abi.CombineArgs()
    a.P, a.B, a.H, a.Dk, a.Dv = 4, 1, 8, 128, 128
    a.transition, a.offset, a.final_state = 0x10000, 0x20000, 0x30000
    return a


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "P", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "H", -2), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "P", 2 ** 60), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "Dv", 64), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: (setattr(a, "Dk", 32), setattr(a, "Dv", 32)), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "transition", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "offset", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "initial_state", 0x40004), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "segment_states", 0x50008), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "final_state", None), _abi.KDA_OK),  # no output requested: nothing to do
    (lambda a: setattr(a, "B", 0), _abi.KDA_OK),
])
def test_combine_validation(lib, mutate, code):
    a = _good_comb()
    mutate(a)
    assert lib.kda_combine_states(ctypes.byref(a), None) == code
    assert lib.kda_combine_states(None, None) == _abi.KDA_ERR_NULL


def _good_var():
    a = _abi.VarlenArgs()
    a.N, a.rows, a.H, a.Dk, a.Dv, a.dtype = 3, 1000, 2, 128, 128, _abi.KDA_BF16
    for f in ("cu_seqlens", "q", "k", "v", "log_alpha", "beta", "gate", "out"):
        setattr(a, f, 0x10000)
    return a


def test_varlen_workspace_size(lib):
    a = _good_var()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_varlen_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    card = 5 * 64 * 128 * 2 + 128 * 4
    chunks = (1000 + 63) // 64 + 3  # the most chunks any offsets can give
    r256 = lambda x: (x + 255) // 256 * 256
    assert n.value == r256(chunks * 2 * card) + 2 * r256(4 * 8) + r256(chunks * 4)
    # the general path (fp32 inputs, default chunk 16; bf16 with chunk 32): one card per
    # chunk of its size, as kda_chunk_fwd sizes a one-chunk call
    for dtype, chunk, c in ((_abi.KDA_F32, 0, 16), (_abi.KDA_BF16, 32, 32)):
        a = _good_var()
        a.dtype, a.chunk = dtype, chunk
        assert lib.kda_chunk_fwd_varlen_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
        one = _good_fwd(B=1, T=c, H=1, D=128, dtype=dtype, chunk=c)
        rc, card = _ws(lib, one)
        assert rc == 0
        chunks = (1000 + c - 1) // c + 3
        assert n.value == r256(chunks * 2 * card) + 2 * r256(4 * 8) + r256(chunks * 4)


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "N", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "rows", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "snapshot_every", -64), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "snapshot_every", 100), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dtype", 7), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "chunk", 48), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: (setattr(a, "dtype", _abi.KDA_F32), setattr(a, "chunk", 64)), _abi.KDA_ERR_UNSUPPORTED),
    # fp32 inputs and the general path's chunk sizes are accepted: the workspace check decides
    (lambda a: setattr(a, "dtype", _abi.KDA_F32), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "chunk", 32), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "Dv", 64), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 16), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "cu_seqlens", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "cu_seqlens", 0x10004), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "gate", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "snapshot_every", 128), _abi.KDA_ERR_NULL),  # no snapshot buffer
    (lambda a: setattr(a, "final_state", 0x10008), _abi.KDA_ERR_ALIGN),
    (lambda a: None, _abi.KDA_ERR_WORKSPACE),
    (lambda a: (setattr(a, "workspace", 0x20000), setattr(a, "workspace_bytes", 4096)), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "N", 0), _abi.KDA_OK),
    (lambda a: setattr(a, "H", 0), _abi.KDA_OK),
])
def test_varlen_validation(lib, mutate, code):
    a = _good_var()
    mutate(a)
    assert lib.kda_chunk_fwd_varlen(ctypes.byref(a), None) == code
    assert lib.kda_chunk_fwd_varlen(None, None) == _abi.KDA_ERR_NULL


def test_binding_refuses_cpu_tensors():
    import torch
    import gated_delta_rule_106_amd as kda
    x = torch.zeros(1, 16, 1, 64)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 16, 1), x)
    with pytest.raises(ValueError):
        kda.decode_step(x[:, 0], x[:, 0], x[:, 0], x[:, 0], torch.zeros(1, 1), x[:, 0],
                        torch.zeros(1, 1, 64, 64))
    with pytest.raises(ValueError):
        kda.chunk_summary(x, x, x, torch.zeros(1, 16, 1))
    with pytest.raises(ValueError):
        kda.combine_states(torch.zeros(2, 1, 1, 64, 64), torch.zeros(2, 1, 1, 64, 64))
    with pytest.raises(ValueError):
        kda.chunk_bwd(x, x, x, x, torch.zeros(1, 16, 1), x, x)
    with pytest.raises(ValueError):
        kda.chunk_bwd_varlen(x[0], x[0], x[0], x[0], torch.zeros(16, 1), x[0], x[0],
                             torch.tensor([0, 16], dtype=torch.int64))


def _good_bwd(B=1, T=100, H=2, D=128):
    a = _abi.BwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv, a.dtype = B, T, H, D, D, _abi.KDA_BF16
    for i, name in enumerate(("q", "k", "v", "log_alpha", "beta", "gate", "d_out", "dq", "dk", "dv",
                              "dlog_alpha", "dbeta", "dgate")):
        setattr(a, name, 0x100000 * (i + 1))
    return a


def test_bwd_workspace_size(lib):
    """Per (b, h, chunk of 64): the sweep's record (3 x 64 x D + D x D + D floats), the
    pair record (64 x D + 3 x 64 x 64 floats), the state at the chunk start and the
    gradient at its end (D x D floats each), every section rounded up to 256 bytes."""
    r256 = lambda x: (x + 255) // 256 * 256
    for B, T, H, D in ((1, 100, 2, 128), (2, 64, 3, 64), (1, 4096, 8, 128), (1, 1, 1, 64)):
        a = _good_bwd(B, T, H, D)
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _abi.KDA_OK
        items = B * H * ((T + 63) // 64)
        rec = 3 * 64 * D + D * D + D
        pairs = 64 * D + 3 * 64 * 64
        want = r256(items * rec * 4) + r256(items * pairs * 4) + 2 * r256(items * D * D * 4)
        assert n.value == want
    a = _good_bwd(T=0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _abi.KDA_OK and n.value == 0
    assert lib.kda_chunk_bwd_workspace_size(None, ctypes.byref(n)) == _abi.KDA_ERR_NULL


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "T", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "T", 2 ** 62), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "dtype", 7), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "Dv", 64), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_NO_SEGMENT_SCAN), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_CARDS_READY), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 32), _abi.KDA_ERR_UNSUPPORTED),
    # the preparation flags are accepted: the next check (no workspace) decides
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_QK_L2NORM | _abi.KDA_FLAG_GATE_LOGITS | _abi.KDA_FLAG_NO_CLAMP),
     _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "d_out", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "dbeta", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "dgate", 0x700008), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "d_initial_state", 0x900004), _abi.KDA_ERR_ALIGN),
    (lambda a: None, _abi.KDA_ERR_WORKSPACE),  # no workspace given
    (lambda a: (setattr(a, "workspace", 0x2000000), setattr(a, "workspace_bytes", 4096)), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "B", 0), _abi.KDA_OK),
    (lambda a: setattr(a, "T", 0), _abi.KDA_OK),  # no tokens and no initial-state gradient asked for
])
def test_bwd_validation(lib, mutate, code):
    a = _good_bwd()
    mutate(a)
    assert lib.kda_chunk_bwd(ctypes.byref(a), None) == code
    assert lib.kda_chunk_bwd(None, None) == _abi.KDA_ERR_NULL


def _good_bwd_var(N=3, rows=1000, H=2, D=128):
    a = _abi.BwdVarlenArgs()
    a.N, a.rows, a.H, a.Dk, a.Dv, a.dtype = N, rows, H, D, D, _abi.KDA_BF16
    for i, name in enumerate(("cu_seqlens", "q", "k", "v", "log_alpha", "beta", "gate", "d_out", "dq", "dk", "dv",
                              "dlog_alpha", "dbeta", "dgate")):
        setattr(a, name, 0x100000 * (i + 1))
    return a


def test_bwd_varlen_workspace_size(lib):
    """The backward's per-chunk sections for the most chunks any offsets can give
    (ceil(rows / 64) + N per head), then the sequence map: N + 1 starts, N + 1 chunk
    offsets (int64) and a sequence index per chunk (int32), each rounded up to 256 bytes."""
    r256 = lambda x: (x + 255) // 256 * 256
    for N, rows, H, D in ((3, 1000, 2, 128), (1, 64, 3, 64), (5, 0, 1, 64)):
        a = _good_bwd_var(N, rows, H, D)
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_bwd_varlen_workspace_size(ctypes.byref(a), ctypes.byref(n)) == _abi.KDA_OK
        chunks = (rows + 63) // 64 + N
        items = H * chunks
        rec = 3 * 64 * D + D * D + D
        pairs = 64 * D + 3 * 64 * 64
        want = r256(items * rec * 4) + r256(items * pairs * 4) + 2 * r256(items * D * D * 4)
        want += 2 * r256((N + 1) * 8) + r256(chunks * 4)
        assert n.value == want
    assert lib.kda_chunk_bwd_varlen_workspace_size(None, ctypes.byref(n)) == _abi.KDA_ERR_NULL


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "N", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "rows", -1), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "rows", 2 ** 62), _abi.KDA_ERR_SHAPE),
    (lambda a: setattr(a, "dtype", 7), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "Dv", 64), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_NO_SEGMENT_SCAN), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", 32), _abi.KDA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "flags", _abi.KDA_FLAG_QK_L2NORM | _abi.KDA_FLAG_GATE_LOGITS | _abi.KDA_FLAG_NO_CLAMP),
     _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "cu_seqlens", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "cu_seqlens", 0x100004), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "d_out", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "dbeta", None), _abi.KDA_ERR_NULL),
    (lambda a: setattr(a, "dgate", 0x700008), _abi.KDA_ERR_ALIGN),
    (lambda a: setattr(a, "d_initial_state", 0x900004), _abi.KDA_ERR_ALIGN),
    (lambda a: None, _abi.KDA_ERR_WORKSPACE),
    (lambda a: (setattr(a, "workspace", 0x2000000), setattr(a, "workspace_bytes", 4096)), _abi.KDA_ERR_WORKSPACE),
    (lambda a: setattr(a, "N", 0), _abi.KDA_OK),
    (lambda a: setattr(a, "H", 0), _abi.KDA_OK),
    (lambda a: setattr(a, "rows", 0), _abi.KDA_OK),  # no tokens and no initial-state gradient asked for
])
def test_bwd_varlen_validation(lib, mutate, code):
    a = _good_bwd_var()
    mutate(a)
    assert lib.kda_chunk_bwd_varlen(ctypes.byref(a), None) == code
    assert lib.kda_chunk_bwd_varlen(None, None) == _abi.KDA_ERR_NULL
