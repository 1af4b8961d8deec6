"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/spattn.h declares, computes the band table bit-exactly
like the oracle, and rejects bad arguments with the documented status codes
before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from structured_sparse_attention_spattn_amd import _lib, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "spattn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(spattn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spattn_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_probe_library_exports_every_declared_symbol():
    """libspattn_probe.so (the measured-denominator microbenchmarks) exports
    what include/spattn_probe.h declares and rejects bad arguments on the host."""
    path = os.path.join(ROOT, "structured_sparse_attention_spattn_amd", "libspattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("libspattn_probe.so not built")
    text = open(os.path.join(ROOT, "include", "spattn_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(spattn_probe_\w+)\s*\(", text, flags=re.M)))
    assert names == ["spattn_probe_atomic", "spattn_probe_lds", "spattn_probe_mfma", "spattn_probe_read"]
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (spattn_probe_\w+)", out))
    lib = ctypes.CDLL(path)
    sink = ctypes.c_void_p(16)  # never dereferenced: every call below fails its argument check
    assert lib.spattn_probe_mfma(2, 1, 1, sink, None) == 1
    assert lib.spattn_probe_mfma(0, 0, 1, sink, None) == 1
    assert lib.spattn_probe_lds(2, 1, 1, sink, None) == 1
    assert lib.spattn_probe_lds(0, 1, 0, sink, None) == 1
    assert lib.spattn_probe_lds(0, 1, 1, None, None) == 1
    lib.spattn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    assert lib.spattn_probe_read(sink, 15, 1, sink, None) == 1
    lib.spattn_probe_atomic.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]
    aligned = ctypes.c_void_p(256)  # never dereferenced either
    assert lib.spattn_probe_atomic(None, 256, 1, 1, None) == 1
    assert lib.spattn_probe_atomic(aligned, 384, 1, 1, None) == 1  # not a power of two
    assert lib.spattn_probe_atomic(aligned, 128, 1, 1, None) == 1  # below 256
    assert lib.spattn_probe_atomic(sink, 256, 1, 1, None) == 1     # not 256-byte aligned
    assert lib.spattn_probe_atomic(aligned, 256, 0, 1, None) == 1
    assert lib.spattn_probe_atomic(aligned, 256, 1, 0, None) == 1


@pytest.mark.parametrize("N", range(1, 65))
def test_band_table_bit_exact_vs_oracle(N):
    for H in range(1, 17):
        lo, hi = ops.band_table(N, H)
        olo, ohi = oracle.band_table(N, H)
        assert np.array_equal(lo, olo) and np.array_equal(hi, ohi)


@pytest.mark.parametrize("N,H", [(1024, 8), (4096, 16), (8192, 32), (10000, 12), (3, 256), (100000, 7)])
def test_band_table_workload_sizes(N, H):
    lo, hi = ops.band_table(N, H)
    olo, ohi = oracle.band_table(N, H)
    assert np.array_equal(lo, olo) and np.array_equal(hi, ohi)


def test_band_table_rejects_bad_args():
    lib = _lib.load()
    buf = (ctypes.c_int32 * 4)()
    assert lib.spattn_band_table(0, 4, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table(4, 0, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table(4, 257, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table(4, 2, None, buf) == _lib.E_ARG


def _fwd(lib, ptr=1, B=1, H=2, N=8, d=64, dtype=_lib.BF16, lo=None, hi=None):
    p = ctypes.c_void_p(ptr)
    return lib.spattn_fwd(p, p, p, p, p, B, H, N, d, dtype, lo, hi, 0.0, None)


def test_fwd_validation_before_launch():
    lib = _lib.load()
    assert _fwd(lib, B=0) == _lib.E_ARG
    assert _fwd(lib, H=0) == _lib.E_ARG
    assert _fwd(lib, N=0) == _lib.E_ARG
    assert _fwd(lib, H=300) == _lib.E_ARG
    assert _fwd(lib, d=96) == _lib.E_UNSUPPORTED
    assert _fwd(lib, dtype=7) == _lib.E_UNSUPPORTED
    assert _fwd(lib, ptr=0) == _lib.E_ARG
    I2 = ctypes.c_int32 * 2
    assert _fwd(lib, lo=I2(0, 5), hi=I2(4, 8)) == _lib.E_ARG       # hi > N - 1
    assert _fwd(lib, lo=I2(0, -1), hi=I2(4, 3)) == _lib.E_ARG      # lo < 0
    assert _fwd(lib, lo=I2(0, 6), hi=I2(4, 4)) == _lib.E_ARG       # lo > hi + 1
    assert _fwd(lib, lo=I2(0, 5), hi=None) == _lib.E_ARG           # only one array


def test_bwd_validation_and_workspace():
    lib = _lib.load()
    p = ctypes.c_void_p(1)
    need = lib.spattn_bwd_workspace_bytes(2, 3, 100, 128, _lib.BF16, _lib.BF16)
    rows = 2 * 3 * 100
    assert need == 2 * ((rows * 4 + 255) // 256 * 256)  # float32 D and -LSE log2(e), 256-byte aligned
    assert lib.spattn_bwd_workspace_bytes(2, 3, 100, 128, _lib.BF16, _lib.F32) == need
    assert lib.spattn_bwd_workspace_bytes(0, 3, 100, 128, _lib.BF16, _lib.BF16) == 0
    assert lib.spattn_bwd_workspace_bytes(1, 3, 100, 96, _lib.BF16, _lib.BF16) == 0

    def bwd(ws, ws_bytes, grad=_lib.BF16, d=128):
        return lib.spattn_bwd(p, p, p, p, p, p, p, p, p, 2, 3, 100, d, _lib.BF16, grad, None, None, 0.0,
                              ctypes.c_void_p(ws), ws_bytes, None)
    assert bwd(0, need) == _lib.E_WORKSPACE
    assert bwd(256, need - 1) == _lib.E_WORKSPACE
    assert bwd(256 + 8, need) == _lib.E_WORKSPACE  # misaligned
    assert bwd(256, need, grad=5) == _lib.E_UNSUPPORTED
    assert bwd(256, need, d=32) == _lib.E_UNSUPPORTED


def test_kernel_tiles_and_status_strings():
    lib = _lib.load()
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    assert lib.spattn_kernel_tiles(128, _lib.BF16, ctypes.byref(bq), ctypes.byref(bk)) == _lib.OK
    assert bq.value > 0 and bk.value > 0 and bq.value % 32 == 0 and bk.value % 32 == 0
    assert lib.spattn_kernel_tiles(96, _lib.BF16, ctypes.byref(bq), ctypes.byref(bk)) == _lib.E_UNSUPPORTED
    for s in range(5):
        assert _lib.status_string(s)
    assert _lib.status_string(99) == "unknown status"


def test_tile_list_validation():
    lib = _lib.load()
    p = ctypes.c_void_p(1)
    assert lib.spattn_tile_list(0, 0, 0, 64, 64, p, p, p, 4, p, None) == _lib.E_ARG
    assert lib.spattn_tile_list(10, 0, 10, 64, 64, p, p, p, 4, p, None) == _lib.E_ARG
    assert lib.spattn_tile_list(10, 0, 5, 0, 64, p, p, p, 4, p, None) == _lib.E_ARG
    assert lib.spattn_tile_list(10, 0, 5, 64, 64, None, p, p, 4, p, None) == _lib.E_ARG


def test_bwd_stage_validation():
    lib = _lib.load()
    p = ctypes.c_void_p(1)
    need = lib.spattn_bwd_workspace_bytes(2, 3, 100, 128, _lib.BF16, _lib.BF16)
    ws = ctypes.c_void_p(256)
    assert lib.spattn_bwd_dq(p, p, p, p, p, p, p, 2, 3, 100, 128, _lib.BF16, _lib.BF16, None, None, 0.0,
                             ctypes.c_void_p(0), need, None) == _lib.E_WORKSPACE
    assert lib.spattn_bwd_dq(p, p, p, None, p, p, p, 2, 3, 100, 128, _lib.BF16, _lib.BF16, None, None, 0.0,
                             ws, need, None) == _lib.E_ARG
    assert lib.spattn_bwd_dq(p, p, p, p, p, p, p, 2, 3, 100, 96, _lib.BF16, _lib.BF16, None, None, 0.0,
                             ws, need, None) == _lib.E_UNSUPPORTED
    assert lib.spattn_bwd_dkdv(p, p, p, p, p, p, p, 2, 3, 100, 128, _lib.BF16, _lib.BF16, None, None, 0.0,
                               ws, need - 4, None) == _lib.E_WORKSPACE
    assert lib.spattn_bwd_dkdv(p, p, p, p, p, None, p, 2, 3, 100, 128, _lib.BF16, _lib.BF16, None, None, 0.0,
                               ws, need, None) == _lib.E_ARG
    assert lib.spattn_bwd_dkdv(p, p, p, p, p, p, p, 0, 3, 100, 128, _lib.BF16, _lib.BF16, None, None, 0.0,
                               ws, need, None) == _lib.E_ARG


def test_local_window_validation_before_launch():
    lib = _lib.load()
    p = ctypes.c_void_p(1)

    def fwd(w, dtype=_lib.BF16):
        return lib.spattn_fwd_local(p, p, p, p, p, 1, 2, 8, 64, dtype, None, None, w, 0.0, None)

    def bwd(w, dtype=_lib.BF16):
        need = lib.spattn_bwd_workspace_bytes(1, 2, 8, 64, dtype, dtype)
        return lib.spattn_bwd_local(p, p, p, p, p, p, p, p, p, 1, 2, 8, 64, dtype, dtype, None, None, w, 0.0,
                                    ctypes.c_void_p(256), need, None)
    assert fwd(-1) == _lib.E_ARG
    assert bwd(-1) == _lib.E_ARG
    assert fwd(-2, dtype=_lib.F32) == _lib.E_ARG
    ptr0 = ctypes.c_void_p(0)
    assert lib.spattn_fwd_local(ptr0, p, p, p, p, 1, 2, 8, 64, _lib.BF16, None, None, 3, 0.0, None) == _lib.E_ARG


@pytest.mark.parametrize("N,H", [(1024, 8), (4096, 16), (7, 3), (5, 9), (10000, 12), (1, 1), (3, 256)])
def test_pattern_tables_match_oracle(N, H):
    """The Figure 2 pattern tables come from the library
    (spattn_band_table_pattern) and equal the oracle's, bit for bit."""
    for w in (0, 1, N // H, N, N + 5):
        lo, hi = ops.window_bands(N, H, w)
        olo, ohi = oracle.band_table_sliding_window(N, H, w)
        assert np.array_equal(lo, olo) and np.array_equal(hi, ohi), w
    lo, hi = ops.gapped_half_bands(N, H)
    olo, ohi = oracle.band_table_gapped_half(N, H)
    assert np.array_equal(lo, olo) and np.array_equal(hi, ohi)
    lo, hi = ops.pattern_bands(N, H, _lib.PATTERN_BDP)
    olo, ohi = oracle.band_table(N, H)
    assert np.array_equal(lo, olo) and np.array_equal(hi, ohi)
    lo, hi = ops.dense_bands(N, H)
    assert np.all(lo == 0) and np.all(hi == N - 1)


def test_pattern_table_rejects_bad_args():
    lib = _lib.load()
    buf = (ctypes.c_int32 * 4)()
    assert lib.spattn_band_table_pattern(8, 4, 9, 0, buf, buf) == _lib.E_ARG             # unknown kind
    assert lib.spattn_band_table_pattern(8, 4, _lib.PATTERN_SLIDING_WINDOW, -1, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table_pattern(0, 4, _lib.PATTERN_BDP, 0, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table_pattern(8, 257, _lib.PATTERN_BDP, 0, buf, buf) == _lib.E_ARG
    assert lib.spattn_band_table_pattern(8, 4, _lib.PATTERN_DENSE, 0, None, buf) == _lib.E_ARG


def test_tile_walk_validation():
    lib = _lib.load()
    p = ctypes.c_void_p(1)

    def walk(kernel=0, dtype=_lib.BF16, B=1, H=1, N=10, lo=0, hi=5, w=0, ptr=p, cap=4, d=128):
        return lib.spattn_tile_walk(kernel, d, dtype, B, H, N, lo, hi, w, ptr, p, p, cap, p, None, None, None)
    assert walk(kernel=3) == _lib.E_ARG
    assert walk(kernel=-1) == _lib.E_ARG
    assert walk(dtype=4) == _lib.E_UNSUPPORTED
    assert walk(N=0) == _lib.E_ARG
    assert walk(B=0) == _lib.E_ARG
    assert walk(hi=10) == _lib.E_ARG
    assert walk(lo=7, hi=5) == _lib.E_ARG
    assert walk(w=-1) == _lib.E_ARG
    assert walk(ptr=None) == _lib.E_ARG
    assert walk(cap=-1) == _lib.E_ARG
    assert walk(d=96) == _lib.E_UNSUPPORTED


def test_decode_validation_before_launch():
    lib = _lib.load()
    p = ctypes.c_void_p(1)

    def dec(w=0, d=128, dtype=_lib.BF16, B=2, ptr=p):
        return lib.spattn_decode(ptr, p, p, p, p, None, B, 4, 64, d, dtype, None, None, w, 0.0, None)
    assert dec(w=-1) == _lib.E_ARG
    assert dec(d=96) == _lib.E_UNSUPPORTED
    assert dec(dtype=9) == _lib.E_UNSUPPORTED
    assert dec(B=0) == _lib.E_ARG
    assert dec(ptr=ctypes.c_void_p(0)) == _lib.E_ARG


def test_varlen_validation_before_launch():
    lib = _lib.load()
    p = ctypes.c_void_p(1)
    I2 = lambda a, b: (ctypes.c_int32 * 2)(a, b)

    def fwd(cu=p, S=2, M=8, T=12, H=2, d=64, dtype=_lib.BF16, lo=None, hi=None, w=0, ptr=p):
        return lib.spattn_fwd_varlen(ptr, p, p, p, p, cu, S, M, T, H, d, dtype, lo, hi, w, 0.0, None)

    def bwd(ws=ctypes.c_void_p(256), nbytes=None, gdt=_lib.BF16, S=2, ptr=p):
        need = lib.spattn_bwd_workspace_bytes(1, 2, 12, 64, _lib.BF16, gdt)
        return lib.spattn_bwd_varlen(ptr, p, p, p, p, p, p, p, p, p, S, 8, 12, 2, 64, _lib.BF16, gdt, None, None,
                                     0, 0.0, ws, need if nbytes is None else nbytes, None)
    assert fwd(cu=None) == _lib.E_ARG
    assert fwd(S=0) == _lib.E_ARG
    assert fwd(M=0) == _lib.E_ARG
    assert fwd(T=0) == _lib.E_ARG
    assert fwd(H=0) == _lib.E_ARG
    assert fwd(w=-1) == _lib.E_ARG
    assert fwd(d=96) == _lib.E_UNSUPPORTED
    assert fwd(dtype=5) == _lib.E_UNSUPPORTED
    assert fwd(ptr=ctypes.c_void_p(0)) == _lib.E_ARG
    assert fwd(lo=I2(0, 4), hi=I2(3, 8)) == _lib.E_ARG   # hi beyond max_seqlen - 1
    assert fwd(lo=I2(0, 4), hi=None) == _lib.E_ARG       # only one array
    assert bwd(S=0) == _lib.E_ARG
    assert bwd(ws=ctypes.c_void_p(0)) == _lib.E_WORKSPACE
    assert bwd(nbytes=16) == _lib.E_WORKSPACE
    assert bwd(gdt=7) == _lib.E_UNSUPPORTED
    assert bwd(ptr=ctypes.c_void_p(0)) == _lib.E_ARG


def test_misaligned_pointers_rejected_before_launch():
    """Tensor pointers must be 16-byte aligned, LSE / lengths / cu_seqlens
    4-byte aligned: one misaligned pointer (all others aligned) is E_ARG,
    checked before anything is launched."""
    lib = _lib.load()
    A = 1 << 20  # aligned stand-in addresses, never dereferenced: each call below fails validation
    P = lambda off=0: ctypes.c_void_p(A + off)
    for i in range(5):
        args = [P(), P(), P(), P(), P()]
        args[i] = P(8 if i < 4 else 2)
        assert lib.spattn_fwd(*args, 1, 2, 64, 64, _lib.BF16, None, None, 0.0, None) == _lib.E_ARG, i
    need = lib.spattn_bwd_workspace_bytes(1, 2, 64, 64, _lib.BF16, _lib.BF16)
    ws = ctypes.c_void_p(A)
    for i in range(9):
        args = [P() for _ in range(9)]
        args[i] = P(2 if i == 4 else 8)  # index 4 is LSE
        assert lib.spattn_bwd(*args, 1, 2, 64, 64, _lib.BF16, _lib.BF16, None, None, 0.0, ws, need,
                              None) == _lib.E_ARG, i
    assert lib.spattn_decode(P(), P(), P(), P(), P(), P(2), 1, 2, 64, 64, _lib.BF16, None, None, 0, 0.0,
                             None) == _lib.E_ARG
    assert lib.spattn_fwd_varlen(P(), P(), P(), P(), P(), P(2), 2, 8, 12, 2, 64, _lib.BF16, None, None, 0, 0.0,
                                 None) == _lib.E_ARG
