"""Torch-facing wrappers of the C ABI (include/spattn.h).

torch provides device memory and the current stream; the computation runs
entirely in libspattn.so.  Tensors are contiguous [B, H, N, d] on the GPU.
"""
import ctypes

import numpy as np
import torch

from . import _lib

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bands_arg(bands, H):
    if bands is None:
        return None, None, None
    lo = np.ascontiguousarray(np.asarray(bands[0], dtype=np.int32))
    hi = np.ascontiguousarray(np.asarray(bands[1], dtype=np.int32))
    if lo.shape != (H,) or hi.shape != (H,):
        raise ValueError(f"band arrays must have shape ({H},)")
    p_lo = lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p_hi = hi.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return p_lo, p_hi, (lo, hi)  # keep the arrays alive for the call


def _check_qkv(*ts):
    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if t0.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t0.dtype}")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.shape != t0.shape or t.dtype != t0.dtype or not t.is_contiguous():
            raise ValueError("q, k, v (and o, dout) must be contiguous with equal shape and dtype")


def band_table(N, H):
    """Balanced Distance Partitioning table from the library: (lo, hi) int32."""
    lo = np.zeros(max(H, 0), dtype=np.int32)
    hi = np.zeros(max(H, 0), dtype=np.int32)
    st = _lib.load().spattn_band_table(
        N, H, lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), hi.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _lib.check(st, "spattn_band_table")
    return lo, hi


def pattern_bands(N, H, kind, width=0):
    """Band table of an attention pattern from the library
    (spattn_band_table_pattern): ``kind`` one of _lib.PATTERN_*."""
    lo = np.zeros(max(H, 0), dtype=np.int32)
    hi = np.zeros(max(H, 0), dtype=np.int32)
    st = _lib.load().spattn_band_table_pattern(
        N, H, int(kind), int(width), lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        hi.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _lib.check(st, "spattn_band_table_pattern")
    return lo, hi


def dense_bands(N, H):
    """Every head sees the whole causal range [0, N-1] (dense causal MHA)."""
    return pattern_bands(N, H, _lib.PATTERN_DENSE)


def window_bands(N, H, window):
    """Sliding-window pattern ("Making Every Head Count", Figure 2): every
    head covers distances [0, window - 1] (window 0: empty bands)."""
    return pattern_bands(N, H, _lib.PATTERN_SLIDING_WINDOW, max(0, int(window)))


def gapped_half_bands(N, H):
    """Gapped-bands pattern (same figure): each head keeps the first half of
    its Balanced Distance Partitioning band (half-width rounded down)."""
    return pattern_bands(N, H, _lib.PATTERN_GAPPED_HALF)


def fwd(q, k, v, bands=None, scale=None, out=None, lse=None, local_window=0):
    """Band attention forward.  Returns (o, lse); lse is float32 [B, H, N].
    ``local_window`` > 0 joins the shared local window [0, w - 1] to every
    head's band (spattn_fwd_local)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_qkv(q, out)
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    if local_window:
        st = _lib.load().spattn_fwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                          _DT[q.dtype], p_lo, p_hi, int(local_window), float(scale or 0.0),
                                          _stream_handle(q.device))
        _lib.check(st, "spattn_fwd_local")
        return out, lse
    st = _lib.load().spattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, _DT[q.dtype],
                                p_lo, p_hi, float(scale or 0.0), _stream_handle(q.device))
    _lib.check(st, "spattn_fwd")
    return out, lse


def _varlen_prep(q, cu_seqlens, max_seqlen):
    """Packed tensors [H, T, d]; cu_seqlens an int32 GPU tensor [S + 1]."""
    if q.dim() != 3:
        raise ValueError("packed tensors must be [H, total, d]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be an int32 GPU tensor [n_seqs + 1]")
    if not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be contiguous with at least two entries")
    H, T, d = q.shape
    # The kernels clamp every sequence to the tensors, but a malformed offsets
    # array would leave rows unwritten: check it once on the host.
    cu = cu_seqlens.cpu().numpy().astype(np.int64)
    lens = np.diff(cu)
    if cu[0] != 0 or cu[-1] != T or np.any(lens < 0):
        raise ValueError(f"cu_seqlens must rise from 0 to the packed length {T} without decreasing")
    if int(lens.max()) > int(max_seqlen):
        raise ValueError(f"a sequence of {int(lens.max())} tokens exceeds max_seqlen = {int(max_seqlen)}")
    return H, T, d, cu_seqlens.numel() - 1, int(max_seqlen)


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, bands=None, scale=None, out=None, lse=None, local_window=0):
    """Forward over a packed batch (spattn_fwd_varlen): q, k, v [H, T, d], the
    sequences at cu_seqlens (int32 GPU [S + 1]); bands None gives every
    sequence its own Balanced Distance Partitioning table.  Returns (o, lse);
    lse float32 [H, T]."""
    H, T, d, S, M = _varlen_prep(q, cu_seqlens, max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    for t in (k, v, out):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v, o must be contiguous GPU tensors of one shape and dtype")
    if q.dtype not in _DT or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous float32 or bfloat16 GPU tensor")
    if lse.dtype != torch.float32 or lse.shape != (H, T) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [H, T]")
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    st = _lib.load().spattn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), S, M, T,
                                       H, d, _DT[q.dtype], p_lo, p_hi, int(local_window), float(scale or 0.0),
                                       _stream_handle(q.device))
    _lib.check(st, "spattn_fwd_varlen")
    return out, lse


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, bands=None, scale=None, grad_dtype=None,
               workspace=None, out=None, local_window=0):
    """Backward over a packed batch (spattn_bwd_varlen).  Returns (dq, dk, dv)."""
    H, T, d, S, M = _varlen_prep(q, cu_seqlens, max_seqlen)
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v, o, dout must be contiguous GPU tensors of one shape and dtype")
    if lse.dtype != torch.float32 or lse.shape != (H, T) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [H, T]")
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    need = bwd_workspace_bytes(1, H, T, d, q.dtype, grad_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = tuple(torch.empty(q.shape, dtype=grad_dtype, device=q.device) for _ in range(3))
    for t in out:
        if t.shape != q.shape or t.dtype != grad_dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("gradient buffers must be contiguous GPU tensors of q's shape and grad_dtype")
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    dq, dk, dv = out
    st = _lib.load().spattn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(cu_seqlens), S, M, T, H, d, _DT[q.dtype],
                                       _DT[grad_dtype], p_lo, p_hi, int(local_window), float(scale or 0.0),
                                       _ptr(workspace), workspace.numel(), _stream_handle(q.device))
    _lib.check(st, "spattn_bwd_varlen")
    return dq, dk, dv


def decode(q, k_cache, v_cache, lengths=None, bands=None, local_window=0, scale=None, out=None, lse=None):
    """Decode step: q [B, H, d] against caches [B, H, Nmax, d]; ``lengths``
    an int32 device tensor [B] of valid cache rows (None: all Nmax).
    Returns (o [B, H, d], lse float32 [B, H])."""
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, H, d] and the caches [B, H, Nmax, d]")
    B, H, Nmax, d = k_cache.shape
    if q.shape != (B, H, d) or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("q and caches disagree in shape or dtype")
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("tensors must be contiguous and on the GPU")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.shape != (B,) or not lengths.is_cuda
                                or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 GPU tensor of shape [B]")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    st = _lib.load().spattn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                   None if lengths is None else _ptr(lengths), B, H, Nmax, d, _DT[q.dtype], p_lo,
                                   p_hi, int(local_window), float(scale or 0.0), _stream_handle(q.device))
    _lib.check(st, "spattn_decode")
    return out, lse


def bwd_workspace_bytes(B, H, N, d, dtype, grad_dtype):
    return int(_lib.load().spattn_bwd_workspace_bytes(B, H, N, d, _DT[dtype], _DT[grad_dtype]))


def _bwd_prep(q, k, v, o, lse, dout, grad_dtype, workspace, out, n_out):
    if o is not None:
        _check_qkv(q, k, v, o, dout)
    else:
        _check_qkv(q, k, v, dout)
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    need = bwd_workspace_bytes(B, H, N, d, q.dtype, grad_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = tuple(torch.empty(q.shape, dtype=grad_dtype, device=q.device) for _ in range(n_out))
    for t in out:
        if t.shape != q.shape or t.dtype != grad_dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("gradient buffers must be contiguous GPU tensors of q's shape and grad_dtype")
    return B, H, N, d, grad_dtype, workspace, out


def bwd_dq(q, k, v, o, lse, dout, workspace, bands=None, scale=None, grad_dtype=None, out=None):
    """First backward stage: D into ``workspace`` and dq.  Returns dq."""
    B, H, N, d, grad_dtype, workspace, out = _bwd_prep(q, k, v, o, lse, dout, grad_dtype, workspace,
                                                       None if out is None else (out,), 1)
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    st = _lib.load().spattn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(out[0]),
                                   B, H, N, d, _DT[q.dtype], _DT[grad_dtype], p_lo, p_hi, float(scale or 0.0),
                                   _ptr(workspace), workspace.numel(), _stream_handle(q.device))
    _lib.check(st, "spattn_bwd_dq")
    return out[0]


def bwd_dkdv(q, k, v, lse, dout, workspace, bands=None, scale=None, grad_dtype=None, out=None):
    """Second backward stage (after bwd_dq with the same workspace): dk, dv."""
    B, H, N, d, grad_dtype, workspace, out = _bwd_prep(q, k, v, None, lse, dout, grad_dtype, workspace, out, 2)
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    st = _lib.load().spattn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(out[0]), _ptr(out[1]),
                                     B, H, N, d, _DT[q.dtype], _DT[grad_dtype], p_lo, p_hi, float(scale or 0.0),
                                     _ptr(workspace), workspace.numel(), _stream_handle(q.device))
    _lib.check(st, "spattn_bwd_dkdv")
    return out


def bwd(q, k, v, o, lse, dout, bands=None, scale=None, grad_dtype=None, workspace=None, out=None,
        local_window=0):
    """Band attention backward.  Returns (dq, dk, dv) of ``grad_dtype``
    (default: the input dtype); ``out`` may supply preallocated (dq, dk, dv).
    ``local_window`` as in ``fwd`` (spattn_bwd_local)."""
    B, H, N, d, grad_dtype, workspace, out = _bwd_prep(q, k, v, o, lse, dout, grad_dtype, workspace, out, 3)
    dq, dk, dv = out
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    if local_window:
        st = _lib.load().spattn_bwd_local(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                          _ptr(dk), _ptr(dv), B, H, N, d, _DT[q.dtype], _DT[grad_dtype], p_lo,
                                          p_hi, int(local_window), float(scale or 0.0), _ptr(workspace),
                                          workspace.numel(), _stream_handle(q.device))
        _lib.check(st, "spattn_bwd_local")
        return dq, dk, dv
    st = _lib.load().spattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, H, N, d, _DT[q.dtype], _DT[grad_dtype], p_lo, p_hi,
                                float(scale or 0.0), _ptr(workspace), workspace.numel(),
                                _stream_handle(q.device))
    _lib.check(st, "spattn_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, bands=None, scale=None, grad_dtype=None, out=None):
    """spattn_bwd_noalloc: the backward with the library's static device
    workspace (no workspace argument).  Calls on one GPU must not overlap."""
    B, H, N, d = q.shape
    _check_qkv(q, k, v, o, dout)
    if lse.dtype != torch.float32 or lse.shape != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    if out is None:
        out = tuple(torch.empty(q.shape, dtype=grad_dtype, device=q.device) for _ in range(3))
    for t in out:
        if t.shape != q.shape or t.dtype != grad_dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("gradient buffers must be contiguous GPU tensors of q's shape and grad_dtype")
    dq, dk, dv = out
    p_lo, p_hi, _keep = _bands_arg(bands, H)
    st = _lib.load().spattn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), B, H, N, d, _DT[q.dtype], _DT[grad_dtype], p_lo, p_hi,
                                        float(scale or 0.0), _stream_handle(q.device))
    _lib.check(st, "spattn_bwd_noalloc")
    return dq, dk, dv


def kernel_tiles(d, dtype):
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    st = _lib.load().spattn_kernel_tiles(d, _DT[dtype], ctypes.byref(bq), ctypes.byref(bk))
    _lib.check(st, "spattn_kernel_tiles")
    return bq.value, bk.value


def tile_list(N, lo, hi, BQ=0, BK=0, device="cuda"):
    """Device-computed query-major tile list (CSR) of one band.
    Returns numpy (row_ptr, tiles, kind)."""
    if BQ == 0 and BK == 0:
        BQ, BK = kernel_tiles(128, torch.bfloat16)
    n_qt = (N + BQ - 1) // BQ
    cap = n_qt * ((N + BK - 1) // BK)
    row_ptr = torch.zeros(n_qt + 1, dtype=torch.int32, device=device)
    tiles = torch.zeros(max(cap, 1), dtype=torch.int32, device=device)
    kind = torch.zeros(max(cap, 1), dtype=torch.uint8, device=device)
    n_out = torch.zeros(1, dtype=torch.int32, device=device)
    st = _lib.load().spattn_tile_list(N, lo, hi, BQ, BK, _ptr(row_ptr), _ptr(tiles), _ptr(kind), cap, _ptr(n_out),
                                      _stream_handle(row_ptr.device))
    _lib.check(st, "spattn_tile_list")
    torch.cuda.current_stream(row_ptr.device).synchronize()
    n = int(n_out.item())
    return row_ptr.cpu().numpy(), tiles[:n].cpu().numpy(), kind[:n].cpu().numpy()


def tile_walk(kernel, N, lo, hi, dtype=torch.bfloat16, B=1, H=1, local_window=0, d=128, device="cuda"):
    """A kernel's actual tile walk for one band (spattn_tile_walk), as numpy
    (ptr, tiles, kind, own_rows, tile_rows): owned tile t visits
    tiles[ptr[t]:ptr[t + 1]] in that order."""
    own, tile = ctypes.c_int32(), ctypes.c_int32()
    lib = _lib.load()
    n_out = torch.zeros(1, dtype=torch.int32, device=device)
    # sizes first (cap 0 writes only ptr and the count)
    probe = torch.zeros(N + 1, dtype=torch.int32, device=device)
    st = lib.spattn_tile_walk(int(kernel), int(d), _DT[dtype], B, H, N, lo, hi, int(local_window), _ptr(probe), None,
                              None, 0, _ptr(n_out), ctypes.byref(own), ctypes.byref(tile), _stream_handle(probe.device))
    _lib.check(st, "spattn_tile_walk")
    torch.cuda.current_stream(probe.device).synchronize()
    n = int(n_out.item())
    n_own = (N + own.value - 1) // own.value
    ptr = torch.zeros(n_own + 1, dtype=torch.int32, device=device)
    tiles = torch.zeros(max(n, 1), dtype=torch.int32, device=device)
    kind = torch.zeros(max(n, 1), dtype=torch.uint8, device=device)
    st = lib.spattn_tile_walk(int(kernel), int(d), _DT[dtype], B, H, N, lo, hi, int(local_window), _ptr(ptr),
                              _ptr(tiles), _ptr(kind), n, _ptr(n_out), None, None, _stream_handle(ptr.device))
    _lib.check(st, "spattn_tile_walk")
    torch.cuda.current_stream(ptr.device).synchronize()
    return (ptr.cpu().numpy(), tiles[:n].cpu().numpy(), kind[:n].cpu().numpy(), own.value, tile.value)


class _BandAttention(torch.autograd.Function):
    """Autograd node over fwd / bwd: saves O and LSE, no recomputation here."""

    @staticmethod
    def forward(ctx, q, k, v, bands, local_window, scale):
        o, lse = fwd(q, k, v, bands=bands, scale=scale, local_window=local_window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.bands, ctx.local_window, ctx.scale = bands, local_window, scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, dout.contiguous(), bands=ctx.bands, scale=ctx.scale,
                         local_window=ctx.local_window)
        return dq, dk, dv, None, None, None


def band_attention(q, k, v, bands=None, local_window=0, scale=None):
    """Differentiable band attention: O = fwd(q, k, v) with a backward through
    bwd.  q, k, v are [B, H, N, d] bfloat16 or float32 on the GPU; ``bands``
    is None (the Balanced Distance Partitioning table of (N, H)) or host
    (lo[H], hi[H]); ``local_window`` joins [0, w - 1] to every band.  Gradients
    come out in the input dtype."""
    return _BandAttention.apply(q.contiguous(), k.contiguous(), v.contiguous(), bands, int(local_window), scale)
