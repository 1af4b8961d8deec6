"""Packed variable-length batches (oracle; test infrastructure only).

Sequences of different lengths stored back to back along the token axis
([H, T, d], sequence s at tokens cu[s] .. cu[s+1] - 1).  Positions restart at
0 in every sequence and attention never crosses a sequence boundary, so each
sequence is the plain band attention of its own length ("Making Every Head
Count": the method is defined on one sequence; Figure 1 caption for the band
table).

Readings (pages silent on packed batches):
* without a caller table, each sequence uses the Balanced Distance
  Partitioning table of its own length n (its heads partition the distances
  [0, n - 1] of that sequence);
* a caller table is shared by all sequences and clipped to each length:
  lo -> min(lo, n), hi -> min(hi, n - 1).
"""
import numpy as np

from .attention import band_attention_bwd, band_attention_fwd
from .band import band_table


def seq_bands(n, H, bands=None):
    """The heads' bands (lo, hi) for one sequence of n >= 1 tokens."""
    if bands is None:
        return band_table(n, H)
    lo = np.minimum(np.asarray(bands[0], dtype=np.int64), n)
    hi = np.minimum(np.asarray(bands[1], dtype=np.int64), n - 1)
    return lo.astype(np.int32), hi.astype(np.int32)


def _segments(cu):
    cu = [int(c) for c in cu]
    return [(cu[s], cu[s + 1] - cu[s]) for s in range(len(cu) - 1)]


def varlen_fwd(q, k, v, cu, bands=None, scale=None, local_window=0):
    """q, k, v: [H, T, d].  Returns (out [H, T, dv], lse [H, T]) in float64;
    tokens of empty sequences (none exist) and outside cu stay 0 / -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, T, _ = q.shape
    out = np.zeros((H, T, v.shape[2]))
    lse = np.full((H, T), -np.inf)
    for o, n in _segments(cu):
        if n <= 0:
            continue
        lo, hi = seq_bands(n, H, bands)
        sl = slice(o, o + n)
        o_s, l_s = band_attention_fwd(q[None, :, sl], k[None, :, sl], v[None, :, sl], lo, hi, scale=scale,
                                      local_window=local_window)
        out[:, sl] = o_s[0]
        lse[:, sl] = l_s[0]
    return out, lse


def varlen_bwd(q, k, v, dout, cu, bands=None, scale=None, local_window=0):
    """Gradients over a packed batch.  Returns (dq, dk, dv, out, lse)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    H, T, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = np.zeros((H, T, v.shape[2]))
    lse = np.full((H, T), -np.inf)
    for o, n in _segments(cu):
        if n <= 0:
            continue
        lo, hi = seq_bands(n, H, bands)
        sl = slice(o, o + n)
        g = band_attention_bwd(q[None, :, sl], k[None, :, sl], v[None, :, sl], dout[None, :, sl], lo, hi,
                               scale=scale, local_window=local_window)
        for dst, src in zip((dq, dk, dv, out, lse), g):
            dst[:, sl] = src[0]
    return dq, dk, dv, out, lse
