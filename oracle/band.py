"""Band table of Balanced Distance Partitioning (oracle; test infrastructure).

Source: "Making Every Head Count: Sparse Attention Without the
Speed-Performance Trade-off", Figure 1 caption: the causal distance spectrum
is cut into H contiguous, non-overlapping bands, each of width floor(N/H) or
ceil(N/H), from the nearest distances (head 0) to the farthest (head H-1);
the TL;DR names the three properties completeness, exclusivity and balance.

Reading (pages silent): the ceil-width bands are the first N mod H heads.
A head whose band is empty (only when H > N) gets lo = N, hi = N - 1.
"""
import numpy as np


def band_table(N, H):
    """Return (lo, hi), int32 arrays of length H, inclusive distance bounds.

    Head h attends the pairs (i, j) with lo[h] <= i - j <= hi[h].  Walk the
    distance axis from 0 upward and give each head its width in turn.
    """
    if N < 1 or H < 1:
        raise ValueError("N and H must be >= 1")
    base, extra = divmod(N, H)
    lo = np.empty(H, dtype=np.int32)
    hi = np.empty(H, dtype=np.int32)
    start = 0
    for h in range(H):
        width = base + (1 if h < extra else 0)
        lo[h] = start
        hi[h] = start + width - 1
        start += width
    assert start == N
    return lo, hi


def band_pairs(N, lo, hi):
    """Number of causal pairs (i, j), 0 <= j <= i < N, whose distance lies in
    [lo, hi]: one term per distance d, each contributing N - d query rows."""
    total = 0
    for dist in range(int(lo), int(hi) + 1):
        if 0 <= dist < N:
            total += N - dist
    return total


def band_table_sliding_window(N, H, window):
    """Figure 2(a) of the SPAttention page: every head is restricted to the
    same local window; it covers distances [0, window - 1]."""
    w = max(0, min(int(window), N))
    lo = np.zeros(H, dtype=np.int32)
    hi = np.full(H, w - 1, dtype=np.int32)
    if w == 0:
        lo[:] = N
        hi[:] = N - 1
    return lo, hi


def band_table_gapped_half(N, H):
    """Figure 2(c) of the SPAttention page (GBHALF): each head attends only the
    first half of its assigned band.  Reading: the half-width rounds down, so a
    width-1 band becomes empty (lo = N, hi = N - 1)."""
    lo, hi = band_table(N, H)
    lo2 = lo.copy()
    hi2 = hi.copy()
    for h in range(H):
        half = (int(hi[h]) - int(lo[h]) + 1) // 2
        if half == 0:
            lo2[h] = N
            hi2[h] = N - 1
        else:
            hi2[h] = lo[h] + half - 1
    return lo2, hi2
