"""Canonical band-tile lists (oracle; test infrastructure only).

The pages give no kernel; this is the plain enumeration a band-aware tile
schedule must reproduce.  Query rows are cut into tiles of BQ rows, key rows
into tiles of BK rows.  For a head whose set of causal distances is the band
[lo, hi] (optionally joined with a shared local window [0, w - 1]), query tile
t meets key tile u iff some pair (i, j) with i in t, j in u, j <= i < N has
i - j in the set.  The tile is FULL (kind 0) iff every pair (i, j) of the tile
with i, j < N has i - j in the set, else PARTIAL (kind 1).

The pairs of a tile have the distances i - j filling the whole integer
interval [i_min - j_max, i_max - j_min], so both tests reduce to interval
tests against the set, written below as sorted, disjoint, non-touching
distance ranges.

Sources: "Making Every Head Count", Figure 1 caption (one contiguous band of
distances per head) and Figure 2 caption (the local sharing that the
exclusive-band ablation removes; reading: a window of distances [0, w - 1]
shared by every head, width not given).  The pages motivate block-aligned
sparsity (the Sparse Attention page, "Then and Now", sections 1, 3 and 6:
irregular index patterns cost memory traffic, block-aligned ones map onto GPU
reads); the tile sizes themselves are implementation parameters.
"""
import numpy as np


def _tile_rows(t, size, n):
    first = t * size
    return first, min(n, first + size) - 1


def distance_ranges(lo, hi, local_window=0):
    """The head's distance set as sorted, disjoint, non-touching inclusive
    ranges: the band [lo, hi] (empty when hi < lo) joined with [0, w - 1]."""
    rs = []
    if hi >= lo:
        rs.append([int(lo), int(hi)])
    if local_window > 0:
        rs.append([0, int(local_window) - 1])
    rs.sort()
    merged = []
    for a, b in rs:
        if merged and a <= merged[-1][1] + 1:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    return merged


def _relation(i_min, i_max, j_min, j_max, ranges):
    """(meets, full) for query rows [i_min, i_max] x key rows [j_min, j_max]."""
    d0, d1 = i_min - j_max, i_max - j_min
    meets = any(d1 >= a and d0 <= b for a, b in ranges)
    full = any(a <= d0 and d1 <= b for a, b in ranges)
    return meets, full


def query_tile_list(N, lo, hi, BQ, BK, local_window=0):
    """CSR list, query-major: for each query tile t, the key tiles u it meets,
    ascending.  Returns (row_ptr int32 [nQT+1], tiles int32, kind uint8)."""
    ranges = distance_ranges(lo, hi, local_window)
    n_qt, n_kt = (N + BQ - 1) // BQ, (N + BK - 1) // BK
    row_ptr = [0]
    tiles, kind = [], []
    for t in range(n_qt):
        i_min, i_max = _tile_rows(t, BQ, N)
        for u in range(n_kt):
            j_min, j_max = _tile_rows(u, BK, N)
            meets, full = _relation(i_min, i_max, j_min, j_max, ranges)
            if meets:
                tiles.append(u)
                kind.append(0 if full else 1)
        row_ptr.append(len(tiles))
    return (np.array(row_ptr, dtype=np.int32), np.array(tiles, dtype=np.int32),
            np.array(kind, dtype=np.uint8))


def key_tile_list(N, lo, hi, BQ, BK, local_window=0):
    """CSR list, key-major: for each key tile u, the query tiles t that meet
    it, ascending, with the same FULL/PARTIAL kind as the query-major list.
    Returns (col_ptr int32 [nKT+1], tiles int32, kind uint8)."""
    ranges = distance_ranges(lo, hi, local_window)
    n_qt, n_kt = (N + BQ - 1) // BQ, (N + BK - 1) // BK
    col_ptr = [0]
    tiles, kind = [], []
    for u in range(n_kt):
        j_min, j_max = _tile_rows(u, BK, N)
        for t in range(n_qt):
            i_min, i_max = _tile_rows(t, BQ, N)
            meets, full = _relation(i_min, i_max, j_min, j_max, ranges)
            if meets:
                tiles.append(t)
                kind.append(0 if full else 1)
        col_ptr.append(len(tiles))
    return (np.array(col_ptr, dtype=np.int32), np.array(tiles, dtype=np.int32),
            np.array(kind, dtype=np.uint8))
