"""Canonical band-tile lists (oracle; test infrastructure only).

The pages give no kernel; this is the plain enumeration a band-aware tile
schedule must reproduce.  Query rows are cut into tiles of BQ rows, key rows
into tiles of BK rows.  For head band [lo, hi] (distance i - j), query tile t
meets key tile u iff some pair (i, j) with i in t, j in u, j <= i < N has
lo <= i - j <= hi.  The tile is FULL (kind 0) iff every pair (i, j) of the
tile with i, j < N is in the band, else PARTIAL (kind 1).

The pages motivate block-aligned sparsity (the Sparse Attention page,
"Then and Now", sections 1, 3 and 6: irregular index patterns cost memory
traffic, block-aligned ones map onto GPU reads); the tile sizes themselves are
implementation parameters.
"""
import numpy as np


def _tile_rows(t, size, n):
    first = t * size
    return first, min(n, first + size) - 1


def query_tile_list(N, lo, hi, BQ, BK):
    """CSR list, query-major: for each query tile t, the key tiles u it meets,
    ascending.  Returns (row_ptr int32 [nQT+1], tiles int32, kind uint8)."""
    n_qt = (N + BQ - 1) // BQ
    row_ptr = [0]
    tiles, kind = [], []
    for t in range(n_qt):
        i_min, i_max = _tile_rows(t, BQ, N)
        if hi >= lo and i_max >= lo:
            j_min = max(0, i_min - hi)
            j_max = i_max - lo
            for u in range(j_min // BK, j_max // BK + 1):
                j0, j1 = _tile_rows(u, BK, N)
                full = (i_min - j1 >= lo) and (i_max - j0 <= hi)
                tiles.append(u)
                kind.append(0 if full else 1)
        row_ptr.append(len(tiles))
    return (np.array(row_ptr, dtype=np.int32), np.array(tiles, dtype=np.int32),
            np.array(kind, dtype=np.uint8))


def key_tile_list(N, lo, hi, BQ, BK):
    """CSR list, key-major: for each key tile u, the query tiles t that meet
    it, ascending, with the same FULL/PARTIAL kind as the query-major list.
    Returns (col_ptr int32 [nKT+1], tiles int32, kind uint8)."""
    n_kt = (N + BK - 1) // BK
    col_ptr = [0]
    tiles, kind = [], []
    for u in range(n_kt):
        j0, j1 = _tile_rows(u, BK, N)
        if hi >= lo and j0 + lo <= N - 1:
            i_first = j0 + lo
            i_last = min(N - 1, j1 + hi)
            for t in range(i_first // BQ, i_last // BQ + 1):
                i_min, i_max = _tile_rows(t, BQ, N)
                full = (i_min - j1 >= lo) and (i_max - j0 <= hi)
                tiles.append(t)
                kind.append(0 if full else 1)
        col_ptr.append(len(tiles))
    return (np.array(col_ptr, dtype=np.int32), np.array(tiles, dtype=np.int32),
            np.array(kind, dtype=np.uint8))
