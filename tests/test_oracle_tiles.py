"""Pins for the oracle's canonical band-tile lists: brute force over element
pairs on small sizes (exclusive bands and bands joined with a shared local
window), and two hand-checked lists at the N = 4096 and N = 10000 workload
bands."""
import numpy as np
import pytest

import oracle


def _brute(N, lo, hi, BQ, BK, w=0):
    n_qt, n_kt = -(-N // BQ), -(-N // BK)
    m = oracle.band_mask(N, N, lo, hi, local_window=w)
    listed, full = {}, {}
    for t in range(n_qt):
        for u in range(n_kt):
            blk = m[t * BQ:(t + 1) * BQ, u * BK:(u + 1) * BK]
            if blk.any():
                listed[(t, u)] = True
                full[(t, u)] = bool(blk.all())
    return listed, full


@pytest.mark.parametrize("w", [0, 1, 3, 9])
@pytest.mark.parametrize("BQ,BK", [(1, 1), (2, 3), (4, 4), (8, 4), (3, 8), (16, 16)])
def test_tile_lists_brute_force(BQ, BK, w):
    for N in (1, 5, 17, 33):
        for H in (1, 2, 3, 5, 40):
            lo_a, hi_a = oracle.band_table(N, H)
            tables = list(zip(lo_a.tolist(), hi_a.tolist())) + [(0, N - 1), (N // 3, N // 2), (N, N - 1)]
            for lo, hi in tables:
                listed, full = _brute(N, lo, hi, BQ, BK, w)
                rp, tl, kd = oracle.query_tile_list(N, lo, hi, BQ, BK, local_window=w)
                got = {}
                for t in range(len(rp) - 1):
                    us = tl[rp[t]:rp[t + 1]].tolist()
                    assert us == sorted(us)
                    for u, kind in zip(us, kd[rp[t]:rp[t + 1]].tolist()):
                        got[(t, u)] = kind
                assert set(got) == set(listed)
                for key, kind in got.items():
                    assert kind == (0 if full[key] else 1)
                cp, tl2, kd2 = oracle.key_tile_list(N, lo, hi, BQ, BK, local_window=w)
                got2 = {}
                for u in range(len(cp) - 1):
                    ts = tl2[cp[u]:cp[u + 1]].tolist()
                    assert ts == sorted(ts)
                    for t, kind in zip(ts, kd2[cp[u]:cp[u + 1]].tolist()):
                        got2[(t, u)] = kind
                assert got2 == got
                # with one distance range, the FULL tiles of a query tile form one contiguous run
                for t in range(len(rp) - 1 if len(oracle.distance_ranges(lo, hi, w)) == 1 else 0):
                    ks = kd[rp[t]:rp[t + 1]].tolist()
                    if 0 in ks:
                        first = ks.index(0)
                        last = len(ks) - 1 - ks[::-1].index(0)
                        assert all(x == 0 for x in ks[first:last + 1])


def test_example_lists():
    # N = 4096, band [256, 511], BQ = 128, BK = 64, query tile 10 (rows 1280..1407)
    rp, tl, kd = oracle.query_tile_list(4096, 256, 511, 128, 64)
    assert tl[rp[10]:rp[11]].tolist() == [12, 13, 14, 15, 16, 17]
    assert kd[rp[10]:rp[11]].tolist() == [1, 1, 0, 0, 1, 1]
    # N = 10000, band [834, 1667], 64 x 64, query tile 20 (rows 1280..1343)
    rp, tl, kd = oracle.query_tile_list(10000, 834, 1667, 64, 64)
    assert tl[rp[20]:rp[21]].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert kd[rp[20]:rp[21]].tolist() == [0, 0, 0, 0, 0, 0, 1, 1]
    # query tiles entirely before the band start are empty
    assert rp[13] - rp[0] == 0  # rows < 832 all < 834


def test_distance_ranges():
    assert oracle.distance_ranges(5, 9) == [[5, 9]]
    assert oracle.distance_ranges(5, 9, 3) == [[0, 2], [5, 9]]   # gap 3..4
    assert oracle.distance_ranges(5, 9, 5) == [[0, 9]]           # window touches the band
    assert oracle.distance_ranges(5, 9, 12) == [[0, 11]]         # window covers it
    assert oracle.distance_ranges(6, 5, 4) == [[0, 3]]           # empty band: the window alone
    assert oracle.distance_ranges(6, 5) == []
