"""Pins for the oracle's band table (Balanced Distance Partitioning).

Source: "Making Every Head Count" -- Figure 1 caption (contiguous,
non-overlapping bands of width floor(N/H) or ceil(N/H), head 0 nearest) and
TL;DR (completeness, exclusivity, balance).  The checks below are properties,
a brute-force search and the figure's own instance -- not a second copy of the
construction.  Together, balance + wider-first + contiguity starting at 0 fix
the table uniquely, which ``test_properties_determine_table`` confirms by
exhaustive search.
"""
import itertools

import numpy as np
import pytest

import oracle


def _check_properties(N, H, lo, hi):
    widths = hi.astype(np.int64) - lo.astype(np.int64) + 1
    floor_w, ceil_w = N // H, -(-N // H)
    # contiguity from distance 0 to N - 1
    assert lo[0] == 0 or (widths[0] == 0)
    pos = 0
    for h in range(H):
        if widths[h] > 0:
            assert lo[h] == pos
            pos = hi[h] + 1
        else:
            assert lo[h] == N and hi[h] == N - 1
    assert pos == N
    # balance
    assert set(widths.tolist()) <= {floor_w, ceil_w}
    # wider bands first
    assert all(widths[h] >= widths[h + 1] for h in range(H - 1))


@pytest.mark.parametrize("N", range(1, 65))
def test_invariants_all_small(N):
    for H in range(1, 17):
        lo, hi = oracle.band_table(N, H)
        assert lo.dtype == np.int32 and hi.dtype == np.int32
        _check_properties(N, H, lo, hi)
        # per-pair: every causal (i, j) falls in exactly one head's band
        counts = np.zeros((N, N), dtype=np.int64)
        for h in range(H):
            counts += oracle.band_mask(N, N, int(lo[h]), int(hi[h]))
        causal = np.tril(np.ones((N, N), dtype=np.int64))
        assert np.array_equal(counts, causal)
        # row sizes: sum over heads of |S_i^h| = i + 1
        assert np.array_equal(counts.sum(axis=1), np.arange(1, N + 1))


def test_properties_determine_table():
    """Exhaustive: among all width vectors summing to N, exactly one is
    balanced and non-increasing; it is the oracle's."""
    for N in range(1, 13):
        for H in range(1, 7):
            found = []
            for widths in itertools.product(range(N + 1), repeat=H):
                if sum(widths) != N:
                    continue
                if max(widths) - min(widths) > 1:
                    continue
                if any(widths[h] < widths[h + 1] for h in range(H - 1)):
                    continue
                found.append(widths)
            assert len(found) == 1
            lo, hi = oracle.band_table(N, H)
            assert tuple((hi - lo + 1).tolist()) == found[0]


def test_figure1_instance():
    # Figure 1: N = 1024, H = 8 -> eight bands of width 128, head 0 = [0, 127]
    lo, hi = oracle.band_table(1024, 8)
    assert lo.tolist() == [128 * h for h in range(8)]
    assert hi.tolist() == [128 * h + 127 for h in range(8)]


def test_uneven_split_n10000_h12():
    # 10000 = 12 * 833 + 4: four bands of 834 first, then eight of 833
    lo, hi = oracle.band_table(10000, 12)
    assert lo.tolist() == [0, 834, 1668, 2502, 3336, 4169, 5002, 5835, 6668, 7501, 8334, 9167]
    assert (hi - lo + 1).tolist() == [834] * 4 + [833] * 8
    assert hi[-1] == 9999


def test_more_heads_than_positions():
    lo, hi = oracle.band_table(3, 5)
    assert lo.tolist() == [0, 1, 2, 3, 3]
    assert hi.tolist() == [0, 1, 2, 2, 2]


def test_pair_count_factor_h():
    """The abstract's factor-H claim: the heads together attend N(N+1)/2
    pairs, a dense causal multi-head layer H * N(N+1)/2."""
    for N, H in [(1024, 8), (4096, 16), (8192, 32), (10000, 12), (7, 3), (5, 9)]:
        lo, hi = oracle.band_table(N, H)
        pairs = [oracle.band_pairs(N, lo[h], hi[h]) for h in range(H)]
        assert sum(pairs) == N * (N + 1) // 2
    lo, hi = oracle.band_table(1024, 8)
    assert [oracle.band_pairs(1024, lo[h], hi[h]) for h in range(8)] == [
        122944, 106560, 90176, 73792, 57408, 41024, 24640, 8256]


def test_band_pairs_brute_force():
    for N in range(1, 20):
        for lo_ in range(0, N + 1):
            for hi_ in range(lo_ - 1, N):
                m = oracle.band_mask(N, N, lo_, hi_)
                assert oracle.band_pairs(N, lo_, hi_) == int(m.sum())


def test_ablation_tables():
    lo, hi = oracle.band_table_sliding_window(1024, 8, 128)
    assert lo.tolist() == [0] * 8 and hi.tolist() == [127] * 8
    lo, hi = oracle.band_table_gapped_half(1024, 8)
    assert lo.tolist() == [128 * h for h in range(8)]
    assert hi.tolist() == [128 * h + 63 for h in range(8)]
    lo, hi = oracle.band_table_gapped_half(10, 4)  # widths 3, 3, 2, 2
    assert lo.tolist() == [0, 3, 6, 8] and hi.tolist() == [0, 3, 6, 8]


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.band_table(0, 4)
    with pytest.raises(ValueError):
        oracle.band_table(4, 0)
