"""Pins for the oracle's local-sharing form (every head's set = its band joined
with a shared local window of distances [0, w - 1]).

Source: "Making Every Head Count", Figure 2 caption -- its exclusive-band
ablation is SPAttention with the local sharing removed.  The window width is
not given on the page; it is a parameter here.

What pins it (independent of the blocked code path that the GPU is compared
with):
* a literal per-element loop whose predicate is written from the set
  definition, and a dense explicit mask built element by element;
* reductions to the already-pinned exclusive-band oracle: w = 0 changes
  nothing; a head with an empty band sees exactly the sliding window
  [0, w - 1]; a window reaching the band (w >= lo) merges into the single band
  [0, max(hi, w - 1)];
* the closed form Q = 0: O_i = mean of v over the set, LSE_i = ln |S_i|, with
  |S_i| counted from the two distance ranges;
* float64 central finite differences for the gradients, and the row-sampling
  API against the full computation.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oatt


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _allowed(lo, hi, w):
    def f(i, j):
        dist = i - j
        return j <= i and ((lo <= dist <= hi) or (0 <= dist <= w - 1))
    return f


def _explicit_mask(N, lo, hi, w):
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(i + 1):
            m[i, j] = (lo <= i - j <= hi) or (i - j < w)
    return m


# (N, H, window): windows below, touching and overlapping the bands, and H > N
CASES = [(12, 3, 2), (12, 3, 4), (12, 3, 6), (16, 4, 3), (9, 12, 2), (20, 2, 1), (13, 5, 0)]


@pytest.mark.parametrize("N,H,w", CASES)
def test_forms_agree(N, H, w, monkeypatch):
    d = 4
    lo, hi = oracle.band_table(N, H)
    q, k, v = (_rand((1, H, N, d), s) for s in (41, 42, 43))
    for block in (256, 5):
        monkeypatch.setattr(oatt, "QUERY_BLOCK", block)
        out_b, lse_b = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
        for h in range(H):
            l, u = int(lo[h]), int(hi[h])
            mask = _explicit_mask(N, l, u, w)
            assert np.array_equal(mask, oracle.band_mask(N, N, l, u, local_window=w))
            out_d, lse_d, _ = oracle.masked_attention_dense(q[0, h], k[0, h], v[0, h], mask)
            out_l, lse_l = oracle.masked_attention_literal(q[0, h], k[0, h], v[0, h], _allowed(l, u, w))
            assert np.max(np.abs(out_l - out_d)) <= 1e-12
            assert np.max(np.abs(out_b[0, h] - out_d)) <= 1e-12
            fin = np.isfinite(lse_l)
            assert np.array_equal(fin, np.isfinite(lse_b[0, h]))
            assert np.max(np.abs(lse_b[0, h][fin] - lse_l[fin]), initial=0) <= 1e-12


def test_zero_window_is_exclusive_bands():
    N, H, d = 40, 4, 6
    lo, hi = oracle.band_table(N, H)
    q, k, v = (_rand((2, H, N, d), s) for s in (1, 2, 3))
    a, la = oracle.band_attention_fwd(q, k, v, lo, hi)
    b, lb = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=0)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_empty_band_is_sliding_window():
    # H > N: heads h >= N have an empty band (lo = N, hi = N - 1); with the
    # window they see exactly the band [0, w - 1] of the plain oracle.
    N, H, d, w = 6, 9, 4, 3
    lo, hi = oracle.band_table(N, H)
    q, k, v = (_rand((1, H, N, d), s) for s in (7, 8, 9))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    lo_w, hi_w = oracle.band_table_sliding_window(N, H, w)
    ref, ref_lse = oracle.band_attention_fwd(q, k, v, lo_w, hi_w)
    for h in range(N, H):
        assert np.max(np.abs(out[0, h] - ref[0, h])) <= 1e-12
        assert np.max(np.abs(lse[0, h] - ref_lse[0, h])) <= 1e-12


def test_window_reaching_band_merges():
    N, H, d = 30, 3, 5
    lo, hi = oracle.band_table(N, H)  # bands [0, 9], [10, 19], [20, 29]
    q, k, v = (_rand((1, H, N, d), s) for s in (11, 12, 13))
    for h in range(H):
        l, u = int(lo[h]), int(hi[h])
        for w in (l, l + 1, u + 3):  # window end w - 1 >= l - 1: touches or overlaps the band
            out, lse = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w, heads=[h])
            m_lo = np.array([0] * H, dtype=np.int32)
            m_hi = np.array([max(u, w - 1)] * H, dtype=np.int32)
            ref, ref_lse = oracle.band_attention_fwd(q, k, v, m_lo, m_hi, heads=[h])
            assert np.max(np.abs(out[0, h] - ref[0, h])) <= 1e-12
            assert np.max(np.abs(lse[0, h] - ref_lse[0, h])) <= 1e-12


@pytest.mark.parametrize("N,H,w", [(24, 3, 3), (17, 4, 5), (10, 12, 2)])
def test_closed_form_zero_queries(N, H, w):
    d = 3
    lo, hi = oracle.band_table(N, H)
    q = np.zeros((1, H, N, d))
    k, v = (_rand((1, H, N, d), s) for s in (21, 22))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    for h in range(H):
        l, u = int(lo[h]), int(hi[h])
        for i in range(N):
            # distances in the band or the window, counted as two ranges minus their overlap
            band = set(range(max(l, 0), min(u, i) + 1)) if u >= l else set()
            win = set(range(0, min(w - 1, i) + 1)) if w > 0 else set()
            dists = band | win
            if not dists:
                assert np.all(out[0, h, i] == 0) and lse[0, h, i] == -np.inf
                continue
            mean = sum(v[0, h, i - t] for t in dists) / len(dists)
            assert np.max(np.abs(out[0, h, i] - mean)) <= 1e-12
            assert abs(lse[0, h, i] - math.log(len(dists))) <= 1e-12


def _loss(q, k, v, g, lo, hi, w):
    out, _ = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    return float((out * g).sum())


@pytest.mark.parametrize("N,H,w", [(9, 3, 2), (8, 10, 2), (12, 2, 4)])
def test_bwd_finite_differences(N, H, w):
    d = 3
    lo, hi = oracle.band_table(N, H)
    q, k, v, g = (_rand((1, H, N, d), s) for s in (50, 51, 52, 53))
    dq, dk, dv, _, _ = oracle.band_attention_bwd(q, k, v, g, lo, hi, local_window=w)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = dict(q=q, k=k, v=v); args_p[name] = xp
            args_m = dict(q=q, k=k, v=v); args_m[name] = xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, lo, hi, w)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], g, lo, hi, w)) / (2 * eps)
        scale = max(1e-3, np.max(np.abs(num)))
        assert np.max(np.abs(num - grad)) / scale <= 1e-6, name


def test_bwd_dense_form():
    N, H, d, w = 14, 4, 4, 2
    lo, hi = oracle.band_table(N, H)
    q, k, v, g = (_rand((1, H, N, d), s) for s in (60, 61, 62, 63))
    dq, dk, dv, _, _ = oracle.band_attention_bwd(q, k, v, g, lo, hi, local_window=w)
    for h in range(H):
        mask = _explicit_mask(N, int(lo[h]), int(hi[h]), w)
        rq, rk, rv = oracle.masked_attention_dense_bwd(q[0, h], k[0, h], v[0, h], g[0, h], mask)
        assert np.max(np.abs(dq[0, h] - rq)) <= 1e-11
        assert np.max(np.abs(dk[0, h] - rk)) <= 1e-11
        assert np.max(np.abs(dv[0, h] - rv)) <= 1e-11


def test_rows_api_matches_full(monkeypatch):
    monkeypatch.setattr(oatt, "QUERY_BLOCK", 7)
    N, H, d, w = 33, 3, 4, 3
    lo, hi = oracle.band_table(N, H)
    q, k, v, g = (_rand((1, H, N, d), s) for s in (70, 71, 72, 73))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    dq, dk, dv, _, _ = oracle.band_attention_bwd(q, k, v, g, lo, hi, local_window=w)
    rows = [0, 1, 5, 10, 11, 20, 32]
    for h in range(H):
        o_r, l_r = oracle.band_attention_fwd_rows(q, k, v, lo, hi, 0, h, rows, local_window=w)
        assert np.max(np.abs(o_r - out[0, h, rows])) <= 1e-12
        fin = np.isfinite(lse[0, h, rows])
        assert np.array_equal(fin, np.isfinite(l_r))
        dq_r, dk_r, dv_r = oracle.band_attention_bwd_rows(q, k, v, g, lo, hi, 0, h, rows, rows, local_window=w)
        assert np.max(np.abs(dq_r - dq[0, h, rows])) <= 1e-11
        assert np.max(np.abs(dk_r - dk[0, h, rows])) <= 1e-11
        assert np.max(np.abs(dv_r - dv[0, h, rows])) <= 1e-11
