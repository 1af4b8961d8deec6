"""Pins for the oracle's single-query decode over a key/value cache.

Independent of the decode code path: (1) the newest query's output equals the
last row of the already-pinned full forward oracle on the same sequence;
(2) Q = 0 gives the mean of v over the key set and LSE = ln |S|; (3) a
single band [0, N - 1] per head is causal attention of the last query, checked
against torch's float64 scaled_dot_product_attention (a library routine);
(4) a literal term-by-term evaluation on tiny inputs; (5) empty key sets give
0 / -inf.
"""
import math

import numpy as np
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_matches_last_row_of_full_forward():
    B, H, N, d = 2, 5, 70, 6
    lo, hi = oracle.band_table(N, H)
    q, k, v = (_rand((B, H, N, d), s) for s in (1, 2, 3))
    for w in (0, 4):
        out, lse = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
        for L in (1, 13, N):
            got, glse = oracle.decode_attention(q[:, :, L - 1], k, v, np.full(B, L), lo, hi, local_window=w)
            ref, rlse = oracle.band_attention_fwd(q[:, :, :L], k[:, :, :L], v[:, :, :L], lo, hi, local_window=w)
            assert np.max(np.abs(got - ref[:, :, L - 1])) <= 1e-12
            fin = np.isfinite(rlse[:, :, L - 1])
            assert np.array_equal(fin, np.isfinite(glse))
            assert np.max(np.abs(glse[fin] - rlse[:, :, L - 1][fin]), initial=0) <= 1e-12
        assert np.max(np.abs(oracle.decode_attention(q[:, :, N - 1], k, v, np.full(B, N), lo, hi,
                                                     local_window=w)[0] - out[:, :, N - 1])) <= 1e-12


def test_zero_query_mean():
    B, H, N, d, w = 1, 4, 50, 3, 5
    lo, hi = oracle.band_table(N, H)
    k, v = (_rand((B, H, N, d), s) for s in (5, 6))
    q = np.zeros((B, H, d))
    for L in (1, 7, 30, 50):
        out, lse = oracle.decode_attention(q, k, v, [L], lo, hi, local_window=w)
        i = L - 1
        for h in range(H):
            dists = [t for t in range(i + 1) if lo[h] <= t <= hi[h] or t < w]
            if not dists:
                assert np.all(out[0, h] == 0) and lse[0, h] == -np.inf
                continue
            mean = sum(v[0, h, i - t] for t in dists) / len(dists)
            assert np.max(np.abs(out[0, h] - mean)) <= 1e-12
            assert abs(lse[0, h] - math.log(len(dists))) <= 1e-12


def test_full_band_is_causal_sdpa_of_last_query():
    B, H, N, d = 2, 3, 40, 8
    q, k, v = (_rand((B, H, N, d), s) for s in (7, 8, 9))
    lo, hi = np.zeros(H, np.int32), np.full(H, N - 1, np.int32)
    got, _ = oracle.decode_attention(q[:, :, N - 1], k, v, np.full(B, N), lo, hi)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, :, N - 1:]), torch.from_numpy(k), torch.from_numpy(v)).numpy()[:, :, 0]
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_literal_terms_and_empty_sets():
    B, H, N, d = 1, 9, 6, 3   # H > N: empty bands
    lo, hi = oracle.band_table(N, H)
    q, k, v = _rand((B, H, d), 10), _rand((B, H, N, d), 11), _rand((B, H, N, d), 12)
    for L in (0, 1, 4, 6):
        out, lse = oracle.decode_attention(q, k, v, [L], lo, hi)
        for h in range(H):
            i = L - 1
            terms = [(math.exp(sum(q[0, h, c] * k[0, h, j, c] for c in range(d)) / math.sqrt(d)), j)
                     for j in range(max(L, 0)) if lo[h] <= i - j <= hi[h]]
            if not terms:
                assert np.all(out[0, h] == 0) and lse[0, h] == -np.inf
                continue
            den = sum(t for t, _ in terms)
            ref = [sum(t * v[0, h, j, c] for t, j in terms) / den for c in range(d)]
            assert np.max(np.abs(out[0, h] - np.array(ref))) <= 1e-12
            assert abs(lse[0, h] - math.log(den)) <= 1e-12
