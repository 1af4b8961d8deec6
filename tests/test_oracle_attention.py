"""Pins for the oracle's band attention, forward and backward.

What pins it (nothing here re-types the oracle's own formula):
* three independent forms agree (literal loop, dense explicit mask, blocked);
* closed forms: Q = 0 gives the mean of V over the key set and LSE = ln |S_i|;
  width-1 bands (H = N) copy v_{i-h}; V = 1 gives 1 on non-empty rows;
* a single band [0, N-1] is textbook causal attention: torch's float64
  scaled_dot_product_attention (a library routine) and its autograd;
* float64 central finite differences of a scalar loss for the gradients;
* gradient invariants (sum_j dK_j = 0, sum_j dV_j = sum of dO over non-empty rows).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sets(N, lo, hi):
    return [[j for j in range(N) if j <= i and lo <= i - j <= hi] for i in range(N)]


TINY_TABLES = [
    (7, 3, None), (9, 4, None), (5, 9, None), (12, 1, None), (10, 10, None),
    (11, 2, ([2, 0], [5, 10])),   # arbitrary (overlapping) bands
]


def _tables(N, H, custom):
    if custom is None:
        return oracle.band_table(N, H)
    return np.array(custom[0], dtype=np.int32), np.array(custom[1], dtype=np.int32)


@pytest.mark.parametrize("N,H,custom", TINY_TABLES)
def test_three_forms_agree(N, H, custom, monkeypatch):
    d = 5
    lo, hi = _tables(N, H, custom)
    q, k, v = (_rand((2, H, N, d), s) for s in (1, 2, 3))
    for block in (256, 3, 4):
        monkeypatch.setattr(oatt, "QUERY_BLOCK", block)
        out_b, lse_b = oracle.band_attention_fwd(q, k, v, lo, hi)
        for b in range(2):
            for h in range(H):
                mask = oracle.band_mask(N, N, int(lo[h]), int(hi[h]))
                out_d, lse_d, _ = oracle.masked_attention_dense(q[b, h], k[b, h], v[b, h], mask)
                out_l, lse_l = oracle.masked_attention_literal(
                    q[b, h], k[b, h], v[b, h], lambda i, j, m=mask: bool(m[i, j]))
                assert np.max(np.abs(out_b[b, h] - out_d)) <= 1e-12
                assert np.max(np.abs(out_l - out_d)) <= 1e-12
                fin = np.isfinite(lse_d)
                assert np.array_equal(fin, np.isfinite(lse_b[b, h])) and np.array_equal(fin, np.isfinite(lse_l))
                assert np.max(np.abs(lse_b[b, h][fin] - lse_d[fin]), initial=0) <= 1e-12
                assert np.max(np.abs(lse_l[fin] - lse_d[fin]), initial=0) <= 1e-12


def test_rows_api_matches_full():
    N, H, d = 37, 3, 4
    lo, hi = oracle.band_table(N, H)
    q, k, v = (_rand((1, H, N, d), s) for s in (4, 5, 6))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi)
    rows = [0, 5, 12, 13, 36]
    for h in range(H):
        o_r, l_r = oracle.band_attention_fwd_rows(q, k, v, lo, hi, 0, h, rows)
        assert np.max(np.abs(o_r - out[0, h, rows])) <= 1e-13
        assert np.array_equal(np.isfinite(l_r), np.isfinite(lse[0, h, rows]))


@pytest.mark.parametrize("N,H", [(13, 3), (40, 6), (64, 8), (9, 12)])
def test_closed_form_zero_queries(N, H):
    """Q = 0: every score is 0, so the softmax is uniform over S_i."""
    d = 6
    lo, hi = oracle.band_table(N, H)
    q = np.zeros((1, H, N, d))
    k = _rand((1, H, N, d), 7)
    v = _rand((1, H, N, d), 8)
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi)
    for h in range(H):
        prefix = np.vstack([np.zeros((1, d)), np.cumsum(v[0, h], axis=0)])
        for i in range(N):
            j_first = max(0, i - int(hi[h]))
            j_last = i - int(lo[h])
            if j_last < j_first:
                assert np.all(out[0, h, i] == 0) and lse[0, h, i] == -np.inf
                continue
            count = j_last - j_first + 1
            mean = (prefix[j_last + 1] - prefix[j_first]) / count
            assert np.max(np.abs(out[0, h, i] - mean)) <= 1e-12
            assert abs(lse[0, h, i] - math.log(count)) <= 1e-12


def test_closed_form_width_one_bands():
    """H = N: head h sees exactly key i - h, so O = v_{i-h} and
    LSE = q_i . k_{i-h} / sqrt(d)."""
    N = H = 11
    d = 4
    lo, hi = oracle.band_table(N, H)
    assert np.array_equal(lo, hi)
    q, k, v = (_rand((1, H, N, d), s) for s in (9, 10, 11))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi)
    for h in range(H):
        for i in range(N):
            if i < h:
                assert np.all(out[0, h, i] == 0) and lse[0, h, i] == -np.inf
            else:
                assert np.max(np.abs(out[0, h, i] - v[0, h, i - h])) <= 1e-14
                assert abs(lse[0, h, i] - q[0, h, i] @ k[0, h, i - h] / 2.0) <= 1e-13


def test_closed_form_unit_values():
    N, H, d = 50, 7, 3
    lo, hi = oracle.band_table(N, H)
    q, k = _rand((2, H, N, d), 12) * 4, _rand((2, H, N, d), 13)
    v = np.ones((2, H, N, d))
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi)
    nonempty = np.isfinite(lse)
    assert np.max(np.abs(out[nonempty] - 1.0)) <= 1e-12
    assert np.all(out[~nonempty] == 0)
    for h in range(H):
        assert np.array_equal(~nonempty[0, h], np.arange(N) < lo[h])


@pytest.mark.parametrize("N,d", [(1, 4), (17, 8), (64, 16), (300, 8)])
def test_single_band_is_causal_sdpa(N, d):
    q, k, v = (_rand((2, 3, N, d), s) for s in (14, 15, 16))
    lo = np.zeros(3, dtype=np.int32)
    hi = np.full(3, N - 1, dtype=np.int32)
    out, lse = oracle.band_attention_fwd(q, k, v, lo, hi)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
    s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    m = s.max(-1, keepdims=True)
    assert np.max(np.abs(lse - (m[..., 0] + np.log(np.exp(s - m).sum(-1))))) <= 1e-12


def test_h1_band_table_is_causal_sdpa():
    N, d = 33, 8
    lo, hi = oracle.band_table(N, 1)
    q, k, v = (_rand((1, 1, N, d), s) for s in (17, 18, 19))
    out, _ = oracle.band_attention_fwd(q, k, v, lo, hi)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_heads_sum_to_dense_causal_weights():
    """Exclusivity + completeness at the level of unnormalised weights: the
    heads' masked exp-score matrices, summed, give the dense causal one."""
    N, H, d = 23, 5, 4
    lo, hi = oracle.band_table(N, H)
    q, k = _rand((N, d), 20), _rand((N, d), 21)
    v = np.eye(N)  # out = P, row-normalised weights
    total = np.zeros((N, N))
    for h in range(H):
        mask = oracle.band_mask(N, N, int(lo[h]), int(hi[h]))
        _, lse, p = oracle.masked_attention_dense(q, k, v, mask)
        w = np.where(np.isfinite(lse)[:, None], p * np.exp(np.where(np.isfinite(lse), lse, 0))[:, None], 0)
        total += w
    s = q @ k.T / 2.0
    dense = np.where(np.tril(np.ones((N, N), dtype=bool)), np.exp(s), 0)
    assert np.max(np.abs(total - dense)) <= 1e-10 * np.max(dense)


# ---------------------------------------------------------------- backward


def _loss(q, k, v, w, lo, hi):
    out, _ = oracle.band_attention_fwd(q, k, v, lo, hi)
    return float((out * w).sum())


@pytest.mark.parametrize("N,H,custom", [(7, 3, None), (10, 4, None), (6, 8, None), (9, 2, ([1, 0], [3, 8]))])
def test_bwd_finite_differences(N, H, custom):
    d = 3
    lo, hi = _tables(N, H, custom)
    q, k, v, w = (_rand((1, H, N, d), s) for s in (30, 31, 32, 33))
    dq, dk, dv, _, _ = oracle.band_attention_bwd(q, k, v, w, lo, hi)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = dict(q=q, k=k, v=v); args_p[name] = xp
            args_m = dict(q=q, k=k, v=v); args_m[name] = xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], w, lo, hi)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], w, lo, hi)) / (2 * eps)
        scale = max(1e-3, np.max(np.abs(num)))
        assert np.max(np.abs(num - g)) / scale <= 1e-6, name


@pytest.mark.parametrize("N,d", [(5, 4), (40, 8)])
def test_bwd_single_band_matches_torch_autograd(N, d, monkeypatch):
    monkeypatch.setattr(oatt, "QUERY_BLOCK", 16)
    q, k, v, do = (_rand((2, 2, N, d), s) for s in (40, 41, 42, 43))
    lo = np.zeros(2, dtype=np.int32)
    hi = np.full(2, N - 1, dtype=np.int32)
    dq, dk, dv, out, _ = oracle.band_attention_bwd(q, k, v, do, lo, hi)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    o.backward(torch.from_numpy(do))
    assert np.max(np.abs(out - o.detach().numpy())) <= 1e-12
    assert np.max(np.abs(dq - tq.grad.numpy())) <= 1e-11
    assert np.max(np.abs(dk - tk.grad.numpy())) <= 1e-11
    assert np.max(np.abs(dv - tv.grad.numpy())) <= 1e-11


@pytest.mark.parametrize("N,H", [(29, 4), (16, 20)])
def test_bwd_dense_form_and_invariants(N, H, monkeypatch):
    monkeypatch.setattr(oatt, "QUERY_BLOCK", 8)
    d = 4
    lo, hi = oracle.band_table(N, H)
    q, k, v, do = (_rand((1, H, N, d), s) for s in (50, 51, 52, 53))
    dq, dk, dv, _, lse = oracle.band_attention_bwd(q, k, v, do, lo, hi)
    for h in range(H):
        mask = oracle.band_mask(N, N, int(lo[h]), int(hi[h]))
        rq, rk, rv = oracle.masked_attention_dense_bwd(q[0, h], k[0, h], v[0, h], do[0, h], mask)
        assert np.max(np.abs(dq[0, h] - rq)) <= 1e-12
        assert np.max(np.abs(dk[0, h] - rk)) <= 1e-12
        assert np.max(np.abs(dv[0, h] - rv)) <= 1e-12
        # sum over keys of dK is 0 (each row of dS sums to 0)
        assert np.max(np.abs(dk[0, h].sum(axis=0))) <= 1e-12
        nonempty = np.isfinite(lse[0, h])
        assert np.max(np.abs(dv[0, h].sum(axis=0) - do[0, h][nonempty].sum(axis=0))) <= 1e-12
        # rows with no keys and keys no query reaches get exactly 0
        assert np.all(dq[0, h][~nonempty] == 0)
        never = np.arange(N) > N - 1 - int(lo[h])
        assert np.all(dk[0, h][never] == 0) and np.all(dv[0, h][never] == 0)


def test_bwd_rows_api_matches_full(monkeypatch):
    monkeypatch.setattr(oatt, "QUERY_BLOCK", 8)
    N, H, d = 41, 3, 5
    lo, hi = oracle.band_table(N, H)
    q, k, v, do = (_rand((1, H, N, d), s) for s in (60, 61, 62, 63))
    dq, dk, dv, _, _ = oracle.band_attention_bwd(q, k, v, do, lo, hi)
    rows = [0, 3, 13, 14, 27, 40]
    for h in range(H):
        rq, rk, rv = oracle.band_attention_bwd_rows(q, k, v, do, lo, hi, 0, h, rows, rows)
        assert np.max(np.abs(rq - dq[0, h, rows])) <= 1e-12
        assert np.max(np.abs(rk - dk[0, h, rows])) <= 1e-12
        assert np.max(np.abs(rv - dv[0, h, rows])) <= 1e-12
