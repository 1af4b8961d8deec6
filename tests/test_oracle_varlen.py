"""Pins for the oracle's packed variable-length form.

The packed batch is the method applied to each sequence on its own (positions
restart at 0, nothing crosses a sequence boundary), with each sequence's own
Balanced Distance Partitioning table ("Making Every Head Count", Figure 1
caption) or a shared caller table clipped to its length.  Pinned by:
* a literal per-element evaluation over the packed token index, whose
  predicate is written from that definition (same sequence, positions, set);
* isolation: changing one sequence's inputs leaves every other sequence's
  outputs and gradients bit-identical;
* the one-sequence batch equals the fixed-length oracle with band_table(T, H);
* float64 central finite differences for the gradients.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _seq_of(cu):
    cu = list(cu)
    seq = []
    for s in range(len(cu) - 1):
        seq += [s] * (cu[s + 1] - cu[s])
    return seq


def _literal(q, k, v, cu, H, bands, w):
    seq = _seq_of(cu)
    out = np.zeros_like(q)
    lse = np.full(q.shape[:2], -np.inf)
    for h in range(H):
        def allowed(t, u, h=h):
            s = seq[t]
            if seq[u] != s:
                return False
            n = cu[s + 1] - cu[s]
            if bands is None:
                base, extra = divmod(n, H)
                lo = h * base + min(h, extra)
                hi = lo + base + (1 if h < extra else 0) - 1
            else:
                lo, hi = min(int(bands[0][h]), n), min(int(bands[1][h]), n - 1)
            i, j = t - cu[s], u - cu[s]
            return j <= i and (lo <= i - j <= hi or i - j < w)
        out[h], lse[h] = oracle.masked_attention_literal(q[h], k[h], v[h], allowed)
    return out, lse


CASES = [
    ([0, 5, 12, 13, 21], 3, None, 0),
    ([0, 9, 9, 17], 4, None, 2),                       # an empty sequence
    ([0, 6, 16, 20], 2, (np.array([0, 3]), np.array([2, 7])), 0),
    ([0, 4, 14], 5, None, 0),                           # H > n for the first sequence
    ([0, 11, 20], 3, (np.array([0, 2, 5]), np.array([1, 4, 9])), 3),
]


@pytest.mark.parametrize("cu,H,bands,w", CASES)
def test_literal_packed(cu, H, bands, w):
    T, d = cu[-1], 3
    q, k, v = (_rand((H, T, d), s) for s in (1, 2, 3))
    out, lse = oracle.varlen_fwd(q, k, v, cu, bands=bands, local_window=w)
    ref, ref_lse = _literal(q, k, v, cu, H, bands, w)
    assert np.max(np.abs(out - ref)) <= 1e-12
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0) <= 1e-12


def test_isolation_between_sequences():
    cu, H, d = [0, 7, 19, 26], 3, 4
    T = cu[-1]
    q, k, v, g = (_rand((H, T, d), s) for s in (11, 12, 13, 14))
    base = oracle.varlen_bwd(q, k, v, g, cu)
    k2, v2, q2, g2 = k.copy(), v.copy(), q.copy(), g.copy()
    sl = slice(cu[1], cu[2])
    for t in (k2, v2, q2, g2):
        t[:, sl] += _rand(t[:, sl].shape, 99)
    pert = oracle.varlen_bwd(q2, k2, v2, g2, cu)
    keep = np.r_[0:cu[1], cu[2]:cu[3]]
    for a, b in zip(base, pert):
        assert np.array_equal(a[:, keep], b[:, keep])


def test_single_sequence_is_fixed_length():
    H, T, d = 4, 23, 5
    q, k, v, g = (_rand((H, T, d), s) for s in (21, 22, 23, 24))
    lo, hi = oracle.band_table(T, H)
    out, lse = oracle.varlen_fwd(q, k, v, [0, T])
    ref, ref_lse = oracle.band_attention_fwd(q[None], k[None], v[None], lo, hi)
    assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref_lse[0])
    dq, dk, dv, _, _ = oracle.varlen_bwd(q, k, v, g, [0, T], local_window=3)
    rq, rk, rv, _, _ = oracle.band_attention_bwd(q[None], k[None], v[None], g[None], lo, hi, local_window=3)
    assert np.array_equal(dq, rq[0]) and np.array_equal(dk, rk[0]) and np.array_equal(dv, rv[0])


def test_seq_bands_clip():
    lo, hi = oracle.seq_bands(5, 3, (np.array([0, 3, 7]), np.array([2, 9, 12])))
    assert list(lo) == [0, 3, 5] and list(hi) == [2, 4, 4]
    lo, hi = oracle.seq_bands(10, 4)
    blo, bhi = oracle.band_table(10, 4)
    assert np.array_equal(lo, blo) and np.array_equal(hi, bhi)


def test_bwd_finite_differences():
    cu, H, d = [0, 4, 9], 2, 3
    T = cu[-1]
    q, k, v, g = (_rand((H, T, d), s) for s in (31, 32, 33, 34))
    dq, dk, dv, _, _ = oracle.varlen_bwd(q, k, v, g, cu, local_window=1)

    def loss(q_, k_, v_):
        o, _ = oracle.varlen_fwd(q_, k_, v_, cu, local_window=1)
        return float((o * g).sum())
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p[name] = xp
            args_m[name] = xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        assert np.max(np.abs(num - grad)) / max(1e-3, np.max(np.abs(num))) <= 1e-6, name
