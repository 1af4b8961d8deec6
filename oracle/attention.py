"""Masked-set attention, forward and backward, in float64 (oracle; test
infrastructure only).

Definition: "Story of Attention -- Part 4: Sparse Attention, Then and Now",
section 1 (Sparse Transformer), the sparse-attention formula: for query i and
its permitted key set S_i,

    out_i = sum_{j in S_i} exp(q_i . k_j / sqrt(d_k)) / sum_{m in S_i} exp(q_i . k_m / sqrt(d_k)) * v_j

i.e. ordinary attention whose softmax runs only over S_i.  SPAttention
("Making Every Head Count", Figure 1 caption and abstract) gives head h the
set S_i^h = { j : 0 <= j <= i, lo_h <= i - j <= hi_h }, one contiguous band of
causal distances per head.

Local sharing: the same page's Figure 2 caption describes its exclusive-band
ablation as SPAttention with the local sharing removed, so the full method
also lets every head see a shared local window.  Reading (width not given):
head h's set becomes S_i^h united with { j : 0 <= i - j <= w - 1 } for a
window width w >= 0 (w = 0 is the exclusive-band method above).  Every
function below takes ``local_window`` = w, default 0.

Readings (pages silent): an empty S_i gives output 0 and LSE = -inf;
LSE_i = ln sum_{j in S_i} exp(scaled score); the backward pass is the
textbook derivative of the formula (D_i = dO_i . O_i, dS = P * (dP - D)).

Three independent forms are kept so the tests can cross-check them:

* ``masked_attention_literal`` -- a per-element Python loop over S_i, written
  exactly as the formula reads (tiny shapes only);
* ``masked_attention_dense`` / ``masked_attention_dense_bwd`` -- one head, a
  full N x N score matrix with an explicit boolean mask;
* ``band_attention_fwd`` / ``band_attention_bwd`` -- all of [B, H, N, d], per
  (b, h) and per block of query rows, gathering only the key rows the band can
  reach and masking element by element.  Used at full workload sizes.
"""
import math

import numpy as np

QUERY_BLOCK = 256


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def masked_attention_literal(q, k, v, allowed, scale=None):
    """One head.  q, k: [N, d]; v: [N, dv]; allowed(i, j) -> bool.

    Returns (out [N, dv], lse [N]).  Every sum is written out term by term.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    dv = v.shape[1]
    sc = _default_scale(d, scale)
    out = np.zeros((n, dv))
    lse = np.full(n, -np.inf)
    for i in range(n):
        s_i = [j for j in range(k.shape[0]) if allowed(i, j)]
        if not s_i:
            continue
        scores = {}
        for j in s_i:
            dot = 0.0
            for c in range(d):
                dot += q[i, c] * k[j, c]
            scores[j] = dot * sc
        denom = 0.0
        for m in s_i:
            denom += math.exp(scores[m])
        for j in s_i:
            w = math.exp(scores[j]) / denom
            for c in range(dv):
                out[i, c] += w * v[j, c]
        lse[i] = math.log(denom)
    return out, lse


def _in_set(dist, lo, hi, local_window=0):
    """Is causal distance `dist` in head (lo, hi)'s set: the band [lo, hi] or
    the shared local window [0, local_window - 1]?"""
    m = (dist >= max(lo, 0)) & (dist <= hi)
    if local_window > 0:
        m = m | ((dist >= 0) & (dist <= local_window - 1))
    return m


def band_mask(n_q, n_k, lo, hi, local_window=0):
    """Boolean [n_q, n_k] mask of head (lo, hi): j <= i and lo <= i - j <= hi
    (or 0 <= i - j < local_window)."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    dist = i - j
    return (j <= i) & _in_set(dist, lo, hi, local_window)


def masked_attention_dense(q, k, v, mask, scale=None):
    """One head with an explicit [N, N] boolean mask.  Returns (out, lse, p)
    where p is the [N, N] probability matrix (0 off the mask)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sc = _default_scale(q.shape[1], scale)
    s = (q @ k.T) * sc
    s = np.where(mask, s, -np.inf)
    row_max = s.max(axis=1)
    nonempty = mask.any(axis=1)
    shift = np.where(nonempty, row_max, 0.0)
    e = np.where(mask, np.exp(s - shift[:, None]), 0.0)
    denom = e.sum(axis=1)
    safe = np.where(nonempty, denom, 1.0)
    p = e / safe[:, None]
    out = p @ v
    lse = np.where(nonempty, shift + np.log(safe), -np.inf)
    return out, lse, p


def masked_attention_dense_bwd(q, k, v, dout, mask, scale=None):
    """Textbook gradient of ``masked_attention_dense`` for one head.

    Returns (dq, dk, dv).  P is recomputed here; D_i = dO_i . O_i uses the
    float64 forward output of this same function.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    sc = _default_scale(q.shape[1], scale)
    out, _, p = masked_attention_dense(q, k, v, mask, sc)
    dv = p.T @ dout
    dp = dout @ v.T
    dcoef = (dout * out).sum(axis=1)
    ds = p * (dp - dcoef[:, None])
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def _key_range(i0, i1, lo, hi):
    """Keys a block of query rows [i0, i1) can reach in band [lo, hi]:
    j from max(0, i0 - hi) to (i1 - 1) - lo inclusive (empty if it ends < 0)."""
    return max(0, i0 - hi), (i1 - 1) - lo


def _key_index(i0, i1, lo, hi, local_window=0):
    """Sorted key rows a block of query rows [i0, i1) can reach: the band's
    range, joined with [max(0, i0 - w + 1), i1 - 1] for a local window w."""
    parts = []
    if hi >= lo:
        j0, j1 = _key_range(i0, i1, lo, hi)
        if j1 >= j0:
            parts.append(np.arange(j0, j1 + 1))
    if local_window > 0:
        parts.append(np.arange(max(0, i0 - local_window + 1), i1))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(parts))


def _query_index(j, lo, hi, N, local_window=0):
    """Query rows i < N whose set contains key row j."""
    parts = []
    if hi >= lo and j + lo <= N - 1:
        parts.append(np.arange(j + lo, min(N - 1, j + hi) + 1))
    if local_window > 0:
        parts.append(np.arange(j, min(N - 1, j + local_window - 1) + 1))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(parts))


def _block_forward(qb, kb, vb, i0, jidx, lo, hi, sc, local_window=0):
    """Forward on one query block against the gathered key rows jidx."""
    n_q = qb.shape[0]
    i = (i0 + np.arange(n_q))[:, None]
    j = np.asarray(jidx)[None, :]
    dist = i - j
    mask = _in_set(dist, lo, hi, local_window)
    s = np.where(mask, (qb @ kb.T) * sc, -np.inf)
    nonempty = mask.any(axis=1)
    shift = np.where(nonempty, s.max(axis=1), 0.0)
    e = np.where(mask, np.exp(s - shift[:, None]), 0.0)
    denom = e.sum(axis=1)
    safe = np.where(nonempty, denom, 1.0)
    p = e / safe[:, None]
    out = p @ vb
    lse = np.where(nonempty, shift + np.log(safe), -np.inf)
    return out, lse, p


def band_attention_fwd(q, k, v, lo, hi, scale=None, heads=None, local_window=0):
    """Band attention over [B, H, N, d] inputs.

    lo, hi: per-head inclusive distance bounds (length H).  Returns
    (out [B, H, N, dv] float64, lse [B, H, N] float64).  ``heads`` optionally
    restricts the work to a subset of head indices (others are left 0/-inf).
    ``local_window`` adds the shared local window to every head's set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    sc = _default_scale(d, scale)
    out = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.full((B, H, N), -np.inf)
    w = int(local_window)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            l, u = int(lo[h]), int(hi[h])
            if u < l and w == 0:
                continue
            for i0 in range(0, N, QUERY_BLOCK):
                i1 = min(N, i0 + QUERY_BLOCK)
                jidx = _key_index(i0, i1, l, u, w)
                if jidx.size == 0:
                    continue
                o_blk, l_blk, _ = _block_forward(q[b, h, i0:i1], k[b, h, jidx], v[b, h, jidx], i0, jidx,
                                                 l, u, sc, w)
                out[b, h, i0:i1] = o_blk
                lse[b, h, i0:i1] = l_blk
    return out, lse


def band_attention_fwd_rows(q, k, v, lo, hi, b, h, rows, scale=None, local_window=0):
    """Forward for selected query rows of one (b, h) only -- each row is
    computed on its own from the definition.  Returns (out [len(rows), dv],
    lse [len(rows)]).  Used to check sampled outputs at full sizes."""
    d = q.shape[3]
    sc = _default_scale(d, scale)
    l, u = int(lo[h]), int(hi[h])
    outs = np.zeros((len(rows), v.shape[3]))
    lses = np.full(len(rows), -np.inf)
    for r, i in enumerate(rows):
        jidx = _key_index(i, i + 1, l, u, int(local_window))
        if jidx.size == 0:
            continue
        qb = np.asarray(q[b, h, i:i + 1], dtype=np.float64)
        kb = np.asarray(k[b, h, jidx], dtype=np.float64)
        vb = np.asarray(v[b, h, jidx], dtype=np.float64)
        o_blk, l_blk, _ = _block_forward(qb, kb, vb, i, jidx, l, u, sc, int(local_window))
        outs[r] = o_blk[0]
        lses[r] = l_blk[0]
    return outs, lses


def band_attention_bwd(q, k, v, dout, lo, hi, scale=None, local_window=0):
    """Gradients of band attention over [B, H, N, d].

    Recomputes the forward in float64 per query block, then per block:
    dV_J += P^T dO, dP = dO V_J^T, dS = P * (dP - D) with D_i = dO_i . O_i,
    dQ = scale * dS K_J, dK_J += scale * dS^T Q.  Rows with an empty key set
    have P = 0 and contribute nothing.  Returns (dq, dk, dv, out, lse).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, N, d = q.shape
    sc = _default_scale(d, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.full((B, H, N), -np.inf)
    w = int(local_window)
    for b in range(B):
        for h in range(H):
            l, u = int(lo[h]), int(hi[h])
            if u < l and w == 0:
                continue
            for i0 in range(0, N, QUERY_BLOCK):
                i1 = min(N, i0 + QUERY_BLOCK)
                jidx = _key_index(i0, i1, l, u, w)
                if jidx.size == 0:
                    continue
                qb = q[b, h, i0:i1]
                kb = k[b, h, jidx]
                vb = v[b, h, jidx]
                dob = dout[b, h, i0:i1]
                o_blk, l_blk, p = _block_forward(qb, kb, vb, i0, jidx, l, u, sc, w)
                out[b, h, i0:i1] = o_blk
                lse[b, h, i0:i1] = l_blk
                dcoef = (dob * o_blk).sum(axis=1)
                dv[b, h, jidx] += p.T @ dob
                dp = dob @ vb.T
                ds = p * (dp - dcoef[:, None])
                dq[b, h, i0:i1] = sc * (ds @ kb)
                dk[b, h, jidx] += sc * (ds.T @ qb)
    return dq, dk, dv, out, lse


def band_attention_bwd_rows(q, k, v, dout, lo, hi, b, h, q_rows, k_rows, scale=None, local_window=0):
    """Gradients for selected rows of one (b, h), each from the definition.

    dq[r] = scale * sum_j dS_ij k_j for query row i = q_rows[r];
    dk[r] = scale * sum_i dS_ij q_i and dv[r] = sum_i P_ij dO_i for key row
    j = k_rows[r], summing over the queries i whose band reaches j.  Every
    query row involved gets its own forward (O_i, LSE_i) and D_i = dO_i . O_i.
    Returns (dq [len(q_rows), d], dk [len(k_rows), d], dv [len(k_rows), dv]).
    """
    d = q.shape[3]
    N = q.shape[2]
    sc = _default_scale(d, scale)
    l, u = int(lo[h]), int(hi[h])
    f64 = lambda x: np.asarray(x, dtype=np.float64)

    w = int(local_window)

    def row_terms(i):
        """(key rows jidx, P_i over them, dS_i over them) or None if empty."""
        jidx = _key_index(i, i + 1, l, u, w)
        if jidx.size == 0:
            return None
        qi = f64(q[b, h, i])
        kb, vb = f64(k[b, h, jidx]), f64(v[b, h, jidx])
        s = (kb @ qi) * sc
        m = s.max()
        e = np.exp(s - m)
        p = e / e.sum()
        o_i = p @ vb
        do_i = f64(dout[b, h, i])
        dcoef = float(do_i @ o_i)
        ds = p * (vb @ do_i - dcoef)
        return jidx, p, ds

    dq = np.zeros((len(q_rows), d))
    for r, i in enumerate(q_rows):
        t = row_terms(i)
        if t is not None:
            jidx, _, ds = t
            dq[r] = sc * (ds @ f64(k[b, h, jidx]))
    dk = np.zeros((len(k_rows), d))
    dv = np.zeros((len(k_rows), v.shape[3]))
    for r, j in enumerate(k_rows):
        for i in _query_index(j, l, u, N, w):
            jidx, p, ds = row_terms(int(i))
            pos = int(np.searchsorted(jidx, j))
            dk[r] += sc * ds[pos] * f64(q[b, h, i])
            dv[r] += p[pos] * f64(dout[b, h, i])
    return dq, dk, dv
