"""Single-query band attention over a key/value cache (oracle; test
infrastructure only).

The decode step of the same method: at sequence position i = L - 1 (L rows
of cache valid), head h attends the cached keys j with i - j in its band
[lo_h, hi_h] ("Making Every Head Count", Figure 1 caption: one contiguous
distance band per head) -- joined with the shared local window [0, w - 1]
when w > 0 (Figure 2 caption reading) -- through the masked-set softmax of
"Sparse Attention, Then and Now", section 1.  The pages measure training only;
this row is the same formula evaluated for the newest query.

Readings: an empty key set gives output 0 and LSE -inf (as in the forward);
LSE is the natural log of the sum of exponentials of scaled scores.
"""
import math

import numpy as np


def decode_key_set(i, lo, hi, local_window=0):
    """Cached key rows j (ascending) that query position i attends."""
    keys = [j for j in range(i + 1) if (lo <= i - j <= hi) or (i - j < local_window)]
    return np.array(keys, dtype=np.int64)


def decode_attention(q, k_cache, v_cache, lengths, lo, hi, local_window=0, scale=None):
    """q: [B, H, d]; k_cache, v_cache: [B, H, Nmax, d]; lengths: [B] (valid
    cache rows per sequence, >= 0).  Returns (out [B, H, d], lse [B, H]) in
    float64."""
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, H, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, H, v_cache.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(lengths[b])
        if L <= 0:
            continue
        i = L - 1
        for h in range(H):
            keys = decode_key_set(i, int(lo[h]), int(hi[h]), int(local_window))
            if keys.size == 0:
                continue
            s = (k_cache[b, h, keys] @ q[b, h]) * sc
            m = s.max()
            e = np.exp(s - m)
            out[b, h] = (e / e.sum()) @ v_cache[b, h, keys]
            lse[b, h] = m + math.log(e.sum())
    return out, lse
