"""GPU parity of the decode step (spattn_decode: one new query per sequence
against a key/value cache) with the float64 decode oracle.

Bars: float32 within 1e-4 max-abs; bfloat16 within 2e-2 max-abs and 1e-2
relative L2; LSE -inf positions (empty key sets) identical.  Small caches are
compared completely, the decode workload (64 sequences of a 4096-row cache,
16 heads, d = 128, ragged lengths) on every output as well.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from structured_sparse_attention_spattn_amd import ops
from structured_sparse_attention_spattn_amd.inputs import as_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(B, H, Nmax, d, dtype, seed):
    """Seeded N(0, 1) query [B, H, d] and caches [B, H, Nmax, d], quantised once."""
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, H, d)).astype(np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((B, H, Nmax, d)).astype(np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((B, H, Nmax, d)).astype(np.float32)).to(tdt)
    return q, k, v


def _compare(o, lse, ro, rl, dtype, what):
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), f"{what}: -inf positions"
    fin = np.isfinite(rl)
    err = float(np.max(np.abs(o - ro)))
    lerr = float(np.max(np.abs(lse[fin] - rl[fin]), initial=0.0))
    if dtype == "f32":
        assert err <= 1e-4 and lerr <= 1e-4, f"{what}: max-abs {err:.3e} lse {lerr:.3e}"
    else:
        den = np.linalg.norm(ro)
        rel = np.linalg.norm(o - ro) / den if den > 0 else np.linalg.norm(o)
        assert err <= 2e-2 and rel <= 1e-2 and lerr <= 2e-2, f"{what}: max-abs {err:.3e} rel {rel:.3e}"


DECODE_SMALL = [
    # (B, H, Nmax, d, dtype, lengths, bands, window, seed)
    (3, 4, 300, 128, "bf16", [300, 1, 157], "bdp", 0, 201),
    (3, 4, 300, 64, "bf16", [0, 299, 75], "bdp", 0, 202),      # an empty cache row count
    (2, 5, 200, 128, "f32", None, "bdp", 0, 203),              # no lengths: all Nmax rows
    (2, 6, 513, 64, "f32", [513, 260], "bdp", 16, 204),        # window below the bands
    (4, 3, 700, 128, "bf16", [700, 10, 400, 233], "bdp", 64, 205),
    (2, 9, 7, 64, "bf16", [7, 3], "bdp", 0, 206),              # H > N: empty bands
    (2, 9, 7, 128, "bf16", [7, 3], "bdp", 2, 207),             # ... which see the window
    (2, 4, 1000, 128, "bf16", [1000, 640], "odd", 5, 208),     # arbitrary bands
]


def _bands(kind, N, H):
    if kind == "bdp":
        return None, oracle.band_table(N, H)
    rng = np.random.default_rng(N + H)
    lo = rng.integers(0, N, H).astype(np.int32)
    hi = np.minimum(N - 1, lo + rng.integers(0, max(1, N // 3), H)).astype(np.int32)
    lo[0], hi[0] = min(N, 3), min(N, 3) - 1
    return (lo, hi), (lo, hi)


@pytest.mark.parametrize("B,H,Nmax,d,dtype,lengths,bk,w,seed", DECODE_SMALL)
def test_decode_small_vs_oracle(B, H, Nmax, d, dtype, lengths, bk, w, seed):
    _say(f"decode small B={B} H={H} Nmax={Nmax} d={d} {dtype} lengths={lengths} {bk} w={w}")
    q, k, v = _inputs(B, H, Nmax, d, dtype, seed)
    band_arg, (lo, hi) = _bands(bk, Nmax, H)
    lens = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device=DEV)
    o, lse = ops.decode(q.to(DEV), k.to(DEV), v.to(DEV), lengths=lens, bands=band_arg, local_window=w)
    torch.cuda.synchronize()
    ref_len = np.full(B, Nmax) if lengths is None else np.array(lengths)
    ro, rl = oracle.decode_attention(as_f64(q), as_f64(k), as_f64(v), ref_len, lo, hi, local_window=w)
    _compare(o, lse, ro, rl, dtype, "decode")


@pytest.mark.parametrize("w", [0, 64])
def test_decode_workload_all_outputs(w):
    B, H, Nmax, d = 64, 16, 4096, 128
    _say(f"decode workload B={B} H={H} Nmax={Nmax} d={d} w={w}")
    q, k, v = _inputs(B, H, Nmax, d, "bf16", 1010)
    rng = np.random.default_rng(1011)
    lengths = rng.integers(1, Nmax + 1, B).astype(np.int32)
    lengths[:3] = [Nmax, 1, 256]
    o, lse = ops.decode(q.to(DEV), k.to(DEV), v.to(DEV), lengths=torch.from_numpy(lengths).to(DEV), local_window=w)
    torch.cuda.synchronize()
    lo, hi = oracle.band_table(Nmax, H)
    ro, rl = oracle.decode_attention(as_f64(q), as_f64(k), as_f64(v), lengths, lo, hi, local_window=w)
    _compare(o, lse, ro, rl, "bf16", "decode workload")
