"""GPU parity of the forward's online softmax where its reference maximum has
to move in the middle of a row's key walk, against the float64 oracle.

The forward keeps one reference maximum per query row and only moves it
(rescaling the accumulated output and row sum) when some score passes it by
more than the rescale window; with N(0, 1) inputs that happens almost only on
a row's first keys.  Here the key rows are scaled along the sequence so that
the largest score of a row keeps growing from one 32-key half to the next
(up), shrinks (down), jumps at a few isolated keys (spike), or steps up at
every 32-key boundary (staircase: most halves then fail the kept reference's
bound and take the update, at d = 64 after recomputing their scores), which
drives the move path, the correction factors and the rows that start with
every key masked.  The masked-set softmax being checked is "Sparse Attention, Then and
Now" section 1 over each head's band ("Making Every Head Count", Figure 1
caption).  Bars as elsewhere: float32 within 1e-4 max-abs; bfloat16 within
2e-2 max-abs and 1e-2 relative L2 (O) and 2e-2 max-abs (LSE); the positions
of LSE = -inf identical.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from structured_sparse_attention_spattn_amd import ops
from structured_sparse_attention_spattn_amd.inputs import as_f64, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
F32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_REL = 1e-2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_o(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    den = np.linalg.norm(ref)
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))
    _say(f"  {what}: max-abs {err:.3e}  rel-L2 {rel:.3e}")
    if dtype == "f32":
        assert err <= F32_TOL, f"{what}: max-abs {err:.3e}"
    else:
        assert err <= BF16_TOL and rel <= BF16_REL, f"{what}: max-abs {err:.3e}, rel-L2 {rel:.3e}"


def _check_lse(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    gi, ri = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"{what}: -inf positions differ"
    fin = ~ri
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    _say(f"  {what}: max-abs {err:.3e} over {int(fin.sum())} finite rows")
    assert err <= (F32_TOL if dtype == "f32" else BF16_TOL), f"{what}: max-abs {err:.3e}"


def _profile(kind, N):
    """Per-key scale factor of the key rows."""
    j = np.arange(N, dtype=np.float64)
    if kind == "up":
        return 1.0 + 16.0 * j / N
    if kind == "down":
        return 1.0 + 16.0 * (N - 1 - j) / N
    if kind == "spike":
        f = np.ones(N)
        f[np.arange(37, N, 211)] = 24.0
        return f
    if kind == "staircase":
        return 1.0 + 2.0 * (j // 32)
    raise ValueError(kind)


def _inputs(B, H, N, d, dtype, seed, kind):
    """Seeded inputs with the key rows scaled by the profile.  V is halved:
    with the attention concentrated on few keys, O is close to single V rows,
    and keeping |O| below about 2 keeps bfloat16's storage rounding of O (an
    ulp is 2^-7 |O|) well inside the bar, so the check measures the softmax."""
    inp = make_inputs(B, H, N, d, dtype=dtype, seed=seed)
    f = torch.from_numpy(_profile(kind, N).astype(np.float32))[None, None, :, None]
    inp["k"] = (inp["k"].float() * f).to(inp["k"].dtype)
    inp["v"] = (inp["v"].float() * 0.5).to(inp["v"].dtype)
    return inp


@pytest.mark.parametrize("kind", ["up", "down", "spike", "staircase"])
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("bands", ["bdp", "dense"])
def test_reference_moves_mid_walk(kind, dtype, d, bands):
    B, H, N = 2, 4, 1000  # ragged last tile, several walks per head
    seed = 4242 + d
    _say(f"reference moves: {kind} {dtype} d={d} bands={bands}")
    inp = _inputs(B, H, N, d, dtype, seed, kind)
    if bands == "bdp":
        lo, hi = oracle.band_table(N, H)
        band_arg = None
    else:
        lo, hi = np.zeros(H, np.int32), np.full(H, N - 1, np.int32)
        band_arg = (lo, hi)
    dv = {n: t.to(DEV) for n, t in inp.items()}
    o, lse = ops.fwd(dv["q"], dv["k"], dv["v"], bands=band_arg)
    torch.cuda.synchronize()
    ro, rl = oracle.band_attention_fwd(as_f64(inp["q"]), as_f64(inp["k"]), as_f64(inp["v"]), lo, hi)
    _check_o(o.float().cpu().numpy(), ro, dtype, "O")
    _check_lse(lse.cpu().numpy(), rl, dtype, "LSE")


@pytest.mark.parametrize("kind", ["up", "spike"])
@pytest.mark.parametrize("d", [64, 128])
def test_reference_moves_with_local_window(kind, d):
    """The two-range distance set (band plus a shared local window): a row's
    walk visits the window's keys and the band's, so the reference can move
    between the two runs."""
    B, H, N, w = 2, 4, 1000, 48
    _say(f"reference moves with window {w}: {kind} d={d}")
    inp = _inputs(B, H, N, d, "bf16", 777 + d, kind)
    lo, hi = oracle.band_table(N, H)
    dv = {n: t.to(DEV) for n, t in inp.items()}
    o, lse = ops.fwd(dv["q"], dv["k"], dv["v"], local_window=w)
    torch.cuda.synchronize()
    ro, rl = oracle.band_attention_fwd(as_f64(inp["q"]), as_f64(inp["k"]), as_f64(inp["v"]), lo, hi,
                                       local_window=w)
    _check_o(o.float().cpu().numpy(), ro, "bf16", "O")
    _check_lse(lse.cpu().numpy(), rl, "bf16", "LSE")
