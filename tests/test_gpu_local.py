"""GPU parity of band attention with a shared local window (spattn_fwd_local /
spattn_bwd_local) against the float64 oracle with the same window.

Source of the variant: "Making Every Head Count", Figure 2 caption (the
exclusive-band ablation is the method with local sharing removed); the window
width is a parameter (not given on the page).  Bars as elsewhere: bfloat16
outputs and gradients within 2e-2 max-abs and 1e-2 relative L2, -inf LSE
positions identical.  The full workload is compared on whole tensors.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from structured_sparse_attention_spattn_amd import ops
from structured_sparse_attention_spattn_amd.inputs import as_f64, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2
REL = 1e-2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / den if den > 0 else np.linalg.norm(got)
    _say(f"  {what}: max-abs {err:.3e}  rel-L2 {rel:.3e}")
    assert err <= TOL and rel <= REL, f"{what}: max-abs {err:.3e}, rel-L2 {rel:.3e}"


def _check_lse(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    gi, ri = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"{what}: -inf positions differ ({int((gi != ri).sum())} rows)"
    fin = ~ri
    if fin.any():
        assert float(np.max(np.abs(got[fin] - ref[fin]))) <= TOL, what


def _bands(kind, N, H):
    if kind == "bdp":
        return None, oracle.band_table(N, H)
    rng = np.random.default_rng(N * 7 + H)
    lo = rng.integers(0, N, H).astype(np.int32)
    hi = np.minimum(N - 1, lo + rng.integers(0, max(1, N // 3), H)).astype(np.int32)
    lo[0], hi[0] = min(N, 3), min(N, 3) - 1  # an empty band: the window alone
    return (lo, hi), (lo, hi)


LOCAL_SMALL = [
    # (B, H, N, d, window, bands, seed)
    (2, 4, 300, 64, 16, "bdp", 101),     # window below bands 1..3, merged into band 0
    (1, 6, 515, 128, 40, "bdp", 102),
    (1, 3, 257, 128, 86, "bdp", 103),    # window touching band 1 ([86, 171]) exactly
    (1, 3, 257, 128, 120, "bdp", 104),   # window overlapping band 1
    (1, 9, 7, 64, 2, "bdp", 105),        # H > N: empty bands see the window alone
    (1, 4, 130, 64, 1, "bdp", 106),      # window = the diagonal only
    (1, 2, 100, 128, 500, "bdp", 107),   # window wider than N
    (2, 5, 451, 64, 33, "odd", 108),     # arbitrary bands
]


@pytest.mark.parametrize("B,H,N,d,w,bk,seed", LOCAL_SMALL)
def test_local_fwd_bwd_small_vs_oracle(B, H, N, d, w, bk, seed):
    _say(f"local window small B={B} H={H} N={N} d={d} w={w} {bk} seed={seed}")
    inp = make_inputs(B, H, N, d, dtype="bf16", seed=seed, with_dout=True)
    band_arg, (lo, hi) = _bands(bk, N, H)
    x = {n: t.to(DEV) for n, t in inp.items()}
    o, lse = ops.fwd(x["q"], x["k"], x["v"], bands=band_arg, local_window=w)
    dq, dk, dv = ops.bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], bands=band_arg, grad_dtype=torch.float32,
                         local_window=w)
    dq16, dk16, dv16 = ops.bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], bands=band_arg, local_window=w)
    torch.cuda.synchronize()
    q, k, v, do = (as_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    ro, rl = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    _check(o.float().cpu().numpy(), ro, "O")
    _check_lse(lse.cpu().numpy(), rl, "LSE")
    rq, rk, rv, _, _ = oracle.band_attention_bwd(q, k, v, do, lo, hi, local_window=w)
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV"),
                         (dq16, rq, "dQ bf16"), (dk16, rk, "dK bf16"), (dv16, rv, "dV bf16")):
        _check(got.float().cpu().numpy(), ref, nm)


def test_zero_window_is_the_plain_entry_point():
    B, H, N, d = 2, 5, 333, 128
    x = {n: t.to(DEV) for n, t in make_inputs(B, H, N, d, dtype="bf16", seed=111, with_dout=True).items()}
    o0, l0 = ops.fwd(x["q"], x["k"], x["v"])
    lib = ops._lib.load()
    o1, l1 = torch.empty_like(o0), torch.empty_like(l0)
    st = lib.spattn_fwd_local(ops._ptr(x["q"]), ops._ptr(x["k"]), ops._ptr(x["v"]), ops._ptr(o1), ops._ptr(l1),
                              B, H, N, d, 1, None, None, 0, 0.0, ops._stream_handle(x["q"].device))
    assert st == 0
    g0 = ops.bwd(x["q"], x["k"], x["v"], o0, l0, x["dout"])
    ws = torch.empty(ops.bwd_workspace_bytes(B, H, N, d, torch.bfloat16, torch.bfloat16), dtype=torch.uint8,
                     device=DEV)
    g1 = tuple(torch.empty_like(o0) for _ in range(3))
    st = lib.spattn_bwd_local(*(ops._ptr(t) for t in (x["q"], x["k"], x["v"], o0, l0, x["dout"], *g1)),
                              B, H, N, d, 1, 1, None, None, 0, 0.0, ops._ptr(ws), ws.numel(),
                              ops._stream_handle(x["q"].device))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert all(torch.equal(a, b) for a, b in zip(g0, g1))


FULL = dict(B=8, H=16, N=4096, d=128, w=64, seed=1005)


def test_local_full_workload_whole_and_invariants():
    B, H, N, d, w = FULL["B"], FULL["H"], FULL["N"], FULL["d"], FULL["w"]
    _say(f"local window full workload B={B} H={H} N={N} d={d} w={w} (whole tensors)")
    inp = make_inputs(B, H, N, d, dtype="bf16", seed=FULL["seed"], with_dout=True)
    x = {n: t.to(DEV) for n, t in inp.items()}
    o, lse = ops.fwd(x["q"], x["k"], x["v"], local_window=w)
    dq, dk, dv = ops.bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], grad_dtype=torch.float32, local_window=w)
    torch.cuda.synchronize()
    lo, hi = oracle.band_table(N, H)
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    dq_h, dk_h, dv_h = (t.cpu().numpy() for t in (dq, dk, dv))
    del x, o, lse, dq, dk, dv
    assert not np.any(np.isneginf(lse_h))  # the window gives every row at least its diagonal
    do = as_f64(inp["dout"])
    for h in range(H):
        sk = dk_h[:, h].astype(np.float64).sum(axis=1)  # sum_j dK_j = 0 per (b, feature)
        assert np.max(np.abs(sk)) <= 2e-2 * max(1.0, np.max(np.abs(dk_h[:, h])) * math.sqrt(N)), h
        sv = dv_h[:, h].astype(np.float64).sum(axis=1)  # every row is non-empty: sum_j dV_j = sum_i dO_i
        ref_sv = do[:, h].sum(axis=1)
        assert np.max(np.abs(sv - ref_sv)) <= 2e-2 * max(1.0, np.max(np.abs(ref_sv))), h
    rq, rk, rv, ro, rl = oracle.band_attention_bwd(*(as_f64(inp[n]) for n in ("q", "k", "v", "dout")), lo, hi,
                                                   local_window=w)
    _check(o_h, ro, "O")
    _check_lse(lse_h, rl, "LSE")
    _check(dq_h, rq, "dQ")
    _check(dk_h, rk, "dK")
    _check(dv_h, rv, "dV")


def test_local_full_closed_form_zero_queries():
    # Q = 0: every score is 0, so O_i is the mean of v over the set and
    # LSE_i = ln |S_i|; checked on every row via prefix sums over the two ranges.
    B, H, N, d, w = 2, FULL["H"], FULL["N"], FULL["d"], FULL["w"]
    inp = make_inputs(B, H, N, d, dtype="bf16", seed=1006)
    q = torch.zeros_like(inp["q"]).to(DEV)
    o, lse = ops.fwd(q, inp["k"].to(DEV), inp["v"].to(DEV), local_window=w)
    torch.cuda.synchronize()
    lo, hi = oracle.band_table(N, H)
    v = inp["v"].double().numpy()
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    i = np.arange(N)
    for h in range(H):
        l, u = int(lo[h]), int(hi[h])
        # keys of row i: the band's [i - u, i - l] and the window's [i - w + 1, i], clipped at 0
        a1, b1 = np.maximum(0, i - u), i - l
        a2, b2 = np.maximum(0, i - w + 1), i
        has1 = b1 >= a1
        joined = has1 & (a2 <= b1 + 1)  # the two key ranges touch or overlap
        for b in range(B):
            pre = np.vstack([np.zeros((1, d)), np.cumsum(v[b, h], axis=0)])
            s2 = pre[b2 + 1] - pre[a2]
            n2 = b2 - a2 + 1
            s1 = np.where(has1[:, None], pre[np.maximum(b1, -1) + 1] - pre[a1], 0.0)
            n1 = np.where(has1, b1 - a1 + 1, 0)
            sj = pre[np.maximum(b1, b2) + 1] - pre[np.minimum(a1, a2)]
            nj = np.maximum(b1, b2) - np.minimum(a1, a2) + 1
            tot = np.where(joined[:, None], sj, s1 + s2)
            cnt = np.where(joined, nj, n1 + n2)
            mean = tot / cnt[:, None]
            err = np.max(np.abs(o_h[b, h] - mean))
            assert err <= TOL, (h, b, err)
            assert np.max(np.abs(lse_h[b, h] - np.log(cnt))) <= 1e-3, h


LOCAL_F32 = [
    # (B, H, N, d, window, bands, seed): float32 inputs and gradients, bar 1e-4 max-abs
    (1, 4, 300, 64, 16, "bdp", 121),
    (2, 3, 257, 128, 120, "bdp", 122),
    (1, 9, 7, 64, 2, "bdp", 123),
    (1, 5, 200, 64, 7, "odd", 124),
    (4, 16, 1024, 64, 40, "bdp", 125),  # 1024 tiles of 64 rows: the two-wave float32 kernels, not the split ones
]


@pytest.mark.parametrize("B,H,N,d,w,bk,seed", LOCAL_F32)
def test_local_f32_vs_oracle(B, H, N, d, w, bk, seed):
    _say(f"local window f32 B={B} H={H} N={N} d={d} w={w} {bk} seed={seed}")
    inp = make_inputs(B, H, N, d, dtype="f32", seed=seed, with_dout=True)
    band_arg, (lo, hi) = _bands(bk, N, H)
    x = {n: t.to(DEV) for n, t in inp.items()}
    o, lse = ops.fwd(x["q"], x["k"], x["v"], bands=band_arg, local_window=w)
    dq, dk, dv = ops.bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], bands=band_arg, local_window=w)
    torch.cuda.synchronize()
    q, k, v, do = (as_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    ro, rl = oracle.band_attention_fwd(q, k, v, lo, hi, local_window=w)
    rq, rk, rv, _, _ = oracle.band_attention_bwd(q, k, v, do, lo, hi, local_window=w)
    lse_h = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lse_h), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(lse_h[fin] - rl[fin]), initial=0) <= 1e-4
    for got, ref, nm in ((o, ro, "O"), (dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - ref)))
        assert err <= 1e-4, f"{nm}: max-abs {err:.3e}"
