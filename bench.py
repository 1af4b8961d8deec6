"""Benchmark of band-partitioned (SPAttention) attention on one MI355X.

One step = the whole hot path over one batch: spattn_fwd (band table, band
tile schedule, scores, masks, online softmax, P V, epilogue) followed by
spattn_bwd's two stages (D = rowsum(dO * O) and band-tiled dQ; then band-tiled
dK / dV), on B = 8, H = 16, N = 4096, d = 128, bfloat16 inputs resident in HBM.

Prints ONE JSON line.  ``value`` is in-band TFLOP/s of fwd+bwd (14 d FLOP per
attended pair; the heads together attend N(N+1)/2 pairs per sequence) with
L2 and the MALL evicted before every timed step (a 512 MiB read outside the
events: the caches then hold only clean lines of an unrelated buffer), so
every input comes from HBM and no step pays for writing back another
buffer's dirty lines; the timed steps follow about 150 ms of untimed steps,
so that they run at the clocks a continuous run holds.  ``fill_flushed``
holds the same steps after a 512 MiB fill instead of the read, and
``cold_start`` the steps of the first run (fill, no settle); ``warm`` holds
the same steps back to back.  Extra keys: per-kernel times and HBM fractions, the roofline
of the dominant kernel, the dense-causal kernel of the same library at the
same shape, the forward of the other workloads (evicted) each next to the
float64 CPU oracle timed on this host, the page's ablation patterns and the
shared local window ("variants"), a decode step, the measured MFMA and HBM
denominators next to the published ones, and the oracle's fwd+bwd time.
"""
import argparse
import ctypes
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

B, H, N, D = 8, 16, 4096, 128
SEED = 1005
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_PEAK_TFLOPS = 157.3  # fp32 matrix (and vector) peak
FLUSH_BYTES = 512 << 20
SETTLE_MS = 150.0  # untimed steps before the headline, for the clocks to settle


class Evictor:
    """Evicts L2 and the MALL before a timed launch.  "read" (the default)
    reads a 512 MiB buffer (one reduction), which leaves only clean lines of
    that buffer in the caches and writes back whatever was dirty there
    before the timed region starts.  "fill" writes 512 MiB instead, which
    leaves the caches full of dirty lines whose write-back then falls inside
    the next timed launch."""

    def __init__(self, dev):
        import torch
        self.rd = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.fill = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def __call__(self, how="read"):
        if how == "fill":
            self.fill.zero_()
        else:
            self.rd.sum()


def kernel_source_hash():
    """sha256 over every file of the HIP sources (name + bytes, sorted)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "structured_sparse_attention_spattn_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (copy-calibrated), or None when the kernel sources have
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_B8_H16_N4096_d128.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["traffic_bytes"])


def pairs_total(lo, hi, local_window=0, seq_len=None, batch=None):
    """Attended causal pairs over all heads and the batch: per head, the
    distances in [lo_h, hi_h] (joined with [0, local_window - 1]), each
    distance d contributing N - d query rows (N, B: the bench workload's
    unless given)."""
    N = seq_len if seq_len is not None else globals()["N"]
    B = batch if batch is not None else globals()["B"]
    tot = 0
    for l, u in zip(lo, hi):
        ranges = []
        if int(u) >= int(l):
            ranges.append([int(l), int(u)])
        if local_window > 0:
            ranges.append([0, min(N, local_window) - 1])
        ranges.sort()
        merged = []
        for a, b in ranges:
            if merged and a <= merged[-1][1] + 1:
                merged[-1][1] = max(merged[-1][1], b)
            else:
                merged.append([a, b])
        for a, b in merged:
            w = b - a + 1
            tot += w * (2 * N - a - b) // 2
    return tot * B


def fwd_bytes(B, H, N, d, esz, lo):
    """Algorithmic HBM bytes of one forward: (minimal I/O, full I/O).
    Full: read Q, K, V; write O and LSE.  Minimal: read only the rows that
    take part in some band (head h: query rows i >= lo_h, key rows
    j <= N - 1 - lo_h, N - lo_h of each); every output row is written."""
    act = B * sum(max(0, N - int(l)) for l in lo)
    row, all_rows = d * esz, B * H * N
    return 3 * row * act + (row + 4) * all_rows, 4 * row * all_rows + 4 * all_rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-causal comparison")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the ablation-pattern, local-window and decode measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload forward measurements (workloads 1-4)")
    ap.add_argument("--no-probe", action="store_true", help="skip the measured MFMA / HBM denominators")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--profile-workload", type=int, default=0, metavar="IDX",
                    help="only run the forward of workload IDX (1-4) --warmup + --steps times, for profilers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the band kernels shard over "
              "(batch, head) with no communication, so multi-GPU throughput is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    # no collector pauses inside the timed regions: collect once now and leave
    # the rest of this short run to reference counting
    gc.collect()
    gc.disable()

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 2, "copy_calibration_bytes_written":
                          dst.numel() * 2}), flush=True)
        return

    from structured_sparse_attention_spattn_amd import ops
    from structured_sparse_attention_spattn_amd.inputs import make_inputs

    dev = torch.device("cuda:0")
    if args.profile_workload:
        profile_workload(args.profile_workload, args.steps, args.warmup, dev)
        return
    inp = make_inputs(B, H, N, D, dtype="bf16", seed=SEED, with_dout=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    lo, hi = ops.band_table(N, H)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(256, ops.bwd_workspace_bytes(B, H, N, D, torch.bfloat16, torch.bfloat16)),
                     dtype=torch.uint8, device=dev)
    evict = Evictor(dev)

    def step(bands=None):
        ops.fwd(q, k, v, bands=bands, out=o, lse=lse)
        ops.bwd(q, k, v, o, lse, do, bands=bands, workspace=ws, out=grads)

    def timed(bands, steps, warmup, flushed, how="read"):
        """`steps` full steps with HIP events around each kernel (recorded on
        the stream the kernels are launched on).  flushed: L2 and the MALL
        evicted before every step, outside the events (`how`: Evictor).
        Returns the wall time and the per-kernel event times (ms)."""
        for _ in range(warmup):
            step(bands)
        torch.cuda.synchronize()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1, e2, e3 in ev:
            if flushed:
                evict(how)
            e0.record()
            ops.fwd(q, k, v, bands=bands, out=o, lse=lse)
            e1.record()
            ops.bwd_dq(q, k, v, o, lse, do, ws, bands=bands, out=grads[0])
            e2.record()
            ops.bwd_dkdv(q, k, v, lse, do, ws, bands=bands, out=grads[1:])
            e3.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        times = {name: [e[i].elapsed_time(e[i + 1]) for e in ev]
                 for i, name in enumerate(("fwd", "bwd_dq", "bwd_dkdv"))}
        times["step"] = [e[0].elapsed_time(e[3]) for e in ev]
        return wall, times

    # ---- the first timed run as it falls, for comparison: fill flush, no settle
    _, ct = timed(None, args.steps, args.warmup, flushed=True, how="fill")
    # ---- settle: untimed evicted steps until SETTLE_MS of wall time has passed
    # (the engine and memory clocks ramp over the first tens of milliseconds
    # of a burst; a continuous run stays at the settled clocks)
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        for _ in range(10):
            evict()
            step()
        torch.cuda.synchronize()
        settle_steps += 10
    # ---- headline: evicted steps
    _, ft = timed(None, args.steps, args.warmup, flushed=True)
    per = {nm: float(np.mean(t)) for nm, t in ft.items()}
    per_median = {nm: float(np.median(t)) for nm, t in ft.items()}
    ms_per_step = per["step"]
    fwd_ms, bwd_ms = per["fwd"], per["bwd_dq"] + per["bwd_dkdv"]
    pairs = pairs_total(lo, hi)
    fl_fwd = 4 * D * pairs
    fl_all = 14 * D * pairs
    value = fl_all / (ms_per_step * 1e-3) / 1e12

    # Full-I/O algorithmic HBM bytes per launch of each kernel (T = one [B,H,N,d] bf16
    # tensor, R = one [B,H,N] fp32 row vector):
    #   fwd      read Q, K, V; write O, LSE                  4T + R
    #   bwd_dq   read Q, K, V, O, dO, LSE; write dQ, D        6T + 2R
    #   bwd_dkdv read Q, K, V, dO, LSE, D; write dK, dV       6T + 2R
    T = B * H * N * D * 2
    R = B * H * N * 4
    alg_full = {"fwd": 4 * T + R, "bwd_dq": 6 * T + 2 * R, "bwd_dkdv": 6 * T + 2 * R}
    # Minimal I/O: only rows that take part in some band are read (head h:
    # query rows i >= lo_h and key rows j <= N - 1 - lo_h, N - lo_h of each);
    # every output row is still written (rows outside all bands get 0).
    # With A active rows and A_all = B H N rows of d bf16 values (e = 2 bytes):
    #   fwd      read Q, K, V of A;  write O, LSE of A_all
    #   bwd_dq   read Q, dO, O, LSE, K, V of A;  write dQ of A_all, D of A
    #   bwd_dkdv read K, V, Q, dO, LSE, D of A;  write dK, dV of A_all
    act_rows = B * sum(max(0, N - int(l)) for l, u in zip(lo, hi) if int(u) >= int(l))
    row, all_rows = D * 2, B * H * N
    alg_min = {"fwd": 3 * row * act_rows + (row + 4) * all_rows,
               "bwd_dq": 5 * row * act_rows + 8 * act_rows + row * all_rows,
               "bwd_dkdv": 4 * row * act_rows + 8 * act_rows + 2 * row * all_rows}
    alg_bytes = alg_min
    kern_names = {"fwd": "fwd_bf16_kernel<128, false>", "bwd_dq": "bwd_dq_kernel<128, false>",
                  "bwd_dkdv": "bwd_dkdv_kernel<128, false>"}
    kernels = ("fwd", "bwd_dq", "bwd_dkdv")
    dom = max(kernels, key=per.get)
    gbs = alg_bytes[dom] / (per[dom] * 1e-3) / 1e9
    roofline = {
        "kernel": kern_names[dom],
        "bound": "hbm",
        "achieved": round(gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(kern_names[dom]),
        "avg_launch_ms": round(per[dom], 4),
        "algorithmic_bytes_per_launch": alg_bytes[dom],
        "io": "minimal (rows outside every band are not read); caches evicted before each step",
        "achieved_full_io": round(alg_full[dom] / (per[dom] * 1e-3) / 1e9, 1),
        "frac_full_io": round(alg_full[dom] / (per[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_full_io": alg_full[dom],
    }

    out = {
        "metric": "in-band TFLOP/s (fwd+bwd) on 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (iid N(0,1), seed 1005)",
        "config": {"workload": "band attention fwd+bwd, bf16, B=8 H=16 N=4096 d=128, BDP bands width 256",
                   "B": B, "H": H, "N": N, "d": D},
        "timing": (f"HIP events per step; {SETTLE_MS:.0f} ms of untimed steps, then {args.warmup} warm-up steps, "
                   "first; L2 and MALL evicted (512 MiB read) before each step, outside the events"),
        "settle": {"ms": SETTLE_MS, "steps": settle_steps},
        "pct_bf16_mfma_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "inband_pairs": pairs,
        "pairs_per_s": round(pairs / (ms_per_step * 1e-3), 1),
        "kernel_ms": {kname: round(per[kname], 4) for kname in kernels},
        "kernel_ms_median": {kname: round(per_median[kname], 4) for kname in kernels},
        "kernel_hbm_frac": {kname: round(alg_bytes[kname] / (per[kname] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                            for kname in kernels},
        "kernel_hbm_frac_full_io": {kname: round(alg_full[kname] / (per[kname] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                    for kname in kernels},
        "fwd_tflops": round(fl_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10 * D * pairs / (bwd_ms * 1e-3) / 1e12, 2),
        "roofline": roofline,
    }

    def summary(tt):
        pm = {nm: float(np.mean(t)) for nm, t in tt.items()}
        return {"ms_per_step": round(pm["step"], 4), "tflops_fwdbwd": round(fl_all / (pm["step"] * 1e-3) / 1e12, 2),
                "kernel_ms": {kname: round(pm[kname], 4) for kname in kernels}}

    # ---- the same steps after a 512 MiB fill (the caches left dirty), settled clocks
    _, fft = timed(None, args.steps, 2, flushed=True, how="fill")
    out["fill_flushed"] = summary(fft)
    out["cold_start"] = dict(summary(ct), timing=f"the first timed run: {args.warmup} warm-up steps, 512 MiB fill "
                                                 "before each step, clocks still ramping")
    # ---- the same steps back to back, caches warm
    wall, wt = timed(None, args.steps, 2, flushed=False)
    wper = {nm: float(np.mean(t)) for nm, t in wt.items()}
    out["warm"] = {
        "ms_per_step_wall": round(wall * 1e3 / args.steps, 4),
        "tflops_fwdbwd_wall": round(fl_all / (wall / args.steps) / 1e12, 2),
        "kernel_ms": {kname: round(wper[kname], 4) for kname in kernels},
        "ms_per_step_events": round(wper["step"], 4),
    }

    if not args.no_dense:
        dlo, dhi = ops.dense_bands(N, H)
        n_dense = max(5, args.steps // 2)
        _, dt = timed((dlo, dhi), n_dense, 2, flushed=True)
        dms = float(np.mean(dt["step"]))
        dfwd, dbwd = float(np.mean(dt["fwd"])), float(np.mean(dt["bwd_dq"])) + float(np.mean(dt["bwd_dkdv"]))
        out["dense_causal"] = {
            "ms_per_step": round(dms, 4), "fwd_ms": round(dfwd, 4), "bwd_ms": round(dbwd, 4),
            "speedup_fwdbwd": round(dms / ms_per_step, 3), "speedup_fwd": round(dfwd / fwd_ms, 3),
            "dense_tflops_fwdbwd": round(14 * D * pairs_total(dlo, dhi) / (dms * 1e-3) / 1e12, 2),
            "timing": "evicted, as the headline",
        }

    if not args.no_configs:
        out["configs"] = workload_forwards(dev, evict, with_cpu=not args.no_cpu)

    if not args.no_variants:
        out["variants"], out["decode"] = variants_and_decode(q, k, v, do, o, lse, ws, grads, lo, hi, args.steps, dev,
                                                             evict)

    if not args.no_probe:
        out["measured_peaks"] = measured_peaks(dev)
        mp = out["measured_peaks"]
        if mp.get("hbm_read_gbs"):
            roofline["peak_measured_read"] = mp["hbm_read_gbs"]
            roofline["frac_of_measured_read"] = round(gbs / mp["hbm_read_gbs"], 4)
        if mp.get("bf16_mfma_tflops"):
            out["pct_measured_bf16_mfma_peak"] = round(100 * value / mp["bf16_mfma_tflops"], 2)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, lo, hi, fl_all)

    print(json.dumps(out), flush=True)


def workload_forwards(dev, evict, with_cpu, reps=20):
    """Forward of workloads 1-4 on seeded inputs of their shapes: HIP events
    around each launch with L2 and the MALL evicted before it (median), the
    warm back-to-back mean, and the whole-workload float64 oracle forward
    timed on the host cores."""
    import numpy as np
    import torch
    from structured_sparse_attention_spattn_amd import ops
    from structured_sparse_attention_spattn_amd.inputs import make_inputs
    from structured_sparse_attention_spattn_amd.workloads import WORKLOADS, seed_for
    per_cfg = {}
    for idx in (1, 2, 3, 4):
        w = WORKLOADS[idx]
        cB, cH, cN, cd = w["B"], w["H"], w["N"], w["d"]
        cinp = make_inputs(cB, cH, cN, cd, dtype=w["dtype"], seed=seed_for(idx), scale=w["scale"])
        cq, ck, cv = (cinp[n].to(dev) for n in ("q", "k", "v"))
        co = torch.empty_like(cq)
        cl = torch.empty((cB, cH, cN), dtype=torch.float32, device=dev)
        for _ in range(3):
            ops.fwd(cq, ck, cv, out=co, lse=cl)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            evict()
            e0.record()
            ops.fwd(cq, ck, cv, out=co, lse=cl)
            e1.record()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(reps):
            ops.fwd(cq, ck, cv, out=co, lse=cl)
        w1.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        warm_ms = w0.elapsed_time(w1) / reps
        clo, chi = ops.band_table(cN, cH)
        cpairs = pairs_total(clo, chi, seq_len=cN, batch=cB)
        tf = 4 * cd * cpairs / (ms * 1e-3) / 1e12
        esz = 4 if w["dtype"] == "f32" else 2
        min_bytes, full_bytes = fwd_bytes(cB, cH, cN, cd, esz, clo)
        peak = FP32_PEAK_TFLOPS if w["dtype"] == "f32" else BF16_PEAK_TFLOPS
        rec = {
            "fwd_us": round(ms * 1e3, 2), "inband_pairs": cpairs,
            "pairs_per_s": round(cpairs / (ms * 1e-3), 1), "tflops": round(tf, 2),
            "pct_peak": round(100 * tf / peak, 2), "peak_tflops": peak,
            "hbm_frac_minimal_io": round(min_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_frac_full_io": round(full_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "median of evicted launches",
            "warm_fwd_us": round(warm_ms * 1e3, 2),
            "warm_tflops": round(4 * cd * cpairs / (warm_ms * 1e-3) / 1e12, 2),
        }
        if w["dtype"] == "f32":
            rec.update(f32_backward(cq, ck, cv, co, cl, seed_for(idx) + 7, dev))
        del cq, ck, cv, co, cl
        if with_cpu:
            rec["cpu_baseline"] = cpu_forward_baseline(cinp, clo, chi, 4 * cd * cpairs, cpairs, w["name"])
        per_cfg[w["name"]] = rec
        del cinp
    # the float32 backward where it is throughput-bound (no workload of its own)
    fB, fH, fN, fd = 2, 16, 4096, 128
    finp = make_inputs(fB, fH, fN, fd, dtype="f32", seed=4242)
    fq, fk, fv = (finp[n].to(dev) for n in ("q", "k", "v"))
    fo, fl = ops.fwd(fq, fk, fv)
    per_cfg[f"bwd_f32_B{fB}_H{fH}_N{fN}_d{fd}"] = f32_backward(fq, fk, fv, fo, fl, 4243, dev)
    return per_cfg


def variants_and_decode(q, k, v, do, o, lse, ws, grads, lo, hi, steps, dev, evict):
    """The page's ablation patterns and the shared local window at the bench
    shape (medians of device time per step), and a decode step (the median of
    launches with L2 and the MALL evicted before each, and the warm mean)."""
    import numpy as np
    import torch
    from structured_sparse_attention_spattn_amd import ops

    def timed_total(bands, lw, steps, warmup):
        for _ in range(warmup):
            ops.fwd(q, k, v, bands=bands, out=o, lse=lse, local_window=lw)
            ops.bwd(q, k, v, o, lse, do, bands=bands, workspace=ws, out=grads, local_window=lw)
        torch.cuda.synchronize()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1, e2 in ev:
            e0.record()
            ops.fwd(q, k, v, bands=bands, out=o, lse=lse, local_window=lw)
            e1.record()
            ops.bwd(q, k, v, o, lse, do, bands=bands, workspace=ws, out=grads, local_window=lw)
            e2.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        # medians: one stalled step must not stand for the variant
        f = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        b = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
        return wall, f, b

    variants = {}
    nvs = max(5, steps // 2)
    wlo, whi = ops.window_bands(N, H, N // H)
    glo, ghi = ops.gapped_half_bands(N, H)
    for name, bands, lw, (plo, phi) in (
            (f"sliding_window_{N // H}", (wlo, whi), 0, (wlo, whi)),
            ("gapped_half_bands", (glo, ghi), 0, (glo, ghi)),
            ("bands_plus_local_window_64", None, 64, (lo, hi))):
        wall_v, f_v, b_v = timed_total(bands, lw, nvs, 3)
        pv = pairs_total(plo, phi, lw)
        variants[name] = {
            "ms_per_step": round(f_v + b_v, 4), "fwd_ms": round(f_v, 4), "bwd_ms": round(b_v, 4),
            "wall_ms_per_step": round(wall_v, 4), "attended_pairs": pv,
            "tflops_fwdbwd": round(14 * D * pv / ((f_v + b_v) * 1e-3) / 1e12, 2),
        }

    # decode step (one new query per sequence) over a full key/value cache
    # of the same head layout; the caches come from a seeded device
    # generator (synthetic N(0, 1), quantised to bfloat16)
    dB = 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED)
    qd = torch.randn((dB, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kc = torch.randn((dB, H, N, D), generator=gen, device=dev).to(torch.bfloat16)
    vc = torch.randn((dB, H, N, D), generator=gen, device=dev).to(torch.bfloat16)
    od = torch.empty_like(qd)
    ld = torch.empty((dB, H), dtype=torch.float32, device=dev)
    for _ in range(5):
        ops.decode(qd, kc, vc, out=od, lse=ld)
    torch.cuda.synchronize()
    # the gathered rows (135 MB here) fit the MALL: back to back, later
    # launches find them there, so the headline decode time evicts first
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in dev_ev:
        evict()
        a.record()
        ops.decode(qd, kc, vc, out=od, lse=ld)
        b.record()
    n_dec = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_dec):
        ops.decode(qd, kc, vc, out=od, lse=ld)
    e1.record()
    torch.cuda.synchronize()
    dec_ms = float(np.median([a.elapsed_time(b) for a, b in dev_ev]))
    warm_dec_ms = e0.elapsed_time(e1) / n_dec
    keys = sum(min(N - 1, int(u)) - int(l_) + 1 for l_, u in zip(lo, hi) if int(u) >= int(l_))  # at i = N - 1
    dec_bytes = dB * (keys * 2 * D * 2 + H * (2 * D * 2 + 4))
    decode = {
        "workload": f"decode, bf16, B={dB} H={H} cache={N} d={D}, BDP bands, full caches",
        "us_per_step": round(dec_ms * 1e3, 2),
        "tokens_per_s": round(dB / (dec_ms * 1e-3), 1),
        "gather_bytes": dec_bytes,
        "gbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": "median of 20 launches, L2 and MALL evicted (512 MiB read) before each",
        "warm_us_per_step": round(warm_dec_ms * 1e3, 2),
    }
    return variants, decode


def measured_peaks(dev):
    """Measured denominators from libspattn_probe.so (spattn_probe.h): bf16
    and fp32 MFMA throughput (4 independent chains per wave, 16 waves per
    CU, registers only), LDS read bandwidth of the two read forms the kernels
    use, float32 atomic-add throughput into 256 MiB and 1 MiB, and the read
    bandwidth of a 4 GiB buffer; the best of 3 launches each.  None where the
    probe library is not built."""
    import torch
    path = os.path.join(ROOT, "structured_sparse_attention_spattn_amd", "libspattn_probe.so")
    if not os.path.exists(path):
        return {"note": "libspattn_probe.so not built"}
    lib = ctypes.CDLL(path)
    lib.spattn_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.spattn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    blocks = 256 * 4  # 4 workgroups of 4 waves per CU
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def best_ms(call, n=3):
        call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    res = {"method": "libspattn_probe.so: 4 independent MFMA chains per wave, 4 workgroups x 4 waves per CU; "
                     "conflict-free LDS reads, 4 workgroups x 4 waves per CU; "
                     "float32 atomic adds without return, 256 B per wave instruction, 4 workgroups per CU; "
                     "16-byte grid-stride reads of a 4 GiB buffer; best of 3 launches"}
    for kind, name, flop in ((0, "bf16_mfma_tflops", 32768), (1, "fp32_mfma_tflops", 4096)):
        iters = 2048 if kind == 0 else 1024
        ms = best_ms(lambda: lib.spattn_probe_mfma(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()), stream))
        res[name] = round(blocks * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12, 1)
    lib.spattn_probe_lds.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    for kind, name in ((0, "lds_read_b128"), (1, "lds_read_b64_tr_b16")):
        iters = 4096
        ms = best_ms(lambda: lib.spattn_probe_lds(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()), stream))
        tbs = blocks * 4 * iters * 8192 / (ms * 1e-3) / 1e12
        # bytes per clock per CU at the 2.4 GHz peak engine clock
        res[name + "_tbs"] = round(tbs, 1)
        res[name + "_bytes_per_clk_cu"] = round(tbs * 1e12 / (256 * 2.4e9), 1)
    # float32 atomic adds (no return) into a buffer the size of an fp32 dQ
    # accumulator at B=8 H=16 N=4096 d=128 (256 MiB) and into 1 MiB (L2)
    lib.spattn_probe_atomic.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]
    for nfl, name in ((1 << 26, "atomic_add_f32_256mib_gbs"), (1 << 18, "atomic_add_f32_1mib_gbs")):
        abuf = torch.zeros(nfl, dtype=torch.float32, device=dev)
        iters = 1024
        ms = best_ms(lambda: lib.spattn_probe_atomic(ctypes.c_void_p(abuf.data_ptr()), nfl, blocks, iters, stream))
        res[name] = round(blocks * 256 * iters * 4 / (ms * 1e-3) / 1e9, 1)
        del abuf
    buf = torch.ones(1 << 30, dtype=torch.float32, device=dev)  # 4 GiB
    nbytes = buf.numel() * 4
    ms = best_ms(lambda: lib.spattn_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, 256 * 8,
                                               ctypes.c_void_p(sink.data_ptr()), stream))
    res["hbm_read_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    res["spec"] = {"bf16_mfma_tflops": BF16_PEAK_TFLOPS, "fp32_mfma_tflops": FP32_PEAK_TFLOPS,
                   "hbm_gbs": HBM_PEAK_GBS}
    del buf
    return res


def profile_workload(idx, steps, warmup, dev):
    """The forward of one workload, on resident seeded inputs, for a profiler
    run: warmup + steps launches, then one JSON line with the HIP-event mean."""
    import numpy as np
    import torch
    from structured_sparse_attention_spattn_amd import ops
    from structured_sparse_attention_spattn_amd.inputs import make_inputs
    from structured_sparse_attention_spattn_amd.workloads import WORKLOADS, seed_for
    w = WORKLOADS[idx]
    cB, cH, cN, cd = w["B"], w["H"], w["N"], w["d"]
    cinp = make_inputs(cB, cH, cN, cd, dtype=w["dtype"], seed=seed_for(idx), scale=w["scale"])
    cq, ck, cv = (cinp[n].to(dev) for n in ("q", "k", "v"))
    co = torch.empty_like(cq)
    cl = torch.empty((cB, cH, cN), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        ops.fwd(cq, ck, cv, out=co, lse=cl)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        ops.fwd(cq, ck, cv, out=co, lse=cl)
        e1.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    print(json.dumps({"workload": w["name"], "launches": steps, "fwd_us_mean": round(1e3 * float(np.mean(ms)), 2),
                      "fwd_us_median": round(1e3 * float(np.median(ms)), 2)}), flush=True)


def f32_backward(q, k, v, o, lse, seed, dev, reps=20):
    """HIP-event times of the float32 backward stages on resident inputs
    (dO seeded N(0, 1)); TFLOP/s counts 10 d per in-band pair."""
    import torch
    from structured_sparse_attention_spattn_amd import ops
    B, H, N, d = q.shape
    g = torch.Generator().manual_seed(seed)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(dev)
    ws = torch.empty(ops.bwd_workspace_bytes(B, H, N, d, torch.float32, torch.float32), dtype=torch.uint8,
                     device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    for _ in range(3):
        ops.bwd_dq(q, k, v, o, lse, do, ws, out=dq)
        ops.bwd_dkdv(q, k, v, lse, do, ws, out=(dk, dv))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(reps):
        ops.bwd_dq(q, k, v, o, lse, do, ws, out=dq)
    ev[1].record()
    for _ in range(reps):
        ops.bwd_dkdv(q, k, v, lse, do, ws, out=(dk, dv))
    ev[2].record()
    torch.cuda.synchronize()
    dq_ms, kv_ms = ev[0].elapsed_time(ev[1]) / reps, ev[1].elapsed_time(ev[2]) / reps
    lo, hi = ops.band_table(N, H)
    pairs = pairs_total(lo, hi, seq_len=N, batch=B)
    tf = 10 * d * pairs / ((dq_ms + kv_ms) * 1e-3) / 1e12
    return {"bwd_us": round((dq_ms + kv_ms) * 1e3, 2), "bwd_dq_us": round(dq_ms * 1e3, 2),
            "bwd_dkdv_us": round(kv_ms * 1e3, 2), "bwd_tflops": round(tf, 2),
            "bwd_pct_peak": round(100 * tf / FP32_PEAK_TFLOPS, 2)}


def _host_info():
    import platform
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(threads), model


def cpu_forward_baseline(inp, lo, hi, flops, pairs, name):
    """The float64 oracle forward (as is) over one whole workload on this host."""
    import oracle
    from structured_sparse_attention_spattn_amd.inputs import as_f64
    q, k, v = (as_f64(inp[n]) for n in ("q", "k", "v"))
    threads, model = _host_info()
    t0 = time.perf_counter()
    oracle.band_attention_fwd(q, k, v, lo, hi)
    dt = time.perf_counter() - t0
    return {"kind": "oracle", "sample": f"whole workload {name}, float64 numpy forward", "seconds": round(dt, 3),
            "gflops": round(flops / dt / 1e9, 2), "pairs_per_s": round(pairs / dt, 1), "cores": threads,
            "cpu": model}


def cpu_baseline(inp, lo, hi, flops_all):
    """The float64 oracle (as is) on this host, fwd+bwd over the whole workload."""
    import oracle
    from structured_sparse_attention_spattn_amd.inputs import as_f64
    threads, model = _host_info()
    q, k, v, do = (as_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    t0 = time.perf_counter()
    oracle.band_attention_bwd(q, k, v, do, lo, hi)  # includes the forward recompute
    dt = time.perf_counter() - t0
    return {
        "value": round(flops_all / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "whole workload (B=8 H=16 N=4096 d=128), float64 numpy, fwd+bwd",
        "seconds": round(dt, 2),
        "cpu": model,
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
    }


if __name__ == "__main__":
    main()
