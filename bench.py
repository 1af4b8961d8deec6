"""Benchmark of band-partitioned (SPAttention) attention on one MI355X.

One step = the whole hot path over one batch: spattn_fwd (band table, band
tile schedule, scores, masks, online softmax, P V, epilogue) followed by
spattn_bwd's two stages (D = rowsum(dO * O) and band-tiled dQ; then band-tiled
dK / dV), on
B = 8, H = 16, N = 4096, d = 128, bfloat16 inputs resident in HBM.

Prints ONE JSON line.  ``value`` is in-band TFLOP/s of fwd+bwd (14 d FLOP per
attended pair; the heads together attend N(N+1)/2 pairs per sequence).
Extra keys report the forward alone, per-kernel medians, the same kernels
with L2 and MALL flushed before each launch ("cold"), the dense-causal kernel
of the same library at the same shape, the roofline of the dominant kernel, the float64
CPU oracle timed on this host and, under "variants", the same shape with the
band tables of the page's ablation patterns (sliding window, gapped half
bands) and with a shared local window joined to every band.
"""
import argparse
import gc
import json
import math
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-causal comparison")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the ablation-pattern and local-window measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload forward measurements (workloads 1-4)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the flushed-cache (cold) per-kernel timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
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
    inp = make_inputs(B, H, N, D, dtype="bf16", seed=SEED, with_dout=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    lo, hi = ops.band_table(N, H)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(256, ops.bwd_workspace_bytes(B, H, N, D, torch.bfloat16, torch.bfloat16)),
                     dtype=torch.uint8, device=dev)

    def step(bands=None):
        ops.fwd(q, k, v, bands=bands, out=o, lse=lse)
        ops.bwd(q, k, v, o, lse, do, bands=bands, workspace=ws, out=grads)

    def timed(bands, steps, warmup):
        """Wall time of `steps` full steps, plus per-kernel HIP-event means and
        medians (every event is recorded on the stream the kernels are launched
        on)."""
        for _ in range(warmup):
            step(bands)
        torch.cuda.synchronize()
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1, e2, e3 in ev:
            e0.record()
            ops.fwd(q, k, v, bands=bands, out=o, lse=lse)
            e1.record()
            ops.bwd_dq(q, k, v, o, lse, do, ws, bands=bands, out=grads[0])
            e2.record()
            ops.bwd_dkdv(q, k, v, lse, do, ws, bands=bands, out=grads[1:])
            e3.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev]))
               for i, name in enumerate(("fwd", "bwd_dq", "bwd_dkdv"))}
        med = {name: float(np.median([e[i].elapsed_time(e[i + 1]) for e in ev]))
               for i, name in enumerate(("fwd", "bwd_dq", "bwd_dkdv"))}
        return wall, per, med

    wall, per, per_median = timed(None, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
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
    dom = max(per, key=per.get)
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
        "io": "minimal (rows outside every band are not read)",
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
        "pct_bf16_mfma_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "inband_pairs": pairs,
        "pairs_per_s": round(pairs / (ms_per_step * 1e-3), 1),
        "kernel_ms": {kname: round(t, 4) for kname, t in per.items()},
        "kernel_hbm_frac": {kname: round(alg_bytes[kname] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                            for kname, t in per.items()},
        "kernel_hbm_frac_full_io": {kname: round(alg_full[kname] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                    for kname, t in per.items()},
        "fwd_tflops": round(fl_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10 * D * pairs / (bwd_ms * 1e-3) / 1e12, 2),
        "roofline": roofline,
    }

    out["kernel_ms_median"] = {kname: round(t, 4) for kname, t in per_median.items()}

    if not args.no_cold:
        # Cold caches: before every kernel a 512 MiB fill (outside the events)
        # evicts the inputs from L2 and the MALL; medians over the repeats.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        n_cold = max(5, args.steps // 2)
        calls = (("fwd", lambda: ops.fwd(q, k, v, out=o, lse=lse)),
                 ("bwd_dq", lambda: ops.bwd_dq(q, k, v, o, lse, do, ws, out=grads[0])),
                 ("bwd_dkdv", lambda: ops.bwd_dkdv(q, k, v, lse, do, ws, out=grads[1:])))
        evs = []
        for _ in range(n_cold):
            for name, call in calls:
                flush.zero_()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                evs.append((name, e0, e1))
        torch.cuda.synchronize()
        cold = {name: float(np.median([a.elapsed_time(b) for n_, a, b in evs if n_ == name]))
                for name, _ in calls}
        cold_step = sum(cold.values())
        out["cold"] = {
            "repeats": n_cold,
            "kernel_ms_median": {kname: round(t, 4) for kname, t in cold.items()},
            "ms_per_step": round(cold_step, 4),
            "tflops_fwdbwd": round(fl_all / (cold_step * 1e-3) / 1e12, 2),
            "kernel_hbm_frac": {kname: round(alg_bytes[kname] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                for kname, t in cold.items()},
        }
        del flush

    if not args.no_dense:
        dlo, dhi = ops.dense_bands(N, H)
        n_dense = max(5, args.steps // 2)
        dwall, dper, _ = timed((dlo, dhi), n_dense, 2)
        dms = dwall * 1e3 / n_dense
        dfwd, dbwd = dper["fwd"], dper["bwd_dq"] + dper["bwd_dkdv"]
        out["dense_causal"] = {
            "ms_per_step": round(dms, 4), "fwd_ms": round(dfwd, 4), "bwd_ms": round(dbwd, 4),
            "speedup_fwdbwd": round(dms / ms_per_step, 3), "speedup_fwd": round(dfwd / fwd_ms, 3),
            "dense_tflops_fwdbwd": round(14 * D * pairs_total(dlo, dhi) / (dms * 1e-3) / 1e12, 2),
        }

    if not args.no_configs:
        # forward throughput of the other workloads (the fp32 N = 1024 one and
        # the bf16 N = 4096 / 8192 / 10000 ones), seeded inputs of their shapes
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
            reps = 20
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                ops.fwd(cq, ck, cv, out=co, lse=cl)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            clo, chi = ops.band_table(cN, cH)
            cpairs = pairs_total(clo, chi, seq_len=cN, batch=cB)
            tf = 4 * cd * cpairs / (ms * 1e-3) / 1e12
            esz = 4 if w["dtype"] == "f32" else 2
            act = cB * sum(max(0, cN - int(l)) for l in clo)
            rowb, allr = cd * esz, cB * cH * cN
            min_bytes = 3 * rowb * act + (rowb + 4) * allr
            peak = FP32_PEAK_TFLOPS if w["dtype"] == "f32" else BF16_PEAK_TFLOPS
            per_cfg[w["name"]] = {
                "fwd_us": round(ms * 1e3, 2), "inband_pairs": cpairs,
                "pairs_per_s": round(cpairs / (ms * 1e-3), 1), "tflops": round(tf, 2),
                "pct_peak": round(100 * tf / peak, 2), "peak_tflops": peak,
                "hbm_frac_minimal_io": round(min_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            if w["dtype"] == "f32":
                per_cfg[w["name"]].update(f32_backward(cq, ck, cv, co, cl, seed_for(idx) + 7, dev))
            del cq, ck, cv, co, cl, cinp
        # the float32 backward where it is throughput-bound (no workload of its own)
        fB, fH, fN, fd = 2, 16, 4096, 128
        finp = make_inputs(fB, fH, fN, fd, dtype="f32", seed=4242)
        fq, fk, fv = (finp[n].to(dev) for n in ("q", "k", "v"))
        fo, fl = ops.fwd(fq, fk, fv)
        per_cfg[f"bwd_f32_B{fB}_H{fH}_N{fN}_d{fd}"] = f32_backward(fq, fk, fv, fo, fl, 4243, dev)
        del fq, fk, fv, fo, fl, finp
        out["configs"] = per_cfg

    if not args.no_variants:
        def timed_total(bands, lw, steps, warmup):
            """fwd and bwd (both stages) of the whole batch with these bands /
            local window; HIP events on the launch stream, median per step
            (and the mean wall time per step)."""
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
        nvs = max(5, args.steps // 2)
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
        out["variants"] = variants

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
        n_dec = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_dec):
            ops.decode(qd, kc, vc, out=od, lse=ld)
        e1.record()
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / n_dec
        keys = sum(min(N - 1, int(u)) - int(l_) + 1 for l_, u in zip(lo, hi) if int(u) >= int(l_))  # at i = N - 1
        dec_bytes = dB * (keys * 2 * D * 2 + H * (2 * D * 2 + 4))
        out["decode"] = {
            "workload": f"decode, bf16, B={dB} H={H} cache={N} d={D}, BDP bands, full caches",
            "us_per_step": round(dec_ms * 1e3, 2),
            "tokens_per_s": round(dB / (dec_ms * 1e-3), 1),
            "gather_bytes": dec_bytes,
            "gbs": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        del kc, vc

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, lo, hi, fl_all)

    print(json.dumps(out), flush=True)


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


def cpu_baseline(inp, lo, hi, flops_all):
    """The float64 oracle (as is) on this host, fwd+bwd over the whole workload."""
    import platform

    import oracle
    from structured_sparse_attention_spattn_amd.inputs import as_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    q, k, v, do = (as_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    t0 = time.perf_counter()
    oracle.band_attention_bwd(q, k, v, do, lo, hi)  # includes the forward recompute
    dt = time.perf_counter() - t0
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(flops_all / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "whole workload (B=8 H=16 N=4096 d=128), float64 numpy, fwd+bwd",
        "seconds": round(dt, 2),
        "cpu": model,
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
    }


if __name__ == "__main__":
    main()
