"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

Holds no attention arithmetic: it draws iid standard normals with numpy's
PCG64 generator in the fixed order Q, K, V (then dO), shape [B, H, N, d] in C
order, multiplies by a per-workload scale, casts to float32 and, for bf16
workloads, rounds to bfloat16 (round-to-nearest-even, torch's conversion).
The quantised tensors are the single source for both the device path and the
float64 CPU check.
"""
import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(B, H, N, d, dtype="bf16", seed=0, scale=1.0, with_dout=False):
    """Return a dict of CPU torch tensors q, k, v (and dout) of ``dtype``."""
    rng = np.random.default_rng(seed)
    names = ["q", "k", "v"] + (["dout"] if with_dout else [])
    out = {}
    for name in names:
        x = rng.standard_normal((B, H, N, d)) * scale
        t = torch.from_numpy(x.astype(np.float32))
        out[name] = t.to(_DTYPES[dtype]).contiguous()
    return out


def as_f64(t):
    """Exact float64 copy of a (possibly bf16) CPU tensor, as numpy."""
    return t.detach().to("cpu").to(torch.float64).numpy()
