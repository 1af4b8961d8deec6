"""The five synthetic workloads the library is tested and measured on.

Shapes follow the SPAttention pages' illustration (Figure 1 of "Making Every
Head Count": N = 1024, H = 8) and single-layer attention shapes at N >= 4096.
Inputs are iid N(0, 1) (scaled by 1/sqrt(2) for the N = 4096 forward
workload) from ``inputs.make_inputs`` with seed 1000 + index.
"""
import math

WORKLOADS = {
    1: dict(name="fwd_f32_B1_H8_N1024_d64", B=1, H=8, N=1024, d=64, dtype="f32", scale=1.0, bwd=False),
    2: dict(name="fwd_bf16_B8_H16_N4096_d128", B=8, H=16, N=4096, d=128, dtype="bf16", scale=1.0 / math.sqrt(2.0), bwd=False),
    3: dict(name="fwd_bf16_B4_H32_N8192_d128", B=4, H=32, N=8192, d=128, dtype="bf16", scale=1.0, bwd=False),
    4: dict(name="fwd_bf16_B2_H12_N10000_d64", B=2, H=12, N=10000, d=64, dtype="bf16", scale=1.0, bwd=False),
    5: dict(name="fwdbwd_bf16_B8_H16_N4096_d128", B=8, H=16, N=4096, d=128, dtype="bf16", scale=1.0, bwd=True),
}


def seed_for(index):
    return 1000 + index
