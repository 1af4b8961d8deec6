"""The allocation-free backward (spattn_bwd_noalloc, for callers that cannot
allocate device memory) against spattn_bwd with a caller workspace: the same
kernels, so the gradients must agree bit for bit.  Two calls in a row on the
GPU's shared scratch array, the second with a smaller input, so a value left
by the first call would show; plus the size limit, checked before any device
work."""
import ctypes
import sys

import pytest
import torch

from structured_sparse_attention_spattn_amd import _lib, ops
from structured_sparse_attention_spattn_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,gdt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                       (torch.float32, torch.float32)])
def test_noalloc_equals_workspace_entry_point(dtype, gdt):
    cases = [(8, 16, 4096, 128, 1005), (1, 4, 515, 64, 1006)]  # the second call is smaller
    if dtype == torch.float32:
        cases = [(2, 16, 4096, 128, 1007), (1, 3, 333, 64, 1008)]
    for B, H, N, d, seed in cases:
        _say(f"noalloc B={B} H={H} N={N} d={d} {dtype}->{gdt}")
        inp = make_inputs(B, H, N, d, dtype="bf16" if dtype == torch.bfloat16 else "f32", seed=seed,
                          with_dout=True)
        x = {n: t.to(DEV) for n, t in inp.items()}
        o, lse = ops.fwd(x["q"], x["k"], x["v"])
        ref = ops.bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], grad_dtype=gdt)
        got = ops.bwd_noalloc(x["q"], x["k"], x["v"], o, lse, x["dout"], grad_dtype=gdt)
        torch.cuda.synchronize()
        for a, b, nm in zip(ref, got, ("dQ", "dK", "dV")):
            assert torch.equal(_bits(a), _bits(b)), f"{nm} differs (B={B} H={H} N={N} d={d})"


def test_noalloc_rejects_sizes_beyond_its_array():
    lib = _lib.load()
    p = ctypes.c_void_p(1 << 20)
    # 8 * 16 * 16385 rows need two vectors of 8 MiB + 256 bytes each: one row over the limit
    st = lib.spattn_bwd_noalloc(p, p, p, p, p, p, p, p, p, 8, 16, 16385, 128, _lib.BF16, _lib.BF16, None, None,
                                0.0, None)
    assert st == _lib.E_WORKSPACE
    need = lib.spattn_bwd_workspace_bytes(8, 16, 16384, 128, _lib.BF16, _lib.BF16)
    assert need == _lib.NOALLOC_SCRATCH_BYTES  # the largest size that fits exactly
