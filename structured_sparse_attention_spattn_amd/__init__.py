"""Band-partitioned (SPAttention) causal attention for AMD MI355X (gfx950).

Every head h attends only the keys whose causal distance i - j lies in its
band [lo_h, hi_h]; Balanced Distance Partitioning gives the heads contiguous,
non-overlapping bands that together cover every causal pair once ("Making
Every Head Count: Sparse Attention Without the Speed-Performance Trade-off",
abstract and Figure 1 caption).  The computation lives in the HIP library
libspattn.so (C ABI in include/spattn.h); ``ops`` wraps it for torch tensors.

    import structured_sparse_attention_spattn_amd as spa
    o = spa.band_attention(q, k, v)          # [B, H, N, d] bf16 on the GPU, BDP bands
    o.float().sum().backward()               # dq, dk, dv through the band backward
    o, lse = spa.fwd(q, k, v)                # the entry points themselves
    dq, dk, dv = spa.bwd(q, k, v, o, lse, dout)
"""
from .ops import (band_attention, band_table, bwd, bwd_dkdv, bwd_dq, bwd_varlen, bwd_workspace_bytes,  # noqa: F401
                  decode, dense_bands, fwd, fwd_varlen, gapped_half_bands, kernel_tiles, tile_list, window_bands)
