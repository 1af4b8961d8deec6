"""Band-partitioned (SPAttention) causal attention for AMD MI355X (gfx950).

Every head h attends only the keys whose causal distance i - j lies in its
band [lo_h, hi_h]; Balanced Distance Partitioning gives the heads contiguous,
non-overlapping bands that together cover every causal pair once ("Making
Every Head Count: Sparse Attention Without the Speed-Performance Trade-off",
abstract and Figure 1 caption).  The computation lives in the HIP library
libspattn.so (C ABI in include/spattn.h); ``ops`` wraps it for torch tensors.
"""
from .ops import (band_table, dense_bands, fwd, bwd, bwd_dq, bwd_dkdv, bwd_workspace_bytes, kernel_tiles,  # noqa: F401
                  tile_list)
