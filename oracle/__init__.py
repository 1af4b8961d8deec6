"""CPU float64 oracle for band-partitioned (SPAttention) causal attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code,
tables or helpers with the HIP library; it takes plain numpy arrays.

Sources (cited by page title and section; no code on any page):

* "Making Every Head Count: Sparse Attention Without the Speed-Performance
  Trade-off" -- abstract (the heads split the attention workload into
  balanced, non-overlapping distance bands, one unique segment each) and the
  Figure 1 caption (Balanced Distance Partitioning: H contiguous,
  non-overlapping bands of width floor(N/H) or ceil(N/H) covering the whole
  causal distance spectrum, head 0 nearest, head H-1 farthest).
* "Story of Attention -- Part 4: Sparse Attention, Then and Now", section 1
  (Sparse Transformer): the masked-set sparse-attention formula, in which the
  softmax runs only over the permitted key set S_i, and its 4x4 worked example.

Readings where the pages are silent (each listed in the design notes):

* wider bands go to the first N mod H heads;
* the diagonal distance 0 belongs to head 0, the distance spectrum is [0, N-1];
* softmax over an empty key set gives output 0 and log-sum-exp -inf, and
  contributes nothing to any gradient;
* scores are divided by sqrt(d_k) (the worked example's printed weights fix
  divide, not multiply);
* LSE is the natural logarithm of the sum of exponentials of scaled scores;
* the backward pass is the textbook derivative of the forward formula (no page
  gives one).

Modules: ``band`` (band table), ``attention`` (forward/backward, three
independent forms; optional shared local window), ``tiles`` (canonical
band-tile lists), ``decode`` (single-query attention over a key/value cache),
``varlen`` (packed batches of sequences of different lengths).
"""
from .band import band_table, band_pairs, band_table_sliding_window, band_table_gapped_half
from .attention import (
    masked_attention_literal,
    masked_attention_dense,
    masked_attention_dense_bwd,
    band_mask,
    band_attention_fwd,
    band_attention_bwd,
    band_attention_fwd_rows,
    band_attention_bwd_rows,
)
from .tiles import query_tile_list, key_tile_list, distance_ranges
from .decode import decode_key_set, decode_attention
from .varlen import seq_bands, varlen_fwd, varlen_bwd

__all__ = [
    "band_table", "band_pairs", "band_table_sliding_window", "band_table_gapped_half",
    "masked_attention_literal", "masked_attention_dense", "masked_attention_dense_bwd",
    "band_mask", "band_attention_fwd", "band_attention_bwd", "band_attention_fwd_rows", "band_attention_bwd_rows",
    "query_tile_list", "key_tile_list", "distance_ranges", "decode_key_set", "decode_attention",
    "seq_bands", "varlen_fwd", "varlen_bwd",
]
