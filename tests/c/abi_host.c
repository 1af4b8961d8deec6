/* Plain C user of the library's C ABI (include/spattn.h), host-side calls
 * only: the Balanced Distance Partitioning table, the pattern tables,
 * workspace sizing, status strings and the argument checks of every entry
 * point that fail before anything is launched (so no GPU is needed).
 * Prints one line per check; the calling tests compare them (also under
 * AddressSanitizer and UndefinedBehaviorSanitizer). */
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>

#include "spattn.h"

int main(void) {
  int32_t lo[8], hi[8];
  int st = spattn_band_table(1024, 8, lo, hi);
  printf("band_table %d", st);
  for (int h = 0; h < 8; ++h) printf(" [%d,%d]", lo[h], hi[h]);
  printf("\n");
  int32_t lo3[3], hi3[3];
  st = spattn_band_table(10, 3, lo3, hi3);  /* widths 4, 3, 3: wider bands first */
  printf("band_table_uneven %d [%d,%d] [%d,%d] [%d,%d]\n", st, lo3[0], hi3[0], lo3[1], hi3[1], lo3[2], hi3[2]);
  printf("band_table_bad %d\n", spattn_band_table(0, 8, lo, hi));
  int32_t plo[3], phi[3];
  st = spattn_band_table_pattern(10, 3, SPATTN_PATTERN_GAPPED_HALF, 0, plo, phi);  /* halves of 4, 3, 3 */
  printf("gapped_half %d [%d,%d] [%d,%d] [%d,%d]\n", st, plo[0], phi[0], plo[1], phi[1], plo[2], phi[2]);
  st = spattn_band_table_pattern(10, 3, SPATTN_PATTERN_SLIDING_WINDOW, 4, plo, phi);
  printf("sliding_window %d [%d,%d] [%d,%d] [%d,%d]\n", st, plo[0], phi[0], plo[1], phi[1], plo[2], phi[2]);
  printf("pattern_bad %d\n", spattn_band_table_pattern(10, 3, 17, 0, plo, phi));

  /* every (N, H) up to the head limit: the partition covers [0, N - 1] exactly */
  int32_t* blo = (int32_t*)malloc(sizeof(int32_t) * SPATTN_MAX_HEADS);
  int32_t* bhi = (int32_t*)malloc(sizeof(int32_t) * SPATTN_MAX_HEADS);
  long bad = 0;
  for (int N = 1; N <= 600; N += 7)
    for (int H = 1; H <= SPATTN_MAX_HEADS; H += 5) {
      if (spattn_band_table(N, H, blo, bhi) != SPATTN_OK) ++bad;
      int next = 0;
      for (int h = 0; h < H && next < N; ++h) {
        if (blo[h] != next || bhi[h] < blo[h]) ++bad;
        next = bhi[h] + 1;
      }
      if (next != N) ++bad;
      for (int kind = 0; kind < 4; ++kind)
        if (spattn_band_table_pattern(N, H, kind, N / 3, blo, bhi) != SPATTN_OK) ++bad;
    }
  printf("band_tables_swept %ld\n", bad);
  free(blo);
  free(bhi);

  printf("workspace %zu\n", spattn_bwd_workspace_bytes(2, 3, 100, 128, SPATTN_BF16, SPATTN_BF16));
  printf("workspace_bad %zu\n", spattn_bwd_workspace_bytes(2, 3, 100, 96, SPATTN_BF16, SPATTN_BF16));
  int32_t bq = 0, bk = 0;
  st = spattn_kernel_tiles(128, SPATTN_BF16, &bq, &bk);
  printf("tiles %d %d %d\n", st, bq, bk);

  /* argument checks that fail before any launch (stand-in addresses, never dereferenced) */
  void* a = (void*)(uintptr_t)(1u << 20);
  void* mis = (void*)((uintptr_t)(1u << 20) + 8);
  float* fa = (float*)a;
  st = spattn_fwd(mis, a, a, a, fa, 1, 2, 64, 64, SPATTN_BF16, NULL, NULL, 0.0f, NULL);
  printf("fwd_misaligned %d %s\n", st, spattn_status_string(st));
  st = spattn_fwd(a, a, a, a, fa, 1, 2, 64, 96, SPATTN_BF16, NULL, NULL, 0.0f, NULL);
  printf("fwd_d96 %d %s\n", st, spattn_status_string(st));
  int32_t bl[2] = {0, 70}, bh[2] = {63, 80};
  printf("fwd_band_past_n %d\n", spattn_fwd(a, a, a, a, fa, 1, 2, 64, 64, SPATTN_BF16, bl, bh, 0.0f, NULL));
  printf("fwd_local_neg %d\n", spattn_fwd_local(a, a, a, a, fa, 1, 2, 64, 64, SPATTN_BF16, NULL, NULL, -1, 0.0f, NULL));
  size_t ws = spattn_bwd_workspace_bytes(1, 2, 64, 64, SPATTN_BF16, SPATTN_BF16);
  printf("bwd_small_ws %d\n", spattn_bwd(a, a, a, a, fa, a, a, a, a, 1, 2, 64, 64, SPATTN_BF16, SPATTN_BF16, NULL,
                                         NULL, 0.0f, a, ws - 1, NULL));
  printf("bwd_grad_dtype %d\n", spattn_bwd(a, a, a, a, fa, a, a, a, a, 1, 2, 64, 64, SPATTN_BF16, 7, NULL, NULL,
                                           0.0f, a, ws, NULL));
  printf("bwd_dq_null %d\n", spattn_bwd_dq(a, a, a, NULL, fa, a, a, 1, 2, 64, 64, SPATTN_BF16, SPATTN_BF16, NULL, NULL,
                                           0.0f, a, ws, NULL));
  printf("bwd_dkdv_heads %d\n", spattn_bwd_dkdv(a, a, a, fa, a, a, a, 1, SPATTN_MAX_HEADS + 1, 64, 64, SPATTN_BF16,
                                                SPATTN_BF16, NULL, NULL, 0.0f, a, ws, NULL));
  printf("bwd_local_neg %d\n", spattn_bwd_local(a, a, a, a, fa, a, a, a, a, 1, 2, 64, 64, SPATTN_BF16, SPATTN_BF16,
                                                NULL, NULL, -3, 0.0f, a, ws, NULL));
  const int32_t* cu = (const int32_t*)a;
  printf("varlen_seqs %d\n", spattn_fwd_varlen(a, a, a, a, fa, cu, 0, 8, 12, 2, 64, SPATTN_BF16, NULL, NULL, 0, 0.0f,
                                               NULL));
  printf("varlen_ws %d\n", spattn_bwd_varlen(a, a, a, a, fa, a, a, a, a, cu, 2, 8, 12, 2, 64, SPATTN_BF16,
                                             SPATTN_BF16, NULL, NULL, 0, 0.0f, a, 16, NULL));
  printf("decode_dtype %d\n", spattn_decode(a, a, a, a, fa, NULL, 2, 4, 64, 128, 9, NULL, NULL, 0, 0.0f, NULL));
  int32_t n_out = 0;
  printf("walk_kernel %d\n", spattn_tile_walk(5, 128, SPATTN_BF16, 1, 1, 10, 0, 5, 0, &n_out, NULL, NULL, 0, &n_out,
                                              NULL, NULL, NULL));
  printf("tile_list_band %d\n", spattn_tile_list(10, 0, 10, 64, 64, &n_out, NULL, NULL, 0, &n_out, NULL));
  printf("status %s|%s\n", spattn_status_string(SPATTN_E_WORKSPACE), spattn_status_string(-5));
  return 0;
}
