/* Plain C user of the library's C ABI (include/spattn.h), host-side calls
 * only: the Balanced Distance Partitioning table, workspace sizing, status
 * strings and argument checks that fail before anything is launched.
 * Prints one line per check; the calling test compares them. */
#include <stdio.h>
#include <stdint.h>

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
  printf("workspace %zu\n", spattn_bwd_workspace_bytes(2, 3, 100, 128, SPATTN_BF16, SPATTN_BF16));
  printf("workspace_bad %zu\n", spattn_bwd_workspace_bytes(2, 3, 100, 96, SPATTN_BF16, SPATTN_BF16));
  int32_t bq = 0, bk = 0;
  st = spattn_kernel_tiles(128, SPATTN_BF16, &bq, &bk);
  printf("tiles %d %d %d\n", st, bq, bk);
  /* a misaligned tensor pointer is rejected before any launch */
  void* a = (void*)(uintptr_t)(1u << 20);
  void* mis = (void*)((uintptr_t)(1u << 20) + 8);
  st = spattn_fwd(mis, a, a, a, (float*)a, 1, 2, 64, 64, SPATTN_BF16, NULL, NULL, 0.0f, NULL);
  printf("fwd_misaligned %d %s\n", st, spattn_status_string(st));
  st = spattn_fwd(a, a, a, a, (float*)a, 1, 2, 64, 96, SPATTN_BF16, NULL, NULL, 0.0f, NULL);
  printf("fwd_d96 %d %s\n", st, spattn_status_string(st));
  return 0;
}
