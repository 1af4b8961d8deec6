// Host-side check of the packed-sequence view every kernel indexes with
// (seq_head in the kernels' common header): whatever the offsets array holds
// -- decreasing, negative, past the packed length, longer than the grid's
// maximum -- the view stays inside the [H, T, d] tensors, and a well-formed
// array gives each sequence exactly its tokens.  Prints "violations <n>".
#include <stdio.h>
#include <stdlib.h>

#include "common.h"

using namespace spattn;

static long check(const int32_t* cu, int S, int T, int N, int H, const Bands& b, bool well_formed) {
  long bad = 0;
  for (int s = 0; s < S; ++s)
    for (int h = 0; h < H; ++h)
      for (int own = 0; own < 2; ++own) {
        const SeqHead v = seq_head(cu, T, own, H, N, b, s, h);
        const long o = (long)v.row0 - (long)h * T;
        if (v.n < 0 || v.n > N || o < 0 || o > T || o + v.n > T) ++bad;
        if (v.n > 0 && (v.lo < 0 || v.hi > v.n - 1 || v.lo > v.hi + 1)) ++bad;
        if (well_formed && (o != cu[s] || v.n != cu[s + 1] - cu[s])) ++bad;
      }
  return bad;
}

int main() {
  const int H = 5;
  Bands b;
  for (int h = 0; h < H; ++h) {
    b.lo[h] = 3 * h;
    b.hi[h] = 3 * h + 40;
  }
  long bad = 0;
  srand(12345);
  for (int trial = 0; trial < 20000; ++trial) {
    const int S = 1 + rand() % 6;
    int32_t cu[8];
    const int T = 1 + rand() % 200;
    const int N = 1 + rand() % 120;
    const bool ok = trial % 2 == 0;
    if (ok) {  // well formed: rising from 0 to T with every length <= N
      cu[0] = 0;
      int left = T;
      for (int s = 1; s <= S; ++s) {
        int len = s == S ? left : rand() % (left + 1);
        if (len > N) len = N;
        cu[s] = cu[s - 1] + len;
        left -= len;
      }
      if (cu[S] != T) continue;
    } else {  // anything at all
      for (int s = 0; s <= S; ++s) cu[s] = rand() % 700 - 250;
    }
    bad += check(cu, S, T, N, H, b, ok);
  }
  printf("violations %ld\n", bad);
  return bad == 0 ? 0 : 1;
}
