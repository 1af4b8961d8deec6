// Host-side check of how the band kernels map workgroups to work items
// (work_item): for many launch shapes and tile sizes, in both tile orders,
// every (sequence, head, tile) is run by exactly one workgroup and all tiles
// of a (sequence, head) pair run on one XCD.  Prints "violations <n>".
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "common.h"

using namespace spattn;

static long check(int B, int H, int N, const WalkShape& ws, bool desc) {
  long bad = 0;
  const int n_tiles = (N + ws.own - 1) / ws.own;
  const long long grid = work_grid(B, H, n_tiles);
  if (grid % 8 != 0) ++bad;
  std::vector<int> hits((size_t)B * H * n_tiles, 0);
  std::vector<int> xcd_of((size_t)B * H, -1);
  for (long long pid = 0; pid < grid; ++pid) {
    const WorkItem wi = work_item((int)pid, B, H, n_tiles, desc);
    if (!wi.valid) continue;
    if (wi.b < 0 || wi.b >= B || wi.h < 0 || wi.h >= H || wi.t < 0 || wi.t >= n_tiles) {
      ++bad;
      continue;
    }
    ++hits[((size_t)wi.h * B + wi.b) * n_tiles + wi.t];
    // all tiles of a pair on one XCD (workgroup i runs on XCD i % 8)
    int& x = xcd_of[(size_t)wi.h * B + wi.b];
    if (x < 0) x = (int)(pid % 8);
    if (x != (int)(pid % 8)) ++bad;
  }
  for (int c : hits) bad += c != 1;
  return bad;
}

int main() {
  long bad = 0;
  const WalkShape shapes[] = {{128, 64, false, true}, {128, 32, false, true}, {64, 32, true, false},
                              {64, 32, false, false}, {32, 32, false, false}, {32, 32, true, false}};
  for (int B = 1; B <= 9; ++B)
    for (int H = 1; H <= 40; H += 3)
      for (int N : {1, 31, 64, 100, 1000, 4096})
        for (const WalkShape& ws : shapes)
          for (int desc = 0; desc < 2; ++desc) bad += check(B, H, N, ws, desc != 0);
  bad += check(8, 256, 300, shapes[0], true);
  printf("violations %ld\n", bad);
  return bad == 0 ? 0 : 1;
}
