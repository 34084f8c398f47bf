// Host-side check of the work-unit scheduler in attn_device.h (no GPU needed).
// For a range of stream and tile counts it verifies that:
//   1. the grid covers every (stream, tile) unit exactly once;
//   2. every XCD (workgroup index mod 8) gets work whenever there are at least
//      8 units, and the unit counts of the XCDs differ by at most one tile row;
//   3. along each XCD's dispatch order the tiles never increase, so under a
//      causal mask the heaviest units of the query-tile kernels start first;
//   4. with a multiple of 8 streams, each XCD keeps to a contiguous range of
//      streams (the heads of one key/value group share an L2).
#include <cstdio>
#include <vector>

#include "attn_device.h"

int check(int BH, int NT) {
  tam::TileSched s{BH, NT, (BH + 7) / 8};
  const long long grid = tam::sched_grid(s);
  std::vector<int> seen((size_t)BH * NT, 0);
  std::vector<long long> per_xcd(8, 0);
  std::vector<int> last_tile(8, 1 << 30), lo(8, 1 << 30), hi(8, -1);
  int bad = 0;
  for (long long b = 0; b < grid; ++b) {
    int bh = -1, qt = -1;
    if (!tam::sched_decode(s, (int)b, &bh, &qt)) continue;
    if (bh < 0 || bh >= BH || qt < 0 || qt >= NT) { ++bad; continue; }
    seen[(size_t)bh * NT + qt]++;
    const int x = (int)(b % 8);
    per_xcd[x]++;
    if (qt > last_tile[x]) ++bad;  // heaviest first along each XCD
    last_tile[x] = qt;
    lo[x] = bh < lo[x] ? bh : lo[x];
    hi[x] = bh > hi[x] ? bh : hi[x];
  }
  for (int v : seen)
    if (v != 1) ++bad;
  long long mn = per_xcd[0], mx = per_xcd[0];
  for (long long c : per_xcd) { mn = c < mn ? c : mn; mx = c > mx ? c : mx; }
  if ((long long)BH * NT >= 8 && mn == 0) ++bad;
  if (mx - mn > (BH % 8 == 0 ? 0 : 1 + NT / 8 + 1)) ++bad;
  if (BH % 8 == 0)
    for (int x = 0; x < 8; ++x)
      if (hi[x] - lo[x] + 1 != BH / 8) ++bad;
  if (bad) printf("BH=%d NT=%d: %d problems (units per XCD %lld..%lld)\n", BH, NT, bad, mn, mx);
  return bad;
}

int main() {
  int bad = 0;
  const int bhs[] = {1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 32, 64, 100, 1024};
  const int nts[] = {1, 2, 5, 8, 32, 640};
  for (int bh : bhs)
    for (int nt : nts) bad += check(bh, nt);
  printf("%s\n", bad ? "FAILED" : "scheduler OK");
  return bad ? 1 : 0;
}
