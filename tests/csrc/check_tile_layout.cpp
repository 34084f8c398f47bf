// Host-side check of the swizzled LDS tile layout in attn_device.h (no GPU needed).
// For D = 64 and 128 it verifies that:
//   1. the 1-KiB direct loads and the element reads agree on where every 16-byte
//      chunk of the tile lives, and cover the tile exactly once;
//   2. a row read (16 lanes, same chunk of 16 consecutive rows) touches 16
//      distinct 16-byte bank groups of the 256-byte bank row;
//   3. a transposed 4x16 read (4 consecutive rows x 4 consecutive chunks)
//      touches 16 distinct bank groups;
//   4. moving by 16 rows moves every address by 16 rows' bytes;
//   5. every address stays inside the tile.
#include <cstdio>
#include <set>

#include "attn_device.h"

template <int D>
int check() {
  using T = tam::SwzTile<D>;
  int bad = 0;
  std::set<int> seen;
  for (int i = 0; i < T::LOADS; ++i)
    for (int l = 0; l < 64; ++l) {
      const int g = T::load_src(i, l);
      const int r = g / T::ROW_BYTES, c = (g % T::ROW_BYTES) / 16;
      if (T::chunk_off(r, c) != 1024 * i + 16 * l) ++bad;
      seen.insert(g);
    }
  if ((int)seen.size() != T::BYTES / 16) ++bad;
  for (int r0 = 0; r0 < T::ROWS; r0 += 16)
    for (int c = 0; c < D / 8; ++c) {
      std::set<int> q;
      for (int r = r0; r < r0 + 16; ++r) q.insert((T::chunk_off(r, c) % 256) / 16);
      if (q.size() != 16) ++bad;
    }
  for (int r0 = 0; r0 < T::ROWS; r0 += 4)
    for (int c0 = 0; c0 < D / 8; c0 += 4) {
      std::set<int> q;
      for (int r = r0; r < r0 + 4; ++r)
        for (int c = c0; c < c0 + 4; ++c) q.insert((T::chunk_off(r, c) % 256) / 16);
      if (q.size() != 16) ++bad;
    }
  for (int r = 0; r + 16 < T::ROWS; ++r)
    for (int c = 0; c < D / 8; ++c)
      if (T::chunk_off(r + 16, c) != T::chunk_off(r, c) + 16 * T::ROW_BYTES) ++bad;
  for (int r = 0; r < T::ROWS; ++r)
    for (int e = 0; e < D; e += 4) {
      const int o = T::elem_off(r, e);
      if (o < 0 || o + 8 > T::BYTES) ++bad;
    }
  return bad;
}

int main() {
  const int b128 = check<128>(), b64 = check<64>();
  std::printf("D=128 violations %d, D=64 violations %d\n", b128, b64);
  return (b128 || b64) ? 1 : 0;
}
