// Host-side check of the work-group -> tile map's division by invariant
// divisors (FastDiv, TileMap in common.hpp), compiled for the host only.
// FastDiv: n / d by multiply and shift must equal the quotient for every
// dividend 0 <= n < 2^31 tried -- all n below 4096, n around multiples of d,
// n near 2^31, pseudo-random n -- and every divisor tried -- all d up to
// 4096, powers of two and their neighbours, pseudo-random d up to 2^31 - 1.
// TileMap: for each tried (tiles_m, tiles_n, group_m, batch), every launch
// position must map to the tile the same raster gives with plain divisions,
// and the positions must cover every (product, tile) exactly once.
// Prints the number of failures and exits non-zero on any.
#include "common.hpp"

#include <cstdio>
#include <cstdint>
#include <vector>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static long failures = 0;

static void check_div(int d, int n) {
  const sgemm::FastDiv f = sgemm::make_fast_div(d);
  if (f(n) != n / d) {
    if (failures < 10) std::printf("FastDiv(%d)(%d) = %d, expected %d\n", d, n, f(n), n / d);
    ++failures;
  }
}

static void check_divisor(int d) {
  for (int n = 0; n < 4096; ++n) check_div(d, n);
  const long top = 2147483647L;
  for (long n = top; n > top - 64; --n) check_div(d, (int)n);
  for (int q : {1, 2, 3, 1000, 65535, 65536, 1 << 20}) {
    const long base = (long)q * d;
    for (long n = base - 2; n <= base + 2; ++n)
      if (n >= 0 && n <= top) check_div(d, (int)n);
  }
  for (long k = top / d; k > top / d - 3 && k >= 0; --k) {
    const long base = k * d;
    for (long n = base - 1; n <= base + 1; ++n)
      if (n >= 0 && n <= top) check_div(d, (int)n);
  }
  for (int i = 0; i < 200; ++i) check_div(d, (int)(next_u32() >> 1));
}

static void check_map(int tiles_m, int tiles_n, int group_m, int batch) {
  const sgemm::TileMap t = sgemm::make_tile_map(tiles_m, tiles_n, group_m);
  const int tiles = tiles_m * tiles_n;
  std::vector<char> seen((size_t)tiles * batch, 0);
  for (int id = 0; id < tiles * batch; ++id) {
    int bidx, tm, tn;
    t.tile(id, bidx, tm, tn);
    // the same raster with plain divisions
    const int eb = id / tiles, in_p = id - eb * tiles;
    const int per_group = group_m * tiles_n, g = in_p / per_group, first = g * group_m;
    const int rows = tiles_m - first < group_m ? tiles_m - first : group_m;
    const int in = in_p - g * per_group;
    const int etm = first + in % rows, etn = in / rows;
    const bool inside = bidx >= 0 && bidx < batch && tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n;
    if (bidx != eb || tm != etm || tn != etn || !inside || seen[((size_t)bidx * tiles_m + tm) * tiles_n + tn]++) {
      if (failures < 10)
        std::printf("TileMap(%d, %d, %d) id %d -> (%d, %d, %d), expected (%d, %d, %d)\n", tiles_m,
                    tiles_n, group_m, id, bidx, tm, tn, eb, etm, etn);
      ++failures;
    }
  }
}

int main() {
  long divisors = 0;
  for (int d = 1; d <= 4096; ++d, ++divisors) check_divisor(d);
  for (int k = 12; k <= 30; ++k)
    for (int e = -1; e <= 1; ++e, ++divisors) check_divisor((1 << k) + e);
  check_divisor(2147483647);
  check_divisor(2147483646);
  for (int i = 0; i < 300; ++i, ++divisors) check_divisor((int)(next_u32() >> 1) | 1);
  long maps = 0;
  for (int tm : {1, 2, 3, 7, 8, 9, 15, 16, 17, 33, 64})
    for (int tn : {1, 2, 5, 8, 13, 16, 31, 32})
      for (int gm : {1, 4, 8})
        for (int b : {1, 3}) check_map(tm, tn, gm, b), ++maps;
  std::printf("divisors %ld, tile maps %ld, failures %ld\n", divisors, maps, failures);
  return failures == 0 ? 0 : 1;
}
