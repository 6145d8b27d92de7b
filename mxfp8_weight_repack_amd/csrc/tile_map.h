// tile_map.h -- workgroup -> output tile mapping of the batched contraction.
//
// On MI355X workgroup i of a launch runs on XCD i % 8 and each XCD has its own
// L2.  When the tile grid splits into whole 8 x 8 super-tiles and their count
// is a multiple of 8, each XCD is given whole super-tiles (64 of its
// consecutive workgroups share 8 operand row tiles and 8 column tiles);
// otherwise tiles go in row-major order.  The mapping is a bijection of
// [0, tiles_m * tiles_n) onto the tile grid (checked on the host by a test).
// Compiles for the host too.
#pragma once

#if defined(__HIPCC__)
#define TM_HD __host__ __device__ __forceinline__
#else
#define TM_HD static inline
#endif

TM_HD void xcd_tile(int p, int tiles_m, int tiles_n, int *tm, int *tn) {
  const int sm = tiles_m / 8, sn = tiles_n / 8;
  if (tiles_m % 8 == 0 && tiles_n % 8 == 0 && (sm * sn) % 8 == 0) {
    const int x = p & 7, j = p >> 3;
    const int sup = (j >> 6) * 8 + x, in = j & 63;
    *tm = (sup / sn) * 8 + (in >> 3);
    *tn = (sup % sn) * 8 + (in & 7);
  } else {
    *tm = p / tiles_n;
    *tn = p - (p / tiles_n) * tiles_n;
  }
}
