// Tile order of the recursive-doubling triangular inverse.
//
// At level h the 128-tiles of L are grouped in blocks of 2h tile rows: block
// q has its first half at tile f0 = 2hq and its second half at s0 = f0 + h,
// with h tile rows in the second half except in the last block, which may
// have fewer (or none). For every tile (r, c) of the second half's
// off-diagonal block, r < rows(q) and c < h:
//   T[r][c]  = sum_{k=c}^{h-1} L[s0+r][f0+k] X[f0+k][f0+c]   (h - c tile products)
//   X[r][c]  = -sum_{k=0}^{r} X[s0+r][s0+k] T[k][c]           (r + 1 tile products)
// Both launches enumerate their tiles heaviest first, and the tiles are taken
// in dispatch order (round-robin over the XCDs), so every XCD gets the same
// mix and the short tiles fill the tail of the launch.
#pragma once
#include <cstdint>

namespace gptq {

// Tile rows in the second half of the last block (<= 0: it has none).
__host__ __device__ inline int level_last_rows(int h, int nt) {
  const int nq = (nt + 2 * h - 1) / (2 * h);
  return nt - (nq - 1) * 2 * h - h;
}

__host__ __device__ inline int level_blocks(int h, int nt) { return (nt + 2 * h - 1) / (2 * h); }

// Number of off-diagonal tiles at level h.
__host__ __device__ inline int level_tiles(int h, int nt) {
  const int nq = level_blocks(h, nt);
  const int last = level_last_rows(h, nt);
  return (nq - 1) * h * h + (last > 0 ? last * h : 0);
}

// T-product tile `id`: c ascending (h - c products, heaviest first), then the
// tile rows of every block in order.
__host__ __device__ inline void level_tile_t(int id, int h, int nt, int& r, int& c, int64_t& f0,
                                             int64_t& s0) {
  const int nq = level_blocks(h, nt);
  const int last = level_last_rows(h, nt);
  const int rows_per_c = (nq - 1) * h + (last > 0 ? last : 0);
  c = id / rows_per_c;
  const int rem = id - c * rows_per_c;
  const int q = rem / h;
  r = rem - q * h;
  f0 = (int64_t)q * 2 * h;
  s0 = f0 + h;
}

// X-update tile `id`: r descending (r + 1 products, heaviest first). Rows
// r >= last exist only in the nq - 1 full blocks; rows below `last` in all nq.
__host__ __device__ inline void level_tile_x(int id, int h, int nt, int& r, int& c, int64_t& f0,
                                             int64_t& s0) {
  const int nq = level_blocks(h, nt);
  const int lastr = level_last_rows(h, nt);
  const int last = lastr > 0 ? lastr : 0;
  const int nfull = nq - 1;
  const int seg1 = (h - last) * nfull * h;  // tiles of the rows only full blocks have
  int q, rem;
  if (id < seg1) {
    const int per = nfull * h;
    const int k = id / per;
    rem = id - k * per;
    r = h - 1 - k;
  } else {
    const int per = (nfull + 1) * h;
    const int id2 = id - seg1;
    const int k = id2 / per;
    rem = id2 - k * per;
    r = last - 1 - k;
  }
  q = rem / h;
  c = rem - q * h;
  f0 = (int64_t)q * 2 * h;
  s0 = f0 + h;
}

}  // namespace gptq
