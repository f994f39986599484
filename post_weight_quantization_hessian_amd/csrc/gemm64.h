// fp64 MFMA tile machinery for gfx950: a 128x128 output tile per 256-thread
// workgroup (4 waves, each a 64x64 quadrant of 4x4 v_mfma_f64_16x16x4 tiles),
// K staged through LDS in chunks of 16, double buffered.
//
// v_mfma_f64_16x16x4f64 operand layout (lane l of 64):
//   A[m][k]: m = l % 16, k = l / 16        B[k][n]: n = l % 16, k = l / 16
//   D[m][n] (4 doubles per lane): n = l % 16, m = l / 16 + 4 * r, r = 0..3
#pragma once
#include "common.h"

namespace gptq {

constexpr int GT = 128;          // tile edge
constexpr int GK = 16;           // K chunk
constexpr int GLD = GT + 8;      // LDS row pitch (doubles), k-major rows
constexpr int GCH = GK * GLD;    // doubles per staged operand chunk

typedef double dbl2 __attribute__((ext_vector_type(2)));

// Wave quadrant MFMA over one staged chunk. As/Bs are k-major: As[k*GLD + m].
__device__ inline void mfma64_chunk(const double* __restrict__ As, const double* __restrict__ Bs,
                                    d4 (&acc)[4][4], int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < GK; kk += 4) {
    const int k = kk + (lane >> 4);
    double a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = As[k * GLD + wm * 64 + i * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = Bs[k * GLD + wn * 64 + i * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Global [k][col] (row stride ld) -> LDS [k][col]. All in bounds, 16B aligned.
struct LdDirect64 {
  const double* base;
  int64_t ld;
  dbl2 r[4];
  __device__ void fetch(int c, int t) {
    const double* p = base + (int64_t)(c * GK + (t >> 4)) * ld + (t & 15) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *reinterpret_cast<const dbl2*>(p + 2 * q);
  }
  __device__ void store(double* s, int t) const {
    double* d = s + (t >> 4) * GLD + (t & 15) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<dbl2*>(d + 2 * q) = r[q];
  }
};

// Global [col][k] (row stride ld) -> LDS [k][col] (transposing). In bounds.
// NEG stores the negated values (a negated operand keeps the epilogue a plain
// store, so the accumulators never leave the matrix registers).
template <bool NEG>
struct LdTrans64T {
  const double* base;
  int64_t ld;
  dbl2 r[4];
  __device__ void fetch(int c, int t) {
    const double* p = base + (int64_t)(t >> 1) * ld + c * GK + (t & 1) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *reinterpret_cast<const dbl2*>(p + 2 * q);
  }
  __device__ void store(double* s, int t) const {
    const int col = t >> 1, kh = (t & 1) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[(kh + 2 * q) * GLD + col] = NEG ? -r[q].x : r[q].x;
      s[(kh + 2 * q + 1) * GLD + col] = NEG ? -r[q].y : r[q].y;
    }
  }
};
using LdTrans64 = LdTrans64T<false>;

// Double-buffered K loop; with SAME the B operand is the A operand (la only).
// The body is straight-line: every iteration fetches the next chunk (the last
// one re-fetches its own chunk, in bounds, into the buffer nobody reads any
// more), so the accumulators stay in the matrix registers across iterations
// instead of being copied out and back around a branchy loop.
template <bool SAME, class LA, class LB>
__device__ inline void gemm64_loop(LA& la, LB& lb, int nchunks, double* sA, double* sB,
                                   d4 (&acc)[4][4]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  la.fetch(0, t);
  if (!SAME) lb.fetch(0, t);
  la.store(sA, t);
  if (!SAME) lb.store(sB, t);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int cur = c & 1;
    const int nx = c + 1 < nchunks ? c + 1 : c;
    la.fetch(nx, t);
    if (!SAME) lb.fetch(nx, t);
    const double* a = sA + cur * GCH;
    const double* b = SAME ? a : sB + cur * GCH;
    mfma64_chunk(a, b, acc, wm, wn, lane);
    la.store(sA + (cur ^ 1) * GCH, t);
    if (!SAME) lb.store(sB + (cur ^ 1) * GCH, t);
    __syncthreads();
  }
}

__device__ inline void zero_acc(d4 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};
}

// C[row][col] += sign * acc for the tile at C (leading dimension ld): all 64
// old values of the thread are loaded before any store, so the loads overlap
// (a load-add-store per element would serialize one memory round trip each).
__device__ inline void acc_update(const d4 (&acc)[4][4], double* C, int64_t ld, double sign) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  double* base = C + (int64_t)(wm * 64 + (lane >> 4)) * ld + wn * 64 + (lane & 15);
  double old[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) old[i][j][r] = base[(int64_t)(i * 16 + 4 * r) * ld + j * 16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        base[(int64_t)(i * 16 + 4 * r) * ld + j * 16] = old[i][j][r] + sign * acc[i][j][r];
}

// acc = the tile at C (leading dimension ld), in the accumulator layout;
// entries at tile-local (row, col) with row >= rows or col >= cols read 0.
// Loads are clamped into range and all issued before use.
__device__ inline void acc_load(d4 (&acc)[4][4], const double* C, int64_t ld, int rows, int cols) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + i * 16 + (lane >> 4) + 4 * r;
        const int col = wn * 64 + j * 16 + (lane & 15);
        const bool ok = row < rows && col < cols;
        const double v = C[ok ? (int64_t)row * ld + col : 0];
        acc[i][j][r] = ok ? v : 0.0;
      }
}

// Visit the tile's accumulators: f(row, col, value) with tile-local row/col.
template <class F>
__device__ inline void for_each_acc(const d4 (&acc)[4][4], F f) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f(wm * 64 + i * 16 + (lane >> 4) + 4 * r, wn * 64 + j * 16 + (lane & 15), acc[i][j][r]);
}

}  // namespace gptq
