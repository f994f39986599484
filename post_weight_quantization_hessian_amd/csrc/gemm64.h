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
// NEG stores the negated values.
template <bool NEG>
struct LdDirect64T {
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
    for (int q = 0; q < 4; ++q) *reinterpret_cast<dbl2*>(d + 2 * q) = NEG ? -r[q] : r[q];
  }
};
using LdDirect64 = LdDirect64T<false>;

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

// Double-buffered K loop over nchunks >= 1 chunks. The body is straight-line:
// every iteration fetches the next chunk (the last one re-fetches its own
// chunk, in bounds, into the buffer nobody reads any more), and there is one
// loop form for every tile (a diagonal tile loads its operand twice). A
// branchy body, or two loop forms in one kernel, made the compiler copy the
// 64 fp64 accumulators between vector and matrix registers around every
// chunk, or keep a second copy of them live across the loop.
template <class LA, class LB>
__device__ inline void gemm64_loop(LA& la, LB& lb, int nchunks, double* sA, double* sB,
                                   d4 (&acc)[4][4]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  la.fetch(0, t);
  lb.fetch(0, t);
  la.store(sA, t);
  lb.store(sB, t);
  __syncthreads();
  int c = 0;
  do {
    const int cur = c & 1;
    const int nx = c + 1 < nchunks ? c + 1 : c;
    la.fetch(nx, t);
    lb.fetch(nx, t);
    mfma64_chunk(sA + cur * GCH, sB + cur * GCH, acc, wm, wn, lane);
    la.store(sA + (cur ^ 1) * GCH, t);
    lb.store(sB + (cur ^ 1) * GCH, t);
    __syncthreads();
  } while (++c < nchunks);
}

__device__ inline void zero_acc(d4 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};
}

// acc = the tile at C (leading dimension ld), staged through LDS 64 rows at a
// time so the values reach the accumulators without a vector-register copy
// that would stay live across the K loop; entries at tile-local (row, col)
// with row >= rows or col >= cols read 0. `stage` holds >= 64 * GT doubles
// and is free on entry; a barrier follows.
__device__ inline void acc_load_lds(d4 (&acc)[4][4], const double* C, int64_t ld, int rows,
                                    int cols, double* stage) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // every load is issued before the first LDS store: `stage` is a generic
    // pointer, so a store between two loads would order them one by one
    double v[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int idx = e * 256 + t;
      const int rr = idx >> 7, cc = idx & 127;
      const int row = 64 * half + rr;
      const bool ok = row < rows && cc < cols;
      v[e] = C[ok ? (int64_t)row * ld + cc : 0];
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int idx = e * 256 + t;
      const int rr = idx >> 7, cc = idx & 127;
      const int row = 64 * half + rr;
      const bool ok = row < rows && cc < cols;
      stage[idx] = ok ? v[e] : 0.0;
    }
    __syncthreads();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = stage[(i * 16 + (lane >> 4) + 4 * r) * GT + wn * 64 + j * 16 + (lane & 15)];
    }
    __syncthreads();
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
