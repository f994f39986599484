// Step 1: S += X^T X in fp64 (CHMC article, Methodik, Schritt 2: the layer
// Hessian from the calibration activations).
//
// One 128x128 tile of S per workgroup, upper-triangular tiles only (a <= b);
// an off-diagonal tile is also written to its mirror position. The token axis
// is the MFMA K axis: fp32 activations are widened to fp64 while staged in
// LDS, so every product is exact and only the fp64 sums round. When the tile
// count alone cannot fill the GPU, the token range is split across
// workgroups that write partial tiles to the workspace; a second kernel adds
// the partials in a fixed order.
#include "gemm64.h"

namespace gptq {

// Global X[token][feature] fp32 -> LDS [k][col] fp64, zero outside the token
// range and the feature range. Branch-free: the row pointer advances by GK
// rows per chunk and is clamped to the last row of the range, feature
// offsets are clamped into the row, every load is issued, and which values
// are in range is kept as a mask applied when the chunk is stored (so the
// load is waited on only then, one chunk of MFMAs later). With VEC (rows
// 16-byte aligned, dim % 4 == 0) each float4 is wholly in or out of range.
template <bool VEC>
struct LdX32 {
  const float* row0;   // this thread's first token row
  const float* rlast;  // the last token row of the range (clamp target)
  int64_t step;        // GK rows
  int64_t left;        // tokens from this thread's first row to the range end
  int f;               // this thread's first feature
  unsigned cols;       // bit q: feature f + q is in range
  f4 r[2];
  unsigned ok;         // bit q: value q of the fetched chunk is in range
  __device__ LdX32(const float* X, int64_t ldx, int64_t t_begin, int64_t t_end, int64_t dim,
                   int64_t f0, int t)
      : row0(X + (t_begin + (t >> 4)) * ldx), rlast(X + (t_end - 1) * ldx), step(GK * ldx),
        left(t_end - t_begin - (t >> 4)), f((int)f0 + (t & 15) * 8), cols(0u), r{}, ok(0u) {
#pragma unroll
    for (int q = 0; q < 8; ++q) cols |= (f + q < dim) ? 1u << q : 0u;
  }
  __device__ void fetch(int c, int) {
    const bool tok_ok = (int64_t)c * GK < left;
    const float* row = tok_ok ? row0 + c * step : rlast;
    ok = tok_ok ? cols : 0u;
    if (VEC) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        r[h] = *reinterpret_cast<const f4*>(row + (((cols >> (4 * h)) & 1u) ? f + 4 * h : 0));
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q >> 2][q & 3] = row[((cols >> q) & 1u) ? f + q : 0];
    }
  }
  __device__ void store(double* s, int t) const {
    double* d = s + (t >> 4) * GLD + (t & 15) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) d[q] = ((ok >> q) & 1u) ? (double)r[q >> 2][q & 3] : 0.0;
  }
};

// Upper-triangle tile id -> (a, b), a <= b, row-major over the triangle of an
// nt x nt tile grid.
__device__ inline void upper_tile(int id, int nt, int& a, int& b) {
  // rows have nt, nt-1, ... tiles; walk with a closed-form guess then fix up
  int row = 0, start = 0;
  // solve start(row) = row*nt - row*(row-1)/2 <= id
  double disc = (2.0 * nt + 1.0) * (2.0 * nt + 1.0) - 8.0 * id;
  row = (int)(((2.0 * nt + 1.0) - sqrt(disc)) * 0.5);
  if (row < 0) row = 0;
  if (row > nt - 1) row = nt - 1;
  while (row > 0 && row * nt - row * (row - 1) / 2 > id) --row;
  while (row + 1 < nt && (row + 1) * nt - (row + 1) * row / 2 <= id) ++row;
  start = row * nt - row * (row - 1) / 2;
  a = row;
  b = row + (id - start);
}

// ACC: add to the old values of S in place (the tile starts from them);
// else the tile starts from zero and overwrites S or writes a partial tile.
// Every workgroup has at least one token: split ranges all start below
// n_tokens.
template <bool VEC, bool ACC>
__global__ __launch_bounds__(256) void hess_tile_kernel(const float* __restrict__ X, int64_t ldx,
                                                        int64_t n_tokens, int64_t dim, int nt,
                                                        int ntiles, int64_t tok_per_split,
                                                        double* __restrict__ S, int64_t lds,
                                                        double* __restrict__ part) {
  __shared__ double sAB[4 * GCH];
  double* sA = sAB;
  double* sB = sAB + 2 * GCH;
  const int nblocks = gridDim.x;
  const int lin = xcd_remap(blockIdx.x, nblocks);
  const int tile = lin % ntiles;
  const int split = lin / ntiles;
  int a, b;
  upper_tile(tile, nt, a, b);
  const int64_t t0 = (int64_t)split * tok_per_split;
  int64_t t1 = t0 + tok_per_split;
  if (t1 > n_tokens) t1 = n_tokens;
  const int nchunks = (int)cdiv(t1 - t0, GK);

  const int64_t fa = (int64_t)a * GT, fb = (int64_t)b * GT;
  const int rows = (int)(dim - fa < GT ? dim - fa : GT);
  const int cols = (int)(dim - fb < GT ? dim - fb : GT);
  // The epilogue is a plain store, so the accumulators stay in the matrix
  // registers through the loop. S is symmetric on entry (every call leaves
  // it so); the mirror tile is rewritten from the upper one.
  d4 acc[4][4];
  if (ACC)
    acc_load_lds(acc, S + fa * lds + fb, lds, rows, cols, sAB);
  else
    zero_acc(acc);
  {
    LdX32<VEC> la(X, ldx, t0, t1, dim, fa, threadIdx.x);
    LdX32<VEC> lb(X, ldx, t0, t1, dim, fb, threadIdx.x);
    gemm64_loop(la, lb, nchunks, sA, sB, acc);
  }
  if (part) {
    double* P = part + ((int64_t)split * ntiles + tile) * (GT * GT);
    for_each_acc(acc, [&](int r, int c, double v) { P[r * GT + c] = v; });
    return;
  }
  for_each_acc(acc, [&](int r, int c, double v) {
    if (r < rows && c < cols) {
      S[(fa + r) * lds + fb + c] = v;
      if (a != b) S[(fb + c) * lds + fa + r] = v;
    }
  });
}

// Sum the token-split partials of every tile in split order and add to S.
// One 64x64 quarter of a tile per workgroup: rows of the partials are read
// and rows of S written along the row; the mirror S[j][i] is written from an
// LDS transpose, so its rows are contiguous too.
__global__ __launch_bounds__(256) void hess_reduce_kernel(const double* __restrict__ part, int nsplit,
                                                          int nt, int ntiles, int64_t dim,
                                                          double* __restrict__ S, int64_t lds,
                                                          bool overwrite) {
  __shared__ double tr[64][65];
  const int tile = blockIdx.y, quarter = blockIdx.x;
  int a, b;
  upper_tile(tile, nt, a, b);
  const int qr = (quarter >> 1) * 64, qc = (quarter & 1) * 64;
  const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int64_t i0 = (int64_t)a * GT + qr, j0 = (int64_t)b * GT + qc;
  const double* src = part + (int64_t)tile * (GT * GT) + qr * GT + qc;
  // all loads of a split (and of the old S) before any store, so they are in
  // flight together
  double acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0;
  for (int p = 0; p < nsplit; ++p) {
    double v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = src[(int64_t)p * ntiles * (GT * GT) + (rg + 4 * m) * GT + c];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] += v[m];
  }
  if (!overwrite) {
    double old[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int64_t i = i0 + rg + 4 * m, j = j0 + c;
      old[m] = (i < dim && j < dim) ? S[i * lds + j] : 0.0;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = old[m] + acc[m];
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int r = rg + 4 * m;
    const int64_t i = i0 + r, j = j0 + c;
    if (i < dim && j < dim) S[i * lds + j] = acc[m];
    tr[r][c] = acc[m];
  }
  if (a == b) return;  // a diagonal tile is its own mirror (uniform per workgroup)
  __syncthreads();
  for (int m = 0; m < 16; ++m) {
    const int r = rg + 4 * m;  // row of the mirror block = column of this block
    const int64_t j = j0 + r, i = i0 + c;
    if (i < dim && j < dim) S[j * lds + i] = tr[c][r];
  }
}

__global__ void hess_zero_kernel(double* __restrict__ S, int64_t count) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * blockDim.x)
    S[e] = 0.0;
}

static void hess_plan(int64_t dim, int64_t n, int& nt, int& ntiles, int& nsplit, int64_t& tps) {
  nt = (int)cdiv(dim, GT);
  ntiles = nt * (nt + 1) / 2;
  int64_t want = cdiv(1024, ntiles);
  int64_t cap_tok = n / 256;
  if (want > cap_tok) want = cap_tok;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  tps = round_up(cdiv(n, want), GK);
  nsplit = (int)cdiv(n, tps);
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_workspace_bytes(int64_t in_features, int64_t n_tokens) {
  if (in_features <= 0 || n_tokens <= 0) return 0;
  int nt, ntiles, nsplit;
  int64_t tps;
  hess_plan(in_features, n_tokens, nt, ntiles, nsplit, tps);
  if (nsplit <= 1) return 0;
  return (size_t)nsplit * ntiles * GT * GT * sizeof(double);
}

extern "C" gptq_status gptq_hessian_accumulate(double* S, int64_t in_features, const float* X,
                                               int64_t n_tokens, int64_t ldx, uint32_t flags,
                                               void* ws, size_t ws_bytes, void* stream) {
  if (in_features < 0 || n_tokens < 0) return GPTQ_EINVAL;
  if (flags & ~GPTQ_FLAG_HESSIAN_OVERWRITE) return GPTQ_EINVAL;
  const bool overwrite = (flags & GPTQ_FLAG_HESSIAN_OVERWRITE) != 0;
  if (in_features == 0 || (n_tokens == 0 && !overwrite)) return GPTQ_OK;
  if (!S) return GPTQ_EINVAL;
  if (in_features > (int64_t)1 << 20) return GPTQ_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (n_tokens == 0) {
    const int64_t cnt = in_features * in_features;
    GPTQ_LAUNCH(K_FILL, st,
                hess_zero_kernel<<<(unsigned)std::min<int64_t>(cdiv(cnt, 256), 65536), 256, 0, st>>>(
                    S, cnt));
    return GPTQ_OK;
  }
  if (!X || ldx < in_features) return GPTQ_EINVAL;
  int nt, ntiles, nsplit;
  int64_t tps;
  hess_plan(in_features, n_tokens, nt, ntiles, nsplit, tps);
  const size_t need = gptq_hessian_workspace_bytes(in_features, n_tokens);
  if (!ws || ws_bytes < need || need == 0) {  // no (usable) workspace: one split
    nsplit = 1;
    tps = round_up(n_tokens, GK);
  }
  const bool vec = (ldx % 4 == 0) && (in_features % 4 == 0) && ((uintptr_t)X % 16 == 0);
  double* part = nsplit > 1 ? (double*)ws : nullptr;
  const int nblocks = ntiles * nsplit;
  // in place only when there is no partial-tile pass (that one adds in the reduce)
  const bool acc_in_place = !overwrite && !part;
#define HESS_TILE(V, A)                                                                       \
  GPTQ_LAUNCH(K_HESS_TILE, st,                                                                 \
              (hess_tile_kernel<V, A><<<nblocks, 256, 0, st>>>(X, ldx, n_tokens, in_features, \
                                                               nt, ntiles, tps, S,            \
                                                               in_features, part)))
  if (vec) {
    if (acc_in_place) HESS_TILE(true, true);
    else HESS_TILE(true, false);
  } else {
    if (acc_in_place) HESS_TILE(false, true);
    else HESS_TILE(false, false);
  }
#undef HESS_TILE
  if (part) {
    dim3 grid(4, ntiles);
    GPTQ_LAUNCH(K_HESS_REDUCE, st,
                hess_reduce_kernel<<<grid, 256, 0, st>>>(part, nsplit, nt, ntiles, in_features, S,
                                                         in_features, overwrite));
  }
  return GPTQ_OK;
}
