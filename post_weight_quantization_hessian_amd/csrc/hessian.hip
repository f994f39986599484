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

// ---------------------------------------------------------------- split8
//
// Digit-sliced route on the int8 matrix cores (the error-free splitting of a
// matrix product into exactly computed integer slice products, Ozaki, Ogita,
// Oishi and Rump; here applied to X^T X). Per call, activation column f gets
// the power-of-two scale 2^e_f with max_k |x_kf| < 2^e_f, and every value of
// the column becomes the integer m = rint(x * 2^(30 - e_f)), |m| < 2^30,
// written as m = d0*2^24 + d1*2^16 + d2*2^8 + d3 with signed-byte digits
// d1..d3 in [-128, 127] and |d0| <= 64. Then
//   x_kf x_kg = 2^(e_f + e_g - 60) * sum_{a,b} d_a d_b 2^(48 - 8(a + b)),
// and for every digit order s = a + b the sum T_s = sum_{a+b=s} D_a^T D_b over
// the tokens is an exact int32 product on v_mfma_i32_32x32x32_i8 (at most
// 4 * 2^14 per token, 16384 tokens per workgroup). Only the orders s <= 4 are
// formed (13 of the 16 digit pairs): the orders 5 and 6 weigh at most
// (2 * 2^14 * 2^8 + 2^14) * 2^(e_f + e_g - 60) < 2^(e_f + e_g - 36.99) per
// token, under 2^-6 of what rounding x to the fixed point may already change
// in a product (up to 2^(e_f + e_g - 30)). Each T_s is added into fp64 accumulators once
// it is complete. What this represents exactly is x rounded to 30 fractional
// bits of its column's scale, less the orders 5 and 6 of its digit products;
// no other error than the fp64 additions.

constexpr int H8_KB = 64;               // tokens per staged chunk
constexpr int H8_LD = 64;               // LDS row pitch in bytes, 16-byte chunks swizzled
constexpr int H8_BUF = 4 * GT * H8_LD;  // one chunk of 128 rows: 4 digit planes
constexpr int H8_GRP = 8;               // tiles are visited in 8x8 groups (L2 reuse)
constexpr int H8_MAXTOK = 16384;        // tokens per workgroup (int32 range of T_s)
constexpr int H8_BAD = 0x40000000;      // exponent of a column holding NaN/Inf
constexpr int H8_ORD = 5;               // digit orders s = a + b formed: 0 .. 4

typedef int i4v __attribute__((ext_vector_type(4)));
typedef int i16v __attribute__((ext_vector_type(16)));

__global__ void h8_zero_kernel(unsigned* __restrict__ p, int64_t count) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = 0u;
}

// colmax[f] = max over the call's tokens of the bits of |x_kf| (as unsigned,
// which orders non-negative floats; NaN/Inf give bits >= 0x7f800000).
// Workgroup: 64 features x 64 tokens, thread t takes feature t % 64 and 16
// tokens of each 64-token block it visits. Grid (cdiv(dim, 64), up to
// 65535), the token blocks strided by the grid's y extent.
__global__ __launch_bounds__(256) void h8_colmax_kernel(const float* __restrict__ X, int64_t ldx,
                                                        int64_t n, int64_t dim,
                                                        unsigned* __restrict__ colmax) {
  const int64_t f = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  if (f >= dim) return;
  unsigned m = 0u;
  for (int64_t k0 = (int64_t)blockIdx.y * 64 + (threadIdx.x >> 6) * 16; k0 < n;
       k0 += (int64_t)gridDim.y * 64) {
    const int cnt = n - k0 < 16 ? (int)(n - k0) : 16;
    unsigned v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = q < cnt ? __float_as_uint(X[(k0 + q) * ldx + f]) : 0u;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const unsigned b = v[q] & 0x7fffffffu;
      m = b > m ? b : m;
    }
  }
  atomicMax(colmax + f, m);
}

__device__ inline int h8_exponent(unsigned bits) {
  if (bits >= 0x7f800000u) return H8_BAD;
  if (bits == 0u) return 0;
  int e;
  (void)frexpf(__uint_as_float(bits), &e);  // max = mant * 2^e, mant in [0.5, 1)
  return e;
}

// Digits of feature f, 64-token chunk c (c < npad / 64) and plane a (0..3)
// at dig[((f * (npad / 64) + c) * 4 + a) * 64 + k % 64] (int8): the four
// planes of one feature and chunk are one contiguous 256-byte block, so that
// the tile kernel's loads of a chunk use whole cache lines. Zero outside the
// token and feature range and in columns holding NaN/Inf. Workgroup: 64 features x 64 tokens; thread t takes
// feature t % 64 and 16 consecutive tokens. Blocks with blockIdx.x == 0 also
// write the column exponents. Grid (npad / 64, dpad / 64).
__global__ __launch_bounds__(256) void h8_split_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t n, int64_t dim,
                                                       const unsigned* __restrict__ colmax,
                                                       int* __restrict__ exps,
                                                       int8_t* __restrict__ dig, int64_t dpad,
                                                       int64_t npad) {
  const int r = threadIdx.x & 63, tg = threadIdx.x >> 6;
  const int64_t f = (int64_t)blockIdx.y * 64 + r;
  const int64_t k0 = (int64_t)blockIdx.x * 64 + tg * 16;
  const int e = f < dim ? h8_exponent(colmax[f]) : 0;
  if (blockIdx.x == 0 && tg == 0) exps[f] = e;
  const bool live = f < dim && e != H8_BAD;
  float x[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) x[q] = (live && k0 + q < n) ? X[(k0 + q) * ldx + f] : 0.0f;
  unsigned w[4][4];  // [digit][token quad], little-endian bytes
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) w[a][qq] = 0u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    int m = __float2int_rn(ldexpf(x[q], 30 - e));
    int d[4];
#pragma unroll
    for (int a = 3; a >= 1; --a) {
      d[a] = (int)(signed char)(m & 0xff);
      m = (m - d[a]) >> 8;
    }
    d[0] = m;
#pragma unroll
    for (int a = 0; a < 4; ++a) w[a][q >> 2] |= ((unsigned)d[a] & 0xffu) << (8 * (q & 3));
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint4 v = make_uint4(w[a][0], w[a][1], w[a][2], w[a][3]);
    *reinterpret_cast<uint4*>(dig + ((f * (npad / H8_KB) + blockIdx.x) * 4 + a) * H8_KB +
                              tg * 16) = v;
  }
}

// 128-tile of a launch slot: the upper triangle of 128x128 tiles is visited
// in groups of 8x8 tiles (row-major over the triangle of groups, row-major
// inside a group), so that the workgroups resident on one XCD share operand
// rows in its L2. Slots of a group that fall below the diagonal or outside
// the matrix have no tile.
__device__ inline bool h8_tile_of(int id, int nt, int& a, int& b) {
  const int ng = (nt + H8_GRP - 1) / H8_GRP;
  int ga, gb;
  upper_tile(id / (H8_GRP * H8_GRP), ng, ga, gb);
  const int loc = id % (H8_GRP * H8_GRP);
  a = ga * H8_GRP + loc / H8_GRP;
  b = gb * H8_GRP + loc % H8_GRP;
  return a <= b && b < nt;
}

// One upper 128-tile of S (a <= b) for one token split per workgroup: eight
// waves (two per SIMD), wave w takes rows 32 (w / 2) .. +31 and columns
// 64 (w % 2) .. +63 as two 32 x 32 v_mfma_i32_32x32x32_i8 blocks that share
// the row operands. Every 64-token chunk stages all four digit planes of the
// 128 rows and of the 128 columns in LDS, and the 13 digit pairs of orders
// s = a + b <= 4 are multiplied from there; each order and column block has
// its own int32 accumulator for the whole token range (2 x 5 x 16 = 160
// registers), combined in fp64 at the end. v_mfma_i32_32x32x32_i8 operands
// (lane l): 16 int8 of row l%32 of A (of column l%32 of B) over the tokens
// 16*(l/32) .. +15 of the 32-token step; A and B are loaded alike, so the
// pairing of their k indices inside the instruction is the same for both.
// D reg x: row 8*(x/4) + 4*(l/32) + x%4, col l%32. The next chunk is loaded
// into registers while the current one is multiplied, and two chunks
// alternate in LDS.
__global__ __launch_bounds__(512, 1) void h8_tile_kernel(const int8_t* __restrict__ dig, int64_t dpad,
                                                         int64_t npad, const int* __restrict__ exps,
                                                         int64_t n_tokens, int64_t dim, int nt,
                                                         int nslots, int64_t tok_per_split,
                                                         double* __restrict__ S, int64_t lds,
                                                         double* __restrict__ part, bool acc_old) {
  __shared__ __attribute__((aligned(16))) int8_t sm[2][2 * H8_BUF];
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int slot = lin % nslots;
  const int split = lin / nslots;
  int ta, tb;
  if (!h8_tile_of(slot, nt, ta, tb)) return;  // uniform per workgroup
  const int64_t fa = (int64_t)ta * GT, fb = (int64_t)tb * GT;
  const int64_t t0 = (int64_t)split * tok_per_split;
  int64_t t1 = t0 + tok_per_split;
  const int64_t tend = round_up(n_tokens, H8_KB);
  if (t1 > tend) t1 = tend;
  const int nst = (int)((t1 - t0) / H8_KB);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;
  // loads: row lrow of all four planes of A and of B; 16-byte chunk lch of
  // the 64 tokens
  const int lrow = tid >> 2, lch = tid & 3;
  // one chunk of a feature: 4 planes x 64 tokens, contiguous (256 bytes)
  constexpr int CHB = 4 * H8_KB;
  const int64_t nchk = npad / H8_KB;
  const int8_t* gA = dig + ((fa + lrow) * nchk + t0 / H8_KB) * CHB + lch * 16;
  const int8_t* gB = dig + ((fb + lrow) * nchk + t0 / H8_KB) * CHB + lch * 16;
  i4v ra[4], rb[4];
  auto fetch = [&](int k) {
    if (k > nst - 1) k = nst - 1;  // past the end: reload the last chunk (never used)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ra[q] = *reinterpret_cast<const i4v*>(gA + (int64_t)k * CHB + q * H8_KB);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rb[q] = *reinterpret_cast<const i4v*>(gB + (int64_t)k * CHB + q * H8_KB);
  };
  // LDS rows of 64 bytes; chunk c of row r sits at position c ^ ((r >> 2) & 3).
  // Stores (four lanes per row, 16 lanes = 4 consecutive rows) cover 64
  // distinct banks, and so do operand reads (16 consecutive rows at one
  // chunk: row r mod 4 picks the 16-bank quarter, the swizzle the 4 banks)
  auto stash = [&](int buf) {
    int8_t* A = sm[buf] + lrow * H8_LD + ((lch ^ ((lrow >> 2) & 3)) << 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<i4v*>(A + q * (GT * H8_LD)) = ra[q];
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<i4v*>(A + H8_BUF + q * (GT * H8_LD)) = rb[q];
  };
  i16v acc[2][H8_ORD];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int o = 0; o < H8_ORD; ++o)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[cb][o][x] = 0;
  // operand rows: wr*32 + l%32 (A), wc*64 + cb*32 + l%32 (B); all have the
  // same swizzle, (l%32 >> 2) & 3, since 32-row offsets leave bits 2-3 alone
  const int sw = ((lane & 31) >> 2) & 3;
  const int arow = (wr * 32 + (lane & 31)) * H8_LD;
  const int brow = H8_BUF + (wc * 64 + (lane & 31)) * H8_LD;
  const int koff[2] = {(((lane >> 5) + 0) ^ sw) << 4, (((lane >> 5) + 2) ^ sw) << 4};
  fetch(0);
  stash(0);
  fetch(1);
  __syncthreads();
  for (int k = 0; k < nst; ++k) {
    const int8_t* base = sm[k & 1];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      i4v av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[q] = *reinterpret_cast<const i4v*>(base + q * (GT * H8_LD) + arow + koff[kh]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        i4v bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bv[q] = *reinterpret_cast<const i4v*>(base + q * (GT * H8_LD) + brow + cb * 32 * H8_LD +
                                                koff[kh]);
#pragma unroll
        for (int da = 0; da < 4; ++da)
#pragma unroll
          for (int db = 0; db < 4; ++db)
            if (da + db < H8_ORD)
              acc[cb][da + db] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[da], bv[db],
                                                                       acc[cb][da + db], 0, 0, 0);
      }
    }
    // unconditional, so that the load counters stay in issue order on every
    // path (after the last chunk this fills the idle buffer)
    stash((k + 1) & 1);
    fetch(k + 2);
    __syncthreads();
  }
  // S_fg = 2^(e_f + e_g - 60) * sum_{s<=4} 2^(48 - 8 s) T_s, smallest terms first
  const int canon = ta * nt - ta * (ta - 1) / 2 + (tb - ta);  // row-major triangle order
  const int ntiles = nt * (nt + 1) / 2;
  double* P = part ? part + ((int64_t)split * ntiles + canon) * (GT * GT) : nullptr;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = wc * 64 + cb * 32 + (lane & 31);  // column inside the tile
    const int ec = exps[fb + c];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int r = wr * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
      const int er = exps[fa + r];
      double t = __builtin_ldexp((double)acc[cb][H8_ORD - 1][x], 48 - 8 * (H8_ORD - 1));
#pragma unroll
      for (int o = H8_ORD - 2; o >= 0; --o)
        t += __builtin_ldexp((double)acc[cb][o][x], 48 - 8 * o);
      const double v = (er == H8_BAD || ec == H8_BAD) ? __builtin_nan("")
                                                      : __builtin_ldexp(t, er + ec - 60);
      if (P) {
        P[r * GT + c] = v;
      } else if (fa + r < dim && fb + c < dim) {
        double* d = S + (fa + r) * lds + fb + c;
        const double o = acc_old ? *d + v : v;
        *d = o;
        // a diagonal tile is written whole (its two triangles are exact
        // integer sums of the same products, so they agree bit for bit)
        if (ta != tb) S[(fb + c) * lds + fa + r] = o;
      }
    }
  }
}

// Token splits: only while the tiles (one workgroup each, one workgroup per
// CU) number fewer than two rounds of the GPU, and whenever a workgroup would
// otherwise take more than H8_MAXTOK tokens.
static void h8_plan(int64_t dim, int64_t n, int& nt, int& ntiles, int& nsplit, int64_t& tps) {
  nt = (int)cdiv(dim, GT);
  ntiles = nt * (nt + 1) / 2;
  int64_t want = cdiv(512, ntiles);
  int64_t cap_tok = n / 512;
  if (want > cap_tok) want = cap_tok;
  if (want > 64) want = 64;
  if (want < cdiv(n, H8_MAXTOK)) want = cdiv(n, H8_MAXTOK);
  if (want < 1) want = 1;
  tps = round_up(cdiv(n, want), H8_KB);
  nsplit = (int)cdiv(n, tps);
}

struct H8Layout {
  int64_t dpad, npad, off_exps, off_dig, off_part, total;
  int nt, ntiles, nsplit, nslots;
  int64_t tps;
  H8Layout(int64_t dim, int64_t n) {
    h8_plan(dim, n, nt, ntiles, nsplit, tps);
    const int ng = (int)cdiv(nt, H8_GRP);
    nslots = ng * (ng + 1) / 2 * H8_GRP * H8_GRP;
    dpad = round_up(dim, GT);
    npad = round_up(n, H8_KB);
    off_exps = round_up(dpad * 4, 256);
    off_dig = off_exps + round_up(dpad * 4, 256);
    off_part = off_dig + round_up(4 * dpad * npad, 256);
    total = off_part + (nsplit > 1 ? (int64_t)nsplit * ntiles * GT * GT * 8 : 0);
  }
};

static gptq_status hess_split8(double* S, int64_t dim, const float* X, int64_t n, int64_t ldx,
                               bool overwrite, void* ws, size_t ws_bytes, hipStream_t st) {
  H8Layout L(dim, n);
  if ((int64_t)L.nslots * L.nsplit > INT32_MAX) return GPTQ_EINVAL;  // one launch grid
  if (!ws || ws_bytes < (size_t)L.total) return GPTQ_EWORKSPACE;
  char* base = (char*)ws;
  unsigned* colmax = (unsigned*)base;
  int* exps = (int*)(base + L.off_exps);
  int8_t* dig = (int8_t*)(base + L.off_dig);
  double* part = L.nsplit > 1 ? (double*)(base + L.off_part) : nullptr;
  GPTQ_LAUNCH(K_FILL, st,
              h8_zero_kernel<<<(unsigned)std::min<int64_t>(cdiv(dim, 256), 4096), 256, 0, st>>>(
                  colmax, dim));
  GPTQ_LAUNCH(K_HESS_DIGITS, st,
              h8_colmax_kernel<<<dim3((unsigned)cdiv(dim, 64),
                                      (unsigned)std::min<int64_t>(cdiv(n, 64), 65535)),
                                 256, 0, st>>>(X, ldx, n, dim, colmax));
  GPTQ_LAUNCH(K_HESS_DIGITS, st,
              h8_split_kernel<<<dim3((unsigned)(L.npad / 64), (unsigned)(L.dpad / 64)), 256, 0,
                                st>>>(X, ldx, n, dim, colmax, exps, dig, L.dpad, L.npad));
  const int nblocks = L.nslots * L.nsplit;
  GPTQ_LAUNCH(K_HESS_SPLIT8, st,
              h8_tile_kernel<<<nblocks, 512, 0, st>>>(dig, L.dpad, L.npad, exps, n, dim, L.nt,
                                                      L.nslots, L.tps, S, dim, part,
                                                      !overwrite));
  if (part) {
    dim3 grid(4, L.ntiles);
    GPTQ_LAUNCH(K_HESS_REDUCE, st,
                hess_reduce_kernel<<<grid, 256, 0, st>>>(part, L.nsplit, L.nt, L.ntiles, dim, S,
                                                         dim, overwrite));
  }
  return GPTQ_OK;
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

extern "C" size_t gptq_hessian_split8_workspace_bytes(int64_t in_features, int64_t n_tokens) {
  if (in_features <= 0 || n_tokens <= 0) return 0;
  if (in_features > (int64_t)1 << 20) return 0;
  return (size_t)H8Layout(in_features, n_tokens).total;
}

extern "C" gptq_status gptq_hessian_accumulate(double* S, int64_t in_features, const float* X,
                                               int64_t n_tokens, int64_t ldx, uint32_t flags,
                                               void* ws, size_t ws_bytes, void* stream) {
  if (in_features < 0 || n_tokens < 0) return GPTQ_EINVAL;
  if (flags & ~(GPTQ_FLAG_HESSIAN_OVERWRITE | GPTQ_FLAG_HESSIAN_SPLIT8)) return GPTQ_EINVAL;
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
  if (flags & GPTQ_FLAG_HESSIAN_SPLIT8)
    return hess_split8(S, in_features, X, n_tokens, ldx, overwrite, ws, ws_bytes, st);
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
