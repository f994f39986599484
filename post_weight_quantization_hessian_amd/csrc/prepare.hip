// Steps 2-3: damping, act-order and the upper factor U of the inverse Hessian
// (CHMC article, Methodik, Schritt 2: H = X^T X/n + lambda*mean(diag H)*I,
// "H^-1 via the Cholesky decomposition", act-order; The Geometry of LLM
// Quantization 2.3: act-order = descending diag H pivot order).
//
// Route: with J the order reversal and Hp the permuted damped Hessian,
//   K = J Hp J = L L^T (lower Cholesky),  U = J L^-1 J,
// which is upper triangular with U^T U = Hp^-1. One Cholesky and one
// triangular inverse, both blocked by 128 in fp64 on MFMA; K is padded to a
// multiple of 128 with an identity block so no kernel needs edge masks.
// The factor form skips the inverse beyond the 128 x 128 diagonal tiles:
// R = J L J = U^-1 is the upper factor of Hp itself (Hp = R R^T), and the
// output holds U's diagonal blocks and R U over each block beyond them (one
// 128 x 128 product per tile of L), which the sweep takes with the
// residuals Q - W in place of the scaled errors (The Geometry of LLM
// Quantization 2.1-2.2: any triangular factor of the Hessian serves the
// nearest-plane step). K is then padded before the matrix, so that its tiles
// end at the matrix end and map onto the sweep's 128-blocks.
#include "gemm64.h"
#include "trtri_order.h"

namespace gptq {

// ---------------------------------------------------------------- damping

// One workgroup: d[k] = c*S[k][k]; lam = damp * mean(d); hd[k] = d[k] + lam.
__global__ __launch_bounds__(1024) void prep_diag_kernel(const double* __restrict__ S, int64_t n,
                                                         double c, double damp,
                                                         double* __restrict__ hd,
                                                         double* __restrict__ lam_out) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < n; k += blockDim.x) {
    const double d = c * S[k * n + k];
    hd[k] = d;
    s += d;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const double lam = damp * (red[0] / (double)n);
  for (int64_t k = threadIdx.x; k < n; k += blockDim.x) hd[k] += lam;
  if (threadIdx.x == 0) *lam_out = lam;
}

// perm[rank(k)] = k with rank(k) = #{j : hd[j] > hd[k] or (hd[j] == hd[k] and
// j < k)}: the stable order of descending damped diagonal. Identity if !act.
// 16 lanes per key, each counting every 16th j of the staged tiles, the 16
// counts summed with lane shuffles: n/16 workgroups of 16 keys, so that a few
// thousand features fill the GPU.
__global__ __launch_bounds__(256) void prep_perm_kernel(const double* __restrict__ hd, int64_t n,
                                                        bool act, int32_t* __restrict__ perm) {
  __shared__ double tile[1024];
  const int kl = threadIdx.x >> 4, jl = threadIdx.x & 15;
  const int64_t k = (int64_t)blockIdx.x * 16 + kl;
  if (!act) {  // uniform
    if (k < n && jl == 0) perm[k] = (int32_t)k;
    return;
  }
  const double mine = k < n ? hd[k] : 0.0;
  int rank = 0;  // < n < 2^31 (perm is int32)
  for (int64_t j0 = 0; j0 < n; j0 += 1024) {
    const int m = (int)((n - j0) < 1024 ? (n - j0) : 1024);
    __syncthreads();
    for (int q = threadIdx.x; q < m; q += blockDim.x) tile[q] = hd[j0 + q];
    __syncthreads();
    if (k < n) {
      for (int q = jl; q < m; q += 16) {
        const double v = tile[q];
        rank += (v > mine) || (v == mine && j0 + q < k);
      }
    }
  }
  rank += __shfl_xor(rank, 1, 16);
  rank += __shfl_xor(rank, 2, 16);
  rank += __shfl_xor(rank, 4, 16);
  rank += __shfl_xor(rank, 8, 16);
  if (k < n && jl == 0) perm[rank] = (int32_t)k;
}

// Lower triangle of K (ip x ip, ld ip): K[a][b] = H[p_a][p_b], p_x =
// perm[n-1-(x-off)], H = c*S + lam*I; the padding (a, b < off or >= off + n)
// is the identity. off = 0 puts the padding after the matrix; off = ip - n
// before it, so that the 128-tiles of K end where the matrix ends and map to
// 128-blocks of the sweep order that start at 0. `split` blocks
// per row, each a contiguous range of b; the blocks of one row are
// consecutive after the XCD remap, so they run on one XCD and the scattered
// reads of the permuted S row are served from its L2. Large matrices take 8
// blocks of 1024 threads per row (with one block per row, the rows in
// flight did not fit the L2s and most reads of a row went to memory again);
// small ones one block of 256 threads, whose rows fit anyway.
constexpr int64_t GATHER_SPLIT_FROM = 8192;  // features from which rows are split
__global__ __launch_bounds__(1024) void prep_gather_kernel(const double* __restrict__ S, int64_t n,
                                                           int64_t ip, double c,
                                                           const double* __restrict__ lam_p,
                                                           const int32_t* __restrict__ perm,
                                                           double* __restrict__ K, int split,
                                                           int64_t off) {
  const int64_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t a = lin / split;
  const int q = (int)(lin % split);
  const int64_t lo = (a + 1) * q / split, hi = (a + 1) * (q + 1) / split;
  const double lam = *lam_p;
  double* row = K + a * ip;
  const int64_t ra = a - off;
  if (ra < 0 || ra >= n) {
    for (int64_t b = lo + threadIdx.x; b < hi; b += blockDim.x) row[b] = (a == b) ? 1.0 : 0.0;
    return;
  }
  // without perm: H itself in the original order (the min-pivot search)
  const int64_t pa = perm ? perm[n - 1 - ra] : ra;
  const double* srow = S + pa * n;
  for (int64_t b = lo + threadIdx.x; b < hi; b += blockDim.x) {
    const int64_t rb = b - off;
    if (rb < 0) {
      row[b] = 0.0;
      continue;
    }
    const int64_t pb = perm ? perm[n - 1 - rb] : rb;
    double v = c * srow[pb];
    if (a == b) v += lam;
    row[b] = v;
  }
}

// ---------------------------------------------------------------- Cholesky
//
// Diagonal 128x128 block of panel p: factor and invert it in LDS, 16 columns
// at a time. The block is held as the 36 lower 16x16 tiles, each stored
// column-major with pitch 17 (conflict-free MFMA fragment reads). Per 16-wide
// step s: one wave factors the 16x16 diagonal tile (no workgroup barrier
// inside), all threads solve the rows below against it by substitution, and
// the waves update the trailing tiles with fp64 MFMA. The inverse then takes
// the eight 16x16 diagonal inverses (one wave each) and assembles the
// off-diagonal tiles by distance from the diagonal:
//     X_ij = -X_ii * sum_{k=j}^{i-1} L_ik X_kj.

constexpr int PT = 17;        // tile pitch (column-major)
constexpr int PTS = 16 * PT;  // doubles per tile
constexpr int NPT = 36;       // lower tiles of an 8x8 tile grid

__device__ inline int ptile(int I, int K) { return (I * (I + 1) / 2 + K) * PTS; }
// tile row I of lower tile number u = I (I + 1) / 2 + K (compile-time in unrolled loops)
__device__ constexpr int tile_row(int u) { return u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : u < 10 ? 3 : u < 15 ? 4 : u < 21 ? 5 : u < 28 ? 6 : 7; }

// Order the LDS accesses of one wave (they execute in order in hardware).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ inline double readlane_f64(double v, int lane) {
  union { double d; int i[2]; } a;
  a.d = v;
  a.i[0] = __builtin_amdgcn_readlane(a.i[0], lane);
  a.i[1] = __builtin_amdgcn_readlane(a.i[1], lane);
  return a.d;
}

// 1/sqrt(d) for d > 0: hardware estimate refined by two Newton steps.
__device__ inline double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  const double h = 0.5 * d;
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

// One wave: in-place Cholesky of the 16x16 tile T (lower part; column-major,
// pitch PT), 1/diag to invd. Lane r (of each 16-lane row of the wave) holds
// row r of the tile in registers; the pivot and the column entries the
// rank-1 update needs are read from their owner lanes with readlane, so no
// column passes through LDS. Entries above the diagonal are updated with
// values that are never read.
__device__ inline void factor16(double* T, double* invd, int lane, bool& bad) {
  const int r = lane & 15;
  double a[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = T[k * PT + r];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    double d = readlane_f64(a[j], j);
    if (!(d > 0.0) || !isfinite(d)) {
      bad = true;
      d = 1.0;
    }
    const double inv = rsqrt_f64(d);
    const double ljj = d * inv;
    a[j] = r > j ? a[j] * inv : (r == j ? ljj : a[j]);
    if (lane == 0) invd[j] = inv;
#pragma unroll
    for (int k = j + 1; k < 16; ++k) a[k] -= a[j] * row_bcast_i(a[j], k);
  }
  if (lane < 16) {
#pragma unroll
    for (int k = 0; k < 16; ++k) T[k * PT + r] = a[k];
  }
}

// One wave: X = L^-1 for the lower 16x16 tile L (column-major, pitch PT;
// rinv = 1/diag L), written to global memory column-major with pitch 16
// (zeros above the diagonal). Lane c solves column c by forward
// substitution; the entries of L it needs are DPP row broadcasts from a
// copy of L held one row per lane.
__device__ inline void inverse16(const double* L, const double* rinv, double* __restrict__ X,
                                 int lane) {
  const int c = lane & 15;
  double lr[16];  // row c of L
#pragma unroll
  for (int k = 0; k < 16; ++k) lr[k] = L[k * PT + c];
  double x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    double s0 = (i == c) ? 1.0 : 0.0, s1 = 0.0;
    // the broadcasts of row i wait for x[i-1]: otherwise all 120 of them are
    // hoisted to the top and held in registers at once
    const double dep = i > 0 ? x[i - 1] : 0.0;
#pragma unroll
    for (int k = 0; k < i; ++k) {
      const double lik = row_bcast_dep_i(lr[k], dep, i);
      if (k & 1)
        s1 = fma(-lik, x[k], s1);
      else
        s0 = fma(-lik, x[k], s0);
    }
    x[i] = (s0 + s1) * rinv[i];
  }
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) X[c * 16 + i] = x[i];
  }
}

// LDS of one diagonal-block factorization (doubles): the 36 tiles, the
// reciprocal diagonals, the per-wave hand-over buffers and a flag.
constexpr int POTRF_LDS = NPT * PTS + 8 * 16 + 4 * 16 + 1;

__device__ __forceinline__ void potrf_block(double* __restrict__ K, double* __restrict__ Dd, int64_t ld, int p,
                            unsigned* __restrict__ status, double* smem) {
  double* A = smem;
  double(*invd)[16] = reinterpret_cast<double(*)[16]>(smem + NPT * PTS);  // 1/diag, 8 tiles
  int& bad_any = *reinterpret_cast<int*>(smem + NPT * PTS + 192);
  double* D = Dd + (int64_t)p * 8 * 256;  // inverted 16x16 diagonal tiles, pitch 16
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t c0 = (int64_t)p * GT;
  if (t == 0) bad_any = 0;
  // Tile-ordered transfers: thread t always handles element (t >> 4, t & 15)
  // of a 16x16 tile, so the LDS offset is fixed and the global address moves
  // by whole tiles; all 36 loads are in flight together.
  const int er = t >> 4, ec = t & 15;
  const int lds_off = ec * PT + er;
  const double* gK = K + (c0 + er) * ld + c0 + ec;
  // four batches of 9 tiles in flight: few enough registers that this block
  // can share a kernel with the fp64 MFMA tile update at two waves per SIMD
#pragma unroll
  for (int u0 = 0; u0 < NPT; u0 += 9) {
    double v[9];
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      const int I = tile_row(u0 + u), Kt = u0 + u - I * (I + 1) / 2;
      v[u] = gK[(int64_t)(16 * I) * ld + 16 * Kt];
    }
#pragma unroll
    for (int u = 0; u < 9; ++u) A[(u0 + u) * PTS + lds_off] = v[u];
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // One 16x16 trailing-tile update C -= L_Is L_Ks^T (one wave, fp64 MFMA).
  auto syrk_tile = [&](int I, int Kc, int s) {
    double* C = A + ptile(I, Kc);
    const double* Li = A + ptile(I, s);
    const double* Lk = A + ptile(Kc, s);
    d4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = C[(lane & 15) * PT + (lane >> 4) + 4 * r];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int q = (lane >> 4) + 4 * kk;
      const double av = -Li[q * PT + (lane & 15)];
      const double bv = Lk[q * PT + (lane & 15)];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) C[(lane & 15) * PT + (lane >> 4) + 4 * r] = acc[r];
  };
  // Two independent tile updates with their MFMA chains interleaved (the
  // second is skipped when `two` is false).
  auto syrk_tile2 = [&](int I1, int K1, int I2, int K2, int s, bool two) {
    double* C1 = A + ptile(I1, K1);
    double* C2 = A + ptile(I2, K2);
    const double* L1i = A + ptile(I1, s);
    const double* L1k = A + ptile(K1, s);
    const double* L2i = A + ptile(I2, s);
    const double* L2k = A + ptile(K2, s);
    const int off = (lane & 15) * PT + (lane >> 4);
    d4 a1, a2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a1[r] = C1[off + 4 * r];
      a2[r] = C2[off + 4 * r];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int q = (lane >> 4) + 4 * kk;
      const double x1 = -L1i[q * PT + (lane & 15)], y1 = L1k[q * PT + (lane & 15)];
      const double x2 = -L2i[q * PT + (lane & 15)], y2 = L2k[q * PT + (lane & 15)];
      a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(x1, y1, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f64_16x16x4f64(x2, y2, a2, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) C1[off + 4 * r] = a1[r];
    if (two) {
#pragma unroll
      for (int r = 0; r < 4; ++r) C2[off + 4 * r] = a2[r];
    }
  };
  auto tile_of = [](int u, int& a, int& b) {
    a = 0;
    while ((a + 1) * (a + 2) / 2 <= u) ++a;
    b = u - a * (a + 1) / 2;
  };

  // Pipelined 16-wide steps: while wave 0 updates and factors the next
  // diagonal tile, waves 1-3 update the other trailing tiles two at a time.
  // The eight 16x16 diagonal inverses are formed at the end (their tiles are
  // final once factored, and only the next launch reads them).
  bool bad = false;
  if (wave == 0) factor16(A + ptile(0, 0), invd[0], lane, bad);
  __syncthreads();
#pragma unroll 1
  for (int s = 0; s < 8; ++s) {
    // rows below the diagonal tile: x L_ss^T = a  (forward substitution)
    if (t >= 16 * (s + 1) && t < GT) {
      double* T = A + ptile(t >> 4, s);
      const double* Ls = A + ptile(s, s);
      const int ri = t & 15;
      double x[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) x[c] = T[c * PT + ri];
      // column c of L_ss and its reciprocal diagonal are read one column
      // ahead, so no LDS latency sits in the dependent chain (a scheduling
      // barrier per column keeps all 120 entries from being hoisted into
      // registers)
      double lc[16], ln[16];
      double dc = invd[s][0], dn = 0.0;
#pragma unroll
      for (int m = 1; m < 16; ++m) lc[m] = Ls[m];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 1 < 16) {
#pragma unroll
          for (int m = c + 2; m < 16; ++m) ln[m] = Ls[(c + 1) * PT + m];
          dn = invd[s][c + 1];
        }
        x[c] *= dc;
#pragma unroll
        for (int m = c + 1; m < 16; ++m) x[m] -= x[c] * lc[m];
#pragma unroll
        for (int m = c + 2; m < 16; ++m) lc[m] = ln[m];
        dc = dn;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) T[c * PT + ri] = x[c];
    }
    __syncthreads();
    if (s == 7) break;
    // trailing tiles (I, Kc), s < Kc <= I < 8; u = 0 is (s+1, s+1)
    if (wave == 0) {
      syrk_tile(s + 1, s + 1, s);
      wave_lds_sync();
      factor16(A + ptile(s + 1, s + 1), invd[s + 1], lane, bad);
    } else {
      const int m = 7 - s;
      const int cnt = m * (m + 1) / 2;  // u = 0 is (s+1, s+1), done by wave 0
      for (int u = wave; u < cnt; u += 6) {
        const bool two = u + 3 < cnt;
        int a1, b1, a2, b2;
        tile_of(u, a1, b1);
        tile_of(two ? u + 3 : u, a2, b2);
        syrk_tile2(s + 1 + a1, s + 1 + b1, s + 1 + a2, s + 1 + b2, s, two);
      }
    }
    __syncthreads();
  }
  if (bad) atomicOr(&bad_any, 1);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    inverse16(A + ptile(wave + 4 * i, wave + 4 * i), invd[wave + 4 * i], D + (wave + 4 * i) * 256,
              lane);
  __syncthreads();

  // L11 back into K (lower tiles); the diagonal inverses went to Dd directly.
  double* gL = K + (c0 + er) * ld + c0 + ec;
  for (int I = 0; I < 8; ++I) {
#pragma unroll
    for (int Kt = 0; Kt < 8; ++Kt)
      if (Kt <= I) gL[(int64_t)(16 * I) * ld + 16 * Kt] = A[(I * (I + 1) / 2 + Kt) * PTS + lds_off];
  }
  if (t == 0 && bad_any) atomicOr(status, ST_NOTSPD);
}

// L21 = A21 L11^-T for one 64-row block below panel p (in place), by
// 16-column blocks: with Y_s = (L21[:, s])^T,
//     Y_s = D_s (A21[:, s]^T - sum_{s'<s} L11[s][s'] Y_s'),   D_s = L11[s][s]^-1,
// so only the lower 16x16 tiles of L11 and the diagonal inverses are needed.
// Each wave owns 16 rows; the Y tiles stay in registers in the MFMA
// accumulator layout, which is also the B-operand layout of the next
// products. The sum over s' is kept in four partial accumulators (one per
// 4-wide K step of the 16x16x4 products) so the dependent chain of each step
// is s MFMAs long instead of 4s.
//
// Workgroups from 2 * mt on (when the inverse X = L^-1 is accumulated beside
// the factorization, as Z = X^T) solve 64 rows each of Z's column block p in
// place: that block holds B^T with B_j = T_pj = -sum_{k<p} L_pk X_kj for
// j < p and B_p = I, and X_pj = L_pp^-1 B_j, so each row of it is the same
// length-128 forward substitution as a row of A21.
__global__ __launch_bounds__(256) void chol_trsm_kernel(double* __restrict__ K,
                                                        const double* __restrict__ Dd,
                                                        double* __restrict__ Z, int64_t ld,
                                                        int p, int mt) {
  __shared__ double Ls[NPT * PTS];
  __shared__ double Ds[8 * PTS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t c0 = (int64_t)p * GT;
  const int64_t r0 = c0 + GT + (int64_t)blockIdx.x * 64;
  {
    const int er = t >> 4, ec = t & 15;
    const double* gK = K + (c0 + er) * ld + c0 + ec;
    double v[NPT];
#pragma unroll
    for (int I = 0; I < 8; ++I)
#pragma unroll
      for (int Kt = 0; Kt <= I; ++Kt) v[I * (I + 1) / 2 + Kt] = gK[(int64_t)(16 * I) * ld + 16 * Kt];
#pragma unroll
    for (int u = 0; u < NPT; ++u) Ls[u * PTS + ec * PT + er] = v[u];
    const double* D = Dd + (int64_t)p * 8 * 256;
#pragma unroll
    for (int i = 0; i < 8; ++i) Ds[i * PTS + ec * PT + er] = D[i * 256 + ec * 16 + er];
  }
  // this wave's 16 rows, transposed into Y tiles: y[s][r] = A21[row][col] with
  // row = 16*wave + (lane & 15), col = 16*s + (lane >> 4) + 4*r; for the
  // inverse, the same with the rows of Z's column block p in place of A21
  const bool xpart = (int)blockIdx.x >= 2 * mt;
  const int64_t row = xpart ? ((int64_t)blockIdx.x - 2 * mt) * 64 + 16 * wave + (lane & 15)
                            : r0 + 16 * wave + (lane & 15);
  double* gA = (xpart ? Z : K) + row * ld + c0 + (lane >> 4);
  const int ident = xpart && row >= c0 ? (int)(row - c0) : -1;  // identity row of B^T
  d4 y[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = 16 * s + (lane >> 4) + 4 * r;
      const double v = gA[16 * s + 4 * r];
      y[s][r] = ident < 0 ? v : (k == ident ? 1.0 : 0.0);
    }
  __syncthreads();
  // The LDS operands of step s+1 (its L11 tiles, negated, and D_s+1) are
  // read while step s multiplies, so no product waits for an LDS read.
  double ops[2][36];
  auto load_ops = [&](int s, double (&o)[36]) {
#pragma unroll
    for (int sp = 0; sp < 7; ++sp)
      if (sp < s) {
        const double* Lt = Ls + ptile(s, sp);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) o[4 * sp + kk] = -Lt[((lane >> 4) + 4 * kk) * PT + (lane & 15)];
      }
    const double* Dt = Ds + s * PTS;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o[32 + kk] = Dt[((lane >> 4) + 4 * kk) * PT + (lane & 15)];
  };
  load_ops(0, ops[0]);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) load_ops(s + 1, ops[(s + 1) & 1]);
    // keeps the reads above this step's products (the scheduler would sink
    // each one next to its use)
    __builtin_amdgcn_sched_barrier(0);
    const double(&o)[36] = ops[s & 1];
    d4 part[4];
    part[0] = y[s];
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) part[kk] = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int sp = 0; sp < s; ++sp)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        part[kk] = __builtin_amdgcn_mfma_f64_16x16x4f64(o[4 * sp + kk], y[sp][kk], part[kk], 0, 0, 0);
    const d4 acc = (part[0] + part[1]) + (part[2] + part[3]);
    d4 out = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      out = __builtin_amdgcn_mfma_f64_16x16x4f64(o[32 + kk], acc[kk], out, 0, 0, 0);
    y[s] = out;
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) gA[16 * s + 4 * r] = y[s][r];
}

// X_pp = L_pp^-1 for every 128x128 diagonal block (one workgroup per block,
// all blocks at once) from its lower 16x16 tiles and the eight 16x16
// diagonal inverses: off-diagonal tiles by distance from the diagonal,
//     X_ij = -X_ii * sum_{k=j}^{i-1} L_ik X_kj.
// Written to the diagonal block of Xb with zero tiles above.
__global__ __launch_bounds__(256) void trtri_diag_kernel(const double* __restrict__ K,
                                                         const double* __restrict__ Dd,
                                                         double* __restrict__ Xb, int64_t ld) {
  __shared__ double A[NPT * PTS];
  __shared__ double X[NPT * PTS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int p = blockIdx.x;
  const int64_t c0 = (int64_t)p * GT;
  const int er = t >> 4, ec = t & 15;
  const int lds_off = ec * PT + er;
  {
    const double* gK = K + (c0 + er) * ld + c0 + ec;
    double v[NPT];
#pragma unroll
    for (int I = 0; I < 8; ++I)
#pragma unroll
      for (int Kt = 0; Kt <= I; ++Kt) v[I * (I + 1) / 2 + Kt] = gK[(int64_t)(16 * I) * ld + 16 * Kt];
#pragma unroll
    for (int u = 0; u < NPT; ++u) A[u * PTS + lds_off] = v[u];
    const double* D = Dd + (int64_t)p * 8 * 256;
#pragma unroll
    for (int i = 0; i < 8; ++i) X[ptile(i, i) + lds_off] = D[i * 256 + ec * 16 + er];
  }
  __syncthreads();
  for (int d = 1; d < 8; ++d) {
    for (int i = d + wave; i < 8; i += 4) {
      const int j = i - d;
      d4 acc = d4{0.0, 0.0, 0.0, 0.0};
      for (int k = j; k < i; ++k) {
        const double* Lik = A + ptile(i, k);
        const double* Xkj = X + ptile(k, j);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int q = (lane >> 4) + 4 * kk;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(Lik[q * PT + (lane & 15)],
                                                     Xkj[(lane & 15) * PT + q], acc, 0, 0, 0);
        }
      }
      const double* Xii = X + ptile(i, i);
      d4 out = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int q = (lane >> 4) + 4 * kk;
        out = __builtin_amdgcn_mfma_f64_16x16x4f64(Xii[q * PT + (lane & 15)], acc[kk], out, 0, 0, 0);
      }
      double* Xij = X + ptile(i, j);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xij[(lane & 15) * PT + (lane >> 4) + 4 * r] = -out[r];
    }
    __syncthreads();
  }
  double* gX = Xb + (c0 + er) * ld + c0 + ec;
  for (int I = 0; I < 8; ++I) {
#pragma unroll
    for (int Kt = 0; Kt < 8; ++Kt)
      gX[(int64_t)(16 * I) * ld + 16 * Kt] =
          Kt <= I ? X[(I * (I + 1) / 2 + Kt) * PTS + lds_off] : 0.0;
  }
}

// C -= A B^T for one 128x128 tile (fp64 MFMA, K = 128): A and B are 128x128
// blocks with K along their rows (leading dimension ld), C starts from its
// first `crows` rows (the others from 0). The first operand is negated as it
// is staged, so the epilogue is a plain store. Every tile update of the
// factorization and of the fused inverse goes through this one call site
// per kernel (a second loop form in a kernel costs registers and copies).
// `smem` holds >= 4 * GCH doubles.
__device__ __forceinline__ void tile_nt_update(const double* A, const double* B, double* C,
                                               int64_t ld, int crows, int kch, double* smem) {
  LdTrans64T<true> la{A, ld, {}};
  LdTrans64 lb{B, ld, {}};
  d4 acc[4][4];
  acc_load_lds(acc, C, ld, crows, GT, smem);
  gemm64_loop(la, lb, kch, smem, smem + 2 * GCH, acc);
  for_each_acc(acc, [&](int r, int c, double v) { C[r * ld + c] = v; });
}

// Tile `id` of the rest of the trailing update of panel p, C -= L_a L_b^T
// over the tiles a >= b >= 1 of the trailing triangle (mt tile rows, in
// trailing-tile coordinates; b = 0 is the next panel's column): first the
// column b = 1 (a = 1 .. mt-1), which the next column update reads, then the
// tiles a >= b >= 2 row by row. With kp = 2 the tile takes panels p - 1 and
// p at once (K = 256: the two panels' columns are adjacent; the products
// enter the accumulators in the same order as two separate updates, so the
// result is the same). Sets the operands of tile_nt_update.
__device__ inline void syrk_tile_args(double* K, int64_t ld, int p, int mt, int id, int kp,
                                      const double*& A, const double*& B, double*& C) {
  int a, b;
  if (id < mt - 1) {
    a = 1 + id;
    b = 1;
  } else {
    const int i2 = id - (mt - 1);
    a = (int)((sqrt(8.0 * i2 + 1.0) - 1.0) * 0.5);
    while (a * (a + 1) / 2 > i2) --a;
    while ((a + 1) * (a + 2) / 2 <= i2) ++a;
    b = i2 - a * (a + 1) / 2;
    a += 2;
    b += 2;
  }
  const int64_t c0 = (int64_t)p * GT, c1 = c0 + GT;
  const int64_t ra = c1 + (int64_t)a * GT, rb = c1 + (int64_t)b * GT;
  const int64_t k0 = c0 - (int64_t)(kp - 1) * GT;
  A = K + ra * ld + k0;
  B = K + rb * ld + k0;
  C = K + ra * ld + rb;
}

// One tile of panel p's step of the inverse accumulated beside the
// factorization, which keeps Z = X^T (upper triangular) for X = L^-1. X is
// built by block rows: once row block p of X is final,
//     T_rj -= L_rp X_pj   for every tile row r > p and column j <= p,
// which leaves T_rj = -sum_{k=j}^{r-1} L_rk X_kj by the time row r is solved
// (X_rj = L_rr^-1 T_rj). Transposed, the update is Z_jr -= Z_jp L_rp^T, the
// same product form as the factorization's trailing update. Tile `id` is
// (r, j) = (p + 1 + id / (p + 1), id % (p + 1)), so the tiles of tile row
// p + 1, which the next panel solve reads, come first; at j = p the tile is
// first written and starts from 0. Sets the operands of tile_nt_update.
__device__ inline void xinv_tile_args(double* K, double* Z, int64_t ld, int p, int id,
                                      const double*& A, const double*& B, double*& C,
                                      int& crows) {
  const int r = p + 1 + id / (p + 1), j = id % (p + 1);
  const int64_t rr = (int64_t)r * GT, cp = (int64_t)p * GT, cj = (int64_t)j * GT;
  A = Z + cj * ld + cp;  // Z_jp
  B = K + rr * ld + cp;  // L_rp
  C = Z + cj * ld + rr;  // Z_jr
  crows = j == p ? 0 : GT;
}

// Background tile `id`: the first nsyrk ids are the trailing-update tiles
// s0, s0 + 1, ... of panel ps (mts trailing tile rows; kps panels ending at
// ps), the others the inverse tiles x0, x0 + 1, ... of panel px's step.
__device__ __forceinline__ void bg_tile(double* K, double* Z, int64_t ld, int ps, int mts, int s0,
                                        int nsyrk, int kps, int px, int x0, int id,
                                        double* smem) {
  const double *A, *B;
  double* C;
  int crows = GT, kch = GT / GK;
  if (id < nsyrk) {
    syrk_tile_args(K, ld, ps, mts, s0 + id, kps, A, B, C);
    kch *= kps;
  } else {
    xinv_tile_args(K, Z, ld, px, x0 + id - nsyrk, A, B, C, crows);
  }
  tile_nt_update(A, B, C, ld, crows, kch, smem);
}

// The next panel's tile column, C(a, p+1) -= L(a, p) L(p+1, p)^T for every
// tile row a below panel p, at a finer grain than the background tiles because
// this update is on the critical path of the factorization: one workgroup
// per 64x64 quadrant (4 per tile), each wave a 32x32 block as 2x2 fp64 MFMA
// tiles. The operands are read from global memory (they are hot in L2)
// straight into the MFMA layout, 8 K-steps (32 columns) at a time, double
// buffered; the accumulators start from C and the row operand is negated.
// A[m][k] = L[row m][c0 + k], B[k][n] = L[col n][c0 + k]: lane l reads row
// (l & 15) of its 16-row group at K offset l >> 4.
//
// Workgroups from 4 * mt on are background tiles, one each: the trailing-
// update tiles s0 .. s0 + nsyrk - 1 of panel p-1 that did not fit beside
// the factor of panel p (none in panel p's column, which this launch
// updates), then the first inverse tiles of panel p's step.
__global__ __launch_bounds__(256, 2) void chol_col_kernel(double* __restrict__ K,
                                                          double* __restrict__ Z, int64_t ld,
                                                          int p, int mt, int s0, int nsyrk,
                                                          int kps) {
  if ((int)blockIdx.x >= 4 * mt) {
    __shared__ double smem[4 * GCH];
    const int nx = (int)gridDim.x - 4 * mt;
    bg_tile(K, Z, ld, p - 1, mt + 1, s0, nsyrk, kps, p, 0,
            xcd_remap((int)blockIdx.x - 4 * mt, nx), smem);
    return;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int tile = blockIdx.x >> 2, quad = blockIdx.x & 3;
  const int64_t c0 = (int64_t)p * GT, c1 = c0 + GT;
  const int64_t row0 = c1 + (int64_t)tile * GT + (quad >> 1) * 64 + (w >> 1) * 32;
  const int64_t col0 = c1 + (quad & 1) * 64 + (w & 1) * 32;
  const double* ar = K + (row0 + (lane & 15)) * ld + c0 + (lane >> 4);
  const double* br = K + (col0 + (lane & 15)) * ld + c0 + (lane >> 4);
  d4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][j][r] = K[(row0 + i * 16 + (lane >> 4) + 4 * r) * ld + col0 + j * 16 + (lane & 15)];
  double a[2][2][8], b[2][2][8];  // [buffer][16-row group][K-step]
  auto load = [&](int buf, int kb) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        a[buf][g][s] = -ar[(int64_t)(g * 16) * ld + kb * 32 + 4 * s];
        b[buf][g][s] = br[(int64_t)(g * 16) * ld + kb * 32 + 4 * s];
      }
  };
  load(0, 0);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < 4) load(cur ^ 1, kb + 1);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[cur][i][s], b[cur][j][s], acc[i][j], 0,
                                                           0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        K[(row0 + i * 16 + (lane >> 4) + 4 * r) * ld + col0 + j * 16 + (lane & 15)] = acc[i][j][r];
}

// The diagonal block of panel p alone.
__global__ __launch_bounds__(256) void chol_potrf_kernel(double* __restrict__ K,
                                                         double* __restrict__ Dd, int64_t ld, int p,
                                                         unsigned* __restrict__ status) {
  __shared__ double smem[POTRF_LDS];
  potrf_block(K, Dd, ld, p, status, smem);
}

// Workgroup 0 factors the diagonal block of panel q (its tile column is
// already updated); the others are background tiles: the first nsyrk tiles
// of the rest of panel q-1's trailing update (which touches no tile of panel
// q's column), then inverse tiles x0, x0 + 1, ... of panel q-1's step. One
// launch for independent pieces of work, so the factor of the next panel
// runs beside the update instead of after it. The factor's registers allow
// this kernel two waves per SIMD only with a few of the factor's values
// spilled to scratch; one round of the GPU then holds about 2 x 255 tiles
// beside the factor (CHOL_MERGE_TILES). Trailing-update tiles beyond that
// round, other than those of the next column, run beside the next column
// update.
constexpr int CHOL_MERGE_TILES = 504;
constexpr int STEP_LDS = POTRF_LDS > 4 * GCH ? POTRF_LDS : 4 * GCH;
__global__ __launch_bounds__(256, 2) void chol_potrf_syrk_kernel(double* __restrict__ K,
                                                              double* __restrict__ Dd,
                                                              double* __restrict__ Z, int64_t ld,
                                                              int q, int mts,
                                                              unsigned* __restrict__ status,
                                                              int nsyrk, int x0, int kps) {
  __shared__ double smem[STEP_LDS];
  if (blockIdx.x == 0)
    potrf_block(K, Dd, ld, q, status, smem);
  else
    bg_tile(K, Z, ld, q - 1, mts, 0, nsyrk, kps, q - 1, x0,
            xcd_remap(blockIdx.x - 1, gridDim.x - 1), smem);
}

// ---------------------------------------------------------------- inverse
//
// X = L^-1 by recursive doubling over the 128-tile grid. At level h (a power
// of two) the tile range is cut into blocks of 2h tiles; in every block the
// inverses X11 (first h tiles) and X22 (the rest) are complete, and
//     X21 = -X22 * (L21 * X11)
// finishes the block. All blocks of a level are independent: one launch for
// T = L21 X11 and one for X21 = -X22 T, with the triangular zeros of X11 and
// X22 skipped in the K ranges.

// The tile products of a doubling level may be cut along their inner sum
// into pieces of `ks` tiles: workgroup id covers piece id % np of tile
// id / np and, with Part, writes its partial 128x128 tile to
// Part + id * GT * GT; trtri_sum_kernel then adds the pieces of every tile in
// piece order. With np == 1 and ks >= h a workgroup computes its whole tile
// and writes it in place. Splitting bounds the serial length of a level at
// ks tiles when the level has too few tiles to fill the GPU.
__global__ __launch_bounds__(256) void trtri_t_kernel(const double* __restrict__ K,
                                                      const double* __restrict__ Xb,
                                                      double* __restrict__ Tb,
                                                      double* __restrict__ Part, int64_t ld, int h,
                                                      int nt, int np, int ks) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int tile = blockIdx.x / np, piece = blockIdx.x % np;
  int r, c;
  int64_t f0, s0;
  level_tile_t(tile, h, nt, r, c, f0, s0);
  // T[r][c] = sum_{k=c}^{h-1} L[s0+r][f0+k] X[f0+k][f0+c]
  const int k0 = c + piece * ks;
  const int k1 = k0 + ks < h ? k0 + ks : h;
  if (k0 >= k1) return;
  LdTrans64 la{K + (s0 + r) * GT * ld + (f0 + k0) * GT, ld, {}};
  LdDirect64 lb{Xb + (f0 + k0) * GT * ld + (f0 + c) * GT, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, (k1 - k0) * (GT / GK), sA, sB, acc);
  if (Part) {
    double* out = Part + (int64_t)blockIdx.x * GT * GT;
    for_each_acc(acc, [&](int rr, int cc, double v) { out[rr * GT + cc] = v; });
  } else {
    double* out = Tb + (s0 + r) * GT * ld + (f0 + c) * GT;
    for_each_acc(acc, [&](int rr, int cc, double v) { out[rr * ld + cc] = v; });
  }
}

__global__ __launch_bounds__(256) void trtri_x_kernel(double* __restrict__ Xb,
                                                      const double* __restrict__ Tb,
                                                      double* __restrict__ Part, int64_t ld, int h,
                                                      int nt, int np, int ks) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int tile = blockIdx.x / np, piece = blockIdx.x % np;
  int r, c;
  int64_t f0, s0;
  level_tile_x(tile, h, nt, r, c, f0, s0);
  // X[s0+r][f0+c] = -sum_{k=0}^{r} X[s0+r][s0+k] T[s0+k][f0+c]
  const int k0 = piece * ks;
  const int k1 = k0 + ks < r + 1 ? k0 + ks : r + 1;
  if (k0 >= k1) return;
  // the X22 operand is negated as it is staged, so the result is stored as is
  LdTrans64T<true> la{Xb + (s0 + r) * GT * ld + (s0 + k0) * GT, ld, {}};
  LdDirect64 lb{Tb + (s0 + k0) * GT * ld + (f0 + c) * GT, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, (k1 - k0) * (GT / GK), sA, sB, acc);
  if (Part) {
    double* out = Part + (int64_t)blockIdx.x * GT * GT;
    for_each_acc(acc, [&](int rr, int cc, double v) { out[rr * GT + cc] = v; });
  } else {
    double* out = Xb + (s0 + r) * GT * ld + (f0 + c) * GT;
    for_each_acc(acc, [&](int rr, int cc, double v) { out[rr * ld + cc] = v; });
  }
}

// Sum of the pieces of every tile of a split level, in piece order, into T
// (xk false) or X (xk true). Eight workgroups per tile (16 rows each); each
// thread sums 4 pairs of adjacent elements, loading up to 8 pieces before
// adding them.
__global__ __launch_bounds__(256) void trtri_sum_kernel(const double* __restrict__ Part,
                                                        double* __restrict__ Dst, int64_t ld, int h,
                                                        int nt, int np, int ks, bool xk) {
  const int tile = blockIdx.x >> 3, band = blockIdx.x & 7;
  int r, c;
  int64_t f0, s0;
  if (xk)
    level_tile_x(tile, h, nt, r, c, f0, s0);
  else
    level_tile_t(tile, h, nt, r, c, f0, s0);
  const int len = xk ? r + 1 : h - c;
  const int cnt = (len + ks - 1) / ks;
  const double* src = Part + (int64_t)tile * np * GT * GT;
  double* dst = Dst + (s0 + r) * GT * ld + (f0 + c) * GT;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = band * 16 * GT + 2 * (u * 256 + threadIdx.x);  // even element of the tile
    dbl2 sum = {0.0, 0.0};
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      dbl2 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q < cnt ? j0 + q : j0;
        v[q] = *reinterpret_cast<const dbl2*>(src + (int64_t)j * GT * GT + e);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q < cnt) {
          sum.x += v[q].x;
          sum.y += v[q].y;
        }
    }
    *reinterpret_cast<dbl2*>(dst + (int64_t)(e >> 7) * ld + (e & 127)) = sum;
  }
}

// Pieces per tile at level h (1: the level is not split): split when the
// level has too few tiles to fill the GPU twice over and its longest inner
// sum is long (>= 16 tiles), within a bound on the partial-tile storage;
// shorter levels do not repay the extra pass over the partial tiles.
constexpr int TRTRI_KS = 4;
constexpr int TRTRI_MAX_PIECES = 4096;
static int trtri_pieces(int h, int nt, bool xk) {
  const int tiles = level_tiles(h, nt);
  const int last = level_last_rows(h, nt);
  const int maxk = xk ? (level_blocks(h, nt) > 1 ? h : (last > 0 ? last : 0)) : h;
  if (tiles >= 512 || maxk < 16) return 1;
  const int np = (maxk + TRTRI_KS - 1) / TRTRI_KS;
  return tiles * np <= TRTRI_MAX_PIECES ? np : 1;
}

static size_t trtri_part_bytes(int nt) {
  size_t mx = 0;
  for (int h = 1; h < nt; h *= 2)
    for (int xk = 0; xk < 2; ++xk) {
      const int np = trtri_pieces(h, nt, xk != 0);
      if (np > 1) mx = std::max(mx, (size_t)level_tiles(h, nt) * np * GT * GT * sizeof(double));
    }
  return mx;
}

// U[j][k] = X[n-1-j][n-1-k] (k >= j), 0 below the diagonal; fp32.
__global__ __launch_bounds__(256) void prep_uout_kernel(const double* __restrict__ Xb, int64_t ld,
                                                        int64_t n, float* __restrict__ U) {
  for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
    const double* xr = Xb + (n - 1 - j) * ld;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x)
      U[j * n + k] = k >= j ? (float)xr[n - 1 - k] : 0.0f;
  }
}

// The factor form, beyond the diagonal tiles: T_ab = L_ab X_bb for every
// tile a > b of K (X_bb = L_bb^-1 from trtri_diag_kernel), in place, one
// workgroup per tile. In sweep order (K front-padded: sweep index j is row
// ip-1-j of K) this is R[blk_a, blk_b] U[blk_b, blk_b] with R = J L J = U^-1
// the upper factor of H itself (H_p = R R^T); the sweep's residuals Q - W
// through it give E U (E = (W - Q) R and, U being upper, R[:j0, :j0]
// U[:j0, blk] = -R[:j0, blk] U[blk, blk]).
__global__ __launch_bounds__(256, 2) void prep_mfac_kernel(double* __restrict__ K,
                                                        const double* __restrict__ Xb,
                                                        int64_t ld) {
  __shared__ double smem[4 * GCH];
  const int id = (int)blockIdx.x;  // strict lower tiles, row-major: a > b
  int a = (int)((1.0 + sqrt(1.0 + 8.0 * id)) * 0.5);
  while (a * (a - 1) / 2 > id) --a;
  while ((a + 1) * a / 2 <= id) ++a;
  const int b = id - a * (a - 1) / 2;
  double* C = K + (int64_t)a * GT * ld + (int64_t)b * GT;
  // A[m][k] = L_ab (K along its rows, staged transposed); B[k][n] = X_bb
  LdTrans64 la{C, ld, {}};
  LdDirect64 lb{Xb + (int64_t)b * GT * ld + (int64_t)b * GT, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, GT / GK, smem, smem + 2 * GCH, acc);
  // every load of the tile has completed in the loop: overwrite it
  for_each_acc(acc, [&](int r, int c, double v) { C[r * ld + c] = v; });
}

// The factor-form matrix (K front-padded: sweep index j is row ip-1-j of K):
//   M[j][k] = U[j][k]  where j and k are in the same 128-block (U's diagonal
//             block: the inverse of the tile of L in Xb, reversed),
//   M[j][k] = T[ip-1-j][ip-1-k] = (R U)[j][k] over k's block  for k in a
//             later block (prep_mfac_kernel),
// 0 below the diagonal; fp32.
__global__ __launch_bounds__(256) void prep_mout_kernel(const double* __restrict__ K,
                                                        const double* __restrict__ Xb, int64_t ld,
                                                        int64_t n, float* __restrict__ M) {
  const int64_t ip = ld;
  for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int64_t a = ip - 1 - j;
    const double* kr = K + a * ld;
    const double* xr = Xb + a * ld;
    const int64_t blk_end = (j / GT + 1) * GT;  // first column of the next block
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x) {
      const int64_t b = ip - 1 - k;
      M[j * n + k] = k < j ? 0.0f : (float)(k < blk_end ? xr[b] : kr[b]);
    }
  }
}

// U[j][k] = Z[n-1-k][n-1-j] (k >= j), 0 below the diagonal; fp32. One 64x64
// tile of U per workgroup, staged through LDS so that the reads of Z and the
// writes of U both run along rows.
__global__ __launch_bounds__(256) void prep_uout_z_kernel(const double* __restrict__ Z,
                                                          int64_t ld, int64_t n,
                                                          float* __restrict__ U) {
  __shared__ double tile[64][65];
  const int64_t j0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const bool below = k0 + 63 < j0;  // the whole tile is below the diagonal
  if (!below) {
    for (int a = ty; a < 64; a += 4) {
      const int64_t k = k0 + a, j = j0 + tx;
      tile[a][tx] = (k < n && j < n) ? Z[(n - 1 - k) * ld + (n - 1 - j)] : 0.0;
    }
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t j = j0 + i, k = k0 + tx;
    if (j < n && k < n) U[j * n + k] = (!below && k >= j) ? (float)tile[tx][i] : 0.0f;
  }
}

__global__ void zero_u32_kernel(unsigned* p) { *p = 0u; }

// ---------------------------------------------------------------- min-pivot
//
// The min-pivot order (The Geometry of LLM Quantization 2.3): the LDL of H
// taking, at every step, the smallest diagonal of the current Schur
// complement as the next pivot, ties to the higher index; the sweep visits
// the columns in the reverse elimination order (perm[n-1-j] = j-th pivot).
// Computed like a blocked pivoted Cholesky, on A = H in the original order
// (lower triangle, in the factorization's K buffer): one launch per pivot,
// panels of 128 pivots, and after every full panel one launch of tile
// updates A -= P P^T over the whole lower triangle (rows of columns already
// eliminated hold zeros in P, so only live entries change). The order found
// is then factored again by the ordinary path; this search only decides it.
//
// Per pivot j (panel column k = j % 128), with d the Schur diagonal of the
// live columns (+inf once eliminated) and Pt = P^T [128 x ip]:
//   p = argmin d (from the previous launch's per-workgroup minima);
//   Pt[k][p] = sqrt(d_p);  for live i != p:
//   Pt[k][i] = (A[i][p] - sum_{k'<k} Pt[k'][i] Pt[k'][p]) / sqrt(d_p),
//   d_i -= Pt[k][i]^2;   eliminated i: Pt[k][i] = 0.
// Every workgroup reduces the previous minima itself (the same result in all
// of them, in a fixed order) and leaves the minimum of its own updated
// entries for the next launch.

struct MinIdx {
  double v;
  int i;
};

// (v, i) before (w, j): smaller value; equal values: the higher index
__device__ inline bool mp_before(double v, int i, double w, int j) {
  return v < w || (v == w && i > j);
}

// Minimum over the wave of (v, i), in every lane (butterfly of lane swaps).
__device__ inline MinIdx mp_wave_min(double v, int i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double w = __shfl_xor(v, off);
    const int j = __shfl_xor(i, off);
    if (mp_before(w, j, v, i)) {
      v = w;
      i = j;
    }
  }
  return MinIdx{v, i};
}

// Minimum over the block of (v, i) (256 threads); result in every thread.
template <int NW = 4>
__device__ inline MinIdx mp_block_min(double v, int i, double* sv, int* si) {
  const MinIdx m = mp_wave_min(v, i);
  const int t = threadIdx.x;
  if ((t & 63) == 0) {
    sv[t >> 6] = m.v;
    si[t >> 6] = m.i;
  }
  __syncthreads();
  MinIdx r{sv[0], si[0]};
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (mp_before(sv[w], si[w], r.v, r.i)) r = MinIdx{sv[w], si[w]};
  return r;
}

// d = diag A for the live columns, +inf for the pad; Pt = 0; minima (the
// second set "none", which a step that found no valid pivot leaves for the
// next); perm = identity, so that it holds valid indices whatever happens.
__global__ __launch_bounds__(256) void mp_init_kernel(const double* __restrict__ A, int64_t ld,
                                                      int64_t n, int64_t ip,
                                                      double* __restrict__ d,
                                                      double* __restrict__ Pt,
                                                      double* __restrict__ mv,
                                                      int* __restrict__ mi,
                                                      int32_t* __restrict__ perm) {
  __shared__ double sv[4];
  __shared__ int si[4];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double v = INFINITY;
  if (i < ip) {
    v = i < n ? A[i * ld + i] : INFINITY;
    d[i] = v;
    for (int k = 0; k < GT; ++k) Pt[(int64_t)k * ip + i] = 0.0;
  }
  if (i < n) perm[i] = (int32_t)i;
  const MinIdx m = mp_block_min(v, (int)i, sv, si);
  if (threadIdx.x == 0) {
    mv[blockIdx.x] = m.v;
    mi[blockIdx.x] = m.i;
    mv[gridDim.x + blockIdx.x] = INFINITY;
    mi[gridDim.x + blockIdx.x] = -1;
  }
}

// Pivot j (column k of its panel). mv_in/mi_in: the previous minima (nwg of
// them), mv_out/mi_out: this launch's.
__global__ __launch_bounds__(256) void mp_step_kernel(const double* __restrict__ A, int64_t ld,
                                                      int64_t n, int64_t ip,
                                                      double* __restrict__ d,
                                                      double* __restrict__ Pt, int j, int k,
                                                      const double* __restrict__ mv_in,
                                                      const int* __restrict__ mi_in,
                                                      double* __restrict__ mv_out,
                                                      int* __restrict__ mi_out,
                                                      int32_t* __restrict__ perm,
                                                      unsigned* __restrict__ status) {
  __shared__ double sv[4];
  __shared__ int si[4];
  // every wave reduces the previous minima itself (no barrier needed)
  const int nwg = gridDim.x, lane = threadIdx.x & 63;
  double bv = INFINITY;
  int bi = -1;
  for (int w = lane; w < nwg; w += 64)
    if (mp_before(mv_in[w], mi_in[w], bv, bi)) {
      bv = mv_in[w];
      bi = mi_in[w];
    }
  const MinIdx m = mp_wave_min(bv, bi);
  const double dp = m.v;
  const int p = __builtin_amdgcn_readfirstlane(m.i);
  if (!(dp > 0.0) || !isfinite(dp) || p < 0 || p >= n) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, ST_NOTSPD);
    return;  // U is garbage after a failed factorization anyway
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) perm[n - 1 - j] = p;
  // the pivot's panel row, once per workgroup
  __shared__ double prow[GT];
  if ((int)threadIdx.x < k) prow[threadIdx.x] = Pt[(int64_t)threadIdx.x * ip + p];
  __syncthreads();
  const double rs = 1.0 / sqrt(dp);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double v = INFINITY;
  if (i < n) {
    const double di = d[i];
    if (i == p) {
      Pt[(int64_t)k * ip + i] = dp * rs;
      d[i] = INFINITY;
    } else if (di == INFINITY) {
      Pt[(int64_t)k * ip + i] = 0.0;
    } else {
      double c = i > p ? A[i * ld + p] : A[(int64_t)p * ld + i];
      // the panel's earlier columns at row i, 16 loads in flight at a time
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      const double* pc = Pt + i;
      int kk = 0;
      for (; kk + 16 <= k; kk += 16) {
        double x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = pc[(int64_t)(kk + u) * ip];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u & 3] = fma(x[u], prow[kk + u], acc[u & 3]);
      }
      for (; kk < k; ++kk) acc[kk & 3] = fma(pc[(int64_t)kk * ip], prow[kk], acc[kk & 3]);
      c -= (acc[0] + acc[1]) + (acc[2] + acc[3]);
      const double l = c * rs;
      Pt[(int64_t)k * ip + i] = l;
      v = di - l * l;
      d[i] = v;
    }
  }
  const MinIdx mo = mp_block_min(v, (int)i, sv, si);
  if (threadIdx.x == 0) {
    mv_out[blockIdx.x] = mo.v;
    mi_out[blockIdx.x] = mo.i;
  }
}

// The pivots of one panel (up to 128) in one cooperative launch, for
// searches whose columns fit few workgroups: the same step as
// mp_step_kernel, with no launch between two pivots. Each workgroup owns
// MP_T columns and keeps their entries of the panel's Pt rows in LDS
// (128 x MP_T fp64), so the dot product of a step reads LDS; the entries
// also go to Pt in global memory for the tile update after the panel.
//
// What one workgroup tells the others travels in tagged 64-bit words: the
// tag j + 1 of step j in the upper half beside 32 bits of payload, each word
// written and read whole with agent-scope atomics (no fences), so a reader
// that sees the tag it waits for sees that step's payload.
//  - slot: the minimum of the workgroup's columns after step j (value low
//    and high words, column index): three words.
//  - candidate: the Pt entries, rows 0..k, of that minimum's column (low
//    and high word each), which are the pivot row of step j + 1 if that
//    column wins.
// Every wave of every workgroup polls all slots of step j - 1 (one lane per
// workgroup) until each holds the tag j, takes the minimum from what it
// read, then reads the winner's candidate (waiting for its tags too).
// Both tables have two halves, by the parity of j: half j & 1 is written
// again only at step j + 2, which needs every workgroup's slot of step j +
// 1, published after it read half j & 1. Every wait is bounded: a wave that
// gives up ends the search with ST_NOTSPD, and so does every wave that then
// waits for it.
constexpr int MP_T = 128;                 // columns per workgroup
constexpr long MP_SPIN = 1L << 20;        // polls before a wait gives up

__global__ void zero_u64_kernel(uint64_t* __restrict__ p, int count) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < count; k += gridDim.x * blockDim.x)
    p[k] = 0;
}

// Minimum over the wave of (v, i), the result uniform: lane moves inside
// quads and rows (DPP), a swizzle across the two row pairs of each half,
// then the two halves' results read from lanes 0 and 32. The order is a
// strict total one on distinct indices, so the result is the same as that of
// any other reduction order.
template <int CTRL>
__device__ inline void mp_dpp_step(double& v, int& i) {
  const double w = dpp_f64<CTRL>(v);
  const int j = __builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false);
  const bool b = mp_before(w, j, v, i);
  v = b ? w : v;
  i = b ? j : i;
}
__device__ inline MinIdx mp_wave_min_u(double v, int i) {
  mp_dpp_step<0xB1>(v, i);   // quad_perm [1,0,3,2]
  mp_dpp_step<0x4E>(v, i);   // quad_perm [2,3,0,1]
  mp_dpp_step<0x141>(v, i);  // row_half_mirror: the other quad of each 8 lanes
  mp_dpp_step<0x140>(v, i);  // row_mirror: the other 8 lanes of each row
  {
    // lane ^ 16 inside each 32 lanes (swizzle, bitmask mode)
    constexpr int SW = 0x1F | (0x10 << 10);
    const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), SW);
    const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), SW);
    const int j = __builtin_amdgcn_ds_swizzle(i, SW);
    const double w = __hiloint2double(hi, lo);
    const bool b = mp_before(w, j, v, i);
    v = b ? w : v;
    i = b ? j : i;
  }
  const double a = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 0),
                                    __builtin_amdgcn_readlane(__double2loint(v), 0));
  const int ai = __builtin_amdgcn_readlane(i, 0);
  const double c = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 32),
                                    __builtin_amdgcn_readlane(__double2loint(v), 32));
  const int ci = __builtin_amdgcn_readlane(i, 32);
  return mp_before(c, ci, a, ai) ? MinIdx{c, ci} : MinIdx{a, ai};
}

// A tagged word: the tag above 32 bits of payload.
__device__ inline uint64_t mp_word(unsigned tag, unsigned payload) {
  return ((uint64_t)tag << 32) | payload;
}
__device__ inline void mp_put(uint64_t* w, unsigned tag, unsigned payload) {
  __hip_atomic_store(w, mp_word(tag, payload), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t mp_get(const uint64_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool mp_tagged(uint64_t w, unsigned tag) { return (unsigned)(w >> 32) == tag; }

__global__ __launch_bounds__(MP_T) void mp_panel_kernel(const double* __restrict__ A, int64_t ld,
                                                        int64_t n, int64_t ip,
                                                        double* __restrict__ d,
                                                        double* __restrict__ Pt, int j0, int kn,
                                                        const double* __restrict__ mv0,
                                                        const int* __restrict__ mi0, int nprev,
                                                        uint64_t* __restrict__ slots,
                                                        uint64_t* __restrict__ cands,
                                                        int32_t* __restrict__ perm,
                                                        unsigned* __restrict__ status) {
  constexpr int NW = MP_T / 64;
  __shared__ double pts[GT][MP_T];  // this workgroup's entries of the panel's Pt rows
  __shared__ double prow[GT];
  __shared__ double sv[NW];
  __shared__ int si[NW];
  __shared__ int fail[NW];
  __shared__ unsigned st0;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int nwg = gridDim.x;
  // a failed step earlier on the stream: the order is garbage already, and
  // the slots of its last step may never have been written
  if (t == 0) st0 = *status;
  __syncthreads();
  if (st0 & ST_NOTSPD) return;
  const int64_t i = (int64_t)blockIdx.x * MP_T + t;
  double di = i < n ? d[i] : INFINITY;
  // j0 is the first column of a panel, so panel column k = j - j0
  for (int k = 0; k < kn; ++k) {
    const int j = j0 + k;
    // the minima of step j - 1: mp_init's (written before this launch) for
    // the first pivot, else the slots
    double bv = INFINITY;
    int bi = -1;
    bool ok = true;
    if (j == 0) {
      for (int w = lane; w < nprev; w += 64)
        if (mp_before(mv0[w], mi0[w], bv, bi)) {
          bv = mv0[w];
          bi = mi0[w];
        }
    } else if (lane < nwg) {
      const uint64_t* sl = slots + ((size_t)((j - 1) & 1) * nwg + lane) * 4;
      uint64_t w0, w1, w2;
      long spins = 0;
      for (;;) {
        w0 = mp_get(sl);
        w1 = mp_get(sl + 1);
        w2 = mp_get(sl + 2);
        if (mp_tagged(w0, j) && mp_tagged(w1, j) && mp_tagged(w2, j)) break;
        if (++spins > MP_SPIN) {
          ok = false;
          break;
        }
      }
      bv = __hiloint2double((int)(unsigned)w1, (int)(unsigned)w0);
      bi = (int)(unsigned)w2;
    }
    const MinIdx m = mp_wave_min_u(bv, bi);
    const double dp = m.v;
    const int p = m.i;
    bool good = __all(ok) && dp > 0.0 && isfinite(dp) && p >= 0 && p < n;
    // the pivot's entries of this panel's earlier rows (its workgroup's
    // candidate of step j - 1), and A's entry (i, p), loaded together from
    // addresses valid in every lane (what a lane does not need is unused)
    const int pc = good ? p : 0;
    const int64_t ic = i < n ? i : pc;
    double c = ic > pc ? A[ic * ld + pc] : A[(int64_t)pc * ld + ic];
    if (good && t < k) {
      const uint64_t* cw = cands + (((size_t)((j - 1) & 1) * nwg + pc / MP_T) * GT + t) * 2;
      uint64_t lo, hi;
      long spins = 0;
      for (;;) {
        lo = mp_get(cw);
        hi = mp_get(cw + 1);
        if (mp_tagged(lo, j) && mp_tagged(hi, j)) break;
        if (++spins > MP_SPIN) {
          good = false;
          break;
        }
      }
      prow[t] = __hiloint2double((int)(unsigned)hi, (int)(unsigned)lo);
    }
    good = __all(good);
    if (lane == 0) fail[wv] = !good;
    __syncthreads();
    bool stop = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) stop |= fail[w] != 0;
    if (stop) {
      if (t == 0) atomicOr(status, ST_NOTSPD);
      break;  // the same decision in every wave of the workgroup
    }
    if (blockIdx.x == 0 && t == 0) perm[n - 1 - j] = p;
    const double rs = 1.0 / sqrt(dp);
    double v = INFINITY;
    if (i < n) {
      double l;
      if (i == p) {
        l = dp * rs;
        di = INFINITY;
      } else if (di == INFINITY) {
        l = 0.0;
      } else {
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        for (int q = 0; q < k; ++q) acc[q & 3] = fma(pts[q][t], prow[q], acc[q & 3]);
        c -= (acc[0] + acc[1]) + (acc[2] + acc[3]);
        l = c * rs;
        di -= l * l;
        v = di;
      }
      pts[k][t] = l;
      Pt[(int64_t)k * ip + i] = l;
    }
    const MinIdx mw = mp_wave_min_u(v, (int)i);
    if (lane == 0) {
      sv[wv] = mw.v;
      si[wv] = mw.i;
    }
    __syncthreads();
    MinIdx r{sv[0], si[0]};
#pragma unroll
    for (int w = 1; w < NW; ++w)
      if (mp_before(sv[w], si[w], r.v, r.i)) r = MinIdx{sv[w], si[w]};
    const unsigned tag = (unsigned)j + 1;
    if (k + 1 < kn && t <= k) {
      // the candidate's column, rows 0..k (the next step of this launch
      // reads it; a launch starts at a panel's first row and reads none)
      const double x = pts[t][r.i - (int)blockIdx.x * MP_T];
      uint64_t* cw = cands + (((size_t)(j & 1) * nwg + blockIdx.x) * GT + t) * 2;
      mp_put(cw, tag, (unsigned)__double2loint(x));
      mp_put(cw + 1, tag, (unsigned)__double2hiint(x));
    }
    if (t == 0) {
      uint64_t* sl = slots + ((size_t)(j & 1) * nwg + blockIdx.x) * 4;
      mp_put(sl, tag, (unsigned)__double2loint(r.v));
      mp_put(sl + 1, tag, (unsigned)__double2hiint(r.v));
      mp_put(sl + 2, tag, (unsigned)r.i);
    }
  }
  if (i < n) d[i] = di;
}

// The panel launches serve searches up to this many workgroups (MP_T columns
// each): their barrier costs grow with the workgroup count, the per-pivot
// launches' cost does not.
constexpr int MP_PANEL_MAX_WG = 64;  // one polling lane per workgroup
constexpr int MP_SLOT_WORDS = 2 * MP_PANEL_MAX_WG * 4;
constexpr int MP_CAND_WORDS = 2 * MP_PANEL_MAX_WG * GT * 2;

// Whether nwg workgroups of mp_panel_kernel can all be resident at once on
// the current device (a cooperative launch needs that).
static bool mp_panel_fits(int nwg) {
  int dev = 0, coop = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
      !coop)
    return false;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)mp_panel_kernel, MP_T, 0) !=
      hipSuccess)
    return false;
  return (int64_t)per * ncu >= nwg;
}

// After a full panel: A -= P P^T on every lower tile (a, b) of the ip grid.
__global__ __launch_bounds__(256) void mp_update_kernel(double* __restrict__ A, int64_t ld,
                                                        int64_t ip,
                                                        const double* __restrict__ Pt) {
  __shared__ double smem[4 * GCH];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  int a = (int)((sqrt(8.0 * id + 1.0) - 1.0) * 0.5);
  while (a * (a + 1) / 2 > id) --a;
  while ((a + 1) * (a + 2) / 2 <= id) ++a;
  const int b = id - a * (a + 1) / 2;
  LdDirect64T<true> la{Pt + (int64_t)a * GT, ip, {}};  // -P rows of tile a, k-major
  LdDirect64 lb{Pt + (int64_t)b * GT, ip, {}};
  double* C = A + (int64_t)a * GT * ld + (int64_t)b * GT;
  d4 acc[4][4];
  acc_load_lds(acc, C, ld, GT, GT, smem);
  gemm64_loop(la, lb, GT / GK, smem, smem + 2 * GCH, acc);
  for_each_acc(acc, [&](int r, int c, double v) { C[r * ld + c] = v; });
}

// ---------------------------------------------------------------- layout

// Up to this many 128-column panels the inverse of L is accumulated by block
// rows inside the factorization's own launches (its tile updates run beside
// the next panel's column update, its row solves beside the panel solve),
// which removes the separate triangular inverse from the dependent chain
// while the factorization is latency-bound. Larger matrices use recursive
// doubling, whose long inner sums run the MFMA units more efficiently and
// read each tile once per level instead of once per panel.
constexpr int CHOL_FUSE_NT = 48;
// panels per trailing update without the fused inverse
constexpr int CHOL_GROUP = 4;

struct PrepLayout {
  int64_t n, ip, nt;
  size_t off_status, off_lam, off_hd, off_K, off_X, off_T, off_D, off_P;
  size_t off_md, off_mpt, off_mv, off_mi, off_mslot, off_mcand;  // min-pivot search
  size_t total;
};

static PrepLayout prep_layout(int64_t n) {
  PrepLayout L;
  L.n = n;
  L.ip = round_up(n, GT);
  L.nt = L.ip / GT;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = (size_t)round_up((int64_t)(o + bytes), 256);
    return at;
  };
  L.off_status = take(4);
  L.off_lam = take(8);
  L.off_hd = take(8 * (size_t)n);
  L.off_K = take(8 * (size_t)L.ip * L.ip);
  L.off_X = take(8 * (size_t)L.ip * L.ip);
  const bool fused = L.nt <= CHOL_FUSE_NT;
  L.off_T = take(L.nt > 1 && !fused ? 8 * (size_t)L.ip * L.ip : 8);
  L.off_D = take(8 * (size_t)L.nt * 8 * 256);
  L.off_P = take(fused ? 8 : std::max<size_t>(trtri_part_bytes((int)L.nt), 8));
  const int64_t nwg = cdiv(L.ip, 256);
  L.off_md = take(8 * (size_t)L.ip);
  L.off_mpt = take(8 * (size_t)GT * L.ip);
  L.off_mv = take(8 * 2 * (size_t)nwg);
  L.off_mi = take(4 * 2 * (size_t)nwg);
  L.off_mslot = take(MP_SLOT_WORDS * 8);
  L.off_mcand = take(MP_CAND_WORDS * 8);
  L.total = o;
  return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_prepare_workspace_bytes(int64_t in_features) {
  if (in_features <= 0) return 0;
  return prep_layout(in_features).total;
}

extern "C" gptq_status gptq_prepare_hinv(const double* S, int64_t in_features, int64_t n_tokens_total,
                                         double damp, uint32_t flags, int32_t* perm, float* U,
                                         void* ws, size_t ws_bytes, void* stream) {
  if (in_features < 0) return GPTQ_EINVAL;
  if (in_features == 0) return GPTQ_OK;
  if (!S || !perm || !U || n_tokens_total <= 0 || !(damp >= 0.0) || !std::isfinite(damp))
    return GPTQ_EINVAL;
  if (flags & ~(GPTQ_FLAG_ACT_ORDER | GPTQ_FLAG_MIN_PIVOT | GPTQ_FLAG_NO_SYNC |
                GPTQ_FLAG_FACTOR_FORM))
    return GPTQ_EINVAL;
  const bool fac = (flags & GPTQ_FLAG_FACTOR_FORM) != 0;
  if ((flags & GPTQ_FLAG_ACT_ORDER) && (flags & GPTQ_FLAG_MIN_PIVOT)) return GPTQ_EINVAL;
  if (in_features > (int64_t)1 << 20) return GPTQ_EINVAL;
  const PrepLayout L = prep_layout(in_features);
  if (!ws || ws_bytes < L.total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  unsigned* status = (unsigned*)(base + L.off_status);
  double* lam = (double*)(base + L.off_lam);
  double* hd = (double*)(base + L.off_hd);
  double* K = (double*)(base + L.off_K);
  double* Xb = (double*)(base + L.off_X);
  double* Tb = (double*)(base + L.off_T);
  double* Dd = (double*)(base + L.off_D);
  double* Pt = (double*)(base + L.off_P);
  const int64_t n = in_features, ip = L.ip;
  const int nt = (int)L.nt;
  const double c = 2.0 / (double)n_tokens_total;

  GPTQ_LAUNCH(K_FILL, st, zero_u32_kernel<<<1, 1, 0, st>>>(status));
  GPTQ_LAUNCH(K_PREP_DIAG, st, prep_diag_kernel<<<1, 1024, 0, st>>>(S, n, c, damp, hd, lam));
  const int gsplit = n >= GATHER_SPLIT_FROM ? 8 : 1, gthreads = gsplit > 1 ? 1024 : 256;
  if (flags & GPTQ_FLAG_MIN_PIVOT) {
    // the order from a pivoted factorization of H in the original order
    double* md = (double*)(base + L.off_md);
    double* Pt = (double*)(base + L.off_mpt);
    double* mv = (double*)(base + L.off_mv);
    int* mi = (int*)(base + L.off_mi);
    uint64_t* mslot = (uint64_t*)(base + L.off_mslot);
    uint64_t* mcand = (uint64_t*)(base + L.off_mcand);
    const int nwg = (int)cdiv(ip, 256);
    const int nwgp = (int)cdiv(ip, MP_T);
    const bool panel = nwgp <= MP_PANEL_MAX_WG && mp_panel_fits(nwgp);
    GPTQ_LAUNCH(K_PREP_GATHER, st,
                prep_gather_kernel<<<(unsigned)(ip * gsplit), gthreads, 0, st>>>(
                    S, n, ip, c, lam, nullptr, K, gsplit, 0));
    GPTQ_LAUNCH(K_MP_STEP, st,
                mp_init_kernel<<<nwg, 256, 0, st>>>(K, ip, n, ip, md, Pt, mv, mi, perm));
    if (panel) {  // no tag of an earlier call may match
      GPTQ_LAUNCH(K_FILL, st, zero_u64_kernel<<<1, 256, 0, st>>>(mslot, MP_SLOT_WORDS));
      GPTQ_LAUNCH(K_FILL, st, zero_u64_kernel<<<64, 256, 0, st>>>(mcand, MP_CAND_WORDS));
    }
    for (int64_t j0 = 0; j0 < n; j0 += GT) {
      const int kn = (int)std::min<int64_t>(GT, n - j0);
      if (panel) {
        // the first pivot reads the minima of mp_init (nwg of them), the
        // others the slots of the step before
        int j0i = (int)j0, nprev = nwg, knv = kn;
        int64_t ldv = ip, nv = n, ipv = ip;
        void* args[] = {&K, &ldv, &nv, &ipv, &md, &Pt, &j0i, &knv, &mv, &mi, &nprev,
                        &mslot, &mcand, &perm, &status};
        GPTQ_LAUNCH(K_MP_STEP, st,
                    GPTQ_HIP(hipLaunchCooperativeKernel((const void*)mp_panel_kernel,
                                                        dim3(nwgp), dim3(MP_T), args, 0, st)));
      } else {
        for (int64_t j = j0; j < j0 + kn; ++j) {
          const int k = (int)(j - j0), par = (int)(j & 1);
          GPTQ_LAUNCH(K_MP_STEP, st,
                      mp_step_kernel<<<nwg, 256, 0, st>>>(
                          K, ip, n, ip, md, Pt, (int)j, k, mv + par * nwg, mi + par * nwg,
                          mv + (1 - par) * nwg, mi + (1 - par) * nwg, perm, status));
        }
      }
      if (j0 + kn < n) {
        const int tiles = (int)(L.nt * (L.nt + 1) / 2);
        GPTQ_LAUNCH(K_MP_UPDATE, st, mp_update_kernel<<<tiles, 256, 0, st>>>(K, ip, ip, Pt));
      }
    }
  } else {
    GPTQ_LAUNCH(K_PREP_PERM, st,
                prep_perm_kernel<<<(unsigned)cdiv(n, 16), 256, 0, st>>>(
                    hd, n, (flags & GPTQ_FLAG_ACT_ORDER) != 0, perm));
  }
  GPTQ_LAUNCH(K_PREP_GATHER, st,
              prep_gather_kernel<<<(unsigned)(ip * gsplit), gthreads, 0, st>>>(
                  S, n, ip, c, lam, perm, K, gsplit, fac ? ip - n : 0));
  // Blocked Cholesky, one stream. Per panel p: solve the panel's column
  // (trsm), update the next panel's tile column, then one launch that
  // factors the next diagonal block beside the rest of the trailing update.
  // With the fused inverse, the panel solve also solves row block p of
  // X = L^-1, and the column update also applies panel p's step of X.
  // Background tiles of panel p (the rest of its trailing update, then its
  // step of the inverse, tile row p + 1 first) go beside the next diagonal
  // block up to CHOL_MERGE_TILES (always the trailing tiles of column p + 2,
  // which the next column update reads); the inverse tiles that do not fit
  // run beside panel p's column update (before the next panel solve, which
  // reads tile row p + 1), the trailing tiles that do not fit beside panel
  // p+1's column update (before panel p+1's own trailing tiles).
  // Without the fused inverse (large matrices, where these tiles are most of
  // the work), the trailing update goes CHOL_GROUP panels at a time: panel
  // p = g0 + r of a group starting at g0 updates only column p + 2, which
  // the next column update reads, with panels g0 .. p (K = 128 (r + 1));
  // the group's last panel applies all of them to the rest at once, so each
  // such tile is read and written once per group. (Column c gets the
  // group's panels up to c - 2 at panel c - 2, and the panels after that
  // from the column updates; a group cut short by the end leaves no tile.)
  // the factor form needs no inverse beyond the diagonal tiles
  const bool fused = !fac && nt <= CHOL_FUSE_NT;
  // grouped trailing updates pay off where the trailing tiles are most of the
  // work; up to CHOL_FUSE_NT panels (the factor form there) every panel
  // applies its own update, as the fused form does, minus the inverse tiles
  const int cgroup = nt <= CHOL_FUSE_NT ? 1 : CHOL_GROUP;
  int sov = 0, sov0 = 0;  // trailing tiles of the previous panel for this column update
  int kpo = 1;            // panels those tiles take
  GPTQ_LAUNCH(K_CHOL_POTRF, st, chol_potrf_kernel<<<1, 256, 0, st>>>(K, Dd, ip, 0, status));
  for (int p = 0; p + 1 < nt; ++p) {
    const int mt = nt - 1 - p;
    const int r = p % cgroup;
    const bool col_only = !fused && r < cgroup - 1;
    const int kp = fused ? 1 : r + 1;
    const int rest = col_only ? mt - 1 : (mt - 1) * mt / 2;
    const int xs = fused ? 2 * (p + 1) : 0;   // inverse row-solve workgroups
    const int xt = fused ? mt * (p + 1) : 0;  // inverse tile updates
    const int ns = std::min(rest, std::max(CHOL_MERGE_TILES, mt - 1));
    const int xstep = std::min(xt, std::max(0, CHOL_MERGE_TILES - ns));
    const int xcol = xt - xstep;
    GPTQ_LAUNCH(K_CHOL_TRSM, st,
                chol_trsm_kernel<<<2 * mt + xs, 256, 0, st>>>(K, Dd, Xb, ip, p, mt));
    GPTQ_LAUNCH(K_CHOL_COL, st,
                chol_col_kernel<<<4 * mt + sov + xcol, 256, 0, st>>>(K, Xb, ip, p, mt, sov0,
                                                                     sov, kpo));
    GPTQ_LAUNCH(K_CHOL_STEP, st,
                chol_potrf_syrk_kernel<<<1 + ns + xstep, 256, 0, st>>>(K, Dd, Xb, ip, p + 1, mt,
                                                                      status, ns, xcol, kp));
    sov = rest - ns;
    sov0 = ns;
    kpo = kp;
  }
  if (fused) {
    // the last block row of X
    GPTQ_LAUNCH(K_CHOL_TRSM, st,
                chol_trsm_kernel<<<2 * nt, 256, 0, st>>>(K, Dd, Xb, ip, nt - 1, 0));
  } else {
    GPTQ_LAUNCH(K_TRTRI_DIAG, st, trtri_diag_kernel<<<nt, 256, 0, st>>>(K, Dd, Xb, ip));
  }
  if (fac) {
    if (nt > 1)
      GPTQ_LAUNCH(K_PREP_UOUT, st,
                  prep_mfac_kernel<<<(unsigned)(nt * (nt - 1) / 2), 256, 0, st>>>(K, Xb, ip));
    dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)std::min<int64_t>(n, 65535));
    GPTQ_LAUNCH(K_PREP_UOUT, st, prep_mout_kernel<<<grid, 256, 0, st>>>(K, Xb, ip, n, U));
    if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
    return gptq_workspace_status(ws, stream);
  }
  for (int h = 1; h < nt && !fused; h *= 2) {
    const int tiles = level_tiles(h, nt);
    const int npt = trtri_pieces(h, nt, false), npx = trtri_pieces(h, nt, true);
    if (npt > 1) {
      GPTQ_LAUNCH(K_TRTRI_ROW, st,
                  trtri_t_kernel<<<tiles * npt, 256, 0, st>>>(K, Xb, Tb, Pt, ip, h, nt, npt,
                                                              TRTRI_KS));
      GPTQ_LAUNCH(K_TRTRI_SUM, st,
                  trtri_sum_kernel<<<8 * tiles, 256, 0, st>>>(Pt, Tb, ip, h, nt, npt, TRTRI_KS,
                                                              false));
    } else {
      GPTQ_LAUNCH(K_TRTRI_ROW, st,
                  trtri_t_kernel<<<tiles, 256, 0, st>>>(K, Xb, Tb, nullptr, ip, h, nt, 1, h));
    }
    if (npx > 1) {
      GPTQ_LAUNCH(K_TRTRI_UPDATE, st,
                  trtri_x_kernel<<<tiles * npx, 256, 0, st>>>(Xb, Tb, Pt, ip, h, nt, npx,
                                                              TRTRI_KS));
      GPTQ_LAUNCH(K_TRTRI_SUM, st,
                  trtri_sum_kernel<<<8 * tiles, 256, 0, st>>>(Pt, Xb, ip, h, nt, npx, TRTRI_KS,
                                                              true));
    } else {
      GPTQ_LAUNCH(K_TRTRI_UPDATE, st,
                  trtri_x_kernel<<<tiles, 256, 0, st>>>(Xb, Tb, nullptr, ip, h, nt, 1, h));
    }
  }
  if (fused) {
    dim3 grid((unsigned)cdiv(n, 64), (unsigned)cdiv(n, 64));
    GPTQ_LAUNCH(K_PREP_UOUT, st, prep_uout_z_kernel<<<grid, 256, 0, st>>>(Xb, ip, n, U));
  } else {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)std::min<int64_t>(n, 65535));
    GPTQ_LAUNCH(K_PREP_UOUT, st, prep_uout_kernel<<<grid, 256, 0, st>>>(Xb, ip, n, U));
  }
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  return gptq_workspace_status(ws, stream);
}
