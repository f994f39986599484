// CHMC frontend (CHMC article, "Methodik. Was ist CHMC", Schritt 1-3): the
// low-rank part of a layer in the norm weighted by the damped activation
// energies, and the residual quantized by the GPTQ sweep with one grid per
// group of output channels and column.
//
//   c_j = S_jj / n + 0.05 * mean(c),  W~ = W diag(sqrt c)
//   randomized subspace iteration (Halko, Martinsson and Tropp, "Finding
//   structure with randomness", 2011, Algorithm 4.4) with the caller's
//   Gaussian sketch Omega [i x r] and 5 power iterations:
//     Q = orth(W~ Omega); 5 times: Q = orth(W~ orth(W~^T Q))
//   Z = W~^T Q (= B^T for B = Q^T W~), Z^T Z = Uh diag(s^2) Uh^T (Jacobi),
//   A = fp16(Q Uh diag(s)) [o x r], B = fp16(diag(1/s) Uh^T Z^T diag(1/sqrt c))
//   R = W - A B, swept in the act-order (perm) with the factor U.
// orth() is CholeskyQR2 (Y^T Y = R^T R, Y R^-1, twice): the iteration depends
// only on the span of each iterate, so any orthonormal basis gives the same
// Q Uh up to the signs of its columns.
// Sizes are those of a layer with a small rank (r <= 64): the products with a
// long inner dimension run as wave dot products (W~ times a thin matrix) or
// one thread per column (W~^T times a thin matrix, the sum over rows split
// over workgroups), the short ones one wave per row; everything is fp64.
#include "common.h"

namespace gptq {

constexpr int CH_RMAX = 64;   // rank (sketch columns) at most
constexpr int CH_NITER = 5;   // power iterations (CHMC article, Schritt 1)
constexpr int CH_QB = 128;    // sweep block width
constexpr int CH_KS = 64;     // shortest K piece of the block update

__global__ void ch_zero_kernel(unsigned* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = 0u;
}

// perm must be a permutation of [0, cols): count each value, then any count
// other than 1 (or a value out of range) sets ST_BADPERM.
__global__ void ch_perm_count_kernel(const int32_t* __restrict__ perm, int64_t cols,
                                     unsigned* __restrict__ cnt, unsigned* __restrict__ status) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < cols;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t v = perm[e];
    if (v < 0 || v >= cols) atomicOr(status, ST_BADPERM);
    else atomicAdd(cnt + v, 1u);
  }
}
__global__ void ch_perm_check_kernel(const unsigned* __restrict__ cnt, int64_t cols,
                                     unsigned* __restrict__ status) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < cols;
       e += (int64_t)gridDim.x * blockDim.x)
    if (cnt[e] != 1u) atomicOr(status, ST_BADPERM);
}

// c_j = S_jj/n + 0.05 mean(S_kk/n), sc_j = sqrt(c_j). One workgroup.
__global__ __launch_bounds__(1024) void ch_energy_kernel(const double* __restrict__ S, int64_t i,
                                                         double inv_n, double* __restrict__ c,
                                                         double* __restrict__ sc,
                                                         unsigned* __restrict__ status) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < i; k += blockDim.x) {
    const double d = S[k * i + k] * inv_n;
    c[k] = d;
    s += d;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double lam = 0.05 * red[0] / (double)i;
  for (int64_t k = threadIdx.x; k < i; k += blockDim.x) {
    const double v = c[k] + lam;
    if (!(v > 0.0) || !isfinite(v)) atomicOr(status, ST_NONFINITE);
    c[k] = v;
    sc[k] = sqrt(v);
  }
}

// Wt[r][j] = W[r][j] * sc[j] (fp64, ld i); a NaN/Inf weight sets ST_NONFINITE.
__global__ void ch_scale_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t o,
                                int64_t i, const double* __restrict__ sc,
                                double* __restrict__ Wt, unsigned* __restrict__ status) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < o * i;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / i, j = e - r * i;
    const double v = f16_to_f64(W[r * ldw + j]);
    if (!isfinite(v)) atomicOr(status, ST_NONFINITE);
    Wt[e] = v * sc[j];
  }
}

// C [m x q] = A [m x k] (ld lda) B [k x q] (ld q): one wave per row of C,
// lane = column of C (q <= 64).
__global__ __launch_bounds__(256) void ch_gemm_nn(const double* __restrict__ A, int64_t lda,
                                                  const double* __restrict__ B, int64_t m,
                                                  int64_t k, int q, double* __restrict__ C) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= m || lane >= q) return;
  const double* a = A + row * lda;
  double acc = 0.0;
#pragma unroll 4
  for (int64_t kk = 0; kk < k; ++kk) acc = fma(a[kk], B[kk * q + lane], acc);
  C[row * q + lane] = acc;
}

// C [m x q] = A [m x k] (ld lda) B [k x q] (ld q) for a long k: one wave per
// row of C, the lanes across k (coalesced reads of the row of A), 8 columns
// of C per blockIdx.y (q0 = 8 y), each summed over the wave at the end.
__global__ __launch_bounds__(256) void ch_rowdot_kernel(const double* __restrict__ A,
                                                        int64_t lda,
                                                        const double* __restrict__ B, int64_t m,
                                                        int64_t k, int q,
                                                        double* __restrict__ C) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q0 = blockIdx.y * 8;
  if (row >= m) return;  // whole waves leave together
  const int nq = q - q0 < 8 ? q - q0 : 8;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  const double* a = A + row * lda;
  for (int64_t kk = lane; kk < k; kk += 64) {
    const double av = a[kk];
    const double* bk = B + kk * q + q0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < nq) acc[j] = fma(av, bk[j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    double v = acc[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    acc[j] = v;
  }
  if (lane < nq) {
    double v = acc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (lane == j) v = acc[j];
    C[row * q + q0 + lane] = v;
  }
}

// C [k x q] = A^T B, A [m x k] (ld lda), B [m x q] (ld q): one thread per
// column of A (coalesced across the workgroup), 8 columns of C per
// blockIdx.z (q0 = 8 z); blockIdx.y = slice s of the sum over m (rows
// [s mc, (s+1) mc)); with one slice the result goes to C, else to part[s]
// (k x q each), summed in slice order by ch_sum_kernel.
__global__ __launch_bounds__(256) void ch_gemm_tn(const double* __restrict__ A, int64_t lda,
                                                  const double* __restrict__ B, int64_t m,
                                                  int64_t k, int q, int64_t mc,
                                                  double* __restrict__ C,
                                                  double* __restrict__ part) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q0 = blockIdx.z * 8;
  if (col >= k) return;
  const int nq = q - q0 < 8 ? q - q0 : 8;
  const int64_t m0 = (int64_t)blockIdx.y * mc;
  const int64_t m1 = m0 + mc < m ? m0 + mc : m;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  // four rows per step, their loads issued together (the sums keep the row
  // order)
  int64_t r = m0;
  for (; r + 4 <= m1; r += 4) {
    double av[4], bv[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = A[(r + u) * lda + col];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[u][j] = j < nq ? B[(r + u) * q + q0 + j] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fma(av[u], bv[u][j], acc[j]);
  }
  for (; r < m1; ++r) {
    const double av = A[r * lda + col];
    const double* br = B + r * q + q0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < nq) acc[j] = fma(av, br[j], acc[j]);
  }
  double* out = gridDim.y == 1 ? C : part + (int64_t)blockIdx.y * k * q;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < nq) out[col * q + q0 + j] = acc[j];
}

__global__ void ch_sum_kernel(const double* __restrict__ part, int ns, int64_t n,
                              double* __restrict__ C) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    double s = 0.0;
#pragma unroll 8
    for (int p = 0; p < ns; ++p) s += part[(int64_t)p * n + e];
    C[e] = s;
  }
}

// G [q x q] symmetric positive definite = R^T R (R upper); Rinv = R^-1. One
// wave, the matrices in LDS: right-looking Cholesky by rows (lane = column),
// then every lane back-substitutes its column of the inverse. A pivot that
// is not above 1e-15 of its diagonal entry of G (the sketch has lost rank:
// the weighted W has rank below q) sets ST_NOTSPD, a pivot that is not
// finite (a NaN or Inf weight) ST_NONFINITE.
__global__ __launch_bounds__(64) void ch_chol_inv_kernel(const double* __restrict__ G, int q,
                                                         double* __restrict__ Rinv,
                                                         unsigned* __restrict__ status) {
  __shared__ double a[CH_RMAX][CH_RMAX + 1];
  __shared__ double x[CH_RMAX][CH_RMAX + 1];
  const int l = threadIdx.x;
  for (int e = l; e < q * q; e += 64) a[e / q][e % q] = G[e];
  __syncthreads();
  bool bad = false, nonfin = false;
  for (int k = 0; k < q; ++k) {
    const double piv = a[k][k];
    const bool fin = isfinite(piv) && isfinite(G[k * q + k]);
    const bool ok = fin && piv > 1e-15 * G[k * q + k];
    bad = bad || (fin && !ok);
    nonfin = nonfin || !fin;
    const double rkk = sqrt(ok ? piv : 1.0);
    __syncthreads();
    if (l > k && l < q) a[k][l] /= rkk;  // row k of R, right of the diagonal
    __syncthreads();
    if (l == k) a[k][k] = rkk;
    if (l > k && l < q)
      for (int r = k + 1; r <= l; ++r) a[r][l] -= a[k][r] * a[k][l];  // trailing upper part
    __syncthreads();
  }
  if (l == 0 && bad) atomicOr(status, ST_NOTSPD);
  if (l == 0 && nonfin) atomicOr(status, ST_NONFINITE);
  // column l of R^-1 (upper triangular) by back substitution
  if (l < q) {
    for (int r = l; r >= 0; --r) {
      double s = r == l ? 1.0 : 0.0;
      for (int k2 = r + 1; k2 <= l; ++k2) s -= a[r][k2] * x[k2][l];
      x[r][l] = s / a[r][r];
    }
    for (int r = 0; r < q; ++r) Rinv[r * q + l] = r <= l ? x[r][l] : 0.0;
  }
}

// Eigen-decomposition of a symmetric q x q matrix M by cyclic Jacobi
// rotations (one wave, LDS), eigenvalues in descending order: Uh [q x q]
// holds the eigenvectors as columns, sig[k] = sqrt(max(lambda_k, 0)).
__global__ __launch_bounds__(64) void ch_jacobi_kernel(const double* __restrict__ M, int q,
                                                       double* __restrict__ Uh,
                                                       double* __restrict__ sig) {
  __shared__ double a[CH_RMAX][CH_RMAX + 1];
  __shared__ double v[CH_RMAX][CH_RMAX + 1];
  __shared__ double cs[2];
  __shared__ int order[CH_RMAX];
  const int l = threadIdx.x;
  for (int e = l; e < q * q; e += 64) {
    a[e / q][e % q] = M[e];
    v[e / q][e % q] = (e / q == e % q) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    double off = 0.0, dg = 0.0;
    for (int r = 0; r < q; ++r)
      for (int k = 0; k < q; ++k) {
        if (r == k) dg += a[r][k] * a[r][k];
        else off += a[r][k] * a[r][k];
      }
    if (off <= 1e-30 * dg) break;  // uniform: every lane reads the same LDS
    for (int p = 0; p < q - 1; ++p)
      for (int r = p + 1; r < q; ++r) {
        if (l == 0) {
          // rotation in the (p, r) plane that zeroes a[p][r]: with
          // theta = (a_rr - a_pp) / (2 a_pr), t = tan = sgn(theta) /
          // (|theta| + sqrt(theta^2 + 1)) (the smaller root)
          const double apr = a[p][r];
          double c = 1.0, s = 0.0;
          if (apr != 0.0) {
            const double th = (a[r][r] - a[p][p]) / (2.0 * apr);
            const double t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(1.0 + th * th));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
          }
          cs[0] = c;
          cs[1] = s;
        }
        __syncthreads();
        const double c = cs[0], s = cs[1];
        if (s != 0.0) {
          if (l < q) {  // columns p, r of A and of V
            const double akp = a[l][p], akr = a[l][r];
            a[l][p] = c * akp - s * akr;
            a[l][r] = s * akp + c * akr;
            const double vkp = v[l][p], vkr = v[l][r];
            v[l][p] = c * vkp - s * vkr;
            v[l][r] = s * vkp + c * vkr;
          }
          __syncthreads();
          if (l < q) {  // rows p, r of A
            const double apk = a[p][l], ark = a[r][l];
            a[p][l] = c * apk - s * ark;
            a[r][l] = s * apk + c * ark;
          }
        }
        __syncthreads();
      }
  }
  if (l == 0) {  // descending eigenvalues, ties in index order
    unsigned long long used = 0ull;
    for (int k = 0; k < q; ++k) {
      int best = -1;
      for (int m = 0; m < q; ++m)
        if (!((used >> m) & 1ull) && (best < 0 || a[m][m] > a[best][best])) best = m;
      used |= 1ull << best;
      order[k] = best;
    }
  }
  __syncthreads();
  if (l < q) {
    const int src = order[l];
    sig[l] = sqrt(fmax(a[src][src], 0.0));
    for (int r = 0; r < q; ++r) Uh[r * q + l] = v[r][src];
  }
}

// A[row][k] = fp16(Ul[row][k] * sig[k]) [o x r]; B[k][j] = fp16(Vz[j][k] /
// sig[k] / sc[j]) [r x i] (Vz = Z Uh). A component with sig = 0 has A = 0
// and B = 0 (its direction carries nothing).
__global__ void ch_factor_kernel(const double* __restrict__ Ul, const double* __restrict__ Vz,
                                 const double* __restrict__ sig, const double* __restrict__ sc,
                                 int64_t o, int64_t i, int r, uint16_t* __restrict__ A,
                                 uint16_t* __restrict__ B) {
  const int64_t na = o * r, nb = (int64_t)r * i;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < na + nb;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < na) {
      const int k = (int)(e % r);
      A[e] = f64_to_f16_rne(Ul[e] * sig[k]);
    } else {
      const int64_t f = e - na, k = f / i, j = f - k * i;
      B[f] = sig[k] > 0.0 ? f64_to_f16_rne(Vz[j * r + k] / sig[k] / sc[j]) : (uint16_t)0;
    }
  }
}

// The residual, stored by column (rows contiguous, the sweep's lane order):
//   ResT[j][row] = W[row][j] - sum_k A[row][k] B[k][j]   (fp64 from fp16).
// One workgroup per 64 x 64 tile: the tile's rows of A and columns of B are
// staged in LDS, W is read along its rows (all 16 loads of a thread issued
// together), the tile is turned in LDS and ResT written along its columns.
__global__ __launch_bounds__(256) void ch_resid_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                       int64_t o, int64_t i,
                                                       const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B, int r,
                                                       double* __restrict__ ResT,
                                                       unsigned* __restrict__ status) {
  __shared__ double T[64][65];
  __shared__ double As[64][CH_RMAX + 1];
  __shared__ double Bs[CH_RMAX][64];
  const int t = threadIdx.x, tx = t & 63, ty = t >> 6;
  const int64_t row0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int64_t j = j0 + tx;
  for (int e = t; e < 64 * r; e += 256) {
    const int rr = e / r, k = e - rr * r;
    As[rr][k] = row0 + rr < o ? f16_to_f64(A[(row0 + rr) * r + k]) : 0.0;
  }
  for (int e = t; e < 64 * r; e += 256) {
    const int k = e >> 6, c = e & 63;
    Bs[k][c] = j0 + c < i ? f16_to_f64(B[(int64_t)k * i + j0 + c]) : 0.0;
  }
  double wv[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int64_t row = row0 + ty + 4 * m;
    wv[m] = (row < o && j < i) ? f16_to_f64(W[row * ldw + j]) : 0.0;
  }
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int rr = ty + 4 * m;
    double acc = 0.0;
    for (int k = 0; k < r; ++k) acc = fma(As[rr][k], Bs[k][tx], acc);
    const double v = wv[m] - acc;
    if (row0 + rr < o && j < i) bad |= !isfinite(v);
    T[rr][tx] = v;
  }
  if (bad) atomicOr(status, ST_NONFINITE);
  __syncthreads();
  const int64_t row = row0 + tx;
  for (int jj = ty; jj < 64; jj += 4)
    if (row < o && j0 + jj < i) ResT[(j0 + jj) * o + row] = T[tx][jj];
}

// Lazy update of the block [j0, j0 + bw) (sweep order) over the errors of
// columns [k_lo, k_hi), k_lo = blockIdx.y * ks, k_hi <= j0:
//   part[y][c][row] = sum_k ET[k][row] U[k][j0 + c]    (c < 128; 0 beyond bw)
// (errors and partial sums stored by column, rows contiguous)
// A workgroup forms 64 rows x 128 columns, thread (tc, tr) = (t / 16, t % 16)
// the rows tr + 16 b and the columns 8 tc .. 8 tc + 7, through 16-deep LDS
// stages of E and U; loads and stores run along the rows (16 consecutive
// rows per column in each wave access).
__global__ __launch_bounds__(256) void ch_update_kernel(const double* __restrict__ ET,
                                                        const float* __restrict__ U,
                                                        int64_t rows, int64_t cols, int64_t j0,
                                                        int bw, int64_t ks,
                                                        double* __restrict__ part,
                                                        int64_t pstride) {
  __shared__ double Es[16][64];
  __shared__ float Us[16][CH_QB];
  const int t = threadIdx.x, tr = t & 15, tc = t >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t k_lo = (int64_t)blockIdx.y * ks;
  const int64_t k_hi = k_lo + ks < j0 ? k_lo + ks : j0;
  double acc[4][8];  // [row tr + 16 b][column 8 tc + a]
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int a = 0; a < 8; ++a) acc[b][a] = 0.0;
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += 16) {
    {
      const int kk = t >> 4;
      const int64_t k = k0 + kk;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int64_t row = r0 + tr + 16 * x;
        Es[kk][tr + 16 * x] = (row < rows && k < k_hi) ? ET[k * rows + row] : 0.0;
      }
    }
    {
      const int kk = t >> 4;
      const int64_t k = k0 + kk;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int c = (t & 15) + 16 * x;
        Us[kk][c] = (k < k_hi && c < bw) ? U[k * cols + j0 + c] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 16; ++kk) {
      double e[4], u[8];
#pragma unroll
      for (int b = 0; b < 4; ++b) e[b] = Es[kk][tr + 16 * b];
#pragma unroll
      for (int a = 0; a < 8; ++a) u[a] = (double)Us[kk][8 * tc + a];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < 8; ++a) acc[b][a] = fma(e[b], u[a], acc[b][a]);
    }
    __syncthreads();
  }
  double* out = part + (int64_t)blockIdx.y * pstride;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t row = r0 + tr + 16 * b;
    if (row < rows)
#pragma unroll
      for (int a = 0; a < 8; ++a) out[(int64_t)(8 * tc + a) * rows + row] = acc[b][a];
  }
}

// The block's current values for the sweep, by block column:
//   cur[c][row] = ResT[perm[j0 + c]][row] - sum_q part[q][c][row]
// (the update pieces summed in piece order; 0 for c >= bw).
__global__ void ch_cur_kernel(const double* __restrict__ part, int np, int64_t pstride,
                              const double* __restrict__ ResT, int64_t rows, int64_t cols,
                              const int32_t* __restrict__ perm, int64_t j0, int bw,
                              double* __restrict__ cur) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < pstride;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e / rows);
    const int64_t row = e - (int64_t)c * rows;
    double v = 0.0;
    if (c < bw) {
      int64_t oc = perm ? (int64_t)perm[j0 + c] : j0 + c;
      if (oc < 0 || oc >= cols) oc = 0;  // reported as ST_BADPERM before the sweep
      double sum = 0.0;
#pragma unroll 8
      for (int q = 0; q < np; ++q) sum += part[(int64_t)q * pstride + e];
      v = ResT[oc * rows + row] - sum;
    }
    cur[e] = v;
  }
}

// binary16 bits of a double that is exactly representable in binary16 and
// not negative (a grid step): exponent and the top 10 fraction bits, or the
// subnormal count of 2^-24; infinity gives 0x7c00.
__device__ inline uint16_t f16_bits_of_exact(double x) {
  if (!(x < 65536.0)) return 0x7c00;
  const long long b = __double_as_longlong(x);
  const int e = (int)((b >> 52) & 0x7ff) - 1023;
  if (e >= -14) return (uint16_t)(((e + 15) << 10) | (int)((b >> 42) & 0x3ff));
  return (uint16_t)(x * 16777216.0);  // 2^24: subnormal (or zero) count
}

// The sweep of the block [j0, j0 + bw) with one grid per group of G output
// channels (rows) and column, starting from the residual ResT[perm[j]][row]
// (first block) or from cur, the residual less the update sum of the
// earlier blocks (by block column, from ch_cur_kernel); codes and grids go to the
// original column perm[j], the scaled errors to ET[j][row] (sweep order,
// by column like the residual and the update sums), the squared errors
// to row_loss (set on the first block). The step and U[j][j] enter as
// reciprocals, as in the GPTQ sweep.
//
// One workgroup of four waves per group of G rows (lane l: rows l + 64 p,
// p < RP; for G = 32 the upper half of the wave holds zeros, which the range
// contains anyway), the block's columns in four stripes of 32 (wave w:
// columns 32 w .. 32 w + 31, in registers). The block is swept in sub-blocks
// of 16 columns, each by the wave that holds it, in a loop that is not
// unrolled: the column under way is always register 0 of the sub-block, and
// the update of the later columns moves each one register down (an fma into
// the next lower register), so the loop body is the same for every column.
// A single wave runs the column chain, so its time is about the count of
// instructions issued per column: the group's range is one reduction over
// the wave in DPP moves (no LDS), every lane quantizes its own rows, and
// codes, errors and grids go to LDS as they are (conversions and global
// stores wait for the end of the block). The sub-block's errors then reach
// the later columns: the other waves apply them while the next sub-block is
// swept, one barrier per sub-block (two error buffers). The U slab stays
// fp32 in LDS, as stored. Errors go to ET from LDS one sub-block later,
// codes and grids after the block (without a permutation, four codes of a
// row per store).
constexpr int CH_SB = 16;  // columns per sub-block

template <int CTRL, int RM>
__device__ inline double ch_dpp(double v) {
  union { double d; int i[2]; } a, b;
  a.d = v;
  if constexpr (RM == 0xF) {  // every lane written
    b.i[0] = __builtin_amdgcn_mov_dpp(a.i[0], CTRL, RM, 0xF, false);
    b.i[1] = __builtin_amdgcn_mov_dpp(a.i[1], CTRL, RM, 0xF, false);
  } else {
    b.i[0] = __builtin_amdgcn_update_dpp(a.i[0], a.i[0], CTRL, RM, 0xF, false);
    b.i[1] = __builtin_amdgcn_update_dpp(a.i[1], a.i[1], CTRL, RM, 0xF, false);
  }
  return b.d;
}
__device__ inline double ch_lane63(double v) {
  union { double d; int i[2]; } a;
  a.d = v;
  a.i[0] = __builtin_amdgcn_readlane(a.i[0], 63);
  a.i[1] = __builtin_amdgcn_readlane(a.i[1], 63);
  return a.d;
}
// min and max over the 64 lanes of the wave, returned uniform: the four
// 16-lane rows reduce in quad and row rotations, rows 1 and 3 then take
// the last lane of rows 0 and 2, rows 2 and 3 the last lane of row 1, so
// that lane 63 holds the whole wave's result (rows left out by a row mask
// keep their value, which min and max leave unchanged)
__device__ inline void ch_wave_minmax(double& mn, double& mx) {
  mn = fmin(mn, ch_dpp<0xB1, 0xF>(mn));  // quad_perm [1,0,3,2]
  mx = fmax(mx, ch_dpp<0xB1, 0xF>(mx));
  mn = fmin(mn, ch_dpp<0x4E, 0xF>(mn));  // quad_perm [2,3,0,1]
  mx = fmax(mx, ch_dpp<0x4E, 0xF>(mx));
  mn = fmin(mn, ch_dpp<0x124, 0xF>(mn)); // row_ror 4
  mx = fmax(mx, ch_dpp<0x124, 0xF>(mx));
  mn = fmin(mn, ch_dpp<0x128, 0xF>(mn)); // row_ror 8
  mx = fmax(mx, ch_dpp<0x128, 0xF>(mx));
  mn = fmin(mn, ch_dpp<0x142, 0xA>(mn)); // row_bcast 15 into rows 1, 3
  mx = fmax(mx, ch_dpp<0x142, 0xA>(mx));
  mn = fmin(mn, ch_dpp<0x143, 0xC>(mn)); // row_bcast 31 into rows 2, 3
  mx = fmax(mx, ch_dpp<0x143, 0xC>(mx));
  mn = ch_lane63(mn);
  mx = ch_lane63(mx);
}

template <int G>
__global__ __launch_bounds__(256) void ch_sweep_rows_kernel(
    const double* __restrict__ ResT, int64_t rows, int64_t cols, int64_t j0, int bw,
    const double* __restrict__ cur, const float* __restrict__ U,
    const int32_t* __restrict__ perm, int bits, double* __restrict__ ET,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
    double* __restrict__ row_loss, unsigned* __restrict__ status, bool fac) {
  constexpr int RP = G >= 64 ? G / 64 : 1;  // rows per lane
  constexpr int NC = CH_QB / 4;             // columns per wave
  constexpr int KPT = CH_SB * G / 256;      // errors per thread in the ET copy
  // the U slab, row-major (fp32 as stored); the shifted update of the last
  // columns reads up to CH_SB - 1 entries past a row's end (zeros at the end)
  __shared__ float Us[CH_QB * CH_QB + CH_SB];
  __shared__ double Es[2][CH_SB][G];  // a sub-block's errors, [column][row]
  __shared__ double Rd[CH_QB];        // 1 / U[jb][jb]
  __shared__ uint8_t Ks[CH_QB][G];    // the block's codes, [column][row]
  __shared__ double Sd[CH_QB], Zd[CH_QB];  // its grids: step, zero point
  __shared__ int Pm[CH_QB];           // original column of each block column
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t grp = blockIdx.x;
  bool rv[RP];
  int64_t row[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    const int lr = lane + 64 * p;
    row[p] = grp * G + lr;
    rv[p] = lr < G && row[p] < rows;
  }
  const double maxq = (double)((1 << bits) - 1);
  const double rmaxq = 1.0 / maxq;
  // every load of the prologue is issued before its first use (each round
  // trip to memory costs about a microsecond)
  if (t < CH_QB) {
    int64_t oc = 0;
    if (t < bw) {
      oc = perm ? (int64_t)perm[j0 + t] : j0 + t;
      if (oc < 0 || oc >= cols) oc = 0;  // reported as ST_BADPERM before the sweep
    }
    Pm[t] = (int)oc;
    Rd[t] = t < bw ? 1.0 / (double)U[(j0 + t) * cols + j0 + t] : 0.0;
  }
  if (t < CH_SB) Us[CH_QB * CH_QB + t] = 0.0f;
  if (bw == CH_QB && (cols & 3) == 0) {
    // 16 float4 per thread, row a = e / 32 of the slab
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = t + 256 * u, a = e >> 5, b4 = e & 31;
      v[u] = *reinterpret_cast<const float4*>(U + (j0 + a) * cols + j0 + 4 * b4);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) reinterpret_cast<float4*>(Us)[t + 256 * u] = v[u];
  } else {
#pragma unroll 1
    for (int e0 = 0; e0 < CH_QB * CH_QB; e0 += 16 * 256) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + t + 256 * u, a = e >> 7, b = e & 127;
        v[u] = (a < bw && b < bw) ? U[(j0 + a) * cols + j0 + b] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) Us[e0 + t + 256 * u] = v[u];
    }
  }
  __syncthreads();
  // current values of the wave's 32 columns (zero for rows outside the group)
  double w[RP][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = NC * wv + c;
    const double* src = cur ? cur + (int64_t)col * rows : ResT + (int64_t)Pm[col] * rows;
#pragma unroll
    for (int p = 0; p < RP; ++p) w[p][c] = (col < bw && rv[p]) ? src[row[p]] : 0.0;
  }
  double lsum[RP], loss0[RP];  // this block's squared errors; the earlier blocks'
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    lsum[p] = 0.0;
    loss0[p] = (j0 > 0 && wv == 0 && rv[p]) ? row_loss[row[p]] : 0.0;
  }
  bool bad = false;

  // the errors of sub-block sb applied to this wave's columns LO .. HI - 1
  // (all of them after the sub-block); the U row and the errors of step
  // k + 1 are read before the products of step k, so no product waits for LDS
  auto apply = [&](int sb, auto lo_c, auto hi_c) {
    constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value, NU = HI - LO;
    const double* es = &Es[sb & 1][0][0];
    const int kn = min(CH_SB, bw - CH_SB * sb);
    const float* ub = Us + (CH_SB * sb) * CH_QB + NC * wv + LO;
    float un[NU];
    double en[RP];
#pragma unroll
    for (int c = 0; c < NU; ++c) un[c] = ub[c];
#pragma unroll
    for (int p = 0; p < RP; ++p) en[p] = lane + 64 * p < G ? es[lane + 64 * p] : 0.0;
#pragma unroll 2
    for (int k = 0; k < kn; ++k) {
      float uc[NU];
      double ev[RP];
#pragma unroll
      for (int c = 0; c < NU; ++c) uc[c] = un[c];
#pragma unroll
      for (int p = 0; p < RP; ++p) ev[p] = en[p];
      const int kx = k + 1 < kn ? k + 1 : k;
#pragma unroll
      for (int c = 0; c < NU; ++c) un[c] = ub[kx * CH_QB + c];
#pragma unroll
      for (int p = 0; p < RP; ++p) en[p] = lane + 64 * p < G ? es[kx * G + lane + 64 * p] : 0.0;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NU; ++c) {
        const double u = (double)uc[c];
#pragma unroll
        for (int p = 0; p < RP; ++p) w[p][LO + c] = fma(-ev[p], u, w[p][LO + c]);
      }
    }
  };

  // the sweep of sub-block sb by its wave, the registers H .. H + 15
  auto sweep = [&](int sb, auto half_c) {
    constexpr int H = decltype(half_c)::value * CH_SB;
    double* es = &Es[sb & 1][0][0];
    const int jbeg = CH_SB * sb, jend = min(jbeg + CH_SB, bw);
    for (int jb = jbeg; jb < jend; ++jb) {
      // this column's row of U and 1 / U[jb][jb] are read first, so the LDS
      // latency passes during the range reduction
      const float* ur = Us + jb * CH_QB + jb + 1;  // columns jb + 1 .. jb + 15
      float uu[CH_SB - 1];
#pragma unroll
      for (int c = 0; c < CH_SB - 1; ++c) uu[c] = ur[c];
      const double rd = Rd[jb];
      __builtin_amdgcn_sched_barrier(0);
      double mn = 0.0, mx = 0.0;  // the range includes 0
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        mn = fmin(mn, w[p][H]);
        mx = fmax(mx, w[p][H]);
      }
      ch_wave_minmax(mn, mx);
      double scale = f16_round_f64((mx - mn) * rmaxq), zero = 0.0;
      bad |= !(scale <= 65504.0);
      const bool degen = mx == mn || scale == 0.0;
      if (degen) scale = 1.0;
      const double rs = 1.0 / scale;
      if (!degen) zero = fmin(fmax(rint(-mn * rs), 0.0), maxq);
      double e[RP];
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        const double v = w[p][H];
        const double k = fmin(fmax(rint(v * rs) + zero, 0.0), maxq);
        e[p] = rv[p] ? (v - scale * (k - zero)) * rd : 0.0;
        lsum[p] = fma(e[p], e[p], lsum[p]);
        if (lane + 64 * p < G) {
          es[(jb - jbeg) * G + lane + 64 * p] = e[p];
          Ks[jb][lane + 64 * p] = (uint8_t)k;
        }
      }
      if (lane == 0) {
        Sd[jb] = scale;
        Zd[jb] = zero;
      }
      // the sub-block's later columns, each one register down
#pragma unroll
      for (int c = 0; c < CH_SB - 1; ++c)
#pragma unroll
        for (int p = 0; p < RP; ++p) w[p][H + c] = fma(-e[p], (double)uu[c], w[p][H + c + 1]);
    }
  };

  // errors of sub-block sb from LDS to ET (sweep order): thread t takes row
  // t % G of the columns KPT (t / G) .. KPT (t / G) + KPT - 1. In the factor
  // form (U holds R U over each block beyond U's diagonal blocks, R = U^-1)
  // ET takes the residual q - r of the swept value r (the residual matrix's
  // entry) instead: the dequantized value from the block's code and grid,
  // the entry (read from ResT while the sub-block was swept, in rv), their
  // difference exact in fp64
  auto store_e = [&](int sb, const double (&rv)[KPT]) {
    const int r = t % G, k0 = KPT * (t / G);
    const int64_t gr = grp * G + r;
    const int kn = min(CH_SB, bw - CH_SB * sb);
    if (gr < rows) {
      const double* es = &Es[sb & 1][0][0];
      double* dst = ET + (j0 + CH_SB * sb) * rows + gr;
      if (fac) {
#pragma unroll
        for (int k = 0; k < KPT; ++k)
          if (k0 + k < kn) {
            const int c = CH_SB * sb + k0 + k;
            const double dq = Sd[c] * ((double)Ks[c][r] - Zd[c]);
            dst[(k0 + k) * rows] = dq - rv[k];
          }
      } else {
#pragma unroll
        for (int k = 0; k < KPT; ++k)
          if (k0 + k < kn) dst[(k0 + k) * rows] = es[(k0 + k) * G + r];
      }
    }
  };

  // factor form: the residual matrix's entries of sub-block sb, loaded when
  // its sweep starts and used by its store one sub-block later
  auto load_r = [&](int sb, double (&rv)[KPT]) {
    const int r = t % G, k0 = KPT * (t / G);
    const int64_t gr = grp * G + r;
    const int kn = min(CH_SB, bw - CH_SB * sb);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      rv[k] = (gr < rows && k0 + k < kn)
                  ? ResT[(int64_t)Pm[CH_SB * sb + k0 + k] * rows + gr] : 0.0;
  };
  double rA[KPT], rB[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) rA[k] = rB[k] = 0.0;
  const int nsb = (bw + CH_SB - 1) / CH_SB;
  for (int sb = 0; sb < nsb; ++sb) {
    const int owner = sb >> 1;
    if (fac) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) rA[k] = rB[k];  // sub-block sb - 1
      load_r(sb, rB);
    }
    if (sb > 0) store_e(sb - 1, rA);
    if (wv == owner) {
      if (sb & 1) {
        if (sb > 0) apply(sb - 1, std::integral_constant<int, CH_SB>{},
                          std::integral_constant<int, NC>{});
        sweep(sb, std::integral_constant<int, 1>{});
      } else {
        if (sb > 0) apply(sb - 1, std::integral_constant<int, 0>{},
                          std::integral_constant<int, CH_SB>{});
        sweep(sb, std::integral_constant<int, 0>{});
        if (sb > 0) apply(sb - 1, std::integral_constant<int, CH_SB>{},
                          std::integral_constant<int, NC>{});
      }
    } else if (sb > 0 && wv > owner) {
      apply(sb - 1, std::integral_constant<int, 0>{}, std::integral_constant<int, NC>{});
    }
    __syncthreads();
  }
  store_e(nsb - 1, rB);
  // codes and grids to the original columns
  if (!perm && bw == CH_QB && (cols & 3) == 0 && ((uintptr_t)codes & 3) == 0) {
    // four consecutive columns of a row per store: lane = column quad
    const int q = t & 31;
#pragma unroll 4
    for (int r = t >> 5; r < G; r += 8) {
      const int64_t gr = grp * G + r;
      const uint32_t v = (uint32_t)Ks[4 * q][r] | ((uint32_t)Ks[4 * q + 1][r] << 8) |
                         ((uint32_t)Ks[4 * q + 2][r] << 16) | ((uint32_t)Ks[4 * q + 3][r] << 24);
      if (gr < rows) *reinterpret_cast<uint32_t*>(codes + gr * cols + j0 + 4 * q) = v;
    }
  } else {
    // lane = block column: without a permutation 64 consecutive bytes of a row
    const int jb = t & (CH_QB - 1);
    if (jb < bw) {
      const int64_t oc = Pm[jb];
#pragma unroll 4
      for (int r = t >> 7; r < G; r += 2) {
        const int64_t gr = grp * G + r;
        if (gr < rows) codes[gr * cols + oc] = Ks[jb][r];
      }
    }
  }
  if (t < bw) {
    const int64_t oc = Pm[t];
    scales[grp * cols + oc] = f16_bits_of_exact(Sd[t]);
    zeros[grp * cols + oc] = f64_to_f16_rne(Zd[t]);
  }
  if (bad && lane == 0) atomicOr(status, ST_NONFINITE);
  // each row's loss over the block: the four waves' sums (each over the
  // columns it swept, in column order), added in wave order
  __syncthreads();  // Es[0] is read by the E copy above
#pragma unroll
  for (int p = 0; p < RP; ++p)
    if (lane + 64 * p < G) Es[0][wv][lane + 64 * p] = lsum[p];
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int p = 0; p < RP; ++p)
      if (rv[p]) {
        const int lr = lane + 64 * p;
        const double l = ((Es[0][0][lr] + Es[0][1][lr]) + Es[0][2][lr]) + Es[0][3][lr];
        row_loss[row[p]] = loss0[p] + l;
      }
  }
}

// Sum over m of A^T B in ns slices: the slice count that gives about 512
// workgroups (each slice at least 64 rows long).
inline int ch_slices(int64_t m, int64_t k) {
  const int64_t wg = std::max<int64_t>(1, cdiv(k, 256));
  int64_t s = cdiv(512, wg);
  s = std::min<int64_t>(s, std::max<int64_t>(1, m / 64));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}

struct CHLayout {
  size_t status, cnt, c, sc, wt, y, q, q1, z, zq, gm, rinv, mm, uh, sig, ul, vz, res, e, tpart,
      part, psum, total;
  int pmax;
  int64_t pstride;
  CHLayout(int64_t o, int64_t i, int r) {
    size_t p = 0;
    auto take = [&](size_t bytes) {
      const size_t at = p;
      p = (size_t)round_up((int64_t)(p + bytes), 256);
      return at;
    };
    const int64_t mx = o > i ? o : i;
    status = take(4);
    cnt = take(4 * i);
    c = take(8 * i);
    sc = take(8 * i);
    wt = take(8 * o * i);
    y = take(8 * o * r);
    q = take(8 * o * r);
    q1 = take(8 * mx * r);
    z = take(8 * i * r);
    zq = take(8 * i * r);
    gm = take(8 * r * r);
    rinv = take(8 * r * r);
    mm = take(8 * r * r);
    uh = take(8 * r * r);
    sig = take(8 * r);
    ul = take(8 * o * r);
    vz = take(8 * i * r);
    res = take(8 * o * i);
    e = take(8 * o * i);
    // slice partials of the A^T B products made: Gram matrices over o and i
    // rows, Z = W~^T Q over o rows
    int64_t tp = std::max<int64_t>((int64_t)ch_slices(o, r), (int64_t)ch_slices(i, r)) * r * r;
    tp = std::max<int64_t>(tp, (int64_t)ch_slices(o, i) * i * r);
    tpart = take(8 * tp);
    const int64_t rt = cdiv(o, 64);
    pmax = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(i, CH_KS), cdiv(1024, rt)));
    pstride = o * CH_QB;
    part = take(8 * (size_t)pmax * pstride);
    psum = take(8 * (size_t)pstride);
    total = p;
  }
};

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_chmc_rank(int64_t rows, int64_t cols, int bits, int group_size,
                              double bpw_target) {
  if (rows <= 0 || cols <= 0 || bits < 2 || bits > 8 || group_size <= 0) return 0;
  // Schritt 3's budget with the residual grid's zero point (bits bits per
  // output group and column) counted beside its fp16 scale
  const double o = (double)rows, i = (double)cols;
  const double r = std::floor((bpw_target * o * i - bits * o * i -
                               (16.0 + bits) * (double)cdiv(rows, group_size) * i) /
                              (16.0 * (o + i)));
  if (!(r > 0.0)) return 0;
  return (int)std::min<double>(r, (double)std::min<int64_t>(std::min(rows, cols), CH_RMAX));
}

extern "C" size_t gptq_chmc_workspace_bytes(int64_t rows, int64_t cols, int rank) {
  if (rows <= 0 || cols <= 0 || rank < 0 || rank > CH_RMAX) return 0;
  return CHLayout(rows, cols, rank).total;
}

extern "C" gptq_status gptq_chmc_layer(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                       const double* S, int64_t n_tokens, const float* U,
                                       const int32_t* perm, const double* omega, int rank,
                                       int bits, int group_size, uint32_t flags, uint16_t* A,
                                       uint16_t* B, uint8_t* codes, uint16_t* scales,
                                       uint16_t* zeros, double* row_loss, void* ws,
                                       size_t ws_bytes, void* stream, void* u_stream) {
  if (flags & ~(GPTQ_FLAG_NO_SYNC | GPTQ_FLAG_FACTOR_FORM)) return GPTQ_EINVAL;
  if (rows <= 0 || cols <= 0 || n_tokens <= 0) return GPTQ_EINVAL;
  const bool fac = (flags & GPTQ_FLAG_FACTOR_FORM) != 0;
  if (bits < 2 || bits > 8) return GPTQ_EINVAL;
  if (group_size != 32 && group_size != 64 && group_size != 128) return GPTQ_EINVAL;
  if (rank < 0 || rank > CH_RMAX || rank > rows || rank > cols) return GPTQ_EINVAL;
  if (!W || !S || !U || !codes || !scales || !zeros || !row_loss || ldw < cols) return GPTQ_EINVAL;
  if (rank > 0 && (!omega || !A || !B)) return GPTQ_EINVAL;
  if (cols > ((int64_t)1 << 20) || rows > ((int64_t)1 << 24)) return GPTQ_EINVAL;
  const CHLayout L(rows, cols, rank);
  if (!ws || ws_bytes < L.total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  unsigned* status = (unsigned*)(b + L.status);
  unsigned* cnt = (unsigned*)(b + L.cnt);
  double *c = (double*)(b + L.c), *sc = (double*)(b + L.sc), *Wt = (double*)(b + L.wt);
  double *Y = (double*)(b + L.y), *Q = (double*)(b + L.q), *Q1 = (double*)(b + L.q1);
  double *Z = (double*)(b + L.z), *Zq = (double*)(b + L.zq), *Gm = (double*)(b + L.gm);
  double *Rinv = (double*)(b + L.rinv), *Mm = (double*)(b + L.mm), *Uh = (double*)(b + L.uh);
  double *sig = (double*)(b + L.sig), *Ul = (double*)(b + L.ul), *Vz = (double*)(b + L.vz);
  double *Res = (double*)(b + L.res), *E = (double*)(b + L.e), *Tp = (double*)(b + L.tpart);
  double* part = (double*)(b + L.part);
  double* psum = (double*)(b + L.psum);
  const int64_t o = rows, i = cols;
  const int r = rank;
  auto grid1 = [](int64_t n) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, 256), 65536));
  };
  auto rowsg = [](int64_t m) { return (unsigned)cdiv(m, 4); };
  GPTQ_LAUNCH(K_FILL, st, ch_zero_kernel<<<1, 64, 0, st>>>(status, 1));
  GPTQ_LAUNCH(K_CH_FRONT, st,
              ch_energy_kernel<<<1, 1024, 0, st>>>(S, i, 1.0 / (double)n_tokens, c, sc, status));
  // C [k x r] = A^T B over m rows, split in slices when that fills the chip
  auto gemm_tn = [&](const double* Am, int64_t lda, const double* Bm, int64_t m, int64_t k,
                     double* C) -> gptq_status {
    const int ns = ch_slices(m, k);
    const int64_t mc = cdiv(m, ns);
    dim3 grid((unsigned)cdiv(k, 256), (unsigned)ns, (unsigned)cdiv(r, 8));
    GPTQ_LAUNCH(K_CH_FRONT, st,
                ch_gemm_tn<<<grid, 256, 0, st>>>(Am, lda, Bm, m, k, r, mc, C, Tp));
    if (ns > 1)
      GPTQ_LAUNCH(K_CH_FRONT, st, ch_sum_kernel<<<grid1(k * r), 256, 0, st>>>(Tp, ns, k * r, C));
    return GPTQ_OK;
  };
  // orth(Y [m x r]) into Qout: CholeskyQR twice
  auto orth = [&](const double* Yin, int64_t m, double* Qout) -> gptq_status {
    const double* src = Yin;
    for (int pass = 0; pass < 2; ++pass) {
      double* dst = pass == 0 ? Q1 : Qout;
      const gptq_status s = gemm_tn(src, r, src, m, r, Gm);
      if (s != GPTQ_OK) return s;
      GPTQ_LAUNCH(K_CH_FRONT, st, ch_chol_inv_kernel<<<1, 64, 0, st>>>(Gm, r, Rinv, status));
      GPTQ_LAUNCH(K_CH_FRONT, st,
                  ch_gemm_nn<<<rowsg(m), 256, 0, st>>>(src, r, Rinv, m, r, r, dst));
      src = dst;
    }
    return GPTQ_OK;
  };
#define CH_TRY(x)                 \
  do {                            \
    const gptq_status _s = (x);   \
    if (_s != GPTQ_OK) return _s; \
  } while (0)
  if (r > 0) {
    GPTQ_LAUNCH(K_CH_FRONT, st,
                ch_scale_kernel<<<grid1(o * i), 256, 0, st>>>(W, ldw, o, i, sc, Wt, status));
    const dim3 gro(rowsg(o), (unsigned)cdiv(r, 8));
    GPTQ_LAUNCH(K_CH_FRONT, st, ch_rowdot_kernel<<<gro, 256, 0, st>>>(Wt, i, omega, o, i, r, Y));
    CH_TRY(orth(Y, o, Q));
    for (int it = 0; it < CH_NITER; ++it) {
      CH_TRY(gemm_tn(Wt, i, Q, o, i, Z));  // Z = W~^T Q [i x r]
      CH_TRY(orth(Z, i, Zq));
      GPTQ_LAUNCH(K_CH_FRONT, st, ch_rowdot_kernel<<<gro, 256, 0, st>>>(Wt, i, Zq, o, i, r, Y));
      CH_TRY(orth(Y, o, Q));
    }
    CH_TRY(gemm_tn(Wt, i, Q, o, i, Z));
    CH_TRY(gemm_tn(Z, r, Z, i, r, Mm));
    GPTQ_LAUNCH(K_CH_FRONT, st, ch_jacobi_kernel<<<1, 64, 0, st>>>(Mm, r, Uh, sig));
    GPTQ_LAUNCH(K_CH_FRONT, st, ch_gemm_nn<<<rowsg(o), 256, 0, st>>>(Q, r, Uh, o, r, r, Ul));
    GPTQ_LAUNCH(K_CH_FRONT, st, ch_gemm_nn<<<rowsg(i), 256, 0, st>>>(Z, r, Uh, i, r, r, Vz));
    GPTQ_LAUNCH(K_CH_FRONT, st,
                ch_factor_kernel<<<grid1(o * r + (int64_t)r * i), 256, 0, st>>>(Ul, Vz, sig, sc,
                                                                                o, i, r, A, B));
  }
#undef CH_TRY
  GPTQ_LAUNCH(K_CH_FRONT, st,
              ch_resid_kernel<<<dim3((unsigned)cdiv(i, 64), (unsigned)cdiv(o, 64)), 256, 0, st>>>(
                  W, ldw, o, i, A, B, r, Res, status));
  // U and perm are read from here on: with u_stream, wait for the work
  // enqueued on it before this call (the frontend above does not need U and
  // overlaps with it)
  if (u_stream && u_stream != stream) {
    hipEvent_t ev;
    GPTQ_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    hipError_t e1 = hipEventRecord(ev, (hipStream_t)u_stream);
    hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(st, ev, 0) : e1;
    hipError_t e3 = hipEventDestroy(ev);
    GPTQ_HIP(e2);
    GPTQ_HIP(e3);
  }
  if (perm) {
    GPTQ_LAUNCH(K_FILL, st, ch_zero_kernel<<<grid1(i), 256, 0, st>>>(cnt, i));
    GPTQ_LAUNCH(K_CH_FRONT, st,
                ch_perm_count_kernel<<<grid1(i), 256, 0, st>>>(perm, i, cnt, status));
    GPTQ_LAUNCH(K_CH_FRONT, st, ch_perm_check_kernel<<<grid1(i), 256, 0, st>>>(cnt, i, status));
  }
  const unsigned ngr = (unsigned)cdiv(o, group_size);
  const unsigned rt = (unsigned)cdiv(o, 64);
  for (int64_t j0 = 0; j0 < i; j0 += CH_QB) {
    const int bw = (int)std::min<int64_t>(CH_QB, i - j0);
    const double* cur = nullptr;  // the block's current values, after the first block
    if (j0 > 0) {
      const int64_t p0 = std::min<int64_t>(L.pmax, cdiv(j0, CH_KS));
      const int64_t ks = round_up(cdiv(j0, p0), 32);
      const int np = (int)cdiv(j0, ks);
      dim3 grid(rt, (unsigned)np);
      GPTQ_LAUNCH(K_CH_UPDATE, st,
                  ch_update_kernel<<<grid, 256, 0, st>>>(E, U, o, i, j0, bw, ks, part, L.pstride));
      // the pieces summed in piece order and taken from the residual, all
      // values at once, so that the sweep reads one value per entry
      GPTQ_LAUNCH(K_CH_UPDATE, st,
                  ch_cur_kernel<<<grid1(L.pstride), 256, 0, st>>>(part, np, L.pstride, Res, o, i,
                                                                  perm, j0, bw, psum));
      cur = psum;
    }
#define CH_SWEEP(GS)                                                                            \
  GPTQ_LAUNCH(K_CH_SWEEP, st,                                                                    \
              ch_sweep_rows_kernel<GS><<<ngr, 256, 0, st>>>(Res, o, i, j0, bw, cur, U, perm,      \
                                                             bits, E, codes, scales, zeros,      \
                                                             row_loss, status, fac))
    if (group_size == 32) CH_SWEEP(32);
    else if (group_size == 64) CH_SWEEP(64);
    else CH_SWEEP(128);
#undef CH_SWEEP
  }
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  return gptq_workspace_status(ws, stream);
}
