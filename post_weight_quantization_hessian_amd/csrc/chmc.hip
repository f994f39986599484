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
constexpr int CH_RP = 2;      // rows per lane in the residual sweep (1 and 4 measured slower)

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

// Res[row][j] = W[row][j] - sum_k A[row][k] B[k][j] (fp64 from the fp16 values).
__global__ void ch_resid_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t o, int64_t i,
                                const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                int r, double* __restrict__ Res, unsigned* __restrict__ status) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < o * i;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / i, j = e - row * i;
    double acc = 0.0;
    for (int k = 0; k < r; ++k)
      acc = fma(f16_to_f64(A[row * r + k]), f16_to_f64(B[k * i + j]), acc);
    const double v = f16_to_f64(W[row * ldw + j]) - acc;
    if (!isfinite(v)) atomicOr(status, ST_NONFINITE);
    Res[e] = v;
  }
}

// Lazy update of the block [j0, j0 + bw) (sweep order) over the errors of
// columns [k_lo, k_hi), k_lo = blockIdx.y * ks, k_hi <= j0:
//   part[y][row][c] = sum_k E[row][k] U[k][j0 + c]    (c < 128; 0 beyond bw)
// A workgroup forms 64 rows x 128 columns, thread (ty, tx) the rows 4 ty..4 ty+3
// and the columns tx + 16 b, through 16-deep LDS stages of E and U.
__global__ __launch_bounds__(256) void ch_update_kernel(const double* __restrict__ E,
                                                        const float* __restrict__ U,
                                                        int64_t rows, int64_t cols, int64_t j0,
                                                        int bw, int64_t ks,
                                                        double* __restrict__ part,
                                                        int64_t pstride) {
  __shared__ double Es[16][64];
  __shared__ float Us[16][CH_QB];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t k_lo = (int64_t)blockIdx.y * ks;
  const int64_t k_hi = k_lo + ks < j0 ? k_lo + ks : j0;
  double acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += 16) {
    {
      const int rr = t >> 2, kk = (t & 3) * 4;
      const int64_t row = r0 + rr;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int64_t k = k0 + kk + x;
        Es[kk + x][rr] = (row < rows && k < k_hi) ? E[row * cols + k] : 0.0;
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
      for (int a = 0; a < 4; ++a) e[a] = Es[kk][ty * 4 + a];
#pragma unroll
      for (int b = 0; b < 8; ++b) u[b] = (double)Us[kk][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = fma(e[a], u[b], acc[a][b]);
    }
    __syncthreads();
  }
  double* out = part + (int64_t)blockIdx.y * pstride;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t row = r0 + ty * 4 + a;
    if (row < rows)
#pragma unroll
      for (int b = 0; b < 8; ++b) out[row * CH_QB + tx + 16 * b] = acc[a][b];
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
// channels (rows) and column: one workgroup of 8 G / RP threads per group;
// thread (row set lr = t / 8, slice cs = t % 8) holds the columns 8 s + cs
// (s < 16) of its RP rows lr RP .. lr RP + RP - 1, starting from
// Res[row][perm[j]] minus the np update sums. For column jj = 8 s + c
// the owners are the lanes with cs = c: each wave reduces its rows' range
// with lane shuffles and one barrier joins the wave ranges; every owner
// quantizes its own rows, and their scaled errors reach the other slices of
// the rows by a shuffle among the 8 lanes, which subtract error * U[jj][col]
// from their later columns. The grid arithmetic is the same in every wave,
// so fewer, fuller waves (RP rows per lane) issue less of it; the step and
// U[jj][jj] enter as reciprocals (one division per column each, the latter
// off the row chain), as in the GPTQ sweep. Codes, errors
// and grids stay in registers until the block is done; codes and grids go
// to the original column perm[j], the errors to E in sweep order, the
// squared errors to row_loss (set on the first block).
template <int G, int RP>
__global__ __launch_bounds__(8 * G / RP) void ch_sweep_kernel(
    const double* __restrict__ Res, int64_t rows, int64_t cols, int64_t j0, int bw,
    const double* __restrict__ part, int np, int64_t pstride, const float* __restrict__ U,
    const int32_t* __restrict__ perm, int bits, double* __restrict__ E,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
    double* __restrict__ row_loss, unsigned* __restrict__ status) {
  constexpr int NT = 8 * G / RP, NW = NT / 64;
  static_assert(NT % 64 == 0, "whole waves");
  __shared__ float Us[CH_QB][CH_QB + 1];
  __shared__ double mm[2][2][NW];
  const int t = threadIdx.x, cs = t & 7, lr = t >> 3, wv = t >> 6, lane = t & 63;
  const int64_t grp = blockIdx.x;
  const int64_t row0 = grp * G + (int64_t)lr * RP;
  bool rv[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) rv[p] = row0 + p < rows;
  const double maxq = (double)((1 << bits) - 1);
  const double rmaxq = 1.0 / maxq;
  for (int e = t; e < CH_QB * CH_QB; e += NT) {
    const int a = e >> 7, b = e & 127;
    Us[a][b] = (a < bw && b < bw) ? U[(j0 + a) * cols + j0 + b] : 0.0f;
  }
  double w[RP][16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int col = 8 * s + cs;
    int64_t oc = 0;
    if (col < bw) {
      oc = perm ? (int64_t)perm[j0 + col] : j0 + col;
      if (oc < 0 || oc >= cols) oc = 0;  // reported as ST_BADPERM before the sweep
    }
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      double v = 0.0;
      if (col < bw && rv[p]) {
        const int64_t row = row0 + p;
        v = Res[row * cols + oc];
        for (int q = 0; q < np; ++q) v -= part[(int64_t)q * pstride + row * CH_QB + col];
      }
      w[p][s] = v;
    }
  }
  uint32_t kq[RP][4];                          // codes of the own columns, 8 bits each
  uint32_t sb[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // their fp16 steps
  uint32_t zb[4] = {0u, 0u, 0u, 0u};          // their zero points
  double lsum[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    lsum[p] = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) kq[p][q] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    for (int c = 0; c < 8; ++c) {
      const int jj = 8 * s + c;
      if (jj >= bw) break;  // uniform
      const bool own = cs == c;
      const double rd = 1.0 / (double)Us[jj][jj];  // off the chain: depends on jj only
      double mn = 0.0, mx = 0.0;  // the range includes 0
#pragma unroll
      for (int p = 0; p < RP; ++p)
        if (own && rv[p]) {
          mn = fmin(mn, w[p][s]);
          mx = fmax(mx, w[p][s]);
        }
#pragma unroll
      for (int off = 8; off < 64; off <<= 1) {
        mn = fmin(mn, __shfl_xor(mn, off, 64));
        mx = fmax(mx, __shfl_xor(mx, off, 64));
      }
      const int buf = jj & 1;
      if (lane == c) {
        mm[buf][0][wv] = mn;
        mm[buf][1][wv] = mx;
      }
      __syncthreads();
      mn = mm[buf][0][0];
      mx = mm[buf][1][0];
#pragma unroll
      for (int k = 1; k < NW; ++k) {
        mn = fmin(mn, mm[buf][0][k]);
        mx = fmax(mx, mm[buf][1][k]);
      }
      double scale = f16_round_f64((mx - mn) * rmaxq), zero = 0.0;
      if (!(scale <= 65504.0) && t == 0) atomicOr(status, ST_NONFINITE);
      const bool degen = mx == mn || scale == 0.0;
      if (degen) scale = 1.0;
      const double rs = 1.0 / scale;
      if (!degen) zero = fmin(fmax(rint(-mn * rs), 0.0), maxq);
      double e[RP];
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        e[p] = 0.0;
        if (own) {
          const double v = w[p][s];
          const double k = fmin(fmax(rint(v * rs) + zero, 0.0), maxq);
          if (rv[p]) e[p] = (v - scale * (k - zero)) * rd;
          kq[p][s >> 2] |= (uint32_t)k << (8 * (s & 3));
          w[p][s] = e[p];
          lsum[p] = fma(e[p], e[p], lsum[p]);
        }
      }
      if (own) {
        sb[s >> 1] |= (uint32_t)f16_bits_of_exact(scale) << (16 * (s & 1));
        zb[s >> 2] |= (uint32_t)zero << (8 * (s & 3));
      }
      const int src = (lane & ~7) | c;
      double eb[RP];
#pragma unroll
      for (int p = 0; p < RP; ++p) eb[p] = __shfl(e[p], src, 64);
      if (cs > c) {
        const double u = (double)Us[jj][8 * s + cs];
#pragma unroll
        for (int p = 0; p < RP; ++p) w[p][s] -= eb[p] * u;
      }
#pragma unroll
      for (int s2 = s + 1; s2 < 16; ++s2) {
        const double u = (double)Us[jj][8 * s2 + cs];
#pragma unroll
        for (int p = 0; p < RP; ++p) w[p][s2] -= eb[p] * u;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int col = 8 * s + cs;
    if (col < bw) {
      int64_t oc = perm ? (int64_t)perm[j0 + col] : j0 + col;
      if (oc < 0 || oc >= cols) oc = 0;
#pragma unroll
      for (int p = 0; p < RP; ++p)
        if (rv[p]) {
          const int64_t row = row0 + p;
          codes[row * cols + oc] = (uint8_t)(kq[p][s >> 2] >> (8 * (s & 3)));
          E[row * cols + j0 + col] = w[p][s];
        }
      if (lr == 0) {
        scales[grp * cols + oc] = (uint16_t)(sb[s >> 1] >> (16 * (s & 1)));
        zeros[grp * cols + oc] = f64_to_f16_rne((double)((zb[s >> 2] >> (8 * (s & 3))) & 0xff));
      }
    }
  }
  // each row's loss: its 8 slices in a fixed order
#pragma unroll
  for (int p = 0; p < RP; ++p) {
    double l = lsum[p];
    l += __shfl_xor(l, 1, 64);
    l += __shfl_xor(l, 2, 64);
    l += __shfl_xor(l, 4, 64);
    if (cs == 0 && rv[p]) row_loss[row0 + p] = (j0 == 0 ? 0.0 : row_loss[row0 + p]) + l;
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
  if (flags & ~GPTQ_FLAG_NO_SYNC) return GPTQ_EINVAL;
  if (rows <= 0 || cols <= 0 || n_tokens <= 0) return GPTQ_EINVAL;
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
              ch_resid_kernel<<<grid1(o * i), 256, 0, st>>>(W, ldw, o, i, A, B, r, Res, status));
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
    int np = 0;
    const double* upd = part;
    if (j0 > 0) {
      const int64_t p0 = std::min<int64_t>(L.pmax, cdiv(j0, CH_KS));
      const int64_t ks = round_up(cdiv(j0, p0), 32);
      np = (int)cdiv(j0, ks);
      dim3 grid(rt, (unsigned)np);
      GPTQ_LAUNCH(K_CH_UPDATE, st,
                  ch_update_kernel<<<grid, 256, 0, st>>>(E, U, o, i, j0, bw, ks, part, L.pstride));
      // the pieces summed in piece order, all values at once, so that the
      // sweep reads one update per value
      if (np > 1) {
        GPTQ_LAUNCH(K_CH_UPDATE, st,
                    ch_sum_kernel<<<grid1(L.pstride), 256, 0, st>>>(part, np, L.pstride, psum));
        upd = psum;
        np = 1;
      }
    }
#define CH_SWEEP(GS)                                                                            \
  GPTQ_LAUNCH(K_CH_SWEEP, st,                                                                    \
              ch_sweep_kernel<GS, CH_RP><<<ngr, 8 * GS / CH_RP, 0, st>>>(Res, o, i, j0, bw, upd, np, L.pstride, \
                                                         U, perm, bits, E, codes, scales, zeros, \
                                                         row_loss, status))
    if (group_size == 32) CH_SWEEP(32);
    else if (group_size == 64) CH_SWEEP(64);
    else CH_SWEEP(128);
#undef CH_SWEEP
  }
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  return gptq_workspace_status(ws, stream);
}
