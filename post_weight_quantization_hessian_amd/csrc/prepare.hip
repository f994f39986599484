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
#include "gemm64.h"

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
__global__ __launch_bounds__(256) void prep_perm_kernel(const double* __restrict__ hd, int64_t n,
                                                        bool act, int32_t* __restrict__ perm) {
  __shared__ double tile[1024];
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!act) {
    if (k < n) perm[k] = (int32_t)k;
    return;
  }
  const double mine = k < n ? hd[k] : 0.0;
  int64_t rank = 0;
  for (int64_t j0 = 0; j0 < n; j0 += 1024) {
    const int64_t m = (n - j0) < 1024 ? (n - j0) : 1024;
    __syncthreads();
    for (int q = threadIdx.x; q < m; q += blockDim.x) tile[q] = hd[j0 + q];
    __syncthreads();
    if (k < n) {
      for (int q = 0; q < m; ++q) {
        const double v = tile[q];
        rank += (v > mine) || (v == mine && j0 + q < k);
      }
    }
  }
  if (k < n) perm[rank] = (int32_t)k;
}

// Lower triangle of K (ip x ip, ld ip): K[a][b] = H[p_a][p_b], p_x = perm[n-1-x],
// H = c*S + lam*I; the padding a, b >= n is the identity. One row per block.
__global__ __launch_bounds__(256) void prep_gather_kernel(const double* __restrict__ S, int64_t n,
                                                          int64_t ip, double c,
                                                          const double* __restrict__ lam_p,
                                                          const int32_t* __restrict__ perm,
                                                          double* __restrict__ K) {
  const int64_t a = blockIdx.x;
  const double lam = *lam_p;
  double* row = K + a * ip;
  if (a >= n) {
    for (int64_t b = threadIdx.x; b <= a; b += blockDim.x) row[b] = (a == b) ? 1.0 : 0.0;
    return;
  }
  const int64_t pa = perm[n - 1 - a];
  const double* srow = S + pa * n;
  for (int64_t b = threadIdx.x; b <= a; b += blockDim.x) {
    const int64_t pb = perm[n - 1 - b];
    double v = c * srow[pb];
    if (a == b) v += lam;
    row[b] = v;
  }
}

// ---------------------------------------------------------------- Cholesky

__device__ inline int pk(int i, int k) { return (i * (i + 1)) / 2 + k; }  // packed lower

// Factor the 128x128 diagonal block of panel p in LDS (right-looking), write
// L11 back, and its inverse (zeros above the diagonal) to Dinv. A pivot that
// is not positive and finite sets ST_NOTSPD and is replaced by 1.
__global__ __launch_bounds__(256) void chol_potrf_kernel(double* __restrict__ K, int64_t ld, int p,
                                                         double* __restrict__ Dinv,
                                                         unsigned* __restrict__ status) {
  __shared__ double Lp[GT * (GT + 1) / 2];
  __shared__ double Xp[GT * (GT + 1) / 2];
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int64_t c0 = (int64_t)p * GT;
  for (int e = t; e < GT * GT; e += 256) {
    const int i = e >> 7, k = e & 127;
    if (k <= i) Lp[pk(i, k)] = K[(c0 + i) * ld + c0 + k];
  }
  for (int e = t; e < GT * (GT + 1) / 2; e += 256) Xp[e] = 0.0;
  __syncthreads();
  bool bad = false;
  for (int j = 0; j < GT; ++j) {
    double d = Lp[pk(j, j)];
    if (!(d > 0.0) || !isfinite(d)) {
      bad = true;
      d = 1.0;
    }
    const double ljj = sqrt(d);
    for (int i = j + 1 + t; i < GT; i += 256) Lp[pk(i, j)] /= ljj;
    __syncthreads();
    if (t == 0) Lp[pk(j, j)] = ljj;
    const int n = GT - 1 - j;
    for (int r = ty; r < n; r += 16) {
      const int i = j + 1 + r;
      const double lij = Lp[pk(i, j)];
      for (int cc = tx; cc <= r; cc += 16) {
        const int k = j + 1 + cc;
        Lp[pk(i, k)] -= lij * Lp[pk(k, j)];
      }
    }
    __syncthreads();
  }
  // X = L^-1, right-looking: row i of X from the accumulated right-hand side,
  // then remove its contribution from the rows below.
  for (int i = 0; i < GT; ++i) {
    const double lii = Lp[pk(i, i)];
    for (int j = t; j <= i; j += 256) Xp[pk(i, j)] = ((j == i ? 1.0 : 0.0) + Xp[pk(i, j)]) / lii;
    __syncthreads();
    for (int r = ty; r < GT - 1 - i; r += 16) {
      const int m = i + 1 + r;
      const double lmi = Lp[pk(m, i)];
      for (int j = tx; j <= i; j += 16) Xp[pk(m, j)] -= lmi * Xp[pk(i, j)];
    }
    __syncthreads();
  }
  double* D = Dinv + (int64_t)p * GT * GT;
  for (int e = t; e < GT * GT; e += 256) {
    const int i = e >> 7, k = e & 127;
    if (k <= i) {
      K[(c0 + i) * ld + c0 + k] = Lp[pk(i, k)];
      D[e] = Xp[pk(i, k)];
    } else {
      D[e] = 0.0;
    }
  }
  if (bad && t == 0) atomicOr(status, ST_NOTSPD);
}

// L21 = A21 * Dinv^T for row block m below panel p (in place).
__global__ __launch_bounds__(256) void chol_trsm_kernel(double* __restrict__ K, int64_t ld, int p,
                                                        const double* __restrict__ Dinv) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int64_t c0 = (int64_t)p * GT;
  const int64_t r0 = c0 + GT + (int64_t)blockIdx.x * GT;
  LdTrans64 la{K + r0 * ld + c0, ld, {}};
  LdTrans64 lb{Dinv + (int64_t)p * GT * GT, GT, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, false, GT / GK, sA, sB, acc);
  for_each_acc(acc, [&](int r, int c, double v) { K[(r0 + r) * ld + c0 + c] = v; });
}

// Lower tiles of the trailing matrix: K22 -= L21 L21^T (tile (a, b), a >= b).
__global__ __launch_bounds__(256) void chol_syrk_kernel(double* __restrict__ K, int64_t ld, int p) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  int a = (int)((sqrt(8.0 * id + 1.0) - 1.0) * 0.5);
  while (a * (a + 1) / 2 > id) --a;
  while ((a + 1) * (a + 2) / 2 <= id) ++a;
  const int b = id - a * (a + 1) / 2;
  const int64_t c0 = (int64_t)p * GT, c1 = c0 + GT;
  const int64_t ra = c1 + (int64_t)a * GT, rb = c1 + (int64_t)b * GT;
  LdTrans64 la{K + ra * ld + c0, ld, {}};
  LdTrans64 lb{K + rb * ld + c0, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, a == b, GT / GK, sA, sB, acc);
  for_each_acc(acc, [&](int r, int c, double v) { K[(ra + r) * ld + rb + c] -= v; });
}

// ---------------------------------------------------------------- inverse

// Step i of the blocked right-looking inverse X = L^-1 (X in Xb, ld ip):
// X[i][j] = Dinv_i * B[i][j] for j < i (B accumulated in place), X[i][i] = Dinv_i.
__global__ __launch_bounds__(256) void trtri_row_kernel(double* __restrict__ Xb, int64_t ld, int i,
                                                        const double* __restrict__ Dinv) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int j = blockIdx.x;
  const double* D = Dinv + (int64_t)i * GT * GT;
  double* blk = Xb + (int64_t)i * GT * ld + (int64_t)j * GT;
  if (j == i) {
    for (int e = threadIdx.x; e < GT * GT; e += 256) blk[(e >> 7) * ld + (e & 127)] = D[e];
    return;
  }
  LdTrans64 la{D, GT, {}};
  LdDirect64 lb{blk, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, false, GT / GK, sA, sB, acc);
  for_each_acc(acc, [&](int r, int c, double v) { blk[r * ld + c] = v; });
}

// B[m][j] -= L[m][i] * X[i][j] for block rows m > i, block columns j <= i.
__global__ __launch_bounds__(256) void trtri_update_kernel(double* __restrict__ Xb,
                                                           const double* __restrict__ K, int64_t ld,
                                                           int i) {
  __shared__ double sA[2 * GCH];
  __shared__ double sB[2 * GCH];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int ncol = i + 1;
  const int m = i + 1 + id / ncol;
  const int j = id % ncol;
  LdTrans64 la{K + (int64_t)m * GT * ld + (int64_t)i * GT, ld, {}};
  LdDirect64 lb{Xb + (int64_t)i * GT * ld + (int64_t)j * GT, ld, {}};
  d4 acc[4][4];
  zero_acc(acc);
  gemm64_loop(la, lb, false, GT / GK, sA, sB, acc);
  double* blk = Xb + (int64_t)m * GT * ld + (int64_t)j * GT;
  for_each_acc(acc, [&](int r, int c, double v) { blk[r * ld + c] -= v; });
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

__global__ void fill_kernel(double* __restrict__ p, int64_t n, double v) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = v;
}

__global__ void zero_u32_kernel(unsigned* p) { *p = 0u; }

// ---------------------------------------------------------------- layout

struct PrepLayout {
  int64_t n, ip, nt;
  size_t off_status, off_lam, off_hd, off_K, off_X, off_D, total;
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
  L.off_D = take(8 * (size_t)L.nt * GT * GT);
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
  if (flags & ~GPTQ_FLAG_ACT_ORDER) return GPTQ_EINVAL;
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
  double* Dinv = (double*)(base + L.off_D);
  const int64_t n = in_features, ip = L.ip;
  const int nt = (int)L.nt;
  const double c = 2.0 / (double)n_tokens_total;

  GPTQ_LAUNCH(K_FILL, st, zero_u32_kernel<<<1, 1, 0, st>>>(status));
  GPTQ_LAUNCH(K_PREP_DIAG, st, prep_diag_kernel<<<1, 1024, 0, st>>>(S, n, c, damp, hd, lam));
  GPTQ_LAUNCH(K_PREP_PERM, st,
              prep_perm_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(
                  hd, n, (flags & GPTQ_FLAG_ACT_ORDER) != 0, perm));
  GPTQ_LAUNCH(K_PREP_GATHER, st,
              prep_gather_kernel<<<(unsigned)ip, 256, 0, st>>>(S, n, ip, c, lam, perm, K));
  for (int p = 0; p < nt; ++p) {
    GPTQ_LAUNCH(K_CHOL_POTRF, st, chol_potrf_kernel<<<1, 256, 0, st>>>(K, ip, p, Dinv, status));
    const int mt = nt - 1 - p;
    if (mt > 0) {
      GPTQ_LAUNCH(K_CHOL_TRSM, st, chol_trsm_kernel<<<mt, 256, 0, st>>>(K, ip, p, Dinv));
      GPTQ_LAUNCH(K_CHOL_SYRK, st, chol_syrk_kernel<<<mt * (mt + 1) / 2, 256, 0, st>>>(K, ip, p));
    }
  }
  {
    const int64_t cnt = ip * ip;
    GPTQ_LAUNCH(K_FILL, st,
                fill_kernel<<<(unsigned)std::min<int64_t>(cdiv(cnt, 256), 65535 * 4), 256, 0, st>>>(
                    Xb, cnt, 0.0));
  }
  for (int i = 0; i < nt; ++i) {
    GPTQ_LAUNCH(K_TRTRI_ROW, st, trtri_row_kernel<<<i + 1, 256, 0, st>>>(Xb, ip, i, Dinv));
    if (i + 1 < nt) {
      const int nb = (nt - 1 - i) * (i + 1);
      GPTQ_LAUNCH(K_TRTRI_UPDATE, st, trtri_update_kernel<<<nb, 256, 0, st>>>(Xb, K, ip, i));
    }
  }
  {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)std::min<int64_t>(n, 65535));
    GPTQ_LAUNCH(K_PREP_UOUT, st, prep_uout_kernel<<<grid, 256, 0, st>>>(Xb, ip, n, U));
  }
  unsigned h_status = 0;
  GPTQ_HIP(hipMemcpyAsync(&h_status, status, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  if (h_status & ST_NOTSPD) return GPTQ_ENOTSPD;
  return GPTQ_OK;
}
