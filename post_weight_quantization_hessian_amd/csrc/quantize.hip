// Steps 4-6: the column sweep (CHMC article, Methodik, Schritt 2: round each
// column to its group's grid, err_j = (col_j - q_j)/U[j,j], later columns -=
// err_j * U[j, j+1:]; The Geometry of LLM Quantization 2.2: this is Babai's
// nearest-plane step).
//
// Lazy blocks of 128 columns, with the update of earlier blocks applied just
// in time: before block [j0, j0+bw) is swept, its current values are
//     W~[:, blk] = W[:, blk] - E[:, :j0] * U[:j0, blk]
// (E = the scaled errors of all earlier columns), the same sums as the
// right-looking update, formed once per block by an fp32-MFMA GEMM whose
// K-chunks are accumulated in fp64. Inside the block the sweep runs in fp64
// registers: 4 lanes per row, lane q of a quad owns columns q, q+4, q+8, ...;
// the register window shifts by one slot every 4 columns so the live column
// is always slot 0, and the scaled error of the live column is broadcast to
// the quad with a DPP quad permute. Group min/max reductions also use DPP.
#include "common.h"

namespace gptq {

constexpr int QB = 128;  // sweep block width
typedef double dbl2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers

template <int CTRL>
__device__ inline double dpp_f64(double v) {
  union { double d; int i[2]; } a, b;
  a.d = v;
  b.i[0] = __builtin_amdgcn_update_dpp(0, a.i[0], CTRL, 0xF, 0xF, false);
  b.i[1] = __builtin_amdgcn_update_dpp(0, a.i[1], CTRL, 0xF, 0xF, false);
  return b.d;
}
// quad_perm controls: broadcast lane q of the quad; xor 1; xor 2
template <int Q>
__device__ inline double quad_bcast(double v) { return dpp_f64<Q * 0x55>(v); }
__device__ inline double quad_xor1(double v) { return dpp_f64<0xB1>(v); }
__device__ inline double quad_xor2(double v) { return dpp_f64<0x4E>(v); }

// ---------------------------------------------------------------- small kernels

// row_loss = 0; invperm = -1 (filled by the permute kernel); g_idx[m] = m / gs
// when there is no permutation (else written by finalize).
__global__ void q_init_kernel(double* __restrict__ row_loss, int64_t rows,
                              const int32_t* __restrict__ perm, int32_t* __restrict__ invperm,
                              int32_t* __restrict__ g_idx, int64_t cols, int gs,
                              unsigned* __restrict__ status) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  if (tid == 0) *status = 0u;
  for (int64_t r = tid; r < rows; r += nthr) row_loss[r] = 0.0;
  for (int64_t k = tid; k < cols; k += nthr) {
    if (perm) invperm[k] = -1;
    else if (g_idx) g_idx[k] = (int32_t)(k / gs);
  }
}

// Wp[r][k] = W[r][perm[k]] (sweep order, ld cols); invperm[perm[k]] = k.
// An entry of perm outside [0, cols) is reported (ST_BADPERM) and skipped.
__global__ __launch_bounds__(256) void q_permute_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                        const int32_t* __restrict__ perm,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t* __restrict__ Wp,
                                                        int32_t* __restrict__ invperm,
                                                        unsigned* __restrict__ status) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint16_t* src = W + r * ldw;
    uint16_t* dst = Wp + r * cols;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < cols;
         k += (int64_t)gridDim.x * blockDim.x) {
      const int64_t pk = perm[k];
      if (pk < 0 || pk >= cols) {
        if (r == 0) atomicOr(status, ST_BADPERM);
        dst[k] = 0;
        continue;
      }
      dst[k] = src[pk];
      if (r == 0) invperm[pk] = (int32_t)k;
    }
  }
}

// codes[r][m] = codes_s[r][invperm[m]]; g_idx[m] = invperm[m] / gs. An unset
// invperm entry (perm was not a permutation) is reported and gives code 0.
__global__ __launch_bounds__(256) void q_finalize_kernel(const uint8_t* __restrict__ codes_s,
                                                         const int32_t* __restrict__ invperm,
                                                         int64_t rows, int64_t cols, int gs,
                                                         uint8_t* __restrict__ codes,
                                                         int32_t* __restrict__ g_idx,
                                                         unsigned* __restrict__ status) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < cols;
         m += (int64_t)gridDim.x * blockDim.x) {
      const int32_t k = invperm[m];
      if (k < 0 || k >= cols) {
        if (r == 0) atomicOr(status, ST_BADPERM);
        codes[r * cols + m] = 0;
        continue;
      }
      codes[r * cols + m] = codes_s[r * cols + k];
      if (r == 0 && g_idx) g_idx[m] = k / gs;
    }
  }
}

// ---------------------------------------------------------------- update GEMM
//
// part[p][r][c] = sum_{l in split p} E[r][l] * U[l][j0 + c], l < j0, c < 128.
// Workgroup tile: 64 rows x 128 columns; wave w owns columns 32w..32w+31 as
// two 32x32 v_mfma_f32_32x32x2f32 tiles (rows 0-31, 32-63). Each 32-wide K
// chunk is summed in fp32 by the MFMA, then added into fp64 accumulators.
//
// v_mfma_f32_32x32x2f32 layout (lane l): A[m][k]: m = l%32, k = l/32;
// B[k][n]: n = l%32, k = l/32; D reg x: row 8*(x/4) + 4*(l/32) + x%4, col l%32.
constexpr int QE_LD = 34;   // Es row pitch (floats)
constexpr int QU_LD = 160;  // Us row pitch (floats)

__global__ __launch_bounds__(256) void q_gemm_kernel(const float* __restrict__ E, int64_t lde,
                                                     const float* __restrict__ U, int64_t ldu,
                                                     const uint16_t* __restrict__ W, int64_t ldw,
                                                     int64_t rows, int64_t j0, int bw,
                                                     int64_t ksplit, double* __restrict__ part,
                                                     int64_t part_stride,
                                                     double* __restrict__ wblk, bool vecU) {
  __shared__ float Es[2][64 * QE_LD];
  __shared__ float Us[2][32 * QU_LD];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int p = blockIdx.y;
  const int64_t k_lo = (int64_t)p * ksplit;
  int64_t k_hi = k_lo + ksplit;
  if (k_hi > j0) k_hi = j0;
  const int nchunks = k_hi > k_lo ? (int)((k_hi - k_lo) / 32) : 0;

  // E loader: row t>>2, 8 floats at (t&3)*8; U loader: row t>>3, 16 floats at (t&7)*16
  const int er = t >> 2, ec = (t & 3) * 8;
  const int ur = t >> 3, uc = (t & 7) * 16;
  f4 eR[2], uR[4];
  auto fetch = [&](int c) {
    const int64_t l0 = k_lo + (int64_t)c * 32;
    if (r0 + er < rows) {
      const float* pe = E + (r0 + er) * lde + l0 + ec;
      eR[0] = *reinterpret_cast<const f4*>(pe);
      eR[1] = *reinterpret_cast<const f4*>(pe + 4);
    } else {
      eR[0] = f4{0, 0, 0, 0};
      eR[1] = f4{0, 0, 0, 0};
    }
    const float* pu = U + (l0 + ur) * ldu + j0 + uc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = uc + 4 * q;
      if (vecU && cc + 3 < bw) {
        uR[q] = *reinterpret_cast<const f4*>(pu + 4 * q);
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) uR[q][x] = (cc + x < bw) ? pu[4 * q + x] : 0.0f;
      }
    }
  };
  auto store = [&](int buf) {
    float* se = &Es[buf][er * QE_LD + ec];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      se[x] = eR[0][x];
      se[4 + x] = eR[1][x];
    }
    float* su = &Us[buf][ur * QU_LD + uc];
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<f4*>(su + 4 * q) = uR[q];
  };

  f16 acc[2];
  double acc64[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      acc[i][x] = 0.0f;
      acc64[i][x] = 0.0;
    }

  if (nchunks > 0) {
    fetch(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const int cur = c & 1;
      const bool more = c + 1 < nchunks;
      if (more) fetch(c + 1);
      const float* es = Es[cur];
      const float* us = Us[cur];
#pragma unroll
      for (int kk = 0; kk < 32; kk += 2) {
        const int k = kk + (lane >> 5);
        const float a0 = es[(lane & 31) * QE_LD + k];
        const float a1 = es[(32 + (lane & 31)) * QE_LD + k];
        const float b = us[k * QU_LD + w * 32 + (lane & 31)];
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc[1], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          acc64[i][x] += (double)acc[i][x];
          acc[i][x] = 0.0f;
        }
      if (more) store(cur ^ 1);
      __syncthreads();
    }
  }
  const int P = gridDim.y;
  const int col = w * 32 + (lane & 31);
  if (P == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int64_t row = r0 + 32 * i + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
        if (row < rows && col < bw)
          wblk[row * QB + col] = f16_to_f64(W[row * ldw + j0 + col]) - acc64[i][x];
      }
    return;
  }
  double* Pp = part + (int64_t)p * part_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int64_t row = r0 + 32 * i + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
      if (row < rows) Pp[row * QB + col] = acc64[i][x];
    }
}

// wblk = W[:, blk] - sum_p part[p] for the split-K partials, summed in split
// order (reproducible). Two adjacent columns per thread.
__global__ __launch_bounds__(256) void q_reduce_kernel(const double* __restrict__ part, int P,
                                                       int64_t part_stride,
                                                       const uint16_t* __restrict__ W, int64_t ldw,
                                                       int64_t rows, int64_t j0, int bw,
                                                       double* __restrict__ wblk) {
  const int64_t e2 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // pair index
  const int64_t row = e2 / (QB / 2);
  const int c = (int)(e2 % (QB / 2)) * 2;
  if (row >= rows) return;
  const int64_t off = row * QB + c;
  dbl2_t sum = {0.0, 0.0};
  for (int q = 0; q < P; q += 4) {
    dbl2_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = q + u < P ? *reinterpret_cast<const dbl2_t*>(part + (int64_t)(q + u) * part_stride + off)
                       : dbl2_t{0.0, 0.0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u < P) {
        sum.x += v[u].x;
        sum.y += v[u].y;
      }
  }
  const uint16_t* wr = W + row * ldw + j0;
  if (c < bw) wblk[off] = f16_to_f64(wr[c]) - sum.x;
  if (c + 1 < bw) wblk[off + 1] = f16_to_f64(wr[c + 1]) - sum.y;
}

// ---------------------------------------------------------------- sweep
//
// One block of columns [j0, j0+bw). 16 rows per wave (4 lanes per row).
template <int GS>
__global__ __launch_bounds__(256) void q_sweep_kernel(
    const uint16_t* __restrict__ W, int64_t ldw, const double* __restrict__ wblk,
    const float* __restrict__ U, int64_t ldu, bool vecU, int64_t rows, int64_t j0, int bw,
    int bits, float* __restrict__ E, int64_t lde, uint8_t* __restrict__ codes, int64_t ldc,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t ldg,
    double* __restrict__ row_loss, unsigned* __restrict__ status) {
  // U slab plus one zero row of padding: slot addresses run up to 3 columns
  // past the end of a row (into the next row or the padding) for slots that
  // are past the block end and never used.
  __shared__ double Us[QB * QB + QB];
  __shared__ double rdiag[QB];  // 1 / U[j][j]
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int q4 = lane & 3;
  const int nthr = blockDim.x;
  const int64_t r = (int64_t)blockIdx.x * (nthr >> 2) + wv * 16 + (lane >> 2);
  const bool rv = r < rows;
  const double maxq = (double)((1 << bits) - 1);

  // U slab of this block; U is zero below its diagonal. Zero outside [0, bw).
  if (vecU && bw == QB) {
    for (int e0 = 0; e0 < QB * QB / 4; e0 += 8 * nthr) {
      f4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * nthr + t;  // float4 index
        const int a = e >> 5, c4 = (e & 31) * 4;
        v[u] = e < QB * QB / 4 ? *reinterpret_cast<const f4*>(U + (j0 + a) * ldu + j0 + c4)
                               : f4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * nthr + t;
        if (e < QB * QB / 4) {
#pragma unroll
          for (int x = 0; x < 4; ++x) Us[e * 4 + x] = (double)v[u][x];
        }
      }
    }
  } else {
    for (int e = t; e < QB * QB; e += nthr) {
      const int a = e >> 7, c = e & 127;
      Us[e] = (a < bw && c < bw && c >= a) ? (double)U[(j0 + a) * ldu + j0 + c] : 0.0;
    }
  }

  for (int j = t; j < QB; j += nthr) {
    rdiag[j] = j < bw ? 1.0 / (double)U[(j0 + j) * ldu + j0 + j] : 0.0;
    Us[QB * QB + j] = 0.0;
  }

  // Current values of this row's columns: W - E[:, :j0] U[:j0, blk], formed by
  // the update GEMM (wblk); the first block reads the weights directly.
  double w[32];
  bool finite = true;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int c = 4 * s + q4;
    double v = 0.0;
    if (rv && c < bw) {
      if (wblk) {
        v = wblk[r * QB + c];
      } else {
        v = f16_to_f64(W[r * ldw + j0 + c]);
      }
      finite = finite && isfinite(v);
    }
    w[s] = v;
  }
  if (!finite) atomicOr(status, ST_NONFINITE);
  __syncthreads();

  double scale = 1.0, rscale = 1.0, zero = 0.0, loss = 0.0;
  const int nt4 = (bw + 3) >> 2;
  for (int tt = 0; tt < nt4; ++tt) {
    if (((4 * tt) % GS) == 0) {
      // grid of the group starting here, from the current values
      double mn = 0.0, mx = 0.0;
#pragma unroll
      for (int s = 0; s < GS / 4; ++s) {
        if (4 * (tt + s) + q4 < bw) {
          mn = fmin(mn, w[s]);
          mx = fmax(mx, w[s]);
        }
      }
      mn = fmin(mn, quad_xor1(mn));
      mx = fmax(mx, quad_xor1(mx));
      mn = fmin(mn, quad_xor2(mn));
      mx = fmax(mx, quad_xor2(mx));
      uint16_t sh = f64_to_f16_rne((mx - mn) / maxq);
      scale = f16_to_f64(sh);
      if ((sh & 0x7fff) >= 0x7c00 && rv) atomicOr(status, ST_NONFINITE);
      if (mx == mn || scale == 0.0) {
        scale = 1.0;
        sh = 0x3c00;
        zero = 0.0;
      } else {
        zero = fmin(fmax(rint(-mn / scale), 0.0), maxq);
      }
      rscale = 1.0 / scale;
      if (rv && q4 == 0) {
        const int64_t g = (j0 + 4 * tt) / GS;
        scales[r * ldg + g] = sh;
        zeros[r * ldg + g] = f64_to_f16_rne(zero);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * tt + jj;
      if (j < bw) {
        // quantize slot 0 (meaningful on the owner lane q4 == jj)
        const double v = w[0];
        double qf = rint(v * rscale) + zero;
        qf = fmin(fmax(qf, 0.0), maxq);
        const double dq = scale * (qf - zero);
        const double e = (v - dq) * rdiag[j];
        double eb;
        if (jj == 0) eb = quad_bcast<0>(e);
        else if (jj == 1) eb = quad_bcast<1>(e);
        else if (jj == 2) eb = quad_bcast<2>(e);
        else eb = quad_bcast<3>(e);
        if (q4 == jj && rv) {
          codes[r * ldc + j0 + j] = (uint8_t)qf;
          E[r * lde + j0 + j] = (float)e;
          loss += e * e;
        }
        // Slot s holds column 4*(tt+s) + q4; slots past the block end are never
        // used again. Whole groups of 8 such slots are skipped (uniform tests);
        // inside a group the reads run past the row end into the next row or
        // the padding, which only feeds dead slots.
        const double* urow = Us + j * QB + 4 * tt + q4;
        {
          const double u0 = urow[0];
          const double nv = w[0] - eb * u0;
          w[0] = q4 > jj ? nv : w[0];
        }
#pragma unroll
        for (int s = 1; s < 8; ++s) w[s] -= eb * urow[4 * s];
        if (tt < 24) {
#pragma unroll
          for (int s = 8; s < 16; ++s) w[s] -= eb * urow[4 * s];
        }
        if (tt < 16) {
#pragma unroll
          for (int s = 16; s < 24; ++s) w[s] -= eb * urow[4 * s];
        }
        if (tt < 8) {
#pragma unroll
          for (int s = 24; s < 32; ++s) w[s] -= eb * urow[4 * s];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 31; ++s) w[s] = w[s + 1];
    w[31] = 0.0;
  }
  loss += quad_xor1(loss);
  loss += quad_xor2(loss);
  if (rv && q4 == 0) row_loss[r] += loss;
}

// ---------------------------------------------------------------- layout

struct QLayout {
  int64_t rows, cols, lde, ng;
  int pmax;
  size_t off_status, off_invperm, off_wp, off_codes, off_E, off_part, off_wblk, total;
};

// Split-K factor of the update GEMM: about 512 workgroups in total.
static int q_pmax(int64_t rows) {
  const int64_t rt = cdiv(rows, 64);
  int64_t p = cdiv(512, rt);
  if (p > 16) p = 16;
  if (p < 1) p = 1;
  return (int)p;
}

static QLayout q_layout(int64_t rows, int64_t cols, int gs) {
  QLayout L;
  L.rows = rows;
  L.cols = cols;
  L.lde = round_up(cols, QB);
  L.ng = cdiv(cols, gs);
  L.pmax = q_pmax(rows);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = (size_t)round_up((int64_t)(o + bytes), 256);
    return at;
  };
  L.off_status = take(4);
  L.off_invperm = take(4 * (size_t)cols);
  L.off_wp = take(2 * (size_t)rows * cols);
  L.off_codes = take((size_t)rows * cols);
  L.off_E = take(4 * (size_t)rows * L.lde);
  L.off_part = take(8 * (size_t)L.pmax * rows * QB);
  L.off_wblk = take(8 * (size_t)rows * QB);
  L.total = o;
  return L;
}

template <int GS>
static gptq_status launch_sweep(hipStream_t st, int nw, const uint16_t* Wsrc, int64_t ldws,
                                const double* wblk, const float* U, int64_t cols, bool vecU,
                                int64_t rows, int64_t j0, int bw, int bits, float* E, int64_t lde,
                                uint8_t* codes, int64_t ldc, uint16_t* scales, uint16_t* zeros,
                                int64_t ldg, double* row_loss, unsigned* status) {
  const unsigned nblk = (unsigned)cdiv(rows, 16 * nw);
  GPTQ_LAUNCH(K_Q_SWEEP, st,
              q_sweep_kernel<GS><<<nblk, 64 * nw, 0, st>>>(Wsrc, ldws, wblk, U, cols, vecU, rows,
                                                           j0, bw, bits, E, lde, codes, ldc,
                                                           scales, zeros, ldg, row_loss, status));
  return GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

static bool valid_gs(int gs) { return gs == 16 || gs == 32 || gs == 64 || gs == 128; }

extern "C" size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t cols, int group_size) {
  if (rows <= 0 || cols <= 0 || !valid_gs(group_size)) return 0;
  return q_layout(rows, cols, group_size).total;
}

extern "C" gptq_status gptq_quantize_layer(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                           const float* U, const int32_t* perm, int bits,
                                           int group_size, uint8_t* codes, uint16_t* scales,
                                           uint16_t* zeros, int32_t* g_idx, double* row_loss,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || cols < 0) return GPTQ_EINVAL;
  if (bits < 2 || bits > 8 || !valid_gs(group_size)) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros || !row_loss || ldw < cols) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 20 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  const QLayout L = q_layout(rows, cols, group_size);
  if (!ws || ws_bytes < L.total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  unsigned* status = (unsigned*)(base + L.off_status);
  int32_t* invperm = (int32_t*)(base + L.off_invperm);
  uint16_t* Wp = (uint16_t*)(base + L.off_wp);
  uint8_t* codes_s = (uint8_t*)(base + L.off_codes);
  float* E = (float*)(base + L.off_E);
  double* part = (double*)(base + L.off_part);
  const int64_t pstride = rows * QB;

  {
    const int64_t n = rows > cols ? rows : cols;
    const unsigned nb = (unsigned)std::min<int64_t>(cdiv(n, 256), 4096);
    GPTQ_LAUNCH(K_Q_INIT, st,
                q_init_kernel<<<nb, 256, 0, st>>>(row_loss, rows, perm, invperm, g_idx, cols,
                                                  group_size, status));
  }
  const uint16_t* Wsrc = W;
  int64_t ldws = ldw;
  uint8_t* csw = codes;  // sweep-order codes
  if (perm) {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(cols, 256), 16),
              (unsigned)std::min<int64_t>(rows, 65535));
    GPTQ_LAUNCH(K_Q_PERMUTE, st,
                q_permute_kernel<<<grid, 256, 0, st>>>(W, ldw, perm, rows, cols, Wp, invperm,
                                                       status));
    Wsrc = Wp;
    ldws = cols;
    csw = codes_s;
  }
  const int nw = 4;
  const bool vecU = (cols % 4 == 0) && ((uintptr_t)U % 16 == 0);
  const int64_t rt = cdiv(rows, 64);
  double* wblk = (double*)(base + L.off_wblk);
  for (int64_t j0 = 0; j0 < cols; j0 += QB) {
    const int bw = (int)std::min<int64_t>(QB, cols - j0);
    const double* cur = nullptr;
    if (j0 > 0) {
      int64_t p = L.pmax;
      if (p > j0 / 128) p = j0 / 128;
      const int64_t ks = round_up(cdiv(j0, p), 32);
      const int P = (int)cdiv(j0, ks);
      dim3 grid((unsigned)rt, (unsigned)P);
      GPTQ_LAUNCH(K_Q_GEMM, st,
                  q_gemm_kernel<<<grid, 256, 0, st>>>(E, L.lde, U, cols, Wsrc, ldws, rows, j0, bw,
                                                      ks, part, pstride, wblk, vecU));
      if (P > 1) {
        const int64_t pairs = rows * (QB / 2);
        GPTQ_LAUNCH(K_Q_REDUCE, st,
                    q_reduce_kernel<<<(unsigned)cdiv(pairs, 256), 256, 0, st>>>(
                        part, P, pstride, Wsrc, ldws, rows, j0, bw, wblk));
      }
      cur = wblk;
    }
    gptq_status s;
    switch (group_size) {
      case 16: s = launch_sweep<16>(st, nw, Wsrc, ldws, cur, U, cols, vecU, rows, j0, bw, bits, E, L.lde, csw, cols, scales, zeros, L.ng, row_loss, status); break;
      case 32: s = launch_sweep<32>(st, nw, Wsrc, ldws, cur, U, cols, vecU, rows, j0, bw, bits, E, L.lde, csw, cols, scales, zeros, L.ng, row_loss, status); break;
      case 64: s = launch_sweep<64>(st, nw, Wsrc, ldws, cur, U, cols, vecU, rows, j0, bw, bits, E, L.lde, csw, cols, scales, zeros, L.ng, row_loss, status); break;
      default: s = launch_sweep<128>(st, nw, Wsrc, ldws, cur, U, cols, vecU, rows, j0, bw, bits, E, L.lde, csw, cols, scales, zeros, L.ng, row_loss, status); break;
    }
    if (s != GPTQ_OK) return s;
  }
  if (perm) {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(cols, 256), 16),
              (unsigned)std::min<int64_t>(rows, 65535));
    GPTQ_LAUNCH(K_Q_FINALIZE, st,
                q_finalize_kernel<<<grid, 256, 0, st>>>(codes_s, invperm, rows, cols, group_size,
                                                        codes, g_idx, status));
  }
  unsigned h_status = 0;
  GPTQ_HIP(hipMemcpyAsync(&h_status, status, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  if (h_status & ST_BADPERM) return GPTQ_EINVAL;
  if (h_status & ST_NONFINITE) return GPTQ_ENONFINITE;
  return GPTQ_OK;
}
