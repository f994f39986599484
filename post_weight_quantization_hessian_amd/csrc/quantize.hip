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
// registers: 16 lanes (one DPP row) per row, lane q owning the columns q,
// q + 16, ..., q + 112 (8 slots); the register window shifts by one slot
// every 16 columns so the live column is always slot 0 of lane j % 16, whose
// residual is broadcast to its row with row_newbcast (one 64-bit DPP move).
// Group min/max and the loss are reduced over the row with quad permutes and
// row rotations.
// In the factor form the matrix beyond U's diagonal blocks is R U over each
// block (R = U^-1, prepare.hip) and E holds the residuals Q - W of the
// original weights: (Q - W)[:, :j0] (R U)[:j0, blk] is the same update sum
// as E[:, :j0] U[:j0, blk] (E = (W - Q) R), so the GEMM and the in-block
// sweep are unchanged and only the stored E differs.
#include <type_traits>

#include "common.h"

namespace gptq {

constexpr int QB = 128;  // sweep block width
typedef double dbl2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers

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
                              unsigned* __restrict__ status,
                              unsigned long long* __restrict__ ocount) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  if (tid == 0) {
    *status = 0u;
    *ocount = 0ull;
  }
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
// The same two gathers with the source row staged in LDS (rows of up to
// QP_LDS_COLS columns, 64 KB of fp16): the row is read once, contiguously,
// and the permuted reads hit LDS instead of scattering 2- or 1-byte loads
// over memory. One block per row (grid-stride over rows).
constexpr int64_t QP_LDS_COLS = 32768;
__global__ __launch_bounds__(1024) void q_permute_lds_kernel(const uint16_t* __restrict__ W,
                                                             int64_t ldw,
                                                             const int32_t* __restrict__ perm,
                                                             int64_t rows, int64_t cols,
                                                             uint16_t* __restrict__ Wp,
                                                             int32_t* __restrict__ invperm,
                                                             unsigned* __restrict__ status) {
  extern __shared__ uint16_t qp_row[];
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* src = W + r * ldw;
    for (int64_t k = threadIdx.x; k < cols; k += blockDim.x) qp_row[k] = src[k];
    __syncthreads();
    uint16_t* dst = Wp + r * cols;
    for (int64_t k = threadIdx.x; k < cols; k += blockDim.x) {
      const int64_t pk = perm[k];
      if (pk < 0 || pk >= cols) {
        if (r == 0) atomicOr(status, ST_BADPERM);
        dst[k] = 0;
        continue;
      }
      dst[k] = qp_row[pk];
      if (r == 0) invperm[pk] = (int32_t)k;
    }
    __syncthreads();
  }
}
__global__ __launch_bounds__(1024) void q_finalize_lds_kernel(const uint8_t* __restrict__ codes_s,
                                                              const int32_t* __restrict__ invperm,
                                                              int64_t rows, int64_t cols, int gs,
                                                              uint8_t* __restrict__ codes,
                                                              int32_t* __restrict__ g_idx,
                                                              unsigned* __restrict__ status) {
  extern __shared__ uint8_t qf_row[];
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint8_t* src = codes_s + r * cols;
    for (int64_t k = threadIdx.x; k < cols; k += blockDim.x) qf_row[k] = src[k];
    __syncthreads();
    for (int64_t m = threadIdx.x; m < cols; m += blockDim.x) {
      const int32_t k = invperm[m];
      if (k < 0 || k >= cols) {
        if (r == 0) atomicOr(status, ST_BADPERM);
        if (codes) codes[r * cols + m] = 0;
        continue;
      }
      if (codes) codes[r * cols + m] = qf_row[k];
      if (r == 0 && g_idx) g_idx[m] = k / gs;
    }
    __syncthreads();
  }
}
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
        if (codes) codes[r * cols + m] = 0;
        continue;
      }
      if (codes) codes[r * cols + m] = codes_s[r * cols + k];
      if (r == 0 && g_idx) g_idx[m] = k / gs;
    }
  }
}

__global__ void q_fill_u32_kernel(unsigned* __restrict__ p, int64_t count) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = 0u;
}

// Histogram of int16 levels into hist[level + 32768] (65536 bins): levels in
// [-1024, 1023] are counted in LDS first, the others straight in global
// memory. Each thread takes 16 consecutive levels.
constexpr int QH_LDS = 2048;
__global__ __launch_bounds__(256) void q_hist_kernel(const int16_t* __restrict__ lv, int64_t n,
                                                     unsigned* __restrict__ hist) {
  __shared__ unsigned h[QH_LDS];
  for (int i = threadIdx.x; i < QH_LDS; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const int64_t e0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t e = e0 + u;
    if (e < n) {
      const int k = lv[e];
      if (k >= -QH_LDS / 2 && k < QH_LDS / 2) atomicAdd(&h[k + QH_LDS / 2], 1u);
      else atomicAdd(&hist[k + 32768], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < QH_LDS; i += blockDim.x)
    if (h[i]) atomicAdd(&hist[i - QH_LDS / 2 + 32768], h[i]);
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

// One 64-row workgroup tile of the update GEMM over l in [k_lo, k_hi): with
// wblk, the whole sum, written as W~ = W - sum into wblk; else the partial
// sum, written to Pp. 256 threads; `lds` holds QG_LDS floats.
constexpr int QG_LDS = 2 * 64 * QE_LD + 2 * 32 * QU_LD;
__device__ __forceinline__ void q_gemm_tile(const float* __restrict__ E, int64_t lde,
                                            const float* __restrict__ U, int64_t ldu,
                                            const uint16_t* __restrict__ W, int64_t ldw,
                                            int64_t rows, int64_t j0, int bw, int64_t r0,
                                            int64_t k_lo, int64_t k_hi, double* __restrict__ Pp,
                                            double* __restrict__ wblk, bool vecU, float* lds) {
  float(*Es)[64 * QE_LD] = reinterpret_cast<float(*)[64 * QE_LD]>(lds);
  float(*Us)[32 * QU_LD] = reinterpret_cast<float(*)[32 * QU_LD]>(lds + 2 * 64 * QE_LD);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nchunks = k_hi > k_lo ? (int)((k_hi - k_lo) / 32) : 0;

  // E loader: row t>>2, 8 floats at (t&3)*8; U loader: row t>>3, 16 floats at (t&7)*16.
  // Chunks are loaded two ahead into two register sets (the E rows come from
  // memory once per block, so a load in flight needs more than one chunk of
  // products to arrive), the loop unrolled by two so that each set keeps its
  // registers.
  const int er = t >> 2, ec = (t & 3) * 8;
  const int ur = t >> 3, uc = (t & 7) * 16;
  const bool vfull = vecU && bw == QB;  // every U load a whole float4
  struct Stage {
    f4 e[2], u[4];
  };
  auto fetch = [&](int c, Stage& S) {
    const int64_t l0 = k_lo + (int64_t)c * 32;
    if (r0 + er < rows) {
      const float* pe = E + (r0 + er) * lde + l0 + ec;
      S.e[0] = *reinterpret_cast<const f4*>(pe);
      S.e[1] = *reinterpret_cast<const f4*>(pe + 4);
    } else {
      S.e[0] = f4{0, 0, 0, 0};
      S.e[1] = f4{0, 0, 0, 0};
    }
    const float* pu = U + (l0 + ur) * ldu + j0 + uc;
    if (vfull) {
#pragma unroll
      for (int q = 0; q < 4; ++q) S.u[q] = *reinterpret_cast<const f4*>(pu + 4 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = uc + 4 * q;
        if (vecU && cc + 3 < bw) {
          S.u[q] = *reinterpret_cast<const f4*>(pu + 4 * q);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) S.u[q][x] = (cc + x < bw) ? pu[4 * q + x] : 0.0f;
        }
      }
    }
  };
  auto store = [&](int buf, const Stage& S) {
    float* se = &Es[buf][er * QE_LD + ec];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      se[x] = S.e[0][x];
      se[4 + x] = S.e[1][x];
    }
    float* su = &Us[buf][ur * QU_LD + uc];
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<f4*>(su + 4 * q) = S.u[q];
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
  auto compute = [&](int cur) {
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
  };

  if (nchunks > 0) {
    Stage A, B;
    fetch(0, A);
    store(0, A);
    if (nchunks > 1) fetch(1, A);
    __syncthreads();
    int c = 0;
    for (;;) {
      // buffer c & 1 holds chunk c, A chunk c + 1
      if (c + 2 < nchunks) fetch(c + 2, B);
      compute(c & 1);
      if (c + 1 < nchunks) store((c + 1) & 1, A);
      __syncthreads();
      if (++c >= nchunks) break;
      // buffer c & 1 holds chunk c, B chunk c + 1
      if (c + 2 < nchunks) fetch(c + 2, A);
      compute(c & 1);
      if (c + 1 < nchunks) store((c + 1) & 1, B);
      __syncthreads();
      if (++c >= nchunks) break;
    }
  }
  const int col = w * 32 + (lane & 31);
  if (wblk) {
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
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int64_t row = r0 + 32 * i + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
      if (row < rows) Pp[row * QB + col] = acc64[i][x];
    }
}

// The update GEMM for the block at j0 over l in [k_base, k_end) in pieces of
// ks (blockIdx.y = piece): the partial of piece p goes to part[p_base + p];
// with wblk (one piece covering all of l < j0) W~ itself goes to wblk.
__global__ __launch_bounds__(256) void q_gemm_kernel(const float* __restrict__ E, int64_t lde,
                                                     const float* __restrict__ U, int64_t ldu,
                                                     const uint16_t* __restrict__ W, int64_t ldw,
                                                     int64_t rows, int64_t j0, int bw,
                                                     int64_t k_base, int64_t ks, int64_t k_end,
                                                     double* __restrict__ part,
                                                     int64_t part_stride, int p_base,
                                                     double* __restrict__ wblk, bool vecU) {
  __shared__ float lds[QG_LDS];
  const int p = blockIdx.y;
  const int64_t k_lo = k_base + (int64_t)p * ks;
  const int64_t k_hi = k_lo + ks < k_end ? k_lo + ks : k_end;
  q_gemm_tile(E, lde, U, ldu, W, ldw, rows, j0, bw, (int64_t)blockIdx.x * 64, k_lo, k_hi,
              part + (int64_t)(p_base + p) * part_stride, wblk, vecU, lds);
}

// ---------------------------------------------------------------- sweep
//
// One block of columns [j0, j0+bw). A row is held by the 16 lanes of one DPP
// row: lane q owns columns q, q+16, ..., q+112 (8 fp64 slots); a wave holds
// 4 rows. Every 16 columns the slots shift down by one, so the live column is
// always slot 0 of lane j % 16, whose scaled error is broadcast to its row
// with row_newbcast. Group min/max and the loss are reduced over the row with
// quad permutes and row rotations.
__device__ inline double row_ror4(double v) { return dpp_f64<0x124>(v); }
// row_newbcast of lane N as a plain DPP move (no "old" operand to keep)
template <int N>
__device__ inline double row_bcast_mov(double v) {
  return row_bcast<N>(v);
}
// the same for a lane index that is a constant after loop unrolling
__device__ inline double row_bcast_mov_i(double v, int n) {
  switch (n) {
    case 0: return row_bcast_mov<0>(v);
    case 1: return row_bcast_mov<1>(v);
    case 2: return row_bcast_mov<2>(v);
    case 3: return row_bcast_mov<3>(v);
    case 4: return row_bcast_mov<4>(v);
    case 5: return row_bcast_mov<5>(v);
    case 6: return row_bcast_mov<6>(v);
    case 7: return row_bcast_mov<7>(v);
    case 8: return row_bcast_mov<8>(v);
    case 9: return row_bcast_mov<9>(v);
    case 10: return row_bcast_mov<10>(v);
    case 11: return row_bcast_mov<11>(v);
    case 12: return row_bcast_mov<12>(v);
    case 13: return row_bcast_mov<13>(v);
    case 14: return row_bcast_mov<14>(v);
    default: return row_bcast_mov<15>(v);
  }
}
__device__ inline double row_ror8(double v) { return dpp_f64<0x128>(v); }

// MODE 1, SSQR (The Geometry of LLM Quantization, section 3): the group's
// step is alpha times the min-max one, with the zero point of the unscaled
// step, and a level outside [0, maxq] makes an outlier: its current value is
// kept as fp16 (mask 1, value in ovals at the original column, only the fp16
// rounding propagates) and its stored code is the clamped one.
// MODE 2, HPTQ (same section): one unbounded grid, step alpha times the
// min-max one, zero point 0, no clipping (the caller passes clip = false);
// the level k goes to ovals (int16 bits) at the original column, and a level
// beyond the int16 range is reported (ST_NONFINITE).
// FAC (MODE 0 only), the factor form: beyond the block's diagonal, the
// matrix passed holds (R U)[blk_a, blk_b] = R[blk_a, blk_b] U[blk_b, blk_b]
// for the factor R = U^-1 of H itself, and E holds the residuals q - w of the
// original weights. Since E = (W - Q) R and, U being upper, R[:j0, :j0]
// U[:j0, blk] = -R[:j0, blk] U[blk, blk], the update sum (Q - W)[:, :j0]
// (R U)[:j0, blk] is E[:, :j0] U[:j0, blk], the same current values; only
// the stored E differs.
template <int GS, int MODE, int RPL, bool FAC = false>
__global__ __launch_bounds__(512) void q_sweep_kernel(
    const uint16_t* __restrict__ W, int64_t ldw, const double* __restrict__ wblk,
    const double* __restrict__ part, int P, int64_t part_stride,
    const float* __restrict__ U, int64_t ldu, bool vecU, int64_t rows, int64_t j0, int bw,
    int bits, float* __restrict__ E, int64_t lde, uint8_t* __restrict__ codes, int64_t ldc,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t ldg,
    double* __restrict__ row_loss, unsigned* __restrict__ status, bool clip, bool late, int nsweep,
    int64_t gj0, int gbw, int64_t gks, int64_t gk_end, double* __restrict__ gpart, double alpha,
    uint8_t* __restrict__ omask, uint16_t* __restrict__ ovals, const int32_t* __restrict__ operm,
    int64_t cols, unsigned long long* __restrict__ ocount) {
  constexpr bool SSQR = MODE == 1;
  constexpr bool HPTQ = MODE == 2;
  // U slab plus three rows of zero padding: the slot reads of a column run up
  // to 112 entries past its row end, into the next row or the padding, only
  // for slots past the block end whose values are never used; rows are read
  // two columns ahead up to row QB + 1. With `late`, the sum over the
  // previous block's errors (16 RPL rows x 128 columns) is left in the front
  // of this array before the slab is staged.
  __shared__ double Us[QB * QB + 3 * QB];
  __shared__ double rdiag[QB];  // 1 / U[j][j]
  if ((int)blockIdx.x >= nsweep) {
    // workgroups past the sweep's own (256 threads each): the next block's
    // update GEMM over the errors of the blocks before this one, l < gk_end,
    // as partials gpart[piece]; they neither read nor write this block
    const int64_t rt = (rows + 63) / 64;
    const int idx = (int)blockIdx.x - nsweep;
    const int piece = (int)(idx / rt);
    const int64_t k_lo = (int64_t)piece * gks;
    const int64_t k_hi = k_lo + gks < gk_end ? k_lo + gks : gk_end;
    q_gemm_tile(E, lde, U, ldu, W, ldw, rows, gj0, gbw, (idx - piece * rt) * 64, k_lo, k_hi,
                gpart + (int64_t)piece * part_stride, nullptr, vecU,
                reinterpret_cast<float*>(Us));
    return;
  }
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int q = lane & 15;
  const int nthr = blockDim.x;
  // the workgroup's rows: 4 per wave and row slot p (16 lanes each), RPL
  // slots; local row lr[p] = 4 RPL wv + 4 p + lane / 16
  const int64_t wg_row0 = (int64_t)blockIdx.x * ((nthr >> 4) * RPL);
  int lr[RPL];
  int64_t r[RPL];
  bool rv[RPL];
#pragma unroll
  for (int p = 0; p < RPL; ++p) {
    lr[p] = 4 * RPL * wv + 4 * p + (lane >> 4);
    r[p] = wg_row0 + lr[p];
    rv[p] = r[p] < rows;
  }
  const double maxq = (double)((1 << bits) - 1);

  // All global loads of the prologue are issued before any is waited on:
  // the U slab (16 float4 per thread for 256 threads), this row's current
  // values, the split-K partials, then the operands of the late sum.
  const bool vec_slab = vecU && bw == QB;
  constexpr int SLAB4 = QB * QB / 4;       // float4s in the slab
  constexpr int PER = SLAB4 / 256;         // per thread with 256 threads
  f4 sv[PER];
  if (vec_slab) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * nthr + t;
      const int a = e >> 5, c4 = (e & 31) * 4;
      sv[u] = e < SLAB4 ? *reinterpret_cast<const f4*>(U + (j0 + a) * ldu + j0 + c4)
                        : f4{0, 0, 0, 0};
    }
  }
  // Current values of this row's columns: W - E[:, :j0] U[:j0, blk]. Either
  // the update GEMM formed them whole (wblk), or it left P split-K partials
  // of the sum over l < j0 (l < j0 - 128 with `late`), which are added here
  // in split order, and with `late` (256 threads) the workgroup forms the
  // sum over the previous block's 128 errors itself, last; the first block
  // reads the weights directly.
  double w[RPL][8];
#pragma unroll
  for (int p = 0; p < RPL; ++p)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 16 * s + q;
      w[p][s] = (rv[p] && c < bw)
                    ? (wblk ? wblk[r[p] * QB + c] : f16_to_f64(W[r[p] * ldw + j0 + c]))
                    : 0.0;
    }
  double acc[RPL][8];
#pragma unroll
  for (int p = 0; p < RPL; ++p)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[p][s] = 0.0;
  if (!wblk && P > 0) {
    constexpr int PR = RPL == 1 ? 4 : 2;  // partials per round
#pragma unroll
    for (int p = 0; p < RPL; ++p) {
      const double* pr = part + (rv[p] ? r[p] : 0) * QB + q;
      for (int p0 = 0; p0 < P; p0 += PR) {
        double v[PR][8];
#pragma unroll
        for (int u = 0; u < PR; ++u) {
          const int pu = p0 + u < P ? p0 + u : p0;
#pragma unroll
          for (int s = 0; s < 8; ++s) v[u][s] = pr[(int64_t)pu * part_stride + 16 * s];
        }
#pragma unroll
        for (int u = 0; u < PR; ++u)
#pragma unroll
          for (int s = 0; s < 8; ++s)
            if (p0 + u < P) acc[p][s] += v[u][s];
      }
    }
  }
  // The late sum, for the workgroup's 16 RPL rows: wave wv takes columns
  // 32 wv .. 32 wv + 31 as 16x16 fp32 MFMA tiles over K = 128 (all operands
  // loaded first), summed in fp32 per 32-wide K chunk and in fp64 across
  // chunks (as the update GEMM does), and leaves them in the front of Us.
  // v_mfma_f32_16x16x4f32 layout (lane l): A[m][k]: m = l%16, k = l/16;
  // B[k][n]: n = l%16, k = l/16; D element i: row 4*(l/16) + i, col l%16.
  double* lt = Us;  // [16 RPL][QB]
  if (late) {
    const int n0 = 32 * wv + (lane & 15);
    const float* ub = U + (j0 - QB + (lane >> 4)) * ldu + j0 + n0;
    const bool cv0 = n0 < bw, cv1 = n0 + 16 < bw;
    double dl[RPL][2][4];
#pragma unroll
    for (int rt = 0; rt < RPL; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dl[rt][0][i] = dl[rt][1][i] = 0.0;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      float av[RPL][8], bv0[8], bv1[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int k = 32 * ch + 4 * st;
        bv0[st] = cv0 ? ub[(int64_t)k * ldu] : 0.0f;
        bv1[st] = cv1 ? ub[(int64_t)k * ldu + 16] : 0.0f;
      }
#pragma unroll
      for (int rt = 0; rt < RPL; ++rt) {
        const int64_t arow = wg_row0 + 16 * rt + (lane & 15);
        const float* ea = E + (arow < rows ? arow : rows - 1) * lde + (j0 - QB) + (lane >> 4);
#pragma unroll
        for (int st = 0; st < 8; ++st) av[rt][st] = ea[32 * ch + 4 * st];
      }
#pragma unroll
      for (int rt = 0; rt < RPL; ++rt) {
        f4 m0 = {0.0f, 0.0f, 0.0f, 0.0f}, m1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          m0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[rt][st], bv0[st], m0, 0, 0, 0);
          m1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[rt][st], bv1[st], m1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dl[rt][0][i] += (double)m0[i];
          dl[rt][1][i] += (double)m1[i];
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < RPL; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lt[(16 * rt + 4 * (lane >> 4) + i) * QB + n0] = dl[rt][0][i];
        lt[(16 * rt + 4 * (lane >> 4) + i) * QB + n0 + 16] = dl[rt][1][i];
      }
  }
  for (int j = t; j < QB; j += nthr) {
    rdiag[j] = j < bw ? 1.0 / (double)U[(j0 + j) * ldu + j0 + j] : 0.0;
    Us[QB * QB + j] = 0.0;
    Us[QB * QB + QB + j] = 0.0;
    Us[QB * QB + 2 * QB + j] = 0.0;
  }
  __syncthreads();
  if (late) {
#pragma unroll
    for (int p = 0; p < RPL; ++p)
#pragma unroll
      for (int s = 0; s < 8; ++s) acc[p][s] += lt[lr[p] * QB + 16 * s + q];
    __syncthreads();  // the slab overwrites lt
  }
  // Row a of the slab is stored divided by U[a][a] (the error broadcast along
  // a row is then the unscaled residual d, and e = d / U[a][a] leaves the
  // dependent chain). Entries on and below the diagonal are zero: a column's
  // own update (its diagonal term) is left out, so the slot holding the
  // column keeps the value it was quantized from until the tile ends, when
  // its code and error are formed from it again.
  if (vec_slab) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * nthr + t;
      if (e < SLAB4) {
        const int a = e >> 5, c4 = (e & 31) * 4;
        const double ra = rdiag[a];
#pragma unroll
        for (int x = 0; x < 4; ++x) Us[e * 4 + x] = c4 + x > a ? (double)sv[u][x] * ra : 0.0;
      }
    }
    // fewer than 256 threads: the rest of the slab
    for (int e = PER * nthr + t; e < SLAB4; e += nthr) {
      const int a = e >> 5, c4 = (e & 31) * 4;
      const f4 v = *reinterpret_cast<const f4*>(U + (j0 + a) * ldu + j0 + c4);
      const double ra = rdiag[a];
#pragma unroll
      for (int x = 0; x < 4; ++x) Us[e * 4 + x] = c4 + x > a ? (double)v[x] * ra : 0.0;
    }
  } else {
    for (int e = t; e < QB * QB; e += nthr) {
      const int a = e >> 7, c = e & 127;
      Us[e] = (a < bw && c < bw && c > a) ? (double)U[(j0 + a) * ldu + j0 + c] * rdiag[a] : 0.0;
    }
  }
  bool finite = true;
#pragma unroll
  for (int p = 0; p < RPL; ++p)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      w[p][s] = (rv[p] && 16 * s + q < bw) ? w[p][s] - acc[p][s] : 0.0;
      finite = finite && isfinite(w[p][s]);
    }
  if (!finite) atomicOr(status, ST_NONFINITE);
  __syncthreads();

  double scale[RPL], rscale[RPL], zero[RPL], loss[RPL];
  double nout[RPL];  // SSQR: outliers of this lane's columns
  // range of the level k = code - zero: [-zero, maxq - zero], or unbounded
  // without clipping (the no-clipping regime of The Geometry of LLM
  // Quantization 2.3, whose codes are stored saturated to [0, 255])
  double klo[RPL], khi[RPL];
#pragma unroll
  for (int p = 0; p < RPL; ++p) {
    scale[p] = rscale[p] = 1.0;
    zero[p] = loss[p] = nout[p] = 0.0;
    klo[p] = -1e300;
    khi[p] = 1e300;
  }
  const int nt16 = (bw + 15) >> 4;
  // U row of column jc as seen from the slots (slot s holds column
  // 16*((jc >> 4) + s) + q; slots past the block end are dead and read into
  // the next row or the padding). Loaded two columns ahead into four
  // rotating register sets (set = column & 3); shared by the RPL rows.
  double ub[4][8];
  auto load_row = [&](int jc, double (&uu)[8]) {
    const double* urow = Us + jc * QB + 16 * (jc >> 4) + q;
#pragma unroll
    for (int s = 0; s < 8; ++s) uu[s] = urow[16 * s];
  };
  load_row(0, ub[0]);
  load_row(1, ub[1]);
  for (int tt = 0; tt < nt16; ++tt) {
    const double* ubase = Us + 16 * tt * QB + 16 * tt + q;
    if (((16 * tt) % GS) == 0) {
      // grid of the group starting here, from the current values
#pragma unroll
      for (int p = 0; p < RPL; ++p) {
        double mn = 0.0, mx = 0.0;
#pragma unroll
        for (int s = 0; s < GS / 16; ++s) {
          if (16 * (tt + s) + q < bw) {
            mn = fmin(mn, w[p][s]);
            mx = fmax(mx, w[p][s]);
          }
        }
        mn = fmin(mn, quad_xor1(mn));
        mx = fmax(mx, quad_xor1(mx));
        mn = fmin(mn, quad_xor2(mn));
        mx = fmax(mx, quad_xor2(mx));
        mn = fmin(mn, row_ror4(mn));
        mx = fmax(mx, row_ror4(mx));
        mn = fmin(mn, row_ror8(mn));
        mx = fmax(mx, row_ror8(mx));
        uint16_t sh = f64_to_f16_rne((mx - mn) / maxq);
        double sc = f16_to_f64(sh);
        if ((sh & 0x7fff) >= 0x7c00 && rv[p]) atomicOr(status, ST_NONFINITE);
        // SSQR: the step used is fp16(alpha * step); the zero point comes
        // from the unscaled one (sc, here), so the grid shrinks about 0
        const uint16_t sha = (SSQR || HPTQ) ? f64_to_f16_rne(alpha * ((mx - mn) / maxq)) : sh;
        const double scale_a = (SSQR || HPTQ) ? f16_to_f64(sha) : sc;
        if ((sha & 0x7fff) >= 0x7c00 && rv[p]) atomicOr(status, ST_NONFINITE);
        double z;
        if (mx == mn || (!HPTQ && sc == 0.0) || scale_a == 0.0) {
          sc = 1.0;
          sh = 0x3c00;
          z = 0.0;
        } else {
          z = HPTQ ? 0.0 : fmin(fmax(rint(-mn / sc), 0.0), maxq);
          sc = scale_a;
          sh = sha;
        }
        scale[p] = sc;
        zero[p] = z;
        rscale[p] = 1.0 / sc;
        klo[p] = clip ? -z : -1e300;
        khi[p] = clip ? maxq - z : 1e300;
        if (rv[p] && q == 0) {
          const int64_t g = (j0 + 16 * tt) / GS;
          scales[r[p] * ldg + g] = sh;
          zeros[r[p] * ldg + g] = f64_to_f16_rne(z);
        }
      }
    }
    // The 16 columns of the tile. Slot s of lane q holds column
    // 16 (tt + s) + q; in a full block only slots s < 8 - tt are inside it
    // (NS live slots), and only those are loaded and updated. Every lane
    // rounds its slot 0 each column, the owner's (lane jj's) residual is
    // broadcast to its row, and later columns take the update; the owner's
    // own slot is left as it was (zero diagonal of the slab). The RPL rows'
    // chains are independent and interleave.
    auto tile = [&](auto ns_c, auto full_c) {
      constexpr int NS = decltype(ns_c)::value;
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        if (FULL || 16 * tt + jj < bw) {
          double (&u)[8] = ub[jj & 3];
          {
            // row 16 tt + jj + 2 at a fixed offset from the tile's base (one
            // address register for the whole tile; rows past the block end
            // are zero rows of the slab or its padding)
            const int jc = jj + 2;
            const double* urow = ubase + jc * QB + 16 * (jc >> 4);
#pragma unroll
            for (int s = 0; s < NS; ++s) ub[(jj + 2) & 3][s] = urow[16 * s];
          }
          double db[RPL];
#pragma unroll
          for (int p = 0; p < RPL; ++p) {
            // code = clamp(rint(v/s) + z, 0, maxq) = k + z with
            // k = clamp(rint(v/s), -z, maxq - z), dequantized s * k
            const double v = w[p][0];
            const double kr = rint(v * rscale[p]);
            double d = fma(-scale[p], fmin(fmax(kr, klo[p]), khi[p]), v);
            if (SSQR && (kr < klo[p] || kr > khi[p])) d = v - f16_round_f64(v);
            db[p] = row_bcast_mov_i(d, jj);
          }
          // later columns: w -= d * U[j][c] / U[j][j] (zero for this column
          // and the ones before it)
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int p = 0; p < RPL; ++p) w[p][s] = fma(-db[p], u[s], w[p][s]);
        }
      }
    };
    // factor form: this tile's original weights for the stored residuals,
    // loaded before its column chain so that the load has arrived by its end
    uint16_t wraw[RPL];
    if constexpr (FAC) {
#pragma unroll
      for (int p = 0; p < RPL; ++p)
        wraw[p] = (rv[p] && 16 * tt + q < bw) ? W[r[p] * ldw + j0 + 16 * tt + q] : (uint16_t)0;
    }
    if (bw == QB) {
      switch (8 - tt) {
        case 8: tile(std::integral_constant<int, 8>{}, std::true_type{}); break;
        case 7: tile(std::integral_constant<int, 7>{}, std::true_type{}); break;
        case 6: tile(std::integral_constant<int, 6>{}, std::true_type{}); break;
        case 5: tile(std::integral_constant<int, 5>{}, std::true_type{}); break;
        case 4: tile(std::integral_constant<int, 4>{}, std::true_type{}); break;
        case 3: tile(std::integral_constant<int, 3>{}, std::true_type{}); break;
        case 2: tile(std::integral_constant<int, 2>{}, std::true_type{}); break;
        default: tile(std::integral_constant<int, 1>{}, std::true_type{}); break;
      }
    } else {
      tile(std::integral_constant<int, 8>{}, std::false_type{});
    }
    // codes and scaled errors of this row's 16 columns, one store each: slot
    // 0 still holds the value the lane's column was quantized from
    {
      const int c = 16 * tt + q;
#pragma unroll
      for (int p = 0; p < RPL; ++p) {
        if (rv[p] && c < bw) {
          const double v = w[p][0];
          const double kr = rint(v * rscale[p]);
          const double k_own = fmin(fmax(kr, klo[p]), khi[p]);
          double d_own = fma(-scale[p], k_own, v);
          const bool o_own = SSQR && (kr < klo[p] || kr > khi[p]);
          const double h_own = SSQR ? f16_round_f64(v) : 0.0;
          if (o_own) d_own = v - h_own;
          const double e = d_own * rdiag[c];
          codes[r[p] * ldc + j0 + c] = (uint8_t)fmin(fmax(k_own + zero[p], 0.0), 255.0);
          if constexpr (FAC) {
            // the residual q - w of the original weight (exact in fp64)
            E[r[p] * lde + j0 + c] = (float)fma(scale[p], k_own, -f16_to_f64(wraw[p]));
          } else {
            E[r[p] * lde + j0 + c] = (float)e;
          }
          loss[p] += e * e;
          if (SSQR || HPTQ) {
            const int64_t oc = operm ? (int64_t)operm[j0 + c] : j0 + c;
            if (oc >= 0 && oc < cols) {  // a bad permutation is reported elsewhere
              if (SSQR) {
                omask[r[p] * cols + oc] = o_own ? 1 : 0;
                ovals[r[p] * cols + oc] = o_own ? f64_to_f16_rne(h_own) : (uint16_t)0;
              } else {
                const double kc = fmin(fmax(k_own, -32768.0), 32767.0);
                if (kc != k_own) atomicOr(status, ST_NONFINITE);
                ovals[r[p] * cols + oc] = (uint16_t)(int16_t)kc;
              }
            }
            if (SSQR) nout[p] += o_own ? 1.0 : 0.0;
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < RPL; ++p) {
#pragma unroll
      for (int s = 0; s < 7; ++s) w[p][s] = w[p][s + 1];
      w[p][7] = 0.0;
    }
  }
#pragma unroll
  for (int p = 0; p < RPL; ++p) {
    double l = loss[p];
    l += quad_xor1(l);
    l += quad_xor2(l);
    l += row_ror4(l);
    l += row_ror8(l);
    if (rv[p] && q == 0) row_loss[r[p]] += l;
    if (SSQR) {
      double no = nout[p];
      no += quad_xor1(no);
      no += quad_xor2(no);
      no += row_ror4(no);
      no += row_ror8(no);
      if (rv[p] && q == 0 && no > 0.0) atomicAdd(ocount, (unsigned long long)no);
    }
  }
}

// ---------------------------------------------------------------- layout

struct QLayout {
  int64_t rows, cols, lde, ng;
  int pmax;
  size_t off_status, off_count, off_hist, off_invperm, off_wp, off_codes, off_E, off_part, off_wblk,
      total;
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
  L.off_count = take(8);
  L.off_hist = take(4 * 65536);
  L.off_invperm = take(4 * (size_t)cols);
  L.off_wp = take(2 * (size_t)rows * cols);
  L.off_codes = take((size_t)rows * cols);
  L.off_E = take(4 * (size_t)rows * L.lde);
  L.off_part = take(8 * 2 * (size_t)(L.pmax + 1) * rows * QB);
  L.off_wblk = take(8 * (size_t)rows * QB);
  L.total = o;
  return L;
}

// One sweep launch: nsweep workgroups of 64 * nw threads for the block at j0
// (with `late`, nw == 4 only, they add the sum over the previous block's
// errors themselves), then ng workgroups (nw == 4 only) of the next block's
// early update GEMM.
struct SweepArgs {
  int nw, rpl, nsweep, ng;
  const uint16_t* W;
  int64_t ldw;
  const double* wblk;
  const double* part;
  int P;
  int64_t pstride;
  const float* U;
  int64_t ldu;
  bool vecU;
  int64_t rows, j0;
  int bw, bits;
  float* E;
  int64_t lde;
  uint8_t* codes;
  int64_t ldc;
  uint16_t* scales;
  uint16_t* zeros;
  int64_t ldg;
  double* row_loss;
  unsigned* status;
  bool clip, late;
  int64_t gj0;
  int gbw;
  int64_t gks, gk_end;
  double* gpart;
  // SSQR (mode 1) / HPTQ (mode 2): outputs at the original columns
  int mode;
  double alpha;
  uint8_t* omask;
  uint16_t* ovals;
  const int32_t* operm;
  int64_t cols;
  unsigned long long* ocount;
  bool fac;  // the factor form (mode 0 only)
};

template <int GS>
static gptq_status launch_sweep(hipStream_t st, const SweepArgs& a) {
#define Q_SWEEP(SS, RP, FC)                                                                    \
  GPTQ_LAUNCH(K_Q_SWEEP, st,                                                                   \
              (q_sweep_kernel<GS, SS, RP, FC><<<a.nsweep + a.ng, 64 * a.nw, 0, st>>>(          \
                  a.W, a.ldw, a.wblk, a.part, a.P, a.pstride, a.U, a.ldu, a.vecU, a.rows, a.j0, \
                  a.bw, a.bits, a.E, a.lde, a.codes, a.ldc, a.scales, a.zeros, a.ldg,          \
                  a.row_loss, a.status, a.clip, a.late, a.nsweep, a.gj0, a.gbw, a.gks,         \
                  a.gk_end, a.gpart, a.alpha, a.omask, a.ovals, a.operm, a.cols, a.ocount)))
  if (a.rpl == 2) {  // the plain sweep only (the SSQR/HPTQ state of two rows spills)
    if (a.fac) Q_SWEEP(0, 2, true);
    else Q_SWEEP(0, 2, false);
  } else {
    if (a.mode == 1) Q_SWEEP(1, 1, false);
    else if (a.mode == 2) Q_SWEEP(2, 1, false);
    else if (a.fac) Q_SWEEP(0, 1, true);
    else Q_SWEEP(0, 1, false);
  }
#undef Q_SWEEP
  return GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

static bool valid_gs(int gs) { return gs == 16 || gs == 32 || gs == 64 || gs == 128; }

extern "C" size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t cols, int group_size) {
  if (rows <= 0 || cols <= 0 || !valid_gs(group_size)) return 0;
  return q_layout(rows, cols, group_size).total;
}

// The whole sweep of a layer; mode 1 (SSQR) and 2 (HPTQ) run those rules
// with their outputs at alpha; mode 3 is the plain sweep in the factor form.
// Arguments are validated by the callers; returns after enqueueing.
static gptq_status quantize_enqueue(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                    const float* U, const int32_t* perm, int bits, int group_size,
                                    bool clip, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                    int32_t* g_idx, double* row_loss, int mode, double alpha,
                                    uint8_t* omask, uint16_t* ovals, void* ws,
                                    hipStream_t st) {
  const bool fac = mode == 3;
  if (fac) mode = 0;
  const QLayout L = q_layout(rows, cols, group_size);
  char* base = (char*)ws;
  unsigned* status = (unsigned*)(base + L.off_status);
  unsigned long long* ocount = (unsigned long long*)(base + L.off_count);
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
                                                  group_size, status, ocount));
  }
  const uint16_t* Wsrc = W;
  int64_t ldws = ldw;
  uint8_t* csw = codes ? codes : codes_s;  // sweep-order codes (HPTQ: none returned)
  if (perm && cols <= QP_LDS_COLS) {
    GPTQ_LAUNCH(K_Q_PERMUTE, st,
                q_permute_lds_kernel<<<(unsigned)std::min<int64_t>(rows, 65535), 1024,
                                       (size_t)cols * 2, st>>>(W, ldw, perm, rows, cols, Wp,
                                                               invperm, status));
    Wsrc = Wp;
    ldws = cols;
    csw = codes_s;
  } else if (perm) {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(cols, 256), 16),
              (unsigned)std::min<int64_t>(rows, 65535));
    GPTQ_LAUNCH(K_Q_PERMUTE, st,
                q_permute_kernel<<<grid, 256, 0, st>>>(W, ldw, perm, rows, cols, Wp, invperm,
                                                       status));
    Wsrc = Wp;
    ldws = cols;
    csw = codes_s;
  }
  // 4 rows per wave and row slot; 8 waves per workgroup once that still
  // gives >= 256 workgroups, else 4 (the U slab fills most of the LDS: one
  // workgroup per CU). Two row slots per lane group (their dependent chains
  // interleave) when one slot would need more than one round of workgroups:
  // 9728 rows, 45.5 -> 36.8 us per launch. (With 4 waves, where the launch
  // also carries the early update GEMM, two slots measured 35 % slower: the
  // split-K partials are loaded per row. The SSQR and HPTQ state of two rows
  // does not fit the registers.)
  const int nw = cdiv(rows, 32) >= 256 ? 8 : 4;
  const int rpl = (mode == 0 && nw == 8 && cdiv(rows, 32) > 256) ? 2 : 1;
  const int nsweep = (int)cdiv(rows, 4 * nw * rpl);
  const bool vecU = (cols % 4 == 0) && ((uintptr_t)U % 16 == 0);
  const int64_t rt = cdiv(rows, 64);
  double* wblk = (double*)(base + L.off_wblk);
  double* partbuf[2] = {part, part + (int64_t)(L.pmax + 1) * pstride};
  // When the sweep leaves CUs idle, the update GEMM of block b+1 is split:
  // the sum over the errors of blocks < b runs in the sweep launch of block b
  // (pieces 0..ep-1, one workgroup per CU beside the sweep's own, while each
  // piece stays short: QEMB_KMAX), and the sum over block b's errors
  // (K = 128) is formed by the sweep workgroups of block b+1 themselves.
  // Otherwise the block's GEMM runs whole before its sweep.
  constexpr int64_t QEMB_KMAX = 512;
  const int emb_max = nw == 4 ? std::min<int64_t>(L.pmax, (256 - nsweep) / rt) : 0;
  int ep = 0;  // early pieces of the current block's GEMM already computed (-1: none)
  for (int64_t j0 = 0, b = 0; j0 < cols; j0 += QB, ++b) {
    const int bw = (int)std::min<int64_t>(QB, cols - j0);
    double* pc = partbuf[b & 1];
    double* pn = partbuf[(b + 1) & 1];
    const double* cur = nullptr;
    int nparts = 0;
    bool late = false;
    if (j0 > 0) {
      if (ep >= 0) {
        late = true;
        nparts = ep;
      } else {
        int64_t p = L.pmax;
        if (p > j0 / 128) p = j0 / 128;
        const int64_t ks = round_up(cdiv(j0, p), 32);
        const int P = (int)cdiv(j0, ks);
        dim3 grid((unsigned)rt, (unsigned)P);
        GPTQ_LAUNCH(K_Q_GEMM, st,
                    q_gemm_kernel<<<grid, 256, 0, st>>>(E, L.lde, U, cols, Wsrc, ldws, rows, j0,
                                                        bw, 0, ks, j0, pc, pstride, 0,
                                                        P == 1 ? wblk : nullptr, vecU));
        // one split: the GEMM wrote W~ itself; else the sweep sums the partials
        if (P == 1) cur = wblk;
        else nparts = P;
      }
    }
    SweepArgs a{nw, rpl, nsweep, 0, Wsrc, ldws, cur, pc, nparts, pstride, U, cols, vecU, rows, j0,
                bw, bits, E, L.lde, csw, cols, scales, zeros, L.ng, row_loss, status, clip,
                late, 0, 0, 0, 0, pn, mode, alpha, omask, ovals, perm, cols, ocount, fac};
    ep = emb_max > 0 ? 0 : -1;
    if (emb_max > 0 && j0 > 0 && j0 + QB < cols) {
      // next block's sum over l < j0 (the errors of blocks < b), in as few
      // pieces of at most QEMB_KMAX as fit (each piece is one more partial
      // for the sweep to add)
      const int64_t pe = std::min<int64_t>(emb_max, cdiv(j0, QEMB_KMAX));
      const int64_t ks = round_up(cdiv(j0, pe), 32);
      if (ks <= QEMB_KMAX) {
        ep = (int)cdiv(j0, ks);
        a.ng = (int)(ep * rt);
        a.gj0 = j0 + QB;
        a.gbw = (int)std::min<int64_t>(QB, cols - j0 - QB);
        a.gks = ks;
        a.gk_end = j0;
      } else {
        ep = -1;
      }
    }
    gptq_status s;
    switch (group_size) {
      case 16: s = launch_sweep<16>(st, a); break;
      case 32: s = launch_sweep<32>(st, a); break;
      case 64: s = launch_sweep<64>(st, a); break;
      default: s = launch_sweep<128>(st, a); break;
    }
    if (s != GPTQ_OK) return s;
  }
  if (perm && cols <= QP_LDS_COLS) {
    GPTQ_LAUNCH(K_Q_FINALIZE, st,
                q_finalize_lds_kernel<<<(unsigned)std::min<int64_t>(rows, 65535), 1024,
                                        (size_t)cols, st>>>(codes_s, invperm, rows, cols,
                                                            group_size, codes, g_idx, status));
  } else if (perm) {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(cols, 256), 16),
              (unsigned)std::min<int64_t>(rows, 65535));
    GPTQ_LAUNCH(K_Q_FINALIZE, st,
                q_finalize_kernel<<<grid, 256, 0, st>>>(codes_s, invperm, rows, cols, group_size,
                                                        codes, g_idx, status));
  }
  return GPTQ_OK;
}

static gptq_status quantize_check(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                  const float* U, int bits, int group_size, const uint8_t* codes,
                                  const uint16_t* scales, const uint16_t* zeros,
                                  const double* row_loss) {
  if (rows < 0 || cols < 0) return GPTQ_EINVAL;
  if (bits < 2 || bits > 8 || !valid_gs(group_size)) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros || !row_loss || ldw < cols) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 20 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  return GPTQ_OK;
}

extern "C" gptq_status gptq_quantize_layer(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                           const float* U, const int32_t* perm, int bits,
                                           int group_size, uint32_t flags, uint8_t* codes,
                                           uint16_t* scales, uint16_t* zeros, int32_t* g_idx,
                                           double* row_loss, void* ws, size_t ws_bytes,
                                           void* stream) {
  if (flags & ~(GPTQ_FLAG_NO_SYNC | GPTQ_FLAG_NO_CLIP | GPTQ_FLAG_FACTOR_FORM)) return GPTQ_EINVAL;
  gptq_status c = quantize_check(W, rows, cols, ldw, U, bits, group_size, codes, scales, zeros,
                                 row_loss);
  if (c != GPTQ_OK || rows == 0 || cols == 0) return c;
  if (!ws || ws_bytes < q_layout(rows, cols, group_size).total) return GPTQ_EWORKSPACE;
  c = quantize_enqueue(W, rows, cols, ldw, U, perm, bits, group_size,
                       !(flags & GPTQ_FLAG_NO_CLIP), codes, scales, zeros, g_idx, row_loss,
                       (flags & GPTQ_FLAG_FACTOR_FORM) ? 3 : 0, 0.0,
                       nullptr, nullptr, ws, (hipStream_t)stream);
  if (c != GPTQ_OK) return c;
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  return gptq_workspace_status(ws, stream);
}

// SSQR: the outlier count of the last sweep on this workspace (synchronizes).
static gptq_status ssqr_count(void* ws, int64_t rows, int64_t cols, int gs, hipStream_t st,
                              uint64_t* n) {
  const QLayout L = q_layout(rows, cols, gs);
  unsigned long long h = 0;
  GPTQ_HIP(hipMemcpyAsync(&h, (char*)ws + L.off_count, sizeof(h), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  *n = (uint64_t)h;
  return GPTQ_OK;
}

extern "C" gptq_status gptq_quantize_layer_ssqr(const uint16_t* W, int64_t rows, int64_t cols,
                                                int64_t ldw, const float* U, const int32_t* perm,
                                                int bits, int group_size, uint32_t flags,
                                                double alpha, uint8_t* codes, uint16_t* scales,
                                                uint16_t* zeros, int32_t* g_idx,
                                                double* row_loss, uint8_t* outlier_mask,
                                                uint16_t* outlier_vals, uint64_t* n_outliers,
                                                void* ws, size_t ws_bytes, void* stream) {
  if (flags & ~GPTQ_FLAG_NO_SYNC) return GPTQ_EINVAL;
  if (!(alpha > 0.0 && alpha <= 16.0)) return GPTQ_EINVAL;
  if ((flags & GPTQ_FLAG_NO_SYNC) && n_outliers) return GPTQ_EINVAL;
  gptq_status c = quantize_check(W, rows, cols, ldw, U, bits, group_size, codes, scales, zeros,
                                 row_loss);
  if (c != GPTQ_OK) return c;
  if (rows == 0 || cols == 0) {
    if (n_outliers) *n_outliers = 0;
    return GPTQ_OK;
  }
  if (!outlier_mask || !outlier_vals) return GPTQ_EINVAL;
  if (!ws || ws_bytes < q_layout(rows, cols, group_size).total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  c = quantize_enqueue(W, rows, cols, ldw, U, perm, bits, group_size, true, codes, scales, zeros,
                       g_idx, row_loss, 1, alpha, outlier_mask, outlier_vals, ws, st);
  if (c != GPTQ_OK) return c;
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  if (n_outliers) {
    c = ssqr_count(ws, rows, cols, group_size, st, n_outliers);
    if (c != GPTQ_OK) return c;
  }
  return gptq_workspace_status(ws, stream);
}

extern "C" gptq_status gptq_ssqr_search(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                        const float* U, const int32_t* perm, int bits,
                                        int group_size, uint32_t flags, double target, int iters,
                                        double alpha_lo, double alpha_hi, double* alpha_out,
                                        uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                        int32_t* g_idx, double* row_loss, uint8_t* outlier_mask,
                                        uint16_t* outlier_vals, uint64_t* n_outliers, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (flags != 0) return GPTQ_EINVAL;
  if (!(target >= 0.0 && target <= 1.0) || iters < 0 || iters > 60) return GPTQ_EINVAL;
  if (!(alpha_lo > 0.0 && alpha_lo < alpha_hi && alpha_hi <= 16.0)) return GPTQ_EINVAL;
  if (!alpha_out) return GPTQ_EINVAL;
  gptq_status c = quantize_check(W, rows, cols, ldw, U, bits, group_size, codes, scales, zeros,
                                 row_loss);
  if (c != GPTQ_OK) return c;
  if (rows == 0 || cols == 0) {
    *alpha_out = alpha_hi;
    if (n_outliers) *n_outliers = 0;
    return GPTQ_OK;
  }
  if (!outlier_mask || !outlier_vals) return GPTQ_EINVAL;
  if (!ws || ws_bytes < q_layout(rows, cols, group_size).total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const double n = (double)rows * (double)cols;
  // every probe is a full sweep into the caller's outputs; the outputs are
  // left from the returned alpha (swept again at the end if the last probe
  // was another one)
  auto probe = [&](double a, uint64_t* cnt) -> gptq_status {
    gptq_status r = quantize_enqueue(W, rows, cols, ldw, U, perm, bits, group_size, true, codes,
                                     scales, zeros, g_idx, row_loss, 1, a, outlier_mask,
                                     outlier_vals, ws, st);
    if (r != GPTQ_OK) return r;
    r = ssqr_count(ws, rows, cols, group_size, st, cnt);
    if (r != GPTQ_OK) return r;
    return gptq_workspace_status(ws, stream);
  };
  double lo = alpha_lo, hi = alpha_hi, last = hi;
  uint64_t cnt = 0, best = 0;
  c = probe(hi, &cnt);
  if (c != GPTQ_OK) return c;
  best = cnt;
  if ((double)cnt / n <= target) {
    for (int it = 0; it < iters; ++it) {
      const double mid = 0.5 * (lo + hi);
      c = probe(mid, &cnt);
      if (c != GPTQ_OK) return c;
      last = mid;
      if ((double)cnt / n <= target) {
        hi = mid;
        best = cnt;
      } else {
        lo = mid;
      }
    }
    if (last != hi) {
      c = probe(hi, &cnt);
      if (c != GPTQ_OK) return c;
    }
  }
  *alpha_out = hi;
  if (n_outliers) *n_outliers = best;
  return GPTQ_OK;
}

// ---------------------------------------------------------------- HPTQ
//
// Bits per weight of a level array: the histogram (device), then on the host
// the total length of a Huffman code for it, which is the sum of the weights
// of all merged subtrees (a single distinct level costs 1 bit each), plus 16
// bits per group step.
#include <functional>
#include <queue>
#include <vector>

static gptq_status hptq_bpw(const int16_t* levels, int64_t rows, int64_t cols, int gs, void* ws,
                            hipStream_t st, double* bpw) {
  const QLayout L = q_layout(rows, cols, gs);
  unsigned* hist = (unsigned*)((char*)ws + L.off_hist);
  const int64_t n = rows * cols;
  GPTQ_LAUNCH(K_FILL, st, q_fill_u32_kernel<<<64, 256, 0, st>>>(hist, 65536));
  GPTQ_LAUNCH(K_Q_HIST, st,
              q_hist_kernel<<<(unsigned)cdiv(n, 256 * 16), 256, 0, st>>>(levels, n, hist));
  std::vector<unsigned> h(65536);
  GPTQ_HIP(hipMemcpyAsync(h.data(), hist, 65536 * sizeof(unsigned), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  std::priority_queue<uint64_t, std::vector<uint64_t>, std::greater<uint64_t>> pq;
  for (unsigned c : h)
    if (c) pq.push(c);
  uint64_t total = 0;
  if (pq.size() == 1) total = pq.top();
  while (pq.size() > 1) {
    const uint64_t a = pq.top();
    pq.pop();
    const uint64_t b = pq.top();
    pq.pop();
    total += a + b;
    pq.push(a + b);
  }
  *bpw = ((double)total + 16.0 * (double)rows * (double)cdiv(cols, gs)) / (double)n;
  return GPTQ_OK;
}

extern "C" gptq_status gptq_quantize_layer_hptq(const uint16_t* W, int64_t rows, int64_t cols,
                                                int64_t ldw, const float* U, const int32_t* perm,
                                                int bits, int group_size, uint32_t flags,
                                                double alpha, int16_t* levels, uint16_t* scales,
                                                uint16_t* zeros, int32_t* g_idx,
                                                double* row_loss, double* bpw, void* ws,
                                                size_t ws_bytes, void* stream) {
  if (flags & ~GPTQ_FLAG_NO_SYNC) return GPTQ_EINVAL;
  if (!(alpha > 0.0 && alpha <= 16.0)) return GPTQ_EINVAL;
  if ((flags & GPTQ_FLAG_NO_SYNC) && bpw) return GPTQ_EINVAL;
  if (rows < 0 || cols < 0) return GPTQ_EINVAL;
  if (bits < 2 || bits > 8 || !valid_gs(group_size)) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) {
    if (bpw) *bpw = 0.0;
    return GPTQ_OK;
  }
  if (!W || !U || !levels || !scales || !zeros || !row_loss || ldw < cols) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 20 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  if (!ws || ws_bytes < q_layout(rows, cols, group_size).total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  gptq_status c = quantize_enqueue(W, rows, cols, ldw, U, perm, bits, group_size, false, nullptr,
                                   scales, zeros, g_idx, row_loss, 2, alpha, nullptr,
                                   (uint16_t*)levels, ws, st);
  if (c != GPTQ_OK) return c;
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  if (bpw) {
    c = hptq_bpw(levels, rows, cols, group_size, ws, st, bpw);
    if (c != GPTQ_OK) return c;
  }
  return gptq_workspace_status(ws, stream);
}

extern "C" gptq_status gptq_hptq_search(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                        const float* U, const int32_t* perm, int bits,
                                        int group_size, uint32_t flags, double budget, int iters,
                                        double alpha_lo, double alpha_hi, double* alpha_out,
                                        int16_t* levels, uint16_t* scales, uint16_t* zeros,
                                        int32_t* g_idx, double* row_loss, double* bpw_out,
                                        void* ws, size_t ws_bytes, void* stream) {
  if (flags != 0) return GPTQ_EINVAL;
  if (!(budget > 0.0) || iters < 0 || iters > 60) return GPTQ_EINVAL;
  if (!(alpha_lo > 0.0 && alpha_lo < alpha_hi && alpha_hi <= 16.0)) return GPTQ_EINVAL;
  if (!alpha_out) return GPTQ_EINVAL;
  if (rows < 0 || cols < 0) return GPTQ_EINVAL;
  if (bits < 2 || bits > 8 || !valid_gs(group_size)) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) {
    *alpha_out = alpha_hi;
    if (bpw_out) *bpw_out = 0.0;
    return GPTQ_OK;
  }
  if (!W || !U || !levels || !scales || !zeros || !row_loss || ldw < cols) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 20 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  if (!ws || ws_bytes < q_layout(rows, cols, group_size).total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  auto probe = [&](double a, double* b) -> gptq_status {
    gptq_status r = quantize_enqueue(W, rows, cols, ldw, U, perm, bits, group_size, false,
                                     nullptr, scales, zeros, g_idx, row_loss, 2, a, nullptr,
                                     (uint16_t*)levels, ws, st);
    if (r != GPTQ_OK) return r;
    r = hptq_bpw(levels, rows, cols, group_size, ws, st, b);
    if (r != GPTQ_OK) return r;
    return gptq_workspace_status(ws, stream);
  };
  double lo = alpha_lo, hi = alpha_hi, last = hi, b = 0.0, best = 0.0;
  gptq_status c = probe(hi, &b);
  if (c != GPTQ_OK) return c;
  best = b;
  if (b <= budget) {
    for (int it = 0; it < iters; ++it) {
      const double mid = 0.5 * (lo + hi);
      c = probe(mid, &b);
      if (c != GPTQ_OK) return c;
      last = mid;
      if (b <= budget) {
        hi = mid;
        best = b;
      } else {
        lo = mid;
      }
    }
    if (last != hi) {
      c = probe(hi, &b);
      if (c != GPTQ_OK) return c;
    }
  }
  *alpha_out = hi;
  if (bpw_out) *bpw_out = best;
  return GPTQ_OK;
}
