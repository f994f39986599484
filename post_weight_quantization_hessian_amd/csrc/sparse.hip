// SSQR's outliers in compressed sparse row form.
//
// The Geometry of LLM Quantization (gist.science), section 3, "Skalengerechte
// SpQR": weights that would overflow the integer grid are kept apart, sparse,
// in floating point. The SSQR sweep marks them at their original columns in a
// dense byte mask with their fp16 values beside it; these kernels compact that
// into CSR: row offsets (int64 [rows + 1]), column indices (int32, increasing
// within a row) and fp16 values.
//
// Three launches, no workspace: the per-row counts go to row_ptr[r + 1], one
// workgroup scans them in place, then one wave per row writes its entries in
// column order (ballot + lane prefix counts over 64 columns at a time).
// Every kernel reads the mask row by row across the wave's lanes, so loads are
// coalesced; the fill pass reads the fp16 values only at set positions.
#include "common.h"

namespace gptq {

constexpr int SP_WAVES = 4;  // rows per workgroup (one wave each)

__global__ void __launch_bounds__(64 * SP_WAVES)
sp_count_kernel(const uint8_t* __restrict__ mask, int64_t rows, int64_t cols,
                int64_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * SP_WAVES + (threadIdx.x >> 6);
  if (r >= rows) return;
  int64_t cnt = 0;
  for (int64_t c = lane; c < cols; c += 64) cnt += mask[r * cols + c] != 0;
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (lane == 0) row_ptr[r + 1] = cnt;
}

// Inclusive scan of row_ptr[1..rows] in place by one workgroup of 1024
// threads, 1024 rows per round; row_ptr[0] = 0.
__global__ void __launch_bounds__(1024)
sp_scan_kernel(int64_t* __restrict__ row_ptr, int64_t rows) {
  __shared__ int64_t part[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) row_ptr[0] = 0;
  int64_t carry = 0;
  for (int64_t base = 0; base < rows; base += 1024) {
    const int64_t r = base + t;
    int64_t v = r < rows ? row_ptr[r + 1] : 0;
    // inclusive scan within the wave
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane == 63) part[w] = v;
    __syncthreads();
    int64_t before = carry;
    for (int k = 0; k < w; ++k) before += part[k];
    int64_t total = carry;
    for (int k = 0; k < 16; ++k) total += part[k];
    if (r < rows) row_ptr[r + 1] = before + v;
    __syncthreads();  // part[] is rewritten next round
    carry = total;
  }
}

__global__ void __launch_bounds__(64 * SP_WAVES)
sp_fill_kernel(const uint8_t* __restrict__ mask, const uint16_t* __restrict__ vals,
               int64_t rows, int64_t cols, const int64_t* __restrict__ row_ptr,
               int32_t* __restrict__ col_idx, uint16_t* __restrict__ out_vals,
               int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * SP_WAVES + (threadIdx.x >> 6);
  if (r >= rows) return;
  if (row_ptr[rows] > capacity) return;  // the caller's arrays are too short
  int64_t pos = row_ptr[r];
  for (int64_t c0 = 0; c0 < cols; c0 += 64) {
    const int64_t c = c0 + lane;
    const bool set = c < cols && mask[r * cols + c] != 0;
    const uint64_t bal = __ballot(set);
    if (set) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      col_idx[pos + below] = (int32_t)c;
      out_vals[pos + below] = vals[r * cols + c];
    }
    pos += __popcll(bal);
  }
}

}  // namespace gptq

using namespace gptq;

extern "C" gptq_status gptq_ssqr_outliers_csr(const uint8_t* mask, const uint16_t* vals,
                                              int64_t rows, int64_t cols, int64_t* row_ptr,
                                              int32_t* col_idx, uint16_t* csr_vals,
                                              int64_t capacity, uint32_t flags, int64_t* nnz,
                                              void* stream) {
  if (flags & ~GPTQ_FLAG_NO_SYNC) return GPTQ_EINVAL;
  if (rows < 0 || cols < 0 || capacity < 0) return GPTQ_EINVAL;
  if (cols > ((int64_t)1 << 31) - 1) return GPTQ_EINVAL;
  if (!row_ptr) return GPTQ_EINVAL;
  if (rows > 0 && cols > 0 && (!mask || !vals)) return GPTQ_EINVAL;
  if (capacity > 0 && (!col_idx || !csr_vals)) return GPTQ_EINVAL;
  if ((flags & GPTQ_FLAG_NO_SYNC) && nnz) return GPTQ_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int64_t nb = cdiv(rows, SP_WAVES);
  if (nb > 0x7fffffff) return GPTQ_EINVAL;
  // (rows == 0: only the scan runs, writing row_ptr[0] = 0; cols == 0: every
  // count is 0 and the fill writes nothing)
  if (rows > 0)
    GPTQ_LAUNCH(K_SP_CSR, st,
                sp_count_kernel<<<(unsigned)nb, 64 * SP_WAVES, 0, st>>>(mask, rows, cols,
                                                                        row_ptr));
  GPTQ_LAUNCH(K_SP_CSR, st, sp_scan_kernel<<<1, 1024, 0, st>>>(row_ptr, rows));
  if (rows > 0 && cols > 0)
    GPTQ_LAUNCH(K_SP_CSR, st,
                sp_fill_kernel<<<(unsigned)nb, 64 * SP_WAVES, 0, st>>>(
                    mask, vals, rows, cols, row_ptr, col_idx, csr_vals, capacity));
  if (flags & GPTQ_FLAG_NO_SYNC) return GPTQ_OK;
  int64_t total = 0;
  GPTQ_HIP(hipMemcpyAsync(&total, row_ptr + rows, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  if (nnz) *nnz = total;
  return total > capacity ? GPTQ_EINVAL : GPTQ_OK;
}
