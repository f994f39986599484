// gptq_quantize_layer for callers that cannot allocate device memory.
//
// The column sweep and its lazy update need scratch beyond the inputs and
// outputs (sweep-order weights and codes, scaled errors, split-K partials,
// the status word), which gptq_quantize_layer takes as a caller workspace.
// This variant takes it from one fixed array of the library instead: a
// file-scope device array, of which every device holds its own copy from the
// first call there until the process ends. Its address on a device is looked
// up once, with that device current, and kept; the kernels receive that
// address exactly as they receive a caller's workspace.
#include <mutex>

#include "common.h"

namespace gptq {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;  // 64 MiB per device
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];  // guarded by g_scratch_mutex

// The device address of `scratch` on the current device (looked up on the
// first call there). The host-side name of the array is not a device
// address; only this pointer is passed on.
static gptq_status scratch_on_current_device(void** out) {
  int dev = -1;
  GPTQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return GPTQ_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    GPTQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return GPTQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

extern "C" gptq_status gptq_quantize_layer_noalloc(const uint16_t* W, int64_t rows, int64_t cols,
                                                   int64_t ldw, const float* U,
                                                   const int32_t* perm, int bits, int group_size,
                                                   uint32_t flags, uint8_t* codes,
                                                   uint16_t* scales, uint16_t* zeros,
                                                   int32_t* g_idx, double* row_loss,
                                                   void* stream) {
  // The argument checks of gptq_quantize_layer itself, before anything is
  // enqueued: with no workspace it returns GPTQ_EINVAL for a bad call,
  // GPTQ_OK for an empty layer (nothing to do) and GPTQ_EWORKSPACE for a
  // valid one.
  const gptq_status v = gptq_quantize_layer(W, rows, cols, ldw, U, perm, bits, group_size, flags,
                                            codes, scales, zeros, g_idx, row_loss, nullptr, 0,
                                            stream);
  if (v != GPTQ_EWORKSPACE) return v;
  const size_t need = gptq_quantize_workspace_bytes(rows, cols, group_size);
  if (need == 0 || need > NOALLOC_SCRATCH_BYTES) return GPTQ_EWORKSPACE;
  int dev = -1;
  GPTQ_HIP(hipGetDevice(&dev));
  if (stream) {
    hipDevice_t sdev = -1;
    GPTQ_HIP(hipStreamGetDevice((hipStream_t)stream, &sdev));
    if (sdev != dev) return GPTQ_EINVAL;
  }
  void* ws = nullptr;
  const gptq_status s = scratch_on_current_device(&ws);
  if (s != GPTQ_OK) return s;
  return gptq_quantize_layer(W, rows, cols, ldw, U, perm, bits, group_size, flags, codes, scales,
                             zeros, g_idx, row_loss, ws, NOALLOC_SCRATCH_BYTES, stream);
}
