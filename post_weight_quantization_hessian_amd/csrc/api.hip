// Status strings, the fp16 rounding utility and the optional HIP-event
// kernel profiler of the GPTQ library.
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace gptq {

static const char* const kKernelNames[K_COUNT] = {
    "hessian_tile", "hessian_reduce", "prepare_diag", "prepare_perm", "prepare_gather",
    "chol_potrf", "chol_trsm", "chol_syrk", "trtri_t", "trtri_x", "prepare_uout",
    "quant_init", "quant_permute", "quant_gemm", "quant_sweep", "quant_finalize", "fill",
    "trtri_diag", "chol_potrf_syrk", "trtri_sum", "chol_col", "minpivot_step",
    "minpivot_update", "hessian_digits", "hessian_split8", "quant_hist", "chmc_front",
    "chmc_update", "chmc_sweep", "ssqr_csr", "hptq_code"};

struct ProfRec {
  int kid;
  hipEvent_t a, b;
};

// The kernel-timing hooks are the library's only state that outlives a call.
// The mask is atomic; the start events of launches in flight are per thread
// (a begin and its end always come from the same call, on one thread); the
// finished records are shared and guarded by a mutex, so calls from several
// host threads on several streams may be timed together.
static std::atomic<uint32_t> g_prof_mask{0u};
static thread_local hipError_t g_last_error = hipSuccess;

void note_hip_error(hipError_t e) { g_last_error = e; }
static std::mutex g_prof_mutex;
static std::vector<ProfRec> g_prof;  // guarded by g_prof_mutex
static thread_local std::vector<hipEvent_t> g_open;  // start events pending an end

static bool selected(int kid) { return (g_prof_mask.load(std::memory_order_relaxed) >> kid) & 1u; }

// A null start event marks a launch whose start could not be recorded; the
// matching prof_end then records nothing.
void prof_begin(int kid, hipStream_t s) {
  if (!selected(kid)) return;
  hipEvent_t a = nullptr;
  if (hipEventCreate(&a) != hipSuccess) {
    a = nullptr;
  } else if (hipEventRecord(a, s) != hipSuccess) {
    (void)hipEventDestroy(a);
    a = nullptr;
  }
  g_open.push_back(a);
}

void prof_end(int kid, hipStream_t s) {
  if (!selected(kid) || g_open.empty()) return;
  hipEvent_t a = g_open.back();
  g_open.pop_back();
  if (!a) return;
  hipEvent_t b;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  (void)hipEventRecord(b, s);
  std::lock_guard<std::mutex> lock(g_prof_mutex);
  g_prof.push_back({kid, a, b});
}

}  // namespace gptq

using namespace gptq;

extern "C" const char* gptq_status_string(gptq_status status) {
  // a C caller may pass any int: read it without an enum-typed load (outside
  // the enumerators' range that load is undefined in C++)
  int code = 0;
  static_assert(sizeof(code) == sizeof(status), "gptq_status is int-sized");
  std::memcpy(&code, &status, sizeof code);
  switch (code) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTSPD: return "damped Hessian is not positive definite";
    case GPTQ_EHIP: return "HIP runtime error";
    case GPTQ_EWORKSPACE: return "workspace missing or too small";
    case GPTQ_ENONFINITE: return "non-finite weight or fp16 scale overflow";
  }
  return "unknown status";
}

extern "C" gptq_status gptq_fp16_round_host(const double* in, uint16_t* out, int64_t n) {
  if (n < 0 || (n > 0 && (!in || !out))) return GPTQ_EINVAL;
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16_rne(in[i]);
  return GPTQ_OK;
}

extern "C" int gptq_version(void) { return 1; }

extern "C" gptq_status gptq_workspace_status(const void* ws, void* stream) {
  if (!ws) return GPTQ_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  unsigned h = 0;
  GPTQ_HIP(hipMemcpyAsync(&h, ws, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  return status_from_bits(h);
}

extern "C" const char* gptq_last_error_string(void) {
  if (g_last_error == hipSuccess) return "no error";
  return hipGetErrorString(g_last_error);
}

extern "C" gptq_status gptq_profile_enable(uint32_t kernel_mask) {
  g_prof_mask.store(kernel_mask, std::memory_order_relaxed);
  return GPTQ_OK;
}

extern "C" int gptq_profile_kernel_count(void) { return K_COUNT; }

extern "C" const char* gptq_profile_kernel_name(int id) {
  if (id < 0 || id >= K_COUNT) return nullptr;
  return kKernelNames[id];
}

extern "C" gptq_status gptq_profile_read(double* totals_ms, int64_t* launches) {
  if (!totals_ms || !launches) return GPTQ_EINVAL;
  for (int k = 0; k < K_COUNT; ++k) {
    totals_ms[k] = 0.0;
    launches[k] = 0;
  }
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    recs.swap(g_prof);
  }
  gptq_status st = GPTQ_OK;
  for (auto& r : recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) st = GPTQ_EHIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      totals_ms[r.kid] += ms;
      launches[r.kid] += 1;
    } else {
      st = GPTQ_EHIP;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  return st;
}
