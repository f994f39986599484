// Shared device/host helpers of the gfx950 GPTQ library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "gptq.h"

namespace gptq {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16 __attribute__((ext_vector_type(16)));

// Device status word bits (first word of every workspace).
enum : unsigned { ST_NOTSPD = 1u, ST_NONFINITE = 2u, ST_BADPERM = 4u };

inline gptq_status status_from_bits(unsigned b) {
  if (b & ST_BADPERM) return GPTQ_EINVAL;
  if (b & ST_NOTSPD) return GPTQ_ENOTSPD;
  if (b & ST_NONFINITE) return GPTQ_ENONFINITE;
  return GPTQ_OK;
}

// Kernel classes for the optional HIP-event profiler.
enum KernelId {
  K_HESS_TILE = 0, K_HESS_REDUCE, K_PREP_DIAG, K_PREP_PERM, K_PREP_GATHER, K_CHOL_POTRF,
  K_CHOL_TRSM, K_CHOL_SYRK, K_TRTRI_ROW, K_TRTRI_UPDATE, K_PREP_UOUT, K_Q_INIT, K_Q_PERMUTE,
  K_Q_GEMM, K_Q_SWEEP, K_Q_FINALIZE, K_FILL, K_TRTRI_DIAG, K_CHOL_STEP, K_TRTRI_SUM, K_CHOL_COL, K_MP_STEP,
  K_MP_UPDATE, K_HESS_DIGITS, K_HESS_SPLIT8, K_Q_HIST, K_CH_FRONT, K_CH_UPDATE, K_CH_SWEEP,
  K_SP_CSR, K_HF, K_COUNT
};

// Launch bracketing for the profiler (defined in api.hip).
void prof_begin(int kid, hipStream_t s);
void prof_end(int kid, hipStream_t s);
// Remember the last HIP error seen by the library (reported by
// gptq_last_error_string).
void note_hip_error(hipError_t e);

struct ProfScope {
  int kid;
  hipStream_t s;
  ProfScope(int k, hipStream_t st) : kid(k), s(st) { prof_begin(kid, s); }
  ~ProfScope() { prof_end(kid, s); }
};

// A launch: clear any stale error left by earlier HIP calls of the process,
// launch, and report a launch failure as GPTQ_EHIP.
#define GPTQ_LAUNCH(kid, stream, ...)                          \
  do {                                                         \
    (void)hipGetLastError();                                   \
    ::gptq::ProfScope _ps((kid), (stream));                    \
    __VA_ARGS__;                                               \
    const hipError_t _e = hipGetLastError();                   \
    if (_e != hipSuccess) {                                    \
      ::gptq::note_hip_error(_e);                              \
      return GPTQ_EHIP;                                        \
    }                                                          \
  } while (0)

#define GPTQ_HIP(call)                                         \
  do {                                                         \
    const hipError_t _e = (call);                              \
    if (_e != hipSuccess) {                                    \
      ::gptq::note_hip_error(_e);                              \
      return GPTQ_EHIP;                                        \
    }                                                          \
  } while (0)

// ---------------------------------------------------------------- fp16 bits

// Nearest-even binary16 of a double, computed from the double's bits directly
// (no intermediate fp32 rounding). Handles subnormals, overflow to Inf, NaN.
__host__ __device__ inline uint16_t f64_to_f16_rne(double x) {
  union { double d; uint64_t u; } c;
  c.d = x;
  const uint64_t b = c.u;
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int e = (int)((b >> 52) & 0x7ff);
  const uint64_t m = b & ((1ull << 52) - 1);
  if (e == 0x7ff) return sign | 0x7c00u | (m ? 0x200u : 0u);
  if (e == 0) return sign;  // fp64 subnormal: far below the fp16 range
  int E = e - 1023;
  const uint64_t mant = (1ull << 52) | m;  // 53 significant bits
  int shift = (E >= -14) ? 42 : 42 + (-14 - E);
  if (shift > 60) return sign;
  uint64_t q = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E >= -14) {
    if (q == 2048) { q = 1024; ++E; }
    if (E > 15) return sign | 0x7c00u;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q & 0x3ff);
  }
  return sign | (uint16_t)q;  // subnormal; q == 1024 is the smallest normal
}

__host__ __device__ inline double f16_to_f64(uint16_t h) {
  const int s = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  double v;
  if (e == 0) v = (double)m * (1.0 / 16777216.0);  // m * 2^-24
  else if (e == 31) v = m ? __builtin_nan("") : __builtin_inf();
  else v = (double)(1024 + m) * __builtin_ldexp(1.0, e - 25);
  return s ? -v : v;
}

// The nearest-even binary16 value of a double, as a double: x scaled by a
// power of two so that one fp16 unit in the last place is 1 (2^(e-10) for
// the binade 2^e, 2^-24 below the normal range), rounded to an integer
// (ties to even), scaled back; beyond the largest finite fp16 value the
// result is infinite. Exact: the scalings are by powers of two.
__device__ inline double f16_round_f64(double x) {
  const int e = (int)((__double_as_longlong(x) >> 52) & 0x7ff) - 1023;
  const int u = e - 10 > -24 ? e - 10 : -24;
  const double r = __builtin_ldexp(__builtin_rint(__builtin_ldexp(x, -u)), u);
  return __builtin_fabs(r) > 65504.0 ? __builtin_copysign(__builtin_inf(), x) : r;
}

// ---------------------------------------------------------------- misc

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Workgroup id remapped so that consecutive logical ids land on the same XCD
// (hardware dispatches workgroup ids round-robin over the 8 XCDs).
// DPP moves of an fp64 value (two 32-bit halves: the quad and row patterns
// exist for 32-bit moves only). Every pattern used writes every lane, so the
// "old" operand is the source itself.
template <int CTRL>
__device__ inline double dpp_f64(double v) {
  union { double d; int i[2]; } a, b;
  a.d = v;
  b.i[0] = __builtin_amdgcn_update_dpp(a.i[0], a.i[0], CTRL, 0xF, 0xF, false);
  b.i[1] = __builtin_amdgcn_update_dpp(a.i[1], a.i[1], CTRL, 0xF, 0xF, false);
  return b.d;
}
// row_newbcast: lane N of each 16-lane row, to the whole row. It is the one
// DPP pattern that also exists for 64-bit moves, so this is a single
// v_mov_b64_dpp rather than a move of each 32-bit half.
template <int N>
__device__ inline double row_bcast(double v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + N, 0xF, 0xF, false);
}
// row_newbcast whose result also depends on `dep` (it is the "old" operand,
// which a full-mask broadcast never uses): keeps the compiler from hoisting
// the broadcast above the computation of dep
template <int N>
__device__ inline double row_bcast_dep(double v, double dep) {
  return __builtin_amdgcn_update_dpp(dep, v, 0x150 + N, 0xF, 0xF, false);
}
__device__ inline double row_bcast_dep_i(double v, double dep, int n) {
  switch (n) {
    case 0: return row_bcast_dep<0>(v, dep);
    case 1: return row_bcast_dep<1>(v, dep);
    case 2: return row_bcast_dep<2>(v, dep);
    case 3: return row_bcast_dep<3>(v, dep);
    case 4: return row_bcast_dep<4>(v, dep);
    case 5: return row_bcast_dep<5>(v, dep);
    case 6: return row_bcast_dep<6>(v, dep);
    case 7: return row_bcast_dep<7>(v, dep);
    case 8: return row_bcast_dep<8>(v, dep);
    case 9: return row_bcast_dep<9>(v, dep);
    case 10: return row_bcast_dep<10>(v, dep);
    case 11: return row_bcast_dep<11>(v, dep);
    case 12: return row_bcast_dep<12>(v, dep);
    case 13: return row_bcast_dep<13>(v, dep);
    case 14: return row_bcast_dep<14>(v, dep);
    default: return row_bcast_dep<15>(v, dep);
  }
}
// the same for an index that is a constant after loop unrolling
__device__ inline double row_bcast_i(double v, int n) {
  switch (n) {
    case 0: return row_bcast<0>(v);
    case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);
    case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);
    case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);
    case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);
    case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v);
    case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v);
    case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v);
    default: return row_bcast<15>(v);
  }
}

__device__ inline int xcd_remap(int bid, int nblocks) {
  const int nx = 8;
  if (nblocks < nx) return bid;
  const int per = nblocks / nx;
  const int rem = nblocks - per * nx;
  const int x = bid % nx;
  const int k = bid / nx;
  // XCD x owns logical ids [start(x), start(x) + count(x)) where the first
  // `rem` XCDs get one extra id.
  if (k >= per + (x < rem ? 1 : 0)) return bid;  // not reached for exact grids
  const int start = x * per + (x < rem ? x : rem);
  return start + k;
}

}  // namespace gptq
