// Shared device/host helpers of the gfx950 GPTQ library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/gptq.h"

namespace gq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQBlock = 128;  // columns per error-feedback tile

// ---------------------------------------------------------------- status
#define GQ_CHECK_ARG(cond)                 \
  do {                                     \
    if (!(cond)) return GPTQ_EINVAL;       \
  } while (0)

#define GQ_HIP(expr)                                   \
  do {                                                 \
    hipError_t _e = (expr);                            \
    if (_e != hipSuccess) return GPTQ_EHIP;            \
  } while (0)

#define GQ_LAUNCHED()                                  \
  do {                                                 \
    if (hipGetLastError() != hipSuccess) return GPTQ_EHIP; \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- timing
enum TimedKind {
  kTimeSyrk = 0,
  kTimeDiag = 1,
  kTimeFactor = 2,
  kTimeBlockQuant = 3,
  kTimeTrailing = 4,
  kTimePack = 5,
  kTimePrep = 6,
  kTimeSyrkReduce = 7,
  kTimeW4Stage = 8,
  kTimeW4Main = 9,
  kTimeAbs = 10,
  kTimeAwqSearch = 11,
  kTimeAwqApply = 12,
  kTimeForward = 13,
  kTimeKinds = 14
};

// Records a start event before and a stop event after a launch when timing
// is enabled (see gptq_timing_enable).
struct TimedScope {
  int kind;
  hipStream_t stream;
  hipEvent_t start = nullptr;
  TimedScope(int k, hipStream_t s);
  ~TimedScope();
};

// ---------------------------------------------------------------- workspace carving
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* r = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += count * sizeof(T);
    return r;
  }
};

// ---------------------------------------------------------------- numeric helpers (device)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// float -> fp16 with round-to-nearest-even (the hardware conversion rounds by
// the default mode, which is nearest-even).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 v = (_Float16)x;
  return __builtin_bit_cast(uint16_t, v);
}

// Scale and zero from the group's range (fp32 decisions, fp16 scale).
// Asymmetric: s = (xmax - xmin) / maxq and z = rne(-xmin / s).  Symmetric:
// s = max(-xmin, xmax) / (2^(bits-1) - 1) and z = 2^(bits-1), so that the
// stored code minus z is the signed code in [-2^(bits-1), 2^(bits-1) - 1].
__device__ __forceinline__ void group_scale_zero(float xmin, float xmax, float maxq, bool sym, float& s,
                                                 float& z, uint16_t& sbits) {
  xmin = fminf(xmin, 0.0f);
  xmax = fmaxf(xmax, 0.0f);
  const float half = 0.5f * (maxq + 1.0f);
  float t = sym ? __fdiv_rn(fmaxf(-xmin, xmax), half - 1.0f) : __fdiv_rn(xmax - xmin, maxq);
  uint16_t h = f32_to_f16_bits(t);
  if ((h & 0x7FFFu) == 0x7C00u) h = 0x7BFFu;          // overflow saturates to 65504
  float sv = f16_bits_to_f32(h);
  if (sv == 0.0f) {
    h = 0x3C00u;                                       // 1.0
    sv = 1.0f;
  }
  s = sv;
  sbits = h;
  z = sym ? half : fminf(fmaxf(rintf(__fdiv_rn(-xmin, sv)), 0.0f), maxq);
}

}  // namespace gq
