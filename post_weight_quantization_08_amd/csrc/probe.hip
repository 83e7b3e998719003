// On-device reference rates for measurement: a loop of MFMAs on registers
// (the matrix-core rate the GPU sustains with random operands, whatever clock
// it holds under that load) and a plain device copy (the HBM rate a simple
// streaming kernel reaches).  They give the phases of the path a measured
// ceiling next to the published one.
#include "common.h"

namespace gq {

typedef double f64x4_p __attribute__((ext_vector_type(4)));

// 32-bit hash of a lane's id and a salt (integer mixing only).
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Two 16-bit values of magnitude in [0.5, 1) with random sign and mantissa
// (fp16: exponent 14; bf16: exponent 126), packed in one word.
template <bool kF16>
__device__ __forceinline__ uint32_t probe_pair(uint32_t h) {
  const uint32_t lo = h & 0xFFFFu, hi = h >> 16;
  uint32_t a, b;
  if constexpr (kF16) {
    a = (lo & 0x83FFu) | 0x3800u;
    b = (hi & 0x83FFu) | 0x3800u;
  } else {
    a = (lo & 0x807Fu) | 0x3F00u;
    b = (hi & 0x807Fu) | 0x3F00u;
  }
  return a | (b << 16);
}

// kKind 0: f16 32x32x16, 1: bf16 32x32x16, 2: f64 16x16x4.  Four independent
// accumulators per wave, so consecutive MFMAs never wait on each other.  The
// operands stay the same from one MFMA to the next (only the accumulators
// change), so the matrix cores' inputs do not toggle: the rate under the
// least data-dependent power (mfma_stream_probe_kernel feeds new operands).
template <int kKind>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  if constexpr (kKind == 2) {
    const double a = 0.5 + (probe_hash(id) & 0xFFFF) * (1.0 / 131072.0);
    const double b = 0.5 + (probe_hash(id ^ 0x9E3779B9u) & 0xFFFF) * (1.0 / 131072.0);
    f64x4_p acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = (f64x4_p){0.0, 0.0, 0.0, 0.0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[k], 0, 0, 0);
    }
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    sink[id] = (float)s;
  } else {
    u32x4 a, b;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[c] = probe_pair<kKind == 0>(probe_hash(id * 8u + c));
      b[c] = probe_pair<kKind == 0>(probe_hash(id * 8u + 4u + c));
    }
    f32x16 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (kKind == 0)
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                         acc[k], 0, 0, 0);
        else
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc[k], 0, 0, 0);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[k][r];
    sink[id] = s;
  }
}

// The same loop with eight random operand sets per lane taken in turn, so
// every MFMA sees new A and B bits, as in a kernel that streams its operands:
// the rate the matrix cores sustain when the power their inputs draw is that
// of random data (kF16: f16, else bf16; 32x32x16).
template <bool kF16>
__global__ __launch_bounds__(256) void mfma_stream_probe_kernel(int iters, float* __restrict__ sink) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  u32x4 a[8], b[8];
#pragma unroll
  for (int v = 0; v < 8; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[v][c] = probe_pair<kF16>(probe_hash(id * 64u + 8u * v + c));
      b[v][c] = probe_pair<kF16>(probe_hash(id * 64u + 8u * v + 4u + c));
    }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int k = v & 3;
      if constexpr (kF16)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[v]), __builtin_bit_cast(f16x8, b[v]),
                                                       acc[k], 0, 0, 0);
      else
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[v]),
                                                        __builtin_bit_cast(bf16x8, b[v]), acc[k], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  sink[id] = s;
}

// dst = src, 16 bytes per lane per step, four steps in flight per lane.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    dst[i] = v0;
    dst[i + stride] = v1;
    dst[i + 2 * stride] = v2;
    dst[i + 3 * stride] = v3;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

constexpr int kProbeBlocks = 2048;   // the largest grid: 8 workgroups (32 waves) per CU

// Best of `reps` timed launches of `launch` (after one untimed one), in ms.
template <class F>
static gptq_status best_ms(hipStream_t st, int reps, F launch, double* out) {
  hipEvent_t e0, e1;
  GQ_HIP(hipEventCreate(&e0));
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return GPTQ_EHIP;
  }
  gptq_status r = GPTQ_OK;
  double best = 1e300;
  for (int i = 0; i <= reps && r == GPTQ_OK; ++i) {
    if (hipEventRecord(e0, st) != hipSuccess) r = GPTQ_EHIP;
    launch();
    if (hipGetLastError() != hipSuccess) r = GPTQ_EHIP;
    if (r == GPTQ_OK && hipEventRecord(e1, st) != hipSuccess) r = GPTQ_EHIP;
    if (r == GPTQ_OK && hipEventSynchronize(e1) != hipSuccess) r = GPTQ_EHIP;
    float ms = 0.f;
    if (r == GPTQ_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) r = GPTQ_EHIP;
    if (i > 0 && ms < best) best = ms;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  *out = best;
  return r;
}

}  // namespace gq

using namespace gq;

extern "C" size_t gptq_probe_sink_bytes(void) { return (size_t)kProbeBlocks * 256 * sizeof(float); }

extern "C" gptq_status gptq_probe_mfma(int32_t kind, int32_t iters, float* sink, double* tflops_out, void* stream) {
  GQ_CHECK_ARG(kind >= 0 && kind <= 4 && iters >= 1 && iters <= (1 << 24) && sink && tflops_out);
  if (kind >= 3) iters += iters & 1;   // the streaming loop takes two steps at a time
  hipStream_t st = static_cast<hipStream_t>(stream);
  const double per = kind == 2 ? 2.0 * 16 * 16 * 4 : 2.0 * 32 * 32 * 16;
  double best = 0.0;
  // 1, 2, 4 and 8 waves per SIMD: the best of them is the rate reported
  for (int blocks = 256; blocks <= kProbeBlocks; blocks *= 2) {
    double ms = 0.0;
    auto launch = [&]() {
      if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, st, iters, sink);
      else if (kind == 1) hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, st, iters, sink);
      else if (kind == 2) hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(blocks), dim3(256), 0, st, iters, sink);
      else if (kind == 3) hipLaunchKernelGGL(mfma_stream_probe_kernel<true>, dim3(blocks), dim3(256), 0, st, iters, sink);
      else hipLaunchKernelGGL(mfma_stream_probe_kernel<false>, dim3(blocks), dim3(256), 0, st, iters, sink);
    };
    gptq_status r = best_ms(st, 3, launch, &ms);
    if (r != GPTQ_OK) return r;
    const double flops = per * 4.0 * iters * (double)blocks * 4.0;   // 4 MFMAs per step, 4 waves per block
    best = std::max(best, flops / (ms * 1e-3) / 1e12);
  }
  *tflops_out = best;
  return GPTQ_OK;
}

extern "C" gptq_status gptq_probe_copy(const void* src, void* dst, size_t bytes, double* gbs_out, double* ms_out,
                                       void* stream) {
  GQ_CHECK_ARG(src && dst && gbs_out && bytes >= 16 && bytes % 16 == 0);
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(src) % 16 == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n16 = (int64_t)(bytes / 16);
  // grids of 1024 .. 16384 workgroups: the fastest is the rate reported
  double best_ms_all = 1e300;
  for (int64_t blocks = 1024; blocks <= 16384; blocks *= 2) {
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(n16, 256), blocks));
    double ms = 0.0;
    auto launch = [&]() {
      hipLaunchKernelGGL(copy_probe_kernel, dim3(grid), dim3(256), 0, st, static_cast<const u32x4*>(src),
                         static_cast<u32x4*>(dst), n16);
    };
    gptq_status r = best_ms(st, 3, launch, &ms);
    if (r != GPTQ_OK) return r;
    best_ms_all = std::min(best_ms_all, ms);
  }
  *gbs_out = 2.0 * (double)bytes / (best_ms_all * 1e-3) / 1e9;
  if (ms_out) *ms_out = best_ms_all;
  return GPTQ_OK;
}
