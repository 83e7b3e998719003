// Dense packing of integer codes ("INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍",
// section 一: 128 four-bit codes take 64 bytes).  Pure byte work, HBM-bound.
#include "common.h"

namespace gq {

// packed[r][c/2] = codes[r][col(c)] | codes[r][col(c+1)] << 4 with col = perm
// or identity; one thread per output byte.
__global__ __launch_bounds__(256) void pack4_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t cols,
                                                    const int32_t* __restrict__ perm, uint8_t* __restrict__ packed) {
  const int64_t half = cols / 2;
  const int64_t n = rows * half;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / half, c = e % half;
    const uint8_t* src = codes + r * cols;
    const int64_t k0 = perm ? perm[2 * c] : 2 * c, k1 = perm ? perm[2 * c + 1] : 2 * c + 1;
    packed[e] = (uint8_t)((src[k0] & 15u) | ((src[k1] & 15u) << 4));
  }
}

// Eight codes of `bits` bits -> `bits` bytes, little-endian bit order.
__global__ __launch_bounds__(256) void packbits_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t cols,
                                                       int bits, uint8_t* __restrict__ packed) {
  const int64_t groups = cols / 8;
  const int64_t n = rows * groups;
  const uint64_t mask = (1u << bits) - 1u;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / groups, gi = e % groups;
    const uint8_t* src = codes + r * cols + gi * 8;
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v |= ((uint64_t)src[i] & mask) << (bits * i);
    uint8_t* dst = packed + r * (cols * bits / 8) + gi * bits;
    for (int i = 0; i < bits; ++i) dst[i] = (uint8_t)(v >> (8 * i));
  }
}

// General case ((cols * bits) % 8 == 0, cols % 8 != 0): one thread per output
// byte gathers its 8 stream bits.
__global__ __launch_bounds__(256) void packbits_bytewise_kernel(const uint8_t* __restrict__ codes, int64_t rows,
                                                                int64_t cols, int bits, uint8_t* __restrict__ packed) {
  const int64_t rb = cols * bits / 8;
  const int64_t n = rows * rb;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / rb, byte = e % rb;
    uint32_t v = 0;
    for (int bit = 0; bit < 8; ++bit) {
      const int64_t sb = byte * 8 + bit;
      const uint32_t code = codes[r * cols + sb / bits];
      v |= ((code >> (sb % bits)) & 1u) << bit;
    }
    packed[e] = (uint8_t)v;
  }
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_pack_int4(const uint8_t* codes, int64_t rows, int64_t cols, uint8_t* packed,
                                      void* stream) {
  GQ_CHECK_ARG(rows >= 0 && cols >= 0 && cols % 2 == 0);
  if (rows == 0 || cols == 0) return GPTQ_OK;
  GQ_CHECK_ARG(codes && packed);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n = rows * (cols / 2);
  TimedScope ts(kTimePack, st);
  hipLaunchKernelGGL(pack4_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st, codes,
                     rows, cols, nullptr, packed);
  GQ_LAUNCHED();
  return GPTQ_OK;
}

extern "C" gptq_status gptq_pack_int4_permuted(const uint8_t* codes, int64_t rows, int64_t cols, const int32_t* perm,
                                               uint8_t* packed, void* stream) {
  GQ_CHECK_ARG(rows >= 0 && cols >= 0 && cols % 2 == 0);
  if (rows == 0 || cols == 0) return GPTQ_OK;
  GQ_CHECK_ARG(codes && packed && perm);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n = rows * (cols / 2);
  TimedScope ts(kTimePack, st);
  hipLaunchKernelGGL(pack4_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st, codes,
                     rows, cols, perm, packed);
  GQ_LAUNCHED();
  return GPTQ_OK;
}

extern "C" gptq_status gptq_pack_bits(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits,
                                      uint8_t* packed, void* stream) {
  GQ_CHECK_ARG(rows >= 0 && cols >= 0 && bits >= 2 && bits <= 8 && (cols * bits) % 8 == 0);
  if (rows == 0 || cols == 0) return GPTQ_OK;
  GQ_CHECK_ARG(codes && packed);
  hipStream_t st = static_cast<hipStream_t>(stream);
  TimedScope ts(kTimePack, st);
  if (cols % 8 == 0) {
    const int64_t n = rows * (cols / 8);
    hipLaunchKernelGGL(packbits_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, st,
                       codes, rows, cols, (int)bits, packed);
  } else {
    const int64_t n = rows * (cols * bits / 8);
    hipLaunchKernelGGL(packbits_bytewise_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256),
                       0, st, codes, rows, cols, (int)bits, packed);
  }
  GQ_LAUNCHED();
  return GPTQ_OK;
}
