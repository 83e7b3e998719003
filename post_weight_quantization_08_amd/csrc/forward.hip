// Forward of a quantized layer for sequential calibration ("3. 模型量化技术(下)",
// section "GPTQ：基于二阶信息的后训练量化", pseudocode: every layer is calibrated
// on its own inputs; here the next layer's inputs are the outputs of the
// already quantized one):  Y = round(act(X Q^T)) with Q the dequantized
// weights (fp32), act none / ReLU / SiLU, and Y in the activations' 16-bit
// format (round to nearest even).
//
// MFMA (v_mfma_f32_32x32x16_bf16) on split operands: Q as two bf16 terms
// (hi + lo, relative error about 2^-17), X exactly (bf16: one term; fp16:
// two), products hi*hi + hi*lo (+ lo*hi for fp16 activations), fp32
// accumulation.  Workgroup tile 128 tokens x 128 output channels, 4 waves of
// 64 x 64; the k dimension staged through LDS 32 at a time.
#include "common.h"

namespace gq {

constexpr int kFwTile = 128;
constexpr int kFwK = 32;

// Eight consecutive values of a row, as loaded (fp32: two 16-byte halves).
template <int kDt>
struct Raw8 {
  u32x4 v[kDt == GPTQ_F32 ? 2 : 1];
};

template <int kDt>
__device__ __forceinline__ Raw8<kDt> fw_load8(const void* p, size_t i, bool live) {
  Raw8<kDt> r;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  if constexpr (kDt == GPTQ_F32) {
    r.v[0] = live ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(p) + i) : z4;
    r.v[1] = live ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(p) + i + 4) : z4;
  } else {
    r.v[0] = live ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i) : z4;
  }
  return r;
}

// The eight values as two bf16 terms (hi, lo).
template <int kDt>
__device__ __forceinline__ void fw_split8(const Raw8<kDt>& r, u32x4& hi, u32x4& lo) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (kDt == GPTQ_F32) {
      v[e] = __uint_as_float(r.v[e >> 2][e & 3]);
    } else {
      const uint32_t h = (r.v[0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      v[e] = kDt == GPTQ_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
    }
  }
  uint32_t h4[4] = {0u, 0u, 0u, 0u}, l4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = f32_to_bf16_bits(v[e]);
    h4[e >> 1] |= h << (16 * (e & 1));
    l4[e >> 1] |= f32_to_bf16_bits(v[e] - bf16_bits_to_f32(h)) << (16 * (e & 1));
  }
  hi = u32x4{h4[0], h4[1], h4[2], h4[3]};
  lo = u32x4{l4[0], l4[1], l4[2], l4[3]};
}

__device__ __forceinline__ float fw_act(float v, int act) {
  if (act == 1) return fmaxf(v, 0.0f);
  if (act == 2) return v / (1.0f + expf(-v));
  return v;
}

// kDt: activations' format (fp16 / bf16; fp32 inputs and outputs also work).
template <int kDt>
__global__ __launch_bounds__(256) void forward_kernel(const void* __restrict__ X, int64_t ld_x, int64_t n_tok, int d,
                                                      const float* __restrict__ Q, int64_t ld_q, int64_t d_out, int act,
                                                      void* __restrict__ Y, int64_t ld_y) {
  constexpr bool kXlo = kDt != GPTQ_BF16;
  constexpr int kAT = kXlo ? 2 : 1;
  constexpr int kLd = kFwK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sA[kAT][kFwTile * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kFwTile * kLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kFwTile;   // tokens
  const int64_t n0 = (int64_t)blockIdx.y * kFwTile;   // output channels
  const int wt = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const int srow = tid >> 2, sk = (tid & 3) * 8;
  // the next k-step's rows are loaded into registers while this one computes
  Raw8<kDt> rx[2];
  Raw8<GPTQ_F32> rq[2];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = srow + 64 * h;
      const int64_t ta = t0 + rr, nb = n0 + rr;
      rx[h] = fw_load8<kDt>(X, (size_t)(ta < n_tok ? ta : 0) * ld_x + k0 + sk, ta < n_tok);
      rq[h] = fw_load8<GPTQ_F32>(Q, (size_t)(nb < d_out ? nb : 0) * ld_q + k0 + sk, nb < d_out);
    }
  };
  load_step(0);
  for (int k0 = 0; k0 < d; k0 += kFwK) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = srow + 64 * h;
      u32x4 xh, xl, qh, ql;
      fw_split8<kDt>(rx[h], xh, xl);
      fw_split8<GPTQ_F32>(rq[h], qh, ql);
      *reinterpret_cast<u32x4*>(&sA[0][rr * kLd + sk]) = xh;
      if constexpr (kXlo) *reinterpret_cast<u32x4*>(&sA[kAT - 1][rr * kLd + sk]) = xl;
      *reinterpret_cast<u32x4*>(&sB[0][rr * kLd + sk]) = qh;
      *reinterpret_cast<u32x4*>(&sB[1][rr * kLd + sk]) = ql;
    }
    __syncthreads();
    if (k0 + kFwK < d) load_step(k0 + kFwK);
#pragma unroll
    for (int ks = 0; ks < kFwK; ks += 16) {
      const int kk = ks + 8 * (lane >> 5);
      u32x4 a[kAT][2], b[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int term = 0; term < kAT; ++term)
          a[term][i] = *reinterpret_cast<const u32x4*>(&sA[term][(wt + 32 * i + (lane & 31)) * kLd + kk]);
#pragma unroll
        for (int term = 0; term < 2; ++term)
          b[term][i] = *reinterpret_cast<const u32x4*>(&sB[term][(wn + 32 * i + (lane & 31)) * kLd + kk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0][i]),
                                                              __builtin_bit_cast(bf16x8, b[0][j]), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0][i]),
                                                              __builtin_bit_cast(bf16x8, b[1][j]), acc[i][j], 0, 0, 0);
          if constexpr (kXlo)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kAT - 1][i]),
                                                                __builtin_bit_cast(bf16x8, b[0][j]), acc[i][j], 0, 0,
                                                                0);
        }
    }
    __syncthreads();
  }
  // D lane layout (32 x 32 block): element e of lane l is row 8 (e / 4) +
  // 4 (l / 32) + e % 4 (token), column l % 32 (output channel)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = t0 + wt + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t n = n0 + wn + 32 * j + (lane & 31);
        if (t < n_tok && n < d_out) {
          const float v = fw_act(acc[i][j][e], act);
          if constexpr (kDt == GPTQ_F32) static_cast<float*>(Y)[(size_t)t * ld_y + n] = v;
          else if constexpr (kDt == GPTQ_F16) static_cast<uint16_t*>(Y)[(size_t)t * ld_y + n] = f32_to_f16_bits(v);
          else static_cast<uint16_t*>(Y)[(size_t)t * ld_y + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_layer_forward(const void* X, int32_t x_dtype, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                          const float* Q, int64_t d_out, int64_t ld_q, int32_t act, void* Y,
                                          int64_t ld_y, void* stream) {
  GQ_CHECK_ARG(X && Q && Y);
  GQ_CHECK_ARG(x_dtype == GPTQ_F32 || x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(act >= 0 && act <= 2);
  GQ_CHECK_ARG(n_tok >= 0 && d_out >= 1 && d_in >= kFwK && d_in % kFwK == 0);
  GQ_CHECK_ARG(ld_x >= d_in && ld_q >= d_in && ld_y >= d_out);
  const int64_t es = x_dtype == GPTQ_F32 ? 4 : 2;
  GQ_CHECK_ARG((ld_x * es) % 16 == 0 && ld_q % 4 == 0);
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(X) % 16 == 0 && reinterpret_cast<uintptr_t>(Q) % 16 == 0);
  GQ_CHECK_ARG(n_tok <= ((int64_t)1 << 31) * kFwTile && d_out <= (int64_t)65535 * kFwTile);
  if (n_tok == 0) return GPTQ_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TimedScope ts(kTimeForward, st);
  const dim3 grid((unsigned)cdiv(n_tok, kFwTile), (unsigned)cdiv(d_out, kFwTile));
  if (x_dtype == GPTQ_F32)
    hipLaunchKernelGGL(forward_kernel<GPTQ_F32>, grid, dim3(256), 0, st, X, ld_x, n_tok, (int)d_in, Q, ld_q, d_out, act,
                       Y, ld_y);
  else if (x_dtype == GPTQ_F16)
    hipLaunchKernelGGL(forward_kernel<GPTQ_F16>, grid, dim3(256), 0, st, X, ld_x, n_tok, (int)d_in, Q, ld_q, d_out, act,
                       Y, ld_y);
  else
    hipLaunchKernelGGL(forward_kernel<GPTQ_BF16>, grid, dim3(256), 0, st, X, ld_x, n_tok, (int)d_in, Q, ld_q, d_out,
                       act, Y, ld_y);
  GQ_LAUNCHED();
  return GPTQ_OK;
}
