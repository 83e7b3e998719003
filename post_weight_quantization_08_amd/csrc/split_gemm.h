// C = A B^T on MFMA with operands held as two 16-bit terms (hi + lo), shared
// by the activation-aware scale search (sum of squares of C) and the forward
// of a quantized layer (C through an activation, rounded to 16 bits).
//
// A: rows m (row stride lda), B: rows n (row stride ldb), both [rows][k] of
// bf16 words (or fp16 words with kF16), hi, and lo when present.
// Products per 32 x 32 x 16 block: Ah Bh, + Al Bh when A has a low term,
// + Ah Bl when B has one (the lo*lo term is below fp32's resolution).
// Workgroup tile 2 kWaveM (m) x 256 (n), 8 waves of kWaveM x 64 (blocks of
// 32 x 32 x 16 MFMA), k staged through LDS 64 at a time; the next stage's
// 16-byte pieces are loaded into registers while this one computes.  A wave
// height of 128 halves the LDS reads per MFMA against 64; the three-product
// form takes 64 (at 128 it runs out of registers).
// Rows past M or N load as zeros.
#pragma once

#include "common.h"

namespace gq {

constexpr int kSgTileN = 256;   // 8 waves: 2 along m, 4 along n (64 columns each)
constexpr int kSgK = 64;        // k per LDS stage
constexpr int kSgKAlign = 32;   // K must be a multiple of this (a half stage loads zeros)

// Rows of m per workgroup for a wave height (32 x 32 blocks per wave: kWaveM / 32).
constexpr int sg_tile_m(int wave_m) { return 2 * wave_m; }

// rows x cols values of kDt (row stride ld) as two bf16 terms, dense [rows][cols].
template <int kDt>
__global__ __launch_bounds__(256) void split_rows_kernel(const void* __restrict__ src, int64_t ld, int64_t rows,
                                                         int cols, uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo) {
  const int64_t total = rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t t = e / cols;
    const int c = (int)(e - t * cols);
    float x;
    if constexpr (kDt == GPTQ_F32) x = static_cast<const float*>(src)[(size_t)t * ld + c];
    else if constexpr (kDt == GPTQ_F16) x = f16_bits_to_f32(static_cast<const uint16_t*>(src)[(size_t)t * ld + c]);
    else x = bf16_bits_to_f32(static_cast<const uint16_t*>(src)[(size_t)t * ld + c]);
    const uint32_t h = f32_to_bf16_bits(x);
    hi[e] = (uint16_t)h;
    if (lo) lo[e] = (uint16_t)f32_to_bf16_bits(x - bf16_bits_to_f32(h));
  }
}

enum SgEpilogue { kSgSumSquares = 0, kSgActRound = 1 };

struct SgArgs {
  const uint16_t *Ah, *Al, *Bh, *Bl;   // [M][lda], [N][ldb]
  int64_t M, N;
  int K;
  int64_t lda, ldb;                    // row strides, elements (multiples of 8)
  int64_t strideA, strideB;            // per blockIdx.z (batched A / B), elements
  double* part;                        // kSgSumSquares: [z][tiles]
  void* Y;                             // kSgActRound: [M][ld_y] of y_dtype
  const float* col_scale;              // kSgActRound: C[m][n] *= col_scale[n] first (NULL: none)
  int64_t ld_y;
  int act, y_dtype;
};

template <bool kF16>
__device__ __forceinline__ f32x16 sg_mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

__device__ __forceinline__ float sg_act(float v, int act) {
  if (act == 1) return fmaxf(v, 0.0f);
  if (act == 2) return v / (1.0f + expf(-v));
  return v;
}

template <bool kALo, bool kBLo, int kEpi, bool kF16, int kWaveM>
__global__ __launch_bounds__(512) void split_gemm_kernel(SgArgs g) {
  constexpr int kLd = kSgK + 8;   // padded rows (halves) against LDS bank conflicts
  constexpr int kAT = kALo ? 2 : 1, kBT = kBLo ? 2 : 1;
  constexpr int kTileM = sg_tile_m(kWaveM);
  __shared__ __attribute__((aligned(16))) uint16_t sA[kAT][kTileM * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBT][kSgTileN * kLd];
  __shared__ double red[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* Ah = g.Ah + (size_t)blockIdx.z * g.strideA;
  const uint16_t* Al = kALo ? g.Al + (size_t)blockIdx.z * g.strideA : nullptr;
  const uint16_t* Bh = g.Bh + (size_t)blockIdx.z * g.strideB;
  const uint16_t* Bl = kBLo ? g.Bl + (size_t)blockIdx.z * g.strideB : nullptr;
  const int64_t m0 = (int64_t)blockIdx.x * kTileM;
  const int64_t n0 = (int64_t)blockIdx.y * kSgTileN;
  constexpr int kBi = kWaveM / 32;
  const int wm = (wave >> 2) * kWaveM, wn = (wave & 3) * 64;
  f32x16 acc[kBi][2];
#pragma unroll
  for (int i = 0; i < kBi; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // staging: 16-byte pieces (8 k); kPieces threads per row, kRows rows per pass
  constexpr int kPieces = kSgK / 8, kRows = 512 / kPieces;
  constexpr int kPassA = kTileM / kRows, kPassB = kSgTileN / kRows;
  const int srow = tid / kPieces, sk = (tid % kPieces) * 8;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  u32x4 pa[kPassA][kAT], pb[kPassB][kBT];
  auto load_step = [&](int k0) {
    const bool kin = k0 + sk < g.K;   // the second half of a last half stage loads zeros
#pragma unroll
    for (int h = 0; h < kPassA; ++h) {
      const int64_t r = m0 + srow + kRows * h;
      const bool live = kin && r < g.M;
      const size_t o = live ? (size_t)r * g.lda + k0 + sk : 0;
      pa[h][0] = live ? *reinterpret_cast<const u32x4*>(Ah + o) : z4;
      if constexpr (kALo) pa[h][kAT - 1] = live ? *reinterpret_cast<const u32x4*>(Al + o) : z4;
    }
#pragma unroll
    for (int h = 0; h < kPassB; ++h) {
      const int64_t r = n0 + srow + kRows * h;
      const bool live = kin && r < g.N;
      const size_t o = live ? (size_t)r * g.ldb + k0 + sk : 0;
      pb[h][0] = live ? *reinterpret_cast<const u32x4*>(Bh + o) : z4;
      if constexpr (kBLo) pb[h][kBT - 1] = live ? *reinterpret_cast<const u32x4*>(Bl + o) : z4;
    }
  };
  load_step(0);
  for (int k0 = 0; k0 < g.K; k0 += kSgK) {
#pragma unroll
    for (int h = 0; h < kPassA; ++h)
#pragma unroll
      for (int t = 0; t < kAT; ++t) *reinterpret_cast<u32x4*>(&sA[t][(srow + kRows * h) * kLd + sk]) = pa[h][t];
#pragma unroll
    for (int h = 0; h < kPassB; ++h)
#pragma unroll
      for (int t = 0; t < kBT; ++t) *reinterpret_cast<u32x4*>(&sB[t][(srow + kRows * h) * kLd + sk]) = pb[h][t];
    __syncthreads();
    if (k0 + kSgK < g.K) load_step(k0 + kSgK);
#pragma unroll
    for (int ks = 0; ks < kSgK; ks += 16) {
      const int kk = ks + 8 * (lane >> 5);
      u32x4 a[kAT][kBi], b[kBT][2];
#pragma unroll
      for (int i = 0; i < kBi; ++i)
#pragma unroll
        for (int t = 0; t < kAT; ++t)
          a[t][i] = *reinterpret_cast<const u32x4*>(&sA[t][(wm + 32 * i + (lane & 31)) * kLd + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < kBT; ++t)
          b[t][j] = *reinterpret_cast<const u32x4*>(&sB[t][(wn + 32 * j + (lane & 31)) * kLd + kk]);
#pragma unroll
      for (int i = 0; i < kBi; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = sg_mfma<kF16>(a[0][i], b[0][j], acc[i][j]);
          if constexpr (kALo) acc[i][j] = sg_mfma<kF16>(a[kAT - 1][i], b[0][j], acc[i][j]);
          if constexpr (kBLo) acc[i][j] = sg_mfma<kF16>(a[0][i], b[kBT - 1][j], acc[i][j]);
        }
    }
    __syncthreads();
  }
  if constexpr (kEpi == kSgSumSquares) {
    double sq = 0.0;
#pragma unroll
    for (int i = 0; i < kBi; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const double y = (double)acc[i][j][e];
          sq = fma(y, y, sq);
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o);
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < 8; ++w) t += red[w];
      g.part[((size_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x] = t;
    }
  } else {
    // D lane layout (32 x 32 block): element e of lane l is row 8 (e / 4) +
    // 4 (l / 32) + e % 4, column l % 32
#pragma unroll
    for (int i = 0; i < kBi; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int64_t n = n0 + wn + 32 * j + (lane & 31);
          if (m < g.M && n < g.N) {
            const float c = g.col_scale ? acc[i][j][e] * g.col_scale[n] : acc[i][j][e];
            const float v = sg_act(c, g.act);
            const size_t o = (size_t)m * g.ld_y + n;
            if (g.y_dtype == GPTQ_F32) static_cast<float*>(g.Y)[o] = v;
            else if (g.y_dtype == GPTQ_F16) static_cast<uint16_t*>(g.Y)[o] = f32_to_f16_bits(v);
            else static_cast<uint16_t*>(g.Y)[o] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
  }
}

}  // namespace gq
