// Activation-aware per-channel scaling as a pre-pass to GPTQ (ipipp.com page,
// section 二: scale each input channel's weights by an activation statistic,
// choose among candidate scales by the output error, divide the scale back
// out in the previous layer; "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍",
// section 四: the transform is exact before rounding).
//
// Search, per candidate alpha of the caller's grid:
//   s_c = fp32(max(a_c, 1e-6)^alpha) with a_c = sum |x| / N        (awq_scale_kernel)
//   D = W - RTN(W diag(s)) diag(s)^-1, group-wise with the path's
//   own quantizer, split into two bf16 terms                        (awq_delta_kernel)
//   E = ||D Xs^T||_F^2 on a token sample Xs: split-bf16 MFMA GEMM,
//   squares summed per tile, tiles summed in a fixed order  (split_gemm_kernel, awq_sum_kernel)
// then the first alpha with the smallest E is kept (awq_pick_kernel).
// Apply: S'_ij = S_ij / (s_i s_j), D'_i = D_i / s_i^2, W' = fp32(W s).
#include "split_gemm.h"

namespace gq {

constexpr double kAwqFloor = 1e-6;
constexpr int kAwqTileMin = sg_tile_m(64);   // fewest rows per output tile of the error GEMM
constexpr int kAwqTokTile = kSgTileN;        // tokens per output tile
constexpr int kAwqK = kSgKAlign;             // d_in is a multiple of this

template <int kDt>
__device__ __forceinline__ float awq_load(const void* p, size_t i) {
  if constexpr (kDt == GPTQ_F32) return static_cast<const float*>(p)[i];
  else if constexpr (kDt == GPTQ_F16) return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

constexpr int kAwqMaxAlpha = 256;
struct AwqAlphas {
  float a[kAwqMaxAlpha];
};

// s[j][c] = fp32(max(A[c] / n, 1e-6) ^ alpha[j]) (power in fp64).
__global__ __launch_bounds__(256) void awq_scale_kernel(const double* __restrict__ A, const int64_t* __restrict__ n,
                                                        AwqAlphas alphas, int d, float* __restrict__ s) {
  const int j = blockIdx.y;
  const double al = (double)alphas.a[j];
  const double nt = (double)*n;
  for (int c = blockIdx.x * 256 + threadIdx.x; c < d; c += gridDim.x * 256) {
    const double a = fmax(A[c] / nt, kAwqFloor);
    s[(size_t)j * d + c] = al == 0.0 ? 1.0f : (float)pow(a, al);
  }
}

// One wave per (row, group): v = fp32(w s), the group's range -> scale and
// zero, q = clamp(rne(v / scale) + z), dq = fp32(scale (q - z)) / s, and the
// residual w - dq as a sum of two bf16 values.
template <int kDt>
__global__ __launch_bounds__(256) void awq_delta_kernel(const void* __restrict__ W, int64_t ld_w, int64_t d_out, int d,
                                                        int g, const float* __restrict__ s, float maxq, int sym,
                                                        uint16_t* __restrict__ Dh, uint16_t* __restrict__ Dl) {
  // candidate blockIdx.z of the batch: its scales and its residual slot
  s += (size_t)blockIdx.z * d;
  Dh += (size_t)blockIdx.z * d_out * d;
  Dl += (size_t)blockIdx.z * d_out * d;
  const int lane = threadIdx.x & 63;
  const int ng = d / g;
  const int64_t units = d_out * ng;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
    const int64_t r = u / ng;
    const int c0 = (int)(u - r * ng) * g;
    const size_t wrow = (size_t)r * ld_w;
    float lo = 3.402823466e38f, hi = -3.402823466e38f;
    for (int c = lane; c < g; c += 64) {
      const float v = awq_load<kDt>(W, wrow + c0 + c) * s[c0 + c];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    float sc, z;
    uint16_t sb;
    group_scale_zero(lo, hi, maxq, sym != 0, sc, z, sb);
    for (int c = lane; c < g; c += 64) {
      const float w = awq_load<kDt>(W, wrow + c0 + c);
      const float sv = s[c0 + c];
      const float v = w * sv;
      const float q = fminf(fmaxf(rintf(__fdiv_rn(v, sc)) + z, 0.0f), maxq);
      const float dq = __fdiv_rn(sc * (q - z), sv);
      const float e = w - dq;
      const uint32_t h = f32_to_bf16_bits(e);
      const size_t o = (size_t)r * d + c0 + c;
      Dh[o] = (uint16_t)h;
      Dl[o] = (uint16_t)f32_to_bf16_bits(e - bf16_bits_to_f32(h));
    }
  }
}

// The same residual, 8 consecutive weights per lane (16-byte code of the
// group's lanes: g / 8 of them, 4 to 64), for g = 32 .. 512: the group's
// range is reduced across its lanes and the weights stay in registers.
template <int kDt>
__device__ __forceinline__ void awq_load8(const void* W, size_t i, float (&w)[8]) {
  if constexpr (kDt == GPTQ_F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = a[e];
      w[e + 4] = b[e];
    }
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      w[e] = kDt == GPTQ_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
    }
  }
}

template <int kDt>
__global__ __launch_bounds__(256) void awq_delta8_kernel(const void* __restrict__ W, int64_t ld_w, int64_t d_out,
                                                         int d, int g, const float* __restrict__ s, float maxq,
                                                         int sym, uint16_t* __restrict__ Dh, uint16_t* __restrict__ Dl) {
  s += (size_t)blockIdx.z * d;
  Dh += (size_t)blockIdx.z * d_out * d;
  Dl += (size_t)blockIdx.z * d_out * d;
  const int lpg = g / 8;   // lanes per group (a power of two, 4 .. 64)
  const int64_t units = d_out * (d / 8);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += stride) {
    // every lane of a wave takes a unit in the same trip: the shuffles below
    // stay inside one group (units of a group are lpg consecutive lanes)
    const int64_t r = u / (d / 8);
    const int c = (int)(u - r * (d / 8)) * 8;
    float w[8], sv[8], v[8];
    awq_load8<kDt>(W, (size_t)r * ld_w + c, w);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + c);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + c + 4);
    float lo = 3.402823466e38f, hi = -3.402823466e38f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = e < 4 ? s0[e] : s1[e - 4];
      v[e] = w[e] * sv[e];
      lo = fminf(lo, v[e]);
      hi = fmaxf(hi, v[e]);
    }
    for (int o = lpg >> 1; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    float sc, z;
    uint16_t sb;
    group_scale_zero(lo, hi, maxq, sym != 0, sc, z, sb);
    uint32_t ho[4] = {0u, 0u, 0u, 0u}, lw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = fminf(fmaxf(rintf(__fdiv_rn(v[e], sc)) + z, 0.0f), maxq);
      const float dq = __fdiv_rn(sc * (q - z), sv[e]);
      const float x = w[e] - dq;
      const uint32_t h = f32_to_bf16_bits(x);
      ho[e >> 1] |= h << (16 * (e & 1));
      lw[e >> 1] |= f32_to_bf16_bits(x - bf16_bits_to_f32(h)) << (16 * (e & 1));
    }
    const size_t o = (size_t)r * d + c;
    *reinterpret_cast<u32x4*>(Dh + o) = u32x4{ho[0], ho[1], ho[2], ho[3]};
    *reinterpret_cast<u32x4*>(Dl + o) = u32x4{lw[0], lw[1], lw[2], lw[3]};
  }
}

// err[j] = sum of the candidate's tile partials, in tile order.
__global__ __launch_bounds__(64) void awq_sum_kernel(const double* __restrict__ part, int tiles,
                                                     double* __restrict__ err) {
  const int j = blockIdx.x;
  __shared__ double red[64];
  double s = 0.0;
  const int per = (tiles + 63) / 64;
  const int i0 = threadIdx.x * per, i1 = min(tiles, i0 + per);
  for (int i = i0; i < i1; ++i) s += part[(size_t)j * tiles + i];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < 64; ++i) t += red[i];
    err[j] = t;
  }
}

// best = first index of the smallest error; s_out = that candidate's scales.
__global__ __launch_bounds__(256) void awq_pick_kernel(const double* __restrict__ err, int n_alpha,
                                                       const float* __restrict__ s_all, int d,
                                                       float* __restrict__ s_out, int32_t* __restrict__ best_out) {
  int best = 0;
  for (int j = 1; j < n_alpha; ++j)
    if (err[j] < err[best]) best = j;
  if (blockIdx.x == 0 && threadIdx.x == 0) *best_out = best;
  for (int c = blockIdx.x * 256 + threadIdx.x; c < d; c += gridDim.x * 256) s_out[c] = s_all[(size_t)best * d + c];
}

// S (lower triangle incl. the diagonal, fp32) / (s_i s_j) and D / s_i^2 in
// fp64; W' = fp32(w s).
__global__ __launch_bounds__(256) void awq_apply_s_kernel(float* __restrict__ S, double* __restrict__ D,
                                                          const float* __restrict__ s, int d) {
  const int i = blockIdx.x;
  const double si = (double)s[i];
  for (int j = threadIdx.x; j <= i; j += 256) {
    float* p = S + (size_t)i * d + j;
    *p = (float)((double)*p / (si * (double)s[j]));
  }
  if (threadIdx.x == 0) D[i] = D[i] / (si * si);
}

template <int kDt>
__global__ __launch_bounds__(256) void awq_apply_w_kernel(const void* __restrict__ W, int64_t ld_w, int64_t d_out,
                                                          int d, const float* __restrict__ s, float* __restrict__ Wo) {
  const int64_t r = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) Wo[(size_t)r * d + c] = awq_load<kDt>(W, (size_t)r * ld_w + c) * s[c];
}

struct AwqPlan {
  size_t off_s, off_dh, off_dl, off_xh, off_xl, off_part, total;
  int tiles_m, tiles_t, batch;
};

// Candidates per launch: as many residuals as fit in 2 GiB (at least one),
// so that layers with few rows still give the GPU enough tiles.
AwqPlan awq_plan(int64_t d_out, int64_t d_in, int64_t n_s, int64_t n_alpha) {
  AwqPlan p;
  p.tiles_m = (int)cdiv(d_out, kAwqTileMin);   // the most tiles any GEMM form launches
  p.tiles_t = (int)cdiv(n_s, kAwqTokTile);
  const int64_t res_bytes = d_out * d_in * 4;
  p.batch = (int)std::max<int64_t>(1, std::min<int64_t>(n_alpha, ((int64_t)2 << 30) / res_bytes));
  Carver cv(nullptr);
  p.off_s = 0;
  cv.take<float>((size_t)n_alpha * d_in);
  p.off_dh = align_up(cv.used, 256);
  cv.take<uint16_t>((size_t)p.batch * d_out * d_in);
  p.off_dl = align_up(cv.used, 256);
  cv.take<uint16_t>((size_t)p.batch * d_out * d_in);
  p.off_xh = align_up(cv.used, 256);
  cv.take<uint16_t>((size_t)n_s * d_in);
  p.off_xl = align_up(cv.used, 256);
  cv.take<uint16_t>((size_t)n_s * d_in);
  p.off_part = align_up(cv.used, 256);
  cv.take<double>((size_t)n_alpha * p.tiles_m * p.tiles_t);
  p.total = cv.used + 256;
  return p;
}

size_t awq_search_workspace_bytes(int64_t d_out, int64_t d_in, int64_t n_s, int64_t n_alpha) {
  return awq_plan(d_out, d_in, n_s, n_alpha).total;
}

}  // namespace gq

using namespace gq;

bool gq_params_ok(const gptq_params* p, int64_t d_in);

extern "C" gptq_status gptq_awq_search(const void* W, int32_t w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                                       const double* A, const int64_t* n_tokens, const void* Xs, int32_t xs_dtype,
                                       int64_t n_s, int64_t ld_xs, const gptq_params* p, const float* alphas,
                                       int32_t n_alpha, double* err_out, float* s_out, int32_t* best_out,
                                       void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(W && A && n_tokens && Xs && p && alphas && err_out && s_out && best_out);
  GQ_CHECK_ARG(w_dtype == GPTQ_F32 || w_dtype == GPTQ_F16 || w_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(xs_dtype == GPTQ_F32 || xs_dtype == GPTQ_F16 || xs_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(d_out >= 1 && d_out <= (int64_t)1 << 24 && n_s >= 1 && n_s <= (int64_t)1 << 20);
  GQ_CHECK_ARG(d_in >= kAwqK && d_in % kAwqK == 0 && d_in <= 65536);
  GQ_CHECK_ARG(ld_w >= d_in && ld_xs >= d_in && n_alpha >= 1 && n_alpha <= kAwqMaxAlpha);
  if (!gq_params_ok(p, d_in)) return GPTQ_EINVAL;
  for (int j = 0; j < n_alpha; ++j) GQ_CHECK_ARG(alphas[j] >= 0.0f && alphas[j] <= 4.0f);
  const AwqPlan pl = awq_plan(d_out, d_in, n_s, n_alpha);
  if (workspace == nullptr || ws_bytes < pl.total) return GPTQ_ENOMEM;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* s_all = reinterpret_cast<float*>(ws + pl.off_s);
  uint16_t* Dh = reinterpret_cast<uint16_t*>(ws + pl.off_dh);
  uint16_t* Dl = reinterpret_cast<uint16_t*>(ws + pl.off_dl);
  uint16_t* Xh = reinterpret_cast<uint16_t*>(ws + pl.off_xh);
  uint16_t* Xl = reinterpret_cast<uint16_t*>(ws + pl.off_xl);
  double* part = reinterpret_cast<double*>(ws + pl.off_part);
  const int d = (int)d_in;

  TimedScope ts(kTimeAwqSearch, st);
  AwqAlphas al{};
  for (int j = 0; j < n_alpha; ++j) al.a[j] = alphas[j];
  hipLaunchKernelGGL(awq_scale_kernel, dim3((unsigned)cdiv(d, 256), (unsigned)n_alpha), dim3(256), 0, st, A,
                     n_tokens, al, d, s_all);
  GQ_LAUNCHED();
  const int64_t nx = n_s * d_in;
  const unsigned gx = (unsigned)std::min<int64_t>(cdiv(nx, 256), 16384);
  // Xs rows as two bf16 terms (exact for fp16 and bf16 inputs; fp32 keeps the
  // first 16 bits of its significand)
  if (xs_dtype == GPTQ_F32) hipLaunchKernelGGL(split_rows_kernel<GPTQ_F32>, dim3(gx), dim3(256), 0, st, Xs, ld_xs, n_s, d, Xh, Xl);
  else if (xs_dtype == GPTQ_F16) hipLaunchKernelGGL(split_rows_kernel<GPTQ_F16>, dim3(gx), dim3(256), 0, st, Xs, ld_xs, n_s, d, Xh, Xl);
  else hipLaunchKernelGGL(split_rows_kernel<GPTQ_BF16>, dim3(gx), dim3(256), 0, st, Xs, ld_xs, n_s, d, Xh, Xl);
  GQ_LAUNCHED();
  const float maxq = (float)((1 << p->bits) - 1);
  const int64_t units = d_out * (d_in / p->group_size);
  const unsigned gd = (unsigned)std::min<int64_t>(cdiv(units, 4), 16384);
  // GEMM form: bf16 tokens, two products on 128-row waves; otherwise three on 64-row waves
  const bool x_lo = xs_dtype != GPTQ_BF16;
  const int tiles_m = (int)cdiv(d_out, sg_tile_m(x_lo ? 64 : 128));
  const int tiles = tiles_m * pl.tiles_t;
  // 8 weights per lane when a group spans 4 .. 64 lanes and the rows keep
  // 16-byte alignment
  const int g = p->group_size;
  const int64_t es = w_dtype == GPTQ_F32 ? 4 : 2;
  const bool v8 = g >= 32 && g <= 512 && (g & (g - 1)) == 0 && (ld_w * es) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(W) % 16 == 0;
  const int64_t units8 = d_out * (d_in / 8);
  const unsigned g8 = (unsigned)std::min<int64_t>(cdiv(units8, 256), 65536);
  for (int j = 0; j < n_alpha; j += pl.batch) {
    const int nb = std::min(pl.batch, n_alpha - j);
    const float* sj = s_all + (size_t)j * d;
#define GQ_DELTA(DT)                                                                                                 \
  do {                                                                                                               \
    if (v8)                                                                                                          \
      hipLaunchKernelGGL(awq_delta8_kernel<DT>, dim3(g8, 1, nb), dim3(256), 0, st, W, ld_w, d_out, d, g, sj, maxq, p->sym, Dh, \
                         Dl);                                                                                        \
    else                                                                                                             \
      hipLaunchKernelGGL(awq_delta_kernel<DT>, dim3(gd, 1, nb), dim3(256), 0, st, W, ld_w, d_out, d, g, sj, maxq, p->sym, Dh,  \
                         Dl);                                                                                        \
  } while (0)
    if (w_dtype == GPTQ_F32) GQ_DELTA(GPTQ_F32);
    else if (w_dtype == GPTQ_F16) GQ_DELTA(GPTQ_F16);
    else GQ_DELTA(GPTQ_BF16);
#undef GQ_DELTA
    GQ_LAUNCHED();
    // tiles of Y = D Xs^T (128 or 256 rows x 256 tokens), one candidate per
    // blockIdx.z; products Dh Xh + Dl Xh (+ Dh Xl when the activations have a
    // low term)
    const dim3 ge((unsigned)tiles_m, (unsigned)pl.tiles_t, (unsigned)nb);
    SgArgs ga{};
    ga.Ah = Dh;
    ga.Al = Dl;
    ga.Bh = Xh;
    ga.Bl = Xl;
    ga.M = d_out;
    ga.N = n_s;
    ga.K = d;
    ga.lda = d_in;
    ga.ldb = d_in;
    ga.strideA = d_out * d_in;
    ga.part = part + (size_t)j * tiles;
    if (x_lo)
      hipLaunchKernelGGL((split_gemm_kernel<true, true, kSgSumSquares, false, 64>), ge, dim3(512), 0, st, ga);
    else
      hipLaunchKernelGGL((split_gemm_kernel<true, false, kSgSumSquares, false, 128>), ge, dim3(512), 0, st, ga);
    GQ_LAUNCHED();
  }
  hipLaunchKernelGGL(awq_sum_kernel, dim3((unsigned)n_alpha), dim3(64), 0, st, part, tiles, err_out);
  GQ_LAUNCHED();
  hipLaunchKernelGGL(awq_pick_kernel, dim3((unsigned)cdiv(d, 256)), dim3(256), 0, st, err_out, n_alpha, s_all, d,
                     s_out, best_out);
  GQ_LAUNCHED();
  return GPTQ_OK;
}

extern "C" gptq_status gptq_awq_apply(float* S, double* D, int64_t d_in, const float* s, const void* W,
                                      int32_t w_dtype, int64_t d_out, int64_t ld_w, float* W_out, void* stream) {
  GQ_CHECK_ARG(S && D && s && W && W_out);
  GQ_CHECK_ARG(w_dtype == GPTQ_F32 || w_dtype == GPTQ_F16 || w_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(d_in >= 1 && d_in <= 65536 && d_out >= 1 && d_out <= (int64_t)1 << 24 && ld_w >= d_in);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = (int)d_in;
  TimedScope ts(kTimeAwqApply, st);
  hipLaunchKernelGGL(awq_apply_s_kernel, dim3((unsigned)d), dim3(256), 0, st, S, D, s, d);
  GQ_LAUNCHED();
  const dim3 gw((unsigned)d_out);
  if (w_dtype == GPTQ_F32) hipLaunchKernelGGL(awq_apply_w_kernel<GPTQ_F32>, gw, dim3(256), 0, st, W, ld_w, d_out, d, s, W_out);
  else if (w_dtype == GPTQ_F16) hipLaunchKernelGGL(awq_apply_w_kernel<GPTQ_F16>, gw, dim3(256), 0, st, W, ld_w, d_out, d, s, W_out);
  else hipLaunchKernelGGL(awq_apply_w_kernel<GPTQ_BF16>, gw, dim3(256), 0, st, W, ld_w, d_out, d, s, W_out);
  GQ_LAUNCHED();
  return GPTQ_OK;
}
