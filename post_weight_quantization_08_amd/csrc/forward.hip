// Forward of a quantized layer for sequential calibration ("3. 模型量化技术(下)",
// section "GPTQ：基于二阶信息的后训练量化", pseudocode: every layer is calibrated
// on its own inputs; here the next layer's inputs are the outputs of the
// already quantized one):  Y = round(act(X Q^T)) with Q the dequantized
// weights (fp32), act none / ReLU / SiLU, and Y in the activations' 16-bit
// format (round to nearest even).
//
// MFMA with fp32 accumulation on 16-bit operand terms (split_gemm.h; tokens
// on the MFMA row side so that the output stores are contiguous):
//   fp16 activations (16-byte rows): X enters v_mfma_f32_32x32x16_f16 as it
//     is (exact); each row of Q is scaled by a power of two and split into
//     two fp16 terms (about 2^-22 relative), two products; the epilogue
//     takes the power of two back out (exact).
//   bf16 activations (16-byte rows): X as it is, Q as two bf16 terms (about
//     2^-17 relative), two bf16 products.
//   otherwise (fp32 activations, other strides): X copied as one (bf16) or
//     two (fp16 / fp32) bf16 terms, Q as two; three products.
// The splits run as their own passes into the workspace, so the GEMM's inner
// loop only moves 16-bit words.
#include "split_gemm.h"

namespace gq {

// Rows of an fp32 matrix as two fp16 terms of the row scaled by a power of
// two: with e chosen so that the row's largest |value| times 2^e lies in
// [2^14, 2^15), hi = fp16(2^e v) and lo = fp16(2^e v - hi) (both round to
// nearest even; the difference is exact in fp32), and inv[row] = 2^-e.  The
// scaling keeps lo out of fp16's subnormal range, so hi + lo carries about 22
// significant bits of every value near the row's magnitude.  One workgroup
// per row.
__global__ __launch_bounds__(256) void split_rows_f16_scaled_kernel(const float* __restrict__ src, int64_t ld,
                                                                    int cols, uint16_t* __restrict__ hi,
                                                                    uint16_t* __restrict__ lo,
                                                                    float* __restrict__ inv) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const float* row = src + (size_t)r * ld;
  float m = 0.0f;
  for (int c = threadIdx.x; c < cols; c += 256) m = fmaxf(m, fabsf(row[c]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int k = 0;
  if (m > 0.0f && m <= 3.0e38f) (void)frexpf(m, &k);   // m = f 2^k, f in [0.5, 1)
  const int e = m > 0.0f && m <= 3.0e38f ? min(110, max(-110, 15 - k)) : 0;
  const float sc = ldexpf(1.0f, e);
  if (threadIdx.x == 0) inv[r] = ldexpf(1.0f, -e);
  uint16_t* h = hi + (size_t)r * cols;
  uint16_t* l = lo + (size_t)r * cols;
  for (int c = threadIdx.x; c < cols; c += 256) {
    const float v = row[c] * sc;
    const uint32_t hb = f32_to_f16_bits(v);
    h[c] = (uint16_t)hb;
    l[c] = (uint16_t)f32_to_f16_bits(v - f16_bits_to_f32(hb));
  }
}

struct ForwardPlan {
  size_t off_qh, off_ql, off_xh, off_xl, off_inv, total;
};

ForwardPlan forward_plan(int64_t n_tok, int64_t d_in, int64_t d_out) {
  ForwardPlan p{};
  const size_t q = (size_t)d_out * d_in * 2, x = (size_t)n_tok * d_in * 2;
  p.off_qh = 0;
  p.off_ql = align_up(p.off_qh + q, 256);
  p.off_xh = align_up(p.off_ql + q, 256);
  p.off_xl = align_up(p.off_xh + x, 256);
  p.off_inv = align_up(p.off_xl + x, 256);
  p.total = align_up(p.off_inv + (size_t)d_out * 4, 256);
  return p;
}

size_t forward_workspace_bytes(int64_t n_tok, int64_t d_in, int64_t d_out) {
  return forward_plan(n_tok, d_in, d_out).total;
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_layer_forward(const void* X, int32_t x_dtype, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                          const float* Q, int64_t d_out, int64_t ld_q, int32_t act, void* Y,
                                          int64_t ld_y, void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(X && Q && Y);
  GQ_CHECK_ARG(x_dtype == GPTQ_F32 || x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(act >= 0 && act <= 2);
  GQ_CHECK_ARG(n_tok >= 0 && d_out >= 1 && d_in >= kSgKAlign && d_in % kSgKAlign == 0 &&
               d_in <= ((int64_t)1 << 30));
  GQ_CHECK_ARG(ld_x >= d_in && ld_q >= d_in && ld_y >= d_out);
  GQ_CHECK_ARG(n_tok <= ((int64_t)1 << 31) * sg_tile_m(64) && d_out <= (int64_t)65535 * kSgTileN);
  if (n_tok == 0) return GPTQ_OK;
  const ForwardPlan pl = forward_plan(n_tok, d_in, d_out);
  if (workspace == nullptr || ws_bytes < pl.total) return GPTQ_ENOMEM;
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(workspace) % 256 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* Qh = reinterpret_cast<uint16_t*>(ws + pl.off_qh);
  uint16_t* Ql = reinterpret_cast<uint16_t*>(ws + pl.off_ql);
  uint16_t* Xh = reinterpret_cast<uint16_t*>(ws + pl.off_xh);
  uint16_t* Xl = reinterpret_cast<uint16_t*>(ws + pl.off_xl);
  float* inv = reinterpret_cast<float*>(ws + pl.off_inv);
  const int d = (int)d_in;
  // 16-bit activations whose rows keep 16-byte alignment feed the MFMA directly
  const bool direct = x_dtype != GPTQ_F32 && (ld_x * 2) % 16 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0;
  const bool f16 = direct && x_dtype == GPTQ_F16;
  const bool x_lo = !direct && x_dtype != GPTQ_BF16;
  TimedScope ts(kTimeForward, st);
  if (f16) {
    hipLaunchKernelGGL(split_rows_f16_scaled_kernel, dim3((unsigned)d_out), dim3(256), 0, st, Q, ld_q, d, Qh, Ql,
                       inv);
  } else {
    const unsigned gq_blocks = (unsigned)std::min<int64_t>(cdiv(d_out * d_in, 256), 65536);
    hipLaunchKernelGGL(split_rows_kernel<GPTQ_F32>, dim3(gq_blocks), dim3(256), 0, st, Q, ld_q, d_out, d, Qh, Ql);
  }
  GQ_LAUNCHED();
  if (!direct) {
    const unsigned gx_blocks = (unsigned)std::min<int64_t>(cdiv(n_tok * d_in, 256), 65536);
    if (x_dtype == GPTQ_F32)
      hipLaunchKernelGGL(split_rows_kernel<GPTQ_F32>, dim3(gx_blocks), dim3(256), 0, st, X, ld_x, n_tok, d, Xh, Xl);
    else if (x_dtype == GPTQ_F16)
      hipLaunchKernelGGL(split_rows_kernel<GPTQ_F16>, dim3(gx_blocks), dim3(256), 0, st, X, ld_x, n_tok, d, Xh, Xl);
    else
      hipLaunchKernelGGL(split_rows_kernel<GPTQ_BF16>, dim3(gx_blocks), dim3(256), 0, st, X, ld_x, n_tok, d, Xh,
                         (uint16_t*)nullptr);
    GQ_LAUNCHED();
  }
  SgArgs g{};
  g.Ah = direct ? static_cast<const uint16_t*>(X) : Xh;
  g.Al = x_lo ? Xl : nullptr;
  g.lda = direct ? ld_x : d_in;
  g.Bh = Qh;
  g.Bl = Ql;
  g.ldb = d_in;
  g.M = n_tok;
  g.N = d_out;
  g.K = d;
  g.Y = Y;
  g.ld_y = ld_y;
  g.col_scale = f16 ? inv : nullptr;
  g.act = act;
  g.y_dtype = x_dtype;
  // two products on 128-token waves; the three-product form on 64-token waves
  const dim3 grid((unsigned)cdiv(n_tok, sg_tile_m(x_lo ? 64 : 128)), (unsigned)cdiv(d_out, kSgTileN));
  if (f16)
    hipLaunchKernelGGL((split_gemm_kernel<false, true, kSgActRound, true, 128>), grid, dim3(512), 0, st, g);
  else if (x_lo)
    hipLaunchKernelGGL((split_gemm_kernel<true, true, kSgActRound, false, 64>), grid, dim3(512), 0, st, g);
  else
    hipLaunchKernelGGL((split_gemm_kernel<false, true, kSgActRound, false, 128>), grid, dim3(512), 0, st, g);
  GQ_LAUNCHED();
  return GPTQ_OK;
}
