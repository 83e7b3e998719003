// W4A16 consumer of the packed format: Y = X Q^T with Q dequantized on the fly
// from 4-bit codes, fp16 scales and integer zeros ("INT4/INT8 量化推理：从 GPTQ
// 到 AWQ 的取舍", section 六: weights in 4 bits, activations in 16-bit floating
// point, the saving is memory traffic while the products run on 16-bit matrix
// units; section 一: the stored group).
//
// The kernel streams the packed weights once from HBM and multiplies on MFMA
// (v_mfma_f32_16x16x32_{f16,bf16}): a wave owns 16 output rows, each lane
// loads 16 bytes (32 codes) of its row per 128-channel chunk, and the four
// lanes of a row cover the chunk.  The codes become MFMA operands with two
// bit operations per pair: OR-ing a nibble into the mantissa of 1024.0 (fp16)
// or 128.0 (bf16) gives 1024 + q (128 + q) exactly.
//   fp16: one packed fp16 add of -(1024 + z) leaves q - z exactly, so every
//         product x (q - z) is exact and the chunk's sum is scaled once.
//   bf16: there is no packed bf16 add; the chunk's MFMA sum of x (128 + q) is
//         corrected by (128 + z) times the chunk's activation sum, computed
//         once per call when the activations are staged.
// Nibble pairs come out as (c0, c4), (c1, c5), (c2, c6), (c3, c7) of each
// 8-code word, so the staged activations carry the same order within every
// 8 channels.  With an act-order permutation the staging also gathers the
// activations into quantization order, and the codes are packed in that
// order too: every group is then a run of consecutive chunks.
#include "common.h"

namespace gq {

constexpr int kW4Rows = 64;    // output rows per workgroup: 4 waves x 16
constexpr int kW4Chunk = 128;  // input channels per lane load (16 bytes of codes)

struct W4Args {
  const u32x4* qw;         // [d_out][d_in / 32]: 16-byte units of the packed rows
  const uint16_t* scales;  // [d_out][ng] fp16 bits
  const uint8_t* zeros;    // [d_out][ng]
  const u32x4* Xs;         // [Mp][d_in / 8]: staged activations
  const float* xsum;       // [nchunks][Mp]: activation sum of every chunk
  float* Y;                // [M][ld_y]
  float* part;             // [S][M][d_out] partial sums of each k-split
  uint32_t* cnt;           // [nblocks] arrivals per row block
  int64_t d_out, ld_y;
  int K, ng, gch, M, Mp, S, nchunks;
};

// Order of the 8 channels of a staged 8-channel unit: position i holds
// channel pair8(i) = 0, 4, 1, 5, 2, 6, 3, 7 of the unit (the order in which
// the codes' nibble pairs come out).
__device__ __forceinline__ int pair8(int i) { return (i >> 1) | ((i & 1) << 2); }

template <int kDt>
__device__ __forceinline__ float act_f32(uint16_t v) {
  if constexpr (kDt == GPTQ_F16) return f16_bits_to_f32(v);
  else return bf16_bits_to_f32(v);
}

// Xs[m][k] = X[m][col(k')] with k' the unit-swizzled channel, col = perm or
// identity; rows m >= M are zero.  xsum[c][m] = sum of the chunk's 128
// staged values (fp32, fixed order).  Also clears the split-K arrival
// counters for the main kernel that follows on the same stream.
template <int kDt>
__global__ __launch_bounds__(256) void w4_stage_kernel(const uint16_t* __restrict__ X, int64_t ld_x, int M, int Mp,
                                                       int K, const int32_t* __restrict__ perm,
                                                       uint16_t* __restrict__ Xs, float* __restrict__ xsum,
                                                       uint32_t* __restrict__ cnt, int ncnt) {
  const int c = blockIdx.x;
  const int e = threadIdx.x & 15;
  const int k0 = c * kW4Chunk + e * 8;
  for (int m = threadIdx.x >> 4; m < Mp; m += 16) {
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + pair8(i);
      const int col = perm ? perm[k] : k;
      const uint16_t v = m < M ? X[(size_t)m * ld_x + col] : (uint16_t)0;
      h[i >> 1] |= (uint32_t)v << (16 * (i & 1));
      s += act_f32<kDt>(v);
    }
    u32x4 o;
    o[0] = h[0];
    o[1] = h[1];
    o[2] = h[2];
    o[3] = h[3];
    *reinterpret_cast<u32x4*>(Xs + (size_t)m * K + k0) = o;
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    if (e == 0) xsum[(size_t)c * Mp + m] = s;
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < ncnt; i += gridDim.x * 256) cnt[i] = 0u;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 codes of one word -> MFMA operand (pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7)).
template <int kDt>
__device__ __forceinline__ u32x4 w4_operand(uint32_t w, uint32_t zc) {
  u32x4 r;
  if constexpr (kDt == GPTQ_F16) {
    const f16x2 zz = __builtin_bit_cast(f16x2, zc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;   // 1024 + q, exact
      r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v) + zz);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ((w >> (4 * i)) & 0x000F000Fu) | 0x43004300u;   // 128 + q, exact
  }
  return r;
}

template <int kDt>
__device__ __forceinline__ f32x4 w4_mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (kDt == GPTQ_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
}

// Workgroup (nb, s): rows nb*64 .. +63, chunks of k-split s.  Lane l of wave w:
// output row nb*64 + 16w + l%16, codes 32*(l/16) .. +31 of every chunk; MFMA
// lane layout: A (activations) row l%16 = token, B (codes) column l%16 = row,
// both with 8 channels per lane at 8*(l/16); D lane l holds tokens 4*(l/16)
// .. +3 of row l%16.  kMT token tiles of 16, kU chunks in flight per lane.
template <int kDt, int kMT, int kU>
__global__ __launch_bounds__(256) void w4_main_kernel(W4Args a) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int nb = blockIdx.x, sp = blockIdx.y;
  const int64_t row = (int64_t)nb * kW4Rows + (threadIdx.x >> 6) * 16 + (lane & 15);
  const int64_t rowc = row < a.d_out ? row : a.d_out - 1;
  const int c0 = (int)((int64_t)a.nchunks * sp / a.S);
  const int c1 = (int)((int64_t)a.nchunks * (sp + 1) / a.S);
  const u32x4* wrow = a.qw + rowc * (a.K / 32) + q;
  const uint16_t* srow = a.scales + rowc * a.ng;
  const uint8_t* zrow = a.zeros + rowc * a.ng;

  f32x4 tot[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) tot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = c0; c < c1; c += kU) {
    u32x4 wq[kU];
    u32x4 A[kU][kMT][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int cc = c + u < c1 ? c + u : c1 - 1;   // clamped: loads stay in the live range
      wq[u] = wrow[(size_t)cc * 4];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int tok = mt * 16 + (lane & 15);
        const u32x4* xp = a.Xs + (size_t)tok * (a.K / 8) + cc * 16 + q * 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) A[u][mt][t] = tok < a.M ? xp[t] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c + u >= c1) break;
      const int gi = (c + u) / a.gch;
      const float sc = f16_bits_to_f32(srow[gi]);
      const uint32_t z = zrow[gi];
      const uint32_t zc = (0xE400u | z) * 0x00010001u;   // fp16 -(1024 + z) in both halves
      f32x4 acc[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 b = w4_operand<kDt>(wq[u][t], zc);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[mt] = w4_mfma<kDt>(A[u][mt][t], b, acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if constexpr (kDt == GPTQ_BF16) {
          const f32x4 xs = *reinterpret_cast<const f32x4*>(a.xsum + (size_t)(c + u) * a.Mp + mt * 16 + 4 * q);
          const float zb = -(128.0f + (float)z);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][r] = fmaf(zb, xs[r], acc[mt][r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[mt][r] = fmaf(sc, acc[mt][r], tot[mt][r]);
      }
    }
  }

  const bool live = row < a.d_out;
  if (a.S == 1) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = mt * 16 + 4 * q + r;
        if (live && tok < a.M) a.Y[(size_t)tok * a.ld_y + row] = tot[mt][r];
      }
    return;
  }
  // k-split: publish this split's sums; the last workgroup of the row block
  // to arrive adds the S partials in split order (a fixed order, so the
  // result does not depend on arrival order).
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = mt * 16 + 4 * q + r;
      if (live && tok < a.M) a.part[((size_t)sp * a.M + tok) * a.d_out + row] = tot[mt][r];
    }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.cnt + nb, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = old == (uint32_t)(a.S - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int e = threadIdx.x; e < a.M * kW4Rows; e += 256) {
    const int tok = e / kW4Rows;
    const int64_t r = (int64_t)nb * kW4Rows + e % kW4Rows;
    if (r >= a.d_out) continue;
    float s = 0.0f;
    for (int k = 0; k < a.S; ++k) s += a.part[((size_t)k * a.M + tok) * a.d_out + r];
    a.Y[(size_t)tok * a.ld_y + r] = s;
  }
}

struct W4Plan {
  int Mp, S, nchunks, nblocks;
  size_t off_xs, off_xsum, off_part, off_cnt, total;
};

static W4Plan w4_plan(int64_t M, int64_t d_in, int64_t d_out) {
  W4Plan p;
  p.Mp = M <= 16 ? 16 : M <= 32 ? 32 : 64;
  p.nchunks = (int)(d_in / kW4Chunk);
  p.nblocks = (int)cdiv(d_out, kW4Rows);
  // enough workgroups to keep every CU streaming, at least 4 chunks each
  const int64_t want = cdiv(1024, p.nblocks);
  p.S = (int)std::max<int64_t>(1, std::min<int64_t>(want, p.nchunks / 4));
  Carver cv(nullptr);
  cv.take<uint16_t>((size_t)p.Mp * d_in);
  p.off_xs = 0;
  p.off_xsum = align_up(cv.used, 256);
  cv.take<float>((size_t)p.nchunks * p.Mp);
  p.off_part = align_up(cv.used, 256);
  cv.take<float>(p.S > 1 ? (size_t)p.S * M * d_out : 0);
  p.off_cnt = align_up(cv.used, 256);
  cv.take<uint32_t>((size_t)p.nblocks);
  p.total = cv.used + 256;
  return p;
}

size_t w4a16_workspace_bytes(int64_t M, int64_t d_in, int64_t d_out) { return w4_plan(M, d_in, d_out).total; }

template <int kDt, int kMT, int kU>
static void launch_w4(const W4Args& a, int nblocks, hipStream_t st) {
  hipLaunchKernelGGL((w4_main_kernel<kDt, kMT, kU>), dim3((unsigned)nblocks, (unsigned)a.S), dim3(256), 0, st, a);
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_w4a16_matmul(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                                         const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                                         const int32_t* perm, int64_t d_out, int32_t group_size, float* Y,
                                         int64_t ld_y, void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(X && qweight && scales && zeros && Y);
  GQ_CHECK_ARG(x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(M >= 1 && d_out >= 1 && d_out <= (int64_t)1 << 24);
  GQ_CHECK_ARG(d_in >= kW4Chunk && d_in % kW4Chunk == 0 && d_in <= 65536);
  GQ_CHECK_ARG(ld_x >= d_in && ld_y >= d_out);
  GQ_CHECK_ARG(group_size >= 1 && d_in % group_size == 0);
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(qweight) % 16 == 0);
  if (group_size % kW4Chunk != 0 || M > 64) return GPTQ_EUNSUPPORTED;
  const W4Plan pl = w4_plan(M, d_in, d_out);
  if (workspace == nullptr || ws_bytes < pl.total) return GPTQ_ENOMEM;

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* Xs = reinterpret_cast<uint16_t*>(ws + pl.off_xs);
  float* xsum = reinterpret_cast<float*>(ws + pl.off_xsum);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + pl.off_cnt);
  const int K = (int)d_in;
  {
    TimedScope ts(kTimeW4Stage, st);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    if (x_dtype == GPTQ_F16)
      hipLaunchKernelGGL(w4_stage_kernel<GPTQ_F16>, dim3((unsigned)pl.nchunks), dim3(256), 0, st, Xh, ld_x, (int)M,
                         pl.Mp, K, perm, Xs, xsum, cnt, pl.nblocks);
    else
      hipLaunchKernelGGL(w4_stage_kernel<GPTQ_BF16>, dim3((unsigned)pl.nchunks), dim3(256), 0, st, Xh, ld_x, (int)M,
                         pl.Mp, K, perm, Xs, xsum, cnt, pl.nblocks);
    GQ_LAUNCHED();
  }
  W4Args a;
  a.qw = reinterpret_cast<const u32x4*>(qweight);
  a.scales = scales;
  a.zeros = zeros;
  a.Xs = reinterpret_cast<const u32x4*>(Xs);
  a.xsum = xsum;
  a.Y = Y;
  a.part = part;
  a.cnt = cnt;
  a.d_out = d_out;
  a.ld_y = ld_y;
  a.K = K;
  a.ng = (int)(d_in / group_size);
  a.gch = group_size / kW4Chunk;
  a.M = (int)M;
  a.Mp = pl.Mp;
  a.S = pl.S;
  a.nchunks = pl.nchunks;
  {
    TimedScope ts(kTimeW4Main, st);
    const int mt = pl.Mp / 16;
    if (x_dtype == GPTQ_F16) {
      if (mt == 1) launch_w4<GPTQ_F16, 1, 4>(a, pl.nblocks, st);
      else if (mt == 2) launch_w4<GPTQ_F16, 2, 2>(a, pl.nblocks, st);
      else launch_w4<GPTQ_F16, 4, 1>(a, pl.nblocks, st);
    } else {
      if (mt == 1) launch_w4<GPTQ_BF16, 1, 4>(a, pl.nblocks, st);
      else if (mt == 2) launch_w4<GPTQ_BF16, 2, 2>(a, pl.nblocks, st);
      else launch_w4<GPTQ_BF16, 4, 1>(a, pl.nblocks, st);
    }
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}
