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
#include <mutex>

#include "common.h"

namespace gq {

constexpr int kW4Chunk = 128;  // input channels per lane load (16 bytes of codes)

struct W4Args {
  const u32x4* qw;         // [d_out][d_in / 32]: 16-byte units of the packed rows
  const uint16_t* scales;  // [d_out][ng] fp16 bits
  const uint8_t* zeros;    // [d_out][ng]
  const u32x4* Xs;         // [Mp][d_in / 8]: staged activations
  const float* xsum;       // [nchunks][Mp]: activation sum of every chunk
  float* Y;                // [M][ld_y]
  int64_t d_out, ld_y;
  int K, ng, gch, M, Mp, nchunks;
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
// staged values (fp32, fixed order).
template <int kDt>
__global__ __launch_bounds__(256) void w4_stage_kernel(const uint16_t* __restrict__ X, int64_t ld_x, int M, int Mp,
                                                       int K, const int32_t* __restrict__ perm,
                                                       uint16_t* __restrict__ Xs, float* __restrict__ xsum) {
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
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// (x & 0x000F000F) | magic.  The caller keeps the mask in an SGPR and the
// magic number in a VGPR, both opaque to the compiler, so the pair becomes one
// v_and_or_b32 (a VOP3 takes no 32-bit literal and one scalar operand).  It is
// plain code, not inline asm: the compiler's hazard check counts an asm
// result as ready for an MFMA one wait state too early, and the bf16 operands
// go straight from here into the MFMA.
__device__ __forceinline__ uint32_t nib_pair(uint32_t x, uint32_t mask_s, uint32_t magic_v) {
  return (x & mask_s) | magic_v;
}

// 8 codes of one word -> MFMA operand (pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7)).
// magic_v: 0x64006400 (fp16 1024, 1024) or 0x43004300 (bf16 128, 128).
template <int kDt>
__device__ __forceinline__ u32x4 w4_operand(uint32_t w, uint32_t zc, uint32_t mask_s, uint32_t magic_v) {
  u32x4 r;
  r[0] = nib_pair(w, mask_s, magic_v);
  r[1] = nib_pair(w >> 4, mask_s, magic_v);
  r[2] = nib_pair(w >> 8, mask_s, magic_v);
  r[3] = nib_pair(w >> 12, mask_s, magic_v);
  if constexpr (kDt == GPTQ_F16) {
    const f16x2 zz = __builtin_bit_cast(f16x2, zc);   // -(1024 + z): leaves q - z exactly
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = r[i];   // a scalar copy: bit_cast of a vector element reads element 0
      r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v) + zz);
    }
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

__host__ __device__ constexpr int align_lds(int b) { return (b + 15) / 16 * 16; }

// Dynamic LDS of the main kernel: [scales 16 x ng fp16][zeros 16 x ng]
// then, with the activations in LDS (kLX), [X: M x K halves][chunk sums:
// nchunks x 16 fp32], then the waves' partial sums.
__host__ __device__ inline int w4_lds_x(int ng) { return align_lds(48 * ng); }
__host__ __device__ inline int w4_lds_xsum(int ng, int M, int K) { return align_lds(w4_lds_x(ng) + M * K * 2); }
__host__ __device__ inline int w4_lds_red(int ng, int M, int K, int nchunks, bool lx) {
  return w4_lds_x(ng);
}
__host__ __device__ inline int w4_lds_total(int ng, int M, int K, int nchunks, bool lx, int red_bytes) {
  const int x_end = lx ? align_lds(w4_lds_xsum(ng, M, K) + nchunks * 16 * 4) : w4_lds_x(ng);
  return std::max(x_end, w4_lds_x(ng) + red_bytes);
}

// Workgroup nb: output rows nb*16 .. +15; its kW waves split the chunks
// (wave w takes chunks w*C/kW .. (w+1)*C/kW - 1) and their sums meet in LDS,
// added in wave order (a fixed order, so results are reproducible).  Lane l:
// output row nb*16 + l%16, codes 32*(l/16) .. +31 of every chunk; MFMA lane
// layout: A (activations) row l%16 = token, B (codes) column l%16 = row, both
// with 8 channels per lane at 8*(l/16); D lane l holds tokens 4*(l/16) .. +3
// of row l%16.  kMT token tiles of 16, kU chunks in flight per lane.
// kLX (a few tokens): the workgroup copies the staged activations and chunk
// sums into LDS once and reads each chunk's operands from there, which frees
// the registers that would hold mostly-zero activation tiles for a deeper
// stream of codes.
template <int kDt, int kMT, int kU, int kW, bool kLX>
__global__ __launch_bounds__(64 * kW) void w4_main_kernel(W4Args a) {
  static_assert(!kLX || kMT == 1, "activations in LDS only for a single token tile");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: chunk loop stays scalar
  const int q = lane >> 4;
  const int64_t row = (int64_t)blockIdx.x * 16 + (lane & 15);
  const int64_t rowc = row < a.d_out ? row : a.d_out - 1;
  const int c0 = a.nchunks * wave / kW;
  const int c1 = a.nchunks * (wave + 1) / kW;
  const u32x4* wrow = a.qw + rowc * (a.K / 32) + q;
  extern __shared__ __attribute__((aligned(16))) uint8_t w4_lds[];
  f32x4 tot[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) tot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // activation tiles in registers (not kLX): lanes whose token is past M
  // never load and keep zeros
  constexpr int kUA = kLX ? 1 : kU;
  u32x4 A[kUA][kMT][4];
#pragma unroll
  for (int u = 0; u < kUA; ++u)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) A[u][mt][t] = u32x4{0u, 0u, 0u, 0u};
  u32x4 wq[kU];
  f32x4 xs[kUA][kMT];
  // every load of an iteration (codes; without kLX also chunk sums and
  // activations) goes out before its arithmetic, so waits never drain later
  // loads
  auto load_iter = [&](int c) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int cc = c + u < c1 ? c + u : c1 - 1;   // clamped: loads stay in the live range
      wq[u] = wrow[(size_t)cc * 4];
      if constexpr (!kLX) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          if constexpr (kDt == GPTQ_BF16)
            xs[u][mt] = *reinterpret_cast<const f32x4*>(a.xsum + (size_t)cc * a.Mp + mt * 16 + 4 * q);
          const int tok = mt * 16 + (lane & 15);
          if (tok < a.M) {
            const u32x4* xp = a.Xs + (size_t)tok * (a.K / 8) + cc * 16 + q * 4;
#pragma unroll
            for (int t = 0; t < 4; ++t) A[u][mt][t] = xp[t];
          }
        }
      }
    }
  };
  if (c0 < c1) load_iter(c0);

  // the workgroup's 16 rows of scales and zeros (and with kLX the staged
  // activations and chunk sums), copied once with coalesced loads while the
  // first codes are in flight (per-chunk gathers of scales and zeros from
  // global memory cost as much as the codes' stream itself)
  uint16_t* s_lds = reinterpret_cast<uint16_t*>(w4_lds);
  uint8_t* z_lds = w4_lds + 32 * a.ng;
  const u32x4* x_lds = reinterpret_cast<const u32x4*>(w4_lds + w4_lds_x(a.ng));
  const f32x4* xsum_lds = reinterpret_cast<const f32x4*>(w4_lds + w4_lds_xsum(a.ng, a.M, a.K));
  {
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    for (int e = threadIdx.x; e < 16 * a.ng; e += 64 * kW) {
      const int rr = e / a.ng;
      const int64_t rs = r0 + rr < a.d_out ? r0 + rr : a.d_out - 1;
      const size_t src = (size_t)rs * a.ng + (e - rr * a.ng);
      s_lds[e] = a.scales[src];
      z_lds[e] = a.zeros[src];
    }
    if constexpr (kLX) {
      u32x4* xd = reinterpret_cast<u32x4*>(w4_lds + w4_lds_x(a.ng));
      for (int e = threadIdx.x; e < a.M * (a.K / 8); e += 64 * kW) xd[e] = a.Xs[e];
      float* sd = reinterpret_cast<float*>(w4_lds + w4_lds_xsum(a.ng, a.M, a.K));
      for (int e = threadIdx.x; e < a.nchunks * 16; e += 64 * kW) sd[e] = a.xsum[(size_t)(e >> 4) * a.Mp + (e & 15)];
    }
    __syncthreads();
  }
  const uint16_t* srow = s_lds + (lane & 15) * a.ng;
  const uint8_t* zrow = z_lds + (lane & 15) * a.ng;
  uint32_t magic_v = kDt == GPTQ_F16 ? 0x64006400u : 0x43004300u;
  uint32_t mask_s = 0x000F000Fu;
  asm volatile("" : "+v"(magic_v));   // a VGPR the compiler cannot fold
  asm volatile("" : "+s"(mask_s));    // an SGPR the compiler cannot fold

  for (int c = c0; c < c1; c += kU) {
    if (c != c0) load_iter(c);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c + u >= c1) break;
      if constexpr (kLX) {
        const int tok = lane & 15;
        if (tok < a.M) {
#pragma unroll
          for (int t = 0; t < 4; ++t) A[0][0][t] = x_lds[tok * (a.K / 8) + (c + u) * 16 + q * 4 + t];
        }
        if constexpr (kDt == GPTQ_BF16) xs[0][0] = xsum_lds[(c + u) * 4 + q];
      }
      const int gi = (c + u) / a.gch;
      const float sc = f16_bits_to_f32(srow[gi]);
      const uint32_t zb = zrow[gi];
      const uint32_t zc = (0xE400u | zb) * 0x00010001u;   // fp16 -(1024 + z) in both halves
      f32x4 acc[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 b = w4_operand<kDt>(wq[u][t], zc, mask_s, magic_v);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[mt] = w4_mfma<kDt>(A[kLX ? 0 : u][mt][t], b, acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if constexpr (kDt == GPTQ_BF16) {
          const float zf = -(128.0f + (float)zb);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][r] = fmaf(zf, xs[kLX ? 0 : u][mt][r], acc[mt][r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[mt][r] = fmaf(sc, acc[mt][r], tot[mt][r]);
      }
    }
  }

  const bool live = row < a.d_out;
  if constexpr (kW == 1) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = mt * 16 + 4 * q + r;
        if (live && tok < a.M) a.Y[(size_t)tok * a.ld_y + row] = tot[mt][r];
      }
  } else {
    // the waves' sums meet in LDS over the staged activations
    if constexpr (kLX) __syncthreads();
    f32x4(*red)[kMT][64] =
        reinterpret_cast<f32x4(*)[kMT][64]>(w4_lds + w4_lds_red(a.ng, a.M, a.K, a.nchunks, kLX));
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) red[wave][mt][lane] = tot[mt];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        f32x4 v = red[0][mt][lane];
        for (int w = 1; w < kW; ++w) {
          const f32x4 o = red[w][mt][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += o[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = mt * 16 + 4 * q + r;
          if (live && tok < a.M) a.Y[(size_t)tok * a.ld_y + row] = v[r];
        }
      }
    }
  }
}

struct W4Plan {
  int Mp, W, nchunks, nblocks;
  size_t off_xs, off_xsum, total;
};

static W4Plan w4_plan(int64_t M, int64_t d_in, int64_t d_out) {
  W4Plan p;
  p.Mp = M <= 16 ? 16 : M <= 32 ? 32 : 64;
  p.nchunks = (int)(d_in / kW4Chunk);
  p.nblocks = (int)cdiv(d_out, 16);
  // waves per workgroup splitting the chunks: at most 4 (measured faster than
  // 8 or 2 on the 70B and MoE shapes), each with >= 4 chunks
  p.W = 1;
  while (p.W < 4 && p.nchunks / (2 * p.W) >= 4) p.W *= 2;
  Carver cv(nullptr);
  cv.take<uint16_t>((size_t)p.Mp * d_in);
  p.off_xs = 0;
  p.off_xsum = align_up(cv.used, 256);
  cv.take<float>((size_t)p.nchunks * p.Mp);
  p.total = cv.used + 256;
  return p;
}

size_t w4a16_workspace_bytes(int64_t M, int64_t d_in, int64_t d_out) { return w4_plan(M, d_in, d_out).total; }

// Activations in LDS when few tokens fit beside the staged scales in 64 KB.
static bool w4_lx(int64_t M, int64_t d_in, int ng, int nchunks, int W) {
  return M <= 4 && w4_lds_total(ng, (int)M, (int)d_in, nchunks, true, W * 64 * 16) <= 65536;
}

template <int kDt, int kMT, int kU, bool kLX>
static void launch_w4(const W4Args& a, const W4Plan& pl, hipStream_t st) {
  const dim3 grid((unsigned)pl.nblocks);
  const size_t lds = w4_lds_total(a.ng, a.M, a.K, a.nchunks, kLX, pl.W * kMT * 64 * (int)sizeof(f32x4));
  switch (pl.W) {
    case 1: hipLaunchKernelGGL((w4_main_kernel<kDt, kMT, kU, 1, kLX>), grid, dim3(64), lds, st, a); break;
    case 2: hipLaunchKernelGGL((w4_main_kernel<kDt, kMT, kU, 2, kLX>), grid, dim3(128), lds, st, a); break;
    default: hipLaunchKernelGGL((w4_main_kernel<kDt, kMT, kU, 4, kLX>), grid, dim3(256), lds, st, a); break;
  }
}

// Both entry points: arguments checked, workspace of at least pl.total bytes.
static gptq_status w4a16_enqueue(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                                 const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                                 const int32_t* perm, int64_t d_out, int32_t group_size, float* Y, int64_t ld_y,
                                 const W4Plan& pl, char* ws, bool timed, hipStream_t st) {
  uint16_t* Xs = reinterpret_cast<uint16_t*>(ws + pl.off_xs);
  float* xsum = reinterpret_cast<float*>(ws + pl.off_xsum);
  const int K = (int)d_in;
  {
    TimedScope ts(timed ? kTimeW4Stage : -1, st);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    if (x_dtype == GPTQ_F16)
      hipLaunchKernelGGL(w4_stage_kernel<GPTQ_F16>, dim3((unsigned)pl.nchunks), dim3(256), 0, st, Xh, ld_x, (int)M,
                         pl.Mp, K, perm, Xs, xsum);
    else
      hipLaunchKernelGGL(w4_stage_kernel<GPTQ_BF16>, dim3((unsigned)pl.nchunks), dim3(256), 0, st, Xh, ld_x, (int)M,
                         pl.Mp, K, perm, Xs, xsum);
    GQ_LAUNCHED();
  }
  W4Args a;
  a.qw = reinterpret_cast<const u32x4*>(qweight);
  a.scales = scales;
  a.zeros = zeros;
  a.Xs = reinterpret_cast<const u32x4*>(Xs);
  a.xsum = xsum;
  a.Y = Y;
  a.d_out = d_out;
  a.ld_y = ld_y;
  a.K = K;
  a.ng = (int)(d_in / group_size);
  a.gch = group_size / kW4Chunk;
  a.M = (int)M;
  a.Mp = pl.Mp;
  a.nchunks = pl.nchunks;
  {
    TimedScope ts(timed ? kTimeW4Main : -1, st);
    const int mt = pl.Mp / 16;
    const bool lx = w4_lx(M, d_in, a.ng, pl.nchunks, pl.W);
    if (x_dtype == GPTQ_F16) {
      if (lx) launch_w4<GPTQ_F16, 1, 8, true>(a, pl, st);
      else if (mt == 1) launch_w4<GPTQ_F16, 1, 4, false>(a, pl, st);
      else if (mt == 2) launch_w4<GPTQ_F16, 2, 2, false>(a, pl, st);
      else launch_w4<GPTQ_F16, 4, 1, false>(a, pl, st);
    } else {
      if (lx) launch_w4<GPTQ_BF16, 1, 8, true>(a, pl, st);
      else if (mt == 1) launch_w4<GPTQ_BF16, 1, 4, false>(a, pl, st);
      else if (mt == 2) launch_w4<GPTQ_BF16, 2, 2, false>(a, pl, st);
      else launch_w4<GPTQ_BF16, 4, 1, false>(a, pl, st);
    }
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}

// Argument checks shared by both entry points (before any HIP call).
static gptq_status w4a16_check(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                               const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t d_out,
                               int32_t group_size, const float* Y, int64_t ld_y) {
  GQ_CHECK_ARG(X && qweight && scales && zeros && Y);
  GQ_CHECK_ARG(x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(M >= 1 && d_out >= 1 && d_out <= (int64_t)1 << 24);
  GQ_CHECK_ARG(d_in >= kW4Chunk && d_in % kW4Chunk == 0 && d_in <= 65536);
  GQ_CHECK_ARG(ld_x >= d_in && ld_y >= d_out);
  GQ_CHECK_ARG(group_size >= 1 && d_in % group_size == 0);
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(qweight) % 16 == 0);
  if (group_size % kW4Chunk != 0 || M > 64) return GPTQ_EUNSUPPORTED;
  return GPTQ_OK;
}

// Scratch of the allocation-free entry point: the workspace of the largest
// call the W4A16 path accepts (64 tokens, 65536 input channels).  Each GPU
// the library runs on holds its own copy for the life of the process; host
// code reaches it only through the address hipGetSymbolAddress returns for
// the current device.  Nothing in it has to start at zero: the staging
// kernel writes every element the main kernel reads.
constexpr size_t kW4ScratchBytes = 8519936;
static __device__ __align__(256) char scratch[kW4ScratchBytes];

static std::mutex scratch_mu;
static void* scratch_ptr[64] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device (with the device current) and kept.
static gptq_status scratch_address(void** out) {
  int dev = 0;
  GQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return GPTQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    GQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return GPTQ_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return GPTQ_OK;
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_w4a16_matmul(const void* X, int32_t x_dtype, int64_t M, int64_t d_in, int64_t ld_x,
                                         const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                                         const int32_t* perm, int64_t d_out, int32_t group_size, float* Y,
                                         int64_t ld_y, void* workspace, size_t ws_bytes, void* stream) {
  gptq_status s = w4a16_check(X, x_dtype, M, d_in, ld_x, qweight, scales, zeros, d_out, group_size, Y, ld_y);
  if (s != GPTQ_OK) return s;
  const W4Plan pl = w4_plan(M, d_in, d_out);
  if (workspace == nullptr || ws_bytes < pl.total) return GPTQ_ENOMEM;
  return w4a16_enqueue(X, x_dtype, M, d_in, ld_x, qweight, scales, zeros, perm, d_out, group_size, Y, ld_y, pl,
                       static_cast<char*>(workspace), true, static_cast<hipStream_t>(stream));
}

extern "C" gptq_status gptq_w4a16_matmul_noalloc(const void* X, int32_t x_dtype, int64_t M, int64_t d_in,
                                                 int64_t ld_x, const uint8_t* qweight, const uint16_t* scales,
                                                 const uint8_t* zeros, const int32_t* perm, int64_t d_out,
                                                 int32_t group_size, float* Y, int64_t ld_y, void* stream) {
  gptq_status s = w4a16_check(X, x_dtype, M, d_in, ld_x, qweight, scales, zeros, d_out, group_size, Y, ld_y);
  if (s != GPTQ_OK) return s;
  const W4Plan pl = w4_plan(M, d_in, d_out);
  if (pl.total > kW4ScratchBytes) return GPTQ_ENOMEM;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != GPTQ_OK) return s;
  return w4a16_enqueue(X, x_dtype, M, d_in, ld_x, qweight, scales, zeros, perm, d_out, group_size, Y, ld_y, pl,
                       static_cast<char*>(ws), false, static_cast<hipStream_t>(stream));
}
