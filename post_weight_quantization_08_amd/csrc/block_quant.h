// Block quantization of one 128-column tile: the column loop with in-tile
// error feedback ("INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍", section 三 listing;
// ipipp.com quantize_gptq listing, processed in blocks).
//
// kL lanes (4 or 8) share a weight row; lane j holds the tile's columns j,
// j+kL, ... in registers.  Per column the owner lane's error is broadcast with
// DPP moves and every lane updates its remaining columns from an LDS copy of
// U[tile, tile] laid out per lane, each row divided by its diagonal entry
// (prepared once per layer for every tile by prep_ud_kernel).  The kernel
// template is instantiated per workgroup shape in bq_*.hip, so the large
// unrolled variants compile in parallel.
#pragma once

#include <utility>

#include "common.h"

namespace gq {

// A weight row is held by kL lanes (4 or 8): lane j has the tile's columns
// j, j + kL, ...  (kQBlock / kL of them); a workgroup of kT threads holds
// kT / kL rows.
template <int kL>
constexpr int cols_per_lane() { return kQBlock / kL; }

// position of tile column c (0..127) in the lane-major k order used for Err
// and the transposed U: lane j = c % kL owns slots j * 128 / kL onwards.
__host__ __device__ __forceinline__ int lane_major(int c, int kl) { return (c % kl) * (kQBlock / kl) + c / kl; }

// Slot of element (k, c) of a tile's scaled U rows (c = j + kL i, lane j's
// i-th column) in LDS: row k holds lane 0's kQBlock / kL entries, then lane
// 1's, ...; within a lane's run the 16-byte chunks are swapped pairwise for
// the lanes whose run starts in the second half of the 64 banks, so the
// lanes of a wave reading the same chunk index fall in distinct banks.
__host__ __device__ __forceinline__ int ud_swz(int j, int kl) { return ((j * (kQBlock / kl)) >> 6) & 1; }
__host__ __device__ __forceinline__ int ud_slot(int k, int c, int kl) {
  const int cpl = kQBlock / kl, j = c % kl, i = c / kl;
  return (k * kl + j) * cpl + ((((i >> 2) ^ ud_swz(j, kl)) << 2) | (i & 3));
}

struct QArgs {
  const float* U;      // [batch][d][d]
  const float* Ud;     // [batch][d / 128][128 * 128]: each tile's scaled U rows in ud_slot order
  const int32_t* perm; // [batch][d] or null
  float* Wc;           // [batch][d_out][d]
  uint16_t* ErrH;      // [batch][d_out][d]: every column's error w - dq
  uint16_t* ErrL;
  int err_ld;          // row length of ErrH / ErrL (= d)
  int err_off;         // first column of this tile in ErrH / ErrL
  uint8_t* codes;      // [batch][d_out][d]
  uint16_t* scales;    // [batch][d_out][ng]
  uint8_t* zeros;
  float* Q;            // optional
  int64_t d_out;        // rows of every batch entry (the stride between entries)
  int64_t r0, r1;       // rows [r0, r1) of every entry are quantized by this launch
  int d;
  int ng;
  int g;
  int b0;              // first column of the tile (quantization order)
  float maxq;
  int sym;             // symmetric groups: zero fixed at (maxq + 1) / 2
  const int32_t* gidx; // [batch][d]: group of each original column
};

// v of lane src (compile time) of this lane's group of kL lanes, on every
// lane of the group: a quad_perm broadcast inside each quad; for kL = 8 the
// other quad of the group then copies it from 4 lanes away, writing only its
// own banks (bank_mask), so no select is needed.
template <int kL, int src>
__device__ __forceinline__ float group_bcast(float v) {
  constexpr int qp = (src & 3) * 0x55;   // quad_perm:[s,s,s,s]
  const int q = __builtin_amdgcn_mov_dpp(__float_as_int(v), qp, 0xF, 0xF, false);
  if constexpr (kL == 4) {
    return __int_as_float(q);
  } else {
    constexpr int ctrl = (src & 4) ? 0x104 : 0x114;   // row_shl:4 (lane + 4) / row_shr:4 (lane - 4)
    constexpr int banks = (src & 4) ? 0x5 : 0xA;      // the quads of each 8-lane group that lack the value
    return __int_as_float(__builtin_amdgcn_update_dpp(q, q, ctrl, 0xF, banks, false));
  }
}

template <int kL>
__device__ __forceinline__ float group_min(float v) {
  v = fminf(v, __shfl_xor(v, 1));
  v = fminf(v, __shfl_xor(v, 2));
  if constexpr (kL == 8) v = fminf(v, __shfl_xor(v, 4));
  return v;
}
template <int kL>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  if constexpr (kL == 8) v = fmaxf(v, __shfl_xor(v, 4));
  return v;
}

// Codes are kept as float bits, one register per column.
template <int kL>
constexpr int code_regs() { return cols_per_lane<kL>(); }
template <int kL>
__device__ __forceinline__ uint32_t code_of(const uint32_t (&qv)[code_regs<kL>()], int i) {
  return (uint32_t)__uint_as_float(qv[i]);
}

__device__ __forceinline__ uint32_t bf16_hi(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ uint32_t bf16_lo(float x, uint32_t hi) {
  return f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Per-workgroup state of one tile shared by all column steps.
template <int kL>
struct BQCtx {
  const float* ue;  // LDS: this lane's run of scaled U row 0, for even chunk indices (ud_slot)
  const float* uo;  // the same for odd chunk indices
  const float* wrow;
  uint16_t* scales;
  uint8_t* zeros;
  size_t grow;      // (b * d_out + r) * ng
  int j, b0, g;
  bool live;
  float maxq;
  bool sym;
};

// G = columns of a group inside one tile (group_size if <= 128, else 128);
// kBig: group_size > 128 (a group opens at a tile start and spans tiles).
// G == 0 selects static groups: every group's scale and zero were fixed
// before the loop (groups of original columns), so no step opens a group;
// the lane holds its columns' fp16 scales (two per word) and zeros (four per
// word) in pk[].
template <int G>
constexpr int groups_in_tile() { return G == 0 ? 1 : (G < kQBlock ? kQBlock / G : 1); }
template <int kL, int G>
constexpr int pk_words() { return G == 0 ? cols_per_lane<kL>() / 2 + cols_per_lane<kL>() / 4 : 1; }

template <int kL>
__device__ __forceinline__ float pk_scale(const uint32_t* pk, int i) {
  return f16_bits_to_f32((pk[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
}
template <int kL>
__device__ __forceinline__ float pk_zero(const uint32_t* pk, int i) {
  return (float)((pk[cols_per_lane<kL>() / 2 + (i >> 2)] >> (8 * (i & 3))) & 0xFFu);
}

// The lane's part of scaled U row K, entries i >= K / kL (exactly the ones
// step K multiplies, so every register a load writes is used): the entries
// before the next 16-byte boundary one by one, the rest 16 bytes at a time.
template <int kL, int K>
__device__ __forceinline__ void bq_load_urow(const BQCtx<kL>& c, float (&u)[cols_per_lane<kL>()]) {
  if constexpr (K < kQBlock) {
    constexpr int kCPL = cols_per_lane<kL>();
    constexpr int i0 = K / kL;
    constexpr int ia = (i0 + 3) & ~3;
#pragma unroll
    for (int i = i0; i < ia && i < kCPL; ++i) u[i] = ((i >> 2) & 1 ? c.uo : c.ue)[K * kQBlock + i];
#pragma unroll
    for (int i = ia; i < kCPL; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(((i >> 2) & 1 ? c.uo : c.ue) + K * kQBlock + i);
      u[i] = v.x;
      u[i + 1] = v.y;
      u[i + 2] = v.z;
      u[i + 3] = v.w;
    }
  }
}

// One column step with a compile-time column index K, so the lane's register
// arrays are indexed statically.  The dependent chain from one column to the
// next: broadcast d_K -> update of column K+1 -> q = med3(rne(w / s) + z, 0,
// maxq) -> dq = s q - s z -> d = w - dq.  The owner lane keeps the column's d
// in w[] and its code in qv[] (as float bits; neither is needed by a later
// step).
template <int kL, int K, int G, bool kBig>
__device__ __forceinline__ void bq_step(const BQCtx<kL>& c, float (&w)[cols_per_lane<kL>()],
                                        uint32_t (&qv)[code_regs<kL>()], float& s, float& z, float& sz,
                                        float& y, float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                        const uint32_t (&pk)[pk_words<kL, G>()],
                                        const float (&ucur)[cols_per_lane<kL>()],
                                        float (&unext)[cols_per_lane<kL>()]) {
  constexpr int kCPL = cols_per_lane<kL>();
  constexpr int js = K % kL, is = K / kL;
  bq_load_urow<kL, K + 1>(c, unext);
  if constexpr (G == 0) {
    s = pk_scale<kL>(pk, is);
    z = pk_zero<kL>(pk, is);
    sz = s * z;
    y = __fdiv_rn(1.0f, s);
  } else {
    bool gstart;
    if constexpr (kBig) gstart = (K == 0) && (c.b0 % c.g == 0);
    else gstart = (K % G) == 0;
    if (gstart) {
      float lo = 3.402823466e38f, hi = -3.402823466e38f;
      constexpr int span = (G < kQBlock ? G : kQBlock) / kL;
#pragma unroll
      for (int i = is; i < is + span; ++i) {
        lo = fminf(lo, w[i]);
        hi = fmaxf(hi, w[i]);
      }
      if constexpr (kBig) {
        for (int col = kQBlock + c.j; col < c.g; col += kL) {
          float v = c.live ? c.wrow[c.b0 + col] : 0.0f;
          lo = fminf(lo, v);
          hi = fmaxf(hi, v);
        }
      }
      lo = group_min<kL>(lo);
      hi = group_max<kL>(hi);
      uint16_t sb;
      group_scale_zero(lo, hi, c.maxq, c.sym, s, z, sb);
      y = __fdiv_rn(1.0f, s);
      sz = s * z;
      sg[K / G] = s;
      zg[K / G] = z;
      if (c.j == 0 && c.live) {
        const size_t go = c.grow + (c.b0 + K) / c.g;
        c.scales[go] = sb;
        c.zeros[go] = (uint8_t)z;
      }
    }
  }
  // w / s correctly rounded from y = RN(1 / s): q0 = w y, the remainder
  // w - q0 s is exact under fma, and q0 + r y rounds to RN(w / s) (Markstein's
  // theorem).  s (q - z) is exact in fp32 (an fp16 value times a small
  // integer), so one fma against s z gives it.
  const float wv = w[is];
  const float q0 = wv * y;
  const float qf = fmaf(fmaf(-q0, s, wv), y, q0);
  const float q = __builtin_amdgcn_fmed3f(rintf(qf) + z, 0.0f, c.maxq);
  const float dq = fmaf(s, q, -sz);
  const float dd = wv - dq;
  const bool own = (c.j == js);
  w[is] = own ? dd : w[is];
  qv[is] = own ? __float_as_uint(q) : qv[is];
  // take the select here: left to itself the compiler sinks every step's
  // select to the epilogue and keeps all 128 codes of the tile live (about 130
  // extra registers, which halve the waves a SIMD can hold)
  asm volatile("" : "+v"(qv[is]));
  const float eb = group_bcast<kL, js>(dd);
#pragma unroll
  for (int i = is; i < kCPL; ++i) w[i] = fmaf(-eb, ucur[i], w[i]);
}

template <int kL, int K, int G, bool kBig>
__device__ __forceinline__ void bq_step2(const BQCtx<kL>& c, float (&w)[cols_per_lane<kL>()],
                                         uint32_t (&qv)[code_regs<kL>()], float& s, float& z, float& sz, float& y,
                                         float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                         const uint32_t (&pk)[pk_words<kL, G>()], float (&ua)[cols_per_lane<kL>()],
                                         float (&ub)[cols_per_lane<kL>()]) {
  if constexpr ((K & 1) == 0) bq_step<kL, K, G, kBig>(c, w, qv, s, z, sz, y, sg, zg, pk, ua, ub);
  else bq_step<kL, K, G, kBig>(c, w, qv, s, z, sz, y, sg, zg, pk, ub, ua);
}

template <int kL, int G, bool kBig, int... Ks>
__device__ __forceinline__ void bq_all_steps(std::integer_sequence<int, Ks...>, const BQCtx<kL>& c,
                                             float (&w)[cols_per_lane<kL>()], uint32_t (&qv)[code_regs<kL>()],
                                             float& s, float& z, float& sz, float& y,
                                             float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                             const uint32_t (&pk)[pk_words<kL, G>()]) {
  float ua[cols_per_lane<kL>()], ub[cols_per_lane<kL>()];   // U rows of even / odd steps
  bq_load_urow<kL, 0>(c, ua);
  (bq_step2<kL, Ks, G, kBig>(c, w, qv, s, z, sz, y, sg, zg, pk, ua, ub), ...);
}

template <int kL, int kT, int G, bool kBig>
__global__ __launch_bounds__(kT) void block_quant_kernel(QArgs a) {
  constexpr int kCPL = cols_per_lane<kL>();
  constexpr int kRows = kT / kL;
  __shared__ __attribute__((aligned(16))) float Ul[kQBlock * kQBlock];   // 64 KB
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[kRows][kQBlock];

  const int b = blockIdx.y;
  const int d = a.d;
  const int32_t* perm = a.perm ? a.perm + (size_t)b * d : nullptr;
  const int b0 = a.b0;
  const int tid = threadIdx.x;

  // the tile's scaled U rows, already in LDS order (prep_ud_kernel)
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.Ud + ((size_t)b * (d / kQBlock) + b0 / kQBlock) *
                                                                 (kQBlock * kQBlock));
    u32x4* dst = reinterpret_cast<u32x4*>(Ul);
#pragma unroll 4
    for (int e = tid; e < kQBlock * kQBlock / 4; e += kT) dst[e] = src[e];
  }
  __syncthreads();

  const int rloc = tid / kL;
  const int j = tid % kL;
  const int64_t r = a.r0 + (int64_t)blockIdx.x * kRows + rloc;
  const bool live = r < a.r1;
  const size_t rowoff = ((size_t)b * a.d_out + (live ? r : 0)) * d;
  float* wrow = a.Wc + rowoff;

  float w[kCPL];
  uint32_t qv[code_regs<kL>()];
#pragma unroll
  for (int i = 0; i < kCPL; ++i) w[i] = live ? wrow[b0 + j + kL * i] : 0.0f;
#pragma unroll
  for (int i = 0; i < code_regs<kL>(); ++i) qv[i] = 0u;

  BQCtx<kL> c;
  {
    const int sw = 4 * ud_swz(j, kL);
    c.ue = Ul + j * kCPL + sw;
    c.uo = Ul + j * kCPL - sw;
  }
  c.wrow = wrow;
  c.scales = a.scales;
  c.zeros = a.zeros;
  c.grow = ((size_t)b * a.d_out + (live ? r : 0)) * a.ng;
  c.j = j;
  c.b0 = b0;
  c.g = a.g;
  c.live = live;
  c.maxq = a.maxq;
  c.sym = a.sym != 0;
  float s = 1.0f, z = 0.0f;
  if constexpr (kBig) {
    // a group wider than the tile: a tile that does not open the group uses
    // the scale and zero stored by the tile that did (earlier in stream order)
    if (b0 % a.g != 0 && live) {
      const size_t go = c.grow + b0 / a.g;
      s = f16_bits_to_f32(a.scales[go]);
      z = (float)a.zeros[go];
    }
  }
  constexpr int kNG = groups_in_tile<G>();
  float sg[kNG], zg[kNG];   // scale and zero of each group of the tile
#pragma unroll
  for (int q = 0; q < kNG; ++q) {
    sg[q] = s;
    zg[q] = z;
  }
  uint32_t pk[pk_words<kL, G>()];
#pragma unroll
  for (int i = 0; i < pk_words<kL, G>(); ++i) pk[i] = 0u;
  if constexpr (G == 0) {
    // each of the lane's columns takes its original column's group
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      const int col = b0 + j + kL * i;
      const int oc = perm ? perm[col] : col;
      const size_t go = c.grow + a.gidx[(size_t)b * d + oc];
      const uint32_t sb = live ? (uint32_t)a.scales[go] : 0x3C00u;
      const uint32_t zb = live ? (uint32_t)a.zeros[go] : 0u;
      pk[i >> 1] |= sb << (16 * (i & 1));
      pk[kCPL / 2 + (i >> 2)] |= zb << (8 * (i & 3));
    }
  }
  float y = __fdiv_rn(1.0f, s);   // 1 / s of the group in force
  float sz = s * z;
  bq_all_steps<kL, G, kBig>(std::make_integer_sequence<int, kQBlock>{}, c, w, qv, s, z, sz, y, sg, zg, pk);
  // this lane's codes (columns j, j+kL, ...) into the row's byte buffer
#pragma unroll
  for (int i = 0; i < kCPL; ++i) qbuf[rloc][j + kL * i] = (uint8_t)code_of<kL>(qv, i);

  // errors of the tile (now in w), lane-major (two-term bf16 split) for the GEMM
  if (live) {
    const size_t eo = ((size_t)b * a.d_out + r) * a.err_ld + a.err_off + j * kCPL;
#pragma unroll
    for (int i = 0; i < kCPL; i += 2) {
      uint32_t h0 = bf16_hi(w[i]), h1 = bf16_hi(w[i + 1]);
      uint32_t l0 = bf16_lo(w[i], h0), l1 = bf16_lo(w[i + 1], h1);
      *reinterpret_cast<uint32_t*>(a.ErrH + eo + i) = h0 | (h1 << 16);
      *reinterpret_cast<uint32_t*>(a.ErrL + eo + i) = l0 | (l1 << 16);
    }
    if (a.Q) {
      // dequantized values from the codes; lane column i = tile column
      // j + kL i lies in group kL i / G of the tile (G is a multiple of kL)
      float* qrow = a.Q + ((size_t)b * a.d_out + r) * d;
#pragma unroll
      for (int i = 0; i < kCPL; ++i) {
        const int col = b0 + j + kL * i;
        float sv, zv;
        if constexpr (G == 0) {
          sv = pk_scale<kL>(pk, i);
          zv = pk_zero<kL>(pk, i);
        } else {
          const int gq = kNG > 1 ? (kL * i) / G : 0;
          sv = sg[gq];
          zv = zg[gq];
        }
        qrow[perm ? perm[col] : col] = sv * ((float)code_of<kL>(qv, i) - zv);
      }
    }
  }
  __syncthreads();
  if (live) {
    uint8_t* crow = a.codes + ((size_t)b * a.d_out + r) * d;
    if (perm) {
      for (int col = j * kCPL; col < (j + 1) * kCPL; ++col) crow[perm[b0 + col]] = qbuf[rloc][col];
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(&qbuf[rloc][j * kCPL]);
      u32x4* dst = reinterpret_cast<u32x4*>(crow + b0 + j * kCPL);
#pragma unroll
      for (int v = 0; v < kCPL / 16; ++v) dst[v] = src[v];
    }
  }
}


template <int kL, int kT, int G, bool kBig>
void launch_bq(const QArgs& a, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)cdiv(a.r1 - a.r0, kT / kL), (unsigned)batch);
  hipLaunchKernelGGL((block_quant_kernel<kL, kT, G, kBig>), grid, dim3(kT), 0, st, a);
}

// Every dynamic-group variant of one shape (g 16, 32, 64, 128, or wider than a tile).
template <int kL, int kT>
void launch_bq_g(const QArgs& a, int g, int64_t batch, hipStream_t st) {
  switch (g) {
    case 16: launch_bq<kL, kT, 16, false>(a, batch, st); break;
    case 32: launch_bq<kL, kT, 32, false>(a, batch, st); break;
    case 64: launch_bq<kL, kT, 64, false>(a, batch, st); break;
    case 128: launch_bq<kL, kT, 128, false>(a, batch, st); break;
    default: launch_bq<kL, kT, 128, true>(a, batch, st); break;
  }
}

// Instantiated in bq_*.hip.
void launch_bq_8x256(const QArgs& a, int g, int64_t batch, hipStream_t st);
void launch_bq_8x512(const QArgs& a, int g, int64_t batch, hipStream_t st);
void launch_bq_static(const QArgs& a, int64_t batch, hipStream_t st);

}  // namespace gq
