// Column-by-column group quantization with error feedback, in 128-column tiles.
//
// The loop is the one of "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍" section 三 and
// of the ipipp.com quantize_gptq listing: quantize column k, divide its error by
// the diagonal of the inverse-Hessian factor, subtract error x factor row from
// every later column.  Columns are processed in 128-wide tiles (the same page's
// "按块处理", process in blocks): inside a tile the updates are applied at once
// by `block_quant_kernel`; the later columns receive the tile's updates together
// through GEMMs, W[:, rest] -= Err U[tile, rest] (`update_kernel`), in two
// levels: inside a super-block of up to 1024 columns after every tile, beyond
// it once per super-block.
//
// block_quant: kL lanes (4 or 8) share a weight row; lane j holds the tile's
// columns j, j+kL, ... in registers.  Per column the owner lane's error is
// broadcast with DPP moves (quad_perm, and for 8 lanes a row shift by 4) and
// every lane updates its remaining columns from an LDS copy of U[tile, tile]
// laid out per lane.
//
// trailing: a bf16 MFMA GEMM with three products (hi*hi + hi*lo + lo*hi) of a
// two-term bf16 split of Err and U, so the update keeps about 16 significant
// bits while the working copy stays fp32.
#include <cmath>
#include <utility>

#include "common.h"

bool gq_params_ok(const gptq_params* p, int64_t d_in);

namespace gq {

// A weight row is held by kL lanes (4 or 8): lane j has the tile's columns
// j, j + kL, ...  (kQBlock / kL of them); 256 threads hold 256 / kL rows.
template <int kL>
constexpr int rows_per_wg() { return 256 / kL; }
template <int kL>
constexpr int cols_per_lane() { return kQBlock / kL; }

// position of tile column c (0..127) in the lane-major k order used for Err
// and the transposed U: lane j = c % kL owns slots j * 128 / kL onwards.
__host__ __device__ __forceinline__ int lane_major(int c, int kl) { return (c % kl) * (kQBlock / kl) + c / kl; }

struct QArgs {
  const float* U;      // [batch][d][d]
  const int32_t* perm; // [batch][d] or null
  float* Wc;           // [batch][d_out][d]
  uint16_t* ErrH;      // [batch][d_out][err_ld]: errors of the current super-block
  uint16_t* ErrL;
  int err_ld;          // columns per super-block
  int err_off;         // offset of this tile inside the super-block
  uint8_t* codes;      // [batch][d_out][d]
  uint16_t* scales;    // [batch][d_out][ng]
  uint8_t* zeros;
  float* Q;            // optional
  int64_t d_out;
  int d;
  int ng;
  int g;
  int b0;              // first column of the tile (quantization order)
  float maxq;
  int sym;             // symmetric groups: zero fixed at (maxq + 1) / 2
  const int32_t* gidx; // [batch][d]: group of each original column
};

__device__ __forceinline__ float quad_bcast(float v, int src) {
  int iv = __float_as_int(v);
  int r;
  switch (src) {
    case 0: r = __builtin_amdgcn_mov_dpp(iv, 0x00, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_mov_dpp(iv, 0x55, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(iv, 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_mov_dpp(iv, 0xFF, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

// v of lane src (compile time) of this lane's group of kL lanes.  For kL = 8:
// broadcast inside each quad, then the other quad takes it from 4 lanes away
// (row_shr:4 / row_shl:4 stay inside the 16-lane DPP row).
template <int kL, int src>
__device__ __forceinline__ float group_bcast(float v) {
  const float qv = quad_bcast(v, src & 3);
  if constexpr (kL == 4) {
    return qv;
  } else {
    const int iq = __float_as_int(qv);
    constexpr int ctrl = (src & 4) ? 0x104 : 0x114;   // lower quad gets lane + 4, upper quad lane - 4
    const float other = __int_as_float(__builtin_amdgcn_mov_dpp(iq, ctrl, 0xF, 0xF, false));
    const bool mine = ((threadIdx.x >> 2) & 1) == ((src >> 2) & 1);
    return mine ? qv : other;
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

__device__ __forceinline__ uint32_t bf16_hi(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ uint32_t bf16_lo(float x, uint32_t hi) {
  return f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// w / s rounded to nearest from y = RN(1 / s): q0 = w y, the remainder
// w - q0 s is exact under fma, and one correction q0 + r y rounds to RN(w / s)
// (Markstein's theorem: y within half an ulp of 1 / s, q0 within one ulp of
// w / s).  One reciprocal per group replaces a full division per element.
__device__ __forceinline__ float div_rn(float w, float s, float y) {
  const float q0 = w * y;
  return fmaf(fmaf(-q0, s, w), y, q0);
}

// Per-workgroup state of one tile shared by all column steps.
template <int kL>
struct BQCtx {
  const f32x4 (*Ul)[kL][cols_per_lane<kL>() / 4];
  const float* rinv;
  const float* wrow;
  uint16_t* scales;
  uint8_t* zeros;
  size_t grow;      // (b * d_out + r) * ng
  int rloc, j, b0, g;
  bool live;
  float maxq;
  bool sym;
};

// One column step with a compile-time column index K, so the lane's register
// array is indexed statically.  G = columns of a group inside one tile
// (group_size if <= 128, else 128); kBig: group_size > 128 (a group starts at
// a tile start and spans tiles).
// After its step, the owner lane keeps the column's scaled error in w[] (the
// column's value is not needed again).
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

// The lane's part of U row K + 1 and 1 / U[K+1][K+1] are read from LDS at the
// start of step K, so their latency hides behind step K's dependency chain.
template <int kL, int K>
__device__ __forceinline__ void bq_load_urow(const BQCtx<kL>& c, f32x4 (&u)[cols_per_lane<kL>() / 4], float& rinv) {
  if constexpr (K < kQBlock) {
    const f32x4* urow = &c.Ul[K][c.j][0];
#pragma unroll
    for (int i4 = (K / kL) / 4; i4 < cols_per_lane<kL>() / 4; ++i4) u[i4] = urow[i4];
    rinv = c.rinv[K];
  }
}

template <int kL, int K, int G, bool kBig>
__device__ __forceinline__ void bq_step(const BQCtx<kL>& c, float (&w)[cols_per_lane<kL>()],
                                        uint32_t (&cq)[cols_per_lane<kL>() / 4], float& s, float& z, float& y,
                                        float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                        const uint32_t (&pk)[pk_words<kL, G>()],
                                        const f32x4 (&ucur)[cols_per_lane<kL>() / 4],
                                        f32x4 (&unext)[cols_per_lane<kL>() / 4], const float& rcur, float& rnext) {
  constexpr int kCPL = cols_per_lane<kL>();
  constexpr int js = K % kL, is = K / kL;
  bq_load_urow<kL, K + 1>(c, unext, rnext);
  if constexpr (G == 0) {
    s = pk_scale<kL>(pk, is);
    z = pk_zero<kL>(pk, is);
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
      sg[K / G] = s;
      zg[K / G] = z;
      if (c.j == 0 && c.live) {
        const size_t go = c.grow + (c.b0 + K) / c.g;
        c.scales[go] = sb;
        c.zeros[go] = (uint8_t)z;
      }
    }
  }
  const float wv = w[is];
  const float q = fminf(fmaxf(rintf(div_rn(wv, s, y)) + z, 0.0f), c.maxq);
  const float dq = s * (q - z);
  const float e = (wv - dq) * rcur;
  const bool own = (c.j == js);
  w[is] = own ? e : w[is];
  cq[is >> 2] = own ? (cq[is >> 2] | ((uint32_t)q << (8 * (is & 3)))) : cq[is >> 2];
  const float eb = group_bcast<kL, js>(e);
#pragma unroll
  for (int i4 = is / 4; i4 < kCPL / 4; ++i4) {
    const f32x4 u = ucur[i4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = i4 * 4 + t;
      if (i >= is) w[i] = fmaf(-eb, u[t], w[i]);
    }
  }
}

template <int kL, int K, int G, bool kBig>
__device__ __forceinline__ void bq_step2(const BQCtx<kL>& c, float (&w)[cols_per_lane<kL>()],
                                         uint32_t (&cq)[cols_per_lane<kL>() / 4], float& s, float& z, float& y,
                                         float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                         const uint32_t (&pk)[pk_words<kL, G>()],
                                         f32x4 (&ua)[cols_per_lane<kL>() / 4], f32x4 (&ub)[cols_per_lane<kL>() / 4],
                                         float& ra, float& rb) {
  if constexpr ((K & 1) == 0) bq_step<kL, K, G, kBig>(c, w, cq, s, z, y, sg, zg, pk, ua, ub, ra, rb);
  else bq_step<kL, K, G, kBig>(c, w, cq, s, z, y, sg, zg, pk, ub, ua, rb, ra);
}

template <int kL, int G, bool kBig, int... Ks>
__device__ __forceinline__ void bq_all_steps(std::integer_sequence<int, Ks...>, const BQCtx<kL>& c,
                                             float (&w)[cols_per_lane<kL>()],
                                             uint32_t (&cq)[cols_per_lane<kL>() / 4], float& s, float& z, float& y,
                                             float (&sg)[groups_in_tile<G>()], float (&zg)[groups_in_tile<G>()],
                                             const uint32_t (&pk)[pk_words<kL, G>()]) {
  f32x4 ua[cols_per_lane<kL>() / 4], ub[cols_per_lane<kL>() / 4];   // U rows of even / odd steps
  float ra = 0.f, rb = 0.f;                                         // their 1 / U[k][k]
  bq_load_urow<kL, 0>(c, ua, ra);
  (bq_step2<kL, Ks, G, kBig>(c, w, cq, s, z, y, sg, zg, pk, ua, ub, ra, rb), ...);
}

template <int kL, int G, bool kBig>
__global__ __launch_bounds__(256) void block_quant_kernel(QArgs a) {
  constexpr int kCPL = cols_per_lane<kL>();
  constexpr int kRows = rows_per_wg<kL>();
  __shared__ f32x4 Ul[kQBlock][kL][kCPL / 4];   // 64 KB
  __shared__ float rinv[kQBlock];
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[kRows][kQBlock];   // 16 KB / kL

  const int b = blockIdx.y;
  const int d = a.d;
  const float* U = a.U + (size_t)b * d * d;
  const int32_t* perm = a.perm ? a.perm + (size_t)b * d : nullptr;
  const int b0 = a.b0;
  const int tid = threadIdx.x;

  // U[tile, tile] -> Ul[k][j][i] = U[b0+k][b0+j+kL i] for j+kL i > k, else 0
  for (int e = tid; e < kQBlock * kQBlock; e += 256) {
    int k = e >> 7, col = e & 127;
    float v = (col > k) ? U[(size_t)(b0 + k) * d + b0 + col] : 0.0f;
    int jj = col % kL, i = col / kL;
    reinterpret_cast<float*>(&Ul[k][jj][0])[i] = v;
  }
  if (tid < kQBlock) rinv[tid] = 1.0f / U[(size_t)(b0 + tid) * d + b0 + tid];
  __syncthreads();

  const int rloc = tid / kL;
  const int j = tid % kL;
  const int64_t r = (int64_t)blockIdx.x * kRows + rloc;
  const bool live = r < a.d_out;
  const size_t rowoff = ((size_t)b * a.d_out + (live ? r : 0)) * d;
  float* wrow = a.Wc + rowoff;

  float w[kCPL];
#pragma unroll
  for (int i = 0; i < kCPL; ++i) w[i] = live ? wrow[b0 + j + kL * i] : 0.0f;

  BQCtx<kL> c;
  c.Ul = Ul;
  c.rinv = rinv;
  c.wrow = wrow;
  c.scales = a.scales;
  c.zeros = a.zeros;
  c.grow = ((size_t)b * a.d_out + (live ? r : 0)) * a.ng;
  c.rloc = rloc;
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
  uint32_t cq[kCPL / 4];
#pragma unroll
  for (int i = 0; i < kCPL / 4; ++i) cq[i] = 0u;
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
  bq_all_steps<kL, G, kBig>(std::make_integer_sequence<int, kQBlock>{}, c, w, cq, s, z, y, sg, zg, pk);
  // this lane's codes (columns j, j+kL, ...) into the row's byte buffer
#pragma unroll
  for (int i = 0; i < kCPL; ++i) qbuf[rloc][j + kL * i] = (uint8_t)(cq[i >> 2] >> (8 * (i & 3)));

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
        const int q = (int)((cq[i >> 2] >> (8 * (i & 3))) & 0xFFu);
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
        qrow[perm ? perm[col] : col] = sv * ((float)q - zv);
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

// Static groups: scale and zero of every (row, group of g consecutive
// original columns) from the weights as given, one wave per group (lanes
// stride the group's columns, then a wave-wide min / max).  The index u of a
// group is its position in scales / zeros: ((b * d_out + r) * ng + group).
template <int kDt>
__global__ __launch_bounds__(256) void static_params_kernel(const void* __restrict__ W, int64_t ld_w, int g, int ng,
                                                            int64_t units, float maxq, int sym,
                                                            uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
    const int64_t row = u / ng;
    const size_t base = (size_t)row * ld_w + (size_t)(u - row * ng) * g;
    float lo = 3.402823466e38f, hi = -3.402823466e38f;
    for (int c = lane; c < g; c += 64) {
      float v;
      if constexpr (kDt == 0) v = static_cast<const float*>(W)[base + c];
      else if constexpr (kDt == 1) v = f16_bits_to_f32(static_cast<const uint16_t*>(W)[base + c]);
      else v = bf16_bits_to_f32(static_cast<const uint16_t*>(W)[base + c]);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if (lane == 0) {
      float s, z;
      uint16_t sb;
      group_scale_zero(lo, hi, maxq, sym != 0, s, z, sb);
      scales[u] = sb;
      zeros[u] = (uint8_t)z;
    }
  }
}

// Wc[b][r][k] = W[b][r][perm[k]] as fp32.
template <int kDt>
__global__ __launch_bounds__(256) void prep_w_kernel(const void* __restrict__ W, int64_t ld_w, int64_t d_out, int d,
                                                     const int32_t* __restrict__ perm, float* __restrict__ Wc) {
  const int b = blockIdx.z;
  const int64_t r = blockIdx.x;
  const int32_t* pb = perm ? perm + (size_t)b * d : nullptr;
  const size_t src_row = ((size_t)b * d_out + r) * ld_w;
  float* dst = Wc + ((size_t)b * d_out + r) * d;
  for (int k = blockIdx.y * 256 + threadIdx.x; k < d; k += gridDim.y * 256) {
    const int c = pb ? pb[k] : k;
    float v;
    if constexpr (kDt == 0) v = static_cast<const float*>(W)[src_row + c];
    else if constexpr (kDt == 1) v = f16_bits_to_f32(static_cast<const uint16_t*>(W)[src_row + c]);
    else v = bf16_bits_to_f32(static_cast<const uint16_t*>(W)[src_row + c]);
    dst[k] = v;
  }
}

// UtH/UtL[b][n][t0 + lane_major(k - t0)] = split(U[b][k][n]) for k in tiles
// strictly before n's tile (the only entries the deferred update reads); kl
// is the block quantizer's lanes per row, which fixes the Err column order.
__global__ __launch_bounds__(256) void prep_u_kernel(const float* __restrict__ U, int d, int kl,
                                                     uint16_t* __restrict__ UtH, uint16_t* __restrict__ UtL) {
  const int b = blockIdx.z;
  const float* Ub = U + (size_t)b * d * d;
  __shared__ float t[32][33];
  const int k0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  if ((k0 / kQBlock) >= ((n0 + 31) / kQBlock)) return;   // no entry of this tile is read
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int rr = ty; rr < 32; rr += 8) {
    int k = k0 + rr, n = n0 + tx;
    t[rr][tx] = (k < d && n < d) ? Ub[(size_t)k * d + n] : 0.f;
  }
  __syncthreads();
  for (int rr = ty; rr < 32; rr += 8) {
    int n = n0 + rr, k = k0 + tx;
    if (n < d && k < d && (k / kQBlock) < (n / kQBlock)) {
      float v = t[tx][rr];
      uint32_t h = f32_to_bf16_bits(v);
      uint32_t l = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
      size_t o = (size_t)b * d * d + (size_t)n * d + (k / kQBlock) * kQBlock + lane_major(k % kQBlock, kl);
      UtH[o] = (uint16_t)h;
      UtL[o] = (uint16_t)l;
    }
  }
}

__global__ void gidx_kernel(const int32_t* __restrict__ perm, int d, int g, int batch, int32_t* __restrict__ gidx) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)d * batch) return;
  int b = (int)(e / d), k = (int)(e % d);
  int col = perm ? perm[(size_t)b * d + k] : k;
  gidx[(size_t)b * d + col] = k / g;
}

// Deferred update W[b][:, n0:n1] -= Err[b][:, k0:k0+K] Ut[b][n0:n1][u0:u0+K]^T as a
// split-bf16 MFMA GEMM: 128x128 output tile per workgroup, 4 waves of 64x64
// (2 x 2 blocks of 32x32x16), K staged through LDS 32 at a time, double
// buffered, with the next stage prefetched into registers.
struct UpdArgs {
  float* Wc;
  const uint16_t* ErrH;
  const uint16_t* ErrL;
  const uint16_t* UtH;
  const uint16_t* UtL;
  int64_t d_out;
  int d;
  int err_ld, err_k0;   // Err columns [err_k0, err_k0 + K) of rows of length err_ld
  int u0;               // matching k range in Ut rows
  int K;
  int n0, n1;
};

// W[rows, n0:n1] -= Err[rows, K] Ut[n0:n1, K]^T on MFMA.  A workgroup owns kR
// rows x 128 columns of W; its waves own 64 x 64 blocks.  Both operands are
// K-contiguous rows (Err rows, rows of the transposed U), so they stream
// global -> LDS unchanged (buffer loads straight into LDS, 16 bytes per lane)
// through a ring of three 32-k stages, and every MFMA fragment is one 16-byte
// LDS read.  An LDS row is 64 bytes (32 bf16 of k); its 16-byte k-chunk c sits
// at slot c ^ ((row / 2) % 4), so 8 lanes reading 8 consecutive rows touch 8
// distinct bank groups.  The workgroup's W elements are read at the start,
// so that latency hides behind the K loop.
constexpr int kUK = 32;          // k per LDS stage
constexpr int kURow = kUK * 2;   // bytes per LDS row

template <int kR>
constexpr int upd_stage_bytes() { return 2 * kR * kURow + 2 * 128 * kURow; }

template <int kR>
__global__ __launch_bounds__(2 * kR) void update_kernel(UpdArgs u) {
  constexpr int kW = kR / 32;                        // waves
  constexpr int kStageB = upd_stage_bytes<kR>();
  constexpr int kChunks = kStageB / 1024;            // 1 KiB direct-load chunks per stage
  constexpr int kPerWave = kChunks / kW;
  __shared__ __attribute__((aligned(1024))) char ring0[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring1[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring2[kStageB];
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: picks operand buffers
  const int64_t m0 = (int64_t)blockIdx.y * kR;
  const int nb = u.n0 + blockIdx.x * 128;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  float* W = u.Wc + (size_t)b * u.d_out * u.d;

  // W elements of this thread, read now (indices clamped: the out-of-range
  // ones are never written back)
  float wpre[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = min(m0 + wm + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3), u.d_out - 1);
        const int col = min(nb + wn + jj * 32 + (lane & 31), u.n1 - 1);
        wpre[i][jj][q] = W[(size_t)row * u.d + col];
      }

  // operand buffers rebased at this workgroup's first row; rows past the end
  // of a tensor read as zeros, rows past the live range repeat the last one
  const int64_t er0 = m0;
  const int64_t ur0 = nb;
  const int64_t erows = min((int64_t)kR, u.d_out - er0);
  const int64_t urows = min((int64_t)128, (int64_t)u.n1 - ur0);
  const size_t eoff = ((size_t)b * u.d_out + er0) * u.err_ld;
  const size_t uoff = ((size_t)b * u.d + ur0) * u.d;
  const __amdgpu_buffer_rsrc_t rEH = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(u.ErrH + eoff), (short)0, (int)(erows * u.err_ld * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rEL = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(u.ErrL + eoff), (short)0, (int)(erows * u.err_ld * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rUH = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(u.UtH + uoff), (short)0, (int)(urows * u.d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rUL = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(u.UtL + uoff), (short)0, (int)(urows * u.d * 2), 0x00020000);

  // direct loads: chunk c of a stage = 16 rows of one array ([Eh | El | Uh | Ul]);
  // wave w issues chunks q kW + w, so the array of each of its loads is known
  // at compile time.  Lane -> row lane / 4, slot lane % 4 holding k-chunk
  // slot ^ ((row / 2) % 4).
  const int crow = lane >> 2;
  const int kc = (lane & 3) ^ ((crow >> 1) & 3);
  auto dma = [&](int st, char* buf) {
    const int k0 = st * kUK;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int c = q * kW + wave;
      const auto dst = (__attribute__((address_space(3))) void*)(buf + c * 1024);
      constexpr int kEC = kR / 16;                // chunks per Err array
      if (q * kW < 2 * kEC) {                     // Eh, El
        const bool lo = q * kW >= kEC;
        const int r = (c - (lo ? kEC : 0)) * 16 + crow;
        const uint32_t vo = (uint32_t)(((int64_t)min(r, (int)erows - 1) * u.err_ld + u.err_k0 + k0 + 8 * kc) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lo ? rEL : rEH, dst, 16, vo, 0, 0, 0);
      } else {                                    // Uh, Ul: 8 chunks each
        const bool lo = q * kW >= 2 * kEC + 8;
        const int r = (c - 2 * kEC - (lo ? 8 : 0)) * 16 + crow;
        const uint32_t vo = (uint32_t)(((int64_t)min(r, (int)urows - 1) * u.d + u.u0 + k0 + 8 * kc) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lo ? rUL : rUH, dst, 16, vo, 0, 0, 0);
      }
    }
  };

  // fragment reads: row r, k-chunk 2 ks + (lane / 32) at slot chunk ^ ((r / 2) % 4)
  const int ra = wm + (lane & 31), rb = wn + (lane & 31);
  int offA[2], offB[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    offA[ks] = ra * kURow + 16 * (c ^ ((ra >> 1) & 3));
    offB[ks] = 2 * kR * kURow + rb * kURow + 16 * (c ^ ((rb >> 1) & 3));
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][jj][q] = 0.f;

  auto compute = [&](const char* buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const u32x4*>(buf + offA[ks] + i * 32 * kURow);
        al[i] = *reinterpret_cast<const u32x4*>(buf + offA[ks] + kR * kURow + i * 32 * kURow);
        bh[i] = *reinterpret_cast<const u32x4*>(buf + offB[ks] + i * 32 * kURow);
        bl[i] = *reinterpret_cast<const u32x4*>(buf + offB[ks] + 128 * kURow + i * 32 * kURow);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah[i]),
                                                               __builtin_bit_cast(bf16x8, bh[jj]), acc[i][jj], 0, 0, 0);
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah[i]),
                                                               __builtin_bit_cast(bf16x8, bl[jj]), acc[i][jj], 0, 0, 0);
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al[i]),
                                                               __builtin_bit_cast(bf16x8, bh[jj]), acc[i][jj], 0, 0, 0);
        }
    }
  };

  // Per stage a wave issues kPerWave direct loads, two stages ahead.  At the
  // end of stage s the loads of stage s + 1 must have landed; those of s + 2
  // may still fly.  Stages past K are loaded too (from past the operands'
  // ends or their live ranges) and never multiplied, so every stage issues
  // the same loads.
  constexpr int kWait = (kPerWave & 0xF) | ((kPerWave >> 4) << 14) | (7 << 4) | (0xF << 8);
  const int nst = u.K / kUK;
  dma(0, ring0);
  dma(1, ring1);
  __builtin_amdgcn_s_waitcnt(kWait);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#define GQ_USTAGE(k, CUR, NXT)                                     \
  {                                                                \
    dma(st + (k) + 2, NXT);                                        \
    if (st + (k) < nst) compute(CUR);                              \
    __builtin_amdgcn_s_waitcnt(kWait);                             \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
  }
  for (int st = 0; st < nst; st += 3) {
    GQ_USTAGE(0, ring0, ring2);
    GQ_USTAGE(1, ring1, ring0);
    GQ_USTAGE(2, ring2, ring1);
  }
#undef GQ_USTAGE
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int col = nb + wn + jj * 32 + (lane & 31);
        if (row < u.d_out && col < u.n1) W[(size_t)row * u.d + col] = wpre[i][jj][q] - acc[i][jj][q];
      }
}

static int super_block(int d, int g) {
  int sb = 1024;
  if (g > kQBlock) sb = g * std::max(1, 1024 / g);
  return std::min(sb, d);
}

// ------------------------------------------------------------------ host
size_t quantize_workspace_bytes(const gptq_params* p, int64_t d_out, int64_t d_in, int64_t batch) {
  (void)p;
  size_t bytes = 0;
  bytes += align_up((size_t)batch * d_out * d_in * sizeof(float), 256);       // Wc
  bytes += 2 * align_up((size_t)batch * d_in * d_in * sizeof(uint16_t), 256); // UtH, UtL
  const int sb = super_block((int)d_in, p ? p->group_size : kQBlock);
  bytes += 2 * align_up((size_t)batch * d_out * sb * sizeof(uint16_t), 256);  // ErrH, ErrL
  return bytes + 256;
}

template <int kL, int G, bool kBig>
static void launch_bq(const QArgs& a, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)cdiv(a.d_out, rows_per_wg<kL>()), (unsigned)batch);
  hipLaunchKernelGGL((block_quant_kernel<kL, G, kBig>), grid, dim3(256), 0, st, a);
}

// Lanes per weight row of the block quantizer: 8 when the layer has few rows,
// so twice as many waves share the column chain (each with half the columns),
// 4 otherwise (the quantization arithmetic of a column runs on every lane of
// its row, so more lanes per row cost instructions once the GPU is full).
// Static groups always take 8: their lanes also hold every column's packed
// scale and zero, which at 4 lanes (32 columns each) leaves one wave per SIMD.
static int bq_lanes(int64_t d_out, int64_t batch, bool stat) { return stat || d_out * batch <= 8192 ? 8 : 4; }

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                                           int64_t batch, const float* U, const int32_t* perm, const gptq_params* p,
                                           uint8_t* codes, uint16_t* scales, uint8_t* zeros, int32_t* g_idx,
                                           float* Q_opt, void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(W && U && p && codes && scales && zeros && g_idx);
  GQ_CHECK_ARG(w_dtype == GPTQ_F32 || w_dtype == GPTQ_F16 || w_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(d_out >= 1 && d_out <= (int64_t)1 << 24 && batch >= 1 && batch <= 65535);
  GQ_CHECK_ARG(d_in >= kQBlock && d_in % kQBlock == 0 && d_in <= 65536);
  GQ_CHECK_ARG(ld_w >= d_in);
  GQ_CHECK_ARG(reinterpret_cast<uintptr_t>(codes) % 16 == 0);
  if (!gq_params_ok(p, d_in)) return GPTQ_EINVAL;
  GQ_CHECK_ARG(!p->act_order || perm != nullptr);   // U of an act-order layer is in permuted order
  const int g = p->group_size;
  if (g < kQBlock && g != 16 && g != 32 && g != 64) return GPTQ_EUNSUPPORTED;
  if (ws_bytes < quantize_workspace_bytes(p, d_out, d_in, batch) || workspace == nullptr) return GPTQ_ENOMEM;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = (int)d_in;
  const bool stat = p->static_groups != 0;
  Carver cv(workspace);
  float* Wc = cv.take<float>((size_t)batch * d_out * d);
  uint16_t* UtH = cv.take<uint16_t>((size_t)batch * d * d);
  uint16_t* UtL = cv.take<uint16_t>((size_t)batch * d * d);
  const int sb = super_block(d, g);
  uint16_t* ErrH = cv.take<uint16_t>((size_t)batch * d_out * sb);
  uint16_t* ErrL = cv.take<uint16_t>((size_t)batch * d_out * sb);

  {
    TimedScope ts(kTimePrep, st);
    dim3 grid((unsigned)d_out, (unsigned)std::min<int64_t>(cdiv(d, 256), 16), (unsigned)batch);
    if (w_dtype == GPTQ_F32) hipLaunchKernelGGL(prep_w_kernel<0>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
    else if (w_dtype == GPTQ_F16) hipLaunchKernelGGL(prep_w_kernel<1>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
    else hipLaunchKernelGGL(prep_w_kernel<2>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
    GQ_LAUNCHED();
    dim3 ug((unsigned)cdiv(d, 32), (unsigned)cdiv(d, 32), (unsigned)batch);
    hipLaunchKernelGGL(prep_u_kernel, ug, dim3(256), 0, st, U, d, bq_lanes(d_out, batch, stat), UtH, UtL);
    GQ_LAUNCHED();
    hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)cdiv((int64_t)d * batch, 256)), dim3(256), 0, st,
                       stat ? nullptr : perm, d, g, (int)batch, g_idx);
    GQ_LAUNCHED();
    if (stat) {
      const int64_t units = batch * d_out * (d / g);
      const unsigned nb = (unsigned)std::min<int64_t>(cdiv(units, 4), 16384);
      const float maxq = (float)((1 << p->bits) - 1);
      if (w_dtype == GPTQ_F32)
        hipLaunchKernelGGL(static_params_kernel<0>, dim3(nb), dim3(256), 0, st, W, ld_w, g, d / g, units, maxq, p->sym,
                           scales, zeros);
      else if (w_dtype == GPTQ_F16)
        hipLaunchKernelGGL(static_params_kernel<1>, dim3(nb), dim3(256), 0, st, W, ld_w, g, d / g, units, maxq, p->sym,
                           scales, zeros);
      else
        hipLaunchKernelGGL(static_params_kernel<2>, dim3(nb), dim3(256), 0, st, W, ld_w, g, d / g, units, maxq, p->sym,
                           scales, zeros);
      GQ_LAUNCHED();
    }
  }

  QArgs a;
  a.U = U;
  a.perm = perm;
  a.Wc = Wc;
  a.ErrH = ErrH;
  a.ErrL = ErrL;
  a.codes = codes;
  a.scales = scales;
  a.zeros = zeros;
  a.Q = Q_opt;
  a.d_out = d_out;
  a.d = d;
  a.ng = d / g;
  a.g = g;
  a.maxq = (float)((1 << p->bits) - 1);
  a.sym = p->sym;
  a.gidx = g_idx;
  const int nblk = d / kQBlock;
  const int tiles_per_sb = sb / kQBlock;
  a.err_ld = sb;
  const int kl = bq_lanes(d_out, batch, stat);
  UpdArgs ua;
  ua.Wc = Wc;
  ua.ErrH = ErrH;
  ua.ErrL = ErrL;
  ua.UtH = UtH;
  ua.UtL = UtL;
  ua.d_out = d_out;
  ua.d = d;
  ua.err_ld = sb;
  auto update = [&](int err_k0, int u0, int K, int n0, int n1) -> gptq_status {
    if (n0 >= n1) return GPTQ_OK;
    ua.err_k0 = err_k0;
    ua.u0 = u0;
    ua.K = K;
    ua.n0 = n0;
    ua.n1 = n1;
    TimedScope ts(kTimeTrailing, st);
    // 256-row tiles while they still give every CU one, else 128-row tiles
    const int64_t nt = cdiv(n1 - n0, 128);
    if (nt * cdiv(d_out, 256) * batch >= 256) {
      dim3 grid((unsigned)nt, (unsigned)cdiv(d_out, 256), (unsigned)batch);
      hipLaunchKernelGGL(update_kernel<256>, grid, dim3(512), 0, st, ua);
    } else {
      dim3 grid((unsigned)nt, (unsigned)cdiv(d_out, 128), (unsigned)batch);
      hipLaunchKernelGGL(update_kernel<128>, grid, dim3(256), 0, st, ua);
    }
    GQ_LAUNCHED();
    return GPTQ_OK;
  };
  for (int t = 0; t < nblk; ++t) {
    const int tt = t % tiles_per_sb;
    const int sb0 = (t / tiles_per_sb) * sb;
    const int sb_end = std::min(sb0 + sb, d);
    a.b0 = t * kQBlock;
    a.err_off = tt * kQBlock;
    {
      TimedScope ts(kTimeBlockQuant, st);
      if (stat) launch_bq<8, 0, false>(a, batch, st);
      else switch (g) {
        case 16: kl == 8 ? launch_bq<8, 16, false>(a, batch, st) : launch_bq<4, 16, false>(a, batch, st); break;
        case 32: kl == 8 ? launch_bq<8, 32, false>(a, batch, st) : launch_bq<4, 32, false>(a, batch, st); break;
        case 64: kl == 8 ? launch_bq<8, 64, false>(a, batch, st) : launch_bq<4, 64, false>(a, batch, st); break;
        case 128: kl == 8 ? launch_bq<8, 128, false>(a, batch, st) : launch_bq<4, 128, false>(a, batch, st); break;
        default: kl == 8 ? launch_bq<8, 128, true>(a, batch, st) : launch_bq<4, 128, true>(a, batch, st); break;
      }
      GQ_LAUNCHED();
    }
    const int b1 = a.b0 + kQBlock;
    gptq_status s1 = update(tt * kQBlock, a.b0, kQBlock, b1, sb_end);    // rest of the super-block
    if (s1 != GPTQ_OK) return s1;
    if (b1 == sb_end) {
      s1 = update(0, sb0, sb_end - sb0, sb_end, d);                      // every later column
      if (s1 != GPTQ_OK) return s1;
    }
  }
  return GPTQ_OK;
}
