// Column-by-column group quantization with error feedback, in 128-column tiles.
//
// The loop is the one of "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍" section 三 and
// of the ipipp.com quantize_gptq listing: quantize column k, divide its error by
// the diagonal of the inverse-Hessian factor, subtract error x factor row from
// every later column.  Columns are processed in 128-wide tiles (the same page's
// "按块处理", process in blocks): inside a tile the updates are applied at once
// by `block_quant_kernel`; the later columns receive the tiles' updates through
// GEMMs, W[:, right] -= Err[:, left] U[left, right] (`update_kernel`), on a
// recursive halving of the tile range: quantize the left half, update the
// right half once with all of the left half's errors, quantize the right half.
//
// block_quant (block_quant.h): kL lanes share a weight row, the tile's columns
// in registers, errors broadcast with DPP moves.  The error kept per column is
// d = w - dq; the rows of U carry the division by their diagonal entry.
//
// trailing: a bf16 MFMA GEMM with three products (hi*hi + hi*lo + lo*hi) of a
// two-term bf16 split of Err and of the scaled U, so the update keeps about 16 significant
// bits while the working copy stays fp32.
#include <cmath>
#include <utility>

#include "block_quant.h"

bool gq_params_ok(const gptq_params* p, int64_t d_in);

namespace gq {

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

// Wc[b][r][k] = W[b][r][perm[k]] as fp32, one row per workgroup.  The row is
// read with 16-byte loads (8 or 4 elements a lane); without a permutation the
// values go straight out as 16-byte stores, with one the row is staged in LDS
// (kMaxD elements) and gathered from there, so global memory sees only
// contiguous accesses.  Rows must start 16-byte aligned (checked by the host).
template <int kDt, int kMaxD>
__global__ __launch_bounds__(256) void prep_w_vec_kernel(const void* __restrict__ W, int64_t ld_w, int64_t d_out, int d,
                                                         const int32_t* __restrict__ perm, float* __restrict__ Wc) {
  constexpr int kE = kDt == 0 ? 4 : 8;   // elements per 16-byte load
  const int b = blockIdx.z;
  const int64_t r = blockIdx.x;
  const int32_t* pb = perm ? perm + (size_t)b * d : nullptr;
  const size_t src_row = ((size_t)b * d_out + r) * ld_w;
  float* dst = Wc + ((size_t)b * d_out + r) * d;
  __shared__ __attribute__((aligned(16))) float row[kMaxD > 0 ? kMaxD : 1];
  for (int k0 = threadIdx.x * kE; k0 < d; k0 += 256 * kE) {
    float v[kE];
    if constexpr (kDt == 0) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + src_row + k0);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + src_row + k0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t h = (uint16_t)(q[e >> 1] >> (16 * (e & 1)));
        v[e] = kDt == 1 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
      }
    }
    if constexpr (kMaxD > 0) {
#pragma unroll
      for (int e = 0; e < kE; e += 4) *reinterpret_cast<f32x4*>(&row[k0 + e]) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < kE; e += 4) *reinterpret_cast<f32x4*>(dst + k0 + e) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    }
  }
  if constexpr (kMaxD > 0) {
    __syncthreads();
    for (int k0 = threadIdx.x * 4; k0 < d; k0 += 256 * 4)
      *reinterpret_cast<f32x4*>(dst + k0) = f32x4{row[pb[k0]], row[pb[k0 + 1]], row[pb[k0 + 2]], row[pb[k0 + 3]]};
  }
}

// Wc[b][r][k] = W[b][r][perm[k]] as fp32 (any row alignment).
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

// UtH/UtL[b][n][t0 + lane_major(k - t0)] = split(U[b][k][n] / U[b][k][k]) for
// k in tiles strictly before n's tile (the only entries the deferred update
// reads; Err holds w - dq, so row k carries the division by U[k][k]); kl is
// the block quantizer's lanes per row, which fixes the Err column order.
__global__ __launch_bounds__(256) void prep_u_kernel(const float* __restrict__ U, int d, int kl,
                                                     uint16_t* __restrict__ UtH, uint16_t* __restrict__ UtL) {
  const int b = blockIdx.z;
  const float* Ub = U + (size_t)b * d * d;
  __shared__ float t[32][33];
  __shared__ float dg[32];
  const int k0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  if ((k0 / kQBlock) >= ((n0 + 31) / kQBlock)) return;   // no entry of this tile is read
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (threadIdx.x < 32) dg[threadIdx.x] = (k0 + threadIdx.x < d) ? Ub[(size_t)(k0 + threadIdx.x) * (d + 1)] : 1.f;
  for (int rr = ty; rr < 32; rr += 8) {
    int k = k0 + rr, n = n0 + tx;
    t[rr][tx] = (k < d && n < d) ? Ub[(size_t)k * d + n] : 0.f;
  }
  __syncthreads();
  for (int rr = ty; rr < 32; rr += 8) {
    int n = n0 + rr, k = k0 + tx;
    if (n < d && k < d && (k / kQBlock) < (n / kQBlock)) {
      float v = t[tx][rr] / dg[tx];
      uint32_t h = f32_to_bf16_bits(v);
      uint32_t l = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
      size_t o = (size_t)b * d * d + (size_t)n * d + (k / kQBlock) * kQBlock + lane_major(k % kQBlock, kl);
      UtH[o] = (uint16_t)h;
      UtL[o] = (uint16_t)l;
    }
  }
}

// Ud[b][t][ud_slot(k, c, kl)] = U[b][t0 + k][t0 + c] / U[b][t0 + k][t0 + k] for
// c > k, else 0 (t0 = 128 t): every tile's in-tile feedback rows in the order
// the block quantizer reads them from LDS.
__global__ __launch_bounds__(256) void prep_ud_kernel(const float* __restrict__ U, int d, int kl,
                                                      float* __restrict__ Ud) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int t0 = t * kQBlock;
  const float* Ub = U + (size_t)b * d * d;
  float* out = Ud + ((size_t)b * (d / kQBlock) + t) * (kQBlock * kQBlock);
  __shared__ float dg[kQBlock];
  if (threadIdx.x < kQBlock) dg[threadIdx.x] = Ub[(size_t)(t0 + threadIdx.x) * (d + 1)];
  __syncthreads();
  for (int e = threadIdx.x; e < kQBlock * kQBlock; e += 256) {
    const int k = e >> 7, c = e & 127;
    const float v = c > k ? Ub[(size_t)(t0 + k) * d + t0 + c] / dg[k] : 0.0f;
    out[ud_slot(k, c, kl)] = v;
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
  int64_t d_out;        // rows of every batch entry (the stride between entries)
  int64_t r0, r1;       // rows [r0, r1) of every entry are updated by this launch
  int d;
  int err_ld, err_k0;   // Err columns [err_k0, err_k0 + K) of rows of length err_ld
  int u0;               // matching k range in Ut rows
  int K;
  int n0, n1;
  int band;             // row blocks per band of the tile order, 0: column tiles fastest
};

// W[rows, n0:n1] -= Err[rows, K] Ut[n0:n1, K]^T on MFMA.  A workgroup owns kR
// rows x kC columns of W; its waves own 64 x (kC / 2) blocks.  Both operands
// are K-contiguous rows (Err rows, rows of the transposed U), so they stream
// global -> LDS unchanged (buffer loads straight into LDS, 16 bytes per lane)
// through a ring of 32-k stages, and every MFMA fragment is one 16-byte LDS
// read.  An LDS row is 64 bytes (32 bf16 of k); its 16-byte k-chunk c sits at
// slot c ^ ((row / 4) % 4), so the 32 rows a half-wave reads spread evenly
// over the 64 banks (two accesses per bank, the minimum; with (row / 2) % 4
// they used 32 banks).
//
// kC = 128: a ring of three stages (loads two stages ahead), and the
// workgroup's W elements are read at the start, so that latency hides behind
// the K loop.  kC = 256: each Err fragment feeds twice as many MFMAs, so a
// flop moves a third fewer bytes from L2 into LDS and out of LDS into
// registers; its 64 KB stages allow a ring of two (loads one stage ahead,
// which is as many cycles ahead as two of the smaller stages), and the
// accumulators leave no registers to hold W, which is read at the end.
constexpr int kUK = 32;          // k per LDS stage
constexpr int kURow = kUK * 2;   // bytes per LDS row

template <int kR, int kC>
constexpr int upd_stage_bytes() { return 2 * kR * kURow + 2 * kC * kURow; }

template <int kR, int kC = 128>
__global__ __launch_bounds__(2 * kR) void update_kernel(UpdArgs u) {
  static_assert(kC == 128 || kC == 256, "128 or 256 columns per workgroup");
  constexpr int kW = kR / 32;                        // waves
  constexpr int kJ = kC / 64;                        // 32-column blocks per wave
  constexpr bool kPre = kC == 128;                   // W read at the start
  constexpr int kRing = kC == 128 ? 3 : 2;
  constexpr int kStageB = upd_stage_bytes<kR, kC>();
  constexpr int kChunks = kStageB / 1024;            // 1 KiB direct-load chunks per stage
  constexpr int kPerWave = kChunks / kW;
  static_assert(kRing * kStageB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char ring0[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring1[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring2[kRing == 3 ? kStageB : 1024];
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: picks operand buffers
  // Workgroups are dispatched in blockIdx order, round-robin over the 8 XCDs.
  // With u.band > 0 each XCD takes a contiguous run of tile ids, and tile ids
  // walk bands of u.band row blocks column by column, so the workgroups one
  // XCD runs at a time form a compact block of row blocks x column tiles that
  // share their Err rows and U^T rows in that XCD's L2.  With u.band == 0 the
  // XCDs take interleaved column tiles of the same row blocks, so the Err rows
  // (the larger operand) are shared across XCDs through the memory-side
  // cache; that order moves fewer bytes once a tile's K range no longer fits
  // the L2 of an XCD.
  int rblk = blockIdx.y, ct = blockIdx.x;
  if (u.band > 0) {
    const int nt = gridDim.x, nrb = gridDim.y;
    const int nwg = nt * nrb;
    const int bid = blockIdx.x + nt * blockIdx.y;
    const int per = nwg / 8, extra = nwg % 8, x = bid % 8, i = bid / 8;
    const int g = x * per + min(x, extra) + i;   // this XCD's i-th tile id
    const int band = g / (u.band * nt);
    const int base = band * u.band;
    const int rows_b = min(u.band, nrb - base);
    const int j = g - band * u.band * nt;
    ct = j / rows_b;
    rblk = base + j % rows_b;
  }
  const int64_t m0 = u.r0 + (int64_t)rblk * kR;
  const int nb = u.n0 + ct * kC;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * (kC / 2);
  float* W = u.Wc + (size_t)b * u.d_out * u.d;

  // W elements of this thread, read now (indices clamped: the out-of-range
  // ones are never written back)
  float wpre[2][kPre ? kJ : 1][16];
  if constexpr (kPre) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t row = min(m0 + wm + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3), u.r1 - 1);
          const int col = min(nb + wn + jj * 32 + (lane & 31), u.n1 - 1);
          wpre[i][jj][q] = W[(size_t)row * u.d + col];
        }
  }

  // operand buffers rebased at this workgroup's first row; rows past the end
  // of a tensor read as zeros, rows past the live range repeat the last one
  const int64_t er0 = m0;
  const int64_t ur0 = nb;
  const int64_t erows = min((int64_t)kR, u.r1 - er0);
  const int64_t urows = min((int64_t)kC, (int64_t)u.n1 - ur0);
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
  // at compile time (every array is a multiple of kW chunks).  Lane -> row
  // lane / 4, slot lane % 4 holding k-chunk slot ^ ((row / 4) % 4).
  const int crow = lane >> 2;
  const int kc = (lane & 3) ^ ((crow >> 2) & 3);
  auto dma = [&](int st, char* buf) {
    const int k0 = st * kUK;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int c = q * kW + wave;
      const auto dst = (__attribute__((address_space(3))) void*)(buf + c * 1024);
      constexpr int kEC = kR / 16;                // chunks per Err array
      constexpr int kUC = kC / 16;                // chunks per U array
      static_assert(kEC % kW == 0 && kUC % kW == 0, "chunk split");
      if (q * kW < 2 * kEC) {                     // Eh, El
        const bool lo = q * kW >= kEC;
        const int r = (c - (lo ? kEC : 0)) * 16 + crow;
        const uint32_t vo = (uint32_t)(((int64_t)min(r, (int)erows - 1) * u.err_ld + u.err_k0 + k0 + 8 * kc) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lo ? rEL : rEH, dst, 16, vo, 0, 0, 0);
      } else {                                    // Uh, Ul
        const bool lo = q * kW >= 2 * kEC + kUC;
        const int r = (c - 2 * kEC - (lo ? kUC : 0)) * 16 + crow;
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
    offA[ks] = ra * kURow + 16 * (c ^ ((ra >> 2) & 3));
    offB[ks] = 2 * kR * kURow + rb * kURow + 16 * (c ^ ((rb >> 2) & 3));
  }

  f32x16 acc[2][kJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][jj][q] = 0.f;

  auto compute = [&](const char* buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 ah[2], al[2], bh[kJ], bl[kJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const u32x4*>(buf + offA[ks] + i * 32 * kURow);
        al[i] = *reinterpret_cast<const u32x4*>(buf + offA[ks] + kR * kURow + i * 32 * kURow);
      }
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        bh[jj] = *reinterpret_cast<const u32x4*>(buf + offB[ks] + jj * 32 * kURow);
        bl[jj] = *reinterpret_cast<const u32x4*>(buf + offB[ks] + kC * kURow + jj * 32 * kURow);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) {
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
  // (a ring of two: the loads of stage s + 1 land by the end of stage s)
  constexpr int kAhead = kRing - 1;
  constexpr int kInFlight = kPerWave * (kAhead - 1);
  constexpr int kWait = (kInFlight & 0xF) | ((kInFlight >> 4) << 14) | (7 << 4) | (0xF << 8);
  const int nst = u.K / kUK;
  dma(0, ring0);
  if constexpr (kRing == 3) dma(1, ring1);
  __builtin_amdgcn_s_waitcnt(kWait);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#define GQ_USTAGE(k, CUR, NXT)                                     \
  {                                                                \
    dma(st + (k) + kAhead, NXT);                                   \
    if (st + (k) < nst) compute(CUR);                              \
    __builtin_amdgcn_s_waitcnt(kWait);                             \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
  }
  if constexpr (kRing == 3) {
    for (int st = 0; st < nst; st += 3) {
      GQ_USTAGE(0, ring0, ring2);
      GQ_USTAGE(1, ring1, ring0);
      GQ_USTAGE(2, ring2, ring1);
    }
  } else {
    for (int st = 0; st < nst; st += 2) {
      GQ_USTAGE(0, ring0, ring1);
      GQ_USTAGE(1, ring1, ring0);
    }
  }
#undef GQ_USTAGE
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // without the early read: the row block's W elements in one batch of
    // loads (indices clamped, as above), then the stores
    float wend[kPre ? 1 : kJ][16];
    if constexpr (!kPre) {
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t row = min(m0 + wm + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3), u.r1 - 1);
          const int col = min(nb + wn + jj * 32 + (lane & 31), u.n1 - 1);
          wend[jj][q] = W[(size_t)row * u.d + col];
        }
    }
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int col = nb + wn + jj * 32 + (lane & 31);
        const float wv = kPre ? wpre[i][kPre ? jj : 0][q] : wend[kPre ? 0 : jj][q];
        if (row < u.r1 && col < u.n1) W[(size_t)row * u.d + col] = wv - acc[i][jj][q];
      }
  }
}

// ------------------------------------------------------------------ host
size_t quantize_workspace_bytes(const gptq_params* p, int64_t d_out, int64_t d_in, int64_t batch) {
  (void)p;
  size_t bytes = 0;
  bytes += align_up((size_t)batch * d_out * d_in * sizeof(float), 256);       // Wc
  bytes += 2 * align_up((size_t)batch * d_in * d_in * sizeof(uint16_t), 256); // UtH, UtL
  bytes += 2 * align_up((size_t)batch * d_out * d_in * sizeof(uint16_t), 256); // ErrH, ErrL
  bytes += align_up((size_t)batch * d_in * kQBlock * sizeof(float), 256);      // Ud
  return bytes + 256;
}

// Block quantizer shape: lanes per weight row and threads per workgroup.
// 8 lanes per row always.  Layers with few rows: 32 rows per workgroup, so
// more workgroups share the column chain.  Taller layers: 64 rows per
// workgroup of 512 threads; with the tile's 64 KB of U in LDS and about 100
// registers per lane, two workgroups fit a CU, four waves per SIMD.  (Measured slower: 4
// lanes per row, whose registers allow two waves per SIMD; 2 lanes per row at
// one wave per SIMD, whose column chain is then exposed; and one lane per
// row, whose fully unrolled column loop is four times the code and took 60
// instead of 43 us per tile on the 70B layer.)  Static groups hold every
// column's packed scale and zero as well, so they stay at 256 threads.
struct BqShape {
  int kl, kt;
};
static BqShape bq_shape(int64_t d_out, int64_t batch, bool stat) {
  if (stat || d_out * batch <= 8192) return {8, 256};
  return {8, 512};
}

// The column loop of rows [r0, r1) of every batch entry on stream st: block
// quantization of each tile and the deferred updates, on a recursive halving
// of the tile range: quantize the left half, bring the right half up to date
// with one GEMM of the left half's errors, quantize the right half.  Every
// column then receives each earlier tile's update exactly once, and W
// crosses HBM about log2(tiles) times instead of once per tile.  When a range
// [lo, hi) starts, its columns hold every update of the tiles before lo.  A
// dynamic group wider than a tile opens at its first tile and reads the
// values of its later tiles there, so a range longer than one group is split
// at a group boundary; inside one group any split is fine (the later tiles
// use the stored scale and zero).
constexpr int kUpd256MinK = 1024;

static gptq_status run_slab(QArgs a, UpdArgs ua, int64_t r0, int64_t r1, int64_t batch, int g, bool stat,
                            BqShape shape, hipStream_t st) {
  a.r0 = ua.r0 = r0;
  a.r1 = ua.r1 = r1;
  const int64_t rows = r1 - r0;
  shape = bq_shape(rows, batch, stat);   // workgroup height for this slab's rows
  const int nblk = a.d / kQBlock;
  // W[:, tiles [m, b)] -= Err[:, tiles [a0, m)] U[tiles [a0, m), tiles [m, b)]
  auto update = [&](int a0, int m, int b) -> gptq_status {
    ua.err_k0 = a0 * kQBlock;
    ua.u0 = a0 * kQBlock;
    ua.K = (m - a0) * kQBlock;
    ua.n0 = m * kQBlock;
    ua.n1 = b * kQBlock;
    // measured on the 70B layer: bands of 2 row blocks while K <= 2048,
    // column tiles fastest beyond
    ua.band = ua.K <= 2048 ? 2 : 0;
    TimedScope ts(kTimeTrailing, st);
    // 256 x 256 tiles for long K while they still give every CU one, then
    // 256 x 128, else 128 x 128
    const int64_t nt2 = cdiv(ua.n1 - ua.n0, 256);
    const int64_t nt = cdiv(ua.n1 - ua.n0, 128);
    if (ua.K >= kUpd256MinK && nt2 * cdiv(rows, 256) * batch >= 256) {
      dim3 grid((unsigned)nt2, (unsigned)cdiv(rows, 256), (unsigned)batch);
      hipLaunchKernelGGL((update_kernel<256, 256>), grid, dim3(512), 0, st, ua);
    } else if (nt * cdiv(rows, 256) * batch >= 256) {
      dim3 grid((unsigned)nt, (unsigned)cdiv(rows, 256), (unsigned)batch);
      hipLaunchKernelGGL(update_kernel<256>, grid, dim3(512), 0, st, ua);
    } else {
      dim3 grid((unsigned)nt, (unsigned)cdiv(rows, 128), (unsigned)batch);
      hipLaunchKernelGGL(update_kernel<128>, grid, dim3(256), 0, st, ua);
    }
    GQ_LAUNCHED();
    return GPTQ_OK;
  };
  auto block_quant = [&](int t) -> gptq_status {
    a.b0 = t * kQBlock;
    a.err_off = t * kQBlock;
    TimedScope ts(kTimeBlockQuant, st);
    if (stat) launch_bq_static(a, batch, st);
    else if (shape.kt == 256) launch_bq_8x256(a, g, batch, st);
    else launch_bq_8x512(a, g, batch, st);
    GQ_LAUNCHED();
    return GPTQ_OK;
  };
  const int gt = (!stat && g > kQBlock) ? g / kQBlock : 1;   // tiles per group
  gptq_status rs = GPTQ_OK;
  // explicit stack of (lo, mid, hi): mid < 0 quantizes tiles [lo, hi), mid >= 0
  // is the update of tiles [mid, hi) by tiles [lo, mid)
  struct Item {
    int lo, mid, hi;
  };
  std::vector<Item> stack{{0, -1, nblk}};
  while (!stack.empty() && rs == GPTQ_OK) {
    const Item it = stack.back();
    stack.pop_back();
    if (it.mid >= 0) {
      rs = update(it.lo, it.mid, it.hi);
      continue;
    }
    const int n = it.hi - it.lo;
    if (n == 1) {
      rs = block_quant(it.lo);
      continue;
    }
    int mid;
    if (n > gt) mid = it.lo + gt * std::max(1, (n / gt) / 2);
    else mid = it.lo + n / 2;
    stack.push_back({mid, -1, it.hi});       // right half last
    stack.push_back({it.lo, mid, it.hi});    // the update between them
    stack.push_back({it.lo, -1, mid});       // left half first
  }
  return rs;
}

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
  uint16_t* ErrH = cv.take<uint16_t>((size_t)batch * d_out * d);
  uint16_t* ErrL = cv.take<uint16_t>((size_t)batch * d_out * d);
  float* Ud = cv.take<float>((size_t)batch * d * kQBlock);
  const BqShape shape = bq_shape(d_out, batch, stat);

  {
    TimedScope ts(kTimePrep, st);
    // rows 16-byte aligned (d is a multiple of 128, so whole 16-byte pieces):
    // the vector kernel, with the row staged in LDS when permuted and it fits
    const int64_t es = w_dtype == GPTQ_F32 ? 4 : 2;
    const bool vec = reinterpret_cast<uintptr_t>(W) % 16 == 0 && (ld_w * es) % 16 == 0;
    const bool lds_ok = perm == nullptr || d <= 16384;
    if (vec && lds_ok) {
      const dim3 grid((unsigned)d_out, 1, (unsigned)batch);
#define GQ_PREPW(DT)                                                                                                  \
  do {                                                                                                                \
    if (perm == nullptr) hipLaunchKernelGGL((prep_w_vec_kernel<DT, 0>), grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc); \
    else if (d <= 4096) hipLaunchKernelGGL((prep_w_vec_kernel<DT, 4096>), grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc); \
    else if (d <= 8192) hipLaunchKernelGGL((prep_w_vec_kernel<DT, 8192>), grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc); \
    else hipLaunchKernelGGL((prep_w_vec_kernel<DT, 16384>), grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc); \
  } while (0)
      if (w_dtype == GPTQ_F32) GQ_PREPW(0);
      else if (w_dtype == GPTQ_F16) GQ_PREPW(1);
      else GQ_PREPW(2);
#undef GQ_PREPW
    } else {
      dim3 grid((unsigned)d_out, (unsigned)std::min<int64_t>(cdiv(d, 256), 16), (unsigned)batch);
      if (w_dtype == GPTQ_F32) hipLaunchKernelGGL(prep_w_kernel<0>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
      else if (w_dtype == GPTQ_F16) hipLaunchKernelGGL(prep_w_kernel<1>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
      else hipLaunchKernelGGL(prep_w_kernel<2>, grid, dim3(256), 0, st, W, ld_w, d_out, d, perm, Wc);
    }
    GQ_LAUNCHED();
    dim3 ug((unsigned)cdiv(d, 32), (unsigned)cdiv(d, 32), (unsigned)batch);
    hipLaunchKernelGGL(prep_u_kernel, ug, dim3(256), 0, st, U, d, shape.kl, UtH, UtL);
    GQ_LAUNCHED();
    hipLaunchKernelGGL(prep_ud_kernel, dim3((unsigned)(d / kQBlock), (unsigned)batch), dim3(256), 0, st, U, d,
                       shape.kl, Ud);
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
  a.Ud = Ud;
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
  a.err_ld = d;
  UpdArgs ua;
  ua.Wc = Wc;
  ua.ErrH = ErrH;
  ua.ErrL = ErrL;
  ua.UtH = UtH;
  ua.UtL = UtL;
  ua.d_out = d_out;
  ua.d = d;
  ua.err_ld = d;
  ua.band = 0;

  return run_slab(a, ua, 0, d_out, batch, g, stat, shape, st);
}
