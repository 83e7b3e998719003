// Hessian accumulation S += X^T X (lower triangle) and D += diag(X^T X) in fp64.
//
// The product is the dense contraction of the method ("3. 模型量化技术(下)",
// pseudocode block: H from the layer's inputs; ipipp.com quantize_gptq listing:
// H = 2 (X^T X) / N).  X is token-major, so both MFMA operands are columns of X;
// the transpose happens in the LDS read (see the tiling notes below).
#include "common.h"

namespace gq {

// ------------------------------------------------------------------ tiling
// One workgroup (8 waves) owns a 256 x 256 tile of S and a range of tokens.
// Tokens stream from global memory straight into LDS (global_load_lds, 16
// bytes per lane, no registers) through a ring of four 32-token stages, so
// three stages are in flight while one is multiplied.  A stage is multiplied in
// two 16-token halves: the second half's fragments are read while the first
// half's products run, and after the stage barrier the next stage's first
// half is read while this stage's second half multiplies, so the MFMAs do not
// wait for a whole stage of LDS reads.  An LDS stage holds token
// rows (512 bytes = 256 channels per panel) exactly as X stores them; the MFMA
// operand fragments (8 consecutive tokens of one channel) come out of the
// gfx950 transposing LDS read ds_read_b64_tr_b16, which gives each lane 4
// consecutive tokens of one channel.  The 16-byte octets of token t sit at slot
// octet ^ 4 (t & 3): the four token rows read by one 16-lane group then put
// the four octets they want in four different quarters of the 256-byte bank
// window, so a fragment read touches all 64 LDS banks once per half-wave
// (with octet ^ 2 (t & 3) it touched 32 of them twice).
constexpr int kTile = 256;               // output tile edge (channels)
constexpr int kStage = 32;               // tokens per LDS stage
// 8 waves per workgroup, each a 128 x 64 block of the tile, two waves per
// SIMD.  (4 waves of 128 x 128 each, one per SIMD with the accumulators in
// AGPRs, read a third less LDS per product but measured 10% slower.)
constexpr int kSyrkWaves = 8;
constexpr int kSyrkThreads = 64 * kSyrkWaves;
constexpr int kSyrkCpw = 16 / kSyrkWaves;   // 1 KiB chunks of each panel a wave loads per stage
constexpr int kSyrkBJ = 16 / kSyrkWaves;    // 32-column blocks of B per wave
constexpr int kRowB = 512;               // LDS bytes per token row of a panel
constexpr int kPanelB = kStage * kRowB;  // 16 KiB
constexpr int kStageB = 2 * kPanelB;     // panel I | panel J

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

struct SyrkArgs {
  const uint16_t* X;        // bf16 / fp16 bit patterns
  int64_t ld_x;             // elements
  const int32_t* row_idx;   // gather list (already offset to this entry) or null
  int64_t n_rows;           // rows of this entry
  int64_t x_rows;           // rows of X (gathered indices outside are skipped)
  const uint16_t* zero_row; // d_in zeros: the source of every row that does not exist
  int d;
  int nt;                   // tiles per dimension
  int tiles;                // nt (nt + 1) / 2
  int full;                 // tiles 0 .. full-1: one workgroup each over every token, written to S
  int splits;               // tiles full .. tiles-1: split over tokens into this many parts
  int stages_per_split;     // kStage-token stages per part
  float* S;                 // this entry's S
  float* partial;           // splits > 1: [tiles - full][splits][kTile * kTile]
};

// Lower-triangle tile t in row-major order.
__device__ __forceinline__ void tile_coords(int t, int& bi, int& bj) {
  int b = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((b + 1) * (b + 2) / 2 <= t) ++b;
  while (b * (b + 1) / 2 > t) --b;
  bi = b;
  bj = t - b * (b + 1) / 2;
}

// Lower-triangle tile t of an nt x nt grid in band order: bands of 8 tile
// rows, each walked column by column (the band's rows top to bottom), so 32
// consecutive tiles are 4 columns of 8 rows and read 12 distinct X panels
// (row-major runs of 32 read up to 23).  Bands before R are full and hold
// 32 R^2 + 4 R tiles; only the last band may have fewer than 8 rows.
__device__ __forceinline__ void tile_coords_band(int t, int nt, int& bi, int& bj) {
  int R = (int)((sqrtf(16.0f + 128.0f * (float)t) - 4.0f) * (1.0f / 64.0f));
  while (32 * (R + 1) * (R + 1) + 4 * (R + 1) <= t) ++R;
  while (R > 0 && 32 * R * R + 4 * R > t) --R;
  int tp = t - (32 * R * R + 4 * R);
  const int r0 = 8 * R;
  const int rows = min(8, nt - r0);
  if (tp < rows * r0) {   // the band's columns left of its diagonal block
    bj = tp / rows;
    bi = r0 + tp - bj * rows;
    return;
  }
  tp -= rows * r0;        // its diagonal block, column by column
  int c = 0;
  while (tp >= rows - c) {
    tp -= rows - c;
    ++c;
  }
  bj = r0 + c;
  bi = r0 + c + tp;
}

template <bool kF16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (kF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Work id -> (tile, part).  Consecutive ids are dispatched round-robin over
// the 8 XCDs; the remap gives each XCD a contiguous run of work ids, so tiles
// that share X panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int nx = 8;
  int per = nwg / nx;
  int full = per * nx;
  if (bid >= full) return bid;
  return (bid % nx) * per + bid / nx;
}

// 8 consecutive tokens of one channel as an MFMA operand: two transposing reads
// of 4 token rows each.
__device__ __forceinline__ u32x4 tr_frag(const lds_char* p) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3)))*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3)))*)(p + 4 * kRowB));
  u32x4 r;
  r.x = (uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)lo.y << 16);
  r.y = (uint32_t)(uint16_t)lo.z | ((uint32_t)(uint16_t)lo.w << 16);
  r.z = (uint32_t)(uint16_t)hi.x | ((uint32_t)(uint16_t)hi.y << 16);
  r.w = (uint32_t)(uint16_t)hi.z | ((uint32_t)(uint16_t)hi.w << 16);
  return r;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8); }

// Where a stage's token rows come from.
enum SyrkSource {
  kDenseRows = 0,    // rows t of X; buffer loads, tokens past the end read as zeros
  kGatherSmall = 1,  // rows row_idx[t] of an X below 4 GiB; buffer loads, bad rows read as zeros
  kGatherLarge = 2,  // rows row_idx[t] of any X; 64-bit addresses, bad rows read the zero row
};

template <bool kF16, int kSrc>
__global__ __launch_bounds__(kSyrkThreads, 1) void syrk_dma_kernel(SyrkArgs a) {
  constexpr bool kGather = kSrc != kDenseRows;
  // the ring: four distinct arrays, so the stage a read touches is known statically
  __shared__ __attribute__((aligned(1024))) char ring0[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring1[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring2[kStageB];
  __shared__ __attribute__((aligned(1024))) char ring3[kStageB];

  const int nwg = a.full + (a.tiles - a.full) * a.splits;
  // the two phases are remapped separately, so every XCD gets its share of
  // each (workgroups are dispatched in blockIdx order, round-robin over XCDs)
  const int wid = (int)blockIdx.x < a.full ? xcd_remap(blockIdx.x, a.full)
                                           : a.full + xcd_remap(blockIdx.x - a.full, nwg - a.full);
  // whole tiles first (every token, straight into S), then the remaining
  // tiles' token parts (partial tiles, added to S in part order afterwards),
  // part-major: a run of work ids covers many tiles of one token range, so
  // the X rows an XCD streams are shared by its workgroups in L2
  const bool whole = wid < a.full;
  const int k = wid - a.full;
  const int rest = a.tiles - a.full;
  const int split = whole ? 0 : k / rest;
  const int tile = whole ? wid : a.full + (k - split * rest);
  const int stages_per = whole ? 0x7FFFFFFF : a.stages_per_split;
  int bi, bj;
  tile_coords_band(tile, a.nt, bi, bj);
  const int i0 = bi * kTile, j0 = bj * kTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // A rows: channels 32 wr + 64 i + r; B cols: 32 ((wc & 1) + 4 (wc >> 1) + 2 jb) + c
  const int wr = wave >> 2;
  const int wc = wave & 3;

  const int64_t stage_begin = (int64_t)split * stages_per;
  const int64_t total_stages = (a.n_rows + kStage - 1) / kStage;
  const int64_t stage_end = min(stage_begin + stages_per, total_stages);
  const int nst = (int)(stage_end - stage_begin);
  const int64_t t_end = min(a.n_rows, stage_end * kStage);   // first token past this split
  const uint32_t rowb = (uint32_t)(a.ld_x * 2);

  // ---- direct loads: wave w fills 1 KiB chunks kSyrkCpw w + q (two token
  // rows each) of both panels; lane -> token row trow[q], swizzled octet.
  int trow[kSyrkCpw];
  int cI[kSyrkCpw], cJ[kSyrkCpw];
#pragma unroll
  for (int q = 0; q < kSyrkCpw; ++q) {
    trow[q] = 2 * (kSyrkCpw * wave + q) + (lane >> 5);
    const int o = (lane & 31) ^ (4 * (trow[q] & 3));
    // channels past d_in read a valid channel; they only reach rows and
    // columns of the tile that are never written
    cI[q] = min(i0 + 8 * o, a.d - 8);
    cJ[q] = min(j0 + 8 * o, a.d - 8);
  }
  int32_t idx[4][kSyrkCpw];   // gather: row indices of four stages (stage s in slot s & 3)
  auto load_idx = [&](int srel, int32_t (&slot)[kSyrkCpw]) {
#pragma unroll
    for (int q = 0; q < kSyrkCpw; ++q) {
      // branch-free: tokens past the end read the last valid entry; the
      // direct load drops them (the test is made where the value is used, so
      // the index load is not waited for here)
      const int64_t t = (stage_begin + srel) * kStage + trow[q];
      slot[q] = a.row_idx[t < t_end ? t : t_end - 1];
    }
  };
#define GQ_LDS_DST(buf, panel, q) \
  ((__attribute__((address_space(3))) void*)((buf) + (panel) * kPanelB + (kSyrkCpw * wave + (q)) * 1024))
  auto dma = [&](int srel, char* buf, const int32_t (&slot)[kSyrkCpw]) {
    if constexpr (kSrc == kDenseRows) {
      // the stage's rows as one buffer whose size ends at the split's last
      // token: rows past it read as zeros
      const int64_t t0 = (stage_begin + srel) * kStage;
      int64_t rem = (t_end - t0) * (int64_t)rowb;
      rem = rem < 0 ? 0 : min(rem, (int64_t)kStage * rowb);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.X + (t0 < t_end ? t0 : 0) * a.ld_x), (short)0, (int)rem, 0x00020000);
#pragma unroll
      for (int q = 0; q < kSyrkCpw; ++q) {
        const uint32_t vo = (uint32_t)trow[q] * rowb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQ_LDS_DST(buf, 0, q), 16, vo + 2u * (uint32_t)cI[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQ_LDS_DST(buf, 1, q), 16, vo + 2u * (uint32_t)cJ[q], 0, 0, 0);
      }
    } else if constexpr (kSrc == kGatherSmall) {
      // all of X as one buffer (the host takes this path only when X plus one
      // row stays below 2^32 bytes, so the size and every offset fit the
      // 32-bit buffer arithmetic); a bad row gets the offset of the byte
      // just past X, so its loads are out of range and read zeros
      const uint32_t xbytes = (uint32_t)(a.x_rows * (int64_t)rowb);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)a.X, (short)0, __builtin_bit_cast(int, xbytes), 0x00020000);
#pragma unroll
      for (int q = 0; q < kSyrkCpw; ++q) {
        const int64_t t = (stage_begin + srel) * kStage + trow[q];
        const int64_t r = slot[q];
        const bool ok = t < t_end && r >= 0 && r < a.x_rows;
        const uint32_t vo = ok ? (uint32_t)r * rowb : xbytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQ_LDS_DST(buf, 0, q), 16, vo + 2u * (uint32_t)cI[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQ_LDS_DST(buf, 1, q), 16, vo + 2u * (uint32_t)cJ[q], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < kSyrkCpw; ++q) {
        const int64_t t = (stage_begin + srel) * kStage + trow[q];
        const int64_t r = slot[q];
        const uint16_t* row = a.zero_row;
        if (t < t_end && r >= 0 && r < a.x_rows) row = a.X + r * a.ld_x;
        __builtin_amdgcn_global_load_lds(row + cI[q], GQ_LDS_DST(buf, 0, q), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(row + cJ[q], GQ_LDS_DST(buf, 1, q), 16, 0, 0);
      }
    }
  };

#undef GQ_LDS_DST

  // ---- transposed fragment reads: 16-lane group g reads token rows
  // 8 (g >> 1) + x (x = lane / 4 within the group) at channel quad (lane % 4)
  const int g = lane >> 4, j = lane & 15, x = j >> 2;
  const int lane_row = x * kRowB + (g >> 1) * 8 * kRowB + 8 * (j & 1);
  const int y = 2 * (g & 1) + ((j & 3) >> 1);   // octet within the 32-channel block
  // A block i holds octets 8 i + 4 wr + y, B block jb octets
  // 16 (wc >> 1) + 8 jb + 4 (wc & 1) + y.  With the ^ 4 (t & 3) slots, rows
  // x = 2, 3 find block i at 128 (i ^ 1) bytes: flip moves the even blocks up
  // and the odd blocks down by one.
  const int offA = lane_row + 16 * (4 * (wr ^ (x & 1)) + y);
  const int offB = lane_row + 16 * (4 * ((wc & 1) ^ (x & 1)) + y) + 256 * (wc >> 1) + kPanelB;
  const int flip = 128 * (x >> 1);

  f32x16 acc[4][kSyrkBJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < kSyrkBJ; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jb][r] = 0.0f;

  // fragments of one 16-token half of a stage: A blocks i, B blocks jb
  u32x4 fa0[4], fb0[kSyrkBJ], fa1[4], fb1[kSyrkBJ];
  auto read_half = [&](const char* buf, int ks, u32x4 (&fa)[4], u32x4 (&fb)[kSyrkBJ]) {
    const lds_char* lb = (const lds_char*)buf;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = tr_frag(lb + offA + ((i & 1) ? -flip : flip) + 128 * i + ks * 16 * kRowB);
#pragma unroll
    for (int jb = 0; jb < kSyrkBJ; ++jb)
      fb[jb] = tr_frag(lb + offB + ((jb & 1) ? -flip : flip) + 128 * jb + ks * 16 * kRowB);
  };
  auto mma_half = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[kSyrkBJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jb = 0; jb < kSyrkBJ; ++jb) acc[i][jb] = mfma16<kF16>(fa[i], fb[jb], acc[i][jb]);
  };
  // Per stage a wave issues 2 kSyrkCpw direct loads (and, gathering,
  // kSyrkCpw index loads after them).  At the wait of stage s the loads of
  // stage s + 1 must have landed; everything issued after them (its index
  // loads, stages s + 2, s + 3) may still fly.  Stage s loads stage s + 3
  // into the slot stage s - 1 left (every wave's reads of it ended before the
  // previous barrier).
  constexpr int kPerStage = (kGather ? 3 : 2) * kSyrkCpw;
  constexpr int kWaitNext = vmcnt_imm(2 * kPerStage + (kGather ? kSyrkCpw : 0));
#define GQ_STAGE(k, CUR, NXT, LOAD)                                      \
  {                                                                      \
    dma(s + (k) + 3, LOAD, idx[((k) + 3) & 3]);                          \
    if constexpr (kGather) load_idx(s + (k) + 7, idx[((k) + 3) & 3]);    \
    read_half(CUR, 1, fa1, fb1);                                         \
    mma_half(fa0, fb0);                                                  \
    __builtin_amdgcn_s_waitcnt(kWaitNext);                               \
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");    \
    read_half(NXT, 0, fa0, fb0);                                         \
    mma_half(fa1, fb1);                                                  \
  }
  if constexpr (kGather) {
    load_idx(0, idx[0]);
    load_idx(1, idx[1]);
    load_idx(2, idx[2]);
    load_idx(3, idx[3]);
  }
  dma(0, ring0, idx[0]);
  if constexpr (kGather) load_idx(4, idx[0]);
  dma(1, ring1, idx[1]);
  if constexpr (kGather) load_idx(5, idx[1]);
  dma(2, ring2, idx[2]);
  if constexpr (kGather) load_idx(6, idx[2]);
  __builtin_amdgcn_s_waitcnt(kWaitNext);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  read_half(ring0, 0, fa0, fb0);
  // stages past the split's end read the zero row, so the loop runs whole
  // turns of the ring
  for (int s = 0; s < nst; s += 4) {
    GQ_STAGE(0, ring0, ring1, ring3);
    GQ_STAGE(1, ring1, ring2, ring0);
    GQ_STAGE(2, ring2, ring3, ring1);
    GQ_STAGE(3, ring3, ring0, ring2);
  }
#undef GQ_STAGE
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  // epilogue: D layout of a 32x32 MFMA: register r of lane l is row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the block.
  const int d = a.d;
  float* part = (!whole && a.splits > 1)
                    ? a.partial + ((size_t)(tile - a.full) * a.splits + split) * (kTile * kTile)
                    : nullptr;
  // one block at a time (sched barriers): keeps the compiler from hoisting
  // every block's loads of S ahead of the stores, which spills with 256
  // accumulators
  if (part) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jb = 0; jb < kSyrkBJ; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = 32 * wr + 64 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int lc = 32 * ((wc & 1) + 4 * (wc >> 1) + 2 * jb) + (lane & 31);
          part[lr * kTile + lc] = acc[i][jb][r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jb = 0; jb < kSyrkBJ; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gi = i0 + 32 * wr + 64 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gj = j0 + 32 * ((wc & 1) + 4 * (wc >> 1) + 2 * jb) + (lane & 31);
          if (gi < d && gj < d && gi >= gj) {
            float* p = a.S + (size_t)gi * d + gj;
            *p = *p + acc[i][jb][r];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

__global__ void fill_u16_kernel(uint16_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// S_tile += sum over the token parts of tile first + blockIdx.y, in part order.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(float* __restrict__ S, const float* __restrict__ partial,
                                                          int d, int first, int splits) {
  const int tile = first + blockIdx.y;
  partial += (size_t)blockIdx.y * splits * (kTile * kTile);
  int bi, bj;
  tile_coords_band(tile, (d + kTile - 1) / kTile, bi, bj);
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;   // 4 consecutive columns
  const int lr = e / kTile, lc = e % kTile;
  const int gi = bi * kTile + lr;
  if (gi >= d) return;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    f32x4 v = *reinterpret_cast<const f32x4*>(partial + (size_t)s * (kTile * kTile) + e);
    sum += v;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int gj = bj * kTile + lc + c;
    if (gj < d && gi >= gj) {
      float* p = S + (size_t)gi * d + gj;
      *p = *p + sum[c];
    }
  }
}

// ------------------------------------------------------------------ fp32 inputs
constexpr int kK32 = 32;    // tokens per LDS stage

// fp32 activations: S += X^T X on fp32 MFMA (v_mfma_f32_32x32x2_f32).  A
// workgroup owns a kT x kT lower tile (kT = 128 when that still gives every
// CU a tile, else 64); its four waves each a (kT / 2)-square block of 32 x 32
// MFMA blocks (on a diagonal tile the block above the diagonal is skipped).
// Token rows are staged through LDS 32 at a time as X stores them (channels
// contiguous; the row stride puts the two half-waves' rows 32 banks apart),
// so an operand fragment (one channel per lane, two tokens) is a plain 4-byte
// read; the next stage is loaded into registers (16 bytes per load) while
// this one multiplies.  Rows past the end, and gathered rows outside X, read
// as zeros; channels past d_in (a multiple of 8) likewise.
template <int kT>
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ld_x,
                                                       const int32_t* __restrict__ row_idx, int64_t n_rows,
                                                       int64_t x_rows, int d, float* __restrict__ S) {
  constexpr int kLd = kT + 32;          // LDS row stride (floats)
  constexpr int kB = kT / 64;           // 32 x 32 blocks per wave and dimension
  constexpr int kTpr = kT / 8;          // staging threads per token row (8 floats of each panel each)
  constexpr int kRows = 256 / kTpr;     // token rows staged per pass
  constexpr int kPass = kK32 / kRows;
  __shared__ __attribute__((aligned(16))) float As[kK32 * kLd];
  __shared__ __attribute__((aligned(16))) float Bs[kK32 * kLd];
  int bi, bj;
  tile_coords(blockIdx.x, bi, bj);
  const int i0 = bi * kT, j0 = bj * kT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const bool skip = bi == bj && wi < wj;   // wave-uniform
  const int tk = tid / kTpr, ch = (tid % kTpr) * 8;
  float4 ra[kPass][2], rb[kPass][2];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int64_t t = t0 + tk + p * kRows;
      int64_t row = -1;
      if (t < n_rows) {
        row = row_idx ? (int64_t)row_idx[t] : t;
        if (row < 0 || row >= x_rows) row = -1;
      }
      const float* xr = X + (row >= 0 ? row : 0) * ld_x;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ca = i0 + ch + 4 * q, cb = j0 + ch + 4 * q;
        ra[p][q] = (row >= 0 && ca < d) ? *reinterpret_cast<const float4*>(xr + ca) : float4{0.f, 0.f, 0.f, 0.f};
        rb[p][q] = (row >= 0 && cb < d) ? *reinterpret_cast<const float4*>(xr + cb) : float4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  f32x16 acc[kB][kB];
#pragma unroll
  for (int u = 0; u < kB; ++u)
#pragma unroll
    for (int v = 0; v < kB; ++v)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][v][r] = 0.f;
  const int fa = (lane >> 5) * kLd + wi * (kT / 2) + (lane & 31);
  const int fb = (lane >> 5) * kLd + wj * (kT / 2) + (lane & 31);
  load(0);
  for (int64_t t0 = 0; t0 < n_rows; t0 += kK32) {
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        *reinterpret_cast<float4*>(&As[(tk + p * kRows) * kLd + ch + 4 * q]) = ra[p][q];
        *reinterpret_cast<float4*>(&Bs[(tk + p * kRows) * kLd + ch + 4 * q]) = rb[p][q];
      }
    __syncthreads();
    if (t0 + kK32 < n_rows) load(t0 + kK32);
    if (!skip) {
#pragma unroll
      for (int k = 0; k < kK32; k += 2) {
        float av[kB], bv[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          av[u] = As[fa + k * kLd + 32 * u];
          bv[u] = Bs[fb + k * kLd + 32 * u];
        }
#pragma unroll
        for (int u = 0; u < kB; ++u)
#pragma unroll
          for (int v = 0; v < kB; ++v) acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[v], acc[u][v], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (skip) return;
  // D layout of a 32x32 MFMA: register r of lane l is row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the block.
#pragma unroll
  for (int u = 0; u < kB; ++u)
#pragma unroll
    for (int v = 0; v < kB; ++v)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = i0 + wi * (kT / 2) + 32 * u + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gj = j0 + wj * (kT / 2) + 32 * v + (lane & 31);
        if (gi < d && gj < d && gi >= gj) {
          float* p = S + (size_t)gi * d + gj;
          *p = *p + acc[u][v][r];
        }
      }
}

// ------------------------------------------------------------------ fp64 diagonal
// Eight channels of one row as floats (exact for every input type).
template <int kDt>  // 0 f32, 1 f16, 2 bf16
__device__ __forceinline__ void load_octet(const void* __restrict__ Xv, int64_t row, int64_t ld_x, int ch0, float (&v)[8]) {
  if constexpr (kDt == 0) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(Xv) + row * ld_x + ch0);
    const f32x4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Xv) + row * ld_x + ch0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = q[c];
      if constexpr (kDt == 1) {
        v[2 * c] = f16_bits_to_f32(w & 0xFFFFu);
        v[2 * c + 1] = f16_bits_to_f32(w >> 16);
      } else {
        v[2 * c] = bf16_bits_to_f32(w & 0xFFFFu);
        v[2 * c + 1] = bf16_bits_to_f32(w >> 16);
      }
    }
  }
}

// Each thread owns one channel octet over a token range and accumulates the
// squares in fp64, eight tokens per step with their loads issued together;
// partial[split][channel] is then added to D in split order.  A gathered row
// outside X is read as row 0 and its values replaced by zeros, so the eight
// loads never wait behind a branch.
// kAbs: sums |x| instead of x^2 (the per-channel activation magnitude of
// activation-aware scaling), through the same partial sums and reduction.
template <int kDt, bool kGather, bool kAbs = false>  // kDt: 0 f32, 1 f16, 2 bf16
__global__ __launch_bounds__(256) void diag_partial_kernel(const void* __restrict__ Xv, int64_t ld_x,
                                                           const int32_t* __restrict__ row_idx, int64_t n_rows,
                                                           int64_t x_rows, int d, int64_t tok_per_split,
                                                           double* __restrict__ partial) {
  const int oct = blockIdx.x * 256 + threadIdx.x;
  const int ch0 = oct * 8;
  const int split = blockIdx.y;
  if (ch0 >= d) return;
  const int64_t t0 = (int64_t)split * tok_per_split;
  int64_t t1 = t0 + tok_per_split;
  if (t1 > n_rows) t1 = n_rows;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](const float (&v)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const double x = (double)v[c];
      if constexpr (kAbs) acc[c] += fabs(x);
      else acc[c] = fma(x, x, acc[c]);
    }
  };
  int64_t t = t0;
  for (; t + 8 <= t1; t += 8) {
    int64_t row[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (kGather) {
        const int64_t r = row_idx[t + u];
        ok[u] = r >= 0 && r < x_rows;
        row[u] = ok[u] ? r : 0;
      } else {
        ok[u] = true;   // a dense entry covers rows [0, n_rows) of X
        row[u] = t + u;
      }
    }
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load_octet<kDt>(Xv, row[u], ld_x, ch0, v[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (kGather) {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[u][c] = ok[u] ? v[u][c] : 0.f;
      }
      add(v[u]);
    }
  }
  for (; t < t1; ++t) {
    const int64_t row = kGather ? (int64_t)row_idx[t] : t;
    if (row < 0 || row >= x_rows) continue;
    float v[8];
    load_octet<kDt>(Xv, row, ld_x, ch0, v);
    add(v);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) partial[(size_t)split * d + ch0 + c] = acc[c];
}

// D[i] += sum over splits of partial[split][i]: 32 channels per workgroup, the
// splits cut into 8 contiguous runs (one per thread row, each summed in
// order), the 8 run sums then added in row order: a fixed order throughout.
__global__ __launch_bounds__(256) void diag_reduce_kernel(double* __restrict__ D, const double* __restrict__ partial,
                                                          int d, int splits) {
  __shared__ double part8[8][32];
  const int c = threadIdx.x & 31, row = threadIdx.x >> 5;
  const int i = blockIdx.x * 32 + c;
  const int per = (splits + 7) / 8;
  const int k0 = row * per, k1 = min(splits, k0 + per);
  double s = 0.0;
  if (i < d)
    for (int k = k0; k < k1; ++k) s += partial[(size_t)k * d + i];
  part8[row][c] = s;
  __syncthreads();
  if (row == 0 && i < d) {
    double t = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r) t += part8[r][c];
    D[i] += t;
  }
}

// N[b] += rows of this call that exist: a dense entry adds all of them, a
// gathered entry the indices inside [0, x_rows), counted by gridDim.x
// workgroups whose counts meet in an integer atomic add (an integer sum, so
// the order does not matter).
__global__ __launch_bounds__(256) void count_rows_kernel(const int32_t* __restrict__ idx, int64_t rows,
                                                         int64_t x_rows, int64_t* __restrict__ n) {
  __shared__ int64_t red[256];
  int64_t c = 0;
  if (idx == nullptr) {
    c = (blockIdx.x == 0 && threadIdx.x == 0) ? rows : 0;
  } else {
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < rows; t += (int64_t)gridDim.x * 256) {
      const int64_t r = idx[t];
      c += (r >= 0 && r < x_rows) ? 1 : 0;
    }
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && red[0] != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(n), (unsigned long long)red[0]);
}

// ------------------------------------------------------------------ host side
namespace {

constexpr int kCUs = 256;

// Work decomposition of the MFMA product (one 512-thread workgroup per CU):
// `full` tiles, a whole number of rounds of the CUs, each taken by one
// workgroup over every token and written straight into S; the remaining
// tiles split over tokens into `splits` parts whose partial tiles are added
// to S afterwards.  Chosen by a cost model in stage-times on the critical
// path: rounds x stages per workgroup, plus about 0.08 stage-times per
// partial tile (256 KiB written and read back at full HBM bandwidth).
struct SyrkPlan {
  int full, splits;
};

SyrkPlan choose_plan(int tiles, int64_t stages) {
  SyrkPlan best{0, 1};
  double best_cost = 1e300;
  const int smax = (int)std::max<int64_t>(1, std::min<int64_t>(64, stages / 32));
  for (int rounds : {0, tiles / kCUs}) {
    const int full = rounds * kCUs;
    const int rest = tiles - full;
    for (int s = 1; s <= (rest > 0 ? smax : 1); ++s) {
      double cost = (double)rounds * (double)stages;
      if (rest > 0) {
        cost += (double)cdiv((int64_t)rest * s, kCUs) * (double)cdiv(stages, s);
        if (s > 1) cost += 0.08 * (double)rest * s;
      }
      if (cost < best_cost) {
        best_cost = cost;
        best = SyrkPlan{full, s};
      }
    }
  }
  return best;
}

size_t syrk_partial_bytes(int tiles, const SyrkPlan& pl) {
  return pl.splits > 1 ? (size_t)pl.splits * (tiles - pl.full) * kTile * kTile * sizeof(float) : 0;
}

int diag_splits(int d, int64_t n) {
  int octets = (d + 7) / 8;
  int64_t want = cdiv(256 * 1024, octets);   // about 16 waves per CU
  int64_t cap = std::max<int64_t>(1, n / 256);
  return (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(want, cap), 1024));
}

}  // namespace

size_t hessian_workspace_bytes(int64_t d, int64_t n_rows, int64_t batch, int dtype) {
  (void)batch;
  size_t bytes = 0;
  if (dtype != GPTQ_F32) {
    int nt = (int)cdiv(d, kTile);
    int tiles = nt * (nt + 1) / 2;
    const SyrkPlan pl = choose_plan(tiles, cdiv(std::max<int64_t>(n_rows, 1), kStage));
    bytes += align_up(syrk_partial_bytes(tiles, pl), 256);
    bytes += align_up((size_t)d * sizeof(uint16_t), 256);   // zero row
  }
  bytes += align_up((size_t)diag_splits((int)d, std::max<int64_t>(n_rows, 1)) * d * sizeof(double), 256);
  return bytes + 256;
}

static gptq_status launch_entry(float* S, double* D, int64_t* n_dev, const void* X, int dtype, int64_t n,
                                int64_t x_rows, int64_t d, int64_t ld_x, const int32_t* idx, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  // no row of an empty X can contribute (every gathered index is outside it)
  if (n == 0 || x_rows == 0) return GPTQ_OK;
  Carver cv(ws);
  {
    TimedScope ts(kTimeDiag, stream);
    const unsigned cb = idx == nullptr ? 1u : (unsigned)std::min<int64_t>(cdiv(n, 2048), 256);
    hipLaunchKernelGGL(count_rows_kernel, dim3(cb), dim3(256), 0, stream, idx, n, x_rows, n_dev);
    GQ_LAUNCHED();
  }
  // ---- product
  if (dtype == GPTQ_F32) {
    const int nt128 = (int)cdiv(d, 128), nt64 = (int)cdiv(d, 64);
    const int t128 = nt128 * (nt128 + 1) / 2, t64 = nt64 * (nt64 + 1) / 2;
    TimedScope ts(kTimeSyrk, stream);
    const float* Xf = static_cast<const float*>(X);
    if (t128 >= kCUs) hipLaunchKernelGGL(syrk_f32_kernel<128>, dim3(t128), dim3(256), 0, stream, Xf, ld_x, idx, n, x_rows, (int)d, S);
    else hipLaunchKernelGGL(syrk_f32_kernel<64>, dim3(t64), dim3(256), 0, stream, Xf, ld_x, idx, n, x_rows, (int)d, S);
    GQ_LAUNCHED();
  } else {
    SyrkArgs a;
    a.X = static_cast<const uint16_t*>(X);
    a.ld_x = ld_x;
    a.row_idx = idx;
    a.n_rows = n;
    a.x_rows = x_rows;
    a.d = (int)d;
    a.nt = (int)cdiv(d, kTile);
    a.tiles = a.nt * (a.nt + 1) / 2;
    int64_t stages = cdiv(n, kStage);
    SyrkPlan pl = choose_plan(a.tiles, stages);
    // never more partial tiles than the workspace holds (it is sized for the
    // largest entry of the call; a smaller entry may prefer other splits)
    const size_t fixed_need = align_up((size_t)diag_splits((int)d, n) * d * sizeof(double), 256) +
                              align_up((size_t)d * sizeof(uint16_t), 256) + 256;
    while (pl.splits > 1 && align_up(syrk_partial_bytes(a.tiles, pl), 256) + fixed_need > ws_bytes) --pl.splits;
    a.full = pl.full;
    a.splits = pl.splits;
    size_t pbytes = syrk_partial_bytes(a.tiles, pl);
    a.partial = cv.take<float>(pbytes / sizeof(float));
    uint16_t* zero_row = cv.take<uint16_t>((size_t)d);
    if (cv.used > ws_bytes) return GPTQ_ENOMEM;
    a.zero_row = zero_row;
    a.stages_per_split = (int)cdiv(stages, a.splits);
    a.S = S;
    {
      // a gather over an X whose bytes plus one row stay below 4 GiB addresses
      // it as one buffer (its byte size and every offset, the out-of-range
      // one of a bad row included, fit the 32-bit buffer arithmetic); anything
      // larger takes 64-bit addresses
      const bool small_x = (x_rows + 1) * (ld_x * 2) < ((int64_t)1 << 32);
      const int src = idx == nullptr ? kDenseRows : (small_x ? kGatherSmall : kGatherLarge);
      if (src == kGatherLarge) {
        hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)cdiv(d, 256)), dim3(256), 0, stream, zero_row, (int)d);
        GQ_LAUNCHED();
      }
      TimedScope ts(kTimeSyrk, stream);
      dim3 grid(a.full + (a.tiles - a.full) * a.splits), block(kSyrkThreads);
      if (dtype == GPTQ_F16) {
        if (src == kDenseRows) hipLaunchKernelGGL((syrk_dma_kernel<true, kDenseRows>), grid, block, 0, stream, a);
        else if (src == kGatherSmall) hipLaunchKernelGGL((syrk_dma_kernel<true, kGatherSmall>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((syrk_dma_kernel<true, kGatherLarge>), grid, block, 0, stream, a);
      } else {
        if (src == kDenseRows) hipLaunchKernelGGL((syrk_dma_kernel<false, kDenseRows>), grid, block, 0, stream, a);
        else if (src == kGatherSmall) hipLaunchKernelGGL((syrk_dma_kernel<false, kGatherSmall>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((syrk_dma_kernel<false, kGatherLarge>), grid, block, 0, stream, a);
      }
      GQ_LAUNCHED();
    }
    if (a.splits > 1) {
      TimedScope ts(kTimeSyrkReduce, stream);
      dim3 grid(kTile * kTile / (256 * 4), a.tiles - a.full);
      hipLaunchKernelGGL(syrk_reduce_kernel, grid, dim3(256), 0, stream, S, a.partial, (int)d, a.full, a.splits);
      GQ_LAUNCHED();
    }
  }
  // ---- fp64 diagonal
  {
    int sp = diag_splits((int)d, n);
    double* part = cv.take<double>((size_t)sp * d);
    if (cv.used > ws_bytes) return GPTQ_ENOMEM;
    int64_t tps = cdiv(n, sp);
    TimedScope ts(kTimeDiag, stream);
    dim3 grid((unsigned)cdiv(cdiv(d, 8), 256), sp);
#define GQ_DIAG(DT, G) \
  hipLaunchKernelGGL((diag_partial_kernel<DT, G>), grid, dim3(256), 0, stream, X, ld_x, idx, n, x_rows, (int)d, tps, part)
    if (idx == nullptr) {
      if (dtype == GPTQ_F32) GQ_DIAG(0, false);
      else if (dtype == GPTQ_F16) GQ_DIAG(1, false);
      else GQ_DIAG(2, false);
    } else {
      if (dtype == GPTQ_F32) GQ_DIAG(0, true);
      else if (dtype == GPTQ_F16) GQ_DIAG(1, true);
      else GQ_DIAG(2, true);
    }
#undef GQ_DIAG
    GQ_LAUNCHED();
    hipLaunchKernelGGL(diag_reduce_kernel, dim3((unsigned)cdiv(d, 32)), dim3(256), 0, stream, D, part, (int)d, sp);
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}

size_t abs_workspace_bytes(int64_t d, int64_t n_rows) {
  return align_up((size_t)diag_splits((int)d, std::max<int64_t>(n_rows, 1)) * d * sizeof(double), 256) + 256;
}

// A += sum over the entry's rows of |x| per channel (fp64), with the fp64
// diagonal's kernels.
static gptq_status launch_abs(double* A, const void* X, int dtype, int64_t n, int64_t x_rows, int64_t d, int64_t ld_x,
                              const int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || x_rows == 0) return GPTQ_OK;
  Carver cv(ws);
  const int sp = diag_splits((int)d, n);
  double* part = cv.take<double>((size_t)sp * d);
  if (cv.used > ws_bytes) return GPTQ_ENOMEM;
  const int64_t tps = cdiv(n, sp);
  TimedScope ts(kTimeAbs, stream);
  dim3 grid((unsigned)cdiv(cdiv(d, 8), 256), sp);
#define GQ_ABS(DT, G)                                                                                          \
  hipLaunchKernelGGL((diag_partial_kernel<DT, G, true>), grid, dim3(256), 0, stream, X, ld_x, idx, n, x_rows, \
                     (int)d, tps, part)
  if (idx == nullptr) {
    if (dtype == GPTQ_F32) GQ_ABS(0, false);
    else if (dtype == GPTQ_F16) GQ_ABS(1, false);
    else GQ_ABS(2, false);
  } else {
    if (dtype == GPTQ_F32) GQ_ABS(0, true);
    else if (dtype == GPTQ_F16) GQ_ABS(1, true);
    else GQ_ABS(2, true);
  }
#undef GQ_ABS
  GQ_LAUNCHED();
  hipLaunchKernelGGL(diag_reduce_kernel, dim3((unsigned)cdiv(d, 32)), dim3(256), 0, stream, A, part, (int)d, sp);
  GQ_LAUNCHED();
  return GPTQ_OK;
}

}  // namespace gq

using namespace gq;

extern "C" gptq_status gptq_abs_accumulate(double* A, const void* X, int32_t x_dtype, int64_t n_rows, int64_t d_in,
                                           int64_t ld_x, const int32_t* row_idx, const int64_t* row_ptr,
                                           int64_t batch, void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(A != nullptr);
  GQ_CHECK_ARG(x_dtype == GPTQ_F32 || x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(d_in >= 8 && d_in % 8 == 0 && d_in <= (1 << 20));
  GQ_CHECK_ARG(n_rows >= 0 && ld_x >= d_in && batch >= 1);
  const int64_t es = x_dtype == GPTQ_F32 ? 4 : 2;
  GQ_CHECK_ARG((ld_x * es) % 16 == 0);
  GQ_CHECK_ARG(n_rows == 0 || X != nullptr);
  GQ_CHECK_ARG(X == nullptr || (reinterpret_cast<uintptr_t>(X) % 16) == 0);
  if (row_idx == nullptr) {
    GQ_CHECK_ARG(batch == 1);
  } else {
    GQ_CHECK_ARG(row_ptr != nullptr && row_ptr[0] == 0);
    for (int64_t b = 0; b < batch; ++b) GQ_CHECK_ARG(row_ptr[b + 1] >= row_ptr[b]);
  }
  int64_t max_rows = row_idx ? 0 : n_rows;
  if (row_idx)
    for (int64_t b = 0; b < batch; ++b) max_rows = std::max<int64_t>(max_rows, row_ptr[b + 1] - row_ptr[b]);
  if (ws_bytes < abs_workspace_bytes(d_in, max_rows) || workspace == nullptr) return GPTQ_ENOMEM;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t rows = row_idx ? row_ptr[b + 1] - row_ptr[b] : n_rows;
    const int32_t* idx = row_idx ? row_idx + row_ptr[b] : nullptr;
    gptq_status s = launch_abs(A + (size_t)b * d_in, X, x_dtype, rows, n_rows, d_in, ld_x, idx, workspace, ws_bytes, st);
    if (s != GPTQ_OK) return s;
  }
  return GPTQ_OK;
}

extern "C" gptq_status gptq_hessian_accumulate(float* S, double* D, int64_t* n_tokens, const void* X,
                                               int32_t x_dtype, int64_t n_rows, int64_t d_in, int64_t ld_x,
                                               const int32_t* row_idx, const int64_t* row_ptr, int64_t batch,
                                               void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(S && D && n_tokens);
  GQ_CHECK_ARG(x_dtype == GPTQ_F32 || x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16);
  GQ_CHECK_ARG(d_in >= 8 && d_in % 8 == 0 && d_in <= (1 << 20));
  GQ_CHECK_ARG(n_rows >= 0 && ld_x >= d_in && batch >= 1);
  const int64_t es = x_dtype == GPTQ_F32 ? 4 : 2;
  GQ_CHECK_ARG((ld_x * es) % 16 == 0);
  GQ_CHECK_ARG(n_rows == 0 || X != nullptr);
  GQ_CHECK_ARG(X == nullptr || (reinterpret_cast<uintptr_t>(X) % 16) == 0);
  if (row_idx == nullptr) {
    GQ_CHECK_ARG(batch == 1);
  } else {
    GQ_CHECK_ARG(row_ptr != nullptr && row_ptr[0] == 0);
    for (int64_t b = 0; b < batch; ++b) GQ_CHECK_ARG(row_ptr[b + 1] >= row_ptr[b]);
  }
  size_t need = 0;
  int64_t max_rows = row_idx ? 0 : n_rows;
  if (row_idx)
    for (int64_t b = 0; b < batch; ++b) max_rows = std::max<int64_t>(max_rows, row_ptr[b + 1] - row_ptr[b]);
  need = hessian_workspace_bytes(d_in, max_rows, 1, x_dtype);
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return GPTQ_ENOMEM;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t b = 0; b < batch; ++b) {
    int64_t rows = row_idx ? row_ptr[b + 1] - row_ptr[b] : n_rows;
    const int32_t* idx = row_idx ? row_idx + row_ptr[b] : nullptr;
    gptq_status s = launch_entry(S + (size_t)b * d_in * d_in, D + (size_t)b * d_in, n_tokens + b, X, x_dtype,
                                 rows, n_rows, d_in, ld_x, idx, workspace, ws_bytes, st);
    if (s != GPTQ_OK) return s;
  }
  return GPTQ_OK;
}
