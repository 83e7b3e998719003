// Hessian accumulation S += X^T X (lower triangle) and D += diag(X^T X) in fp64.
//
// The product is the dense contraction of the method ("3. 模型量化技术(下)",
// pseudocode block: H from the layer's inputs; ipipp.com quantize_gptq listing:
// H = 2 (X^T X) / N).  X is token-major, so both MFMA operands are columns of X:
// each thread loads an 8-token x 8-channel block with 16-byte row loads,
// transposes it in registers (v_perm_b32), and stores 8 channels x 8 tokens into
// LDS so that every MFMA operand fragment (8 consecutive tokens of one channel)
// is a single 16-byte LDS read.
#include "common.h"

namespace gq {

// ------------------------------------------------------------------ tiling
constexpr int kTile = 256;      // output tile edge (channels)
constexpr int kStage = 64;      // tokens per LDS stage
constexpr int kSyrkThreads = 512;
constexpr int kRowBytes = kStage * 2;  // one channel row of a stage in LDS

struct SyrkArgs {
  const uint16_t* X;        // bf16 / fp16 bit patterns
  int64_t ld_x;             // elements
  const int32_t* row_idx;   // gather list (already offset to this entry) or null
  int64_t n_rows;           // rows of this entry
  int64_t x_rows;           // rows of X (gathered indices outside are skipped)
  int d;
  int nt;                   // tiles per dimension
  int tiles;                // nt (nt + 1) / 2
  int splits;
  int stages_per_split;
  float* S;                 // this entry's S
  float* partial;           // splits > 1: [splits][tiles][kTile * kTile]
};

__device__ __forceinline__ void tile_coords(int t, int& bi, int& bj) {
  int b = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((b + 1) * (b + 2) / 2 <= t) ++b;
  while (b * (b + 1) / 2 > t) --b;
  bi = b;
  bj = t - b * (b + 1) / 2;
}

// LDS byte offset of (channel row m, 8-token group tg) inside one panel.  The
// 16-byte slot is XOR-swizzled with both the low and the next three bits of m
// so that the transposed stores (8 lanes = 8 rows 8 apart) and the fragment
// loads (8 lanes = 8 consecutive rows) both touch 8 distinct bank groups.
__device__ __forceinline__ int lds_off(int m, int tg) {
  int slot = tg ^ (m & 7) ^ ((m >> 3) & 7);
  return m * kRowBytes + slot * 16;
}

// Swap 16-bit halves between two rows: lo16(a), lo16(b) and hi16(a), hi16(b).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <bool kGather>
__device__ __forceinline__ void load_block(const SyrkArgs& a, int64_t tok0, int ch0, u32x4 (&r)[8]) {
  const bool ch_ok = ch0 < a.d;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t t = tok0 + i;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ch_ok && t < a.n_rows) {
      int64_t row = kGather ? (int64_t)a.row_idx[t] : t;
      if (!kGather || (row >= 0 && row < a.x_rows))
        v = *reinterpret_cast<const u32x4*>(a.X + row * a.ld_x + ch0);
    }
    r[i] = v;
  }
}

// r[i] holds channels ch0..ch0+7 of token i; write channel c's 8 tokens.
__device__ __forceinline__ void store_block_T(char* panel, int mrow0, int tg, const u32x4 (&r)[8]) {
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) {
    u32x4 lo, hi;
    lo.x = pack_lo(r[0][c2], r[1][c2]);
    lo.y = pack_lo(r[2][c2], r[3][c2]);
    lo.z = pack_lo(r[4][c2], r[5][c2]);
    lo.w = pack_lo(r[6][c2], r[7][c2]);
    hi.x = pack_hi(r[0][c2], r[1][c2]);
    hi.y = pack_hi(r[2][c2], r[3][c2]);
    hi.z = pack_hi(r[4][c2], r[5][c2]);
    hi.w = pack_hi(r[6][c2], r[7][c2]);
    int m = mrow0 + 2 * c2;
    *reinterpret_cast<u32x4*>(panel + lds_off(m, tg)) = lo;
    *reinterpret_cast<u32x4*>(panel + lds_off(m + 1, tg)) = hi;
  }
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

// Work id -> (split, tile).  Consecutive ids are dispatched round-robin over
// the 8 XCDs; the remap gives each XCD a contiguous run of tiles of the same
// token split, so tiles that share X panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int nx = 8;
  int per = nwg / nx;
  int full = per * nx;
  if (bid >= full) return bid;
  return (bid % nx) * per + bid / nx;
}

template <bool kF16, bool kGather>
__global__ __launch_bounds__(kSyrkThreads, 1) void syrk_mfma_kernel(SyrkArgs a) {
  // two LDS stages (double buffer), each holding panel I and panel J
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int kPanel = kTile * kRowBytes;

  const int nwg = a.tiles * a.splits;
  const int wid = xcd_remap(blockIdx.x, nwg);
  const int split = wid / a.tiles;
  const int tile = wid - split * a.tiles;
  int bi, bj;
  tile_coords(tile, bi, bj);
  const bool diag = (bi == bj);
  const int i0 = bi * kTile, j0 = bj * kTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 2;   // 0..1 : 128-row half
  const int wc = wave & 3;    // 0..3 : 64-col quarter

  // loader role: threads 0..255 load panel I, 256..511 panel J
  const int half = tid >> 8;
  const int tt = tid & 255;
  const int oc = tt & 31;     // channel octet within the panel
  const int tg = tt >> 5;     // 8-token group within the stage
  const bool loader = !(diag && half == 1);
  const int ch0 = (half ? j0 : i0) + oc * 8;

  const int64_t stage_begin = (int64_t)split * a.stages_per_split;
  int64_t stage_end = stage_begin + a.stages_per_split;
  const int64_t total_stages = (a.n_rows + kStage - 1) / kStage;
  if (stage_end > total_stages) stage_end = total_stages;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 regs[8];
  // prologue: stage 0 into buffer 0, stage 1 into registers
  if (stage_begin < stage_end) {
    if (loader) {
      load_block<kGather>(a, stage_begin * kStage + tg * 8, ch0, regs);
      store_block_T(smem + half * kPanel, oc * 8, tg, regs);
      if (stage_begin + 1 < stage_end) load_block<kGather>(a, (stage_begin + 1) * kStage + tg * 8, ch0, regs);
    }
    __syncthreads();
  }

  for (int64_t s = stage_begin; s < stage_end; ++s) {
    const int buf = (int)((s - stage_begin) & 1);
    const char* pI = smem + buf * 2 * kPanel;
    const char* pB = diag ? pI : pI + kPanel;
#pragma unroll
    for (int ks = 0; ks < kStage / 16; ++ks) {
      const int tgr = ks * 2 + (lane >> 5);
      u32x4 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int m = wr * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const u32x4*>(pI + lds_off(m, tgr));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int n = wc * 64 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const u32x4*>(pB + lds_off(n, tgr));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16<kF16>(af[i], bf[j], acc[i][j]);
    }
    // next stage's registers go to the other buffer (last read one stage ago),
    // then the registers fetch the stage after it
    if (loader && s + 1 < stage_end) {
      store_block_T(smem + (buf ^ 1) * 2 * kPanel + half * kPanel, oc * 8, tg, regs);
      if (s + 2 < stage_end) load_block<kGather>(a, (s + 2) * kStage + tg * 8, ch0, regs);
    }
    __syncthreads();
  }

  // epilogue: D layout of a 32x32 MFMA: register r of lane l is row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
  const int d = a.d;
  float* part = a.splits > 1 ? a.partial + ((size_t)split * a.tiles + tile) * (kTile * kTile) : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int lr = wr * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        int lc = wc * 64 + j * 32 + (lane & 31);
        if (part) {
          part[lr * kTile + lc] = acc[i][j][r];
        } else {
          int gi = i0 + lr, gj = j0 + lc;
          if (gi < d && gj < d && gi >= gj) {
            float* p = a.S + (size_t)gi * d + gj;
            *p = *p + acc[i][j][r];
          }
        }
      }
}

// S_tile += sum over splits of the partial tiles, in split order.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(float* __restrict__ S, const float* __restrict__ partial,
                                                          int d, int tiles, int splits) {
  const int tile = blockIdx.y;
  int bi, bj;
  tile_coords(tile, bi, bj);
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;   // 4 consecutive columns
  const int lr = e / kTile, lc = e % kTile;
  const int gi = bi * kTile + lr;
  if (gi >= d) return;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    f32x4 v = *reinterpret_cast<const f32x4*>(partial + ((size_t)s * tiles + tile) * (kTile * kTile) + e);
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
// A plain VALU product for fp32 activations (64x64 lower tiles, 4x4 per thread).
constexpr int kT32 = 64;
constexpr int kK32 = 16;

__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ld_x,
                                                       const int32_t* __restrict__ row_idx, int64_t n_rows,
                                                       int64_t x_rows, int d, float* __restrict__ S) {
  __shared__ float As[kK32][kT32 + 4];
  __shared__ float Bs[kK32][kT32 + 4];
  int bi, bj;
  tile_coords(blockIdx.x, bi, bj);
  const int i0 = bi * kT32, j0 = bj * kT32;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n_rows; t0 += kK32) {
    for (int e = threadIdx.x; e < kK32 * kT32; e += 256) {
      int k = e / kT32, m = e % kT32;
      int64_t t = t0 + k;
      float va = 0.f, vb = 0.f;
      if (t < n_rows) {
        int64_t row = row_idx ? (int64_t)row_idx[t] : t;
        if (row >= 0 && row < x_rows) {
          if (i0 + m < d) va = X[row * ld_x + i0 + m];
          if (j0 + m < d) vb = X[row * ld_x + j0 + m];
        }
      }
      As[k][m] = va;
      Bs[k][m] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kK32; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[k][ty * 4 + u];
        bv[u] = Bs[k][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int gi = i0 + ty * 4 + u, gj = j0 + tx * 4 + v;
      if (gi < d && gj < d && gi >= gj) {
        float* p = S + (size_t)gi * d + gj;
        *p = *p + acc[u][v];
      }
    }
}

// ------------------------------------------------------------------ fp64 diagonal
// Each thread owns one channel octet over a token range and accumulates the
// squares in fp64; partial[split][channel] is then added to D in split order.
template <int kDt>  // 0 f32, 1 f16, 2 bf16
__global__ __launch_bounds__(256) void diag_partial_kernel(const void* __restrict__ Xv, int64_t ld_x,
                                                           const int32_t* __restrict__ row_idx, int64_t n_rows,
                                                           int64_t x_rows, int d, int64_t tok_per_split,
                                                           double* __restrict__ partial) {
  const int oct = blockIdx.x * 256 + threadIdx.x;
  const int ch0 = oct * 8;
  const int split = blockIdx.y;
  if (ch0 >= d) return;
  int64_t t0 = (int64_t)split * tok_per_split;
  int64_t t1 = t0 + tok_per_split;
  if (t1 > n_rows) t1 = n_rows;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t t = t0; t < t1; ++t) {
    int64_t row = row_idx ? (int64_t)row_idx[t] : t;
    if (row < 0 || row >= x_rows) continue;
    float v[8];
    if constexpr (kDt == 0) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(Xv) + row * ld_x + ch0);
      f32x4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Xv) + row * ld_x + ch0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w = q[c];
        if constexpr (kDt == 1) {
          v[2 * c] = f16_bits_to_f32(w & 0xFFFFu);
          v[2 * c + 1] = f16_bits_to_f32(w >> 16);
        } else {
          v[2 * c] = bf16_bits_to_f32(w & 0xFFFFu);
          v[2 * c + 1] = bf16_bits_to_f32(w >> 16);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      double x = (double)v[c];
      acc[c] = fma(x, x, acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) partial[(size_t)split * d + ch0 + c] = acc[c];
}

__global__ __launch_bounds__(256) void diag_reduce_kernel(double* __restrict__ D, const double* __restrict__ partial,
                                                          int d, int splits) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  double s = 0.0;
  for (int k = 0; k < splits; ++k) s += partial[(size_t)k * d + i];
  D[i] += s;
}

// ------------------------------------------------------------------ host side
namespace {

constexpr int kCUs = 256;

// Number of token splits for the MFMA product: balance tiles x splits over the
// CUs (one 512-thread workgroup per CU), each split at least 16 stages, and
// keep the partial-tile traffic modest.
int choose_splits(int tiles, int64_t stages) {
  int best = 1;
  double best_cost = 1e300;
  const int smax = (int)std::max<int64_t>(1, std::min<int64_t>(64, stages / 16));
  for (int s = 1; s <= smax; ++s) {
    int64_t waves = cdiv((int64_t)tiles * s, kCUs);
    double per = (double)cdiv(stages, s);           // stages per workgroup
    double cost = waves * per;                      // stage-times on the critical path
    // partial tiles: 256 KiB written and read back per workgroup, about 0.08
    // stage-times each at full HBM bandwidth
    if (s > 1) cost += 0.08 * (double)tiles * s;
    if (cost < best_cost * 0.97) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

size_t syrk_partial_bytes(int tiles, int splits) {
  return splits > 1 ? (size_t)splits * tiles * kTile * kTile * sizeof(float) : 0;
}

int diag_splits(int d, int64_t n) {
  int octets = (d + 7) / 8;
  int64_t want = cdiv(64 * 1024, octets);
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
    int splits = choose_splits(tiles, cdiv(std::max<int64_t>(n_rows, 1), kStage));
    bytes += align_up(syrk_partial_bytes(tiles, splits), 256);
  }
  bytes += align_up((size_t)diag_splits((int)d, std::max<int64_t>(n_rows, 1)) * d * sizeof(double), 256);
  return bytes + 256;
}

static gptq_status launch_entry(float* S, double* D, const void* X, int dtype, int64_t n, int64_t x_rows,
                                int64_t d, int64_t ld_x, const int32_t* idx, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (n == 0) return GPTQ_OK;
  Carver cv(ws);
  // ---- product
  if (dtype == GPTQ_F32) {
    int nt = (int)cdiv(d, kT32);
    int tiles = nt * (nt + 1) / 2;
    TimedScope ts(kTimeSyrk, stream);
    hipLaunchKernelGGL(syrk_f32_kernel, dim3(tiles), dim3(256), 0, stream, static_cast<const float*>(X), ld_x,
                       idx, n, x_rows, (int)d, S);
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
    a.splits = choose_splits(a.tiles, stages);
    // never more partial tiles than the workspace holds (it is sized for the
    // largest entry of the call; a smaller entry may prefer other splits)
    const size_t diag_need = align_up((size_t)diag_splits((int)d, n) * d * sizeof(double), 256) + 512;
    while (a.splits > 1 && align_up(syrk_partial_bytes(a.tiles, a.splits), 256) + diag_need > ws_bytes) --a.splits;
    size_t pbytes = syrk_partial_bytes(a.tiles, a.splits);
    a.partial = cv.take<float>(pbytes / sizeof(float));
    if (cv.used > ws_bytes) return GPTQ_ENOMEM;
    a.stages_per_split = (int)cdiv(stages, a.splits);
    a.S = S;
    const size_t lds = 4 * kTile * kRowBytes;   // two stages x two panels
    {
      auto kern = dtype == GPTQ_F16 ? (idx ? syrk_mfma_kernel<true, true> : syrk_mfma_kernel<true, false>)
                                    : (idx ? syrk_mfma_kernel<false, true> : syrk_mfma_kernel<false, false>);
      // more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
      GQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds));
      TimedScope ts(kTimeSyrk, stream);
      dim3 grid(a.tiles * a.splits), block(kSyrkThreads);
      hipLaunchKernelGGL(kern, grid, block, lds, stream, a);
      GQ_LAUNCHED();
    }
    if (a.splits > 1) {
      TimedScope ts(kTimeSyrkReduce, stream);
      dim3 grid(kTile * kTile / (256 * 4), a.tiles);
      hipLaunchKernelGGL(syrk_reduce_kernel, grid, dim3(256), 0, stream, S, a.partial, (int)d, a.tiles, a.splits);
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
    if (dtype == GPTQ_F32)
      hipLaunchKernelGGL(diag_partial_kernel<0>, grid, dim3(256), 0, stream, X, ld_x, idx, n, x_rows, (int)d, tps, part);
    else if (dtype == GPTQ_F16)
      hipLaunchKernelGGL(diag_partial_kernel<1>, grid, dim3(256), 0, stream, X, ld_x, idx, n, x_rows, (int)d, tps, part);
    else
      hipLaunchKernelGGL(diag_partial_kernel<2>, grid, dim3(256), 0, stream, X, ld_x, idx, n, x_rows, (int)d, tps, part);
    GQ_LAUNCHED();
    hipLaunchKernelGGL(diag_reduce_kernel, dim3((unsigned)cdiv(d, 256)), dim3(256), 0, stream, D, part, (int)d, sp);
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}

}  // namespace gq

using namespace gq;

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
    gptq_status s = launch_entry(S + (size_t)b * d_in * d_in, D + (size_t)b * d_in, X, x_dtype, rows, n_rows,
                                 d_in, ld_x, idx, workspace, ws_bytes, st);
    if (s != GPTQ_OK) return s;
    n_tokens[b] += rows;
  }
  return GPTQ_OK;
}
