// Damping, importance order and the inverse-Hessian factor U (U^T U = Hd^-1).
//
// The pages feed each column's rounding error through a row of the inverse
// Hessian and say the inverse is handled through a decomposition in practice
// (ipipp.com, section 一, paragraph before the listing; "1. 项目概述：大模型量化的
// “校准”艺术", section 2.2 step 4).  The exact form of that update uses the upper
// Cholesky factor U of Hd^-1.  With J the reversal permutation and
// J Hd J = L L^T (lower Cholesky), U = J L^-1 J, so one Cholesky and one
// triangular inverse of the reversed matrix give U without ever forming Hd^-1.
// Both are computed in fp64 by a recursive 2x2 block scheme whose work is all
// in fp64 GEMM launches, with 64x64 leaf blocks factored inside one workgroup.
#include <cmath>
#include <mutex>
#include <unordered_map>

#include "common.h"

namespace gq {

constexpr int kLeaf = 64;
typedef double f64x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ small kernels
constexpr int kMaxBatch = 64;

// 2 / N of every entry from the device token counts; an entry without
// calibration rows gets info = -1 (its factor is not meaningful), every
// other entry starts with info = 0.
__global__ void set_scalars_kernel(const int64_t* __restrict__ n, int nb, double* __restrict__ two_over_n,
                                   int32_t* __restrict__ info) {
  const int i = threadIdx.x;
  if (i < nb) {
    const int64_t v = n[i];
    two_over_n[i] = v > 0 ? 2.0 / (double)v : __builtin_nan("");
    info[i] = v > 0 ? 0 : -1;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// lambda_b = damp_rel * mean_i(2 D_b[i] / N_b), fixed-order reduction.
__global__ __launch_bounds__(256) void damping_kernel(const double* __restrict__ D, int d,
                                                      const double* __restrict__ two_over_n, float damp_rel,
                                                      double* __restrict__ lam) {
  const int b = blockIdx.x;
  const double* Db = D + (size_t)b * d;
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) s += Db[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) lam[b] = (double)damp_rel * (two_over_n[b] * red[0] / (double)d);
}

// Stable descending order of D: rank(i) = #{j : D_j > D_i} + #{j < i : D_j == D_i};
// perm[rank(i)] = i.  Exact comparisons, so ties go to the lower index.  A
// workgroup takes 64 entries i (one per lane) and its four waves a quarter of
// the j range each (D_j a wave-uniform scalar load); the four partial counts
// meet in LDS.
__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ D, int d, int32_t* __restrict__ perm) {
  const int b = blockIdx.y;
  const double* Db = D + (size_t)b * d;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * 64 + lane;
  // NaN keys sort as -inf so the ranks always form a permutation
  double di = i < d ? Db[i] : 0.0;
  if (di != di) di = -HUGE_VAL;
  const int j0 = (int)((int64_t)d * w / 4), j1 = (int)((int64_t)d * (w + 1) / 4);
  int rank = 0;
#pragma unroll 8
  for (int j = j0; j < j1; ++j) {
    double v = Db[j];
    if (v != v) v = -HUGE_VAL;
    rank += (v > di) || (v == di && j < i);
  }
  __shared__ int part[4][64];
  part[w][lane] = rank;
  __syncthreads();
  if (w == 0 && i < d) perm[(size_t)b * d + part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane]] = i;
}

__global__ void iota_kernel(int32_t* p, int d, int batch) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)d * batch) p[i] = (int32_t)(i % d);
}

// F[x][y] = 2 S[max][min] / N as a full symmetric fp64 matrix, written through
// a 32x32 LDS tile so that both the lower-triangle reads and the writes are
// row-contiguous.  The diagonal comes from the fp64 D.
__global__ __launch_bounds__(256) void symmetrize_kernel(const float* __restrict__ S, const double* __restrict__ D,
                                                         int d, const double* __restrict__ two_over_n,
                                                         double* __restrict__ F) {
  const int b = blockIdx.z;
  const float* Sb = S + (size_t)b * d * d;
  double* Fb = F + (size_t)b * d * d;
  const double c = two_over_n[b];
  __shared__ float t[32][33];
  const int x0 = blockIdx.y * 32, y0 = blockIdx.x * 32;   // output block rows x0.., cols y0..
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  if (x0 >= y0) {
    // block on or below the diagonal: read S[x][y] directly (S[y][x] for the
    // few x < y entries of diagonal blocks)
    for (int r = ty; r < 32; r += 8) {
      int x = x0 + r, y = y0 + tx;
      if (x < d && y < d) {
        double v;
        if (x == y) v = c * D[(size_t)b * d + x];
        else if (x > y) v = c * (double)Sb[(size_t)x * d + y];
        else v = c * (double)Sb[(size_t)y * d + x];
        Fb[(size_t)x * d + y] = v;
      }
    }
  } else {
    // upper block: F[x][y] = S[y][x]; read S rows y (contiguous in x), transpose
    for (int r = ty; r < 32; r += 8) {
      int y = y0 + r, x = x0 + tx;
      t[r][tx] = (x < d && y < d) ? Sb[(size_t)y * d + x] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
      int x = x0 + r, y = y0 + tx;
      if (x < d && y < d) Fb[(size_t)x * d + y] = c * (double)t[tx][r];
    }
  }
}

// A[i][j] (i >= j) = F[p(d-1-i)][p(d-1-j)] + lambda (i == j): the damped,
// permuted, reversed Hessian.  For the identity order the read runs backwards
// along one row of F.
__global__ __launch_bounds__(256) void build_rev_kernel(const double* __restrict__ F, const int32_t* __restrict__ perm,
                                                        int d, const double* __restrict__ lam, double* __restrict__ A) {
  const int b = blockIdx.z;
  const double* Fb = F + (size_t)b * d * d;
  const int32_t* pb = perm ? perm + (size_t)b * d : nullptr;
  double* Ab = A + (size_t)b * d * d;
  const int i = blockIdx.y;
  const int x = pb ? pb[d - 1 - i] : d - 1 - i;
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= i && j < d; j += gridDim.x * 256) {
    const int y = pb ? pb[d - 1 - j] : d - 1 - j;
    double v = Fb[(size_t)x * d + y];
    if (i == j) v += lam[b];
    Ab[(size_t)i * d + j] = v;
  }
}

// Without a permutation: A[i][j] (i >= j) = 2 S[d-1-j][d-1-i] / N, the
// diagonal 2 D[d-1-i] / N + lambda, straight from the lower triangle of S
// (d-1-j >= d-1-i): a 32 x 32 tile of S read along its rows, turned in LDS and
// written along the rows of A, so both sides stay contiguous.  Tiles above the
// diagonal of A are not written (the factorization reads the lower triangle).
__global__ __launch_bounds__(256) void rev_lower_kernel(const float* __restrict__ S, const double* __restrict__ D,
                                                        int d, const double* __restrict__ two_over_n,
                                                        const double* __restrict__ lam, double* __restrict__ A) {
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  if (j0 > i0) return;
  const int b = blockIdx.z;
  const float* Sb = S + (size_t)b * d * d;
  double* Ab = A + (size_t)b * d * d;
  const double c = two_over_n[b];
  __shared__ float t[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  // source rows y = d-1-j for j in [j0, j0+32), columns x = d-1-i for i in [i0, i0+32)
  const int ys0 = d - 32 - j0, xs0 = d - 32 - i0;
  for (int r = ty; r < 32; r += 8) {
    const int y = ys0 + r, x = xs0 + tx;
    t[r][tx] = (y >= 0 && x >= 0 && x < y) ? Sb[(size_t)y * d + x] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + tx;
    if (i < d && j <= i) {
      double v;
      if (i == j) v = c * D[(size_t)b * d + (d - 1 - i)] + lam[b];
      else v = c * (double)t[31 - tx][31 - r];
      Ab[(size_t)i * d + j] = v;
    }
  }
}

// The same with the permutation: one workgroup per output row i copies row
// p(d-1-i) of F into LDS with coalesced loads and gathers its columns there
// (a gather straight from global memory touches a cache line per element).
// The row buffer holds kMaxD doubles (static LDS: 32, 64 or 128 KiB).
constexpr int kRevLdsMax = 16384;
template <int kMaxD>
__global__ __launch_bounds__(512) void build_rev_lds_kernel(const double* __restrict__ F,
                                                            const int32_t* __restrict__ perm, int d,
                                                            const double* __restrict__ lam, double* __restrict__ A) {
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) double rowv[kMaxD];
  const int b = blockIdx.z;
  const int32_t* pb = perm + (size_t)b * d;
  const int i = blockIdx.y;
  const double* src = F + (size_t)b * d * d + (size_t)pb[d - 1 - i] * d;
  if ((d & 1) == 0) {
    // 16-byte loads, four in flight per thread (rows of an even d start 16-byte aligned)
    const int n2 = d >> 1;
    int y = threadIdx.x;
    for (; y + 3 * 512 < n2; y += 4 * 512) {
      f64x2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = reinterpret_cast<const f64x2*>(src)[y + u * 512];
#pragma unroll
      for (int u = 0; u < 4; ++u) reinterpret_cast<f64x2*>(rowv)[y + u * 512] = v[u];
    }
    for (; y < n2; y += 512) reinterpret_cast<f64x2*>(rowv)[y] = reinterpret_cast<const f64x2*>(src)[y];
  } else {
    for (int y = threadIdx.x; y < d; y += 512) rowv[y] = src[y];
  }
  __syncthreads();
  double* dst = A + (size_t)b * d * d + (size_t)i * d;
  const double l = lam[b];
  for (int j = threadIdx.x; j <= i; j += 512) {
    double v = rowv[pb[d - 1 - j]];
    if (j == i) v += l;
    dst[j] = v;
  }
}

// ------------------------------------------------------------------ diagonal blocks in one workgroup
// A diagonal block of n <= 64 is factored recursively inside the workgroup:
// 64 = 32 + 32, 32 = 16 + 16.  A node (o, m) with halves m1 = m2 = m / 2
// factors its first half, forms L21 = A21 L11^-T, A22 -= L21 L21^T and
// T = L21 L11^-1, factors its second half and finishes L^-1 with
// (L^-1)21 = -L22^-1 T.  Only the inverse is kept: the factor of a block is
// not needed again.  The 16-column leaves and the 32-wide node run in wave 0
// alone, so their column steps need no workgroup barrier (the lanes of one
// wave exchange values through LDS, whose operations a wave issues in
// order); the 64-wide node's 32 x 32 x 32 products take all four waves, one
// 16 x 16 block each.  Every product is a chain of fp64 MFMAs
// (v_mfma_f64_16x16x4f64).
//
// Operands sit in LDS row-major in 64-double rows with their 16-byte chunks
// swizzled: element (r, k) at r * 64 + 2 ((k / 2) ^ (r % 32)) + k % 2.
// Sixteen lanes reading one k of sixteen rows, or sixteen k of one row, then
// touch distinct banks, and a row is still 512 contiguous bytes, so panels
// are copied global -> LDS by the DMA path (the swizzle goes into the global
// address).
//
// Leaf (16 columns, one wave): lane l keeps row r = l % 16 at columns
// c = l / 16 + 4 v (v < 4) of the block and of the eliminator X (unit lower
// triangular, X A = D L^T).  Step j publishes column j (its rows r > j after
// the earlier steps, pivot p_j on the diagonal) and row j of X through LDS;
// every lane then applies a[r][c] -= a[r][j] a[c][j] / p_j and
// x[r] -= (a[r][j] / p_j) x[j] for its rows below j.  With the pivots kept
// unscaled, L^-1 row r is x[r] / sqrt(p_r).  Entries right of the diagonal
// are never read: the published row of X is zero there, and the column
// values a lane reads for rows at or above j are multiplied by zero.
//
// 1/p and 1/sqrt(p): hardware estimates refined by two Newton steps each
// (y <- y (2 - p y) and y <- y (3 - p y^2) / 2; each squares the relative error).
__device__ __forceinline__ double rcp_nr(double x) {
  double y = __builtin_amdgcn_rcp(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(y, fma(-x, y, 1.0), y);
  return y;
}

__device__ __forceinline__ double rsqrt_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-x * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// The barrier orders LDS traffic only; the global stores need no wait.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Within one wave: keeps the compiler from moving LDS accesses across this
// point (the hardware runs a wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int bsw(int r, int k) { return r * 64 + ((((k >> 1) ^ (r & 31)) << 1) | (k & 1)); }

// Per-workgroup scratch of the recursion.
struct LeafShared {
  double col[16];    // leaf step: published column, at slot (c % 4) * 4 + c / 4
  double rowx[16];   // leaf step: published row of X, same slots
  double piv[64];    // pivots of the 64-block's columns
};

// 16 x 16 fp64 MFMA product of one wave: acc (+)= X Y with
// X[i][k] = Pa(ra + i, ca + k) and Y[k][j] = Pb(rb + j, cb + k) (kBT) or
// Pb(rb + k, cb + j), k < K.  D lane layout: rows lane / 16 + 4 e, column lane % 16.
template <bool kBT>
__device__ __forceinline__ void mm16(const double* Pa, int ra, int ca, const double* Pb, int rb, int cb, int K,
                                     f64x4& acc) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, kq = lane >> 4;
  for (int k4 = 0; k4 < K; k4 += 4) {
    const int k = k4 + kq;
    const double a = Pa[bsw(ra + i, ca + k)];
    const double b = kBT ? Pb[bsw(rb + i, cb + k)] : Pb[bsw(rb + k, cb + i)];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ int d_row(int e) { return ((threadIdx.x & 63) >> 4) + 4 * e; }
__device__ __forceinline__ int d_col() { return threadIdx.x & 15; }

// Leaf: the 16 x 16 diagonal block at (o, o) of the panel P (lower
// triangle; rows at or past n are taken as identity rows) -> its L^-1 into
// the panel Q at (o, o), zeros right of the diagonal; pivots into sh.piv.
// Wave 0 only.
__device__ __forceinline__ void leaf16(const double* P, double* Q, int o, int n, LeafShared& sh) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, cq = lane >> 4;
  double a[4], x[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = cq + 4 * v;
    double val = (r == c) ? 1.0 : 0.0;
    if (o + r < n && c <= r) val = P[bsw(o + r, o + c)];
    a[v] = val;
    x[v] = (r == c) ? 1.0 : 0.0;
  }
  double myp = 1.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    constexpr int dummy = 0;
    (void)dummy;
    const int vj = j >> 2, cj = j & 3;
    if (cq == cj) sh.col[(r & 3) * 4 + (r >> 2)] = a[vj];
    if (r == j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sh.rowx[cq * 4 + v] = x[v];
    }
    wave_lds_order();
    const double p = sh.col[cj * 4 + vj];
    const double cr = sh.col[(r & 3) * 4 + (r >> 2)];
    double ck[4], xr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ck[v] = sh.col[cq * 4 + v];
      xr[v] = sh.rowx[cq * 4 + v];
    }
    const double f = (r > j) ? cr * rcp_nr(p) : 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      a[v] = fma(-f, ck[v], a[v]);
      x[v] = fma(-f, xr[v], x[v]);
    }
    if (r == j) myp = p;
    wave_lds_order();
  }
  const double rs = rsqrt_nr(myp);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = cq + 4 * v;
    Q[bsw(o + r, o + c)] = c <= r ? x[v] * rs : 0.0;
  }
  if (cq == 0) sh.piv[o + r] = myp;
}

// The 32-wide node at (o, o): wave 0 only.  T16 is a 16 x 16 scratch block in
// swizzled rows (rows 0..15, columns tc..tc+15 of the panel Tp).
__device__ __forceinline__ void node32(double* P, double* Q, double* Tp, int tc, int o, int n, LeafShared& sh) {
  leaf16(P, Q, o, n, sh);
  wave_lds_order();
  // L21 = A21 Li11^T, over A21
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  mm16<true>(P, o + 16, o, Q, o, o, 16, acc);
  wave_lds_order();
#pragma unroll
  for (int e = 0; e < 4; ++e) P[bsw(o + 16 + d_row(e), o + d_col())] = acc[e];
  wave_lds_order();
  // A22 -= L21 L21^T, T = L21 Li11
  f64x4 up = {0.0, 0.0, 0.0, 0.0}, t = {0.0, 0.0, 0.0, 0.0};
  mm16<true>(P, o + 16, o, P, o + 16, o, 16, up);
  mm16<false>(P, o + 16, o, Q, o, o, 16, t);
  wave_lds_order();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    P[bsw(o + 16 + d_row(e), o + 16 + d_col())] -= up[e];
    Tp[bsw(d_row(e), tc + d_col())] = t[e];
  }
  wave_lds_order();
  leaf16(P, Q, o + 16, n, sh);
  wave_lds_order();
  // (L^-1)21 = -Li22 T
  f64x4 li = {0.0, 0.0, 0.0, 0.0};
  mm16<false>(Q, o + 16, o + 16, Tp, 0, tc, 16, li);
  wave_lds_order();
#pragma unroll
  for (int e = 0; e < 4; ++e) Q[bsw(o + 16 + d_row(e), o + d_col())] = -li[e];
  wave_lds_order();
}

// The 16 x 16 blocks of a panel right of the block diagonal: zero.  No leaf
// or node writes them, so a panel that serves several 64-blocks in turn is
// cleared once.
__device__ __forceinline__ void zero_upper_blocks(double* Q) {
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) Q[bsw(r, c)] = 0.0;
  }
}

// A 64-block (rows at or past n taken as identity) whose lower triangle is in
// the swizzled panel P (overwritten) -> its L^-1 in the panel Q, zeros right
// of the diagonal (the caller has cleared Q's upper blocks and synchronized).
// Tp: a swizzled 32-row scratch panel.  All 256 threads; returns the first
// column whose pivot is not positive (NaN included), or -1.
__device__ __forceinline__ int leaf64(double* P, double* Q, double* Tp, int n, LeafShared& sh) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  if (wave == 0) node32(P, Q, Tp, 32, 0, n, sh);
  __syncthreads();
  // the 64-node's products: wave w owns the 16 x 16 block (w / 2, w % 2) of
  // each 32 x 32 result
  const int bi = wave >> 1, bj = wave & 1;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  mm16<true>(P, 32 + 16 * bi, 0, Q, 16 * bj, 0, 32, acc);   // L21 = A21 Li11^T
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) P[bsw(32 + 16 * bi + d_row(e), 16 * bj + d_col())] = acc[e];
  __syncthreads();
  f64x4 up = {0.0, 0.0, 0.0, 0.0}, t = {0.0, 0.0, 0.0, 0.0};
  if (bi >= bj) mm16<true>(P, 32 + 16 * bi, 0, P, 32 + 16 * bj, 0, 32, up);   // A22 -= L21 L21^T
  mm16<false>(P, 32 + 16 * bi, 0, Q, 0, 16 * bj, 32, t);                      // T = L21 Li11
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (bi >= bj) P[bsw(32 + 16 * bi + d_row(e), 32 + 16 * bj + d_col())] -= up[e];
    Tp[bsw(16 * bi + d_row(e), 16 * bj + d_col())] = t[e];
  }
  __syncthreads();
  if (wave == 0) node32(P, Q, Tp, 32, 32, n, sh);
  __syncthreads();
  f64x4 li = {0.0, 0.0, 0.0, 0.0};
  mm16<false>(Q, 32 + 16 * bi, 32, Tp, 0, 16 * bj, 32, li);   // (L^-1)21 = -Li22 T
#pragma unroll
  for (int e = 0; e < 4; ++e) Q[bsw(32 + 16 * bi + d_row(e), 16 * bj + d_col())] = -li[e];
  __syncthreads();
  // the first pivot that is not positive (NaN included) names the failing column
  const unsigned long long bad = __ballot((tid & 63) < n && !(sh.piv[tid & 63] > 0.0));
  return bad != 0ull ? __ffsll((long long)bad) - 1 : -1;
}

// rows [0, 64) of a 64-column block at src (row stride d) into a swizzled
// panel, two rows per 1 KiB direct load; rows at or past `rows` read as
// zeros.  The last row's 64 doubles may run past the end of the matrix when
// the block is the last one (a ragged d); the workspace holds more buffers
// after it, and those columns are never used.
__device__ __forceinline__ void dma_panel(const double* src, int d, int rows, double* panel) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src, (short)0, (int)(((int64_t)(rows - 1) * d + 64) * 8), 0x00020000);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int pair = q * 4 + wave;                  // rows 2 pair, 2 pair + 1
    const int r = 2 * pair + (lane >> 5);
    const int c = (lane & 31) ^ (r & 31);            // the global chunk held by slot lane % 32
    const uint32_t vo = (uint32_t)(((int64_t)r * d + 2 * c) * 8);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(panel + pair * 128), 16,
                                             vo, 0, 0, 0);
  }
}

// rows [0, n) and columns [0, min(n, 64)) of the lower triangle of a swizzled
// panel -> global (row stride d); with lower, entries right of the diagonal
// are skipped.
__device__ __forceinline__ void store_panel(const double* Q, double* dst, int d, int rows, int cols, bool lower) {
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    if (r < rows && c < cols && (!lower || c <= r)) dst[(size_t)r * d + c] = Q[bsw(r, c)];
  }
}

struct BlockShared {
  double p[4][64 * 64];   // panels: 0 A21 then L21; 1 A22; 2 L^-1 of a 64-block; 3 A11 then T
  double t[32 * 64];      // 32 swizzled rows of scratch for the 64-blocks' recursion
  LeafShared leaf;
};

__global__ __launch_bounds__(256) void leaf_kernel(const double* __restrict__ A, double* __restrict__ Li, int d,
                                                   int o, int n, int32_t* __restrict__ info) {
  const int b = blockIdx.z;
  const size_t off = (size_t)b * d * d + (size_t)o * d + o;
  __shared__ __attribute__((aligned(1024))) double P[64 * 64];
  __shared__ __attribute__((aligned(1024))) double Q[64 * 64];
  __shared__ __attribute__((aligned(1024))) double Tp[32 * 64];
  __shared__ LeafShared sh;
  dma_panel(A + off, d, n, P);
  zero_upper_blocks(Q);
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads have landed
  __syncthreads();
  const int fail = leaf64(P, Q, Tp, n, sh);
  store_panel(Q, Li + off, d, n, n, true);
  if (threadIdx.x == 0 && fail >= 0 && info[b] == 0) info[b] = (d - 1 - (o + fail)) + 1;
}

// acc (+)= A B for this wave's 32 x 32 quadrant of a 64 x 64 product,
// A[i][k] = Pa(i, k) and B[k][j] = Pb(j, k) (kBT) or Pb(k, j)
// The fragments of step k4 + 1 are read while the four MFMAs of step k4 run.
template <bool kBT>
__device__ __forceinline__ void mm64(const double* Pa, const double* Pb, f64x4 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  double av[2][2], bv[2][2];
  auto frag = [&](int k4, int set) {
    const int kr = 4 * k4 + (lane >> 4);
#pragma unroll
    for (int u = 0; u < 2; ++u) av[set][u] = Pa[bsw(wm + 16 * u + (lane & 15), kr)];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int j = wn + 16 * v + (lane & 15);
      bv[set][v] = kBT ? Pb[bsw(j, kr)] : Pb[bsw(kr, j)];
    }
  };
  frag(0, 0);
#pragma unroll
  for (int k4 = 0; k4 < 16; ++k4) {
    if (k4 + 1 < 16) frag(k4 + 1, (k4 + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v)
        acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[k4 & 1][u], bv[k4 & 1][v], acc[u][v], 0, 0, 0);
  }
}

// element e of block (u, v) of this wave's quadrant: row, column
__device__ __forceinline__ int q_row(int u, int e) {
  return ((threadIdx.x >> 6) >> 1) * 32 + 16 * u + ((threadIdx.x & 63) >> 4) + 4 * e;
}
__device__ __forceinline__ int q_col(int v) { return ((threadIdx.x >> 6) & 1) * 32 + 16 * v + (threadIdx.x & 15); }

__device__ __forceinline__ void zero_acc(f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// ------------------------------------------------------------------ block of 65..128 in one workgroup
// The two-level step of the recursion (n1 = 64, n2 = n - 64) without leaving
// the workgroup: L11^-1 by leaf64, L21 = A21 L11^-T, A22 -= L21 L21^T,
// T = L21 L11^-1, L22^-1 by leaf64, (L^-1)21 = -L22^-1 T.  The products are
// 64x64x64 on fp64 MFMA, each wave one 32x32 quadrant.  A11, A21 and A22 are
// copied global -> LDS by the DMA path at the start.
__global__ __launch_bounds__(256) void block128_kernel(const double* __restrict__ A, double* __restrict__ Li, int d,
                                                       int o, int n, int32_t* __restrict__ info) {
  const int b = blockIdx.z;
  const int n2 = n - 64;
  const double* Ab = A + (size_t)b * d * d;
  double* Lb = Li + (size_t)b * d * d;
  __shared__ __attribute__((aligned(1024))) BlockShared sh;
  double* P0 = sh.p[0];
  double* P1 = sh.p[1];
  double* P2 = sh.p[2];
  double* P3 = sh.p[3];

  dma_panel(Ab + (size_t)o * d + o, d, 64, P3);               // A11
  dma_panel(Ab + (size_t)(o + 64) * d + o, d, n2, P0);        // A21
  dma_panel(Ab + (size_t)(o + 64) * d + o + 64, d, n2, P1);   // A22
  zero_upper_blocks(P2);
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads have landed
  __syncthreads();

  const int fail1 = leaf64(P3, P2, sh.t, 64, sh.leaf);
  store_panel(P2, Lb + (size_t)o * d + o, d, 64, 64, true);

  // L21 = A21 Li11^T, written over A21
  f64x4 acc[2][2];
  zero_acc(acc);
  mm64<true>(P0, P2, acc);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) P0[bsw(q_row(u, e), q_col(v))] = acc[u][v][e];
  __syncthreads();

  // A22 -= L21 L21^T (the upper-right quadrant is not needed), T = L21 Li11
  // (over A11, which the first leaf has consumed)
  {
    const int tid = threadIdx.x;
    f64x4 up[2][2];
    zero_acc(up);
    zero_acc(acc);
    if ((tid >> 6) != 1) mm64<true>(P0, P0, up);
    mm64<false>(P0, P2, acc);
    if ((tid >> 6) != 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = q_row(u, e), j = q_col(v);
            if (j <= i) P1[bsw(i, j)] -= up[u][v][e];
          }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) P3[bsw(q_row(u, e), q_col(v))] = acc[u][v][e];
  }
  __syncthreads();

  // L22^-1 over L11^-1 (stored, and last read by the products above)
  const int fail2 = leaf64(P1, P2, sh.t, n2, sh.leaf);
  store_panel(P2, Lb + (size_t)(o + 64) * d + o + 64, d, n2, n2, true);

  // (L^-1)21 = -Li22 T
  zero_acc(acc);
  mm64<false>(P2, P3, acc);
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = q_row(u, e);
        if (i < n2) Lb[(size_t)(o + 64 + i) * d + o + q_col(v)] = -acc[u][v][e];
      }
  if (threadIdx.x == 0 && info[b] == 0) {
    if (fail1 >= 0) info[b] = (d - 1 - (o + fail1)) + 1;
    else if (fail2 >= 0) info[b] = (d - 1 - (o + 64 + fail2)) + 1;
  }
}

// ------------------------------------------------------------------ fp64 GEMM
// C = beta C + alpha op(A) op(B) on kT x kT workgroup tiles with fp64 MFMA
// (v_mfma_f64_16x16x4f64); each of the 4 waves owns a (kT/2) x (kT/2) quarter
// of 16x16 blocks.  op(A) = A (M x K, row-major); op(B) = B (K x N) or, with
// kTB, B^T for B N x K.  kmode: 0 full; 1 A lower (A[i][k] = 0 for k > i);
// 2 B lower, not transposed (B[k][j] = 0 for k < j); 3 B lower, transposed
// (B[j][k] = 0 for k > j).  Zero entries are masked when staged into LDS, so the
// unused triangles may hold anything; with lower_out only i >= j of C is
// written.  beta == 0 never reads C.  kT = 32 and 64 serve the many small
// products of the recursion, kT = 128 the large ones (half the L2 traffic per
// flop of kT = 64).
struct GemmArgs {
  int M, N, K;
  double alpha, beta;
  const double* A;
  int64_t lda, sA;   // sA: batch stride
  const double* B;
  int64_t ldb, sB;
  double* C;
  int64_t ldc, sC;
  int kmode;
  int lower_out;
  int tb;            // op(B) = B^T
};

// One launch may carry two independent products: tiles [0, tiles0) belong to
// g[0], the rest to g[1].
struct GemmPair {
  GemmArgs g[2];
  int tiles0;
  int tiles;   // tiles of both products; a workgroup takes tiles blockIdx.x, + gridDim.x, ...
};

// Tile order: the launch enumerates only the tiles that do work, longest
// first, so the short triangular tiles fill the tail.  lower_out: the lower
// triangle of tiles (uniform K); kmode 1: rows by decreasing i (K ends at the
// row); kmode 3: columns by decreasing j (K ends at the column); otherwise
// columns by increasing j (kmode 2: K starts at the column).
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int kT, int t, int& ti, int& tj) {
  const int mt = (g.M + kT - 1) / kT, nt = (g.N + kT - 1) / kT;
  if (g.lower_out) {
    int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    ti = r;
    tj = t - r * (r + 1) / 2;
  } else if (g.kmode == 1) {
    ti = mt - 1 - t / nt;
    tj = t % nt;
  } else if (g.kmode == 3) {
    tj = nt - 1 - t / mt;
    ti = t % mt;
  } else {
    tj = t / mt;
    ti = t % mt;
  }
}

// kT x kT tile, kW waves: the waves split the tile into 2 columns of
// (kW / 2) row groups, each wave an (2 kT / kW) x (kT / 2) block of 16x16
// MFMA blocks.  kT = 128 and 64 run 8 waves so that one workgroup alone keeps
// two waves on every SIMD (an fp64 MFMA stream needs two to issue at full rate).
// kTBMode: 0 op(B) = B, 1 op(B) = B^T for every tile, 2 per product (g.tb).
// kVec: every run of 8 operand elements along a row is wholly inside or
// outside the live range and 16-byte aligned, so a thread's kE elements load
// as 16-byte pairs; otherwise one element at a time.  kE: elements per thread
// per operand and stage (8, or 4 for half the LDS and so two workgroups of
// 128 x 128 or 64 x 64 on a CU).
template <int kT, int kW, int kTBMode, bool kVec, int kE = 8>
__global__ __launch_bounds__(64 * kW) void dgemm_kernel(GemmPair pair) {
  constexpr int kThreads = 64 * kW;
  constexpr int kGK = kE * kThreads / kT;   // K per LDS stage
  constexpr int kWM = 2 * kT / kW;          // rows per wave
  constexpr int kWN = kT / 2;               // columns per wave
  constexpr int kBM = kWM / 16, kBN = kWN / 16;
  constexpr int kAR = kGK / kE;             // threads per row of a K-contiguous operand
  constexpr int kBR = kT / kE;              // threads per K-row of a row-major B
  // As[k][m], Bs[k][n]: k-major so a 16-lane MFMA fragment is 16 consecutive doubles
  __shared__ double As[2][kGK][kT + 2];
  __shared__ double Bs[2][kGK][kT + 2];
  // one tile per workgroup, or several in turn when the grid was capped (every
  // tile's K loop ends at a barrier after its last LDS read, so the next
  // tile's first stage may overwrite the buffers)
  for (int wt = blockIdx.x; wt < pair.tiles; wt += gridDim.x) {
    const bool second = wt >= pair.tiles0;
    const GemmArgs g = second ? pair.g[1] : pair.g[0];   // a copy: its fields stay in registers
    const bool kTB = kTBMode == 2 ? g.tb != 0 : kTBMode == 1;
    const int b = blockIdx.z;
    int ti, tj;
    gemm_tile(g, kT, second ? wt - pair.tiles0 : wt, ti, tj);
    const int i0 = ti * kT, j0 = tj * kT;
    const double* A = g.A + (size_t)b * g.sA;
    const double* B = g.B + (size_t)b * g.sB;
    double* C = g.C + (size_t)b * g.sC;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = (wave >> 1) * kWM, wn = (wave & 1) * kWN;
    int kb = 0, ke = g.K;
    if (g.kmode == 1) ke = min(g.K, i0 + kT);
    if (g.kmode == 2) kb = (j0 / kGK) * kGK;
    if (g.kmode == 3) ke = min(g.K, j0 + kT);

    f64x4 acc[kBM][kBN];
#pragma unroll
    for (int u = 0; u < kBM; ++u)
#pragma unroll
      for (int v = 0; v < kBN; ++v) acc[u][v] = f64x4{0.0, 0.0, 0.0, 0.0};

    // staging: kT x kGK doubles per operand = kE per thread
    double ra[kE], rb[kE];
    const int rA = tid / kAR, kA = (tid % kAR) * kE;   // K-contiguous operand: row, first k
    const int kBk = tid / kBR, cB = (tid % kBR) * kE;  // row-major B: k, first column
    // Loads never branch: indices are clamped into the operands, and rows,
    // columns and k outside the live range, and the zero triangles, are masked
    // when a stage is written to LDS.  So the loads of the next stage stay in
    // flight through the MFMA work of the current one.
    typedef double f64x2 __attribute__((ext_vector_type(2)));
    auto ld8 = [&](const double* row, int c0, int cmax, double (&r)[kE]) {
      if constexpr (kVec) {
        const f64x2* p = reinterpret_cast<const f64x2*>(row + (c0 <= cmax ? c0 : 0));
#pragma unroll
        for (int q = 0; q < kE / 2; ++q) {
          const f64x2 v = p[q];
          r[2 * q] = v.x;
          r[2 * q + 1] = v.y;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kE; ++u) r[u] = row[min(c0 + u, cmax)];
      }
    };
    auto load_stage = [&](int k0) {
      ld8(A + (size_t)min(i0 + rA, g.M - 1) * g.lda, k0 + kA, g.K - 1, ra);
      if (kTB) ld8(B + (size_t)min(j0 + rA, g.N - 1) * g.ldb, k0 + kA, g.K - 1, rb);
      else ld8(B + (size_t)min(k0 + kBk, g.K - 1) * g.ldb, j0 + cB, g.N - 1, rb);
    };
    // the masks: one test per kE-element run where kVec guarantees the run is
    // wholly live or dead, per element otherwise; the triangle test only for
    // the products that have one (a branch on a kernel argument)
    const bool rowA = i0 + rA < g.M;
    const bool rowB = kTB ? j0 + rA < g.N : true;
    auto put8 = [&](double* dst, int stride, const double (&r)[kE], bool run_live, int first, int lim, bool has_tri,
                    int tri) {
      // element u is live when run_live, first + u < lim (implied under kVec)
      // and, for a product with a zero triangle, first + u <= tri
      if (has_tri) {
#pragma unroll
        for (int u = 0; u < kE; ++u) {
          const bool live = run_live && (kVec || first + u < lim) && first + u <= tri;
          dst[u * stride] = live ? r[u] : 0.0;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kE; ++u) {
          const bool live = run_live && (kVec || first + u < lim);
          dst[u * stride] = live ? r[u] : 0.0;
        }
      }
    };
    auto store_stage = [&](int buf, int k0) {
      const int gk0 = k0 + kA;
      const bool runA = rowA && (!kVec || gk0 < ke);
      put8(&As[buf][kA][rA], kT + 2, ra, runA, gk0, ke, g.kmode == 1, i0 + rA);
      if (kTB) {
        const bool runB = rowB && (!kVec || gk0 < ke);
        put8(&Bs[buf][kA][rA], kT + 2, rb, runB, gk0, ke, g.kmode == 3, j0 + rA);
      } else {
        const int gk = k0 + kBk, gj0 = j0 + cB;
        const bool runB = gk < ke && (!kVec || gj0 < g.N);
        put8(&Bs[buf][kBk][cB], 1, rb, runB, gj0, g.N, g.kmode == 2, gk);
      }
    };
    int buf = 0;
    if (kb < ke) {
      load_stage(kb);
      store_stage(0, kb);
      if (kb + kGK < ke) load_stage(kb + kGK);
      __syncthreads();
    }
    for (int k0 = kb; k0 < ke; k0 += kGK) {
      // the fragments of step k4 + 1 are read while the MFMAs of step k4 run
      double av[2][kBM], bv[2][kBN];
      auto frag = [&](int k4, int set) {
        const int kr = k4 * 4 + (lane >> 4);
#pragma unroll
        for (int u = 0; u < kBM; ++u) av[set][u] = As[buf][kr][wm + u * 16 + (lane & 15)];
#pragma unroll
        for (int v = 0; v < kBN; ++v) bv[set][v] = Bs[buf][kr][wn + v * 16 + (lane & 15)];
      };
      frag(0, 0);
#pragma unroll
      for (int k4 = 0; k4 < kGK / 4; ++k4) {
        if (k4 + 1 < kGK / 4) frag(k4 + 1, (k4 + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of the MFMAs
#pragma unroll
        for (int u = 0; u < kBM; ++u)
#pragma unroll
          for (int v = 0; v < kBN; ++v)
            acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[k4 & 1][u], bv[k4 & 1][v], acc[u][v], 0, 0, 0);
      }
      if (k0 + kGK < ke) {
        store_stage(buf ^ 1, k0 + kGK);
        if (k0 + 2 * kGK < ke) load_stage(k0 + 2 * kGK);
      }
      __syncthreads();
      buf ^= 1;
    }
    // D layout of a 16x16 fp64 MFMA: lane l holds rows l / 16 + 4 e, column l % 16
#pragma unroll
    for (int u = 0; u < kBM; ++u)
#pragma unroll
      for (int v = 0; v < kBN; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = i0 + wm + u * 16 + (lane >> 4) + 4 * e;
          const int gj = j0 + wn + v * 16 + (lane & 15);
          if (gi >= g.M || gj >= g.N) continue;
          if (g.lower_out && gj > gi) continue;
          double* p = C + (size_t)gi * g.ldc + gj;
          double r = g.alpha * acc[u][v][e];
          if (g.beta != 0.0) r += g.beta * *p;
          *p = r;
        }
  }
}

// U[a][c] = Linv[d-1-a][d-1-c] for a <= c, 0 below the diagonal (fp32).
__global__ __launch_bounds__(256) void write_u_kernel(const double* __restrict__ Li, int d, float* __restrict__ U) {
  const int b = blockIdx.z;
  const double* Lb = Li + (size_t)b * d * d;
  float* Ub = U + (size_t)b * d * d;
  const int a = blockIdx.y;
  for (int c = blockIdx.x * 256 + threadIdx.x; c < d; c += gridDim.x * 256) {
    float v = 0.f;
    if (c >= a) v = (float)Lb[(size_t)(d - 1 - a) * d + (d - 1 - c)];
    Ub[(size_t)a * d + c] = v;
  }
}

// ------------------------------------------------------------------ host
namespace {

// Scratch T: every node on a chain of second children holds its n2 x n1 block
// at once; n2 n1 <= n^2 / 4 + 32 n with n halving down the chain, so the sum
// stays below d^2 / 3 + 64 d per batch entry (rounded up to 256 bytes so
// every entry's blocks keep the 16-byte alignment of the first).
inline int64_t t_stride(int64_t d) { return (d * d / 3 + 64 * d + 31) / 32 * 32; }

// A second stream per device for the products that are off the Cholesky
// chain, and the events that order it against the caller's stream.  One
// factorization at a time enqueues on it (the mutex); default priority.
struct SideStream {
  hipStream_t s = nullptr;
  std::vector<hipEvent_t> ev;
  size_t next = 0;
};
std::mutex g_side_mu;
std::unordered_map<int, SideStream> g_side;

struct FactorCtx {
  double* A;
  double* Li;
  double* T;
  int d;
  int batch;
  int32_t* info;
  hipStream_t stream;   // the caller's stream: the chain of diagonal blocks
  SideStream* side;     // products the chain does not wait for
};

// Next event of the pool (created on first use, reused by later calls: a wait
// takes the record that precedes it, so re-recording is safe).
hipEvent_t side_event(const FactorCtx& c) {
  SideStream& ss = *c.side;
  if (ss.next == ss.ev.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    ss.ev.push_back(e);
  }
  return ss.ev[ss.next++];
}

// Work enqueued on `to` after this waits for everything enqueued on `from` so far.
gptq_status stream_order(const FactorCtx& c, hipStream_t from, hipStream_t to) {
  hipEvent_t e = side_event(c);
  if (!e) return GPTQ_EHIP;
  GQ_HIP(hipEventRecord(e, from));
  GQ_HIP(hipStreamWaitEvent(to, e, 0));
  return GPTQ_OK;
}

GemmArgs gemm_args(bool tb, int M, int N, int K, double alpha, const double* A, int64_t lda, const double* B,
                   int64_t ldb, double beta, double* C, int64_t ldc, int kmode, int lower_out, int64_t sA, int64_t sB,
                   int64_t sC) {
  return GemmArgs{M, N, K, alpha, beta, A, lda, sA, B, ldb, sB, C, ldc, sC, kmode, lower_out, tb ? 1 : 0};
}

int64_t gemm_tiles(const GemmArgs& g, int kT) {
  if (g.M <= 0 || g.N <= 0) return 0;
  return g.lower_out ? cdiv(g.M, kT) * (cdiv(g.M, kT) + 1) / 2 : cdiv(g.M, kT) * cdiv(g.N, kT);
}

// Whether every 8-element run a thread loads is 16-byte aligned and wholly
// inside or outside the live k (and, for a row-major B, column) range.
bool vec_ok(const GemmArgs& g) {
  const auto al = [](const double* p, int64_t ld) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && ld % 2 == 0; };
  return g.K % 8 == 0 && (g.tb || g.N % 8 == 0) && al(g.A, g.lda) && al(g.B, g.ldb) && g.sA % 2 == 0 && g.sB % 2 == 0;
}

// Launch one product, or two independent ones together.  Large launches take
// 128 x 128 tiles (8 waves) once that gives every CU two of them; then 64 x 64
// tiles, whose larger count evens out the triangular products' tiles of
// unequal K, while that gives every CU one; the small products near the
// leaves 32 x 32 tiles (4 waves of one 16 x 16 block), so that more CUs share
// their latency-bound K loops.  The 64 x 64 tiles run 8 waves of 16 x 32, so
// that a CU holding one of them (the products of 1024 columns) still has two
// waves on every SIMD; with 4 waves of 32 x 32 the 1024-column levels and the
// factor of d = 8192 took about 4% longer (measured on d = 2048 to 11008).
gptq_status gemm_launch(const FactorCtx& c, hipStream_t st, const GemmArgs& g0, const GemmArgs* g1,
                        int max_wg = 0) {
  for (const GemmArgs* g : {&g0, g1})
    if (g && g->lower_out && g->M != g->N) return GPTQ_EINVAL;   // the lower triangle of a square product
  GemmPair pair;
  pair.g[0] = g0;
  pair.g[1] = g1 ? *g1 : g0;
  const int64_t big = gemm_tiles(g0, 128) + (g1 ? gemm_tiles(*g1, 128) : 0);
  const int64_t mid = gemm_tiles(g0, 64) + (g1 ? gemm_tiles(*g1, 64) : 0);
  const int kT = big * c.batch >= 512 ? 128 : mid * c.batch >= 256 ? 64 : 32;
  if (g1 && kT == 128) {
    // large products fill the GPU on their own: launch each with its B layout fixed
    gptq_status s = gemm_launch(c, st, g0, nullptr, max_wg);
    return s != GPTQ_OK ? s : gemm_launch(c, st, *g1, nullptr, max_wg);
  }
  const int64_t t0 = gemm_tiles(g0, kT);
  const int64_t tiles = t0 + (g1 ? gemm_tiles(*g1, kT) : 0);
  if (tiles == 0) return GPTQ_OK;
  pair.tiles0 = (int)t0;
  pair.tiles = (int)tiles;
  int64_t gx = tiles;
  if (max_wg > 0) gx = std::max<int64_t>(1, std::min<int64_t>(tiles, max_wg / c.batch));
  dim3 grid((unsigned)gx, 1, (unsigned)c.batch);
  bool vec = true;
  for (const GemmArgs* g : {&g0, g1})
    if (g) vec = vec && vec_ok(*g);
  // 128 and 64 tiles stage 4 doubles per thread: half the LDS of 8, so two
  // workgroups share a CU and hide each other's barriers
#define GQ_GEMM(T, W, TB)                                                                                 \
  do {                                                                                                    \
    constexpr int kE = T == 32 ? 8 : 4;                                                                   \
    if (vec) hipLaunchKernelGGL((dgemm_kernel<T, W, TB, true, kE>), grid, dim3(64 * W), 0, st, pair); \
    else hipLaunchKernelGGL((dgemm_kernel<T, W, TB, false, kE>), grid, dim3(64 * W), 0, st, pair);    \
  } while (0)
  if (kT == 32) {
    if (g1) GQ_GEMM(32, 4, 2);
    else if (g0.tb) GQ_GEMM(32, 4, 1);
    else GQ_GEMM(32, 4, 0);
  } else if (kT == 64) {
    if (g1) GQ_GEMM(64, 8, 2);
    else if (g0.tb) GQ_GEMM(64, 8, 1);
    else GQ_GEMM(64, 8, 0);
  } else if (g0.tb) GQ_GEMM(128, 8, 1);
  else GQ_GEMM(128, 8, 0);
#undef GQ_GEMM
  GQ_LAUNCHED();
  return GPTQ_OK;
}

// Factor the diagonal block at offset o of size n: L into A, L^-1 into Li.
// T is this node's scratch for L21 L11^-1; the second child, which runs while
// it is live, gets the scratch after it.
//
// The chain the next diagonal block waits for is: the first child, L21, the
// update of A22, the second child.  T = L21 L11^-1 is needed only by the
// node's last product, (L^-1)21 = -L22^-1 T.  At the root, T runs on the side
// stream beside the whole second half of the chain (after the update, which
// gets the whole GPU), on at most kSideWG workgroups so that the chain's
// diagonal blocks, which need a whole CU's LDS, still find free CUs; the last
// product waits for it.  (The last product itself cannot leave the chain:
// the parent's L21 needs it when the node is a first child, and when it is a
// second child every later product of the chain waits for it through an
// ancestor's last product.)  Inner nodes keep T on the chain: the side stream
// is one in-order queue, so an inner T queued behind the root's would hold
// up the inner node's last product, and an uncapped T makes the next
// diagonal block wait for its last tiles (both measured on d = 11008).  An
// event also holds the chain for several microseconds, so the split pays
// only for roots of at least kSideMin columns.
constexpr int kSideMin = 2048;
// A side-stream product runs on at most this many workgroups (each takes its
// tiles in turn), so CUs stay free for the chain: a diagonal block kernel
// needs a whole CU's LDS and otherwise waits for the product's last tiles
// (measured on d = 11008 with uncapped products: 350-870 us instead of 45 us).
constexpr int kSideWG = 192;
gptq_status rec(const FactorCtx& c, int o, int n, double* T, bool root = false) {
  const int d = c.d;
  const int64_t dd = (int64_t)d * d;
  const int64_t sT = t_stride(d);
  if (n <= kLeaf) {
    hipLaunchKernelGGL(leaf_kernel, dim3(1, 1, c.batch), dim3(256), 0, c.stream, c.A, c.Li, d, o, n, c.info);
    GQ_LAUNCHED();
    return GPTQ_OK;
  }
  if (n <= 2 * kLeaf) {
    hipLaunchKernelGGL(block128_kernel, dim3(1, 1, c.batch), dim3(256), 0, c.stream, c.A, c.Li, d, o, n, c.info);
    GQ_LAUNCHED();
    return GPTQ_OK;
  }
  // the first child a multiple of the 128-column block, so every leaf but the
  // last one of a ragged d is a whole 128-block (n1 * n2 <= n^2 / 4 as before)
  const int n1 = (int)(cdiv(cdiv(n, 2), 2 * kLeaf) * 2 * kLeaf);
  const int n2 = n - n1;
  gptq_status s = rec(c, o, n1, T);
  if (s != GPTQ_OK) return s;
  double* A21 = c.A + (size_t)(o + n1) * d + o;
  double* A22 = c.A + (size_t)(o + n1) * d + (o + n1);
  double* Li11 = c.Li + (size_t)o * d + o;
  double* Li21 = c.Li + (size_t)(o + n1) * d + o;
  double* Li22 = c.Li + (size_t)(o + n1) * d + (o + n1);
  const hipStream_t side = c.side->s;
  // L21 = A21 Li11^T, parked in the Li21 slot
  s = gemm_launch(c, c.stream, gemm_args(true, n2, n1, n1, 1.0, A21, d, Li11, d, 0.0, Li21, d, 3, 0, dd, dd, dd),
                  nullptr);
  if (s != GPTQ_OK) return s;
  if (!root || n < kSideMin) {
    // everything on the chain; the update and T share one launch
    const GemmArgs upd = gemm_args(true, n2, n2, n1, -1.0, Li21, d, Li21, d, 1.0, A22, d, 0, 1, dd, dd, dd);
    const GemmArgs tprod = gemm_args(false, n2, n1, n1, 1.0, Li21, d, Li11, d, 0.0, T, n1, 2, 0, dd, dd, sT);
    s = gemm_launch(c, c.stream, upd, &tprod);
    if (s != GPTQ_OK) return s;
    s = rec(c, o + n1, n2, T + (size_t)n2 * n1);
    if (s != GPTQ_OK) return s;
    return gemm_launch(c, c.stream,
                       gemm_args(false, n2, n1, n2, -1.0, Li22, d, T, n1, 0.0, Li21, d, 1, 0, dd, sT, dd), nullptr);
  }
  // A22 -= L21 L21^T (lower half) on the chain with the whole GPU, then
  // T = L21 Li11 beside the second child's blocks
  s = gemm_launch(c, c.stream, gemm_args(true, n2, n2, n1, -1.0, Li21, d, Li21, d, 1.0, A22, d, 0, 1, dd, dd, dd),
                  nullptr);
  if (s != GPTQ_OK) return s;
  s = stream_order(c, c.stream, side);
  if (s != GPTQ_OK) return s;
  s = gemm_launch(c, side, gemm_args(false, n2, n1, n1, 1.0, Li21, d, Li11, d, 0.0, T, n1, 2, 0, dd, dd, sT),
                  nullptr, kSideWG);
  if (s != GPTQ_OK) return s;
  s = rec(c, o + n1, n2, T + (size_t)n2 * n1);
  if (s != GPTQ_OK) return s;
  // Li21 = -Li22 T, after T
  s = stream_order(c, side, c.stream);
  if (s != GPTQ_OK) return s;
  return gemm_launch(c, c.stream,
                     gemm_args(false, n2, n1, n2, -1.0, Li22, d, T, n1, 0.0, Li21, d, 1, 0, dd, sT, dd), nullptr);
}

}  // namespace

size_t prepare_workspace_bytes(int64_t d, int64_t batch) {
  size_t dd = (size_t)d * d;
  size_t bytes = 0;
  bytes += align_up(batch * dd * sizeof(double), 256);               // A
  bytes += align_up(batch * dd * sizeof(double), 256);               // Li (first F)
  bytes += align_up(batch * t_stride(d) * sizeof(double), 256);      // T
  bytes += align_up(batch * d * sizeof(int32_t), 256);               // perm copy
  bytes += align_up(batch * 2 * sizeof(double), 256);               // lambda, 2/N
  return bytes + 256;
}

}  // namespace gq

using namespace gq;

bool gq_params_ok(const gptq_params* p, int64_t d_in) {
  if (!p) return false;
  if (p->bits < 2 || p->bits > 8) return false;
  if (p->block_size != kQBlock) return false;
  const int g = p->group_size;
  if (g < 4 || d_in % g != 0) return false;
  if (g % kQBlock != 0 && kQBlock % g != 0) return false;
  if (!(p->damp_rel >= 0.0f) || !std::isfinite(p->damp_rel)) return false;
  if (p->sym != 0 && p->sym != 1) return false;
  if (p->static_groups != 0 && p->static_groups != 1) return false;
  return true;
}

extern "C" gptq_status gptq_prepare_hinv(const float* S, const double* D, const int64_t* n_tokens, int64_t d_in,
                                         int64_t batch, const gptq_params* p, float* U, int32_t* perm,
                                         int32_t* info, void* workspace, size_t ws_bytes, void* stream) {
  GQ_CHECK_ARG(S && D && n_tokens && U && info && p);
  GQ_CHECK_ARG(d_in >= 1 && d_in <= 65536 && batch >= 1 && batch <= kMaxBatch);
  GQ_CHECK_ARG(p->damp_rel >= 0.0f && std::isfinite(p->damp_rel));
  GQ_CHECK_ARG(!p->act_order || perm != nullptr);
  if (ws_bytes < prepare_workspace_bytes(d_in, batch) || workspace == nullptr) return GPTQ_ENOMEM;
  const int d = (int)d_in;
  const int nb = (int)batch;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Carver cv(workspace);
  const size_t dd = (size_t)d * d;
  double* A = cv.take<double>(nb * dd);
  double* Li = cv.take<double>(nb * dd);
  double* T = cv.take<double>(nb * t_stride(d));
  int32_t* permw = cv.take<int32_t>((size_t)nb * d);
  double* lam = cv.take<double>((size_t)nb * 2);
  double* two_over_n = lam + nb;
  TimedScope ts(kTimeFactor, st);

  hipLaunchKernelGGL(set_scalars_kernel, dim3(1), dim3(kMaxBatch), 0, st, n_tokens, nb, two_over_n, info);
  GQ_LAUNCHED();
  hipLaunchKernelGGL(damping_kernel, dim3(nb), dim3(256), 0, st, D, d, two_over_n, p->damp_rel, lam);
  GQ_LAUNCHED();
  int32_t* pp = perm ? perm : permw;
  if (p->act_order) {
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)cdiv(d, 64), nb), dim3(256), 0, st, D, d, pp);
  } else {
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)cdiv((int64_t)d * nb, 256)), dim3(256), 0, st, pp, d, nb);
  }
  GQ_LAUNCHED();
  if (!p->act_order) {
    dim3 grid((unsigned)cdiv(d, 32), (unsigned)cdiv(d, 32), nb);
    hipLaunchKernelGGL(rev_lower_kernel, grid, dim3(256), 0, st, S, D, d, two_over_n, lam, A);
    GQ_LAUNCHED();
  } else {
    // F (full symmetric 2S/N) lives in Li until the factorization needs it:
    // its rows make the permuted gather contiguous
    dim3 grid((unsigned)cdiv(d, 32), (unsigned)cdiv(d, 32), nb);
    hipLaunchKernelGGL(symmetrize_kernel, grid, dim3(256), 0, st, S, D, d, two_over_n, Li);
    GQ_LAUNCHED();
    if (d <= kRevLdsMax) {
      const dim3 g(1, d, nb);
      if (d <= 4096) hipLaunchKernelGGL(build_rev_lds_kernel<4096>, g, dim3(512), 0, st, Li, pp, d, lam, A);
      else if (d <= 8192) hipLaunchKernelGGL(build_rev_lds_kernel<8192>, g, dim3(512), 0, st, Li, pp, d, lam, A);
      else if (d <= 12288) hipLaunchKernelGGL(build_rev_lds_kernel<12288>, g, dim3(512), 0, st, Li, pp, d, lam, A);
      else hipLaunchKernelGGL(build_rev_lds_kernel<kRevLdsMax>, g, dim3(512), 0, st, Li, pp, d, lam, A);
    } else {
      dim3 g((unsigned)std::min<int64_t>(cdiv(d, 256), 64), d, nb);
      hipLaunchKernelGGL(build_rev_kernel, g, dim3(256), 0, st, Li, pp, d, lam, A);
    }
    GQ_LAUNCHED();
  }
  gptq_status s;
  {
    int dev = 0;
    GQ_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream& ss = g_side[dev];
    if (!ss.s) GQ_HIP(hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking));
    ss.next = 0;
    FactorCtx c{A, Li, T, d, nb, info, st, &ss};
    // the side stream starts after the work above and ends before what follows
    if (d < kSideMin) {
      s = rec(c, 0, d, T);
    } else {
      s = stream_order(c, st, ss.s);
      if (s == GPTQ_OK) s = rec(c, 0, d, T, true);
      const gptq_status sj = stream_order(c, ss.s, st);
      if (s == GPTQ_OK) s = sj;
    }
  }
  if (s != GPTQ_OK) return s;
  {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(d, 256), 64), d, nb);
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, st, Li, d, U);
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}
