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

#include "common.h"

namespace gq {

constexpr int kLeaf = 64;
typedef double f64x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ small kernels
constexpr int kMaxBatch = 64;
struct BatchScalars {
  double two_over_n[kMaxBatch];
};

__global__ void set_scalars_kernel(BatchScalars s, int nb, double* __restrict__ out) {
  int i = threadIdx.x;
  if (i < nb) out[i] = s.two_over_n[i];
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
// perm[rank(i)] = i.  Exact comparisons, so ties go to the lower index.
__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ D, int d, int32_t* __restrict__ perm) {
  const int b = blockIdx.y;
  const double* Db = D + (size_t)b * d;
  const int i = blockIdx.x * 256 + threadIdx.x;
  __shared__ double tile[256];
  // NaN keys sort as -inf so the ranks always form a permutation
  double di = i < d ? Db[i] : 0.0;
  if (di != di) di = -HUGE_VAL;
  int rank = 0;
  for (int j0 = 0; j0 < d; j0 += 256) {
    __syncthreads();
    if (j0 + threadIdx.x < d) {
      double v = Db[j0 + threadIdx.x];
      tile[threadIdx.x] = (v != v) ? -HUGE_VAL : v;
    }
    __syncthreads();
    int jn = min(256, d - j0);
    for (int u = 0; u < jn; ++u) {
      double v = tile[u];
      int j = j0 + u;
      rank += (v > di) || (v == di && j < i);
    }
  }
  if (i < d) perm[(size_t)b * d + rank] = i;
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

// ------------------------------------------------------------------ leaf: 64x64 Cholesky + inverse
// 256 threads as a 16x16 grid; thread (ti, tk) keeps the trailing matrix and
// the inverse at rows ti + 16u, columns tk + 16v (u, v < 4) in registers.
// Column j is step s = j % 16 of phase ph = j / 16.  The cyclic layout makes
// the finished part uniform across threads: in phase ph the rows and columns
// of groups below ph are done, so the trailing update touches only u, v >= ph
// and the inverse only u >= ph, v <= ph (its row j is zero right of column j).
//
// Step j publishes the pivot, the strictly lower part of column j and row j of
// the (unscaled) inverse through LDS (double buffered, one barrier per step);
// every thread then applies a[i][k] -= a[i][j] a[k][j] / p_j and the same row
// elimination to the inverse, x_i -= (a[i][j] / p_j) x_j.  The published column
// is zero at rows <= j, so finished rows are left alone without masks.  With
// the pivots kept unscaled, L^-1 row i is x_i / sqrt(p_i); the rows stay in
// registers until the last step and are scaled and stored once.  Only the
// inverse is stored: the factor of a diagonal block is not needed again.  A
// block smaller than 64 is padded with the identity, which leaves it unchanged.
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

// The barrier orders LDS traffic only; the global stores of the last phase
// need no wait.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct LeafShared {
  double colv[2][kLeaf];
  double rowv[2][kLeaf];
  double piv[kLeaf];
};

template <int PH, int BUF>
__device__ __forceinline__ void leaf_step(int s, int ti, int tk, double (&a)[4][4], double (&x)[4][4],
                                          LeafShared& sh) {
  const int j = 16 * PH + s;
  if (tk == s) {
#pragma unroll
    for (int u = PH; u < 4; ++u) sh.colv[BUF][ti + 16 * u] = (u > PH || ti > s) ? a[u][PH] : 0.0;
    if (ti == s) sh.piv[j] = a[PH][PH];
  }
  if (ti == s) {
#pragma unroll
    for (int v = 0; v <= PH; ++v) sh.rowv[BUF][tk + 16 * v] = x[PH][v];
  }
  lds_barrier();
  const double rp = rcp_nr(sh.piv[j]);
  double f[4], ck[4], xr[4];
#pragma unroll
  for (int u = PH; u < 4; ++u) f[u] = sh.colv[BUF][ti + 16 * u] * rp;
#pragma unroll
  for (int v = PH; v < 4; ++v) ck[v] = sh.colv[BUF][tk + 16 * v];
#pragma unroll
  for (int v = 0; v <= PH; ++v) xr[v] = sh.rowv[BUF][tk + 16 * v];
#pragma unroll
  for (int u = PH; u < 4; ++u) {
#pragma unroll
    for (int v = PH; v < 4; ++v) a[u][v] = fma(-f[u], ck[v], a[u][v]);
#pragma unroll
    for (int v = 0; v <= PH; ++v) x[u][v] = fma(-f[u], xr[v], x[u][v]);
  }
}

template <int PH>
__device__ __forceinline__ void leaf_phase(int ti, int tk, double (&a)[4][4], double (&x)[4][4], LeafShared& sh) {
  for (int s = 0; s < 16; s += 2) {
    leaf_step<PH, 0>(s, ti, tk, a, x, sh);
    leaf_step<PH, 1>(s + 1, ti, tk, a, x, sh);
  }
}

// Factor one block of n <= 64 whose lower triangle is read at src (row stride
// ld) into the registers of the 256 threads: on return x holds rows ti + 16u,
// columns tk + 16v of L^-1 (zero right of the diagonal; identity rows past n)
// and the return value is the first failing column, or -1.
__device__ __forceinline__ int leaf64(const double* src, int64_t ld, int n, LeafShared& sh, double (&x)[4][4]) {
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tk = tid & 15;
  double a[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ti + 16 * u, k = tk + 16 * v;
      double val = (i == k) ? 1.0 : 0.0;
      if (i < n && k <= i) val = src[(size_t)i * ld + k];
      a[u][v] = val;
      x[u][v] = (i == k) ? 1.0 : 0.0;
    }
  leaf_phase<0>(ti, tk, a, x, sh);
  leaf_phase<1>(ti, tk, a, x, sh);
  leaf_phase<2>(ti, tk, a, x, sh);
  leaf_phase<3>(ti, tk, a, x, sh);
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const double rs = rsqrt_nr(sh.piv[ti + 16 * u]);
#pragma unroll
    for (int v = 0; v < 4; ++v) x[u][v] *= rs;
  }
  // the first pivot that is not positive (NaN included) names the failing column
  const unsigned long long bad = __ballot((tid & 63) < n && !(sh.piv[tid & 63] > 0.0));
  return bad != 0ull ? __ffsll((long long)bad) - 1 : -1;
}

__device__ __forceinline__ void store_inverse(double* __restrict__ Lb, int64_t ld, int n, const double (&x)[4][4]) {
  const int ti = threadIdx.x >> 4, tk = threadIdx.x & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = ti + 16 * u;
    if (i < n)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (tk + 16 * v <= i) Lb[(size_t)i * ld + tk + 16 * v] = x[u][v];
  }
}

__global__ __launch_bounds__(256) void leaf_kernel(const double* __restrict__ A, double* __restrict__ Li, int d,
                                                   int o, int n, int32_t* __restrict__ info) {
  const int b = blockIdx.z;
  const size_t off = (size_t)b * d * d + (size_t)o * d + o;
  __shared__ LeafShared sh;
  double x[4][4];
  const int fail = leaf64(A + off, d, n, sh, x);
  store_inverse(Li + off, d, n, x);
  if (threadIdx.x == 0 && fail >= 0 && info[b] == 0) info[b] = (d - 1 - (o + fail)) + 1;
}

// ------------------------------------------------------------------ block of 65..128 in one workgroup
// The two-level step of the recursion (n1 = 64, n2 = n - 64) without leaving
// the workgroup: L11^-1 by the leaf, L21 = A21 L11^-T, A22 -= L21 L21^T,
// T = L21 L11^-1, L22^-1 by the leaf, L21^-1 block = -L22^-1 T.  The products
// are 64x64x64 on fp64 MFMA, each wave one 32x32 quadrant.
//
// Every 64x64 operand sits in LDS row-major with its 16-byte chunks swizzled:
// element (r, k) at r * 64 + 2 ((k / 2) ^ (r % 32)) + k % 2.  Sixteen lanes
// reading one k of sixteen rows, or sixteen k of one row, then touch distinct
// banks, and a row is still 512 contiguous bytes, so A21 and A22 are copied
// global -> LDS by the DMA path (the swizzle goes into the global address)
// while the first leaf runs.
__device__ __forceinline__ int bsw(int r, int k) { return r * 64 + ((((k >> 1) ^ (r & 31)) << 1) | (k & 1)); }

struct BlockShared {
  double p[4][64 * 64];   // 0: A21 then L21; 1: A22; 2: Li11 then Li22; 3: T
  LeafShared leaf;
};

// Factor a leaf whose lower triangle is in a swizzled LDS panel (see leaf64).
__device__ __forceinline__ int leaf64_lds(const double* P, int n, LeafShared& sh, double (&x)[4][4]) {
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tk = tid & 15;
  double a[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ti + 16 * u, k = tk + 16 * v;
      double val = (i == k) ? 1.0 : 0.0;
      if (i < n && k <= i) val = P[bsw(i, k)];
      a[u][v] = val;
      x[u][v] = (i == k) ? 1.0 : 0.0;
    }
  leaf_phase<0>(ti, tk, a, x, sh);
  leaf_phase<1>(ti, tk, a, x, sh);
  leaf_phase<2>(ti, tk, a, x, sh);
  leaf_phase<3>(ti, tk, a, x, sh);
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const double rs = rsqrt_nr(sh.piv[ti + 16 * u]);
#pragma unroll
    for (int v = 0; v < 4; ++v) x[u][v] *= rs;
  }
  const unsigned long long bad = __ballot((tid & 63) < n && !(sh.piv[tid & 63] > 0.0));
  return bad != 0ull ? __ffsll((long long)bad) - 1 : -1;
}

// acc (+)= A B for this wave's quadrant, A[i][k] = Pa(i, k) and
// B[k][j] = Pb(j, k) (kBT) or Pb(k, j)
template <bool kBT>
__device__ __forceinline__ void mm64(const double* Pa, const double* Pb, f64x4 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
#pragma unroll
  for (int k4 = 0; k4 < 16; ++k4) {
    const int kr = 4 * k4 + (lane >> 4);
    double av[2], bv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) av[u] = Pa[bsw(wm + 16 * u + (lane & 15), kr)];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int j = wn + 16 * v + (lane & 15);
      bv[v] = kBT ? Pb[bsw(j, kr)] : Pb[bsw(kr, j)];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u], bv[v], acc[u][v], 0, 0, 0);
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

// rows [0, 64) of a 64-column block at src (row stride d) into a swizzled
// panel, two rows per 1 KiB direct load; rows at or past `rows` read as zeros
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

__global__ __launch_bounds__(256) void block128_kernel(const double* __restrict__ A, double* __restrict__ Li, int d,
                                                       int o, int n, int32_t* __restrict__ info) {
  const int b = blockIdx.z;
  const int n2 = n - 64;
  const double* Ab = A + (size_t)b * d * d;
  double* Lb = Li + (size_t)b * d * d;
  __shared__ __attribute__((aligned(1024))) BlockShared sh;
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tk = tid & 15;
  double* P0 = sh.p[0];
  double* P1 = sh.p[1];
  double* P2 = sh.p[2];
  double* P3 = sh.p[3];

  dma_panel(Ab + (size_t)(o + 64) * d + o, d, n2, P0);        // A21
  dma_panel(Ab + (size_t)(o + 64) * d + o + 64, d, n2, P1);   // A22

  double x[4][4];
  const int fail1 = leaf64(Ab + (size_t)o * d + o, d, 64, sh.leaf, x);
  store_inverse(Lb + (size_t)o * d + o, d, 64, x);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) P2[bsw(ti + 16 * u, tk + 16 * v)] = x[u][v];
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads have landed
  __syncthreads();

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
  {
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

  const int fail2 = leaf64_lds(P1, n2, sh.leaf, x);
  store_inverse(Lb + (size_t)(o + 64) * d + o + 64, d, n2, x);
  // Li22 over Li11 (last read by the products before the barrier above)
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) P2[bsw(ti + 16 * u, tk + 16 * v)] = x[u][v];
  __syncthreads();

  // Li21 = -Li22 T
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
  if (tid == 0 && info[b] == 0) {
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
// MFMA blocks.  kT = 128 runs 8 waves so that one workgroup alone keeps two
// waves on every SIMD (an fp64 MFMA stream needs two to issue at full rate).
// kTBMode: 0 op(B) = B, 1 op(B) = B^T for every tile, 2 per product (g.tb).
// kVec: every run of 8 operand elements along a row is wholly inside or
// outside the live range and 16-byte aligned, so a thread's kE elements load
// as 16-byte pairs; otherwise one element at a time.  kE: elements per thread
// per operand and stage (8, or 4 for half the LDS and so two workgroups of
// 128 x 128 on a CU).
template <int kT, int kW, int kTBMode, bool kVec, int kE = 8>
__global__ __launch_bounds__(64 * kW) void dgemm_kernel(GemmPair pair) {
  constexpr int kThreads = 64 * kW;
  constexpr int kGK = kE * kThreads / kT;   // K per LDS stage
  constexpr int kWM = 2 * kT / kW;          // rows per wave
  constexpr int kWN = kT / 2;               // columns per wave
  constexpr int kBM = kWM / 16, kBN = kWN / 16;
  constexpr int kAR = kGK / kE;             // threads per row of a K-contiguous operand
  constexpr int kBR = kT / kE;              // threads per K-row of a row-major B
  const bool second = (int)blockIdx.x >= pair.tiles0;
  const GemmArgs g = second ? pair.g[1] : pair.g[0];   // a copy: its fields stay in registers
  const bool kTB = kTBMode == 2 ? g.tb != 0 : kTBMode == 1;
  const int b = blockIdx.z;
  int ti, tj;
  gemm_tile(g, kT, second ? (int)blockIdx.x - pair.tiles0 : (int)blockIdx.x, ti, tj);
  const int i0 = ti * kT, j0 = tj * kT;
  const double* A = g.A + (size_t)b * g.sA;
  const double* B = g.B + (size_t)b * g.sB;
  double* C = g.C + (size_t)b * g.sC;
  // As[k][m], Bs[k][n]: k-major so a 16-lane MFMA fragment is 16 consecutive doubles
  __shared__ double As[2][kGK][kT + 2];
  __shared__ double Bs[2][kGK][kT + 2];
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

struct FactorCtx {
  double* A;
  double* Li;
  double* T;
  int d;
  int batch;
  int32_t* info;
  hipStream_t stream;
};

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
// (4 waves), whose larger count evens out the triangular products' tiles of
// unequal K, while that gives every CU one; the small products near the
// leaves 32 x 32 tiles (4 waves of one 16 x 16 block), so that more CUs share
// their latency-bound K loops.
gptq_status gemm_launch(const FactorCtx& c, const GemmArgs& g0, const GemmArgs* g1) {
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
    gptq_status s = gemm_launch(c, g0, nullptr);
    return s != GPTQ_OK ? s : gemm_launch(c, *g1, nullptr);
  }
  const int64_t t0 = gemm_tiles(g0, kT);
  const int64_t tiles = t0 + (g1 ? gemm_tiles(*g1, kT) : 0);
  if (tiles == 0) return GPTQ_OK;
  pair.tiles0 = (int)t0;
  dim3 grid((unsigned)tiles, 1, (unsigned)c.batch);
  bool vec = true;
  for (const GemmArgs* g : {&g0, g1})
    if (g) vec = vec && vec_ok(*g);
  // 128 and 64 tiles stage 4 doubles per thread: half the LDS of 8, so two
  // (four) workgroups share a CU and hide each other's barriers
#define GQ_GEMM(T, W, TB)                                                                                 \
  do {                                                                                                    \
    constexpr int kE = T == 32 ? 8 : 4;                                                                   \
    if (vec) hipLaunchKernelGGL((dgemm_kernel<T, W, TB, true, kE>), grid, dim3(64 * W), 0, c.stream, pair); \
    else hipLaunchKernelGGL((dgemm_kernel<T, W, TB, false, kE>), grid, dim3(64 * W), 0, c.stream, pair);    \
  } while (0)
  if (kT == 32) {
    if (g1) GQ_GEMM(32, 4, 2);
    else if (g0.tb) GQ_GEMM(32, 4, 1);
    else GQ_GEMM(32, 4, 0);
  } else if (g1) GQ_GEMM(64, 4, 2);
  else if (kT == 128 && g0.tb) GQ_GEMM(128, 8, 1);
  else if (kT == 128) GQ_GEMM(128, 8, 0);
  else if (g0.tb) GQ_GEMM(64, 4, 1);
  else GQ_GEMM(64, 4, 0);
#undef GQ_GEMM
  GQ_LAUNCHED();
  return GPTQ_OK;
}

// Factor the diagonal block at offset o of size n: L into A, L^-1 into Li.
// T is this node's scratch for L21 L11^-1; the second child, which runs while
// it is live, gets the scratch after it.
gptq_status rec(const FactorCtx& c, int o, int n, double* T) {
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
  const int n1 = (int)(cdiv(cdiv(n, 2), kLeaf) * kLeaf);
  const int n2 = n - n1;
  gptq_status s = rec(c, o, n1, T);
  if (s != GPTQ_OK) return s;
  double* A21 = c.A + (size_t)(o + n1) * d + o;
  double* A22 = c.A + (size_t)(o + n1) * d + (o + n1);
  double* Li11 = c.Li + (size_t)o * d + o;
  double* Li21 = c.Li + (size_t)(o + n1) * d + o;
  double* Li22 = c.Li + (size_t)(o + n1) * d + (o + n1);
  // L21 = A21 Li11^T, parked in the Li21 slot
  s = gemm_launch(c, gemm_args(true, n2, n1, n1, 1.0, A21, d, Li11, d, 0.0, Li21, d, 3, 0, dd, dd, dd), nullptr);
  if (s != GPTQ_OK) return s;
  // together: A22 -= L21 L21^T (lower half) and T = L21 Li11
  const GemmArgs upd = gemm_args(true, n2, n2, n1, -1.0, Li21, d, Li21, d, 1.0, A22, d, 0, 1, dd, dd, dd);
  const GemmArgs tprod = gemm_args(false, n2, n1, n1, 1.0, Li21, d, Li11, d, 0.0, T, n1, 2, 0, dd, dd, sT);
  s = gemm_launch(c, upd, &tprod);
  if (s != GPTQ_OK) return s;
  s = rec(c, o + n1, n2, T + (size_t)n2 * n1);
  if (s != GPTQ_OK) return s;
  // Li21 = -Li22 T
  return gemm_launch(c, gemm_args(false, n2, n1, n2, -1.0, Li22, d, T, n1, 0.0, Li21, d, 1, 0, dd, sT, dd), nullptr);
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
  for (int64_t b = 0; b < batch; ++b) GQ_CHECK_ARG(n_tokens[b] > 0);
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

  {
    BatchScalars sc;
    for (int b = 0; b < nb; ++b) sc.two_over_n[b] = 2.0 / (double)n_tokens[b];
    hipLaunchKernelGGL(set_scalars_kernel, dim3(1), dim3(kMaxBatch), 0, st, sc, nb, two_over_n);
    GQ_LAUNCHED();
  }
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)cdiv(nb, 256)), dim3(256), 0, st, info, (int64_t)nb, 0);
  GQ_LAUNCHED();
  hipLaunchKernelGGL(damping_kernel, dim3(nb), dim3(256), 0, st, D, d, two_over_n, p->damp_rel, lam);
  GQ_LAUNCHED();
  int32_t* pp = perm ? perm : permw;
  if (p->act_order) {
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)cdiv(d, 256), nb), dim3(256), 0, st, D, d, pp);
  } else {
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)cdiv((int64_t)d * nb, 256)), dim3(256), 0, st, pp, d, nb);
  }
  GQ_LAUNCHED();
  // F (full symmetric 2S/N) lives in Li until the factorization needs it
  {
    dim3 grid((unsigned)cdiv(d, 32), (unsigned)cdiv(d, 32), nb);
    hipLaunchKernelGGL(symmetrize_kernel, grid, dim3(256), 0, st, S, D, d, two_over_n, Li);
    GQ_LAUNCHED();
  }
  {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(d, 256), 64), d, nb);
    hipLaunchKernelGGL(build_rev_kernel, grid, dim3(256), 0, st, Li, p->act_order ? pp : nullptr, d, lam, A);
    GQ_LAUNCHED();
  }
  FactorCtx c{A, Li, T, d, nb, info, st};
  gptq_status s = rec(c, 0, d, T);
  if (s != GPTQ_OK) return s;
  {
    dim3 grid((unsigned)std::min<int64_t>(cdiv(d, 256), 64), d, nb);
    hipLaunchKernelGGL(write_u_kernel, grid, dim3(256), 0, st, Li, d, U);
    GQ_LAUNCHED();
  }
  return GPTQ_OK;
}
