// From H to U, the upper factor of the damped, permuted inverse Hessian, on gfx950.
//
// Steps ("GPTQ Architecture, in depth", "The algorithm in code"; "Same Ruler, Smarter
// Placement: GPTQ", 1.6 dampening, 1.7 the Cholesky trick, 1.9 activation ordering):
//   1. dead inputs (zero fp64 diagonal) count as diagonal 1;
//   2. ActOrder: perm sorts the fp64 diagonal in descending order, ties by index
//      (computed as exact ranks, so the order is the same as a stable sort);
//   3. lambda = damp * mean(diagonal), fp64;
//   4. U with H_p^-1 = U^T U.  Route: A = J H_p J (index-reversed, gathered in one pass
//      with the permutation), L = chol(A) lower, U = J L^-1 J.  Then H_p = (J L J)(J L J)^T
//      with J L J upper, so H_p^-1 = (J L^-1 J)^T (J L^-1 J) and U is the unique
//      positive-diagonal upper factor the pages obtain with chol / cholesky_inverse / chol,
//      at 2/3 d^3 instead of 4/3 d^3 flops.
//
// Cholesky blocked by 128 columns (chol_blocked below) and the triangular inverse by
// doubling (TriInverse, its early parts beside the factorization's later steps): one
// workgroup factors and inverts each 128-column diagonal
// block in LDS (by recursive halving inside the kernel); everything else is fp32
// matrix-core products.  A non-positive or non-finite pivot sets a device flag that
// the host reads back (GPTQ_ERR_NOT_SPD).
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int NB = 128;   // panel width (must equal the GEMM tile)

// key[c] = diag_key[c], or 1 for a dead input; dead[c] = (diag_key[c] == 0).
// Also clears the rank counters of actorder_rank_kernel.
__global__ __launch_bounds__(256) void keys_kernel(const double* __restrict__ diag_key, int d_in,
                                                   double* __restrict__ key, uint8_t* __restrict__ dead,
                                                   int32_t* __restrict__ rank) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d_in) return;
  const int64_t o = static_cast<int64_t>(e) * d_in + c;
  const double v = diag_key[o];
  key[o] = (v == 0.0) ? 1.0 : v;
  dead[o] = (v == 0.0) ? 1 : 0;
  rank[o] = 0;
}

// rank(c) = #{j: key_j > key_c} + #{j < c: key_j == key_c}, the position of c in a stable
// descending sort.  Block (x, y): 256 candidates c against a slice of RANK_SLICE keys j;
// the integer partial counts are summed with atomics (order-independent, exact).  Slices of
// 256 keys give d_in 4096 its 256 workgroups, one per CU.
constexpr int RANK_SLICE = 256;
__global__ __launch_bounds__(256) void actorder_rank_kernel(const double* __restrict__ key, int d_in,
                                                            int32_t* __restrict__ rank) {
  __shared__ double sk[RANK_SLICE];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int j0 = blockIdx.y * RANK_SLICE;
  const int e = blockIdx.z;
  const double* k = key + static_cast<int64_t>(e) * d_in;
  for (int i = threadIdx.x; i < RANK_SLICE; i += 256) sk[i] = (j0 + i < d_in) ? k[j0 + i] : 0.0;
  __syncthreads();
  if (c >= d_in) return;
  const double kc = k[c];
  const int jn = min(RANK_SLICE, d_in - j0);
  int cnt = 0;
  for (int j = 0; j < jn; ++j) {
    const double kj = sk[j];
    cnt += (kj > kc) || (kj == kc && j0 + j < c);
  }
  if (cnt) atomicAdd(rank + static_cast<int64_t>(e) * d_in + c, cnt);
}

// perm[rank(c)] = c (ActOrder), or the identity.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ rank, int d_in,
                                                           int act_order, int32_t* __restrict__ perm) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d_in) return;
  const int64_t o = static_cast<int64_t>(e) * d_in;
  if (!act_order) {
    perm[o + c] = c;
    return;
  }
  const int r = min(max(rank[o + c], 0), d_in - 1);
  perm[o + r] = c;
}

// lambda[e] = damp * mean(key[e]) (fixed-order tree sum in fp64).
__global__ __launch_bounds__(256) void damping_kernel(const double* __restrict__ key, int d_in,
                                                      double damp, double* __restrict__ lambda,
                                                      int* __restrict__ flag) {
  __shared__ double red[256];
  const int e = blockIdx.x;
  const double* k = key + static_cast<int64_t>(e) * d_in;
  double s = 0.0;
  for (int c = threadIdx.x; c < d_in; c += 256) s += k[c];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lambda[e] = damp * red[0] / static_cast<double>(d_in);
    flag[e] = 0;
  }
}

// A[r][c] = H[p(r)][p(c)] with p(r) = perm[d-1-r]; diagonal key[p(r)] + lambda.
// Only the blocks on and below the 128-block diagonal are written: nothing reads the others.
// The reversed permutation of the problem and one source row of H are staged in LDS, so H is
// read row by row in 16-byte vectors and the scatter happens in LDS.  kVec: H rows are
// 16-byte aligned.  DMAX bounds d_in.
constexpr int GATHER_ROWS = 4;  // output rows per workgroup
template <int DMAX, bool kVec>
__global__ __launch_bounds__(256) void gather_reversed_kernel(const float* __restrict__ H, int64_t bsh,
                                                              const int32_t* __restrict__ perm,
                                                              const double* __restrict__ key,
                                                              const double* __restrict__ lambda, int d_in,
                                                              float* __restrict__ A) {
  __shared__ __attribute__((aligned(16))) float srow[DMAX];
  __shared__ uint16_t sidx[DMAX];
  const int e = blockIdx.y, t = threadIdx.x;
  const int32_t* pe = perm + static_cast<int64_t>(e) * d_in;
  // indices are clamped so that a malformed permutation can never address outside H
  batched_copy<256>(t, d_in, [&](int c) { return pe[d_in - 1 - c]; },
                    [&](int c, int32_t p) { sidx[c] = static_cast<uint16_t>(min(max(p, 0), d_in - 1)); });
  const float* He = H + static_cast<int64_t>(e) * bsh;
  for (int i = 0; i < GATHER_ROWS; ++i) {
    const int r = blockIdx.x * GATHER_ROWS + i;
    if (r >= d_in) break;
    __syncthreads();  // sidx written / the previous row fully consumed
    const int pr = sidx[r];
    const float* src = He + static_cast<int64_t>(pr) * d_in;
    if constexpr (kVec) {
      batched_copy<256>(t, d_in / 4, [&](int c4) { return reinterpret_cast<const float4*>(src)[c4]; },
                        [&](int c4, float4 v) { reinterpret_cast<float4*>(srow)[c4] = v; });
    } else {
      batched_copy<256>(t, d_in, [&](int c) { return src[c]; }, [&](int c, float v) { srow[c] = v; });
    }
    __syncthreads();
    const int cend = min(d_in, (r / NB + 1) * NB);
    const float dg = static_cast<float>(key[static_cast<int64_t>(e) * d_in + pr] + lambda[e]);
    float* dst = A + (static_cast<int64_t>(e) * d_in + r) * d_in;
    for (int c = 4 * t; c < cend; c += 1024) {
      float4 v = make_float4(srow[sidx[c]], srow[sidx[c + 1]], srow[sidx[c + 2]], srow[sidx[c + 3]]);
      if (r - c >= 0 && r - c < 4) {
        if (r == c) v.x = dg;
        if (r == c + 1) v.y = dg;
        if (r == c + 2) v.z = dg;
        if (r == c + 3) v.w = dg;
      }
      *reinterpret_cast<float4*>(dst + c) = v;
    }
  }
}

// The same gather one element per thread, for d_in beyond the largest staged row.
__global__ __launch_bounds__(256) void gather_reversed_scalar_kernel(const float* __restrict__ H, int64_t bsh,
                                                                     const int32_t* __restrict__ perm,
                                                                     const double* __restrict__ key,
                                                                     const double* __restrict__ lambda,
                                                                     int d_in, float* __restrict__ A) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (c >= d_in || c >= (r / NB + 1) * NB) return;
  const int32_t* pe = perm + static_cast<int64_t>(e) * d_in;
  const int pr = min(max(pe[d_in - 1 - r], 0), d_in - 1);
  const int pc = min(max(pe[d_in - 1 - c], 0), d_in - 1);
  const float v = (r == c) ? static_cast<float>(key[static_cast<int64_t>(e) * d_in + pr] + lambda[e])
                           : H[static_cast<int64_t>(e) * bsh + static_cast<int64_t>(pr) * d_in + pc];
  A[(static_cast<int64_t>(e) * d_in + r) * d_in + c] = v;
}

// Factor the diagonal block at (k0, k0) of A: writes L_kk into Lbuf and L_kk^-1 into Linv
// (full 128x128 blocks, zeros above the diagonal).  Only the lower triangle of A is read.
//
// The block and its inverse stay in LDS for the whole kernel, and a recursive halving
// runs inside it down to 16-column leaves:
//   node(o, S):  node(o, S/2);  L21 = A21 X11^T;  S22 = A22 - L21 L21^T and T = L21 X11;
//                node(o + S/2, S/2);  X21 = -X22 T
// (X = L^-1).  A 16-column leaf is factored and inverted by one wave with the 16 rows in
// lanes 0..15 and the columns in registers; values move between lanes by readlane, so a
// leaf needs no barrier.  Products are 16x16 output tiles on the fp32 matrix cores,
// dealt round-robin to the LEAF_WAVES waves, with one barrier per product.
constexpr int LLD = NB + 4;   // LDS row stride (floats): 16-byte aligned rows, banks spread
// Waves of the diagonal-block kernel: the 16x16 tile products of a level are dealt to them
// (at the top level 26 tiles: 2 rounds with 16 waves, 7 with 4).
constexpr int LEAF_WAVES = 16;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bcast_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// acc += sum over k in [k0, k0 + 16 KS) of A(i0 + i, k) * B(k, j0 + j) for a 16x16 tile,
// with A(i, k) = pa[i * LLD + k] and B(k, j) = pb[j * LLD + k] (kBT) or pb[k * LLD + j].
// The K range is split in four contiguous quarters, one per k-slot of the 16x16x4
// instruction, so each lane reads its A (and B^T) values 4 at a time; all reads are issued
// before the first product.
template <bool kBT, int KS>
__device__ __forceinline__ f32x4v tile_mma_n(f32x4v acc, const float* pa, const float* pb, int k0, int lane) {
  const int q = lane >> 4, rc = lane & 15;
  const float* ar = pa + rc * LLD + k0 + q * 4 * KS;
  const float* br = kBT ? pb + rc * LLD + k0 + q * 4 * KS : pb + (k0 + q * 4 * KS) * LLD + rc;
  float4 av[KS], bv[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    av[s] = *reinterpret_cast<const float4*>(ar + 4 * s);
    if (kBT) {
      bv[s] = *reinterpret_cast<const float4*>(br + 4 * s);
    } else {
      bv[s] = make_float4(br[(4 * s) * LLD], br[(4 * s + 1) * LLD], br[(4 * s + 2) * LLD], br[(4 * s + 3) * LLD]);
    }
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s].x, bv[s].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s].y, bv[s].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s].z, bv[s].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s].w, bv[s].w, acc, 0, 0, 0);
  }
  return acc;
}

// Same over [k0, k1), k1 - k0 a multiple of 16 up to 64.
template <bool kBT>
__device__ __forceinline__ f32x4v tile_mma(f32x4v acc, const float* pa, const float* pb, int k0, int k1,
                                           int lane) {
  switch ((k1 - k0) >> 4) {
    case 1: return tile_mma_n<kBT, 1>(acc, pa, pb, k0, lane);
    case 2: return tile_mma_n<kBT, 2>(acc, pa, pb, k0, lane);
    case 3: return tile_mma_n<kBT, 3>(acc, pa, pb, k0, lane);
    default: return tile_mma_n<kBT, 4>(acc, pa, pb, k0, lane);
  }
}

// 16x16 tile (rows 4*(lane/16) + r, column lane%16) of a result, to or from LDS.
__device__ __forceinline__ void tile_store(float* p, f32x4v v, int lane) {
  float* d = p + 4 * (lane >> 4) * LLD + (lane & 15);
  d[0] = v[0]; d[LLD] = v[1]; d[2 * LLD] = v[2]; d[3 * LLD] = v[3];
}
__device__ __forceinline__ f32x4v tile_load(const float* p, int lane) {
  const float* s = p + 4 * (lane >> 4) * LLD + (lane & 15);
  f32x4v v;
  v[0] = s[0]; v[1] = s[LLD]; v[2] = s[2 * LLD]; v[3] = s[3 * LLD];
  return v;
}

// Cholesky and inverse of the 16x16 diagonal block at (o, o), by the calling wave, and,
// when kPanel, the solve L21 = A21 L11^-T of the 16 rows below it (rows o+16..o+31).
// Column k of the Cholesky takes pivot d = a_kk, scales l_rk = a_rk / sqrt(d) and then
// a_rj -= l_rk l_jk for every later column j; forward substitution of L X = I takes
// x_k /= l_kk and x_j -= l_jk x_k; the panel rows follow the Cholesky rows.  All three are
// v_j -= v_k l_jk after v_k is scaled, so one register file v[] serves them:
//   lanes  0..15: row r of the diagonal block,
//   lanes 16..31: column r of X = L^-1 (starts as e_r),
//   lanes 32..47: row r of the panel (kPanel).
// The broadcast l_jk comes out of lane j by readlane; no barrier is needed.
template <bool kPanel>
__device__ __forceinline__ void leaf16(float* sA, float* sX, int o, int lane, int* bad) {
  float v[16];
  const int r = lane & 15, part = lane >> 4;
  if (part == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (r == i) ? 1.0f : 0.0f;
  } else {
    const int row = o + r + ((kPanel && part >= 2) ? 16 : 0);
    const float* src = sA + row * LLD + o;
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
      const float4 u = *reinterpret_cast<const float4*>(src + c);
      v[c] = u.x; v[c + 1] = u.y; v[c + 2] = u.z; v[c + 3] = u.w;
    }
  }
  bool ok = true;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float d = bcast_lane(v[k], k);
    ok = ok && (d > 0.0f) && (d < INFINITY);
    // 1/sqrt(d) by the hardware reciprocal square root (1 ulp); l_kk = d / sqrt(d)
    const float il = __builtin_amdgcn_rsqf(d);
    v[k] = (lane == k) ? d * il : v[k] * il;
#pragma unroll
    for (int j = k + 1; j < 16; ++j) v[j] = fmaf(-v[k], bcast_lane(v[k], j), v[j]);
  }
  if (!ok) *bad = 1;
  if (part == 0) {
    float* dl = sA + (o + r) * LLD + o;
#pragma unroll
    for (int c = 0; c < 16; ++c) dl[c] = (c <= r) ? v[c] : 0.0f;
  } else if (part == 1) {
    float* dx = sX + o * LLD + o + r;
#pragma unroll
    for (int i = 0; i < 16; ++i) dx[i * LLD] = v[i];
  } else if (kPanel && part == 2) {
    float* dl = sA + (o + 16 + r) * LLD + o;
#pragma unroll
    for (int c = 0; c < 16; c += 4) *reinterpret_cast<float4*>(dl + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
  }
}

// kFirst: the node is the first half of its parent, and for S == 16 the leaf also solves
// the parent's 16 panel rows (so a node of 32 needs no product for its L21).
template <int S, bool kFirst>
__device__ __forceinline__ void leaf_node(float* sA, float* sX, int o, int wave, int lane, int* bad) {
  if constexpr (S == 16) {
    if (wave == 0) leaf16<kFirst>(sA, sX, o, lane, bad);
    __syncthreads();
  } else {
    constexpr int H = S / 2, NT = H / 16, NTT = NT * NT, PER = (NTT + LEAF_WAVES - 1) / LEAF_WAVES;
    leaf_node<H, true>(sA, sX, o, wave, lane, bad);
    const f32x4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4v res[PER];
    if constexpr (H > 16) {
      // L21 = A21 X11^T (X11 lower: k < 16 (tj + 1)), in place over A21
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = wave + LEAF_WAVES * u;
        if (t < NTT) {
          const int ti = t / NT, tj = t % NT;
          res[u] = tile_mma<true>(zero, sA + (o + H + 16 * ti) * LLD + o, sX + (o + 16 * tj) * LLD + o, 0,
                                  16 * (tj + 1), lane);
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int t = wave + LEAF_WAVES * u;
        if (t < NTT) tile_store(sA + (o + H + 16 * (t / NT)) * LLD + o + 16 * (t % NT), res[u], lane);
      }
      __syncthreads();
    }
    // S22 = A22 - L21 L21^T (lower tiles) and T = L21 X11 (X11 lower: k >= 16 tj) into X21
    constexpr int NLOW = NT * (NT + 1) / 2;
    for (int t = wave; t < NLOW + NTT; t += LEAF_WAVES) {
      if (t < NLOW) {
        int ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
        const int tj = t - ti * (ti + 1) / 2;
        float* c = sA + (o + H + 16 * ti) * LLD + o + H + 16 * tj;
        const f32x4v p = tile_mma<true>(zero, sA + (o + H + 16 * ti) * LLD + o, sA + (o + H + 16 * tj) * LLD + o,
                                        0, H, lane);
        tile_store(c, tile_load(c, lane) - p, lane);
      } else {
        const int u = t - NLOW, ti = u / NT, tj = u % NT;
        const f32x4v p = tile_mma<false>(zero, sA + (o + H + 16 * ti) * LLD + o, sX + o * LLD + o + 16 * tj,
                                         16 * tj, H, lane);
        tile_store(sX + (o + H + 16 * ti) * LLD + o + 16 * tj, p, lane);
      }
    }
    __syncthreads();
    leaf_node<H, false>(sA, sX, o + H, wave, lane, bad);
    // X21 = -X22 T (X22 lower: k < 16 (ti + 1)), in place over T
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = wave + LEAF_WAVES * u;
      if (t < NTT) {
        const int ti = t / NT, tj = t % NT;
        res[u] = tile_mma<false>(zero, sX + (o + H + 16 * ti) * LLD + o + H, sX + (o + H) * LLD + o + 16 * tj, 0,
                                 16 * (ti + 1), lane);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = wave + LEAF_WAVES * u;
      if (t < NTT) tile_store(sX + (o + H + 16 * (t / NT)) * LLD + o + 16 * (t % NT), -res[u], lane);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64 * LEAF_WAVES) void potrf_block_kernel(const float* __restrict__ A, float* __restrict__ Lbuf,
                                                          int64_t bsl, float* __restrict__ Linv, int d_in,
                                                          int k0, int* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) float sA[NB * LLD];
  __shared__ __attribute__((aligned(16))) float sX[NB * LLD];
  __shared__ int bad;
  const int e = blockIdx.x;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  const float* Ae = A + e * dd + static_cast<int64_t>(k0) * d_in + k0;
  if (t == 0) bad = 0;
  // 128 rows x 32 float4: thread t loads float4 column t%32 of rows t/32 + RS m, all loads
  // issued before the first LDS store
  constexpr int RS = 2 * LEAF_WAVES, NM = NB / RS;
  float4 ld[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
    ld[m] = *reinterpret_cast<const float4*>(Ae + static_cast<int64_t>(t / 32 + RS * m) * d_in + 4 * (t % 32));
#pragma unroll
  for (int m = 0; m < NM; ++m) *reinterpret_cast<float4*>(sA + (t / 32 + RS * m) * LLD + 4 * (t % 32)) = ld[m];
  __syncthreads();
  leaf_node<NB, false>(sA, sX, 0, wave, lane, &bad);
  if (t == 0 && bad) flag[e] = 1;
  float* Le = Lbuf + e * bsl + static_cast<int64_t>(k0) * d_in + k0;
  float* Xe = Linv + e * dd + static_cast<int64_t>(k0) * d_in + k0;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int row = t / 32 + RS * m, c = 4 * (t % 32);
    const float4 l = *reinterpret_cast<const float4*>(sA + row * LLD + c);
    const float4 x = *reinterpret_cast<const float4*>(sX + row * LLD + c);
    *reinterpret_cast<float4*>(Le + static_cast<int64_t>(row) * d_in + c) =
        make_float4(c <= row ? l.x : 0.0f, c + 1 <= row ? l.y : 0.0f, c + 2 <= row ? l.z : 0.0f,
                    c + 3 <= row ? l.w : 0.0f);
    *reinterpret_cast<float4*>(Xe + static_cast<int64_t>(row) * d_in + c) =
        make_float4(c <= row ? x.x : 0.0f, c + 1 <= row ? x.y : 0.0f, c + 2 <= row ? x.z : 0.0f,
                    c + 3 <= row ? x.w : 0.0f);
  }
}

// U[i][j] = Linv[d-1-i][d-1-j] for j >= i, 0 below the diagonal.  Each thread writes 4
// consecutive j of REV_ROWS rows (one reversed float4 of the source row each).
constexpr int REV_ROWS = 8;
__global__ __launch_bounds__(256) void reverse_to_upper_kernel(const float* __restrict__ Linv, int d_in,
                                                               float* __restrict__ U, int64_t bsu) {
  const int j = 4 * (blockIdx.x * 256 + threadIdx.x);
  const int e = blockIdx.z;
  if (j >= d_in) return;
#pragma unroll 2
  for (int q = 0; q < REV_ROWS; ++q) {
    const int i = blockIdx.y * REV_ROWS + q;
    if (i >= d_in) break;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j + 3 >= i) {
      const float4 s = *reinterpret_cast<const float4*>(
          Linv + (static_cast<int64_t>(e) * d_in + (d_in - 1 - i)) * d_in + (d_in - 4 - j));
      v = make_float4(j >= i ? s.w : 0.0f, j + 1 >= i ? s.z : 0.0f, j + 2 >= i ? s.y : 0.0f, s.x);
    }
    *reinterpret_cast<float4*>(U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(i) * d_in + j) = v;
  }
}

// Groups of the triangular inverse's doubling level with halves of hb blocks (nb blocks in
// all): the full groups of 2 hb blocks, then a ragged last one when the blocks left over
// exceed one half.
int tri_groups(int nb, int hb) {
  const int full = nb / (2 * hb);
  return full + (nb - full * 2 * hb > hb ? 1 : 0);
}

// Floats of T per problem for the triangular inverse: an h x h product per group and level,
// kept from the T product of a group to its X21 product (the two may be issued at different
// points of the factorization).
size_t trtri_t_floats(int nb) {
  size_t m = 0;
  for (int hb = 1; hb < nb; hb *= 2) {
    const size_t h = static_cast<size_t>(hb) * NB;
    m += static_cast<size_t>(tri_groups(nb, hb)) * h * h;
  }
  return m;
}

struct PrepWs {
  double* key;
  int32_t* rank;
  double* lambda;
  int* flag;
  float* A;
  float* Linv;
  float* T;
  size_t bytes;
};

PrepWs carve(void* ws, int batch, int d_in) {
  Carver cv(ws);
  PrepWs w{};
  const size_t dd = static_cast<size_t>(d_in) * d_in;
  w.key = cv.take<double>(static_cast<size_t>(batch) * d_in);
  w.rank = cv.take<int32_t>(static_cast<size_t>(batch) * d_in);
  w.lambda = cv.take<double>(batch);
  w.flag = cv.take<int>(batch);
  w.A = cv.take<float>(batch * dd);
  w.Linv = cv.take<float>(batch * dd);
  w.T = cv.take<float>(static_cast<size_t>(batch) * trtri_t_floats(d_in / NB));
  w.bytes = cv.used;
  return w;
}

// X = L^-1 from L and its inverted diagonal blocks, by doubling: at the level of groups of
// 2 hb blocks (hb = 1, 2, 4, ...), group [o, o + 2h) (h = 128 hb) gets
//   T = L21 X11,   X21 = -X22 T
// (X11 = L11^-1 lower: the K range of an output column of T starts at it; X22 lower: the
// K range of an output row of X21 ends at it); a ragged last group has a full first half
// and a shorter second half, itself inverted at the levels below.  T needs the columns of L
// under the group's first half and that half's inverse only, so it can run as soon as the
// factorization has passed the first half; X21 waits for the second half.  issue(ready)
// enqueues every product of the inverse whose operands lie in the first `ready` factored
// block columns and that is not yet enqueued, level by level upward, one batched product
// per run of groups: called as the factorization proceeds, the early levels and the T
// products overlap the rest of the factorization; called once with ready = nb, it is the
// plain level-by-level order.  Each group's T has its own place (trtri_t_floats).
struct TriInverse {
  static constexpr int kLevels = 32;
  int d_in, nb, batch;
  const float* L;
  int64_t bsl;
  float* Linv;
  float* T;
  int next_t[kLevels] = {}, next_x[kLevels] = {};   // per level: first group not enqueued

  gptq_status issue(int ready, hipStream_t stream, int max_cus, int max_hb = 1 << 30) {
    const int64_t dd = static_cast<int64_t>(d_in) * d_in;
    const int64_t tstride = static_cast<int64_t>(trtri_t_floats(nb));   // T floats per problem
    int64_t tbase = 0;
    int lv = 0;
    for (int hb = 1; hb < nb && hb <= max_hb; hb *= 2, ++lv) {
      const int h = hb * NB;
      const int full = nb / (2 * hb);
      const int groups = tri_groups(nb, hb);
      const int64_t gs = static_cast<int64_t>(2 * h) * (d_in + 1);   // next group, same level
      const int64_t hh = static_cast<int64_t>(h) * h;
      float* Tl = T + tbase;
      tbase += groups * hh;
      int t_end = next_t[lv], x_end = next_x[lv];
      while (t_end < groups && t_end * 2 * hb + hb <= ready) ++t_end;
      while (x_end < groups && (x_end < full ? (x_end + 1) * 2 * hb <= ready : ready == nb)) ++x_end;
      // groups [a, b) in runs of full groups, the ragged one alone (a shorter second half)
      for (int pass = 0; pass < 2; ++pass) {
        const bool is_t = pass == 0;
        int a = is_t ? next_t[lv] : next_x[lv];
        const int b = is_t ? t_end : x_end;
        while (a < b) {
          const int e = a < full ? std::min(b, full) : b;
          const int h2 = a < full ? h : (nb - full * 2 * hb - hb) * NB;
          const int64_t o = static_cast<int64_t>(a) * 2 * h;
          GemmArgs g{};
          g.batch = batch; g.batch2 = e - a; g.max_cus = max_cus;
          g.M = h2; g.N = h; g.transB = 0;
          if (is_t) {
            g.K = h;
            g.A = L + (o + h) * d_in + o; g.lda = d_in; g.sA = bsl; g.sA2 = gs;
            g.B = Linv + o * d_in + o; g.ldb = d_in; g.sB = dd; g.sB2 = gs;
            g.C = Tl + a * hh; g.ldc = h; g.sC = tstride; g.sC2 = hh;
            g.alpha = 1.0f; g.beta = 0.0f; g.flags = kBLower;
          } else {
            g.K = h2;
            g.A = Linv + (o + h) * d_in + o + h; g.lda = d_in; g.sA = dd; g.sA2 = gs;
            g.B = Tl + a * hh; g.ldb = h; g.sB = tstride; g.sB2 = hh;
            g.C = Linv + (o + h) * d_in + o; g.ldc = d_in; g.sC = dd; g.sC2 = gs;
            g.alpha = -1.0f; g.beta = 0.0f; g.flags = kALower;
          }
          gptq_status st = gemm_f32(g, stream);
          if (st != GPTQ_OK) return st;
          a = e;
        }
      }
      next_t[lv] = t_end;
      next_x[lv] = x_end;
    }
    return GPTQ_OK;
  }
};

// Cholesky of A (lower, in place) into L, blocked by 128 columns, right-looking with
// lookahead.  For each block column k, on the main stream:
//   leaf(k):  L_kk and X_kk = L_kk^-1 from the updated diagonal block (potrf_block_kernel);
//   panel(k): L[k+1:, k] = A[k+1:, k] X_kk^T;
//   near(k):  A[k+1:, k+1] -= L[k+1:, F:k+1] L[k+1, F:k+1]^T, the panels F..k that no far
//             update has brought to block column k+1, so that leaf(k+1) and panel(k+1) can start;
// and on the side stream, every G panels (k + 1 - f == G, f = first panel not yet given to a
// far update):
//   far(k):   A[k+3:, k+3:] -= L[k+3:, f:k+1] L[k+3:, f:k+1]^T  (lower tiles, K = 128 G).
// A far update covers the columns from k+3 on, so near(k+1), which writes column k+2, does
// not wait for the far update of panel k: the side stream runs up to two steps behind the
// chain.  near(c-1) waits for the last far update that covers column c (the one launched at
// a checkpoint <= c-3).  Aggregating G panels per far update reads and rewrites the trailing
// matrix once per G panels (with K = 128 these updates are bound by that traffic); the near
// updates then carry K = 2..G+1 panels.  Every block receives the updates of all earlier
// panels exactly once before it is factored.
// From this many problems per call on, the Cholesky runs left-looking (chol_left).
constexpr int kLeftLookingBatch = 4;

// Block columns between the points where the triangular inverse's ready products are
// enqueued beside the factorization, and the CUs they may take there (0: all).
constexpr int kTriStep = 8;
constexpr int kTriMaxHb = 1 << 30;
int tri_cus(int nb) { return 0; }

struct Sched {
  hipStream_t main;
  SideStream* side;
  int nb, batch;
};

float* block_at(float* base, int d_in, int bi, int bj) {
  return base + static_cast<int64_t>(bi) * NB * d_in + static_cast<int64_t>(bj) * NB;
}

// Left-looking variant for many problems at once: block column k first takes the
// contributions of all earlier columns in one product,
//   A[k:, k] -= L[k:, :k] L[k, :k]^T   (K = 128 k),
// then the leaf factors its diagonal block and the panel solve gives L[k+1:, k].  With a
// batch of problems the early steps already fill the chip, and the trailing matrix is not
// read and written back once per block column as in the right-looking order.  The later
// steps cover fewer and fewer rows, and the inverse's products over the columns already
// factored run beside them on the second side stream.
gptq_status chol_left(int d_in, float* A, float* L, int64_t bsl, float* Linv, int* flag, const Sched& sc,
                      TriInverse& tri) {
  const int nb = sc.nb, batch = sc.batch;
  hipStream_t s0 = sc.main, s2 = sc.side->s2;
  bool tri_forked = false;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  for (int k = 0; k < nb; ++k) {
    gptq_status st;
    if (k > 0) {
      GemmArgs u{};
      u.batch = batch;
      u.M = (nb - k) * NB; u.N = NB; u.K = k * NB;
      u.A = block_at(L, d_in, k, 0); u.lda = d_in; u.sA = bsl;
      u.B = u.A; u.ldb = d_in; u.sB = bsl;                         // block row k of L
      u.C = block_at(A, d_in, k, k); u.ldc = d_in; u.sC = dd;
      u.alpha = -1.0f; u.beta = 1.0f; u.transB = 1; u.flags = 0;
      if ((st = gemm_f32(u, s0)) != GPTQ_OK) return st;
    }
    GPTQ_LAUNCH(potrf_block_kernel, dim3(batch), dim3(64 * LEAF_WAVES), 0, s0, A, L, bsl, Linv, d_in, k * NB, flag);
    const int rest = nb - k - 1;
    if (rest == 0) break;
    GemmArgs g{};
    g.batch = batch;
    g.M = rest * NB; g.N = NB; g.K = NB;
    g.A = block_at(A, d_in, k + 1, k); g.lda = d_in; g.sA = dd;
    g.B = block_at(Linv, d_in, k, k); g.ldb = d_in; g.sB = dd;
    g.C = block_at(L, d_in, k + 1, k); g.ldc = d_in; g.sC = bsl;
    g.alpha = 1.0f; g.beta = 0.0f; g.transB = 1; g.flags = kBtLower;
    if ((st = gemm_f32(g, s0)) != GPTQ_OK) return st;
    // columns 0..k of L are final: the inverse's products over them beside the later steps,
    // whose products shrink with the columns left
    if ((k + 1) % kTriStep == 0) {
      GPTQ_HIP_TRY(hipEventRecord(sc.side->fork2, s0));
      GPTQ_HIP_TRY(hipStreamWaitEvent(s2, sc.side->fork2, 0));
      if ((st = tri.issue(k + 1, s2, 0)) != GPTQ_OK) return st;
      tri_forked = true;
    }
  }
  if (tri_forked) {
    GPTQ_HIP_TRY(hipEventRecord(sc.side->join3, s2));
    GPTQ_HIP_TRY(hipStreamWaitEvent(s0, sc.side->join3, 0));
  }
  return tri.issue(nb, s0, 0);
}

// Panels per far update.  While the chain of small products is the critical path (d_in <=
// 4096) two: every fork/join between the streams adds a few microseconds to the chain, and
// near updates of up to three panels are still short (d_in 4096: prepare 2.73 ms with one,
// 2.63 with two, 2.66 with three).  Four for wide layers, where the trailing passes bound
// the factorization (d_in 14336: 26.9 ms with one pass per panel, 22.5 with 2, 21.4 with
// 4, 22.0 with 8).
int far_group(int nb) { return nb <= 32 ? 2 : 4; }

// CUs a far update may occupy (one workgroup each) out of the 256 of the chip, for d_in up
// to 4096: the others are left to the chain's diagonal-block kernel (135 KB of LDS: it
// needs a whole CU), and the occupied ones keep room for the chain's 64-wide products.  On
// every CU (three workgroups each), a far update holds each chain kernel issued during it
// until it has finished (d_in 4096: prepare 2.59 -> 2.51 ms when limited).  Wider layers keep
// the full-chip far updates: one workgroup per CU runs their long updates 1.5x slower, more
// than the chain gains (d_in 14336: prepare 17.9 -> 18.4 ms when limited).
constexpr int kFarCUs = 240;
int far_cus(int nb) { return nb <= 32 ? kFarCUs : 0; }


gptq_status chol_blocked(int d_in, float* A, float* L, int64_t bsl, float* Linv, int* flag, const Sched& sc,
                         TriInverse& tri) {
  const int nb = sc.nb, batch = sc.batch;
  const int G = far_group(nb);
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  hipStream_t s0 = sc.main, s1 = sc.side->s, s2 = sc.side->s2;
  bool tri_forked = false;
  hipEvent_t far_done[2] = {sc.side->join, sc.side->join2};   // far update i records far_done[i % 2]
  // checkpoints of the last two far updates (their checkpoints differ by G >= 1, so when
  // the last one is too recent to cover a column, the one before it does)
  int last_k[2] = {-1, -1};   // [0]: the one before the last, [1]: the last
  int nfar = 0;
  int f = 0;   // first panel not yet given to a far update
  for (int k = 0; k < nb; ++k) {
    GPTQ_LAUNCH(potrf_block_kernel, dim3(batch), dim3(64 * LEAF_WAVES), 0, s0, A, L, bsl, Linv, d_in, k * NB, flag);
    const int rest = nb - k - 1;   // block rows below the diagonal block k
    if (rest == 0) break;
    gptq_status st;
    GemmArgs g{};
    g.batch = batch;
    g.M = rest * NB; g.N = NB; g.K = NB;
    g.A = block_at(A, d_in, k + 1, k); g.lda = d_in; g.sA = dd;
    g.B = block_at(Linv, d_in, k, k); g.ldb = d_in; g.sB = dd;
    g.C = block_at(L, d_in, k + 1, k); g.ldc = d_in; g.sC = bsl;
    g.alpha = 1.0f; g.beta = 0.0f; g.transB = 1; g.flags = kBtLower;
    if ((st = gemm_f32(g, s0)) != GPTQ_OK) return st;
    // columns 0..k of L are final: the inverse's products over them, on the second side stream
    if ((k + 1) % kTriStep == 0) {
      GPTQ_HIP_TRY(hipEventRecord(sc.side->fork2, s0));
      GPTQ_HIP_TRY(hipStreamWaitEvent(s2, sc.side->fork2, 0));
      if ((st = tri.issue(k + 1, s2, tri_cus(nb), kTriMaxHb)) != GPTQ_OK) return st;
      tri_forked = true;
    }
    // near(k) writes column c = k + 1: the last far update covering it has checkpoint <= k - 2
    int F = 0, wait = -1;
    if (nfar >= 1 && last_k[1] <= k - 2) {
      F = last_k[1] + 1;
      wait = nfar - 1;
    } else if (nfar >= 2 && last_k[0] <= k - 2) {
      F = last_k[0] + 1;
      wait = nfar - 2;
    }
    // a far update at checkpoint k: panels f..k onto the columns from k + 3 on
    const bool far_now = (k + 1 - f == G) && (k + 3 <= nb - 1);
    if (far_now) GPTQ_HIP_TRY(hipEventRecord(sc.side->fork, s0));   // panel(k) done
    if (wait >= 0) GPTQ_HIP_TRY(hipStreamWaitEvent(s0, far_done[wait & 1], 0));
    GemmArgs n{};
    n.batch = batch;
    n.M = rest * NB; n.N = NB; n.K = (k + 1 - F) * NB;
    n.A = block_at(L, d_in, k + 1, F); n.lda = d_in; n.sA = bsl;
    n.B = n.A; n.ldb = d_in; n.sB = bsl;                         // block row k+1 of L
    n.C = block_at(A, d_in, k + 1, k + 1); n.ldc = d_in; n.sC = dd;
    n.alpha = -1.0f; n.beta = 1.0f; n.transB = 1; n.flags = 0;
    if ((st = gemm_f32(n, s0)) != GPTQ_OK) return st;
    if (far_now) {
      GPTQ_HIP_TRY(hipStreamWaitEvent(s1, sc.side->fork, 0));
      GemmArgs u{};
      u.batch = batch;
      u.M = (nb - k - 3) * NB; u.N = u.M; u.K = (k + 1 - f) * NB;
      u.A = block_at(L, d_in, k + 3, f); u.lda = d_in; u.sA = bsl;
      u.B = u.A; u.ldb = d_in; u.sB = bsl;
      u.C = block_at(A, d_in, k + 3, k + 3); u.ldc = d_in; u.sC = dd;
      u.alpha = -1.0f; u.beta = 1.0f; u.transB = 1; u.flags = kLowerOut;
      u.max_cus = far_cus(nb);
      if ((st = gemm_f32(u, s1)) != GPTQ_OK) return st;
      GPTQ_HIP_TRY(hipEventRecord(far_done[nfar & 1], s1));
      last_k[0] = last_k[1];
      last_k[1] = k;
      ++nfar;
      f = k + 1;
    }
  }
  // every far update has been joined by a later near update; join the last one anyway
  if (nfar > 0) GPTQ_HIP_TRY(hipStreamWaitEvent(s0, far_done[(nfar - 1) & 1], 0));
  // the rest of the inverse on the main stream, after what the second side stream holds
  if (tri_forked) {
    GPTQ_HIP_TRY(hipEventRecord(sc.side->join3, s2));
    GPTQ_HIP_TRY(hipStreamWaitEvent(s0, sc.side->join3, 0));
  }
  return tri.issue(nb, s0, 0);
}

}  // namespace

size_t prepare_workspace(int batch, int d_in) {
  if (batch < 1 || d_in < NB || d_in % NB) return 0;
  return carve(nullptr, batch, d_in).bytes + 256;
}

gptq_status prepare_enqueue(int batch, int d_in, const float* H, int64_t bsh, const double* diag_key,
                            const gptq_params& p, float* U, int64_t bsu, int32_t* perm, uint8_t* dead,
                            void* ws, size_t ws_bytes, hipStream_t stream, int* not_spd) {
  PrepWs w = carve(ws, batch, d_in);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_ERR_WORKSPACE;
  const dim3 blk(256);
  const int cb = (d_in + 255) / 256;
  GPTQ_LAUNCH(keys_kernel, dim3(cb, batch), blk, 0, stream, diag_key, d_in, w.key, dead, w.rank);
  if (p.act_order) {
    GPTQ_LAUNCH(actorder_rank_kernel, dim3(cb, (d_in + RANK_SLICE - 1) / RANK_SLICE, batch), blk, 0, stream, w.key,
                d_in, w.rank);
  }
  GPTQ_LAUNCH(perm_scatter_kernel, dim3(cb, batch), blk, 0, stream, w.rank, d_in, p.act_order, perm);
  GPTQ_LAUNCH(damping_kernel, dim3(batch), blk, 0, stream, w.key, d_in, static_cast<double>(p.damp),
              w.lambda, w.flag);
  {
    const bool vec = reinterpret_cast<uintptr_t>(H) % 16 == 0 && (batch == 1 || bsh % 4 == 0);
    const dim3 gg((d_in + GATHER_ROWS - 1) / GATHER_ROWS, batch);
#define GPTQ_GATHER(DMAX)                                                                                   \
  do {                                                                                                     \
    if (vec) GPTQ_LAUNCH((gather_reversed_kernel<DMAX, true>), gg, blk, 0, stream, H, bsh, perm, w.key, w.lambda, \
                         d_in, w.A);                                                                       \
    else GPTQ_LAUNCH((gather_reversed_kernel<DMAX, false>), gg, blk, 0, stream, H, bsh, perm, w.key, w.lambda,    \
                     d_in, w.A);                                                                           \
  } while (0)
    if (d_in <= 2048) GPTQ_GATHER(2048);
    else if (d_in <= 4096) GPTQ_GATHER(4096);
    else if (d_in <= 8192) GPTQ_GATHER(8192);
    else if (d_in <= 16384) GPTQ_GATHER(16384);
    else GPTQ_LAUNCH(gather_reversed_scalar_kernel, dim3(cb, d_in, batch), blk, 0, stream, H, bsh, perm, w.key,
                     w.lambda, d_in, w.A);
#undef GPTQ_GATHER
  }
  // L is built in the U buffer (same shape), then replaced by U at the end.
  {
    std::lock_guard<std::mutex> lk(side_mutex());
    Sched sc{stream, nullptr, d_in / NB, batch};
    gptq_status st = side_stream(&sc.side);
    if (st != GPTQ_OK) return st;
    TriInverse tri{d_in, d_in / NB, batch, U, bsu, w.Linv, w.T};
    st = batch >= kLeftLookingBatch ? chol_left(d_in, w.A, U, bsu, w.Linv, w.flag, sc, tri)
                                    : chol_blocked(d_in, w.A, U, bsu, w.Linv, w.flag, sc, tri);
    if (st != GPTQ_OK) return st;
  }
  GPTQ_LAUNCH(reverse_to_upper_kernel, dim3((d_in / 4 + 255) / 256, (d_in + REV_ROWS - 1) / REV_ROWS, batch), blk, 0,
              stream, w.Linv, d_in, U, bsu);

  // read back the per-problem pivot flags
  int any = 0;
  for (int e0 = 0; e0 < batch; e0 += 64) {
    int buf[64];
    const int n = std::min(64, batch - e0);
    GPTQ_HIP_TRY(hipMemcpyAsync(buf, w.flag + e0, sizeof(int) * n, hipMemcpyDeviceToHost, stream));
    GPTQ_HIP_TRY(hipStreamSynchronize(stream));
    for (int i = 0; i < n; ++i) any |= buf[i];
  }
  *not_spd = any;
  return GPTQ_OK;
}

}  // namespace gptq
