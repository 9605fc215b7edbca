// GPTQ column sweep on gfx950.
//
// "Same Ruler, Smarter Placement: GPTQ", 1.5 (quantize a column, scale its error by the
// inverse-Hessian diagonal, push it along that row of the inverse), 1.7 (the rows come
// from the upper factor U), 1.8 (lazy batches of 128 columns); "GPTQ Architecture, in
// depth", "The algorithm in code" (asymmetric min-max grid refitted at each group start,
// dead inputs, undoing the permutation, group index of each original column).
//
// Data path for one problem:
//   permute_weight:  W (bf16/fp16/fp32, original order) -> W_p fp32 [d_out, d_in] in
//                    processing order, dead columns zeroed                 (workspace)
//   row_grid:        per-row grid only: min/max of each whole row -> scale, zero
//   per block b of 128 columns:
//     block_sweep:   16 lanes per row keep the row's 128 block columns in registers
//                    (8 each); the column value is broadcast within the row by DPP and
//                    quantized by all 16; U's diagonal block sits in LDS.  Outputs codes
//                    (processing order), the group scale/zero, and the block's columns
//                    of Err.
//     lazy update:   hierarchical (see sweep_range): W_p[:, right] -= Err[:, left] @ U[left,
//                    right] on the fp32 matrix cores, Err [d_out, d_in] in processing order.
//   unpermute:       codes back to original column order; g_idx.
#include <type_traits>
#include <utility>

#include "common.h"

namespace gptq {
namespace {

// Rows and index tables are staged in LDS: the per-problem table (source column, or a
// sentinel for dead columns) once per workgroup, then each row of W read in 16-byte vectors
// and gathered from LDS into float4 stores.  kVec: W rows are 16-byte aligned.
constexpr int STAGE_ROWS = 8;       // rows per workgroup of the staged permutes
constexpr int kStagedMax = 16384;   // largest d_in whose row and index table are staged
constexpr uint16_t kDeadCol = 0xFFFF;
template <typename T, int DMAX, bool kVec>
__global__ __launch_bounds__(256) void permute_weight_staged_kernel(const T* __restrict__ W, int64_t ldw,
                                                                    int64_t bsw, const int32_t* __restrict__ perm,
                                                                    const uint8_t* __restrict__ dead, int d_out,
                                                                    int d_in, float* __restrict__ Wp) {
  __shared__ __attribute__((aligned(16))) float srow[DMAX];
  __shared__ uint16_t sidx[DMAX];
  const int e = blockIdx.y, t = threadIdx.x;
  for (int j = t; j < d_in; j += 256) {
    // a malformed permutation is clamped into range rather than addressing outside W
    const int c = min(max(perm[static_cast<int64_t>(e) * d_in + j], 0), d_in - 1);
    sidx[j] = dead[static_cast<int64_t>(e) * d_in + c] ? kDeadCol : static_cast<uint16_t>(c);
  }
  for (int i = 0; i < STAGE_ROWS; ++i) {
    const int r = blockIdx.x * STAGE_ROWS + i;
    if (r >= d_out) break;
    __syncthreads();  // sidx written / the previous row fully consumed
    const T* src = W + static_cast<int64_t>(e) * bsw + static_cast<int64_t>(r) * ldw;
    if constexpr (kVec && sizeof(T) == 2) {
      for (int c8 = t; c8 < d_in / 8; c8 += 256) {
        const uint4 v = reinterpret_cast<const uint4*>(src)[c8];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          T lo, hi;
          lo.bits = static_cast<uint16_t>(u[q] & 0xFFFFu);
          hi.bits = static_cast<uint16_t>(u[q] >> 16);
          f[2 * q] = load_as_f32(&lo);
          f[2 * q + 1] = load_as_f32(&hi);
        }
        reinterpret_cast<float4*>(srow)[2 * c8] = make_float4(f[0], f[1], f[2], f[3]);
        reinterpret_cast<float4*>(srow)[2 * c8 + 1] = make_float4(f[4], f[5], f[6], f[7]);
      }
    } else if constexpr (kVec) {
      for (int c4 = t; c4 < d_in / 4; c4 += 256)
        reinterpret_cast<float4*>(srow)[c4] = reinterpret_cast<const float4*>(src)[c4];
    } else {
      for (int c = t; c < d_in; c += 256) srow[c] = load_as_f32(src + c);
    }
    __syncthreads();
    float* dst = Wp + (static_cast<int64_t>(e) * d_out + r) * d_in;
    for (int j = 4 * t; j < d_in; j += 1024) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint16_t c = sidx[j + q];
        v[q] = c == kDeadCol ? 0.0f : srow[c];
      }
      *reinterpret_cast<float4*>(dst + j) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// One element per thread, for d_in beyond the largest staged row.
template <typename T>
__global__ __launch_bounds__(256) void permute_weight_kernel(const T* __restrict__ W, int64_t ldw, int64_t bsw,
                                                             const int32_t* __restrict__ perm,
                                                             const uint8_t* __restrict__ dead, int d_out,
                                                             int d_in, float* __restrict__ Wp) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (j >= d_in) return;
  // a malformed permutation is clamped into range rather than addressing outside W
  const int c = min(max(perm[static_cast<int64_t>(e) * d_in + j], 0), d_in - 1);
  const bool isdead = dead[static_cast<int64_t>(e) * d_in + c] != 0;
  const float v = isdead ? 0.0f : load_as_f32(W + static_cast<int64_t>(e) * bsw + static_cast<int64_t>(r) * ldw + c);
  Wp[(static_cast<int64_t>(e) * d_out + r) * d_in + j] = v;
}

__global__ __launch_bounds__(256) void inverse_perm_kernel(const int32_t* __restrict__ perm, int d_in,
                                                           int32_t* __restrict__ inv) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (j >= d_in) return;
  const int c = min(max(perm[static_cast<int64_t>(e) * d_in + j], 0), d_in - 1);
  inv[static_cast<int64_t>(e) * d_in + c] = j;
}

// One grid per row, fitted on the whole (dead-zeroed) row at the first column.
__global__ __launch_bounds__(256) void row_grid_kernel(const float* __restrict__ Wp, int d_out, int d_in,
                                                       float maxq, float* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros) {
  __shared__ float slo[256], shi[256];
  const int r = blockIdx.x, e = blockIdx.y;
  const float* row = Wp + (static_cast<int64_t>(e) * d_out + r) * d_in;
  float lo = 0.0f, hi = 0.0f;
  for (int j = threadIdx.x; j < d_in; j += 256) {
    lo = fminf(lo, row[j]);
    hi = fmaxf(hi, row[j]);
  }
  slo[threadIdx.x] = lo;
  shi[threadIdx.x] = hi;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      slo[threadIdx.x] = fminf(slo[threadIdx.x], slo[threadIdx.x + w]);
      shi[threadIdx.x] = fmaxf(shi[threadIdx.x], shi[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float s = fmaxf((shi[0] - slo[0]) / maxq, 1e-8f);
    scales[static_cast<int64_t>(e) * d_out + r] = s;
    zeros[static_cast<int64_t>(e) * d_out + r] = static_cast<uint8_t>(rintf(-slo[0] / s));
  }
}

// DPP within a row of 16 lanes: broadcast of lane `src`, and rotation by `n`.
template <int src>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + src, 0xF, 0xF, false));
}
template <int n>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + n, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_min(float v) {
  v = fminf(v, row_ror<8>(v));
  v = fminf(v, row_ror<4>(v));
  v = fminf(v, row_ror<2>(v));
  return fminf(v, row_ror<1>(v));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

constexpr int SW_ROWS = 16;   // rows of W per workgroup: 16 lanes per row, 4 rows per wave

// One 128-column block of the sweep.  G = group size (16, 32, 64 or 128), or 0 for the
// per-row grid already written by row_grid_kernel.
//
// A row of W is spread over one DPP row of 16 lanes: lane k keeps columns 16m + k
// (m = 0..7) in registers.  For column j the owner lane's value is broadcast to the row
// (row_newbcast), every lane of the row quantizes it (so all 16 hold err_j and code_j),
// and each lane updates its own later columns.  The U block sits in LDS as
// Ul[j][8k + m] = U[j0 + j][j0 + 16m + k] with its diagonal zeroed (1/U_jj kept apart):
// a lane's update reads are contiguous, the four rows of a wave read the same words, and
// columns at or before j get a zero factor.  At a group start the grid is fitted on the
// row's current values of the group's columns (min/max reduced over the 16 lanes).
template <int G>
__global__ __launch_bounds__(256) void block_sweep_kernel(const float* __restrict__ Wp, const float* __restrict__ U,
                                                          int64_t bsu, int d_out, int d_in, int blk, float maxq,
                                                          float* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                          uint8_t* __restrict__ codes_p, float* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) float Ul[kBlock * kBlock];
  __shared__ float inv_d[kBlock];
  const int e = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blk * kBlock;
  const float* Ub = U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(j0) * d_in + j0;
  const int r = blockIdx.x * SW_ROWS + (tid >> 4);
  const int k = tid & 15;
  const bool live = r < d_out;
  // the row's block columns are fetched first, so they arrive while U is staged
  const float* wrow = Wp + (static_cast<int64_t>(e) * d_out + (live ? r : 0)) * d_in + j0;
  float w[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) w[m] = wrow[16 * m + k];
  // stage the U block: thread (row j, lane kk) gathers U[j][16m + kk], m = 0..7 (each load
  // instruction reads 16 consecutive floats across the lanes) and writes them as 8
  // consecutive floats
#pragma unroll 2
  for (int i = tid; i < kBlock * 16; i += 256) {
    const int j = i >> 4, kk = i & 15;
    const float* src = Ub + static_cast<int64_t>(j) * d_in + kk;
    float v[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = src[16 * m];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (16 * m + kk == j) {
        inv_d[j] = 1.0f / v[m];
        v[m] = 0.0f;
      }
    }
    float4* dst = reinterpret_cast<float4*>(Ul + j * kBlock + 8 * kk);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();
  if (!live) return;   // whole rows of 16 lanes leave together; no barrier follows
  const int n_groups = G ? d_in / G : 1;
  float* sc = scales + static_cast<int64_t>(e) * n_groups * d_out;
  uint8_t* zr = zeros + static_cast<int64_t>(e) * n_groups * d_out;
  float s = 1.0f, z = 0.0f, inv_s = 1.0f;
  if constexpr (G == 0) {
    s = sc[r];
    z = static_cast<float>(zr[r]);
    inv_s = 1.0f / s;
  }
  // lane k stores the codes of columns 8k..8k+7 (two words)
  uint32_t cw0 = 0u, cw1 = 0u;
  const float* ul_k = Ul + 8 * k;
  // U row j is read into registers one column ahead (two alternating sets), so that the
  // LDS latency stays off the column-to-column chain
  float4 ua0 = *reinterpret_cast<const float4*>(ul_k), ua1 = *reinterpret_cast<const float4*>(ul_k + 4);
  float4 ub0, ub1;
  float dja = inv_d[0], djb = 0.0f;

  static_for(std::make_integer_sequence<int, kBlock>{}, [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int mj = j >> 4;
    float4& cur0 = (j & 1) ? ub0 : ua0;
    float4& cur1 = (j & 1) ? ub1 : ua1;
    float4& nxt0 = (j & 1) ? ua0 : ub0;
    float4& nxt1 = (j & 1) ? ua1 : ub1;
    const float dj = (j & 1) ? djb : dja;
    if constexpr (j + 1 < kBlock) {
      const float* un = ul_k + (j + 1) * kBlock;
      if constexpr (((j + 1) >> 4) < 4) nxt0 = *reinterpret_cast<const float4*>(un);
      nxt1 = *reinterpret_cast<const float4*>(un + 4);
      if constexpr (j & 1) dja = inv_d[j + 1];
      else djb = inv_d[j + 1];
      // the scheduler would sink these reads next to their use in the next column
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (G != 0 && j % G == 0) {
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int m = j / 16; m < (j + G) / 16; ++m) {
        lo = fminf(lo, w[m]);
        hi = fmaxf(hi, w[m]);
      }
      lo = row_min(lo);
      hi = row_max(hi);
      s = fmaxf((hi - lo) / maxq, 1e-8f);
      z = rintf(-lo / s);
      inv_s = 1.0f / s;
      if (k == 0) {
        const int gi = (j0 + j) / G;
        sc[static_cast<int64_t>(gi) * d_out + r] = s;
        zr[static_cast<int64_t>(gi) * d_out + r] = static_cast<uint8_t>(z);
      }
    }
    const float wj = row_bcast<j & 15>(w[mj]);
    const float q = fminf(fmaxf(rintf(wj * inv_s) + z, 0.0f), maxq);
    const float wq = s * (q - z);
    const float e_j = (wj - wq) * dj;
    const uint32_t qb = (k == (j >> 3)) ? (static_cast<uint32_t>(q) << (8 * (j & 3))) : 0u;
    if constexpr ((j & 4) == 0) cw0 |= qb;
    else cw1 |= qb;
    const float u[8] = {cur0.x, cur0.y, cur0.z, cur0.w, cur1.x, cur1.y, cur1.z, cur1.w};
#pragma unroll
    for (int m = mj; m < 8; ++m) w[m] = fmaf(-e_j, u[m], w[m]);
    if (k == (j & 15)) w[mj] = e_j;   // the owner keeps err_j in place of w_j
  });
  uint2* cdst = reinterpret_cast<uint2*>(codes_p + (static_cast<int64_t>(e) * d_out + r) * d_in + j0);
  cdst[k] = make_uint2(cw0, cw1);
  float* edst = err + (static_cast<int64_t>(e) * d_out + r) * d_in + j0;
#pragma unroll
  for (int m = 0; m < 8; ++m) edst[16 * m + k] = w[m];
}

// codes[:, c] = codes_p[:, inv[c]]; g_idx[c] = inv[c] / group.  Staged like the weight
// permute: inv once per workgroup, each codes_p row in LDS, 16 codes per thread per store.
// kVec: the codes rows are 16-byte aligned.
template <int DMAX, bool kVec>
__global__ __launch_bounds__(256) void unpermute_staged_kernel(const uint8_t* __restrict__ codes_p,
                                                               const int32_t* __restrict__ inv, int d_out,
                                                               int d_in, int group, uint8_t* __restrict__ codes,
                                                               int32_t* __restrict__ g_idx) {
  __shared__ __attribute__((aligned(16))) uint8_t srow[DMAX];
  __shared__ uint16_t sidx[DMAX];
  const int e = blockIdx.y, t = threadIdx.x;
  for (int c = t; c < d_in; c += 256) {
    const int j = min(max(inv[static_cast<int64_t>(e) * d_in + c], 0), d_in - 1);
    sidx[c] = static_cast<uint16_t>(j);
    if (blockIdx.x == 0) g_idx[static_cast<int64_t>(e) * d_in + c] = group > 0 ? j / group : 0;
  }
  for (int i = 0; i < STAGE_ROWS; ++i) {
    const int r = blockIdx.x * STAGE_ROWS + i;
    if (r >= d_out) break;
    __syncthreads();
    const int64_t ro = (static_cast<int64_t>(e) * d_out + r) * d_in;
    // codes_p rows start at multiples of d_in (a multiple of 128) in a 256-byte aligned workspace
    for (int c16 = t; c16 < d_in / 16; c16 += 256)
      reinterpret_cast<uint4*>(srow)[c16] = reinterpret_cast<const uint4*>(codes_p + ro)[c16];
    __syncthreads();
    if constexpr (kVec) {
      for (int c = 16 * t; c < d_in; c += 4096) {
        uint32_t u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          u[q] = static_cast<uint32_t>(srow[sidx[c + 4 * q]]) | (static_cast<uint32_t>(srow[sidx[c + 4 * q + 1]]) << 8) |
                 (static_cast<uint32_t>(srow[sidx[c + 4 * q + 2]]) << 16) |
                 (static_cast<uint32_t>(srow[sidx[c + 4 * q + 3]]) << 24);
        *reinterpret_cast<uint4*>(codes + ro + c) = make_uint4(u[0], u[1], u[2], u[3]);
      }
    } else {
      for (int c = t; c < d_in; c += 256) codes[ro + c] = srow[sidx[c]];
    }
  }
}

// One element per thread, for d_in beyond the largest staged row.
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ codes_p,
                                                        const int32_t* __restrict__ inv, int d_out, int d_in,
                                                        int group, uint8_t* __restrict__ codes,
                                                        int32_t* __restrict__ g_idx) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (c >= d_in) return;
  const int j = min(max(inv[static_cast<int64_t>(e) * d_in + c], 0), d_in - 1);
  const int64_t ro = (static_cast<int64_t>(e) * d_out + r) * d_in;
  codes[ro + c] = codes_p[ro + j];
  if (r == 0) g_idx[static_cast<int64_t>(e) * d_in + c] = group > 0 ? j / group : 0;
}

struct QuantWs {
  float* Wp;
  float* err;
  uint8_t* codes_p;
  int32_t* inv;
  size_t bytes;
};

QuantWs carve(void* ws, int batch, int d_out, int d_in) {
  Carver cv(ws);
  QuantWs w{};
  const size_t rows = static_cast<size_t>(batch) * d_out;
  w.Wp = cv.take<float>(rows * d_in);
  w.err = cv.take<float>(rows * d_in);
  w.codes_p = cv.take<uint8_t>(rows * d_in);
  w.inv = cv.take<int32_t>(static_cast<size_t>(batch) * d_in);
  w.bytes = cv.used;
  return w;
}

template <int G>
gptq_status launch_sweep(dim3 grid, hipStream_t stream, const float* Wp, const float* U, int64_t bsu, int d_out,
                         int d_in, int blk, float maxq, float* scales, uint8_t* zeros, uint8_t* codes_p,
                         float* err) {
  GPTQ_LAUNCH(block_sweep_kernel<G>, grid, dim3(256), 0, stream, Wp, U, bsu, d_out, d_in, blk, maxq, scales,
              zeros, codes_p, err);
  return GPTQ_OK;
}

gptq_status sweep_block(int b, int G, dim3 sg, hipStream_t stream, int d_out, int d_in, const QuantWs& w,
                        const float* U, int64_t bsu, float maxq, float* scales, uint8_t* zeros) {
  switch (G) {
    case 0: return launch_sweep<0>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err);
    case 16: return launch_sweep<16>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err);
    case 32: return launch_sweep<32>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err);
    case 64: return launch_sweep<64>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err);
    case 128: return launch_sweep<128>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err);
    default: return GPTQ_ERR_UNSUPPORTED;
  }
}

// Blocks [b0, b1) of the sweep.  The lazy batch update is applied hierarchically: after
// the left half of a range is swept, its errors are pushed into the right half of the
// same range in one product, W_p[:, right] -= Err[:, left] @ U[left, right].  Every pair
// of columns j < k in different blocks meets exactly once, at the range where they are
// split, after j's error is known and before k is quantized, so the updates are the same
// as applying each block's errors to all later columns right after the block; only the
// time at which they land changes.  Most of the flops move into a few large products.
gptq_status sweep_range(int b0, int b1, int G, dim3 sg, hipStream_t stream, int batch, int d_out, int d_in,
                        const QuantWs& w, const float* U, int64_t bsu, float maxq, float* scales, uint8_t* zeros) {
  if (b1 - b0 == 1) return sweep_block(b0, G, sg, stream, d_out, d_in, w, U, bsu, maxq, scales, zeros);
  const int bm = b0 + (b1 - b0) / 2;
  gptq_status st = sweep_range(b0, bm, G, sg, stream, batch, d_out, d_in, w, U, bsu, maxq, scales, zeros);
  if (st != GPTQ_OK) return st;
  GemmArgs g{};
  g.M = d_out; g.N = (b1 - bm) * kBlock; g.K = (bm - b0) * kBlock;
  g.A = w.err + static_cast<int64_t>(b0) * kBlock; g.lda = d_in; g.sA = static_cast<int64_t>(d_out) * d_in;
  g.B = U + static_cast<int64_t>(b0) * kBlock * d_in + static_cast<int64_t>(bm) * kBlock; g.ldb = d_in; g.sB = bsu;
  g.C = w.Wp + static_cast<int64_t>(bm) * kBlock; g.ldc = d_in; g.sC = static_cast<int64_t>(d_out) * d_in;
  g.alpha = -1.0f; g.beta = 1.0f; g.transB = 0; g.flags = 0; g.batch = batch;
  if ((st = gemm_f32(g, stream)) != GPTQ_OK) return st;
  return sweep_range(bm, b1, G, sg, stream, batch, d_out, d_in, w, U, bsu, maxq, scales, zeros);
}

}  // namespace

size_t quantize_workspace(int batch, int d_out, int d_in, const gptq_params&) {
  if (batch < 1 || d_out < 1 || d_in < kBlock) return 0;
  return carve(nullptr, batch, d_out, d_in).bytes + 256;
}

gptq_status quantize_enqueue(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W, int64_t ldw,
                             int64_t bsw, const float* U, int64_t bsu, const int32_t* perm, const uint8_t* dead,
                             const gptq_params& p, uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  QuantWs w = carve(ws, batch, d_out, d_in);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_ERR_WORKSPACE;
  const int G = p.group_size == -1 ? 0 : p.group_size;
  const float maxq = static_cast<float>((1 << p.bits) - 1);
  const dim3 blk(256);
  const int cb = (d_in + 255) / 256;
  const dim3 pg(cb, d_out, batch);
  const dim3 sgr((d_out + STAGE_ROWS - 1) / STAGE_ROWS, batch);
  {
    const size_t tb = w_dtype == GPTQ_F32 ? 4 : 2;
    const bool vec = reinterpret_cast<uintptr_t>(W) % 16 == 0 && (ldw * tb) % 16 == 0 &&
                     (batch == 1 || (bsw * tb) % 16 == 0);
    gptq_status st = GPTQ_OK;
    auto staged = [&](auto tag, auto dmax) {
      using T = decltype(tag);
      constexpr int DM = decltype(dmax)::value;
      const T* Wt = static_cast<const T*>(W);
      if (vec) GPTQ_LAUNCH((permute_weight_staged_kernel<T, DM, true>), sgr, blk, 0, stream, Wt, ldw, bsw, perm, dead,
                           d_out, d_in, w.Wp);
      else GPTQ_LAUNCH((permute_weight_staged_kernel<T, DM, false>), sgr, blk, 0, stream, Wt, ldw, bsw, perm, dead,
                       d_out, d_in, w.Wp);
      return GPTQ_OK;
    };
    auto by_dtype = [&](auto dmax) {
      switch (w_dtype) {
        case GPTQ_F32: return staged(float{}, dmax);
        case GPTQ_BF16: return staged(BF16{}, dmax);
        case GPTQ_F16: return staged(F16{}, dmax);
      }
      return GPTQ_ERR_INVALID_ARG;
    };
    if (d_in <= 2048) st = by_dtype(std::integral_constant<int, 2048>{});
    else if (d_in <= 4096) st = by_dtype(std::integral_constant<int, 4096>{});
    else if (d_in <= 8192) st = by_dtype(std::integral_constant<int, 8192>{});
    else if (d_in <= kStagedMax) st = by_dtype(std::integral_constant<int, kStagedMax>{});
    else {
      switch (w_dtype) {
        case GPTQ_F32:
          GPTQ_LAUNCH(permute_weight_kernel<float>, pg, blk, 0, stream, static_cast<const float*>(W), ldw, bsw, perm,
                      dead, d_out, d_in, w.Wp);
          break;
        case GPTQ_BF16:
          GPTQ_LAUNCH(permute_weight_kernel<BF16>, pg, blk, 0, stream, static_cast<const BF16*>(W), ldw, bsw, perm,
                      dead, d_out, d_in, w.Wp);
          break;
        case GPTQ_F16:
          GPTQ_LAUNCH(permute_weight_kernel<F16>, pg, blk, 0, stream, static_cast<const F16*>(W), ldw, bsw, perm,
                      dead, d_out, d_in, w.Wp);
          break;
      }
    }
    if (st != GPTQ_OK) return st;
  }
  GPTQ_LAUNCH(inverse_perm_kernel, dim3(cb, batch), blk, 0, stream, perm, d_in, w.inv);
  if (G == 0) {
    GPTQ_LAUNCH(row_grid_kernel, dim3(d_out, batch), blk, 0, stream, w.Wp, d_out, d_in, maxq, scales, zeros);
  }
  const dim3 sg((d_out + SW_ROWS - 1) / SW_ROWS, batch);
  const gptq_status st = sweep_range(0, d_in / kBlock, G, sg, stream, batch, d_out, d_in, w, U, bsu, maxq, scales,
                                     zeros);
  if (st != GPTQ_OK) return st;
  {
    const bool vec = reinterpret_cast<uintptr_t>(codes) % 16 == 0;
    auto staged = [&](auto dmax) {
      constexpr int DM = decltype(dmax)::value;
      if (vec) GPTQ_LAUNCH((unpermute_staged_kernel<DM, true>), sgr, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G,
                           codes, g_idx);
      else GPTQ_LAUNCH((unpermute_staged_kernel<DM, false>), sgr, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G,
                       codes, g_idx);
      return GPTQ_OK;
    };
    gptq_status st = GPTQ_OK;
    if (d_in <= 4096) st = staged(std::integral_constant<int, 4096>{});
    else if (d_in <= kStagedMax) st = staged(std::integral_constant<int, kStagedMax>{});
    else GPTQ_LAUNCH(unpermute_kernel, pg, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G, codes, g_idx);
    if (st != GPTQ_OK) return st;
  }
  return GPTQ_OK;
}

}  // namespace gptq
