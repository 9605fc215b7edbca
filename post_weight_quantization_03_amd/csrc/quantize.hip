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
//     block_sweep:   one lane per row keeps the row's 128 block columns in registers;
//                    every lane quantizes its own row, so the column recurrence needs no
//                    cross-lane traffic.  U's diagonal block is wave-uniform and is read
//                    through the scalar cache.  Outputs codes (processing order), the
//                    group scale/zero, and the block's columns of Err.
//     lazy update:   hierarchical (see sweep_range): W_p[:, right] -= Err[:, left] @ U[left,
//                    right] on the fp32 matrix cores, Err [d_out, d_in] in processing order.
//   unpermute:       codes back to original column order; g_idx.
#include "common.h"

namespace gptq {
namespace {

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

// One 128-column block of the sweep.  G = group size (a divisor of 128), or 0 for the
// per-row grid already written by row_grid_kernel.  One lane = one row.
template <int G>
__global__ __launch_bounds__(64) void block_sweep_kernel(const float* __restrict__ Wp, const float* __restrict__ U,
                                                         int64_t bsu, int d_out, int d_in, int blk, float maxq,
                                                         float* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                         uint8_t* __restrict__ codes_p, float* __restrict__ err) {
  const int e = blockIdx.y;
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= d_out) return;
  const int j0 = blk * kBlock;
  const int n_groups = G ? d_in / G : 1;
  float w[kBlock];
  const float4* src = reinterpret_cast<const float4*>(Wp + (static_cast<int64_t>(e) * d_out + r) * d_in + j0);
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) {
    const float4 v = src[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  const float* Ub = U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(j0) * d_in + j0;
  float* sc = scales + static_cast<int64_t>(e) * n_groups * d_out;
  uint8_t* zr = zeros + static_cast<int64_t>(e) * n_groups * d_out;
  float s = 1.0f, z = 0.0f, inv_s = 1.0f;
  if constexpr (G == 0) {
    s = sc[r];
    z = static_cast<float>(zr[r]);
    inv_s = 1.0f / s;
  }
  uint32_t cw[kBlock / 4];
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) cw[i] = 0u;

#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    if constexpr (G != 0) {
      if (j % G == 0) {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int k = 0; k < G; ++k) {
          lo = fminf(lo, w[j + k]);
          hi = fmaxf(hi, w[j + k]);
        }
        s = fmaxf((hi - lo) / maxq, 1e-8f);
        z = rintf(-lo / s);
        inv_s = 1.0f / s;
        const int gi = (j0 + j) / G;
        sc[static_cast<int64_t>(gi) * d_out + r] = s;
        zr[static_cast<int64_t>(gi) * d_out + r] = static_cast<uint8_t>(z);
      }
    }
    const float q = fminf(fmaxf(rintf(w[j] * inv_s) + z, 0.0f), maxq);
    const float wq = s * (q - z);
    const float e_j = (w[j] - wq) * (1.0f / Ub[j * d_in + j]);
    cw[j / 4] |= static_cast<uint32_t>(q) << (8 * (j % 4));
#pragma unroll
    for (int k = j + 1; k < kBlock; ++k) w[k] = fmaf(-e_j, Ub[j * d_in + k], w[k]);
    w[j] = e_j;
  }
  uint4* cdst = reinterpret_cast<uint4*>(codes_p + (static_cast<int64_t>(e) * d_out + r) * d_in + j0);
#pragma unroll
  for (int i = 0; i < kBlock / 16; ++i) cdst[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
  float4* edst = reinterpret_cast<float4*>(err + (static_cast<int64_t>(e) * d_out + r) * d_in + j0);
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) edst[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

// Broadcast lane `src` of each group of four lanes (DPP quad_perm).
template <int src>
__device__ __forceinline__ float quad_bcast(float v) {
  constexpr int ctrl = src | (src << 2) | (src << 4) | (src << 6);
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // [1,0,3,2]
  return fminf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // [2,3,0,1]
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
}

constexpr int QP = 36;   // LDS stride (floats) of one lane's 32 U values of a row

// One 128-column block of the sweep with four lanes per row: lane k of a quad keeps
// columns 4m + k (m = 0..31) of its row in registers.  For column j, the owner lane's
// value is broadcast to the quad (DPP), every lane of the quad quantizes it (so all four
// hold err_j and code_j), and each lane updates its own later columns.  The U block sits
// in LDS as Ul[j][k][m] = U[j0 + j][j0 + 4m + k] with its diagonal zeroed (1/U_jj kept
// apart), so a lane's update reads are contiguous and columns at or before j get a zero
// factor.  A workgroup of 256 threads handles 64 rows.
template <int G>
__global__ __launch_bounds__(256) void block_sweep_quad_kernel(const float* __restrict__ Wp, const float* __restrict__ U,
                                                               int64_t bsu, int d_out, int d_in, int blk, float maxq,
                                                               float* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                               uint8_t* __restrict__ codes_p, float* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) float Ul[kBlock][4][QP];
  __shared__ float inv_d[kBlock];
  const int e = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blk * kBlock;
  const float* Ub = U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(j0) * d_in + j0;
  // stage the U block: thread handles float4 chunks (row j, columns 4m..4m+3)
  for (int i = tid; i < kBlock * kBlock / 4; i += 256) {
    const int j = i >> 5, m = i & 31;
    const float4 v = *reinterpret_cast<const float4*>(Ub + static_cast<int64_t>(j) * d_in + 4 * m);
    Ul[j][0][m] = (4 * m + 0 == j) ? 0.0f : v.x;
    Ul[j][1][m] = (4 * m + 1 == j) ? 0.0f : v.y;
    Ul[j][2][m] = (4 * m + 2 == j) ? 0.0f : v.z;
    Ul[j][3][m] = (4 * m + 3 == j) ? 0.0f : v.w;
    if (4 * m <= j && j < 4 * m + 4) {
      const float dj = (j == 4 * m) ? v.x : (j == 4 * m + 1) ? v.y : (j == 4 * m + 2) ? v.z : v.w;
      inv_d[j] = 1.0f / dj;
    }
  }
  __syncthreads();
  const int r = blockIdx.x * 64 + (tid >> 2);
  const int k = tid & 3;
  if (r >= d_out) return;
  const int n_groups = G ? d_in / G : 1;
  const float* wrow = Wp + (static_cast<int64_t>(e) * d_out + r) * d_in + j0;
  float w[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) w[m] = wrow[4 * m + k];
  float* sc = scales + static_cast<int64_t>(e) * n_groups * d_out;
  uint8_t* zr = zeros + static_cast<int64_t>(e) * n_groups * d_out;
  float s = 1.0f, z = 0.0f, inv_s = 1.0f;
  if constexpr (G == 0) {
    s = sc[r];
    z = static_cast<float>(zr[r]);
    inv_s = 1.0f / s;
  }
  uint32_t cw[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) cw[i] = 0u;
  const float* ul_k = &Ul[0][k][0];

#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const int mj = j >> 2;
    if constexpr (G != 0) {
      if (j % G == 0) {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int m = j / 4; m < (j + G) / 4; ++m) {
          lo = fminf(lo, w[m]);
          hi = fmaxf(hi, w[m]);
        }
        lo = quad_min(lo);
        hi = quad_max(hi);
        s = fmaxf((hi - lo) / maxq, 1e-8f);
        z = rintf(-lo / s);
        inv_s = 1.0f / s;
        if (k == 0) {
          const int gi = (j0 + j) / G;
          sc[static_cast<int64_t>(gi) * d_out + r] = s;
          zr[static_cast<int64_t>(gi) * d_out + r] = static_cast<uint8_t>(z);
        }
      }
    }
    float wj;
    switch (j & 3) {
      case 0: wj = quad_bcast<0>(w[mj]); break;
      case 1: wj = quad_bcast<1>(w[mj]); break;
      case 2: wj = quad_bcast<2>(w[mj]); break;
      default: wj = quad_bcast<3>(w[mj]); break;
    }
    const float q = fminf(fmaxf(rintf(wj * inv_s) + z, 0.0f), maxq);
    const float wq = s * (q - z);
    const float e_j = (wj - wq) * inv_d[j];
    cw[j >> 2] |= static_cast<uint32_t>(q) << (8 * (j & 3));
    // update this lane's columns 4m + k > j (the LDS factor is zero for columns <= j)
    const float* urow = ul_k + j * (4 * QP);
#pragma unroll
    for (int m = mj; m < 32; ++m) w[m] = fmaf(-e_j, urow[m], w[m]);
    if (k == (j & 3)) w[mj] = e_j;   // the owner keeps err_j in place of w_j
  }
  // codes: every lane holds all 128; lane k stores words [8k, 8k+8)
  uint32_t* cdst = reinterpret_cast<uint32_t*>(codes_p + (static_cast<int64_t>(e) * d_out + r) * d_in + j0);
  // lane-dependent word choice by masks (keeps cw[] in registers; no dynamic indexing)
  const uint32_t m0 = k == 0 ? ~0u : 0u, m1 = k == 1 ? ~0u : 0u, m2 = k == 2 ? ~0u : 0u, m3 = k == 3 ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    cdst[8 * k + i] = (cw[i] & m0) | (cw[8 + i] & m1) | (cw[16 + i] & m2) | (cw[24 + i] & m3);
  float* edst = err + (static_cast<int64_t>(e) * d_out + r) * d_in + j0;
#pragma unroll
  for (int m = 0; m < 32; ++m) edst[4 * m + k] = w[m];
}

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
  GPTQ_LAUNCH(block_sweep_quad_kernel<G>, grid, dim3(256), 0, stream, Wp, U, bsu, d_out, d_in, blk, maxq, scales,
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
  GPTQ_LAUNCH(inverse_perm_kernel, dim3(cb, batch), blk, 0, stream, perm, d_in, w.inv);
  if (G == 0) {
    GPTQ_LAUNCH(row_grid_kernel, dim3(d_out, batch), blk, 0, stream, w.Wp, d_out, d_in, maxq, scales, zeros);
  }
  const dim3 sg((d_out + 63) / 64, batch);
  const gptq_status st = sweep_range(0, d_in / kBlock, G, sg, stream, batch, d_out, d_in, w, U, bsu, maxq, scales,
                                     zeros);
  if (st != GPTQ_OK) return st;
  GPTQ_LAUNCH(unpermute_kernel, pg, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G, codes, g_idx);
  return GPTQ_OK;
}

}  // namespace gptq
