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
//                    group scale/zero, and Err [d_out, 128].
//     lazy update:   W_p[:, j2:] -= Err @ U[b-block, j2:] on the fp32 matrix cores.
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
  float4* edst = reinterpret_cast<float4*>(err + (static_cast<int64_t>(e) * d_out + r) * kBlock);
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) edst[i] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
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
  w.err = cv.take<float>(rows * kBlock);
  w.codes_p = cv.take<uint8_t>(rows * d_in);
  w.inv = cv.take<int32_t>(static_cast<size_t>(batch) * d_in);
  w.bytes = cv.used;
  return w;
}

template <int G>
gptq_status launch_sweep(dim3 grid, hipStream_t stream, const float* Wp, const float* U, int64_t bsu, int d_out,
                         int d_in, int blk, float maxq, float* scales, uint8_t* zeros, uint8_t* codes_p,
                         float* err) {
  GPTQ_LAUNCH(block_sweep_kernel<G>, grid, dim3(64), 0, stream, Wp, U, bsu, d_out, d_in, blk, maxq, scales,
              zeros, codes_p, err);
  return GPTQ_OK;
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
  const int nblk = d_in / kBlock;
  for (int b = 0; b < nblk; ++b) {
    gptq_status st;
    switch (G) {
      case 0: st = launch_sweep<0>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err); break;
      case 16: st = launch_sweep<16>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err); break;
      case 32: st = launch_sweep<32>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err); break;
      case 64: st = launch_sweep<64>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err); break;
      case 128: st = launch_sweep<128>(sg, stream, w.Wp, U, bsu, d_out, d_in, b, maxq, scales, zeros, w.codes_p, w.err); break;
      default: return GPTQ_ERR_UNSUPPORTED;
    }
    if (st != GPTQ_OK) return st;
    const int j2 = (b + 1) * kBlock;
    if (j2 < d_in) {
      GemmArgs g{};
      g.M = d_out; g.N = d_in - j2; g.K = kBlock;
      g.A = w.err; g.lda = kBlock; g.sA = static_cast<int64_t>(d_out) * kBlock;
      g.B = U + static_cast<int64_t>(b) * kBlock * d_in + j2; g.ldb = d_in; g.sB = bsu;
      g.C = w.Wp + j2; g.ldc = d_in; g.sC = static_cast<int64_t>(d_out) * d_in;
      g.alpha = -1.0f; g.beta = 1.0f; g.transB = 0; g.flags = 0; g.batch = batch;
      st = gemm_f32(g, stream);
      if (st != GPTQ_OK) return st;
    }
  }
  GPTQ_LAUNCH(unpermute_kernel, pg, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G, codes, g_idx);
  return GPTQ_OK;
}

}  // namespace gptq
