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
//   static_grid:     static groups only: the grid of every group of original columns,
//                    fitted on W before the sweep
//   per block b of 128 columns:
//     block_sweep:   (sweep.h) 16 lanes per row keep the row's 128 block columns in registers
//                    (8 each); the column value is broadcast within the row by DPP and
//                    quantized by all 16; U's diagonal block sits in LDS.  Outputs codes
//                    (processing order), the group scale/zero, and the block's columns
//                    of Err.
//     lazy update:   hierarchical (see sweep_range): W_p[:, right] -= Err[:, left] @ U[left,
//                    right] as fp32-accurate matrix-core products (split-bf16 when large),
//                    Err [d_out, d_in] in processing order.
//   unpermute:       codes back to original column order; g_idx.
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "sweep.h"

// Scratch of the allocation-free entry point (gptq_quantize_layer_noalloc): a fixed array
// of device memory, one per GPU that the library runs on, held until the process ends.
// Host code never uses the array's name as an address: its device address is looked up
// once per device (scratch_address below) and kept.
static __device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

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
  // a malformed permutation is clamped into range rather than addressing outside W
  batched_copy<256>(
      t, d_in,
      [&](int j) -> uint16_t {
        const int c = min(max(perm[static_cast<int64_t>(e) * d_in + j], 0), d_in - 1);
        return dead[static_cast<int64_t>(e) * d_in + c] ? kDeadCol : static_cast<uint16_t>(c);
      },
      [&](int j, uint16_t v) { sidx[j] = v; });
  for (int i = 0; i < STAGE_ROWS; ++i) {
    const int r = blockIdx.x * STAGE_ROWS + i;
    if (r >= d_out) break;
    __syncthreads();  // sidx written / the previous row fully consumed
    const T* src = W + static_cast<int64_t>(e) * bsw + static_cast<int64_t>(r) * ldw;
    if constexpr (kVec && sizeof(T) == 2) {
      batched_copy<256>(t, d_in / 8, [&](int c8) { return reinterpret_cast<const uint4*>(src)[c8]; },
                        [&](int c8, uint4 v) {
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
                        });
    } else if constexpr (kVec) {
      batched_copy<256>(t, d_in / 4, [&](int c4) { return reinterpret_cast<const float4*>(src)[c4]; },
                        [&](int c4, float4 v) { reinterpret_cast<float4*>(srow)[c4] = v; });
    } else {
      batched_copy<256>(t, d_in, [&](int c) { return load_as_f32(src + c); }, [&](int c, float v) { srow[c] = v; });
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
                                                       float maxq, int sym, float* __restrict__ scales,
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
    float s, z;
    fit_grid(slo[0], shi[0], maxq, sym != 0, s, z);
    scales[static_cast<int64_t>(e) * d_out + r] = s;
    zeros[static_cast<int64_t>(e) * d_out + r] = static_cast<uint8_t>(z);
  }
}

// Static groups: the grid of every group of G consecutive ORIGINAL columns, fitted once on
// the dead-zeroed W before the sweep -> scales / zeros [e][group][row].  One thread per
// (group, row), rows fastest so that the stores are coalesced.
template <typename T>
__global__ __launch_bounds__(256) void static_grid_kernel(const T* __restrict__ W, int64_t ldw, int64_t bsw,
                                                          const uint8_t* __restrict__ dead, int d_out, int d_in,
                                                          int G, float maxq, int sym, float* __restrict__ scales,
                                                          uint8_t* __restrict__ zeros) {
  const int ng = d_in / G;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (i >= static_cast<int64_t>(ng) * d_out) return;
  const int r = static_cast<int>(i % d_out), gi = static_cast<int>(i / d_out);
  const T* row = W + static_cast<int64_t>(e) * bsw + static_cast<int64_t>(r) * ldw + static_cast<int64_t>(gi) * G;
  const uint8_t* de = dead + static_cast<int64_t>(e) * d_in + static_cast<int64_t>(gi) * G;
  float lo = 0.0f, hi = 0.0f;
  for (int c = 0; c < G; ++c) {
    const float v = de[c] ? 0.0f : load_as_f32(row + c);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  float s, z;
  fit_grid(lo, hi, maxq, sym != 0, s, z);
  const int64_t o = (static_cast<int64_t>(e) * ng + gi) * d_out + r;
  scales[o] = s;
  zeros[o] = static_cast<uint8_t>(z);
}


// codes[:, c] = codes_p[:, inv[c]]; g_idx[c] = inv[c] / group.  Staged like the weight
// permute: inv once per workgroup, each codes_p row in LDS, 16 codes per thread per store.
// kVec: the codes rows are 16-byte aligned.
// by_orig (static groups): g_idx[c] = c / group.
template <int DMAX, bool kVec>
__global__ __launch_bounds__(256) void unpermute_staged_kernel(const uint8_t* __restrict__ codes_p,
                                                               const int32_t* __restrict__ inv, int d_out,
                                                               int d_in, int group, int by_orig,
                                                               uint8_t* __restrict__ codes,
                                                               int32_t* __restrict__ g_idx) {
  __shared__ __attribute__((aligned(16))) uint8_t srow[DMAX];
  __shared__ uint16_t sidx[DMAX];
  const int e = blockIdx.y, t = threadIdx.x;
  batched_copy<256>(t, d_in, [&](int c) { return min(max(inv[static_cast<int64_t>(e) * d_in + c], 0), d_in - 1); },
                    [&](int c, int j) {
                      sidx[c] = static_cast<uint16_t>(j);
                      if (blockIdx.x == 0)
                        g_idx[static_cast<int64_t>(e) * d_in + c] = group > 0 ? (by_orig ? c : j) / group : 0;
                    });
  for (int i = 0; i < STAGE_ROWS; ++i) {
    const int r = blockIdx.x * STAGE_ROWS + i;
    if (r >= d_out) break;
    __syncthreads();
    const int64_t ro = (static_cast<int64_t>(e) * d_out + r) * d_in;
    // codes_p rows start at multiples of d_in (a multiple of 128) in a 256-byte aligned workspace
    batched_copy<256>(t, d_in / 16, [&](int c16) { return reinterpret_cast<const uint4*>(codes_p + ro)[c16]; },
                      [&](int c16, uint4 v) { reinterpret_cast<uint4*>(srow)[c16] = v; });
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
                                                        int group, int by_orig, uint8_t* __restrict__ codes,
                                                        int32_t* __restrict__ g_idx) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (c >= d_in) return;
  const int j = min(max(inv[static_cast<int64_t>(e) * d_in + c], 0), d_in - 1);
  const int64_t ro = (static_cast<int64_t>(e) * d_out + r) * d_in;
  codes[ro + c] = codes_p[ro + j];
  if (r == 0) g_idx[static_cast<int64_t>(e) * d_in + c] = group > 0 ? (by_orig ? c : j) / group : 0;
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

// The U block takes 64 KB of LDS, so at most two workgroups share a CU.  With rows enough
// for about one wave per SIMD at 4 lanes per row (16 rows per wave), rows get 4 lanes;
// else 16.  At 16 lanes, the largest workgroup that still gives every CU at least one.  At
// 4 lanes the sweep is bound by VALU issue and LDS reads, so its time goes with the rows
// the busiest CU takes, ceil(workgroups / 256) x rows per workgroup: of the workgroup sizes
// below, with one or two rows per lane, the one that makes this smallest, a lane's second
// row counted as half a row (it shares the lane's U reads and loop overhead).  64 experts
// of 1408 rows: 704 threads with two rows per lane, one workgroup of 352 rows per CU
// (sweep 74 -> 55 us against two rounds of 176 rows at one row per lane, where 1024
// threads at one row left a third of the chip idle in the second round); 14336 rows: one
// row per lane (two would leave half the SIMDs without a wave).  Groups of 64 at 4 lanes
// per row stop at 512 threads and one row (their registers would not fit more).  The small
// groups (16, 32) keep 16 lanes and 256 threads: their sweeps need too many registers for
// more than one wave per SIMD.
constexpr int kCUs = 256;
SweepShape sweep_shape(int G, bool stat, int batch, int d_out) {
  // static groups keep 16 lanes per row: each lane also holds the grids of its columns
  const bool wide_ok = !stat && (G == 0 || G == 64 || G == 128);
  const int64_t rows = static_cast<int64_t>(batch) * d_out;
  const int lpr = (wide_ok && rows / 16 >= 768) ? 4 : 16;
  int nt = 256, rpl = 1;
  if (wide_ok && lpr == 16) {
    for (int cand : {1024, 512}) {
      const int rpw = cand / lpr;
      if (static_cast<int64_t>((d_out + rpw - 1) / rpw) * batch >= kCUs) {
        nt = cand;
        break;
      }
    }
  } else if (wide_ok) {
    // cost in row-steps of the busiest CU; a lane's second row costs half a row (4 x the
    // cost compared against 3 x for two rows per lane)
    int64_t best = -1;
    for (int two = 0; two < 2; ++two) {
      if (two && G == 64) continue;   // would spill registers
      for (int cand : {1024, 704, 512, 256}) {
        if ((G == 64 || two) && cand > 512 + 192 * two) continue;   // would spill registers
        const int rpw = cand / lpr * (two + 1);
        const int64_t wgs = static_cast<int64_t>((d_out + rpw - 1) / rpw) * batch;
        const int64_t cost = (wgs + kCUs - 1) / kCUs * rpw * (two ? 3 : 4);
        if (best < 0 || cost < best) {
          best = cost;
          nt = cand;
          rpl = two + 1;
        }
      }
    }
  }
  const int rpw = nt / lpr * rpl;
  return {nt, lpr, rpl, dim3((d_out + rpw - 1) / rpw, batch)};
}

gptq_status sweep_block(int b, int G, bool stat, const SweepShape& sg, hipStream_t stream, const SweepArgs& a) {
  if (stat) return launch_sweep_static(sg, stream, a, b);
  switch (G) {
    case 0: return launch_sweep_nt<0>(sg, stream, a, b);
    case 16: return launch_sweep_nt<16>(sg, stream, a, b);
    case 32: return launch_sweep_nt<32>(sg, stream, a, b);
    case 64: return launch_sweep_nt<64>(sg, stream, a, b);
    case 128: return launch_sweep_nt<128>(sg, stream, a, b);
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
gptq_status sweep_range(int b0, int b1, int G, bool stat, const SweepShape& sg, hipStream_t stream, int batch,
                        const SweepArgs& a) {
  if (b1 - b0 == 1) return sweep_block(b0, G, stat, sg, stream, a);
  const int bm = b0 + (b1 - b0) / 2;
  gptq_status st = sweep_range(b0, bm, G, stat, sg, stream, batch, a);
  if (st != GPTQ_OK) return st;
  const int d_in = a.d_in;
  GemmArgs g{};
  g.M = a.d_out; g.N = (b1 - bm) * kBlock; g.K = (bm - b0) * kBlock;
  g.A = a.err + static_cast<int64_t>(b0) * kBlock; g.lda = d_in; g.sA = static_cast<int64_t>(a.d_out) * d_in;
  g.B = a.U + static_cast<int64_t>(b0) * kBlock * d_in + static_cast<int64_t>(bm) * kBlock; g.ldb = d_in; g.sB = a.bsu;
  g.C = const_cast<float*>(a.Wp) + static_cast<int64_t>(bm) * kBlock; g.ldc = d_in;
  g.sC = static_cast<int64_t>(a.d_out) * d_in;
  g.alpha = -1.0f; g.beta = 1.0f; g.transB = 0; g.flags = 0; g.batch = batch; g.role = 1;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (a.timed) timing_pair(GPTQ_TIME_LAZY_GEMM, &ev0, &ev1);
  if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
  if ((st = gemm_f32(g, stream)) != GPTQ_OK) return st;
  if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
  return sweep_range(bm, b1, G, stat, sg, stream, batch, a);
}

}  // namespace

size_t quantize_workspace(int batch, int d_out, int d_in, const gptq_params&) {
  if (batch < 1 || d_out < 1 || d_in < kBlock) return 0;
  return carve(nullptr, batch, d_out, d_in).bytes + 256;
}

namespace {

gptq_status quantize_impl(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W, int64_t ldw,
                          int64_t bsw, const float* U, int64_t bsu, const int32_t* perm, const uint8_t* dead,
                          const gptq_params& p, uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                          void* ws, size_t ws_bytes, hipStream_t stream, bool timed) {
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
  const bool stat = p.static_groups != 0 && G > 0;
  if (G == 0) {
    GPTQ_LAUNCH(row_grid_kernel, dim3(d_out, batch), blk, 0, stream, w.Wp, d_out, d_in, maxq, p.sym, scales, zeros);
  } else if (stat) {
    const dim3 gg(static_cast<unsigned>((static_cast<int64_t>(d_in / G) * d_out + 255) / 256), batch);
    switch (w_dtype) {
      case GPTQ_F32:
        GPTQ_LAUNCH(static_grid_kernel<float>, gg, blk, 0, stream, static_cast<const float*>(W), ldw, bsw, dead, d_out,
                    d_in, G, maxq, p.sym, scales, zeros);
        break;
      case GPTQ_BF16:
        GPTQ_LAUNCH(static_grid_kernel<BF16>, gg, blk, 0, stream, static_cast<const BF16*>(W), ldw, bsw, dead, d_out,
                    d_in, G, maxq, p.sym, scales, zeros);
        break;
      case GPTQ_F16:
        GPTQ_LAUNCH(static_grid_kernel<F16>, gg, blk, 0, stream, static_cast<const F16*>(W), ldw, bsw, dead, d_out,
                    d_in, G, maxq, p.sym, scales, zeros);
        break;
    }
  }
  const SweepShape sg = sweep_shape(G, stat, batch, d_out);
  const SweepArgs sa{w.Wp, U, bsu, d_out, d_in, maxq, p.sym, perm, G, scales, zeros, w.codes_p, w.err, timed};
  const gptq_status st = sweep_range(0, d_in / kBlock, stat ? 0 : G, stat, sg, stream, batch, sa);
  if (st != GPTQ_OK) return st;
  {
    const bool vec = reinterpret_cast<uintptr_t>(codes) % 16 == 0;
    auto staged = [&](auto dmax) {
      constexpr int DM = decltype(dmax)::value;
      if (vec) GPTQ_LAUNCH((unpermute_staged_kernel<DM, true>), sgr, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G,
                           int(stat), codes, g_idx);
      else GPTQ_LAUNCH((unpermute_staged_kernel<DM, false>), sgr, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G,
                       int(stat), codes, g_idx);
      return GPTQ_OK;
    };
    gptq_status st = GPTQ_OK;
    if (d_in <= 4096) st = staged(std::integral_constant<int, 4096>{});
    else if (d_in <= kStagedMax) st = staged(std::integral_constant<int, kStagedMax>{});
    else GPTQ_LAUNCH(unpermute_kernel, pg, blk, 0, stream, w.codes_p, w.inv, d_out, d_in, G, int(stat), codes, g_idx);
    if (st != GPTQ_OK) return st;
  }
  return GPTQ_OK;
}

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
gptq_status scratch_address(void** out) {
  int dev = 0;
  GPTQ_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices) return GPTQ_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(::scratch)) != hipSuccess || ptr == nullptr) return GPTQ_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GPTQ_OK;
}

}  // namespace

gptq_status quantize_enqueue(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W, int64_t ldw,
                             int64_t bsw, const float* U, int64_t bsu, const int32_t* perm, const uint8_t* dead,
                             const gptq_params& p, uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  return quantize_impl(batch, d_out, d_in, w_dtype, W, ldw, bsw, U, bsu, perm, dead, p, codes, scales, zeros, g_idx,
                       ws, ws_bytes, stream, true);
}

// The same kernels with the scratch array as the workspace.  Everything the kernels read
// from the scratch they have written earlier in the same call (the permuted weights, the
// errors, the processing-order codes, the inverse permutation), so nothing needs clearing.
// No event is recorded (the timing hook would create events).
gptq_status quantize_noalloc_enqueue(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W,
                                     int64_t ldw, int64_t bsw, const float* U, int64_t bsu, const int32_t* perm,
                                     const uint8_t* dead, const gptq_params& p, uint8_t* codes, float* scales,
                                     uint8_t* zeros, int32_t* g_idx, hipStream_t stream) {
  if (carve(nullptr, batch, d_out, d_in).bytes > kNoAllocScratchBytes) return GPTQ_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (const gptq_status st = scratch_address(&ws); st != GPTQ_OK) return st;
  return quantize_impl(batch, d_out, d_in, w_dtype, W, ldw, bsw, U, bsu, perm, dead, p, codes, scales, zeros, g_idx,
                       ws, kNoAllocScratchBytes, stream, false);
}

}  // namespace gptq
