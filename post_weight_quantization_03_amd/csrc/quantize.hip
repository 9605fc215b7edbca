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
//     block_sweep:   16 lanes per row keep the row's 128 block columns in registers
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

// Grid of one row segment from its range widened to contain 0, [lo, hi] with lo <= 0 <=
// hi ("GPTQ Architecture, in depth", "The algorithm in code" and "Groups, act-order and
// other knobs"): asymmetric, step (hi - lo) / maxq and zero level rne(-lo / step); or
// symmetric, step max|w| / (2^(bits-1) - 1) and zero level fixed at 2^(bits-1) (the grid
// of "Same Ruler, Smarter Placement: GPTQ", 1.11).  The step is never below 1e-8.
__device__ __forceinline__ void fit_grid(float lo, float hi, float maxq, bool sym, float& s, float& z) {
  if (sym) {
    const float half = 0.5f * (maxq + 1.0f);
    s = fmaxf(fmaxf(-lo, hi) / (half - 1.0f), 1e-8f);
    z = half;
  } else {
    s = fmaxf((hi - lo) / maxq, 1e-8f);
    z = rintf(-lo / s);
  }
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

// A row of W is spread over LPR lanes (16: one DPP row; 4: one DPP quad).  Broadcast of
// lane `src` of the group, and min / max over the group.
template <int LPR, int src>
__device__ __forceinline__ float grp_bcast(float v) {
  if constexpr (LPR == 16) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + src, 0xF, 0xF, false));
  else return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), src * 0x55, 0xF, 0xF, false));
}
template <int ctrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}
// row_ror:n = 0x120 + n; quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E
template <int LPR>
__device__ __forceinline__ float grp_min(float v) {
  if constexpr (LPR == 16) {
    v = fminf(v, dpp_f<0x128>(v));
    v = fminf(v, dpp_f<0x124>(v));
    v = fminf(v, dpp_f<0x122>(v));
    return fminf(v, dpp_f<0x121>(v));
  } else {
    v = fminf(v, dpp_f<0xB1>(v));
    return fminf(v, dpp_f<0x4E>(v));
  }
}
template <int LPR>
__device__ __forceinline__ float grp_max(float v) {
  if constexpr (LPR == 16) {
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x122>(v));
    return fmaxf(v, dpp_f<0x121>(v));
  } else {
    v = fmaxf(v, dpp_f<0xB1>(v));
    return fmaxf(v, dpp_f<0x4E>(v));
  }
}

// One 128-column block of the sweep.  G = group size (16, 32, 64 or 128), or 0 for the
// per-row grid already written by row_grid_kernel.  kStatic (with G = 0): every column
// takes the grid of its original group, perm[column] / gsz, written before the sweep by
// static_grid_kernel; each lane loads the grids of its own columns once and the column's
// owner broadcasts them with the column value.  sym selects the symmetric grid at group
// starts.  NT threads per workgroup, LPR lanes per row of W, so NT / LPR rows per workgroup.
//
// Lane k of a row keeps the C = 128 / LPR columns LPR m + k (m = 0..C-1) in registers.
// For column j the owner lane's value is broadcast to the row's lanes, every lane of the
// row quantizes it (so all hold err_j and code_j), and each lane updates its own later
// columns: with the columns interleaved every lane has the same number of them, so the
// update loop starts at a compile-time index.  Fewer lanes per row repeat the per-column
// quantization on fewer lanes (4 lanes: a quarter of the instructions per row and column
// of 16), but need 4x the rows to fill the chip.  The U block sits in LDS as
// Ul[j][CP k + m] = U[j0 + j][j0 + LPR m + k] with its diagonal zeroed (1/U_jj kept apart):
// a lane's update reads are contiguous, the rows of a wave read the same words, and
// columns at or before j get a zero factor.  At a group start the grid is fitted on the
// row's current values of the group's columns (min/max reduced over the row's lanes).
template <int G, int NT, int LPR, bool kStatic>
__global__ __launch_bounds__(NT) void block_sweep_kernel(const float* __restrict__ Wp, const float* __restrict__ U,
                                                         int64_t bsu, int d_out, int d_in, int blk, float maxq,
                                                         int sym, const int32_t* __restrict__ perm, int gsz,
                                                         float* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                         uint8_t* __restrict__ codes_p, float* __restrict__ err) {
  constexpr int C = kBlock / LPR;   // columns per lane
  constexpr int CW = C / 4;         // code words per lane
  constexpr int CQ = C / 4;         // float4 of a U row per lane
  // a lane's slice of a U row in LDS: padded at 4 lanes per row, so that the four lanes'
  // 16-byte reads start on different banks (unpadded, 32 floats apart, they collide)
  constexpr int CP = LPR == 4 ? C + 4 : C;
  constexpr int UR = LPR * CP;      // floats per staged U row
  static_assert(G == 0 || G % LPR == 0, "a group spans whole registers");
  static_assert(!kStatic || G == 0, "static groups are fitted before the sweep");
  __shared__ __attribute__((aligned(16))) float Ul[kBlock * UR];
  __shared__ float inv_d[kBlock];
  const int e = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blk * kBlock;
  const float* Ub = U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(j0) * d_in + j0;
  const int r = blockIdx.x * (NT / LPR) + tid / LPR;
  const int k = tid % LPR;
  const bool live = r < d_out;
  // the row's block columns are fetched first, so they arrive while U is staged
  const float* wrow = Wp + (static_cast<int64_t>(e) * d_out + (live ? r : 0)) * d_in + j0;
  float w[C];
#pragma unroll
  for (int m = 0; m < C; ++m) w[m] = wrow[LPR * m + k];
  // stage the U block: item i = (row j, lane kk) gathers U[j][LPR m + kk], m = 0..C-1 (each
  // load instruction reads LPR consecutive floats per row) and writes them as C
  // consecutive floats.  A thread's items are all loaded before any is stored, so their
  // loads overlap (one item at a time left the block's 64 KB as SI serial load latencies).
  constexpr int ITEMS = kBlock * LPR;
  constexpr int SI = (ITEMS + NT - 1) / NT;   // items per thread
  {
    float v[SI][C];
#pragma unroll
    for (int s = 0; s < SI; ++s) {
      const int i = tid + s * NT;
      if (ITEMS % NT == 0 || i < ITEMS) {
        const float* src = Ub + static_cast<int64_t>(i / LPR) * d_in + i % LPR;
#pragma unroll
        for (int m = 0; m < C; ++m) v[s][m] = src[LPR * m];
      }
    }
#pragma unroll
    for (int s = 0; s < SI; ++s) {
      const int i = tid + s * NT;
      if (ITEMS % NT == 0 || i < ITEMS) {
        const int j = i / LPR, kk = i % LPR;
#pragma unroll
        for (int m = 0; m < C; ++m) {
          if (LPR * m + kk == j) {
            inv_d[j] = 1.0f / v[s][m];
            v[s][m] = 0.0f;
          }
        }
        float4* dst = reinterpret_cast<float4*>(Ul + j * UR + CP * kk);
#pragma unroll
        for (int q = 0; q < CQ; ++q)
          dst[q] = make_float4(v[s][4 * q], v[s][4 * q + 1], v[s][4 * q + 2], v[s][4 * q + 3]);
      }
    }
  }
  __syncthreads();
  if (!live) return;   // whole rows leave together; no barrier follows
  const int n_groups = G ? d_in / G : (kStatic ? d_in / gsz : 1);
  float* sc = scales + static_cast<int64_t>(e) * n_groups * d_out;
  uint8_t* zr = zeros + static_cast<int64_t>(e) * n_groups * d_out;
  float s = 1.0f, z = 0.0f, inv_s = 1.0f;
  // static groups: the grid of each of this lane's columns (scale, 1 / scale, zero)
  constexpr int CS = kStatic ? C : 1;
  float g_s[CS], g_is[CS], g_z[CS];
  if constexpr (kStatic) {
    const int32_t* pe = perm + static_cast<int64_t>(e) * d_in + j0;
#pragma unroll
    for (int m = 0; m < C; ++m) {
      const int c = min(max(pe[LPR * m + k], 0), d_in - 1);
      const int64_t o = static_cast<int64_t>(c / gsz) * d_out + r;
      g_s[m] = sc[o];
      g_z[m] = static_cast<float>(zr[o]);
      g_is[m] = 1.0f / g_s[m];
    }
  } else if constexpr (G == 0) {
    s = sc[r];
    z = static_cast<float>(zr[r]);
    inv_s = 1.0f / s;
  }
  // Codes.  16 lanes per row: the owner of a column keeps its code, as it keeps its error,
  // and each lane stores the codes of its own columns.  4 lanes per row: lane k packs the
  // codes of columns C k .. C k + C - 1 (every lane has every code).
  constexpr bool kOwnCodes = LPR == 16;
  float qv[kOwnCodes ? C : 1];
  uint32_t cw[kOwnCodes ? 1 : CW];
  if constexpr (!kOwnCodes) {
#pragma unroll
    for (int q = 0; q < CW; ++q) cw[q] = 0u;
  }
  float zmax = maxq - z;   // upper clamp of code - zero for the current group
  const float* ul_k = Ul + CP * k;
  // U row j is read into registers one column ahead (two alternating sets), so that the
  // LDS latency stays off the column-to-column chain
  float4 ua[CQ], ub[CQ];
#pragma unroll
  for (int q = 0; q < CQ; ++q) ua[q] = reinterpret_cast<const float4*>(ul_k)[q];
  float dja = inv_d[0], djb = 0.0f;

  static_for(std::make_integer_sequence<int, kBlock>{}, [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int mj = j / LPR;
    float4* cur = (j & 1) ? ub : ua;
    float4* nxt = (j & 1) ? ua : ub;
    const float dj = (j & 1) ? djb : dja;
    if constexpr (j + 1 < kBlock) {
      const float4* un = reinterpret_cast<const float4*>(ul_k + (j + 1) * UR);
      static_for(std::make_integer_sequence<int, CQ>{}, [&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (4 * q + 3 >= (j + 1) / LPR) nxt[q] = un[q];
      });
      if constexpr (j & 1) dja = inv_d[j + 1];
      else djb = inv_d[j + 1];
      // the scheduler would sink these reads next to their use in the next column
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (G != 0 && j % G == 0) {
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int m = j / LPR; m < (j + G) / LPR; ++m) {
        lo = fminf(lo, w[m]);
        hi = fmaxf(hi, w[m]);
      }
      lo = grp_min<LPR>(lo);
      hi = grp_max<LPR>(hi);
      fit_grid(lo, hi, maxq, sym != 0, s, z);
      inv_s = 1.0f / s;
      zmax = maxq - z;
      if (k == 0) {
        const int gi = (j0 + j) / G;
        sc[static_cast<int64_t>(gi) * d_out + r] = s;
        zr[static_cast<int64_t>(gi) * d_out + r] = static_cast<uint8_t>(z);
      }
    }
    if constexpr (kStatic) {
      s = grp_bcast<LPR, j % LPR>(g_s[mj]);
      inv_s = grp_bcast<LPR, j % LPR>(g_is[mj]);
      z = grp_bcast<LPR, j % LPR>(g_z[mj]);
    }
    const float wj = grp_bcast<LPR, j % LPR>(w[mj]);
    // t = code - zero: round(w / s) clamped to [-z, maxq - z] (the code clamp(round(w / s)
    // + z, 0, maxq) less z, exactly), so that the dequantized value is s t and the scaled
    // error (w - s t) / U_jj takes one fused multiply-add and a multiply
    const float zq = kStatic ? maxq - z : zmax;
    const float t = __builtin_amdgcn_fmed3f(rintf(wj * inv_s), -z, zq);
    const float e_j = fmaf(-s, t, wj) * dj;
    const float q = t + z;
    if constexpr (kOwnCodes) {
      if (k == j % LPR) qv[mj] = q;   // the owner keeps the code of its column
    } else {
      cw[(j % C) / 4] |= (k == j / C) ? (static_cast<uint32_t>(q) << (8 * (j & 3))) : 0u;
    }
#pragma unroll
    for (int m = mj; m < C; ++m) {
      const float4 u4 = cur[m / 4];
      const float u = (m & 3) == 0 ? u4.x : (m & 3) == 1 ? u4.y : (m & 3) == 2 ? u4.z : u4.w;
      w[m] = fmaf(-e_j, u, w[m]);
    }
    if (k == j % LPR) w[mj] = e_j;   // the owner keeps err_j in place of w_j
  });
  uint8_t* crow = codes_p + (static_cast<int64_t>(e) * d_out + r) * d_in + j0;
  if constexpr (kOwnCodes) {
#pragma unroll
    for (int m = 0; m < C; ++m) crow[LPR * m + k] = static_cast<uint8_t>(qv[m]);
  } else {
    uint32_t* cdst = reinterpret_cast<uint32_t*>(crow + C * k);
#pragma unroll
    for (int q = 0; q < CW; q += 4) *reinterpret_cast<uint4*>(cdst + q) = make_uint4(cw[q], cw[q + 1], cw[q + 2], cw[q + 3]);
  }
  float* edst = err + (static_cast<int64_t>(e) * d_out + r) * d_in + j0;
#pragma unroll
  for (int m = 0; m < C; ++m) edst[LPR * m + k] = w[m];
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

// Launch geometry of the sweep: NT threads per workgroup, LPR lanes per row, the grid.
struct SweepShape {
  int nt, lpr;
  dim3 grid;
};

// The U block takes 64 KB of LDS, so at most two workgroups share a CU.  With rows enough
// for about one wave per SIMD at 4 lanes per row (16 rows per wave), rows get 4 lanes;
// else 16.  At 16 lanes, the largest workgroup that still gives every CU at least one.  At
// 4 lanes the sweep is bound by VALU issue and LDS reads, so its time goes with the rows
// the busiest CU takes, ceil(workgroups / 256) x rows per workgroup: of the workgroup sizes
// below, the one that makes this smallest (64 experts of 1408 rows: 704 threads, 8 x 64
// workgroups of 176 rows in two even rounds, where 1024 threads left a third of the chip
// idle in the second round).  Groups of 64 at 4 lanes per row stop at 512 threads (their
// registers would not fit more).  The small groups (16, 32) keep 16 lanes and 256
// threads: their sweeps need too many registers for more than one wave per SIMD.
constexpr int kCUs = 256;
SweepShape sweep_shape(int G, bool stat, int batch, int d_out) {
  // static groups keep 16 lanes per row: each lane also holds the grids of its columns
  const bool wide_ok = !stat && (G == 0 || G == 64 || G == 128);
  const int64_t rows = static_cast<int64_t>(batch) * d_out;
  const int lpr = (wide_ok && rows / 16 >= 768) ? 4 : 16;
  int nt = 256;
  if (wide_ok && lpr == 16) {
    for (int cand : {1024, 512}) {
      const int rpw = cand / lpr;
      if (static_cast<int64_t>((d_out + rpw - 1) / rpw) * batch >= kCUs) {
        nt = cand;
        break;
      }
    }
  } else if (wide_ok) {
    int64_t best = -1;
    for (int cand : {1024, 704, 512, 256}) {
      if (G == 64 && cand > 512) continue;   // would spill registers
      const int rpw = cand / lpr;
      const int64_t wgs = static_cast<int64_t>((d_out + rpw - 1) / rpw) * batch;
      const int64_t cost = (wgs + kCUs - 1) / kCUs * rpw;
      if (best < 0 || cost < best) {
        best = cost;
        nt = cand;
      }
    }
  }
  const int rpw = nt / lpr;
  return {nt, lpr, dim3((d_out + rpw - 1) / rpw, batch)};
}

// Arguments of every sweep launch of one quantize call.
struct SweepArgs {
  const float* Wp;
  const float* U;
  int64_t bsu;
  int d_out, d_in;
  float maxq;
  int sym;
  const int32_t* perm;   // static groups: processing position -> original column
  int gsz;               // static groups: group size
  float* scales;
  uint8_t* zeros;
  uint8_t* codes_p;
  float* err;
  bool timed;            // the launch-timing hook may bracket these launches
};

template <int G, int NT, int LPR, bool kStatic>
gptq_status launch_sweep(dim3 grid, hipStream_t stream, const SweepArgs& a, int blk) {
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (a.timed) timing_pair(GPTQ_TIME_SWEEP, &ev0, &ev1);
  if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
  GPTQ_LAUNCH((block_sweep_kernel<G, NT, LPR, kStatic>), grid, dim3(NT), 0, stream, a.Wp, a.U, a.bsu, a.d_out, a.d_in,
              blk, a.maxq, a.sym, a.perm, a.gsz, a.scales, a.zeros, a.codes_p, a.err);
  if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
  return GPTQ_OK;
}

template <int G>
gptq_status launch_sweep_nt(const SweepShape& sh, hipStream_t stream, const SweepArgs& a, int blk) {
  if constexpr (G == 0 || G == 64 || G == 128) {
#define GPTQ_SWEEP(NT, LPR) \
  if (sh.nt == NT && sh.lpr == LPR) return launch_sweep<G, NT, LPR, false>(sh.grid, stream, a, blk);
    GPTQ_SWEEP(512, 16)   // 1024 threads at 16 lanes: never chosen (4 lanes take over first)
    if constexpr (G != 64) {
      GPTQ_SWEEP(1024, 4)
      GPTQ_SWEEP(704, 4)
    }
    GPTQ_SWEEP(512, 4)
    GPTQ_SWEEP(256, 4)
#undef GPTQ_SWEEP
  }
  if (sh.nt != 256 || sh.lpr != 16) return GPTQ_ERR_UNSUPPORTED;
  return launch_sweep<G, 256, 16, false>(sh.grid, stream, a, blk);
}

gptq_status sweep_block(int b, int G, bool stat, const SweepShape& sg, hipStream_t stream, const SweepArgs& a) {
  if (stat) {
    if (sg.nt != 256 || sg.lpr != 16) return GPTQ_ERR_UNSUPPORTED;
    return launch_sweep<0, 256, 16, true>(sg.grid, stream, a, b);
  }
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
