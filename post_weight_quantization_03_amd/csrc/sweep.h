// Column sweep of the GPTQ quantizer on gfx950: the block sweep kernel, its launch shape
// and its launchers ("Same Ruler, Smarter Placement: GPTQ", 1.5 and 1.8; "GPTQ
// Architecture, in depth", "The algorithm in code").  The kernel's instantiations are
// compiled in sources of their own (sweep_g0.hip, sweep_g128.hip, sweep_misc.hip), which
// build in parallel; quantize.hip launches them through launch_sweep_nt and
// launch_sweep_static.
#pragma once

#include <utility>

#include "common.h"

namespace gptq {

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
// starts.  NT threads per workgroup, LPR lanes per row of W, RPL rows per lane (1, or 2 at
// 4 lanes per row: the two rows, NT / LPR apart, are independent chains that share every
// read of U and halve its LDS traffic per row), so RPL NT / LPR rows per workgroup.
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
template <int G, int NT, int LPR, bool kStatic, int RPL>
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
  constexpr int RW = NT / LPR;      // rows of one pass over the workgroup's lanes
  static_assert(G == 0 || G % LPR == 0, "a group spans whole registers");
  static_assert(!kStatic || G == 0, "static groups are fitted before the sweep");
  static_assert(RPL == 1 || (RPL == 2 && !kStatic), "two rows per lane: not with static groups");
  __shared__ __attribute__((aligned(16))) float Ul[kBlock * UR];
  __shared__ float inv_d[kBlock];
  const int e = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blk * kBlock;
  const float* Ub = U + static_cast<int64_t>(e) * bsu + static_cast<int64_t>(j0) * d_in + j0;
  const int k = tid % LPR;
  // rows rw[i] = first + i RW: a lane's rows are independent chains that share every U read
  int rw[RPL];
  bool live[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    rw[i] = blockIdx.x * (RW * RPL) + i * RW + tid / LPR;
    live[i] = rw[i] < d_out;
  }
  // the rows' block columns are fetched first, so they arrive while U is staged (a row past
  // d_out reads row 0 and stores nothing)
  float w[RPL][C];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const float* wrow = Wp + (static_cast<int64_t>(e) * d_out + (live[i] ? rw[i] : 0)) * d_in + j0;
#pragma unroll
    for (int m = 0; m < C; ++m) w[i][m] = wrow[LPR * m + k];
  }
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
  if (!live[0]) return;   // whole rows leave together (the later rows too); no barrier follows
  const int n_groups = G ? d_in / G : (kStatic ? d_in / gsz : 1);
  float* sc = scales + static_cast<int64_t>(e) * n_groups * d_out;
  uint8_t* zr = zeros + static_cast<int64_t>(e) * n_groups * d_out;
  float s[RPL], z[RPL], inv_s[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    s[i] = 1.0f;
    z[i] = 0.0f;
    inv_s[i] = 1.0f;
  }
  // static groups: the grid of each of this lane's columns (scale, 1 / scale, zero)
  constexpr int CS = kStatic ? C : 1;
  float g_s[CS], g_is[CS], g_z[CS];
  if constexpr (kStatic) {
    const int32_t* pe = perm + static_cast<int64_t>(e) * d_in + j0;
#pragma unroll
    for (int m = 0; m < C; ++m) {
      const int c = min(max(pe[LPR * m + k], 0), d_in - 1);
      const int64_t o = static_cast<int64_t>(c / gsz) * d_out + rw[0];
      g_s[m] = sc[o];
      g_z[m] = static_cast<float>(zr[o]);
      g_is[m] = 1.0f / g_s[m];
    }
  } else if constexpr (G == 0) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int rr = live[i] ? rw[i] : rw[0];
      s[i] = sc[rr];
      z[i] = static_cast<float>(zr[rr]);
      inv_s[i] = 1.0f / s[i];
    }
  }
  // Codes.  16 lanes per row: the owner of a column keeps its code, as it keeps its error,
  // and each lane stores the codes of its own columns.  4 lanes per row: lane k packs the
  // codes of columns C k .. C k + C - 1 (every lane has every code).
  constexpr bool kOwnCodes = LPR == 16;
  float qv[RPL][kOwnCodes ? C : 1];
  uint32_t cw[RPL][kOwnCodes ? 1 : CW];
  if constexpr (!kOwnCodes) {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int q = 0; q < CW; ++q) cw[i][q] = 0u;
  }
  float zmax[RPL];   // upper clamp of code - zero for the current group
#pragma unroll
  for (int i = 0; i < RPL; ++i) zmax[i] = maxq - z[i];
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
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int m = j / LPR; m < (j + G) / LPR; ++m) {
          lo = fminf(lo, w[i][m]);
          hi = fmaxf(hi, w[i][m]);
        }
        lo = grp_min<LPR>(lo);
        hi = grp_max<LPR>(hi);
        fit_grid(lo, hi, maxq, sym != 0, s[i], z[i]);
        inv_s[i] = 1.0f / s[i];
        zmax[i] = maxq - z[i];
        if (k == 0 && live[i]) {
          const int gi = (j0 + j) / G;
          sc[static_cast<int64_t>(gi) * d_out + rw[i]] = s[i];
          zr[static_cast<int64_t>(gi) * d_out + rw[i]] = static_cast<uint8_t>(z[i]);
        }
      }
    }
    if constexpr (kStatic) {
      s[0] = grp_bcast<LPR, j % LPR>(g_s[mj]);
      inv_s[0] = grp_bcast<LPR, j % LPR>(g_is[mj]);
      z[0] = grp_bcast<LPR, j % LPR>(g_z[mj]);
    }
    float e_j[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float wj = grp_bcast<LPR, j % LPR>(w[i][mj]);
      // t = code - zero: round(w / s) clamped to [-z, maxq - z] (the code clamp(round(w / s)
      // + z, 0, maxq) less z, exactly), so that the dequantized value is s t and the scaled
      // error (w - s t) / U_jj takes one fused multiply-add and a multiply
      const float zq = kStatic ? maxq - z[i] : zmax[i];
      const float t = __builtin_amdgcn_fmed3f(rintf(wj * inv_s[i]), -z[i], zq);
      e_j[i] = fmaf(-s[i], t, wj) * dj;
      const float q = t + z[i];
      if constexpr (kOwnCodes) {
        if (k == j % LPR) qv[i][mj] = q;   // the owner keeps the code of its column
      } else {
        cw[i][(j % C) / 4] |= (k == j / C) ? (static_cast<uint32_t>(q) << (8 * (j & 3))) : 0u;
        // packed here: left to itself the compiler sinks the packing of two rows' codes and
        // keeps the codes live across columns (256 registers and spills instead of 168)
        if constexpr (RPL == 2) asm volatile("" : "+v"(cw[i][(j % C) / 4]));
      }
    }
#pragma unroll
    for (int m = mj; m < C; ++m) {
      const float4 u4 = cur[m / 4];
      const float u = (m & 3) == 0 ? u4.x : (m & 3) == 1 ? u4.y : (m & 3) == 2 ? u4.z : u4.w;
#pragma unroll
      for (int i = 0; i < RPL; ++i) w[i][m] = fmaf(-e_j[i], u, w[i][m]);
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (k == j % LPR) w[i][mj] = e_j[i];   // the owner keeps err_j in place of w_j
  });
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    if (!live[i]) continue;
    uint8_t* crow = codes_p + (static_cast<int64_t>(e) * d_out + rw[i]) * d_in + j0;
    if constexpr (kOwnCodes) {
#pragma unroll
      for (int m = 0; m < C; ++m) crow[LPR * m + k] = static_cast<uint8_t>(qv[i][m]);
    } else {
      uint32_t* cdst = reinterpret_cast<uint32_t*>(crow + C * k);
#pragma unroll
      for (int q = 0; q < CW; q += 4)
        *reinterpret_cast<uint4*>(cdst + q) = make_uint4(cw[i][q], cw[i][q + 1], cw[i][q + 2], cw[i][q + 3]);
    }
    float* edst = err + (static_cast<int64_t>(e) * d_out + rw[i]) * d_in + j0;
#pragma unroll
    for (int m = 0; m < C; ++m) edst[LPR * m + k] = w[i][m];
  }
}

// Launch geometry of the sweep: NT threads per workgroup, LPR lanes per row, the grid.
struct SweepShape {
  int nt, lpr, rpl;   // rpl: rows per lane
  dim3 grid;
};

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

template <int G, int NT, int LPR, bool kStatic, int RPL = 1>
gptq_status launch_sweep(dim3 grid, hipStream_t stream, const SweepArgs& a, int blk) {
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (a.timed) timing_pair(GPTQ_TIME_SWEEP, &ev0, &ev1);
  if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
  GPTQ_LAUNCH((block_sweep_kernel<G, NT, LPR, kStatic, RPL>), grid, dim3(NT), 0, stream, a.Wp, a.U, a.bsu, a.d_out, a.d_in,
              blk, a.maxq, a.sym, a.perm, a.gsz, a.scales, a.zeros, a.codes_p, a.err);
  if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
  return GPTQ_OK;
}

template <int G>
gptq_status launch_sweep_nt(const SweepShape& sh, hipStream_t stream, const SweepArgs& a, int blk) {
  if constexpr (G == 0 || G == 64 || G == 128) {
#define GPTQ_SWEEP(NT, LPR, RPL) \
  if (sh.nt == NT && sh.lpr == LPR && sh.rpl == RPL) return launch_sweep<G, NT, LPR, false, RPL>(sh.grid, stream, a, blk);
    GPTQ_SWEEP(512, 16, 1)   // 1024 threads at 16 lanes: never chosen (4 lanes take over first)
    if constexpr (G != 64) {
      GPTQ_SWEEP(1024, 4, 1)
      GPTQ_SWEEP(704, 4, 1)
      GPTQ_SWEEP(704, 4, 2)
      GPTQ_SWEEP(512, 4, 2)
      GPTQ_SWEEP(256, 4, 2)
    }
    GPTQ_SWEEP(512, 4, 1)
    GPTQ_SWEEP(256, 4, 1)
#undef GPTQ_SWEEP
  }
  if (sh.nt != 256 || sh.lpr != 16 || sh.rpl != 1) return GPTQ_ERR_UNSUPPORTED;
  return launch_sweep<G, 256, 16, false>(sh.grid, stream, a, blk);
}

// one 128-column block with static groups (256 threads, 16 lanes per row)
gptq_status launch_sweep_static(const SweepShape& sh, hipStream_t stream, const SweepArgs& a, int blk);

// instantiated in the sweep sources
extern template gptq_status launch_sweep_nt<0>(const SweepShape&, hipStream_t, const SweepArgs&, int);
extern template gptq_status launch_sweep_nt<16>(const SweepShape&, hipStream_t, const SweepArgs&, int);
extern template gptq_status launch_sweep_nt<32>(const SweepShape&, hipStream_t, const SweepArgs&, int);
extern template gptq_status launch_sweep_nt<64>(const SweepShape&, hipStream_t, const SweepArgs&, int);
extern template gptq_status launch_sweep_nt<128>(const SweepShape&, hipStream_t, const SweepArgs&, int);

}  // namespace gptq
