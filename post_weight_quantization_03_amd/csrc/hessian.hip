// Hessian accumulation H += 2 X^T X on gfx950.
//
// "Same Ruler, Smarter Placement: GPTQ", 1.4: each output row's loss is a quadratic form
// in X X^T, so one d_in x d_in Hessian serves every row; "GPTQ Architecture, in depth",
// "The algorithm in code": it is accumulated per calibration batch.
//
// bf16/fp16 inputs: a symmetric rank-k update on the MFMA units.  Each workgroup owns a
// 256 x 256 tile on or below the diagonal and a slice of the tokens; products of two
// 16-bit values are exact in fp32 and are summed in fp32 by v_mfma_f32_32x32x16_{bf16,f16}.
// Token-major X is staged through LDS transposed (channel-major, 8 tokens per MFMA
// operand), double-buffered so global loads of the next stage overlap the MFMAs.
// Off-diagonal tiles are mirrored into the upper triangle, so H is exactly symmetric.
// When the tiles alone cannot fill the 256 CUs the tokens are split and the fp32
// partial tiles are summed in a fixed order by a second kernel (deterministic, no
// atomics).  fp32 inputs use a plain FMA tile kernel (small layers only).
//
// The fp64 diagonal key 2 * sum_t x^2 (exact products, fp64 sums) is accumulated by its
// own kernel pair: it decides the ActOrder permutation, where fp32 sums are not precise
// enough to order nearly equal channels reproducibly.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int ST = 256;        // output tile edge
constexpr int SBK = 32;        // tokens per LDS stage
constexpr int LDK = SBK + 4;   // LDS row (one channel) length in 16-bit elements
constexpr int SYRK_THREADS = 256;
constexpr int kMinTokensPerSplit = 2048;

__device__ __forceinline__ void lower_tile_coords(int t, int& I, int& J) {
  // t enumerates (0,0), (1,0), (1,1), (2,0), ... row by row.
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

template <bool kF16>
__device__ __forceinline__ f32x16 mfma16(const uint2 a[2], const uint2 b[2], f32x16 c) {
  uint4 av = make_uint4(a[0].x, a[0].y, a[1].x, a[1].y);
  uint4 bv = make_uint4(b[0].x, b[0].y, b[1].x, b[1].y);
  if constexpr (kF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                  __builtin_bit_cast(f16x8, bv), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
  }
}

// One 256x256 lower tile (blockIdx.x), token slice (blockIdx.y), problem (blockIdx.z).
// partial == nullptr: H += 2 * tile (and its mirror).  Otherwise the raw tile is stored
// to partial[e][split][tile][256][256] for syrk_reduce_kernel.
template <bool kF16>
__global__ __launch_bounds__(SYRK_THREADS) void syrk_mfma_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t bsx, int64_t n_tokens, int d_in,
    int64_t tokens_per_split, float* __restrict__ H, int64_t bsh, float* __restrict__ partial,
    int ntiles) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][ST * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][ST * LDK];

  const int e = blockIdx.z;
  const int split = blockIdx.y;
  int I, J;
  lower_tile_coords(blockIdx.x, I, J);
  const bool diag = (I == J);
  const int I0 = I * ST, J0 = J * ST;
  const int64_t t_begin = static_cast<int64_t>(split) * tokens_per_split;
  const int64_t t_end = min(n_tokens, t_begin + tokens_per_split);
  const uint16_t* Xe = X + static_cast<int64_t>(e) * bsx;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader unit of a thread: tokens [4*lq, 4*lq+4) of the stage, channels [8*loct, 8*loct+8)
  const int lq = tid & 7, loct = tid >> 3;

  uint4 ra[4], rb[4];
  auto gload = [&](int64_t t0, int C0, uint4* r) {
    const int c = C0 + 8 * loct;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = t0 + 4 * lq + k;
      if (t < t_end && c < d_in) {
        r[k] = *reinterpret_cast<const uint4*>(Xe + t * ldx + c);
      } else {
        r[k] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  // Transpose 4 tokens x 8 channels in registers: channel i gets its 4 tokens as 8 bytes.
  auto swrite = [&](uint16_t* s, const uint4* r) {
    const uint32_t w[4][4] = {{r[0].x, r[0].y, r[0].z, r[0].w},
                              {r[1].x, r[1].y, r[1].z, r[1].w},
                              {r[2].x, r[2].y, r[2].z, r[2].w},
                              {r[3].x, r[3].y, r[3].z, r[3].w}};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(w[1][i >> 1], w[0][i >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(w[3][i >> 1], w[2][i >> 1], sel);
      *reinterpret_cast<uint2*>(s + (8 * loct + i) * LDK + 4 * lq) = make_uint2(lo, hi);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int am = lane & 31, ak = (lane >> 5) * 8;
  const int nstages = static_cast<int>((t_end - t_begin + SBK - 1) / SBK);

  if (nstages > 0) {
    gload(t_begin, I0, ra);
    if (!diag) gload(t_begin, J0, rb);
    swrite(sA[0], ra);
    if (!diag) swrite(sB[0], rb);
  }
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    const bool more = (s + 1 < nstages);
    if (more) {
      const int64_t tn = t_begin + static_cast<int64_t>(s + 1) * SBK;
      gload(tn, I0, ra);
      if (!diag) gload(tn, J0, rb);
    }
    const uint16_t* as = sA[buf];
    const uint16_t* bs = diag ? sA[buf] : sB[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint2 av[4][2], bv[4][2];
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        const uint16_t* p = as + (128 * wm + 32 * bm + am) * LDK + 16 * ks + ak;
        av[bm][0] = *reinterpret_cast<const uint2*>(p);
        av[bm][1] = *reinterpret_cast<const uint2*>(p + 4);
      }
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const uint16_t* p = bs + (128 * wn + 32 * bn + am) * LDK + 16 * ks + ak;
        bv[bn][0] = *reinterpret_cast<const uint2*>(p);
        bv[bn][1] = *reinterpret_cast<const uint2*>(p + 4);
      }
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = mfma16<kF16>(av[bm], bv[bn], acc[bm][bn]);
    }
    if (more) {
      swrite(sA[buf ^ 1], ra);
      if (!diag) swrite(sB[buf ^ 1], rb);
    }
    __syncthreads();
  }

  // Accumulator layout of a 32x32 MFMA block: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (partial != nullptr) {
    float* P = partial + ((static_cast<int64_t>(e) * gridDim.y + split) * ntiles + blockIdx.x) *
                             static_cast<int64_t>(ST * ST);
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 128 * wm + 32 * bm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int n = 128 * wn + 32 * bn + (lane & 31);
          P[m * ST + n] = acc[bm][bn][r];
        }
    return;
  }
  float* He = H + static_cast<int64_t>(e) * bsh;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int m0 = 128 * wm + 32 * bm + 8 * rq + 4 * (lane >> 5);
        const int n = 128 * wn + 32 * bn + (lane & 31);
        const int col = J0 + n;
        if (col >= d_in) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + q;
          const int row = I0 + m;
          if (row >= d_in || (diag && m < n)) continue;
          const float v = 2.0f * acc[bm][bn][4 * rq + q];
          He[static_cast<int64_t>(row) * d_in + col] += v;
          if (!diag || m > n) He[static_cast<int64_t>(col) * d_in + row] += v;
        }
      }
}

// Sums the token-slice partials of each lower tile in slice order and adds twice the
// sum to H and to its mirror.  Block: 64x64 sub-block of one tile; mirror writes go
// through LDS so both stores are coalesced.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ partial,
                                                          int nsplit, int ntiles, int d_in,
                                                          float* __restrict__ H, int64_t bsh) {
  __shared__ float tr[64][65];
  const int e = blockIdx.z;
  const int tile = blockIdx.y;
  const int sub = blockIdx.x;  // 16 sub-blocks of 64x64
  const int sm = (sub >> 2) * 64, sn = (sub & 3) * 64;
  int I, J;
  lower_tile_coords(tile, I, J);
  const bool diag = (I == J);
  if (diag && sm < sn) return;  // strictly-upper sub-block of a diagonal tile
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  float* He = H + static_cast<int64_t>(e) * bsh;
  const int64_t tstride = static_cast<int64_t>(ST) * ST;
  const float* P0 = partial + (static_cast<int64_t>(e) * nsplit * ntiles + tile) * tstride;
  for (int i = ty; i < 64; i += 4) {
    const int m = sm + i, n = sn + tx;
    float s = 0.0f;
    for (int k = 0; k < nsplit; ++k) s += P0[static_cast<int64_t>(k) * ntiles * tstride + m * ST + n];
    const float v = 2.0f * s;
    tr[i][tx] = v;
    const int row = I * ST + m, col = J * ST + n;
    if (row < d_in && col < d_in && (!diag || m >= n)) He[static_cast<int64_t>(row) * d_in + col] += v;
  }
  __syncthreads();
  // mirror: H[col][row] for the same sub-block, written along rows of the transpose
  for (int i = ty; i < 64; i += 4) {
    const int n = sn + i, m = sm + tx;       // element (m, n) of the tile
    const int row = I * ST + m, col = J * ST + n;
    if (row < d_in && col < d_in && (!diag || m > n))
      He[static_cast<int64_t>(col) * d_in + row] += tr[tx][i];
  }
}

// fp32 inputs: 64x64 lower tiles, 256 threads with 4x4 outputs each, FMA in fp32.
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t bsx, int64_t n_tokens, int d_in,
                                                       float* __restrict__ H, int64_t bsh) {
  __shared__ float sa[16][64];
  __shared__ float sb[16][64];
  const int e = blockIdx.z;
  int I, J;
  lower_tile_coords(blockIdx.x, I, J);
  const int I0 = I * 64, J0 = J * 64;
  const float* Xe = X + static_cast<int64_t>(e) * bsx;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n_tokens; t0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int k = i >> 6, c = i & 63;
      const int64_t t = t0 + k;
      const bool okt = t < n_tokens;
      sa[k][c] = (okt && I0 + c < d_in) ? Xe[t * ldx + I0 + c] : 0.0f;
      sb[k][c] = (okt && J0 + c < d_in) ? Xe[t * ldx + J0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = sa[k][ty * 4 + q];
        b[q] = sb[k][tx * 4 + q];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
    }
    __syncthreads();
  }
  float* He = H + static_cast<int64_t>(e) * bsh;
  const bool diag = (I == J);
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = ty * 4 + p, n = tx * 4 + q;
      const int row = I0 + m, col = J0 + n;
      if (row >= d_in || col >= d_in || (diag && m < n)) continue;
      const float v = 2.0f * acc[p][q];
      He[static_cast<int64_t>(row) * d_in + col] += v;
      if (!diag || m > n) He[static_cast<int64_t>(col) * d_in + row] += v;
    }
}

// fp64 channel energy of one token slice: part[e][split][c] = sum_t x[t][c]^2.
template <typename T>
__global__ __launch_bounds__(256) void channel_energy_kernel(const T* __restrict__ X, int64_t ldx,
                                                             int64_t bsx, int64_t n_tokens, int d_in,
                                                             int64_t tokens_per_split,
                                                             double* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int split = blockIdx.y, e = blockIdx.z;
  if (c >= d_in) return;
  const int64_t t0 = static_cast<int64_t>(split) * tokens_per_split;
  const int64_t t1 = min(n_tokens, t0 + tokens_per_split);
  const T* Xe = X + static_cast<int64_t>(e) * bsx + c;
  double acc0 = 0.0, acc1 = 0.0;
  int64_t t = t0;
  for (; t + 1 < t1; t += 2) {
    const double a = static_cast<double>(load_as_f32(Xe + t * ldx));
    const double b = static_cast<double>(load_as_f32(Xe + (t + 1) * ldx));
    acc0 = fma(a, a, acc0);
    acc1 = fma(b, b, acc1);
  }
  if (t < t1) {
    const double a = static_cast<double>(load_as_f32(Xe + t * ldx));
    acc0 = fma(a, a, acc0);
  }
  part[(static_cast<int64_t>(e) * gridDim.y + split) * d_in + c] = acc0 + acc1;
}

__global__ __launch_bounds__(256) void channel_energy_reduce_kernel(const double* __restrict__ part,
                                                                    int nsplit, int d_in,
                                                                    double* __restrict__ diag_key,
                                                                    int64_t* __restrict__ n_seen,
                                                                    int64_t n_tokens) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c < d_in) {
    double s = 0.0;
    for (int k = 0; k < nsplit; ++k) s += part[(static_cast<int64_t>(e) * nsplit + k) * d_in + c];
    diag_key[static_cast<int64_t>(e) * d_in + c] += 2.0 * s;
  }
  if (c == 0) n_seen[e] += n_tokens;
}

struct HessianPlan {
  bool mfma;
  int ntiles;            // lower tiles per problem
  int ksplit;            // token slices of the MFMA SYRK
  int64_t kchunk;        // tokens per slice (multiple of SBK)
  int esplit;            // token slices of the energy kernel
  int64_t echunk;
};

HessianPlan make_plan(int batch, int d_in, int64_t n_tokens, bool mfma) {
  HessianPlan pl{};
  pl.mfma = mfma;
  const int tile = mfma ? ST : 64;
  const int nt = (d_in + tile - 1) / tile;
  pl.ntiles = nt * (nt + 1) / 2;
  pl.ksplit = 1;
  pl.kchunk = n_tokens;
  if (mfma) {
    const int64_t want = (1024 + static_cast<int64_t>(pl.ntiles) * batch - 1) /
                         (static_cast<int64_t>(pl.ntiles) * batch);
    const int64_t cap = std::max<int64_t>(1, n_tokens / kMinTokensPerSplit);
    pl.ksplit = static_cast<int>(std::min<int64_t>(std::min(want, cap), 64));
    pl.kchunk = (n_tokens + pl.ksplit - 1) / pl.ksplit;
    pl.kchunk = (pl.kchunk + SBK - 1) / SBK * SBK;
    if (pl.kchunk == 0) pl.kchunk = SBK;
    pl.ksplit = static_cast<int>((n_tokens + pl.kchunk - 1) / pl.kchunk);
    if (pl.ksplit < 1) pl.ksplit = 1;
  }
  const int cblocks = (d_in + 255) / 256;
  const int64_t ewant = (2048 + static_cast<int64_t>(cblocks) * batch - 1) /
                        (static_cast<int64_t>(cblocks) * batch);
  const int64_t ecap = std::max<int64_t>(1, n_tokens / 256);
  pl.esplit = static_cast<int>(std::min<int64_t>(std::min(ewant, ecap), 1024));
  pl.echunk = (n_tokens + pl.esplit - 1) / pl.esplit;
  if (pl.echunk == 0) pl.echunk = 1;
  pl.esplit = static_cast<int>(std::max<int64_t>(1, (n_tokens + pl.echunk - 1) / pl.echunk));
  return pl;
}

size_t plan_bytes(const HessianPlan& pl, int batch, int d_in, float** partial, double** epart,
                  void* ws) {
  Carver cv(ws);
  float* p = nullptr;
  if (pl.mfma && pl.ksplit > 1)
    p = cv.take<float>(static_cast<size_t>(batch) * pl.ksplit * pl.ntiles * ST * ST);
  double* q = cv.take<double>(static_cast<size_t>(batch) * pl.esplit * d_in);
  if (partial) *partial = p;
  if (epart) *epart = q;
  return cv.used + 256;
}

}  // namespace

size_t hessian_workspace(int batch, int d_in, int64_t n_tokens) {
  if (batch < 1 || d_in < 8 || n_tokens < 0) return 0;
  const HessianPlan a = make_plan(batch, d_in, std::max<int64_t>(n_tokens, 1), true);
  const HessianPlan b = make_plan(batch, d_in, std::max<int64_t>(n_tokens, 1), false);
  return std::max(plan_bytes(a, batch, d_in, nullptr, nullptr, nullptr),
             plan_bytes(b, batch, d_in, nullptr, nullptr, nullptr));
}

gptq_status hessian_enqueue(int batch, int d_in, int64_t n_tokens, gptq_dtype x_dtype, const void* X,
                            int64_t ldx, int64_t bsx, float* H, int64_t bsh, double* diag_key,
                            int64_t* n_seen, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_tokens == 0) return GPTQ_OK;
  const bool mfma = (x_dtype == GPTQ_BF16 || x_dtype == GPTQ_F16);
  const HessianPlan pl = make_plan(batch, d_in, n_tokens, mfma);
  float* partial = nullptr;
  double* epart = nullptr;
  const size_t need = plan_bytes(pl, batch, d_in, &partial, &epart, ws);
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  // the carver aligned from the workspace base; recompute pointers from the real base
  plan_bytes(pl, batch, d_in, &partial, &epart, ws);

  const dim3 blk(256);
  if (mfma) {
    const dim3 grid(pl.ntiles, pl.ksplit, batch);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    float* part = pl.ksplit > 1 ? partial : nullptr;
    if (x_dtype == GPTQ_F16) {
      GPTQ_LAUNCH(syrk_mfma_kernel<true>, grid, blk, 0, stream, Xh, ldx, bsx, n_tokens, d_in,
                  pl.kchunk, H, bsh, part, pl.ntiles);
    } else {
      GPTQ_LAUNCH(syrk_mfma_kernel<false>, grid, blk, 0, stream, Xh, ldx, bsx, n_tokens, d_in,
                  pl.kchunk, H, bsh, part, pl.ntiles);
    }
    if (pl.ksplit > 1) {
      GPTQ_LAUNCH(syrk_reduce_kernel, dim3(16, pl.ntiles, batch), blk, 0, stream, partial,
                  pl.ksplit, pl.ntiles, d_in, H, bsh);
    }
  } else {
    GPTQ_LAUNCH(syrk_f32_kernel, dim3(pl.ntiles, 1, batch), blk, 0, stream,
                static_cast<const float*>(X), ldx, bsx, n_tokens, d_in, H, bsh);
  }
  const dim3 eg((d_in + 255) / 256, pl.esplit, batch);
  switch (x_dtype) {
    case GPTQ_F32:
      GPTQ_LAUNCH(channel_energy_kernel<float>, eg, blk, 0, stream, static_cast<const float*>(X), ldx,
                  bsx, n_tokens, d_in, pl.echunk, epart);
      break;
    case GPTQ_BF16:
      GPTQ_LAUNCH(channel_energy_kernel<BF16>, eg, blk, 0, stream, static_cast<const BF16*>(X), ldx,
                  bsx, n_tokens, d_in, pl.echunk, epart);
      break;
    case GPTQ_F16:
      GPTQ_LAUNCH(channel_energy_kernel<F16>, eg, blk, 0, stream, static_cast<const F16*>(X), ldx,
                  bsx, n_tokens, d_in, pl.echunk, epart);
      break;
  }
  GPTQ_LAUNCH(channel_energy_reduce_kernel, dim3((d_in + 255) / 256, batch), blk, 0, stream, epart,
              pl.esplit, d_in, diag_key, n_seen, n_tokens);
  return GPTQ_OK;
}

}  // namespace gptq
