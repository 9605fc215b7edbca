// W4A16 serving product on gfx950: Y = X What^T read straight from the packed checkpoint.
//
// "GPTQ Architecture, in depth", "Packing, tooling and serving": serving kernels keep the
// 4-bit weights packed and dequantize them in registers right before the matrix product
// with 16-bit activations; decode is bound by reading the weights.  "Same Ruler, Smarter
// Placement: GPTQ", 1.9: with act-order the weight columns are permuted, and the
// activations are permuted the same way at inference time.  Layout of the checkpoint:
// "04 — GPTQ: ...", section 8 (qweight [d_in/8, d_out], nibble k of word i is input
// 8 i + k; qzeros [groups, d_out/8]; fp16 scales [groups, d_out]; g_idx [d_in]).
//
// Serving order.  A group's scale and zero can be applied once per group only if the
// group's inputs are contiguous along K.  gptq_w4a16_repack sorts the inputs by group
// (stable: ascending original index inside a group) and rewrites qweight in that order;
// the product then gathers the activations by the same order when it stages them in LDS.
// With static groups or without act-order g_idx is already sorted and nothing moves.
//
// The product (decode batches: up to 16 activation rows per pass, more in further passes):
//   y[m, o] = sum over groups g of  s[g, o] * (A_g[m, o] - z[g, o] * S_g[m]),
//   A_g[m, o] = sum_{k in g} x[m, k] q[o, k],   S_g[m] = sum_{k in g} x[m, k].
// The codes q (integers 0..15) are exact in bf16 / fp16, so A_g and S_g come out of the
// 16-bit matrix cores with exact products and fp32 sums (v_mfma_f32_16x16x32_{bf16,f16};
// S_g from the same activations against a column of ones); the fold with the fp16 scale
// and the integer zero runs in fp32 per group.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int SV_WAVES = 4;                 // waves per workgroup, side by side over outputs
constexpr int SV_OUT_WAVE = 64;             // outputs per wave: lane group j holds 4 consecutive outputs
constexpr int SV_OUT = SV_WAVES * SV_OUT_WAVE;
constexpr int SV_M = 16;                    // activation rows per pass (MFMA rows)
constexpr int SV_KMAX = 512;                // largest K chunk per workgroup (its weights all in flight)
constexpr int SV_SEG = 128;                 // fold period of a per-row grid

// ---------------------------------------------------------------------------- repack

// pos[c] = g * gs + (number of inputs before c in the same group); order[pos[c]] = c.  A
// group index outside [0, n_groups) or a group with more than gs members sets *bad.  Each
// thread counts its input's rank against g_idx tiles staged in LDS.
constexpr int RK_TILE = 1024;
__global__ __launch_bounds__(256) void group_order_kernel(const int32_t* __restrict__ g_idx, int d_in, int n_groups,
                                                          int gs, int32_t* __restrict__ order, int* __restrict__ bad) {
  __shared__ int32_t tile[RK_TILE];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  const int32_t* ge = g_idx + static_cast<int64_t>(e) * d_in;
  const int gc = c < d_in ? ge[c] : -1;
  int rank = 0;
  // only inputs before c count; the workgroup's last input bounds the tiles it needs
  const int cmax = min(d_in, static_cast<int>(blockIdx.x + 1) * 256);
  for (int t0 = 0; t0 < cmax; t0 += RK_TILE) {
    __syncthreads();
    for (int i = threadIdx.x; i < RK_TILE; i += 256) tile[i] = (t0 + i < d_in) ? ge[t0 + i] : -1;
    __syncthreads();
    const int n = min(RK_TILE, c - t0);
    for (int i = 0; i < n; ++i) rank += (tile[i] == gc);
  }
  if (c >= d_in) return;
  if (gc < 0 || gc >= n_groups || rank >= gs) {
    *bad = 1;
    return;
  }
  order[static_cast<int64_t>(e) * d_in + static_cast<int64_t>(gc) * gs + rank] = c;
}

// qweight_s[i][o] = the codes of inputs order[8 i .. 8 i + 7] of output o, nibble t for
// order[8 i + t].  One thread per output word; consecutive threads take consecutive outputs.
__global__ __launch_bounds__(256) void repack_qweight_kernel(const int32_t* __restrict__ qweight,
                                                             const int32_t* __restrict__ order, int d_out, int d_in,
                                                             int32_t* __restrict__ qweight_s) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;
  const int e = blockIdx.z;
  if (o >= d_out) return;
  const int64_t qs = static_cast<int64_t>(d_in / 8) * d_out;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(qweight) + e * qs;
  const int32_t* oe = order + static_cast<int64_t>(e) * d_in;
  uint32_t word = 0u;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c = min(max(oe[8 * i + t], 0), d_in - 1);
    const uint32_t q = (src[static_cast<int64_t>(c / 8) * d_out + o] >> (4 * (c % 8))) & 15u;
    word |= q << (4 * t);
  }
  reinterpret_cast<uint32_t*>(qweight_s)[e * qs + static_cast<int64_t>(i) * d_out + o] = word;
}

// ---------------------------------------------------------------------------- product

// Eight codes of one qweight word (nibble t = input t of the word) as eight 16-bit values
// in input order, the MFMA operand of one lane.
template <bool kBF16>
__device__ __forceinline__ s16x8 codes16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  uint32_t p[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 v = {static_cast<float>((lo >> (8 * b)) & 0xFFu), static_cast<float>((hi >> (8 * b)) & 0xFFu)};
    if constexpr (kBF16) p[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else p[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  return __builtin_bit_cast(s16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

template <bool kBF16>
__device__ __forceinline__ f32x4 mma16(s16x8 a, s16x8 b, f32x4 c) {
  if constexpr (kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
}

struct ServeArgs {
  int m, d_out, d_in;
  int gs;               // inputs per group (d_in for one grid per row)
  int kchunk;           // inputs per workgroup (a multiple of 32 and of min(gs, SV_SEG))
  const uint16_t* X;    // [m, d_in] 16-bit activations, row stride ldx
  int64_t ldx;
  const int32_t* order; // serving position -> input, or null (identity)
  const int32_t* qweight;   // [d_in / 8, d_out], serving order
  const int32_t* qzeros;    // [groups, d_out / 8]
  const uint16_t* scales;   // [groups, d_out] fp16 bits
  float* out;           // Y [m, d_out] (ldy) when one K chunk, else partials [chunks][m][d_out]
  int64_t ldy;
};

// One workgroup: 256 consecutive outputs (64 per wave), one K chunk of at most SV_KMAX
// inputs, 16 activation rows (blockIdx.z selects the pass).  Every lane issues the loads
// of all its qweight vectors of the chunk (one 16-byte vector per 32-input step: 4
// consecutive outputs of one 8-input row), so a wave keeps up to 16 KB of weights in
// flight, and meanwhile all of the activations it gathers into LDS in serving order (rows
// past m are zero).  Each step turns the 4 words of its vector into the B operands of 4
// MFMAs against the same activations, and a fifth MFMA against ones adds the activation
// sums.  Lane l owns outputs o0 + 4 (l % 16) + t, t = 0..3; after every SEG inputs (a
// group, or SEG inputs of a wider group) its sums are folded with the scale and zero.
template <bool kBF16, int SEG>
__global__ __launch_bounds__(256) void w4a16_kernel(ServeArgs a) {
  constexpr int LDX = SV_KMAX + 8;   // LDS row pitch (16-bit elements): rows start 16 bytes apart mod 128
  constexpr int NS = SEG / 32;       // 32-input steps per segment
  constexpr int NSEG = SV_KMAX / SEG;
  __shared__ __attribute__((aligned(16))) uint16_t xs[SV_M * LDX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.y * a.kchunk;
  const int kn = min(a.kchunk, a.d_in - k0);   // a multiple of SEG
  const int m0 = blockIdx.z * SV_M;

  const int o0 = blockIdx.x * SV_OUT + wave * SV_OUT_WAVE;
  const int j = lane & 15, q = lane >> 4;
  const int ob = o0 + 4 * j;                  // this lane's first output (4 consecutive)
  const bool live = ob < a.d_out;             // d_out is a multiple of 8, so all 4 are live
  const int obc = live ? ob : 0;
  const uint4* qw = reinterpret_cast<const uint4*>(a.qweight + obc);
  const int64_t row4 = a.d_out / 4;           // uint4 per qweight row

  // Loads in three waves, ordered for the wave's in-order memory counter: the serving-order
  // indices of the thread's two chunk inputs k = tid, tid + 256 first, then the weights and
  // grids, then the activations at those indices, which wait only for the indices while
  // the weights are in flight (loaded after the weights, the gather waited for all of them,
  // and one pass of 16 rows went through it in serial batches)
  static_assert(SV_KMAX <= 2 * 256, "two chunk inputs per thread");
  int kc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = tid + 256 * h;
    kc[h] = k >= kn ? -1 : a.order ? min(max(a.order[k0 + k], 0), a.d_in - 1) : k0 + k;
  }
  // step i covers inputs k0 + 32 i + 8 q .. + 7: qweight row k0 / 8 + 4 i + q
  uint4 w[NSEG * NS];
#pragma unroll
  for (int i = 0; i < NSEG * NS; ++i)
    if (32 * i < kn) w[i] = qw[static_cast<int64_t>(k0 / 8 + 4 * i + q) * row4];
  // the scales (4 fp16) and zeros (one qzeros word) of every segment's group, also up front
  uint2 sv[NSEG];
  uint32_t zw[NSEG];
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    if (sg * SEG < kn) {
      const int g = (k0 + sg * SEG) / a.gs;
      sv[sg] = *reinterpret_cast<const uint2*>(a.scales + static_cast<int64_t>(g) * a.d_out + obc);
      zw[sg] = static_cast<uint32_t>(a.qzeros[static_cast<int64_t>(g) * (a.d_out / 8) + obc / 8]);
    }
  }
  // the activations: element (r, k) = X[m0 + r][order[k0 + k]], zero for rows past m
  const int mrows = min(SV_M, a.m - m0);
  uint16_t xv[SV_M][2];
#pragma unroll
  for (int r = 0; r < SV_M; ++r)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      xv[r][h] = (r < mrows && kc[h] >= 0) ? a.X[static_cast<int64_t>(m0 + r) * a.ldx + kc[h]] : uint16_t{0};
#pragma unroll
  for (int r = 0; r < SV_M; ++r)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (kc[h] >= 0) xs[r * LDX + tid + 256 * h] = xv[r][h];
  __syncthreads();

  const s16x8 ones = kBF16 ? s16x8{0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80}
                           : s16x8{0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00};
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 y[4] = {zero4, zero4, zero4, zero4};
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    const int s0 = sg * SEG;
    if (s0 < kn) {
      f32x4 acc[4] = {zero4, zero4, zero4, zero4};
      f32x4 sacc = zero4;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const uint4 wv = w[sg * NS + t];
        const s16x8 av = *reinterpret_cast<const s16x8*>(xs + j * LDX + s0 + 32 * t + 8 * q);
        acc[0] = mma16<kBF16>(av, codes16<kBF16>(wv.x), acc[0]);
        acc[1] = mma16<kBF16>(av, codes16<kBF16>(wv.y), acc[1]);
        acc[2] = mma16<kBF16>(av, codes16<kBF16>(wv.z), acc[2]);
        acc[3] = mma16<kBF16>(av, codes16<kBF16>(wv.w), acc[3]);
        sacc = mma16<kBF16>(av, ones, sacc);
      }
      // fold with the segment's group: the lane's 4 outputs share one qzeros word
      const uint32_t sh[2] = {sv[sg].x, sv[sg].y};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sh[t / 2] >> (16 * (t & 1)))));
        const float z = static_cast<float>((zw[sg] >> (4 * ((obc % 8) + t))) & 15u);
#pragma unroll
        for (int r = 0; r < 4; ++r) y[t][r] = fmaf(s, fmaf(-z, sacc[r], acc[t][r]), y[t][r]);
      }
    }
  }
  if (!live) return;
  // lane holds rows 4 q + r of the pass, outputs ob .. ob + 3
  const bool one_chunk = gridDim.y == 1;
  float* base = one_chunk ? a.out : a.out + static_cast<int64_t>(blockIdx.y) * a.m * a.d_out;
  const int64_t ld = one_chunk ? a.ldy : a.d_out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mm = m0 + 4 * q + r;
    if (mm < a.m) *reinterpret_cast<float4*>(base + mm * ld + ob) = make_float4(y[0][r], y[1][r], y[2][r], y[3][r]);
  }
}

__global__ void clear_flag_kernel(int* __restrict__ flag) { *flag = 0; }

// Y[m][o] = sum over chunks of the partials, in chunk order.  The loads of up to 32 chunks
// are issued together before they are added (one load after another would put every
// load's latency on the chain; 8 at a time left a decode call's 28 chunks four latencies).
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float* __restrict__ part, int chunks, int m,
                                                           int d_out, float* __restrict__ Y, int64_t ldy) {
  constexpr int B = 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(m) * d_out;
  if (i >= n) return;
  float s = 0.0f;
  for (int c0 = 0; c0 < chunks; c0 += B) {
    float v[B];
#pragma unroll
    for (int c = 0; c < B; ++c) v[c] = c0 + c < chunks ? part[static_cast<int64_t>(c0 + c) * n + i] : 0.0f;
#pragma unroll
    for (int c = 0; c < B; ++c) s += v[c];
  }
  const int64_t r = i / d_out, o = i - r * d_out;
  Y[r * ldy + o] = s;
}

// K chunk per workgroup: whole fold segments, at most SV_KMAX inputs, about 2 workgroups
// per CU over the output tiles and passes.
int serve_chunk(int m, int d_out, int d_in, int gs) {
  const int seg = std::min(gs, SV_SEG);
  const int64_t tiles = static_cast<int64_t>((d_out + SV_OUT - 1) / SV_OUT) * ((m + SV_M - 1) / SV_M);
  const int64_t want = std::max<int64_t>(1, (512 + tiles - 1) / tiles);      // chunks wanted
  int chunk = static_cast<int>((d_in + want - 1) / want);
  chunk = (chunk + seg - 1) / seg * seg;
  chunk = std::min(std::max(chunk, seg), std::max(seg, SV_KMAX / seg * seg));
  return std::min(chunk, d_in);
}

}  // namespace

size_t serve_workspace(int m, int d_out, int d_in, int n_groups) {
  if (m < 1 || d_out < 1 || d_in < 1 || n_groups < 1) return 0;
  const int gs = d_in / n_groups;
  const int chunk = serve_chunk(m, d_out, d_in, gs);
  const int chunks = (d_in + chunk - 1) / chunk;
  return chunks > 1 ? static_cast<size_t>(chunks) * m * d_out * sizeof(float) + 256 : 256;
}

gptq_status repack_enqueue(int batch, int d_out, int d_in, int n_groups, const int32_t* qweight,
                           const int32_t* g_idx, int32_t* qweight_s, int32_t* order, int* flag,
                           hipStream_t stream) {
  const int gs = d_in / n_groups;
  GPTQ_LAUNCH(clear_flag_kernel, dim3(1), dim3(1), 0, stream, flag);
  GPTQ_LAUNCH(group_order_kernel, dim3((d_in + 255) / 256, batch), dim3(256), 0, stream, g_idx, d_in, n_groups, gs,
              order, flag);
  GPTQ_LAUNCH(repack_qweight_kernel, dim3((d_out + 255) / 256, d_in / 8, batch), dim3(256), 0, stream, qweight, order,
              d_out, d_in, qweight_s);
  return GPTQ_OK;
}

gptq_status serve_enqueue(int m, int d_out, int d_in, int n_groups, gptq_dtype x_dtype, const void* X, int64_t ldx,
                          const int32_t* order, const int32_t* qweight, const int32_t* qzeros,
                          const uint16_t* scales, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  const int gs = d_in / n_groups;
  const int chunk = serve_chunk(m, d_out, d_in, gs);
  const int chunks = (d_in + chunk - 1) / chunk;
  if (ws_bytes < serve_workspace(m, d_out, d_in, n_groups) || (chunks > 1 && ws == nullptr))
    return GPTQ_ERR_WORKSPACE;
  ServeArgs a{};
  a.m = m; a.d_out = d_out; a.d_in = d_in; a.gs = gs; a.kchunk = chunk;
  a.X = static_cast<const uint16_t*>(X); a.ldx = ldx; a.order = order;
  a.qweight = qweight; a.qzeros = qzeros; a.scales = scales;
  a.out = chunks > 1 ? static_cast<float*>(ws) : Y;
  a.ldy = ldy;
  const dim3 grid((d_out + SV_OUT - 1) / SV_OUT, chunks, (m + SV_M - 1) / SV_M);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  timing_pair(GPTQ_TIME_W4A16, &ev0, &ev1);
  if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
  const int seg = std::min(gs, SV_SEG);
#define GPTQ_SERVE(SEG)                                                                             \
  if (seg == SEG) {                                                                                 \
    if (x_dtype == GPTQ_BF16) GPTQ_LAUNCH((w4a16_kernel<true, SEG>), grid, dim3(256), 0, stream, a); \
    else GPTQ_LAUNCH((w4a16_kernel<false, SEG>), grid, dim3(256), 0, stream, a);                      \
  }
  GPTQ_SERVE(32)
  GPTQ_SERVE(64)
  GPTQ_SERVE(128)
#undef GPTQ_SERVE
  if (chunks > 1) {
    const int64_t n = static_cast<int64_t>(m) * d_out;
    GPTQ_LAUNCH(w4a16_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                static_cast<const float*>(ws), chunks, m, d_out, Y, ldy);
  }
  if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
  return GPTQ_OK;
}

}  // namespace gptq
