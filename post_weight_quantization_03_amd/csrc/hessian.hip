// Hessian accumulation H += 2 X^T X on gfx950.
//
// "Same Ruler, Smarter Placement: GPTQ", 1.4: each output row's loss is a quadratic form
// in X X^T, so one d_in x d_in Hessian serves every row; "GPTQ Architecture, in depth",
// "The algorithm in code": it is accumulated per calibration batch.
//
// bf16/fp16 inputs: a symmetric rank-k update on the MFMA units.  Each workgroup (8 waves)
// owns a 256 x 256 tile on or below the diagonal and a slice of the tokens; products of two
// 16-bit values are exact in fp32 and are summed in fp32 by v_mfma_f32_32x32x16_{bf16,f16}.
// Token-major X is copied to LDS as it lies in memory by direct global->LDS loads (no
// register staging; XOR-swizzled 16-byte chunks), one 64-token stage in flight
// under the MFMAs; the MFMA operands (8 consecutive tokens of one channel per
// lane) come out of LDS through the transposing ds_read_b64_tr_b16.
// The tokens are split into slices (about 2048 workgroups in all); every workgroup writes
// its fp32 tile to a partial buffer, and a second kernel sums the slices in a fixed order
// (deterministic, no atomics) and adds twice the sum to H and its mirror, so H is exactly
// symmetric.  fp32 inputs use a plain FMA tile kernel (small layers only).
//
// The fp64 diagonal key 2 * sum_t x^2 (exact products, fp64 sums) decides the ActOrder
// permutation, where fp32 sums are not precise enough to order nearly equal channels
// reproducibly.  For 16-bit inputs the SYRK's diagonal tiles add it up from the tokens
// they already hold in LDS (X is read once); for fp32 inputs a separate memory-bound kernel
// does.  Per-slice fp64 partials are summed in a fixed order.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int ST = 256;        // output tile edge
constexpr int SBK = 64;        // tokens per LDS stage
// Two stage buffers per operand: while stage s is multiplied, the copy of stage s + 1 is in
// flight.  Each wave drains its own LDS reads of stage s (lgkmcnt(0)) before the stage's one
// barrier, after which the copy of stage s + 2 goes into stage s's buffer.  64-token stages
// (four 16-token MFMA steps per barrier) ran 7-10% faster than 32-token stages with three
// buffers and the same bytes in flight; with 32-token stages, two stages in flight beat
// three and four (fewer outstanding copies keep more of each channel panel's lines in L2
// for the other tiles of the round that read it).
constexpr int DEPTH = 2;                  // stages loaded before the first barrier
constexpr int NBUF = 2;                   // LDS stage buffers per operand
// 8 waves per 256 x 256 tile: 2 (rows) x 4 (columns) of 128 x 64, two waves per SIMD.
// (4 waves of 128 x 128, one per SIMD with the accumulators in AGPRs, read a third fewer
// operand bytes from LDS but ran slower: one wave per SIMD hides less latency.)
constexpr int SYRK_WAVES = 8;
constexpr int kMinTokensPerSplit = 2048;
// At most this many tokens per slice: the workgroups of a round stream their panels
// together, and the longer a slice the further apart they drift, so that panels fetched
// for one are gone from the caches before the others read them (d_in 14336 over 262144
// tokens: SYRK 46.1 ms with 4 slices of 65536 tokens, 45.6 with 8, 44.3 with 16 of 16384;
// d_in 4096 over 131072 tokens: 15 slices of 8738 tokens already fill its rounds).
constexpr int64_t kMaxTokensPerSplit = 16384;

// Lower tiles (J <= I) of the tile rectangle rows [r0, r1) x columns [c0, c1).
__device__ __forceinline__ int lower_count(int r0, int r1, int c0, int c1) {
  int n = 0;
  for (int i = r0; i < r1; ++i) n += max(0, min(c1, i + 1) - c0);
  return n;
}

// (I, J) of lower tile t of an nt x nt tile grid, in an order whose aligned runs of 256
// tiles (one round of one workgroup per CU on all 256 CUs) stay inside one block of 16 x
// 16 tiles, and whose runs of 32 (the share of one XCD in a round) stay inside one 4 x 8
// sub-block of it: super-blocks of 16 x 16 tiles row by row, inside a super-block its 8
// sub-blocks (4 tile rows x 8 tile columns) row by row, inside a sub-block tiles row by
// row.  A round then reads 32 channel panels (16 + 16) for up to 256 tiles, all from one
// token slice, so concurrent workgroups of all XCDs share their panels in the last-level
// cache; an XCD's 32 tiles share 4 + 8 panels in its L2.  Scalar loops of at most a few
// dozen iterations.
__device__ __forceinline__ void round_tile_coords(int t, int nt, int& I, int& J) {
  const int nsb = (nt + 15) / 16;
  int A = 0, Bc = 0;
  for (A = 0; A < nsb; ++A) {
    bool found = false;
    for (Bc = 0; Bc <= A; ++Bc) {
      const int n = lower_count(16 * A, min(16 * A + 16, nt), 16 * Bc, min(16 * Bc + 16, nt));
      if (t < n) {
        found = true;
        break;
      }
      t -= n;
    }
    if (found) break;
  }
  const int R0 = 16 * A, R1 = min(R0 + 16, nt), C0 = 16 * Bc, C1 = min(C0 + 16, nt);
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 2; ++b) {
      const int r0 = R0 + 4 * a, r1 = min(r0 + 4, R1), c0 = C0 + 8 * b, c1 = min(c0 + 8, C1);
      if (r0 >= r1 || c0 >= c1) continue;
      const int n = lower_count(r0, r1, c0, c1);
      if (t >= n) {
        t -= n;
        continue;
      }
      for (int i = r0; i < r1; ++i) {
        const int w = max(0, min(c1, i + 1) - c0);
        if (t < w) {
          I = i;
          J = c0 + t;
          return;
        }
        t -= w;
      }
    }
  }
  I = 0;   // not reached for t < nt (nt + 1) / 2
  J = 0;
}

__device__ __forceinline__ void lower_tile_coords(int t, int& I, int& J) {
  // t enumerates (0,0), (1,0), (1,1), (2,0), ... row by row.
  int i = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

// Rows of problem e in its activation buffer: [start, start + count).  Without token
// offsets every problem has n_tokens rows from its own buffer (X + e * bsx).  With offsets
// (grouped calls: one buffer, problem e owns rows offsets[e] .. offsets[e + 1]) the range
// is clamped to the buffer's total_rows rows and to n_tokens, the most rows the launch
// covers per problem, so no access leaves the buffer whatever the offsets hold.
struct Rows {
  int64_t start, count;
};
__device__ __forceinline__ Rows problem_rows(const int64_t* offsets, int e, int64_t n_tokens, int64_t total_rows) {
  if (offsets == nullptr) return {0, n_tokens};
  const int64_t a = min(max(offsets[e], static_cast<int64_t>(0)), total_rows);
  const int64_t b = min(max(offsets[e + 1], a), total_rows);
  return {a, min(b - a, n_tokens)};
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Direct global->LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes
// land at LDS byte address base + 16 l; base must be wave-uniform (a scalar register).  Issued from inline
// assembly so that the compiler does not fence every later LDS read on it; the caller
// waits for completion with s_waitcnt vmcnt.  m0 is saved and restored around the copy.
__device__ __forceinline__ void lds_dma16(const void* src, unsigned base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left at their no-wait maxima); the
// counter's low four bits sit in bits 3:0 of the immediate, its high two in bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

template <bool kF16>
__device__ __forceinline__ f32x16 mfma16(s16x4 a0, s16x4 a1, s16x4 b0, s16x4 b1, f32x16 c) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const s16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  if constexpr (kF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
}

// LDS stage layout: SBK token rows of 256 channels (512 bytes), stored as 32 chunks of 16
// bytes.  A transposing operand read takes, per 16 lanes, 4 consecutive token rows x 2
// chunks, and the next 16 lanes the same rows 2 chunks further on; every token row starts
// on the same bank (512-byte rows, 256 bytes of banks).  Chunk c of row t therefore sits at
//   phys(t, c) = (c ^ 8 * bit1(c)) ^ 2 * (t & 3):
// the token term spreads the 4 rows of one 16-lane group over 8 chunks (128 bytes), and
// the bit-1 term puts the two chunk pairs of a half wave into different 128-byte halves,
// so the 32 lanes of a half wave cover all 64 banks once.
__device__ __forceinline__ int chunk_phys(int t, int c) { return (c ^ (((c >> 1) & 1) << 3)) ^ (2 * (t & 3)); }
// the logical chunk stored at physical position p of row t (inverse of chunk_phys)
__device__ __forceinline__ int chunk_logical(int t, int p) {
  const int q = p ^ (2 * (t & 3));
  return q ^ (((q >> 1) & 1) << 3);
}

// One 256x256 lower tile and token slice per workgroup of NW waves (2 x NW/2 waves).
// (tile, slice) pairs are assigned so that each XCD (workgroups are dealt to the 8 XCDs
// round-robin) works through a contiguous run of tiles of the same slice, which share
// operand blocks in its L2.
//
// Global->LDS copies run one stage ahead of the math, and within the math the operand
// reads (transposing LDS reads) of the next 16-token step are in flight while the
// MFMAs of the current one issue, so neither the copies nor the LDS reads serialise with
// the matrix cores.
//
// The raw tile goes to partial[e][slice][tile][256][256]; syrk_reduce_kernel sums the
// slices in order and adds twice the sum to H and its mirror.
template <bool kF16, int NW>
__global__ __launch_bounds__(64 * NW) void syrk_mfma_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t bsx, int64_t n_tokens, const int64_t* __restrict__ offsets,
    int64_t total_rows, int d_in, int64_t tokens_per_split, int ksplit, float* __restrict__ partial, int ntiles,
    double* __restrict__ epart) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[NBUF][SBK * ST];
  __shared__ __attribute__((aligned(16))) uint16_t sB[NBUF][SBK * ST];

  // (problem, slice, tile) of this workgroup.  Workgroups start in linear order over the
  // whole grid (x fastest), dealt to the 8 XCDs round-robin (XCD = id % 8), one per CU, so
  // the running ones form a window of about 256 consecutive ids.  Positions are problem-
  // then slice-major; inside each full run of 256 ids, the workgroup dealt to XCD x in slot
  // s takes position 32 x + s, so every XCD works on 32 consecutive positions (one sub-block
  // of round_tile_coords) of the same problem and token slice.
  const int total = ntiles * ksplit;
  const int all = total * static_cast<int>(gridDim.y);
  const int lin = static_cast<int>(blockIdx.y) * total + static_cast<int>(blockIdx.x);
  const int rnd = lin >> 8, p = lin & 255;
  const int gidx = (rnd + 1) * 256 <= all ? (rnd << 8) + 32 * (p & 7) + (p >> 3) : lin;
  const int e = gidx / total;
  const int idx = gidx - e * total;
  const int split = idx / ntiles;
  const int tile = idx - split * ntiles;
  int I, J;
  round_tile_coords(tile, (d_in + ST - 1) / ST, I, J);
  const bool diag = (I == J);
  const int I0 = I * ST, J0 = J * ST;
  const Rows pr = problem_rows(offsets, e, n_tokens, total_rows);
  const int64_t t_begin = static_cast<int64_t>(split) * tokens_per_split;
  const int64_t t_end = min(pr.count, t_begin + tokens_per_split);   // an empty slice writes a zero tile
  const uint16_t* Xe = X + static_cast<int64_t>(e) * bsx + pr.start * ldx;
  const bool full_cols = (I0 + ST <= d_in) && (J0 + ST <= d_in);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int WN = NW / 2;              // waves along the columns
  constexpr int WC = ST / WN;              // columns per wave: 64 or 128
  constexpr int BN = WC / 32;              // 32-column MFMA blocks per wave
  constexpr int RPW = SBK / NW;            // token rows each wave copies per operand and stage
  constexpr int CPO = RPW / 2;             // 2-row copies per operand per wave and stage
  const int wm = wave / WN, wn = wave % WN;

  // Stage loader.  Fast path (all 32 rows and all 256 channels valid): each wave issues CPO
  // direct global->LDS copies of 2 token rows (64 lanes x 16 bytes, lane-linear in LDS)
  // per operand; lane l fills physical chunk l%32 of its row, i.e. fetches logical chunk
  // chunk_logical(row, l%32).  The per-lane sources of stage 0 and the wave's LDS offsets are
  // computed once; stage k adds k * SBK rows.  Copy i covers rows crow + 2 i; the swizzle
  // repeats every 4 rows, so copies i and i + 2 share a source pattern 4 rows apart.
  // Tail stages go through registers with zero fill.
  const int crow = RPW * wave + (lane >> 5);
  const uint16_t* srcA0 = Xe + (t_begin + crow) * ldx + I0 + 8 * chunk_logical(crow, lane & 31);
  const uint16_t* srcA1 = Xe + (t_begin + crow + 2) * ldx + I0 + 8 * chunk_logical(crow + 2, lane & 31);
  const uint16_t* srcB0 = Xe + (t_begin + crow) * ldx + J0 + 8 * chunk_logical(crow, lane & 31);
  const uint16_t* srcB1 = Xe + (t_begin + crow + 2) * ldx + J0 + 8 * chunk_logical(crow + 2, lane & 31);
  constexpr unsigned kBufBytes = SBK * ST * 2, kRowBytes = ST * 2;
  const unsigned ldsA = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void*)(&sA[0][0]))) +
                        RPW * wave * kRowBytes;
  const unsigned ldsB = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void*)(&sB[0][0]))) +
                        RPW * wave * kRowBytes;
  auto load_stage = [&](int k) {
    const int64_t t0 = t_begin + static_cast<int64_t>(k) * SBK;
    const int buf = k % NBUF;
    const int rows = static_cast<int>(min<int64_t>(SBK, t_end - t0));
    if (rows == SBK && full_cols) {
      const int64_t off = static_cast<int64_t>(k) * SBK * ldx;
      const unsigned lb = buf * kBufBytes;
#pragma unroll
      for (int i = 0; i < CPO; i += 2) {
        const int64_t o4 = off + static_cast<int64_t>(2 * i) * ldx;   // 4 rows per pair of copies
        lds_dma16(srcA0 + o4, ldsA + lb + 2 * i * kRowBytes);
        lds_dma16(srcA1 + o4, ldsA + lb + (2 * i + 2) * kRowBytes);
      }
      if (!diag) {
#pragma unroll
        for (int i = 0; i < CPO; i += 2) {
          const int64_t o4 = off + static_cast<int64_t>(2 * i) * ldx;
          lds_dma16(srcB0 + o4, ldsB + lb + 2 * i * kRowBytes);
          lds_dma16(srcB1 + o4, ldsB + lb + (2 * i + 2) * kRowBytes);
        }
      }
    } else {
      for (int op = 0; op < (diag ? 1 : 2); ++op) {
        const int C0 = op ? J0 : I0;
        uint16_t* dst = op ? sB[buf] : sA[buf];
#pragma unroll
        for (int i = 0; i < CPO; ++i) {
          const int r = RPW * wave + 2 * i + (lane >> 5);
          const int p = lane & 31;
          const int c = chunk_logical(r, p);
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (r < rows && C0 + 8 * c < d_in) v = *reinterpret_cast<const uint4*>(Xe + (t0 + r) * ldx + C0 + 8 * c);
          *reinterpret_cast<uint4*>(dst + r * ST + 8 * p) = v;
        }
      }
    }
  };

  f32x16 acc[4][BN];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < BN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // transposing-read coordinates of this lane within a 32x16 operand block
  const int g16 = lane >> 4, j16 = lane & 15;
  const int rq = j16 >> 2, ra = j16 & 3;
  const int op_ch = 16 * (g16 & 1) + 4 * ra;         // + 32*block
  const int op_tok = 8 * (g16 >> 1) + rq;            // + 16*ks + 4*half
  const int nstages = static_cast<int>((t_end - t_begin + SBK - 1) / SBK);

  auto operand = [&](const uint16_t* stage, int ch0, int tok0) -> s16x4 {
    const int ch = ch0 + op_ch;
    const int t = tok0 + op_tok;
    const int byte = t * (2 * ST) + 16 * chunk_phys(t, ch >> 3) + 2 * (ch & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(reinterpret_cast<const char*>(stage) + byte));
  };

  // fp64 channel energies, on diagonal tiles only (each token slice of each channel passes
  // through exactly one of them): thread (cg = tid % 64, tg = tid / 64) adds the squares of
  // channels I0 + 4 cg .. + 3 over tokens 8 tg .. 8 tg + 7 of every stage, in token order
  // (squares of 16-bit values are exact in fp64).
  static_assert(NW == 8 && SBK == 64, "energy thread map: 64 channel quads x 8 token octets");
  const int e_cg = tid & 63, e_tg = tid >> 6;
  double en[4] = {0.0, 0.0, 0.0, 0.0};
  auto energies = [&](int stage) {
    const char* base = reinterpret_cast<const char*>(sA[stage % NBUF]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 8 * e_tg + i;
      const uint2 raw =
          *reinterpret_cast<const uint2*>(base + t * (2 * ST) + 16 * chunk_phys(t, e_cg >> 1) + 8 * (e_cg & 1));
      const uint32_t hw[4] = {raw.x & 0xFFFFu, raw.x >> 16, raw.y & 0xFFFFu, raw.y >> 16};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double x = static_cast<double>(kF16 ? f16_to_f32(static_cast<uint16_t>(hw[c]))
                                                  : bf16_to_f32(static_cast<uint16_t>(hw[c])));
        en[c] = fma(x, x, en[c]);
      }
    }
  };

  // Copies in flight per wave per stage (the fast path; tail stages load through
  // registers and are complete when issued).  Waiting for a stage means allowing the
  // copies of the `later` stages issued after it to stay outstanding.
  auto wait_copies = [&](int later) {
    const int n = later * (diag ? CPO : 2 * CPO);
    switch (n) {
      case 0: wait_vmcnt<0>(); break;
      case 2: wait_vmcnt<2>(); break;
      case 4: wait_vmcnt<4>(); break;
      case 6: wait_vmcnt<6>(); break;
      case 8: wait_vmcnt<8>(); break;
      default: wait_vmcnt<12>(); break;
    }
  };
  // operands of one 16-token step
  struct Ops {
    s16x4 a0[4], a1[4], b0[BN], b1[BN];
  };
  auto read_ops = [&](int stage, int ks, Ops& o) {
    const uint16_t* as = sA[stage % NBUF];
    const uint16_t* bs = diag ? as : sB[stage % NBUF];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      o.a0[bm] = operand(as, 128 * wm + 32 * bm, 16 * ks);
      o.a1[bm] = operand(as, 128 * wm + 32 * bm, 16 * ks + 4);
    }
#pragma unroll
    for (int bn = 0; bn < BN; ++bn) {
      o.b0[bn] = operand(bs, WC * wn + 32 * bn, 16 * ks);
      o.b1[bn] = operand(bs, WC * wn + 32 * bn, 16 * ks + 4);
    }
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < BN; ++bn) acc[bm][bn] = mfma16<kF16>(o.a0[bm], o.a1[bm], o.b0[bn], o.b1[bn], acc[bm][bn]);
    // keep the MFMAs ahead of the following wait/barrier (the compiler would otherwise sink
    // them below it and serialise them with the operand reads)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < BN; ++bn) asm volatile("" : "+v"(acc[bm][bn]));
  };

  for (int k = 0; k < DEPTH && k < nstages; ++k) load_stage(k);
  Ops P, Q;   // operand sets of alternate 16-token steps
  if (nstages > 0) {
    wait_copies(min(DEPTH, nstages) - 1);
    __syncthreads();
    read_ops(0, 0, P);
  }
  // Each stage runs in four 16-token steps; in each, the MFMAs of one step are issued while
  // the operand reads of the next step are in flight (P and Q alternate):
  //   read (s, 1) | MFMAs (s, 0);  read (s, 2) | MFMAs (s, 1);  read (s, 3) | MFMAs (s, 2);
  //   wait for the copies of stage s+1 and for this wave's reads of stage s, barrier;
  //   start the copy of stage s+2 into stage s's buffer;
  //   read (s+1, 0) | MFMAs (s, 3)
  for (int s = 0; s < nstages; ++s) {
    read_ops(s, 1, Q);
    mma(P);
    if (diag) energies(s);
    read_ops(s, 2, P);
    mma(Q);
    read_ops(s, 3, Q);
    mma(P);
    if (s + 1 < nstages) wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of stage s are done
    __syncthreads();
    if (s + 2 < nstages) load_stage(s + 2);   // into the buffer of stage s
    if (s + 1 < nstages) read_ops(s + 1, 0, P);
    mma(Q);
  }
  // Accumulator layout of a 32x32 MFMA block: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* Pt = partial + ((static_cast<int64_t>(e) * ksplit + split) * ntiles + tile) * static_cast<int64_t>(ST * ST);
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < BN; ++bn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 128 * wm + 32 * bm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = WC * wn + 32 * bn + (lane & 31);
        Pt[m * ST + n] = acc[bm][bn][r];
      }
  if (diag) {
    // the 8 token octets of each channel summed in order through LDS (free after the loop),
    // then this slice's energies of the tile's channels to epart[e][split][channel]
    __syncthreads();
    double* red = reinterpret_cast<double*>(&sA[0][0]);   // [8][256]
#pragma unroll
    for (int c = 0; c < 4; ++c) red[e_tg * ST + 4 * e_cg + c] = en[c];
    __syncthreads();
    if (tid < ST && I0 + tid < d_in) {
      double sum = 0.0;
#pragma unroll
      for (int g = 0; g < 8; ++g) sum += red[g * ST + tid];
      epart[(static_cast<int64_t>(e) * ksplit + split) * d_in + I0 + tid] = sum;
    }
  }
}

// Sums the token-slice partials of each lower tile in slice order and adds twice the
// sum to H and to its mirror.  Block: 64x64 sub-block of one tile, each thread 4 rows of
// 4 consecutive columns (16-byte loads; the slice loop is unrolled so several slices'
// loads are in flight, the additions keep slice order).  Mirror writes go through LDS so
// both stores are coalesced.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(const float* __restrict__ partial,
                                                          int nsplit, int ntiles, int d_in,
                                                          float* __restrict__ H, int64_t bsh) {
  __shared__ float tr[64][65];
  const int e = blockIdx.z;
  const int tile = blockIdx.y;
  const int sub = blockIdx.x;  // 16 sub-blocks of 64x64
  const int sm = (sub >> 2) * 64, sn = (sub & 3) * 64;
  int I, J;
  round_tile_coords(tile, (d_in + ST - 1) / ST, I, J);
  const bool diag = (I == J);
  if (diag && sm < sn) return;  // strictly-upper sub-block of a diagonal tile
  const int c4 = 4 * (threadIdx.x & 15), r0 = threadIdx.x >> 4;   // rows r0 + 16 q
  float* He = H + static_cast<int64_t>(e) * bsh;
  const int64_t tstride = static_cast<int64_t>(ST) * ST;
  const int64_t kstride = static_cast<int64_t>(ntiles) * tstride;
  const float* P0 = partial + (static_cast<int64_t>(e) * nsplit * ntiles + tile) * tstride + sm * ST + sn + c4;
  // The old values of H under the sub-block and under its mirror are loaded first, so that
  // their latency overlaps the partials' (after the sum, one read-modify-write and then the
  // other put two more latencies on every workgroup).  Each element of H belongs to one
  // sub-block, as lower value or as mirror, so no other workgroup writes what these read.
  // The four columns of a thread's row take one 16-byte read-modify-write where all four
  // are inside H and on or below the diagonal (and H's rows are 16-byte aligned).
  const bool vec_rows = (d_in % 4 == 0) && (reinterpret_cast<uintptr_t>(He) % 16 == 0);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  float4 hlo[4];
  bool hvec[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = sm + r0 + 16 * q;
    const int row = I * ST + m, col0 = J * ST + sn + c4;
    hvec[q] = vec_rows && row < d_in && col0 + 3 < d_in && (!diag || m >= sn + c4 + 3);
    if (hvec[q]) hlo[q] = *reinterpret_cast<const float4*>(He + static_cast<int64_t>(row) * d_in + col0);
  }
  float hmir[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int n = sn + ty + 4 * u, m = sm + tx;   // element (m, n) of the tile
    const int row = I * ST + m, col = J * ST + n;
    hmir[u] = (row < d_in && col < d_in && (!diag || m > n)) ? He[static_cast<int64_t>(col) * d_in + row] : 0.0f;
  }
  float4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int k = 0; k < nsplit; ++k) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(P0 + k * kstride + (r0 + 16 * q) * ST);
      acc[q].x += v.x; acc[q].y += v.y; acc[q].z += v.z; acc[q].w += v.w;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = r0 + 16 * q, m = sm + i;
    const float v[4] = {2.0f * acc[q].x, 2.0f * acc[q].y, 2.0f * acc[q].z, 2.0f * acc[q].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) tr[i][c4 + t] = v[t];
    const int row = I * ST + m, col0 = J * ST + sn + c4;
    if (hvec[q]) {
      float4 o = hlo[q];
      o.x += v[0]; o.y += v[1]; o.z += v[2]; o.w += v[3];
      *reinterpret_cast<float4*>(He + static_cast<int64_t>(row) * d_in + col0) = o;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = sn + c4 + t;
        const int col = col0 + t;
        if (row < d_in && col < d_in && (!diag || m >= n)) He[static_cast<int64_t>(row) * d_in + col] += v[t];
      }
    }
  }
  __syncthreads();
  // mirror: H[col][row] for the same sub-block, written along rows of the transpose
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int i = ty + 4 * u;
    const int n = sn + i, m = sm + tx;       // element (m, n) of the tile
    const int row = I * ST + m, col = J * ST + n;
    if (row < d_in && col < d_in && (!diag || m > n))
      He[static_cast<int64_t>(col) * d_in + row] = hmir[u] + tr[tx][i];
  }
}

// fp32 inputs: 64x64 lower tiles (blockIdx.x) and token slices (blockIdx.y), 256 threads
// with 4x4 outputs each, FMA in fp32.  With one slice the tile is added to H directly;
// otherwise it goes to partial[e][slice][tile][64][64] for syrk_f32_reduce_kernel.
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t bsx, int64_t n_tokens,
                                                       const int64_t* __restrict__ offsets, int64_t total_rows,
                                                       int d_in, int64_t tokens_per_split, int ntiles,
                                                       float* __restrict__ partial, float* __restrict__ H,
                                                       int64_t bsh) {
  __shared__ float sa[16][64];
  __shared__ float sb[16][64];
  const int e = blockIdx.z, split = blockIdx.y;
  int I, J;
  lower_tile_coords(blockIdx.x, I, J);
  const int I0 = I * 64, J0 = J * 64;
  const Rows pr = problem_rows(offsets, e, n_tokens, total_rows);
  const int64_t tb = static_cast<int64_t>(split) * tokens_per_split;
  const int64_t te = min(pr.count, tb + tokens_per_split);
  const float* Xe = X + static_cast<int64_t>(e) * bsx + pr.start * ldx;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = tb; t0 < te; t0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      const int k = i >> 6, c = i & 63;
      const int64_t t = t0 + k;
      const bool okt = t < te;
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
  if (gridDim.y > 1) {
    float* Pt = partial + ((static_cast<int64_t>(e) * gridDim.y + split) * ntiles + blockIdx.x) * 4096;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<float4*>(Pt + (ty * 4 + p) * 64 + tx * 4) = make_float4(acc[p][0], acc[p][1], acc[p][2],
                                                                              acc[p][3]);
    return;
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

// Sums the token slices of each 64x64 fp32 tile in slice order and adds twice the sum to H
// and its mirror (exactly symmetric).  Thread t takes elements t + 256 k of the tile.
__global__ __launch_bounds__(256) void syrk_f32_reduce_kernel(const float* __restrict__ partial, int nsplit,
                                                              int ntiles, int d_in, float* __restrict__ H,
                                                              int64_t bsh) {
  const int tile = blockIdx.x, e = blockIdx.y;
  int I, J;
  lower_tile_coords(tile, I, J);
  const bool diag = (I == J);
  float* He = H + static_cast<int64_t>(e) * bsh;
  const float* P0 = partial + (static_cast<int64_t>(e) * nsplit * ntiles + tile) * 4096;
  const int64_t kstride = static_cast<int64_t>(ntiles) * 4096;
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int idx = threadIdx.x + 256 * k, m = idx >> 6, n = idx & 63;
    float sum = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) sum += P0[sp * kstride + idx];
    const int row = I * 64 + m, col = J * 64 + n;
    if (row >= d_in || col >= d_in || (diag && m < n)) continue;
    const float v = 2.0f * sum;
    He[static_cast<int64_t>(row) * d_in + col] += v;
    if (!diag || m > n) He[static_cast<int64_t>(col) * d_in + row] += v;
  }
}

// fp64 channel energies sum_t x_tc^2 of one token slice: part[e][slice][c].  A thread
// owns V = 16 / sizeof(T) consecutive channels and reads them 16 bytes at a time (the
// squares are exact in fp64).
template <typename T>
__global__ __launch_bounds__(256) void channel_energy_kernel(const T* __restrict__ X, int64_t ldx,
                                                             int64_t bsx, int64_t n_tokens,
                                                             const int64_t* __restrict__ offsets, int64_t total_rows,
                                                             int d_in, int64_t tokens_per_split,
                                                             double* __restrict__ part) {
  constexpr int V = 16 / sizeof(T);
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * V;
  const int split = blockIdx.y, e = blockIdx.z;
  if (c0 >= d_in) return;
  const Rows pr = problem_rows(offsets, e, n_tokens, total_rows);
  const int64_t t0 = static_cast<int64_t>(split) * tokens_per_split;
  const int64_t t1 = min(pr.count, t0 + tokens_per_split);
  const T* Xe = X + static_cast<int64_t>(e) * bsx + pr.start * ldx + c0;
  double acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0;
#pragma unroll 4
  for (int64_t t = t0; t < t1; ++t) {
    const uint4 raw = *reinterpret_cast<const uint4*>(Xe + t * ldx);
    const T* x = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const double xv = static_cast<double>(load_as_f32(x + v));
      acc[v] = fma(xv, xv, acc[v]);
    }
  }
  double* dst = part + (static_cast<int64_t>(e) * gridDim.y + split) * d_in + c0;
#pragma unroll
  for (int v = 0; v < V; ++v) dst[v] = acc[v];
}

__global__ __launch_bounds__(256) void channel_energy_reduce_kernel(const double* __restrict__ part,
                                                                    int nsplit, int d_in,
                                                                    double* __restrict__ diag_key,
                                                                    int64_t* __restrict__ n_seen,
                                                                    int64_t n_tokens,
                                                                    const int64_t* __restrict__ offsets,
                                                                    int64_t total_rows) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c < d_in) {
    double s = 0.0;
#pragma unroll 8
    for (int k = 0; k < nsplit; ++k) s += part[(static_cast<int64_t>(e) * nsplit + k) * d_in + c];
    diag_key[static_cast<int64_t>(e) * d_in + c] += 2.0 * s;
  }
  if (c == 0) n_seen[e] += problem_rows(offsets, e, n_tokens, total_rows).count;
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
    // About 2048 workgroups (8 per CU): shorter token slices balance the CUs better than
    // the extra partial tiles cost in the reduction.  Then, among slice counts from 1/16
    // fewer up to 64, the one with the fewest rounds x tokens per slice (one workgroup fills
    // a CU; each partial tile costs the reduction about two tokens' worth of SYRK time): 15
    // rather than 16 slices at 136 tiles fill 8 rounds instead of leaving a ninth half empty.
    // Fewer slices than that never: longer fp32 accumulation chains make H less accurate.
    const int64_t tiles = static_cast<int64_t>(pl.ntiles) * batch;
    const int64_t want = (2048 + tiles - 1) / tiles;
    const int64_t cap = std::max<int64_t>(1, n_tokens / kMinTokensPerSplit);
    const int64_t kmin = std::min<int64_t>((n_tokens + kMaxTokensPerSplit - 1) / kMaxTokensPerSplit, 64);
    const int64_t base = std::max(kmin, std::min<int64_t>(std::min(want, cap), 64));
    const int n_cu = 256;
    double best = -1.0;
    for (int64_t k = std::max<int64_t>(kmin, std::max<int64_t>(1, base - base / 16)); k <= 64; ++k) {
      int64_t chunk = (n_tokens + k - 1) / k;
      chunk = std::max<int64_t>(SBK, (chunk + SBK - 1) / SBK * SBK);
      if (k > base && chunk < kMinTokensPerSplit) break;
      const int64_t ks = (n_tokens + chunk - 1) / chunk;
      const int64_t rounds = (tiles * ks + n_cu - 1) / n_cu;
      const double cost = static_cast<double>(rounds) * static_cast<double>(chunk) + 2.0 * static_cast<double>(ks * tiles);
      if (best < 0.0 || cost < best) {
        best = cost;
        pl.kchunk = chunk;
        pl.ksplit = static_cast<int>(std::max<int64_t>(1, ks));
      }
    }
  }
  if (!mfma) {
    // fp32 inputs (small layers): about 512 workgroups over tiles and token slices of at
    // least 128 tokens, at most 64 slices
    const int64_t tiles = static_cast<int64_t>(pl.ntiles) * batch;
    const int64_t k = std::min<int64_t>(std::min<int64_t>((512 + tiles - 1) / tiles, 64),
                                        std::max<int64_t>(1, n_tokens / 128));
    pl.kchunk = ((n_tokens + k - 1) / k + 15) / 16 * 16;
    pl.ksplit = static_cast<int>((n_tokens + pl.kchunk - 1) / pl.kchunk);
  }
  if (mfma) {   // energies from the SYRK's diagonal tiles, one partial per token slice
    pl.esplit = pl.ksplit;
    pl.echunk = pl.kchunk;
    return pl;
  }
  // energy kernel: 16-byte loads of 16 / elem_bytes channels per thread, ~1024 workgroups,
  // at least 256 tokens per slice, at most 256 slices (their sum is one thread per channel)
  const int vec = mfma ? 8 : 4;
  const int cblocks = (d_in + 256 * vec - 1) / (256 * vec);
  const int64_t ewant = (1024 + static_cast<int64_t>(cblocks) * batch - 1) /
                        (static_cast<int64_t>(cblocks) * batch);
  const int64_t ecap = std::max<int64_t>(1, n_tokens / 256);
  pl.esplit = static_cast<int>(std::min<int64_t>(std::min(ewant, ecap), 256));
  pl.echunk = (n_tokens + pl.esplit - 1) / pl.esplit;
  if (pl.echunk == 0) pl.echunk = 1;
  pl.esplit = static_cast<int>(std::max<int64_t>(1, (n_tokens + pl.echunk - 1) / pl.echunk));
  return pl;
}

size_t plan_bytes(const HessianPlan& pl, int batch, int d_in, float** partial, double** epart,
                  void* ws) {
  Carver cv(ws);
  float* p = nullptr;
  if (pl.mfma)
    p = cv.take<float>(static_cast<size_t>(batch) * pl.ksplit * pl.ntiles * ST * ST);
  else if (pl.ksplit > 1)
    p = cv.take<float>(static_cast<size_t>(batch) * pl.ksplit * pl.ntiles * 64 * 64);
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
                            int64_t ldx, int64_t bsx, const int64_t* offsets, int64_t total_rows, float* H,
                            int64_t bsh, double* diag_key, int64_t* n_seen, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
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
    // The fp64 channel energies come out of the SYRK's diagonal tiles (epart[e][slice][c]).
    const dim3 sblk(64 * SYRK_WAVES);
    const dim3 grid(pl.ntiles * pl.ksplit, batch);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    // Tiles always go through the partial buffer and the ordered reduction, also with a
    // single token slice: the reduction writes the mirror half through LDS with coalesced
    // stores, where an epilogue in the SYRK would add to H column by column (one 4-byte
    // read-modify-write per 128-byte line).
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    timing_pair(GPTQ_TIME_SYRK, &ev0, &ev1);
    if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
    if (x_dtype == GPTQ_F16) {
      GPTQ_LAUNCH((syrk_mfma_kernel<true, SYRK_WAVES>), grid, sblk, 0, stream, Xh, ldx, bsx, n_tokens, offsets,
                  total_rows, d_in, pl.kchunk, pl.ksplit, partial, pl.ntiles, epart);
    } else {
      GPTQ_LAUNCH((syrk_mfma_kernel<false, SYRK_WAVES>), grid, sblk, 0, stream, Xh, ldx, bsx, n_tokens, offsets,
                  total_rows, d_in, pl.kchunk, pl.ksplit, partial, pl.ntiles, epart);
    }
    if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
    GPTQ_LAUNCH(syrk_reduce_kernel, dim3(16, pl.ntiles, batch), blk, 0, stream, partial, pl.ksplit, pl.ntiles, d_in,
                H, bsh);
  } else {
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    timing_pair(GPTQ_TIME_SYRK, &ev0, &ev1);
    if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
    GPTQ_LAUNCH(syrk_f32_kernel, dim3(pl.ntiles, pl.ksplit, batch), blk, 0, stream, static_cast<const float*>(X), ldx,
                bsx, n_tokens, offsets, total_rows, d_in, pl.kchunk, pl.ntiles, partial, H, bsh);
    if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
    if (pl.ksplit > 1)
      GPTQ_LAUNCH(syrk_f32_reduce_kernel, dim3(pl.ntiles, batch), blk, 0, stream, partial, pl.ksplit, pl.ntiles, d_in,
                  H, bsh);
    const dim3 egrid((d_in + 1023) / 1024, pl.esplit, batch);
    GPTQ_LAUNCH(channel_energy_kernel<float>, egrid, blk, 0, stream, static_cast<const float*>(X), ldx, bsx, n_tokens,
                offsets, total_rows, d_in, pl.echunk, epart);
  }
  GPTQ_LAUNCH(channel_energy_reduce_kernel, dim3((d_in + 255) / 256, batch), blk, 0, stream, epart,
              pl.esplit, d_in, diag_key, n_seen, n_tokens, offsets, total_rows);
  return GPTQ_OK;
}

}  // namespace gptq
