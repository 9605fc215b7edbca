// fp32-accurate GEMM on the gfx950 matrix cores:
//   C = alpha * op(A) * op(B) + beta * C,   A [M, K], op(B) = B [K, N] or B^T (B [N, K]),
// batched over blockIdx.z (two nested batch strides).
//
// Used for the blocked Cholesky (panel solve as a product with the inverted diagonal
// block, trailing symmetric update), the triangular inverse, and GPTQ's lazy batch update
// W[:, later] -= Err @ U[block, later] ("Same Ruler, Smarter Placement: GPTQ", 1.8).
// Products and sums are fp32, as the quantizer's arithmetic requires.
//
// Two kernels:
//  * gemm_x6_kernel, for products that fill the chip with 128 x 128 tiles: the operands
//    split into three bf16 parts each and six bf16 MFMAs per block (fp32 accuracy at 2.7x
//    the rate of the fp32 matrix instruction; see the comment at the kernel);
//  * gemm_f32_kernel (v_mfma_f32_32x32x2_f32), 128 x 128 x 32 tiles for large products
//    whose shapes are not multiples of 4, and 64 x 64 x 64 tiles for the small products of
//    the Cholesky chain.
// Both: 256 threads = 4 waves, each owning a quarter of the tile as 32 x 32 MFMA blocks;
// triangular operands shrink the K range per tile; a lower-only output skips tiles above
// the diagonal.
#include <algorithm>
#include <type_traits>

#include "common.h"


namespace gptq {
namespace {

// TT = output tile edge (128 or 64); each of the 4 waves owns a (TT/2) x (TT/2) quarter as
// MB x MB blocks of 32 x 32.  The 64-wide tile takes 64 k per stage: with one workgroup per
// CU its stage is otherwise too short to cover the latency of the next stage's loads.
// kVec: K, N and the leading dimensions are multiples of 4 and the operands 16-byte aligned;
// loads are then unconditional 16-byte loads from clamped addresses, with the elements
// outside the product zeroed when the stage is stored to LDS.  (Editing a loaded register
// right after its load, as the general path does for a partial vector, makes the compiler
// wait for every load as it is issued.)
// kRole: 0 for the factorization's products, 1 for the quantizer's lazy trailing updates
// (identical code; separate instantiations so that kernel traces tell them apart).
template <bool kTransB, int TT, bool kVec, int kRole>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int GT = TT;
  constexpr int GK = TT == 64 ? 64 : 32;
  // LDS row lengths.  Rows written by the transposing scalar stores get an odd length, so
  // the 8 k rows x 4 tile rows that half a wave writes fall on 32 different banks; rows
  // written as float4 (B already k-major) keep 16-byte alignment.
  constexpr int GPA = GT + 1;
  constexpr int GPB = kTransB ? GT + 1 : GT + 4;
  constexpr int MB = TT / 64;
  constexpr int RQ = GT * GK / 1024;  // float4 loads per thread per operand and stage
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, so with 8 column tiles
  // per row XCD c would get every tile of column c.  Triangular operands and lower-only
  // outputs make the work of a tile depend on its column, so the column index is rotated
  // by the row and batch index: every XCD gets a mix of columns.
  const int bx = static_cast<int>((blockIdx.x + blockIdx.y + blockIdx.z) % gridDim.x);
  const int n0 = bx * GT, m0 = blockIdx.y * GT;
  if ((g.flags & kLowerOut) && n0 > m0) return;
  const int zo = blockIdx.z / g.batch2, zi = blockIdx.z % g.batch2;
  const float* A = g.A + static_cast<int64_t>(zo) * g.sA + static_cast<int64_t>(zi) * g.sA2;
  const float* B = g.B + static_cast<int64_t>(zo) * g.sB + static_cast<int64_t>(zi) * g.sB2;
  float* C = g.C + static_cast<int64_t>(zo) * g.sC + static_cast<int64_t>(zi) * g.sC2;

  int kb = 0, ke = g.K;
  if (g.flags & kALower) ke = min(ke, m0 + GT);
  if (g.flags & kBtLower) ke = min(ke, n0 + GT);
  if (g.flags & kBLower) kb = max(kb, n0);
  kb = kb / GK * GK;

  __shared__ __attribute__((aligned(16))) float sA[2][GK][GPA];
  __shared__ __attribute__((aligned(16))) float sB[2][GK][GPB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // loads run two stages ahead through a ring of two register sets
  float4 ra[2][RQ], rb[2][RQ];
  // Row-major tile [GT rows][GK k] read as float4: half a wave covers 4 rows x 8 k-vectors
  // (row lr + RS q, k 4 lc .. 4 lc + 3), which makes its transposing LDS stores conflict-free.
  constexpr int RS = 1024 / GK;  // rows per pass of the workgroup
  const int lc = GK == 32 ? (lane & 7) : (lane & 7) + 8 * (lane >> 5);
  const int lr = GK == 32 ? (lane >> 3) + 8 * wave : ((lane >> 3) & 3) + 4 * wave;
  auto load_rows = [&](const float* P, int64_t ld, int r0, int rlim, int k0, float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int row = r0 + lr + RS * q;
      const int k = k0 + 4 * lc;
      if constexpr (kVec) {
        r[q] = *reinterpret_cast<const float4*>(P + static_cast<int64_t>(min(row, rlim - 1)) * ld + min(k, ke - 4));
        continue;
      }
      if (row < rlim && k < ke) {
        r[q] = *reinterpret_cast<const float4*>(P + static_cast<int64_t>(row) * ld + k);
        if (k + 4 > ke) {  // partial K vector: zero the tail
          if (k + 1 >= ke) r[q].y = 0.0f;
          if (k + 2 >= ke) r[q].z = 0.0f;
          if (k + 3 >= ke) r[q].w = 0.0f;
        }
      } else {
        r[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_rows = [&](auto s, const float4* r, int r0, int rlim, int k0) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int row = lr + RS * q;
      const int k = 4 * lc;
      float4 v = r[q];
      if constexpr (kVec) {
        if (!(r0 + row < rlim && k0 + k < ke)) v = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      s[k + 0][row] = v.x;
      s[k + 1][row] = v.y;
      s[k + 2][row] = v.z;
      s[k + 3][row] = v.w;
    }
  };
  // B tile [GK k][GT n] (no transpose): thread loads k = tid / (GT/4) + (256*4/GT) q,
  // n = 4 * (tid % (GT/4))
  constexpr int NV = GT / 4;        // float4 per k row
  constexpr int KS = 256 / NV;      // k rows covered by one pass of the block
  auto load_kmajor = [&](int k0, float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int k = k0 + tid / NV + KS * q;
      const int n = n0 + 4 * (tid % NV);
      if constexpr (kVec) {
        r[q] = *reinterpret_cast<const float4*>(B + static_cast<int64_t>(min(k, ke - 1)) * g.ldb + min(n, g.N - 4));
        continue;
      }
      if (k < ke && n < g.N) {
        if (n + 4 <= g.N) {
          r[q] = *reinterpret_cast<const float4*>(B + static_cast<int64_t>(k) * g.ldb + n);
        } else {
          const float* p = B + static_cast<int64_t>(k) * g.ldb + n;
          r[q].x = p[0];
          r[q].y = (n + 1 < g.N) ? p[1] : 0.0f;
          r[q].z = (n + 2 < g.N) ? p[2] : 0.0f;
          r[q].w = 0.0f;
        }
      } else {
        r[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_kmajor = [&](float (*s)[GPB], const float4* r, int k0) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int k = tid / NV + KS * q;
      float4 v = r[q];
      if constexpr (kVec) {
        if (!(k0 + k < ke && n0 + 4 * (tid % NV) < g.N)) v = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      *reinterpret_cast<float4*>(&s[k][4 * (tid % NV)]) = v;
    }
  };
  auto load_b = [&](int k0, float4* r) {
    if constexpr (kTransB) load_rows(B, g.ldb, n0, g.N, k0, r);
    else load_kmajor(k0, r);
  };
  auto store_b = [&](float (*s)[GPB], const float4* r, int k0) {
    if constexpr (kTransB) store_rows(s, r, n0, g.N, k0);
    else store_kmajor(s, r, k0);
  };

  f32x16 acc[MB][MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int l32 = lane & 31, kh = lane >> 5;
  // 32x32 accumulator layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  // 64-wide tiles (one 32 x 32 block per wave, short K loops): with beta != 0 the old C
  // values are loaded before the K loop, so that their latency overlaps it rather than
  // following it (C never overlaps A or B).
  const bool has_beta = g.beta != 0.0f;
  constexpr bool kPreC = (MB == 1);
  float preC[16];
  if constexpr (kPreC) {
    const int n = n0 + (GT / 2) * wn + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + (GT / 2) * wm + 8 * (r >> 2) + 4 * kh + (r & 3);
      preC[r] = (has_beta && m < g.M && n < g.N) ? C[static_cast<int64_t>(m) * g.ldc + n] : 0.0f;
    }
  }
  const int nk = ke > kb ? (ke - kb + GK - 1) / GK : 0;
  if (nk > 0) {
    load_rows(A, g.lda, m0, g.M, kb, ra[0]);
    load_b(kb, rb[0]);
    if (nk > 1) {
      load_rows(A, g.lda, m0, g.M, kb + GK, ra[1]);
      load_b(kb + GK, rb[1]);
    }
    store_rows(sA[0], ra[0], m0, g.M, kb);
    store_b(sB[0], rb[0], kb);
  }
  __syncthreads();
  // iteration s: loads of stage s + 2 into the register set of stage s (stored to LDS one
  // iteration earlier) | products of LDS buffer s % 2 | stage s + 1 from the other register
  // set into the other buffer.  Unrolled by two so that the register sets are fixed.
  auto iteration = [&](int s, auto bc) {
    constexpr int buf = decltype(bc)::value;
    if (s + 2 < nk) {
      load_rows(A, g.lda, m0, g.M, kb + (s + 2) * GK, ra[buf]);
      load_b(kb + (s + 2) * GK, rb[buf]);
    }
#pragma unroll
    for (int kk = 0; kk < GK / 2; ++kk) {
      float av[MB], bv[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        av[b] = sA[buf][2 * kk + kh][(GT / 2) * wm + 32 * b + l32];
        bv[b] = sB[buf][2 * kk + kh][(GT / 2) * wn + 32 * b + l32];
      }
#pragma unroll
      for (int bm = 0; bm < MB; ++bm)
#pragma unroll
        for (int bn = 0; bn < MB; ++bn)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[bm], bv[bn], acc[bm][bn], 0, 0, 0);
    }
    if (s + 1 < nk) {
      store_rows(sA[buf ^ 1], ra[buf ^ 1], m0, g.M, kb + (s + 1) * GK);
      store_b(sB[buf ^ 1], rb[buf ^ 1], kb + (s + 1) * GK);
    }
    __syncthreads();
  };
  for (int s = 0; s < nk; s += 2) {
    iteration(s, std::integral_constant<int, 0>{});
    if (s + 1 < nk) iteration(s + 1, std::integral_constant<int, 1>{});
  }

  // With beta != 0 (128-wide tiles) the 16 old values of a block are all loaded before any
  // of its stores: element by element, every load would have to wait for the previous
  // store (the compiler cannot tell that they never overlap).
#pragma unroll
  for (int bm = 0; bm < MB; ++bm)
#pragma unroll
    for (int bn = 0; bn < MB; ++bn) {
      const int n = n0 + (GT / 2) * wn + 32 * bn + l32;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (GT / 2) * wm + 32 * bm + 8 * (r >> 2) + 4 * kh + (r & 3);
        if constexpr (kPreC) old[r] = preC[r];
        else old[r] = (has_beta && m < g.M && n < g.N) ? C[static_cast<int64_t>(m) * g.ldc + n] : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (GT / 2) * wm + 32 * bm + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (m < g.M && n < g.N) {
          const float v = g.alpha * acc[bm][bn][r];
          C[static_cast<int64_t>(m) * g.ldc + n] = has_beta ? fmaf(g.beta, old[r], v) : v;
        }
      }
    }
}


// ---------------------------------------------------------------------------------------
// The same product on the bf16 matrix cores, at fp32 accuracy, by splitting the operands.
// Each fp32 value is written as x = x0 + x1 + x2 with x0 = bf16(x), x1 = bf16(x - x0),
// x2 = bf16(x - x0 - x1) (round to nearest even, unit roundoff 2^-8 for bf16's 8-bit
// significand; every difference is exact in fp32), so |x - x0 - x1 - x2| <= 2^-24 |x|.  Of
// the nine cross products a_i b_j the six with i + j <= 2 are kept; the dropped ones and the
// two residuals change a product by at most about 2^-22 |a b|, the order of the fp32
// roundings of the accumulation itself.  Products of two bf16 values are exact in fp32 and
// the sums are fp32, as in the fp32 kernel: the operands are never rounded to a 16-bit type
// as a whole.
// Six v_mfma_f32_32x32x16_bf16 per 32x32x16 block run at 2500 / 6 = 417 TFLOP/s of fp32
// products against 157 TFLOP/s for v_mfma_f32_32x32x2_f32.
//
// Tile 128 x 128 x 16, 256 threads = 4 waves of 64 x 64 (2 x 2 blocks of 32 x 32), three
// workgroups per CU.  The three parts are stored in LDS as bf16 planes: A (and B^T)
// with K contiguous per row, 32 bytes = two 16-byte chunks per row, the chunks of rows
// 8..15 (mod 16) swapped, so that a 16-lane read of 16 bytes per lane (rows r..r+15, one k
// half) and a 32-lane write of 8 bytes per lane (8 whole rows) each cover all 64 banks
// once; B [K, N] with N contiguous, 256-byte k rows with the 8-byte n-quads of rows k+1..3
// (mod 4) moved by 64 bytes each, read with the transposing ds_read_b64_tr_b16 (a half wave
// covers all banks once).  48 KB of LDS per workgroup either way: three fit a CU.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short s16x4v __attribute__((ext_vector_type(4)));
typedef short s16x8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4v lds_s16x4v;

// 16-byte chunk swap of K-contiguous plane rows 8..15 (mod 16)
__device__ __forceinline__ int chunk_swz(int row) { return (row >> 3) & 1; }
// physical 8-byte n-quad of quad q in k row k of an N-contiguous plane (256-byte rows): rows
// k, k+1, k+2, k+3 move their quads by 64 bytes each, so the 4 rows x 8 quads of a half
// wave's transposing read, and a 32-lane write of one row, cover all 64 banks once
__device__ __forceinline__ int quad_swz(int k, int q) { return q ^ (8 * (k & 3)); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// parts (x0, x1, x2) of 4 consecutive values, each as 4 packed bf16
__device__ __forceinline__ void split3(const float4 v, uint2& p0, uint2& p1, uint2& p2) {
  const uint32_t a0 = pack_bf16(v.x, v.y), b0 = pack_bf16(v.z, v.w);
  const float rx = v.x - bf16_lo(a0), ry = v.y - bf16_hi(a0), rz = v.z - bf16_lo(b0), rw = v.w - bf16_hi(b0);
  const uint32_t a1 = pack_bf16(rx, ry), b1 = pack_bf16(rz, rw);
  const uint32_t a2 = pack_bf16(rx - bf16_lo(a1), ry - bf16_hi(a1)), b2 = pack_bf16(rz - bf16_lo(b1), rw - bf16_hi(b1));
  p0 = make_uint2(a0, b0);
  p1 = make_uint2(a1, b1);
  p2 = make_uint2(a2, b2);
}

// v where `in`, else zeros, as bitwise ANDs (a select here compiles to a branch, which
// would split the loop body into blocks that the scheduler cannot interleave)
__device__ __forceinline__ float4 masked(const float4 v, bool in) {
  const uint32_t k = in ? 0xFFFFFFFFu : 0u;
  return make_float4(__uint_as_float(__float_as_uint(v.x) & k), __uint_as_float(__float_as_uint(v.y) & k),
                     __uint_as_float(__float_as_uint(v.z) & k), __uint_as_float(__float_as_uint(v.w) & k));
}

// One 128 x 128 tile (column tile bx, row tile by, product bz) of the split-bf16 product.
template <bool kTransB>
__device__ __forceinline__ void gemm_x6_tile(const GemmArgs& g, int bx, int by, int bz) {
  constexpr int GT = 128, GK = 16;
  constexpr int PA = GK;                       // bf16 per K-contiguous row (two 16-byte chunks)
  constexpr int PB = GT;                       // bf16 per k row of the N-contiguous layout
  constexpr int A_PLANE = GT * PA;
  constexpr int B_PLANE = kTransB ? GT * PA : GK * PB;
  constexpr int RQ = GT * GK / 1024;           // float4 per thread per operand and stage (2)
  const int n0 = bx * GT, m0 = by * GT;
  if ((g.flags & kLowerOut) && n0 > m0) return;
  const int zo = bz / g.batch2, zi = bz % g.batch2;
  const float* A = g.A + static_cast<int64_t>(zo) * g.sA + static_cast<int64_t>(zi) * g.sA2;
  const float* B = g.B + static_cast<int64_t>(zo) * g.sB + static_cast<int64_t>(zi) * g.sB2;
  float* C = g.C + static_cast<int64_t>(zo) * g.sC + static_cast<int64_t>(zi) * g.sC2;

  int kb = 0, ke = g.K;
  if (g.flags & kALower) ke = min(ke, m0 + GT);
  if (g.flags & kBtLower) ke = min(ke, n0 + GT);
  if (g.flags & kBLower) kb = max(kb, n0);
  kb = kb / GK * GK;

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][3 * A_PLANE];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][3 * B_PLANE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global loads run two stages ahead through a ring of two register sets (a 16-deep
  // stage is too short to cover their latency on its own)
  float4 ra[2][RQ], rb[2][RQ];
  // Loads are unconditional 16-byte loads from clamped (always valid) addresses; whether
  // an element is inside the product is applied when the stage is split into LDS.  No
  // branch or register write touches a load's destination before that, so the loads of a
  // stage stay in flight until then.  (The host uses this kernel only when K, N and the
  // leading dimensions are multiples of 4 and the operands 16-byte aligned, so a vector
  // with k < ke lies entirely inside the K range.)
  // K-contiguous rows: float4 f = tid + 256 q is (row f / 4, k 4 (f % 4))
  auto load_rows = [&](const float* P, int64_t ld, int r0, int rlim, int k0, float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int f = tid + 256 * q;
      const int row = min(r0 + f / 4, rlim - 1), k = min(k0 + 4 * (f % 4), ke - 4);
      r[q] = *reinterpret_cast<const float4*>(P + static_cast<int64_t>(row) * ld + k);
    }
  };
  auto store_rows = [&](uint16_t* s, const float4* r, int r0, int rlim, int k0) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int f = tid + 256 * q;
      const bool in = (r0 + f / 4 < rlim) && (k0 + 4 * (f % 4) < ke);
      const float4 v = masked(r[q], in);
      uint2 p0, p1, p2;
      split3(v, p0, p1, p2);
      const int row = f / 4, k4 = f % 4;
      uint16_t* d = s + row * PA + 8 * ((k4 >> 1) ^ chunk_swz(row)) + 4 * (k4 & 1);
      *reinterpret_cast<uint2*>(d) = p0;
      *reinterpret_cast<uint2*>(d + A_PLANE) = p1;
      *reinterpret_cast<uint2*>(d + 2 * A_PLANE) = p2;
    }
  };
  // B [K, N], N contiguous: float4 f = tid + 256 q is (k f / 32, n 4 (f % 32))
  auto load_kmajor = [&](int k0, float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int f = tid + 256 * q;
      const int k = min(k0 + f / (GT / 4), ke - 1);
      const int n = min(n0 + 4 * (f % (GT / 4)), g.N - 4);
      r[q] = *reinterpret_cast<const float4*>(B + static_cast<int64_t>(k) * g.ldb + n);
    }
  };
  auto store_kmajor = [&](uint16_t* s, const float4* r, int k0) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int f = tid + 256 * q;
      const bool in = (k0 + f / (GT / 4) < ke) && (n0 + 4 * (f % (GT / 4)) < g.N);
      const float4 v = masked(r[q], in);
      uint2 p0, p1, p2;
      split3(v, p0, p1, p2);
      const int k = f / (GT / 4);
      uint16_t* d = s + k * PB + 4 * quad_swz(k, f % (GT / 4));
      *reinterpret_cast<uint2*>(d) = p0;
      *reinterpret_cast<uint2*>(d + B_PLANE) = p1;
      *reinterpret_cast<uint2*>(d + 2 * B_PLANE) = p2;
    }
  };
  auto load_stage = [&](int st, int slot) {
    load_rows(A, g.lda, m0, g.M, kb + st * GK, ra[slot]);
    if constexpr (kTransB) load_rows(B, g.ldb, n0, g.N, kb + st * GK, rb[slot]);
    else load_kmajor(kb + st * GK, rb[slot]);
  };
  auto store_stage = [&](int st, int buf, int slot) {
    store_rows(sA[buf], ra[slot], m0, g.M, kb + st * GK);
    if constexpr (kTransB) store_rows(sB[buf], rb[slot], n0, g.N, kb + st * GK);
    else store_kmajor(sB[buf], rb[slot], kb + st * GK);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // operand of a 32 x 16 block from a K-contiguous plane: lane l holds row l % 32,
  // k 8 (l / 32) .. + 7
  const int l32 = lane & 31, kh = lane >> 5;
  auto rd_rows = [&](const uint16_t* plane, int r0) -> s16x8v {
    const int row = r0 + l32;
    return *reinterpret_cast<const s16x8v*>(plane + row * PA + 8 * (kh ^ chunk_swz(row)));
  };
  // operand of a 16 x 32 block from the N-contiguous plane by two transposing reads
  // (4 k rows x 4 n-quads per 16 lanes; the second read is 4 k rows further on)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int tr_n = 16 * (g16 & 1) + 4 * (j16 & 3);
  const int tr_k = 8 * (g16 >> 1) + (j16 >> 2);
  auto rd_tr = [&](const uint16_t* plane, int c0) -> s16x8v {
    const int q = (c0 + tr_n) >> 2;   // the lane's n-quad; rows tr_k and tr_k + 4 share k mod 4
    const uint16_t* p = plane + tr_k * PB + 4 * quad_swz(tr_k, q);
    const s16x4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4v*)(p));
    const s16x4v y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4v*)(p + 4 * PB));
    return s16x8v{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  };

  // Stages past the K range split to zeros, so the stage count is rounded up to even and
  // every load and store below is unconditional: with a fixed number of loads in flight
  // the compiler waits for exactly the stage it stores, never for the one just issued.
  const int nk = ke > kb ? (ke - kb + GK - 1) / GK : 0;
  if (nk > 0) {
    const int nk2 = (nk + 1) & ~1;
    load_stage(0, 0);
    load_stage(1, 1);
    store_stage(0, 0, 0);
    __syncthreads();
    // iteration s: loads of stage s + 2 into register slot s % 2 | products of LDS buffer
    // s % 2 | stage s + 1 (loaded one iteration earlier, slot (s + 1) % 2) into the other
    // buffer.  Unrolled by two so that the slots are compile-time registers.
    auto iteration = [&](int s, auto bc) {
      constexpr int buf = decltype(bc)::value;
      load_stage(min(s + 2, nk2 - 1), buf);
      // operand parts are read in the order the products below first need them (a0 b0,
      // b1, a1, b2, a2), so the first products wait for two reads, not for all twelve
      s16x8v av[3][2], bv[3][2];
      auto rd_a = [&](int p) {
#pragma unroll
        for (int b = 0; b < 2; ++b) av[p][b] = rd_rows(sA[buf] + p * A_PLANE, 64 * wm + 32 * b);
      };
      auto rd_b = [&](int p) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if constexpr (kTransB) bv[p][b] = rd_rows(sB[buf] + p * B_PLANE, 64 * wn + 32 * b);
          else bv[p][b] = rd_tr(sB[buf] + p * B_PLANE, 64 * wn + 32 * b);
        }
      };
      rd_a(0);
      rd_b(0);
      rd_b(1);
      rd_a(1);
      rd_b(2);
      rd_a(2);
      // parts (i, j) with i + j <= 2; the four blocks interleave so that consecutive
      // products never wait on one accumulator
      constexpr int PI[6] = {0, 0, 1, 1, 0, 2};
      constexpr int PJ[6] = {0, 1, 0, 1, 2, 0};
#pragma unroll
      for (int t = 0; t < 6; ++t)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
          for (int bn = 0; bn < 2; ++bn)
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[PI[t]][bm]),
                                                                  __builtin_bit_cast(bf16x8, bv[PJ[t]][bn]),
                                                                  acc[bm][bn], 0, 0, 0);
      store_stage(s + 1, buf ^ 1, buf ^ 1);   // past the last stage: zeros, never read
      // The next stage's split (VALU) and LDS stores are independent of this stage's
      // products: interleave them, a few instructions after every MFMA, so that the matrix
      // core keeps issuing while they run (left to itself the scheduler issues all MFMAs
      // first, and the waves of a workgroup, in step between barriers, then all split at
      // once with the matrix core idle).
      static_for(std::make_integer_sequence<int, 24>{}, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
        if constexpr (i % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // an LDS store
      });
      __syncthreads();
    };
    for (int s = 0; s < nk2; s += 2) {
      iteration(s, std::integral_constant<int, 0>{});
      iteration(s + 1, std::integral_constant<int, 1>{});
    }
  }

  // 32x32 accumulator layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  // With beta != 0 each block's 16 old values are loaded before the previous block's
  // stores, so that the loads of the next block are in flight while a block is written
  // (the compiler cannot move them there itself, not knowing that the blocks never
  // overlap); all four blocks at once would keep 64 more addresses and values live.
  const bool has_beta = g.beta != 0.0f;
  float old[2][16];
  auto load_old = [&](int blk, float* o) {
    const int bm = blk >> 1, bn = blk & 1;
    const int n = n0 + 64 * wn + 32 * bn + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 64 * wm + 32 * bm + 8 * (r >> 2) + 4 * kh + (r & 3);
      o[r] = (has_beta && m < g.M && n < g.N) ? C[static_cast<int64_t>(m) * g.ldc + n] : 0.0f;
    }
  };
  load_old(0, old[0]);
  static_for(std::make_integer_sequence<int, 4>{}, [&](auto bc) {
    constexpr int blk = decltype(bc)::value;
    constexpr int bm = blk >> 1, bn = blk & 1;
    if constexpr (blk + 1 < 4) load_old(blk + 1, old[(blk + 1) & 1]);
    const int n = n0 + 64 * wn + 32 * bn + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 64 * wm + 32 * bm + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (m < g.M && n < g.N) {
        const float v = g.alpha * acc[bm][bn][r];
        C[static_cast<int64_t>(m) * g.ldc + n] = has_beta ? fmaf(g.beta, old[blk & 1][r], v) : v;
      }
    }
  });
}

// Tile of this workgroup.  Workgroups start in linear order (x fastest), dealt to the 8
// XCDs round-robin (XCD = id % 8), so XCD x runs ids x, x + 8, x + 16, ...  The tiles are
// ordered in bands of kBand tile rows (the rows of all batch entries stacked), column by
// column inside a band, and XCD x takes the x-th of 8 consecutive runs of that order, one
// tile per id in its turn.  The ~96 workgroups an XCD holds at once then cover about 24
// columns of 4 rows, whose 28 operand panels its L2 shares, instead of tiles strewn over
// the grid.  col_bands: the same with rows and columns exchanged (bands of kBand tile
// columns, row by row), for products whose work per tile grows with the row, so that
// every band, and so every XCD's run, holds light and heavy rows alike.
constexpr int kBand = 4;
__device__ __forceinline__ void xcd_band_tile(bool col_bands, int& bx, int& by, int& bz) {
  const int nx = gridDim.x, ny = gridDim.y;
  const int total = nx * ny * static_cast<int>(gridDim.z);
  const int lin = static_cast<int>(blockIdx.x) + nx * (static_cast<int>(blockIdx.y) + ny * static_cast<int>(blockIdx.z));
  const int x = lin & 7, s = lin >> 3;
  // ids on XCD x: ceil((total - x) / 8); the runs before x hold those of XCDs 0 .. x-1
  const int q = total >> 3, r = total & 7;
  const int t = x * q + min(x, r) + s;
  const int rows = ny * static_cast<int>(gridDim.z);
  const int lines = col_bands ? nx : rows;     // what the bands cut
  const int across = col_bands ? rows : nx;    // what a band runs along
  const int band = t / (kBand * across);
  const int hb = min(kBand, lines - band * kBand);
  const int u = t - band * kBand * across;
  const int along = u / hb, line = band * kBand + u % hb;
  const int row = col_bands ? along : line;
  bx = col_bands ? line : along;
  by = row % ny;
  bz = row / ny;
}

// kPersist: a grid of fewer workgroups than tiles, each taking every gridDim.x-th tile in
// turn (lower tiles only with kLowerOut, row by row).  Otherwise one tile per workgroup:
// the lazy updates, plain products and those with one triangular operand in the XCD band
// order above; lower-only outputs (and the remaining flag combinations) with the column
// index rotated by the row and batch index, so that the XCDs, dealt workgroups round-robin
// by linear id, mix tiles whose work depends on the column.
template <bool kTransB, int kRole, bool kPersist = false>
__global__ __launch_bounds__(256, 2) void gemm_x6_kernel(GemmArgs g) {
  if constexpr (kPersist) {
    const int tm = (g.M + 127) / 128, tn = (g.N + 127) / 128;
    const bool lower = (g.flags & kLowerOut) != 0;
    const int per = lower ? tm * (tm + 1) / 2 : tm * tn;   // lower: C is square
    const int total = per * g.batch * g.batch2;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
      const int z = t / per, u = t - z * per;
      int by, bx;
      if (lower) {
        by = static_cast<int>((sqrtf(8.0f * static_cast<float>(u) + 1.0f) - 1.0f) * 0.5f);
        while ((by + 1) * (by + 2) / 2 <= u) ++by;
        while (by * (by + 1) / 2 > u) --by;
        bx = u - by * (by + 1) / 2;
      } else {
        by = u / tn;
        bx = u - by * tn;
      }
      gemm_x6_tile<kTransB>(g, bx, by, z);
      __syncthreads();   // the next tile refills the LDS stages
    }
  } else if (kRole == 1 || g.flags == 0 || g.flags == kBLower || g.flags == kALower) {
    // rectangular products, and triangular ones whose work varies along one axis only
    int bx, by, bz;
    xcd_band_tile(g.flags == kALower, bx, by, bz);
    gemm_x6_tile<kTransB>(g, bx, by, bz);
  } else {
    const int bx = static_cast<int>((blockIdx.x + blockIdx.y + blockIdx.z) % gridDim.x);
    gemm_x6_tile<kTransB>(g, bx, blockIdx.y, blockIdx.z);
  }
}

}  // namespace

// Dynamic LDS of a CU-limited split-bf16 product: 48 KB static + this exceeds half of the
// CU's 160 KB, and leaves the 66.5 KB of a 64-wide fp32 tile.
constexpr size_t kOneWgPerCuLds = 33 * 1024;

gptq_status gemm_f32(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0 || g.batch2 <= 0) return GPTQ_OK;
  const int nz = g.batch * g.batch2;
  // 128-wide tiles when they give every CU one workgroup (the split-bf16 kernel, 2.7x the
  // fp32 rate, even where triangular operands leave some tiles with less work) or, for the
  // fp32 kernel, two (one for a plain product); else 64-wide fp32 tiles
  const int64_t tiles128 = static_cast<int64_t>((g.N + 127) / 128) * ((g.M + 127) / 128) * nz;
  // the split-bf16 kernel loads unmasked 16-byte vectors
  const auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool vec4 = g.K % 4 == 0 && g.N % 4 == 0 && g.lda % 4 == 0 && g.ldb % 4 == 0 && g.sA % 4 == 0 &&
                    g.sB % 4 == 0 && g.sA2 % 4 == 0 && g.sB2 % 4 == 0 && al16(g.A) && al16(g.B);
  const bool big = vec4 ? tiles128 >= 256 : (tiles128 >= 512 || (g.flags == 0 && tiles128 >= 256));
  const int T = big ? 128 : 64;
  const dim3 grid((g.N + T - 1) / T, (g.M + T - 1) / T, nz);
  if (g.role == 1) {   // lazy trailing updates: never transposed
    if (g.transB) return GPTQ_ERR_UNSUPPORTED;
    // split-bf16 from half a chip of 128-wide tiles: their K grows with N, and the fp32
    // kernel's 64-wide tiles take the long-K mid levels at under half the rate (d_in 14336:
    // N = K = 896 at 96 us; quantize -0.12 ms)
    if (vec4 && tiles128 >= 128)
      GPTQ_LAUNCH((gemm_x6_kernel<false, 1>), dim3((g.N + 127) / 128, (g.M + 127) / 128, nz), dim3(256), 0, stream, g);
    else if (big) GPTQ_LAUNCH((gemm_f32_kernel<false, 128, false, 1>), grid, dim3(256), 0, stream, g);
    else if (vec4) GPTQ_LAUNCH((gemm_f32_kernel<false, 64, true, 1>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 64, false, 1>), grid, dim3(256), 0, stream, g);
    return GPTQ_OK;
  }
  if (big && vec4 && g.max_cus > 0 && (!(g.flags & kLowerOut) || g.M == g.N)) {
    // At most max_cus workgroups, each with enough (unused) dynamic LDS that no second one
    // fits its CU: the product occupies max_cus CUs, one workgroup each, and leaves every
    // other CU free and every occupied CU room for a 64-wide fp32 tile.
    const int64_t tm = (g.M + 127) / 128, tn = (g.N + 127) / 128;
    const int64_t total = ((g.flags & kLowerOut) ? tm * (tm + 1) / 2 : tm * tn) * nz;
    const int wgs = static_cast<int>(std::min<int64_t>(total, g.max_cus));
    if (g.transB) GPTQ_LAUNCH((gemm_x6_kernel<true, 0, true>), dim3(wgs), dim3(256), kOneWgPerCuLds, stream, g);
    else GPTQ_LAUNCH((gemm_x6_kernel<false, 0, true>), dim3(wgs), dim3(256), kOneWgPerCuLds, stream, g);
  } else if (big && vec4) {
    if (g.transB) GPTQ_LAUNCH((gemm_x6_kernel<true, 0>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_x6_kernel<false, 0>), grid, dim3(256), 0, stream, g);
  } else if (big) {
    if (g.transB) GPTQ_LAUNCH((gemm_f32_kernel<true, 128, false, 0>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 128, false, 0>), grid, dim3(256), 0, stream, g);
  } else if (vec4) {
    if (g.transB) GPTQ_LAUNCH((gemm_f32_kernel<true, 64, true, 0>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 64, true, 0>), grid, dim3(256), 0, stream, g);
  } else {
    if (g.transB) GPTQ_LAUNCH((gemm_f32_kernel<true, 64, false, 0>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 64, false, 0>), grid, dim3(256), 0, stream, g);
  }
  return GPTQ_OK;
}

}  // namespace gptq
