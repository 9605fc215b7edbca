// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32):
//   C = alpha * op(A) * op(B) + beta * C,   A [M, K], op(B) = B [K, N] or B^T (B [N, K]),
// batched over blockIdx.z (two nested batch strides).
//
// Used for the blocked Cholesky (panel solve as a product with the inverted diagonal
// block, trailing symmetric update), the triangular inverse, and GPTQ's lazy batch update
// W[:, later] -= Err @ U[block, later] ("Same Ruler, Smarter Placement: GPTQ", 1.8).
// Products and sums are fp32, as the quantizer's arithmetic requires; the operands are
// never rounded to a 16-bit type.
//
// Tile 128 x 128 x 32 (or 64 x 64 x 32 when the grid would be small), 256 threads = 4
// waves, each owning a quarter of the tile as 32 x 32 MFMA blocks.
// Operands are staged k-major in LDS so that lanes 0..31 of an MFMA operand read 32
// consecutive floats.  Triangular operands shrink the K range per tile; a lower-only
// output skips tiles above the diagonal.
#include "common.h"

namespace gptq {
namespace {

// TT = output tile edge (128 or 64); each of the 4 waves owns a (TT/2) x (TT/2) quarter as
// MB x MB blocks of 32 x 32.  The 64-wide tile takes 64 k per stage: with one workgroup per
// CU its stage is otherwise too short to cover the latency of the next stage's loads.
template <bool kTransB, int TT>
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

  float4 ra[RQ], rb[RQ];
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
  auto store_rows = [&](auto s, const float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int row = lr + RS * q;
      const int k = 4 * lc;
      s[k + 0][row] = r[q].x;
      s[k + 1][row] = r[q].y;
      s[k + 2][row] = r[q].z;
      s[k + 3][row] = r[q].w;
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
  auto store_kmajor = [&](float (*s)[GPB], const float4* r) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int k = tid / NV + KS * q;
      *reinterpret_cast<float4*>(&s[k][4 * (tid % NV)]) = r[q];
    }
  };
  auto load_b = [&](int k0) {
    if constexpr (kTransB) load_rows(B, g.ldb, n0, g.N, k0, rb);
    else load_kmajor(k0, rb);
  };
  auto store_b = [&](float (*s)[GPB]) {
    if constexpr (kTransB) store_rows(s, rb);
    else store_kmajor(s, rb);
  };

  f32x16 acc[MB][MB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int nk = ke > kb ? (ke - kb + GK - 1) / GK : 0;
  if (nk > 0) {
    load_rows(A, g.lda, m0, g.M, kb, ra);
    load_b(kb);
    store_rows(sA[0], ra);
    store_b(sB[0]);
  }
  __syncthreads();
  const int l32 = lane & 31, kh = lane >> 5;
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nk;
    if (more) {
      load_rows(A, g.lda, m0, g.M, kb + (s + 1) * GK, ra);
      load_b(kb + (s + 1) * GK);
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
    if (more) {
      store_rows(sA[buf ^ 1], ra);
      store_b(sB[buf ^ 1]);
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  // With beta != 0 the 16 old values of a block are all loaded before any of its stores:
  // element by element, every load would have to wait for the previous store (the
  // compiler cannot tell that they never overlap).
  const bool has_beta = g.beta != 0.0f;
#pragma unroll
  for (int bm = 0; bm < MB; ++bm)
#pragma unroll
    for (int bn = 0; bn < MB; ++bn) {
      const int n = n0 + (GT / 2) * wn + 32 * bn + l32;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (GT / 2) * wm + 32 * bm + 8 * (r >> 2) + 4 * kh + (r & 3);
        old[r] = (has_beta && m < g.M && n < g.N) ? C[static_cast<int64_t>(m) * g.ldc + n] : 0.0f;
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

}  // namespace

gptq_status gemm_f32(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0 || g.batch2 <= 0) return GPTQ_OK;
  const int nz = g.batch * g.batch2;
  // 128-wide tiles when they give every CU two workgroups, or one for a plain product
  // (triangular operands leave some tiles with far less work, a lower-only output skips
  // half of them); else 64-wide
  const int64_t tiles128 = static_cast<int64_t>((g.N + 127) / 128) * ((g.M + 127) / 128) * nz;
  const bool big = tiles128 >= 512 || (g.flags == 0 && tiles128 >= 256);
  const int T = big ? 128 : 64;
  const dim3 grid((g.N + T - 1) / T, (g.M + T - 1) / T, nz);
  if (big) {
    if (g.transB) GPTQ_LAUNCH((gemm_f32_kernel<true, 128>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 128>), grid, dim3(256), 0, stream, g);
  } else {
    if (g.transB) GPTQ_LAUNCH((gemm_f32_kernel<true, 64>), grid, dim3(256), 0, stream, g);
    else GPTQ_LAUNCH((gemm_f32_kernel<false, 64>), grid, dim3(256), 0, stream, g);
  }
  return GPTQ_OK;
}

}  // namespace gptq
