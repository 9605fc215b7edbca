// From H to U, the upper factor of the damped, permuted inverse Hessian, on gfx950.
//
// Steps ("GPTQ Architecture, in depth", "The algorithm in code"; "Same Ruler, Smarter
// Placement: GPTQ", 1.6 dampening, 1.7 the Cholesky trick, 1.9 activation ordering):
//   1. dead inputs (zero fp64 diagonal) count as diagonal 1;
//   2. ActOrder: perm sorts the fp64 diagonal in descending order, ties by index
//      (computed as exact ranks, so the order is the same as a stable sort);
//   3. lambda = damp * mean(diagonal), fp64;
//   4. U with H_p^-1 = U^T U.  Route: A = J H_p J (index-reversed, gathered in one pass
//      with the permutation), L = chol(A) lower, U = J L^-1 J.  Then H_p = (J L J)(J L J)^T
//      with J L J upper, so H_p^-1 = (J L^-1 J)^T (J L^-1 J) and U is the unique
//      positive-diagonal upper factor the pages obtain with chol / cholesky_inverse / chol,
//      at 2/3 d^3 instead of 4/3 d^3 flops.
//
// Cholesky and inverse together by recursive halving (chol_inv below): one workgroup
// factors and inverts each 128-column diagonal block in registers/LDS; everything else is
// fp32 matrix-core products.  A non-positive or non-finite pivot sets a device flag that
// the host reads back (GPTQ_ERR_NOT_SPD).
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int NB = 128;   // panel width (must equal the GEMM tile)
constexpr int LP = NB + 1;

// key[c] = diag_key[c], or 1 for a dead input; dead[c] = (diag_key[c] == 0).
// Also clears the rank counters of actorder_rank_kernel.
__global__ __launch_bounds__(256) void keys_kernel(const double* __restrict__ diag_key, int d_in,
                                                   double* __restrict__ key, uint8_t* __restrict__ dead,
                                                   int32_t* __restrict__ rank) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d_in) return;
  const int64_t o = static_cast<int64_t>(e) * d_in + c;
  const double v = diag_key[o];
  key[o] = (v == 0.0) ? 1.0 : v;
  dead[o] = (v == 0.0) ? 1 : 0;
  rank[o] = 0;
}

// rank(c) = #{j: key_j > key_c} + #{j < c: key_j == key_c}, the position of c in a stable
// descending sort.  Block (x, y): 256 candidates c against a slice of RANK_SLICE keys j;
// the integer partial counts are summed with atomics (order-independent, exact).
constexpr int RANK_SLICE = 512;
__global__ __launch_bounds__(256) void actorder_rank_kernel(const double* __restrict__ key, int d_in,
                                                            int32_t* __restrict__ rank) {
  __shared__ double sk[RANK_SLICE];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int j0 = blockIdx.y * RANK_SLICE;
  const int e = blockIdx.z;
  const double* k = key + static_cast<int64_t>(e) * d_in;
  for (int i = threadIdx.x; i < RANK_SLICE; i += 256) sk[i] = (j0 + i < d_in) ? k[j0 + i] : 0.0;
  __syncthreads();
  if (c >= d_in) return;
  const double kc = k[c];
  const int jn = min(RANK_SLICE, d_in - j0);
  int cnt = 0;
  for (int j = 0; j < jn; ++j) {
    const double kj = sk[j];
    cnt += (kj > kc) || (kj == kc && j0 + j < c);
  }
  if (cnt) atomicAdd(rank + static_cast<int64_t>(e) * d_in + c, cnt);
}

// perm[rank(c)] = c (ActOrder), or the identity.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ rank, int d_in,
                                                           int act_order, int32_t* __restrict__ perm) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d_in) return;
  const int64_t o = static_cast<int64_t>(e) * d_in;
  if (!act_order) {
    perm[o + c] = c;
    return;
  }
  const int r = min(max(rank[o + c], 0), d_in - 1);
  perm[o + r] = c;
}

// lambda[e] = damp * mean(key[e]) (fixed-order tree sum in fp64).
__global__ __launch_bounds__(256) void damping_kernel(const double* __restrict__ key, int d_in,
                                                      double damp, double* __restrict__ lambda,
                                                      int* __restrict__ flag) {
  __shared__ double red[256];
  const int e = blockIdx.x;
  const double* k = key + static_cast<int64_t>(e) * d_in;
  double s = 0.0;
  for (int c = threadIdx.x; c < d_in; c += 256) s += k[c];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lambda[e] = damp * red[0] / static_cast<double>(d_in);
    flag[e] = 0;
  }
}

// A[r][c] = H[p(r)][p(c)] with p(r) = perm[d-1-r]; diagonal key[p(r)] + lambda.
__global__ __launch_bounds__(256) void gather_reversed_kernel(const float* __restrict__ H, int64_t bsh,
                                                              const int32_t* __restrict__ perm,
                                                              const double* __restrict__ key,
                                                              const double* __restrict__ lambda, int d_in,
                                                              float* __restrict__ A) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  const int e = blockIdx.z;
  if (c >= d_in) return;
  const int32_t* pe = perm + static_cast<int64_t>(e) * d_in;
  // indices are clamped so that a malformed permutation can never address outside H
  const int pr = min(max(pe[d_in - 1 - r], 0), d_in - 1);
  const int pc = min(max(pe[d_in - 1 - c], 0), d_in - 1);
  float v;
  if (r == c) {
    v = static_cast<float>(key[static_cast<int64_t>(e) * d_in + pr] + lambda[e]);
  } else {
    v = H[static_cast<int64_t>(e) * bsh + static_cast<int64_t>(pr) * d_in + pc];
  }
  A[(static_cast<int64_t>(e) * d_in + r) * d_in + c] = v;
}

// Factor the diagonal block k of A (lower part): writes L_kk into Lbuf and L_kk^-1 into
// Linv (both full 128x128 blocks, zeros above the diagonal).
//
// Each of the 256 threads keeps an 8x8 sub-block of the 128x128 block in registers
// (thread t: block row t/16, block column t%16; a wave covers 32 consecutive rows).
// Cholesky, right-looking on unscaled columns: at step j every element with
// j < c, j < i takes a_ic -= a_ij a_cj / a_jj; column j (zeros at rows <= j) and the pivot
// a_jj are broadcast through LDS by the threads that own them, so each step costs one
// barrier.  Afterwards l_ij = a_ij / sqrt(a_jj).  The inverse X = L^-1 is then formed the
// same way, row by row: row k of X is final once divided by l_kk, and every row i > k
// subtracts l_ik times it.  Loops over columns are unrolled by 8 so that register
// indices stay compile-time constants.
__global__ __launch_bounds__(256) void potrf_block_kernel(const float* __restrict__ A, float* __restrict__ Lbuf,
                                                          int64_t bsl, float* __restrict__ Linv, int d_in,
                                                          int k0, int* __restrict__ flag) {
  __shared__ float sL[NB][LP];
  __shared__ float colbuf[2][NB];
  __shared__ float piv[NB];
  const int e = blockIdx.x;
  const int t = threadIdx.x;
  const int br = t >> 4, bc = t & 15;
  const int r0 = 8 * br, c0 = 8 * bc;
  const int wave_last_row = 32 * (t >> 6) + 31;
  const float* Ae = A + static_cast<int64_t>(e) * d_in * d_in + static_cast<int64_t>(k0) * d_in + k0;

  float a[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float4* src = reinterpret_cast<const float4*>(Ae + static_cast<int64_t>(r0 + r) * d_in + c0);
    const float4 u = src[0], v = src[1];
    a[r][0] = u.x; a[r][1] = u.y; a[r][2] = u.z; a[r][3] = u.w;
    a[r][4] = v.x; a[r][5] = v.y; a[r][6] = v.z; a[r][7] = v.w;
  }
  // publish column 0
  if (bc == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) colbuf[0][r0 + r] = (r0 + r > 0) ? a[r][0] : 0.0f;
    if (br == 0) piv[0] = a[0][0];
  }
  __syncthreads();
  for (int jb = 0; jb < NB / 8; ++jb) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * jb + jj;
      const int buf = jj & 1;
      if (wave_last_row > j) {
        const float rp = 1.0f / piv[j];
        float ci[8], cc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) ci[r] = colbuf[buf][r0 + r] * rp;
#pragma unroll
        for (int c = 0; c < 8; ++c) cc[c] = colbuf[buf][c0 + c];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) a[r][c] = fmaf(-ci[r], cc[c], a[r][c]);
      }
      // publish column j + 1 (its owners are block column (j+1)/8, local column (jj+1)%8)
      const int jn = j + 1;
      if (jn < NB && bc == (jn >> 3)) {
#pragma unroll
        for (int r = 0; r < 8; ++r) colbuf[buf ^ 1][r0 + r] = (r0 + r > jn) ? a[r][(jj + 1) & 7] : 0.0f;
        if (br == bc) piv[jn] = a[(jj + 1) & 7][(jj + 1) & 7];
      }
      __syncthreads();
    }
  }
  // every pivot must be positive and finite
  if (t == 0) {
    bool bad = false;
    for (int j = 0; j < NB; ++j) bad |= !(piv[j] > 0.0f) || !isfinite(piv[j]);
    if (bad) flag[e] = 1;
  }
  // scale: l_ic = a_ic / sqrt(a_cc), l_cc = sqrt(a_cc)
  float sq[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sq[c] = sqrtf(piv[c0 + c]);
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i = r0 + r, cg = c0 + c;
      const float v = (i > cg) ? a[r][c] / sq[c] : (i == cg ? sq[c] : 0.0f);
      a[r][c] = v;
      sL[i][cg] = v;
    }
  float* Le = Lbuf + static_cast<int64_t>(e) * bsl + static_cast<int64_t>(k0) * d_in + k0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float4* dst = reinterpret_cast<float4*>(Le + static_cast<int64_t>(r0 + r) * d_in + c0);
    dst[0] = make_float4(a[r][0], a[r][1], a[r][2], a[r][3]);
    dst[1] = make_float4(a[r][4], a[r][5], a[r][6], a[r][7]);
  }
  // X = L^-1: start from the identity; row 0 of X is e_0 / l_00.
  float x[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) x[r][c] = (r0 + r == c0 + c) ? 1.0f : 0.0f;
  __syncthreads();   // sL complete
  if (br == 0) {
    const float inv0 = 1.0f / sL[0][0];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      x[0][c] *= inv0;
      colbuf[0][c0 + c] = x[0][c];
    }
  }
  __syncthreads();
  for (int kb = 0; kb < NB / 8; ++kb) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = 8 * kb + kk;
      const int buf = kk & 1;
      if (wave_last_row > k) {
        float m[8], xr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) m[r] = (r0 + r > k) ? sL[r0 + r][k] : 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) xr[c] = colbuf[buf][c0 + c];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) x[r][c] = fmaf(-m[r], xr[c], x[r][c]);
      }
      // row k + 1 is now final up to its diagonal scale: its owners scale and publish it
      const int kn = k + 1;
      if (kn < NB && br == (kn >> 3)) {
        const float inv = 1.0f / sL[kn][kn];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          x[(kk + 1) & 7][c] *= inv;
          colbuf[buf ^ 1][c0 + c] = x[(kk + 1) & 7][c];
        }
      }
      __syncthreads();
    }
  }
  float* Xe = Linv + static_cast<int64_t>(e) * d_in * d_in + static_cast<int64_t>(k0) * d_in + k0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float4* dst = reinterpret_cast<float4*>(Xe + static_cast<int64_t>(r0 + r) * d_in + c0);
    dst[0] = make_float4(x[r][0], x[r][1], x[r][2], x[r][3]);
    dst[1] = make_float4(x[r][4], x[r][5], x[r][6], x[r][7]);
  }
}

// U[i][j] = Linv[d-1-i][d-1-j] for j >= i, 0 below the diagonal.
__global__ __launch_bounds__(256) void reverse_to_upper_kernel(const float* __restrict__ Linv, int d_in,
                                                               float* __restrict__ U, int64_t bsu) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;
  const int e = blockIdx.z;
  if (j >= d_in) return;
  float v = 0.0f;
  if (j >= i) v = Linv[(static_cast<int64_t>(e) * d_in + (d_in - 1 - i)) * d_in + (d_in - 1 - j)];
  U[static_cast<int64_t>(e) * bsu + static_cast<int64_t>(i) * d_in + j] = v;
}

struct PrepWs {
  double* key;
  int32_t* rank;
  double* lambda;
  int* flag;
  float* A;
  float* Linv;
  float* T;
  size_t bytes;
};

PrepWs carve(void* ws, int batch, int d_in) {
  Carver cv(ws);
  PrepWs w{};
  const size_t dd = static_cast<size_t>(d_in) * d_in;
  w.key = cv.take<double>(static_cast<size_t>(batch) * d_in);
  w.rank = cv.take<int32_t>(static_cast<size_t>(batch) * d_in);
  w.lambda = cv.take<double>(batch);
  w.flag = cv.take<int>(batch);
  w.A = cv.take<float>(batch * dd);
  w.Linv = cv.take<float>(batch * dd);
  w.T = cv.take<float>(batch * dd / 4 + static_cast<size_t>(NB) * d_in);
  w.bytes = cv.used;
  return w;
}

// Recursive Cholesky with the inverse, over the block range [b0, b1) of A (in place):
//   [A11  .  ]   [L11  0 ]            L11, L11^-1 = recurse(A11)
//   [A21 A22 ] = [L21 L22] [..]^T     L21 = A21 L11^-T           (product with L11^-1)
//                                     S   = A22 - L21 L21^T      (lower tiles, in place)
//                                     L22, L22^-1 = recurse(S)
//   L^-1 = [[L11^-1, 0], [-L22^-1 L21 L11^-1, L22^-1]].
// Leaves are single 128-column blocks (potrf_block_kernel).  Every product runs on the
// fp32 matrix cores with triangular operands trimming the K range; most of the flops land
// in the large products near the top of the recursion.
gptq_status chol_inv(int b0, int b1, int batch, int d_in, float* A, float* L, int64_t bsl, float* Linv, float* T,
                     int* flag, hipStream_t stream) {
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  if (b1 - b0 == 1) {
    GPTQ_LAUNCH(potrf_block_kernel, dim3(batch), dim3(256), 0, stream, A, L, bsl, Linv, d_in, b0 * NB, flag);
    return GPTQ_OK;
  }
  const int bm = b0 + (b1 - b0) / 2;
  const int o1 = b0 * NB, o2 = bm * NB, h1 = (bm - b0) * NB, h2 = (b1 - bm) * NB;
  gptq_status st = chol_inv(b0, bm, batch, d_in, A, L, bsl, Linv, T, flag, stream);
  if (st != GPTQ_OK) return st;
  GemmArgs g{};
  // L21 = A21 * (L11^-1)^T
  g.M = h2; g.N = h1; g.K = h1;
  g.A = A + static_cast<int64_t>(o2) * d_in + o1; g.lda = d_in; g.sA = dd;
  g.B = Linv + static_cast<int64_t>(o1) * d_in + o1; g.ldb = d_in; g.sB = dd;
  g.C = L + static_cast<int64_t>(o2) * d_in + o1; g.ldc = d_in; g.sC = bsl;
  g.alpha = 1.0f; g.beta = 0.0f; g.transB = 1; g.flags = kBtLower; g.batch = batch;
  if ((st = gemm_f32(g, stream)) != GPTQ_OK) return st;
  // S = A22 - L21 L21^T (lower tiles)
  g.M = h2; g.N = h2; g.K = h1;
  g.A = L + static_cast<int64_t>(o2) * d_in + o1; g.lda = d_in; g.sA = bsl;
  g.B = g.A; g.ldb = d_in; g.sB = bsl;
  g.C = A + static_cast<int64_t>(o2) * d_in + o2; g.ldc = d_in; g.sC = dd;
  g.alpha = -1.0f; g.beta = 1.0f; g.transB = 1; g.flags = kLowerOut;
  if ((st = gemm_f32(g, stream)) != GPTQ_OK) return st;
  if ((st = chol_inv(bm, b1, batch, d_in, A, L, bsl, Linv, T, flag, stream)) != GPTQ_OK) return st;
  // T = L21 * L11^-1   (L11^-1 lower: the K range of an output column starts at it)
  g.M = h2; g.N = h1; g.K = h1;
  g.A = L + static_cast<int64_t>(o2) * d_in + o1; g.lda = d_in; g.sA = bsl;
  g.B = Linv + static_cast<int64_t>(o1) * d_in + o1; g.ldb = d_in; g.sB = dd;
  g.C = T; g.ldc = h1; g.sC = static_cast<int64_t>(h2) * h1;
  g.alpha = 1.0f; g.beta = 0.0f; g.transB = 0; g.flags = kBLower;
  if ((st = gemm_f32(g, stream)) != GPTQ_OK) return st;
  // Linv21 = -L22^-1 * T   (L22^-1 lower: the K range of an output row ends at it)
  g.M = h2; g.N = h1; g.K = h2;
  g.A = Linv + static_cast<int64_t>(o2) * d_in + o2; g.lda = d_in; g.sA = dd;
  g.B = T; g.ldb = h1; g.sB = static_cast<int64_t>(h2) * h1;
  g.C = Linv + static_cast<int64_t>(o2) * d_in + o1; g.ldc = d_in; g.sC = dd;
  g.alpha = -1.0f; g.beta = 0.0f; g.transB = 0; g.flags = kALower;
  return gemm_f32(g, stream);
}

}  // namespace

size_t prepare_workspace(int batch, int d_in) {
  if (batch < 1 || d_in < NB || d_in % NB) return 0;
  return carve(nullptr, batch, d_in).bytes + 256;
}

gptq_status prepare_enqueue(int batch, int d_in, const float* H, int64_t bsh, const double* diag_key,
                            const gptq_params& p, float* U, int64_t bsu, int32_t* perm, uint8_t* dead,
                            void* ws, size_t ws_bytes, hipStream_t stream, int* not_spd) {
  PrepWs w = carve(ws, batch, d_in);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_ERR_WORKSPACE;
  const dim3 blk(256);
  const int cb = (d_in + 255) / 256;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  GPTQ_LAUNCH(keys_kernel, dim3(cb, batch), blk, 0, stream, diag_key, d_in, w.key, dead, w.rank);
  if (p.act_order) {
    GPTQ_LAUNCH(actorder_rank_kernel, dim3(cb, (d_in + RANK_SLICE - 1) / RANK_SLICE, batch), blk, 0, stream, w.key,
                d_in, w.rank);
  }
  GPTQ_LAUNCH(perm_scatter_kernel, dim3(cb, batch), blk, 0, stream, w.rank, d_in, p.act_order, perm);
  GPTQ_LAUNCH(damping_kernel, dim3(batch), blk, 0, stream, w.key, d_in, static_cast<double>(p.damp),
              w.lambda, w.flag);
  GPTQ_LAUNCH(gather_reversed_kernel, dim3(cb, d_in, batch), blk, 0, stream, H, bsh, perm, w.key,
              w.lambda, d_in, w.A);
  // L is built in the U buffer (same shape), then replaced by U at the end.
  gptq_status st = chol_inv(0, d_in / NB, batch, d_in, w.A, U, bsu, w.Linv, w.T, w.flag, stream);
  if (st != GPTQ_OK) return st;
  GPTQ_LAUNCH(reverse_to_upper_kernel, dim3(cb, d_in, batch), blk, 0, stream, w.Linv, d_in, U, bsu);

  // read back the per-problem pivot flags
  int any = 0;
  for (int e0 = 0; e0 < batch; e0 += 64) {
    int buf[64];
    const int n = std::min(64, batch - e0);
    GPTQ_HIP_TRY(hipMemcpyAsync(buf, w.flag + e0, sizeof(int) * n, hipMemcpyDeviceToHost, stream));
    GPTQ_HIP_TRY(hipStreamSynchronize(stream));
    for (int i = 0; i < n; ++i) any |= buf[i];
  }
  *not_spd = any;
  return GPTQ_OK;
}

}  // namespace gptq
