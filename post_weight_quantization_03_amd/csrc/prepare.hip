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
// Cholesky: right-looking with 128-column panels.  A single workgroup factors the
// diagonal block in LDS and inverts it; the panel below is the product of the panel with
// that inverse (transposed), and the trailing lower tiles take a symmetric rank-128
// update — both on the fp32 matrix cores.  The inverse L^-1 is assembled bottom-up:
// diagonal blocks come from the panel kernel, off-diagonal blocks from
// inv([[L11, 0], [L21, L22]]) = [[L11^-1, 0], [-L22^-1 L21 L11^-1, L22^-1]] over a
// recursive split.  A non-positive or non-finite pivot sets a device flag that the host
// reads back (GPTQ_ERR_NOT_SPD).
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int NB = 128;   // panel width (must equal the GEMM tile)
constexpr int LP = NB + 1;

// key[c] = diag_key[c], or 1 for a dead input; dead[c] = (diag_key[c] == 0).
__global__ __launch_bounds__(256) void keys_kernel(const double* __restrict__ diag_key, int d_in,
                                                   double* __restrict__ key, uint8_t* __restrict__ dead) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d_in) return;
  const int64_t o = static_cast<int64_t>(e) * d_in + c;
  const double v = diag_key[o];
  key[o] = (v == 0.0) ? 1.0 : v;
  dead[o] = (v == 0.0) ? 1 : 0;
}

// perm[rank(c)] = c, rank(c) = #{j: key_j > key_c} + #{j < c: key_j == key_c}.
__global__ __launch_bounds__(256) void actorder_rank_kernel(const double* __restrict__ key, int d_in,
                                                            int act_order, int32_t* __restrict__ perm) {
  __shared__ double sk[256];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  const double* k = key + static_cast<int64_t>(e) * d_in;
  if (!act_order) {
    if (c < d_in) perm[static_cast<int64_t>(e) * d_in + c] = c;
    return;
  }
  const double kc = (c < d_in) ? k[c] : 0.0;
  int rank = 0;
  for (int j0 = 0; j0 < d_in; j0 += 256) {
    __syncthreads();
    sk[threadIdx.x] = (j0 + threadIdx.x < d_in) ? k[j0 + threadIdx.x] : 0.0;
    __syncthreads();
    const int jn = min(256, d_in - j0);
    for (int j = 0; j < jn; ++j) {
      const double kj = sk[j];
      rank += (kj > kc) || (kj == kc && j0 + j < c);
    }
  }
  if (c < d_in) perm[static_cast<int64_t>(e) * d_in + rank] = c;
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

// Factor the diagonal block k of A (lower part) in LDS: writes L_kk into Lbuf and
// L_kk^-1 into Linv (both full 128x128 blocks, zeros above the diagonal).
__global__ __launch_bounds__(256) void potrf_block_kernel(const float* __restrict__ A, float* __restrict__ Lbuf,
                                                          int64_t bsl, float* __restrict__ Linv, int d_in,
                                                          int k0, int* __restrict__ flag) {
  __shared__ float sa[NB][LP];
  __shared__ float sx[NB][LP];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const float* Ae = A + static_cast<int64_t>(e) * d_in * d_in;
  for (int i = tid; i < NB * NB; i += 256) {
    const int r = i / NB, c = i % NB;
    sa[r][c] = (c <= r) ? Ae[static_cast<int64_t>(k0 + r) * d_in + k0 + c] : 0.0f;
  }
  __syncthreads();
  // Right-looking elimination on unscaled columns: at step j, a_ic -= a_ij a_cj / a_jj for
  // j < c <= i.  Afterwards l_ij = a_ij / sqrt(a_jj).
  bool bad = false;
  for (int j = 0; j < NB; ++j) {
    const float piv = sa[j][j];
    if (!(piv > 0.0f) || !isfinite(piv)) bad = true;
    const float rp = 1.0f / piv;
    const int m = NB - 1 - j;                 // trailing size
    const int cnt = m * (m + 1) / 2;
    for (int t = tid; t < cnt; t += 256) {
      // t -> (i, c) with j < c <= i, enumerated row by row of the trailing triangle
      int ii = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
      while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
      while (ii * (ii + 1) / 2 > t) --ii;
      const int cc = t - ii * (ii + 1) / 2;
      const int i = j + 1 + ii, c = j + 1 + cc;
      sa[i][c] = fmaf(-sa[i][j] * rp, sa[c][j], sa[i][c]);
    }
    __syncthreads();
  }
  if (bad && tid == 0) flag[e] = 1;
  // scale columns: l_ij = a_ij / sqrt(a_jj); the diagonal becomes sqrt(a_jj)
  for (int i = tid; i < NB * NB; i += 256) {
    const int r = i / NB, c = i % NB;
    if (c < r) sa[r][c] = sa[r][c] / sqrtf(sa[c][c]);
  }
  __syncthreads();
  for (int r = tid; r < NB; r += 256) sa[r][r] = sqrtf(sa[r][r]);
  __syncthreads();
  // X = L^-1 by elimination on the identity: at step k every row i > k subtracts
  // (l_ik / l_kk) times the (still unscaled) row k; finally row k is divided by l_kk.
  for (int i = tid; i < NB * NB; i += 256) sx[i / NB][i % NB] = (i / NB == i % NB) ? 1.0f : 0.0f;
  __syncthreads();
  for (int k = 0; k < NB - 1; ++k) {
    const float rk = 1.0f / sa[k][k];
    const int rows = NB - 1 - k, cols = k + 1;
    for (int t = tid; t < rows * cols; t += 256) {
      const int i = k + 1 + t / cols, c = t % cols;
      sx[i][c] = fmaf(-sa[i][k] * rk, sx[k][c], sx[i][c]);
    }
    __syncthreads();
  }
  for (int i = tid; i < NB * NB; i += 256) {
    const int r = i / NB, c = i % NB;
    if (c <= r) sx[r][c] = sx[r][c] / sa[r][r];
  }
  __syncthreads();
  float* Le = Lbuf + static_cast<int64_t>(e) * bsl;
  float* Xe = Linv + static_cast<int64_t>(e) * d_in * d_in;
  for (int i = tid; i < NB * NB; i += 256) {
    const int r = i / NB, c = i % NB;
    Le[static_cast<int64_t>(k0 + r) * d_in + k0 + c] = (c <= r) ? sa[r][c] : 0.0f;
    Xe[static_cast<int64_t>(k0 + r) * d_in + k0 + c] = (c <= r) ? sx[r][c] : 0.0f;
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
  w.lambda = cv.take<double>(batch);
  w.flag = cv.take<int>(batch);
  w.A = cv.take<float>(batch * dd);
  w.Linv = cv.take<float>(batch * dd);
  w.T = cv.take<float>(batch * dd / 4 + static_cast<size_t>(NB) * d_in);
  w.bytes = cv.used;
  return w;
}

// Off-diagonal blocks of L^-1 for the block range [b0, b1) (block = NB columns).
gptq_status tri_inverse(int b0, int b1, int batch, int d_in, const float* L, int64_t bsl, float* Linv,
                        float* T, hipStream_t stream) {
  if (b1 - b0 <= 1) return GPTQ_OK;
  const int bm = b0 + (b1 - b0) / 2;
  gptq_status st = tri_inverse(b0, bm, batch, d_in, L, bsl, Linv, T, stream);
  if (st != GPTQ_OK) return st;
  st = tri_inverse(bm, b1, batch, d_in, L, bsl, Linv, T, stream);
  if (st != GPTQ_OK) return st;
  const int o1 = b0 * NB, o2 = bm * NB, h1 = (bm - b0) * NB, h2 = (b1 - bm) * NB;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  // T = L21 * L11^-1     (L11^-1 lower: K starts at the output column)
  GemmArgs g{};
  g.M = h2; g.N = h1; g.K = h1;
  g.A = L + static_cast<int64_t>(o2) * d_in + o1; g.lda = d_in; g.sA = bsl;
  g.B = Linv + static_cast<int64_t>(o1) * d_in + o1; g.ldb = d_in; g.sB = dd;
  g.C = T; g.ldc = h1; g.sC = static_cast<int64_t>(h2) * h1;
  g.alpha = 1.0f; g.beta = 0.0f; g.transB = 0; g.flags = kBLower; g.batch = batch;
  st = gemm_f32(g, stream);
  if (st != GPTQ_OK) return st;
  // Linv21 = -L22^-1 * T   (L22^-1 lower: K ends at the output row)
  GemmArgs h{};
  h.M = h2; h.N = h1; h.K = h2;
  h.A = Linv + static_cast<int64_t>(o2) * d_in + o2; h.lda = d_in; h.sA = dd;
  h.B = T; h.ldb = h1; h.sB = static_cast<int64_t>(h2) * h1;
  h.C = Linv + static_cast<int64_t>(o2) * d_in + o1; h.ldc = d_in; h.sC = dd;
  h.alpha = -1.0f; h.beta = 0.0f; h.transB = 0; h.flags = kALower; h.batch = batch;
  return gemm_f32(h, stream);
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
  GPTQ_LAUNCH(keys_kernel, dim3(cb, batch), blk, 0, stream, diag_key, d_in, w.key, dead);
  GPTQ_LAUNCH(actorder_rank_kernel, dim3(cb, batch), blk, 0, stream, w.key, d_in, p.act_order, perm);
  GPTQ_LAUNCH(damping_kernel, dim3(batch), blk, 0, stream, w.key, d_in, static_cast<double>(p.damp),
              w.lambda, w.flag);
  GPTQ_LAUNCH(gather_reversed_kernel, dim3(cb, d_in, batch), blk, 0, stream, H, bsh, perm, w.key,
              w.lambda, d_in, w.A);
  // L is built in the U buffer (same shape), then replaced by U at the end.
  float* L = U;
  const int nblk = d_in / NB;
  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * NB;
    GPTQ_LAUNCH(potrf_block_kernel, dim3(batch), blk, 0, stream, w.A, L, bsu, w.Linv, d_in, k0, w.flag);
    const int rest = d_in - k0 - NB;
    if (rest == 0) break;
    // panel: L[k0+NB:, k-block] = A[k0+NB:, k-block] * (L_kk^-1)^T
    GemmArgs g{};
    g.M = rest; g.N = NB; g.K = NB;
    g.A = w.A + static_cast<int64_t>(k0 + NB) * d_in + k0; g.lda = d_in; g.sA = dd;
    g.B = w.Linv + static_cast<int64_t>(k0) * d_in + k0; g.ldb = d_in; g.sB = dd;
    g.C = L + static_cast<int64_t>(k0 + NB) * d_in + k0; g.ldc = d_in; g.sC = bsu;
    g.alpha = 1.0f; g.beta = 0.0f; g.transB = 1; g.flags = kBtLower; g.batch = batch;
    gptq_status st = gemm_f32(g, stream);
    if (st != GPTQ_OK) return st;
    // trailing: A[k0+NB:, k0+NB:] -= P P^T (lower tiles)
    GemmArgs h{};
    h.M = rest; h.N = rest; h.K = NB;
    h.A = L + static_cast<int64_t>(k0 + NB) * d_in + k0; h.lda = d_in; h.sA = bsu;
    h.B = h.A; h.ldb = d_in; h.sB = bsu;
    h.C = w.A + static_cast<int64_t>(k0 + NB) * d_in + k0 + NB; h.ldc = d_in; h.sC = dd;
    h.alpha = -1.0f; h.beta = 1.0f; h.transB = 1; h.flags = kLowerOut; h.batch = batch;
    st = gemm_f32(h, stream);
    if (st != GPTQ_OK) return st;
  }
  gptq_status st = tri_inverse(0, nblk, batch, d_in, L, bsu, w.Linv, w.T, stream);
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
