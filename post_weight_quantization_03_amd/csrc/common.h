// Internal helpers shared by the HIP translation units of libgptq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "gptq.h"

#define GPTQ_HIP_TRY(expr)                         \
  do {                                             \
    if ((expr) != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

// A kernel launch: enqueue, then report a failed launch as GPTQ_ERR_HIP.
#define GPTQ_LAUNCH(kernel, grid, block, lds, stream, ...)                    \
  do {                                                                       \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);       \
    if (hipGetLastError() != hipSuccess) return GPTQ_ERR_HIP;                \
  } while (0)

namespace gptq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;  // columns per lazy batch

// f(std::integral_constant<int, I>) for every I of the sequence, in order (a loop whose
// index is a compile-time constant in its body)
template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// store(i, load(i)) for i = t, t + NT, t + 2 NT, ... < n, the loads of up to B consecutive
// iterations issued before their stores: a plain loop waits for each global load before
// its LDS store, one full load latency per iteration.
template <int NT, int B = 8, typename Load, typename Store>
__device__ __forceinline__ void batched_copy(int t, int n, Load&& load, Store&& store) {
  for (int base = t; base < n; base += NT * B) {
    decltype(load(0)) v[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (base + NT * u < n) v[u] = load(base + NT * u);
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (base + NT * u < n) store(base + NT * u, v[u]);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }

// 16-bit storage types are carried as raw bits; the tag selects the decoding.
struct BF16 { uint16_t bits; };
struct F16 { uint16_t bits; };
template <>
__device__ __forceinline__ float load_as_f32<BF16>(const BF16* p) { return bf16_to_f32(p->bits); }
template <>
__device__ __forceinline__ float load_as_f32<F16>(const F16* p) { return f16_to_f32(p->bits); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves consecutive 256-byte aligned regions out of one workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

}  // namespace gptq

// Internal entry points of the translation units (host side).
namespace gptq {
// offsets (device, batch + 1 entries) or null: see problem_rows in hessian.hip.
gptq_status hessian_enqueue(int batch, int d_in, int64_t n_tokens, gptq_dtype x_dtype, const void* X,
                            int64_t ldx, int64_t bsx, const int64_t* offsets, int64_t total_rows, float* H,
                            int64_t bsh, double* diag_key, int64_t* n_seen, void* ws, size_t ws_bytes,
                            hipStream_t stream);
size_t hessian_workspace(int batch, int d_in, int64_t n_tokens);

gptq_status prepare_enqueue(int batch, int d_in, const float* H, int64_t bsh, const double* diag_key,
                            const gptq_params& p, float* U, int64_t bsu, int32_t* perm, uint8_t* dead,
                            void* ws, size_t ws_bytes, hipStream_t stream, int* not_spd);
size_t prepare_workspace(int batch, int d_in);

gptq_status quantize_enqueue(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W,
                             int64_t ldw, int64_t bsw, const float* U, int64_t bsu, const int32_t* perm,
                             const uint8_t* dead, const gptq_params& p, uint8_t* codes, float* scales,
                             uint8_t* zeros, int32_t* g_idx, void* ws, size_t ws_bytes,
                             hipStream_t stream);
size_t quantize_workspace(int batch, int d_out, int d_in, const gptq_params& p);
// The same call with the library's fixed device scratch array instead of a workspace
// (GPTQ_NOALLOC_SCRATCH_BYTES); GPTQ_ERR_TOO_LARGE when the problem needs more.
constexpr size_t kNoAllocScratchBytes = GPTQ_NOALLOC_SCRATCH_BYTES;
gptq_status quantize_noalloc_enqueue(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W,
                                     int64_t ldw, int64_t bsw, const float* U, int64_t bsu, const int32_t* perm,
                                     const uint8_t* dead, const gptq_params& p, uint8_t* codes, float* scales,
                                     uint8_t* zeros, int32_t* g_idx, hipStream_t stream);

size_t serve_workspace(int m, int d_out, int d_in, int n_groups);
gptq_status repack_enqueue(int batch, int d_out, int d_in, int n_groups, const int32_t* qweight,
                           const int32_t* g_idx, int32_t* qweight_s, int32_t* order, int* flag,
                           hipStream_t stream);
gptq_status serve_enqueue(int m, int d_out, int d_in, int n_groups, gptq_dtype x_dtype, const void* X, int64_t ldx,
                          const int32_t* order, const int32_t* qweight, const int32_t* qzeros,
                          const uint16_t* scales, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t stream);

gptq_status pack_enqueue(int batch, int d_out, int d_in, int n_groups, const uint8_t* codes,
                         const float* scales, const uint8_t* zeros, int32_t* qweight, int32_t* qzeros,
                         uint16_t* scales_f16, hipStream_t stream);

// Launch timing (gptq_timing_enable / gptq_timing_read): returns the event pair to record
// around the next launch of the given class, or nulls when timing is off.
constexpr int kTimedKinds = 5;
void timing_pair(gptq_timed_kernel kind, hipEvent_t* start, hipEvent_t* stop);

// Two more streams per device for work that can overlap the caller's stream, with events
// that fork work onto them and join it back.  Created on first use, kept for the life of
// the process.  Callers hold side_mutex() while they enqueue on them.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t join2 = nullptr;   // a second join event, for two side-stream stages in flight
  hipStream_t s2 = nullptr;     // the second side stream
  hipEvent_t fork2 = nullptr, join3 = nullptr;
};
std::mutex& side_mutex();
gptq_status side_stream(SideStream** out);   // of the current device

// fp32-accurate matrix-core GEMM: C = alpha * op(A) op(B) + beta * C (row-major, batched by
// blockIdx.z); large products as split-bf16 products, small ones on the fp32 instruction.
struct GemmArgs {
  int M, N, K;
  const float* A; int64_t lda, sA;   // A [M, K]
  const float* B; int64_t ldb, sB;   // B [K, N], or [N, K] when transB
  float* C; int64_t ldc, sC;         // C [M, N]
  float alpha, beta;
  int transB;
  int flags;                         // GemmFlags
  int batch;
  // optional inner batch: product z = zo * batch2 + zi sits at zo * s + zi * s2
  int batch2 = 1;
  int64_t sA2 = 0, sB2 = 0, sC2 = 0;
  int role = 0;                      // 1: a lazy trailing update of the quantizer (see gemm.hip)
  // > 0: a product that runs next to a latency-bound chain on another stream; it is given
  // at most this many CUs, one workgroup each (see gemm.hip), so that the chain's kernels
  // find free CUs
  int max_cus = 0;
};
enum GemmFlags {
  kLowerOut = 1,   // C square: only tiles on or below the diagonal are computed
  kALower = 2,     // A lower triangular: K range of a row tile ends at its last row
  kBLower = 4,     // op(B) = B lower triangular (B[k][n] = 0 for k < n): K starts at n0
  kBtLower = 8,    // op(B) = B^T with B lower (B^T[k][n] = 0 for k > n): K ends at n0 + TN
};
gptq_status gemm_f32(const GemmArgs& g, hipStream_t stream);
}  // namespace gptq
