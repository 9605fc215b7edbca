// C ABI of libgptq: argument validation and dispatch to the kernel enqueuers.
// Every function declared in include/gptq.h is defined here.
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_bytes(gptq_dtype t) { return t == GPTQ_F32 ? 4 : 2; }

bool valid_dtype(int t) { return t == GPTQ_F32 || t == GPTQ_BF16 || t == GPTQ_F16; }

// Quantizer parameters accepted by prepare/quantize.
gptq_status check_params(const gptq_params* p, int d_in, bool need_grid) {
  if (p == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (!(p->damp >= 0.0f) || !std::isfinite(p->damp)) return GPTQ_ERR_INVALID_ARG;
  if (!need_grid) return GPTQ_OK;
  if (p->bits < 2 || p->bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (p->block_size != gptq::kBlock) return GPTQ_ERR_INVALID_ARG;
  const int g = p->group_size;
  if (g != -1) {
    if (g < 1 || gptq::kBlock % g != 0 || d_in % g != 0) return GPTQ_ERR_INVALID_ARG;
    if (g != 16 && g != 32 && g != 64 && g != 128) return GPTQ_ERR_UNSUPPORTED;
  }
  return GPTQ_OK;
}

// Launch timing state: recorded (start, stop) pairs per kernel class and a pool of
// reusable events.
struct TimingState {
  std::mutex mu;
  int mask = 0;   // bit k: class k is timed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recorded[gptq::kTimedKinds], pool;
};
TimingState& timing() {
  static TimingState t;
  return t;
}

}  // namespace

namespace gptq {
namespace {
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
}  // namespace

std::mutex& side_mutex() {
  static std::mutex mu;
  return mu;
}

gptq_status side_stream(SideStream** out) {
  int dev = 0;
  GPTQ_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return GPTQ_ERR_HIP;
  SideStream& ss = g_side[dev];
  // each handle created once; a failed creation is retried on the next call
  for (hipStream_t* st : {&ss.s, &ss.s2})
    if (*st == nullptr) GPTQ_HIP_TRY(hipStreamCreateWithFlags(st, hipStreamNonBlocking));
  for (hipEvent_t* ev : {&ss.fork, &ss.join, &ss.join2, &ss.fork2, &ss.join3})
    if (*ev == nullptr) GPTQ_HIP_TRY(hipEventCreateWithFlags(ev, hipEventDisableTiming));
  *out = &ss;
  return GPTQ_OK;
}

void timing_pair(gptq_timed_kernel kind, hipEvent_t* start, hipEvent_t* stop) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  *start = *stop = nullptr;
  if (kind < 0 || kind >= kTimedKinds || !(t.mask & (1 << kind))) return;
  std::pair<hipEvent_t, hipEvent_t> p{nullptr, nullptr};
  if (!t.pool.empty()) {
    p = t.pool.back();
    t.pool.pop_back();
  } else if (hipEventCreate(&p.first) != hipSuccess || hipEventCreate(&p.second) != hipSuccess) {
    return;
  }
  t.recorded[kind].push_back(p);
  *start = p.first;
  *stop = p.second;
}
}  // namespace gptq

extern "C" {

gptq_status gptq_timing_enable(int mask) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.mask = mask & ((1 << gptq::kTimedKinds) - 1);
  return GPTQ_OK;
}

gptq_status gptq_timing_read(gptq_timed_kernel which, double* total_ms, int64_t* launches) {
  if (total_ms == nullptr || launches == nullptr || which < 0 || which >= gptq::kTimedKinds)
    return GPTQ_ERR_INVALID_ARG;
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  double sum = 0.0;
  gptq_status st = GPTQ_OK;
  auto& rec = t.recorded[which];
  for (auto& p : rec) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.second) != hipSuccess || hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess) {
      st = GPTQ_ERR_HIP;
    }
    sum += ms;
    t.pool.push_back(p);
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(rec.size());
  rec.clear();
  return st;
}


gptq_status gptq_accumulate_hessian(int batch, int d_in, int64_t n_tokens, gptq_dtype x_dtype, const void* X,
                                    int64_t ldx, int64_t batch_stride_x, float* H, int64_t batch_stride_h,
                                    double* diag_key, int64_t* n_seen, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (batch < 1 || d_in < 8 || d_in % 8 != 0 || n_tokens < 0 || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
  if (H == nullptr || diag_key == nullptr || n_seen == nullptr) return GPTQ_ERR_INVALID_ARG;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  if (batch_stride_h < dd && batch > 1) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(H, 16) || (batch > 1 && batch_stride_h % 4 != 0)) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  const int64_t vec = 16 / static_cast<int64_t>(dtype_bytes(x_dtype));
  if (X == nullptr || ldx < d_in || ldx % vec != 0 || !aligned(X, 16)) return GPTQ_ERR_INVALID_ARG;
  if (batch > 1 && (batch_stride_x < ldx * n_tokens || batch_stride_x % vec != 0)) return GPTQ_ERR_INVALID_ARG;
  return gptq::hessian_enqueue(batch, d_in, n_tokens, x_dtype, X, ldx, batch_stride_x, nullptr, 0, H,
                               batch > 1 ? batch_stride_h : dd, diag_key, n_seen, workspace, workspace_bytes,
                               stream);
}

gptq_status gptq_accumulate_hessian_grouped(int batch, int d_in, int64_t total_tokens,
                                            int64_t max_tokens_per_problem, gptq_dtype x_dtype, const void* X,
                                            int64_t ldx, const int64_t* token_offsets, float* H,
                                            int64_t batch_stride_h, double* diag_key, int64_t* n_seen,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch < 1 || d_in < 8 || d_in % 8 != 0 || total_tokens < 0 || max_tokens_per_problem < 0 ||
      !valid_dtype(x_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (H == nullptr || diag_key == nullptr || n_seen == nullptr || token_offsets == nullptr ||
      !aligned(token_offsets, 8))
    return GPTQ_ERR_INVALID_ARG;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  if (batch_stride_h < dd && batch > 1) return GPTQ_ERR_INVALID_ARG;
  if (!aligned(H, 16) || (batch > 1 && batch_stride_h % 4 != 0)) return GPTQ_ERR_INVALID_ARG;
  if (max_tokens_per_problem == 0 || total_tokens == 0) return GPTQ_OK;
  const int64_t vec = 16 / static_cast<int64_t>(dtype_bytes(x_dtype));
  if (X == nullptr || ldx < d_in || ldx % vec != 0 || !aligned(X, 16)) return GPTQ_ERR_INVALID_ARG;
  return gptq::hessian_enqueue(batch, d_in, max_tokens_per_problem, x_dtype, X, ldx, 0, token_offsets, total_tokens,
                               H, batch > 1 ? batch_stride_h : dd, diag_key, n_seen, workspace, workspace_bytes,
                               stream);
}

gptq_status gptq_prepare_hinv(int batch, int d_in, const float* H, int64_t batch_stride_h, const double* diag_key,
                              const gptq_params* p, float* U, int64_t batch_stride_u, int32_t* perm, uint8_t* dead,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch < 1 || d_in < gptq::kBlock || d_in % gptq::kBlock != 0) return GPTQ_ERR_INVALID_ARG;
  if (H == nullptr || diag_key == nullptr || U == nullptr || perm == nullptr || dead == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  const gptq_status ps = check_params(p, d_in, false);
  if (ps != GPTQ_OK) return ps;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  if (batch > 1 && (batch_stride_h < dd || batch_stride_u < dd || batch_stride_u % 4 != 0))
    return GPTQ_ERR_INVALID_ARG;
  if (!aligned(U, 16)) return GPTQ_ERR_INVALID_ARG;
  int not_spd = 0;
  const gptq_status st = gptq::prepare_enqueue(batch, d_in, H, batch > 1 ? batch_stride_h : dd, diag_key, *p, U,
                                               batch > 1 ? batch_stride_u : dd, perm, dead, workspace,
                                               workspace_bytes, stream, &not_spd);
  if (st != GPTQ_OK) return st;
  return not_spd ? GPTQ_ERR_NOT_SPD : GPTQ_OK;
}

namespace {
// Arguments shared by gptq_quantize_layer and its allocation-free variant.
gptq_status check_quantize(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W, int64_t ldw,
                           int64_t batch_stride_w, const float* U, int64_t batch_stride_u, const int32_t* perm,
                           const uint8_t* dead, const gptq_params* p, uint8_t* codes, float* scales,
                           uint8_t* zeros, int32_t* g_idx) {
  if (batch < 1 || d_out < 1 || d_in < gptq::kBlock || d_in % gptq::kBlock != 0 || !valid_dtype(w_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (W == nullptr || U == nullptr || perm == nullptr || dead == nullptr || codes == nullptr || scales == nullptr ||
      zeros == nullptr || g_idx == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  const gptq_status ps = check_params(p, d_in, true);
  if (ps != GPTQ_OK) return ps;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  if (ldw < d_in) return GPTQ_ERR_INVALID_ARG;
  if (batch > 1 && (batch_stride_w < ldw * d_out || batch_stride_u < dd || batch_stride_u % 4 != 0))
    return GPTQ_ERR_INVALID_ARG;
  if (!aligned(U, 16)) return GPTQ_ERR_INVALID_ARG;
  return GPTQ_OK;
}
}  // namespace

gptq_status gptq_quantize_layer(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W, int64_t ldw,
                                int64_t batch_stride_w, const float* U, int64_t batch_stride_u, const int32_t* perm,
                                const uint8_t* dead, const gptq_params* p, uint8_t* codes, float* scales,
                                uint8_t* zeros, int32_t* g_idx, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  const gptq_status st = check_quantize(batch, d_out, d_in, w_dtype, W, ldw, batch_stride_w, U, batch_stride_u, perm,
                                        dead, p, codes, scales, zeros, g_idx);
  if (st != GPTQ_OK) return st;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  return gptq::quantize_enqueue(batch, d_out, d_in, w_dtype, W, ldw, batch > 1 ? batch_stride_w : ldw * d_out, U,
                                batch > 1 ? batch_stride_u : dd, perm, dead, *p, codes, scales, zeros, g_idx,
                                workspace, workspace_bytes, stream);
}

gptq_status gptq_quantize_layer_noalloc(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W,
                                        int64_t ldw, int64_t batch_stride_w, const float* U, int64_t batch_stride_u,
                                        const int32_t* perm, const uint8_t* dead, const gptq_params* p,
                                        uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                                        hipStream_t stream) {
  const gptq_status st = check_quantize(batch, d_out, d_in, w_dtype, W, ldw, batch_stride_w, U, batch_stride_u, perm,
                                        dead, p, codes, scales, zeros, g_idx);
  if (st != GPTQ_OK) return st;
  const int64_t dd = static_cast<int64_t>(d_in) * d_in;
  return gptq::quantize_noalloc_enqueue(batch, d_out, d_in, w_dtype, W, ldw,
                                        batch > 1 ? batch_stride_w : ldw * d_out, U, batch > 1 ? batch_stride_u : dd,
                                        perm, dead, *p, codes, scales, zeros, g_idx, stream);
}

gptq_status gptq_pack_int4(int batch, int d_out, int d_in, int n_groups, const uint8_t* codes, const float* scales,
                           const uint8_t* zeros, int32_t* qweight, int32_t* qzeros, uint16_t* scales_f16,
                           hipStream_t stream) {
  if (batch < 1 || d_out < 8 || d_out % 8 != 0 || d_in < 8 || d_in % 8 != 0 || n_groups < 1)
    return GPTQ_ERR_INVALID_ARG;
  if (codes == nullptr || scales == nullptr || zeros == nullptr || qweight == nullptr || qzeros == nullptr ||
      scales_f16 == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  return gptq::pack_enqueue(batch, d_out, d_in, n_groups, codes, scales, zeros, qweight, qzeros, scales_f16, stream);
}

gptq_status gptq_w4a16_repack(int batch, int d_out, int d_in, int n_groups, const int32_t* qweight,
                              const int32_t* g_idx, int32_t* qweight_s, int32_t* order, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (batch < 1 || d_out < 8 || d_out % 8 != 0 || d_in < 8 || d_in % 8 != 0 || n_groups < 1 || d_in % n_groups != 0)
    return GPTQ_ERR_INVALID_ARG;
  if (qweight == nullptr || g_idx == nullptr || qweight_s == nullptr || order == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < sizeof(int) || !aligned(workspace, 4)) return GPTQ_ERR_WORKSPACE;
  int* flag = static_cast<int*>(workspace);
  gptq_status st = gptq::repack_enqueue(batch, d_out, d_in, n_groups, qweight, g_idx, qweight_s, order, flag, stream);
  if (st != GPTQ_OK) return st;
  int bad = 0;
  GPTQ_HIP_TRY(hipMemcpyAsync(&bad, flag, sizeof(int), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_TRY(hipStreamSynchronize(stream));
  return bad ? GPTQ_ERR_INVALID_ARG : GPTQ_OK;
}

gptq_status gptq_w4a16_matmul(int m, int d_out, int d_in, int n_groups, gptq_dtype x_dtype, const void* X,
                              int64_t ldx, const int32_t* qweight_s, const int32_t* order, const int32_t* qzeros,
                              const uint16_t* scales_f16, float* Y, int64_t ldy, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (m < 1 || d_out < 8 || d_out % 8 != 0 || d_in < 128 || d_in % 128 != 0 || n_groups < 1 ||
      d_in % n_groups != 0)
    return GPTQ_ERR_INVALID_ARG;
  const int gs = d_in / n_groups;
  if (!(n_groups == 1 || gs == 32 || gs == 64 || gs == 128)) return GPTQ_ERR_UNSUPPORTED;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F16) return GPTQ_ERR_INVALID_ARG;
  if (X == nullptr || qweight_s == nullptr || qzeros == nullptr || scales_f16 == nullptr || Y == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  if (ldx < d_in || ldy < d_out || ldy % 4 != 0 || !aligned(Y, 16) || !aligned(qweight_s, 16) ||
      !aligned(scales_f16, 8))
    return GPTQ_ERR_INVALID_ARG;
  return gptq::serve_enqueue(m, d_out, d_in, n_groups, x_dtype, X, ldx, order, qweight_s, qzeros, scales_f16, Y, ldy,
                             workspace, workspace_bytes, stream);
}

size_t gptq_workspace_size(gptq_ws_call which, int batch, int d_out, int d_in, int64_t n_tokens_hint,
                           const gptq_params* p) {
  switch (which) {
    case GPTQ_WS_HESSIAN:
      if (d_in % 8 != 0) return 0;
      return gptq::hessian_workspace(batch, d_in, n_tokens_hint);
    case GPTQ_WS_PREPARE:
      return gptq::prepare_workspace(batch, d_in);
    case GPTQ_WS_QUANTIZE: {
      if (p == nullptr) return 0;
      return gptq::quantize_workspace(batch, d_out, d_in, *p);
    }
    case GPTQ_WS_W4A16_REPACK:
      return 256;
    case GPTQ_WS_W4A16: {
      if (p == nullptr || n_tokens_hint < 1 || n_tokens_hint > INT32_MAX) return 0;
      const int ng = p->group_size == -1 ? 1 : (p->group_size > 0 && d_in % p->group_size == 0 ? d_in / p->group_size : 0);
      if (ng == 0) return 0;
      return gptq::serve_workspace(static_cast<int>(n_tokens_hint), d_out, d_in, ng);
    }
  }
  return 0;
}

const char* gptq_status_string(gptq_status s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_SPD: return "damped Hessian is not positive definite";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GPTQ_ERR_UNSUPPORTED: return "unsupported parameters";
    case GPTQ_ERR_TOO_LARGE: return "problem exceeds the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

const char* gptq_version(void) { return "0.2.0"; }

}  // extern "C"
