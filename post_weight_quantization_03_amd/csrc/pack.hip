// Checkpoint packing on gfx950 ("04 — GPTQ: ...", section 8; "GPTQ Architecture, in
// depth", "Packing, tooling and serving"): eight 4-bit values per int32, element k in
// bits [4k, 4k + 4); qweight packs along the input dimension, qzeros along the output
// dimension; scales become fp16 with round-to-nearest-even.
//
// qweight [d_in/8, d_out] is the transpose of the code layout [d_out, d_in]: a workgroup
// stages a 64-row x 256-column code tile in LDS with coalesced 16-byte loads, then writes
// 32 x 64 int32 words with consecutive lanes on consecutive output columns.
#include "common.h"

namespace gptq {
namespace {

constexpr int PR = 64;    // code rows (output features) per workgroup
constexpr int PC = 256;   // code columns (input features) per workgroup

__global__ __launch_bounds__(256) void pack_qweight_kernel(const uint8_t* __restrict__ codes, int d_out, int d_in,
                                                           int32_t* __restrict__ qweight) {
  __shared__ __attribute__((aligned(16))) uint8_t sc[PR][PC + 16];
  const int o0 = blockIdx.x * PR, c0 = blockIdx.y * PC, e = blockIdx.z;
  const uint8_t* ce = codes + static_cast<int64_t>(e) * d_out * d_in;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = tid / 16 + 16 * q, c16 = (tid % 16) * 16;
    const int o = o0 + row, c = c0 + c16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (o < d_out) {
      const uint8_t* src = ce + static_cast<int64_t>(o) * d_in + c;
      if (c + 16 <= d_in && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
        v = *reinterpret_cast<const uint4*>(src);
      } else {
        uint8_t b[16];
        for (int k = 0; k < 16; ++k) b[k] = (c + k < d_in) ? src[k] : 0;
        v = *reinterpret_cast<const uint4*>(b);
      }
    }
    *reinterpret_cast<uint4*>(&sc[row][c16]) = v;
  }
  __syncthreads();
  const int ol = tid % PR;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int il = tid / PR + 4 * q;          // word row within the tile (0..31)
    const int o = o0 + ol, i = c0 / 8 + il;
    if (o >= d_out || 8 * i >= d_in) continue;
    uint32_t word = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) word |= (static_cast<uint32_t>(sc[ol][8 * il + k]) & 15u) << (4 * k);
    qweight[static_cast<int64_t>(e) * (d_in / 8) * d_out + static_cast<int64_t>(i) * d_out + o] =
        static_cast<int32_t>(word);
  }
}

__global__ __launch_bounds__(256) void pack_meta_kernel(const float* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, int64_t n_meta,
                                                        int d_out, int32_t* __restrict__ qzeros,
                                                        uint16_t* __restrict__ scales_f16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // over batch*n_groups*d_out
  if (i >= n_meta) return;
  scales_f16[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(scales[i]));
  if ((i % 8) == 0) {
    uint32_t word = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) word |= (static_cast<uint32_t>(zeros[i + k]) & 15u) << (4 * k);
    qzeros[i / 8] = static_cast<int32_t>(word);
  }
}

}  // namespace

gptq_status pack_enqueue(int batch, int d_out, int d_in, int n_groups, const uint8_t* codes, const float* scales,
                         const uint8_t* zeros, int32_t* qweight, int32_t* qzeros, uint16_t* scales_f16,
                         hipStream_t stream) {
  const dim3 grid((d_out + PR - 1) / PR, (d_in + PC - 1) / PC, batch);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  timing_pair(GPTQ_TIME_PACK, &ev0, &ev1);
  if (ev0) GPTQ_HIP_TRY(hipEventRecord(ev0, stream));
  GPTQ_LAUNCH(pack_qweight_kernel, grid, dim3(256), 0, stream, codes, d_out, d_in, qweight);
  const int64_t n_meta = static_cast<int64_t>(batch) * n_groups * d_out;
  GPTQ_LAUNCH(pack_meta_kernel, dim3(static_cast<unsigned>((n_meta + 255) / 256)), dim3(256), 0, stream, scales,
              zeros, n_meta, d_out, qzeros, scales_f16);
  if (ev1) GPTQ_HIP_TRY(hipEventRecord(ev1, stream));
  return GPTQ_OK;
}

}  // namespace gptq
