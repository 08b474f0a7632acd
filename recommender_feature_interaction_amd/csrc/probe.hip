// Measurement aid: the rate at which this GPU retires dense bf16 MFMA work
// (v_mfma_f32_16x16x32_bf16, the instruction of the Linear kernels) when
// every SIMD is kept busy and consecutive instructions take different
// operands, as in a GEMM main loop.  A loop on constant operands toggles far
// fewer bits and runs at a higher clock, so it would overstate the ceiling.
// The benchmark reports it beside the published peak (Kunlun technical
// summary, section 1, measures recommender modules by their fraction of the
// MFMA peak).
#include "wk_device.h"

namespace wk {
namespace {

constexpr int kProbeThreads = 512;  // 8 waves: two per SIMD

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const u32x4* __restrict__ ops,
                                                                   float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(8 + i) * 64 + lane];
  }
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = mfma16x16x32(a[i & 7], b[(3 * i + 1) & 7], acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace wk

extern "C" int32_t wukong_probe_mfma_bf16(const void* operands, void* sink, int32_t blocks, int32_t iters,
                                          void* stream) {
  if (operands == nullptr || sink == nullptr || blocks <= 0 || iters <= 0) return 1;  // WK_ERR_INVALID_ARG
  hipLaunchKernelGGL(wk::mfma_probe_kernel, dim3((unsigned)blocks), dim3(wk::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const wk::u32x4*>(operands),
                     static_cast<float*>(sink), iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;  // WK_OK : WK_ERR_HIP
}
