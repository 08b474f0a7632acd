// The prediction head's last Linear and logistic function (Wukong paper,
// section 2.2: after the interaction layers an MLP produces the prediction).
//
// prob[m, o] = 1 / (1 + exp(-(sum_k A[m, k] W[o, k] + bias[o])))
//
// The last Linear of a prediction head has one (or a few) outputs, far too
// narrow for an MFMA tile: it is a dot product per (example, output) pair,
// HBM-bound on reading A once.  One wave per pair: each lane accumulates a
// strided slice of K in fp32 (16-byte loads of 8 bf16, or coalesced fp32
// loads), a wave-wide xor reduction sums the slices, lane 0 applies the bias
// and the logistic function in its overflow-free form.
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float logistic(float z) {
  if (z >= 0.f) return 1.f / (1.f + expf(-z));
  const float e = expf(z);
  return e / (1.f + e);
}

__global__ __launch_bounds__(kWavesPerBlock * 64) void head_out_bf16_kernel(HeadOutArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t q = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);  // (example, output) pair
  if (q >= p.M * p.N) return;  // wave-uniform
  const int64_t m = q / p.N;
  const int o = (int)(q - m * p.N);
  const uint16_t* a = static_cast<const uint16_t*>(p.a) + m * p.K;
  const uint16_t* w = static_cast<const uint16_t*>(p.w) + (int64_t)o * p.K;
  float acc = 0.f;
  for (int k0 = lane * 8; k0 < p.K; k0 += 64 * 8) {  // K % 8 == 0
    const u32x4 av = *reinterpret_cast<const u32x4*>(a + k0);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16lo(av[i]) * bf16lo(wv[i]) + bf16hi(av[i]) * bf16hi(wv[i]);
  }
  acc = xor_sum<1>(acc);
  if (lane == 0) {
    const float b = p.bias ? bf16_to_f32(static_cast<const uint16_t*>(p.bias)[o]) : 0.f;
    p.prob[q] = logistic(acc + b);
  }
}

__global__ __launch_bounds__(kWavesPerBlock * 64) void head_out_f32_kernel(HeadOutArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t q = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (q >= p.M * p.N) return;  // wave-uniform
  const int64_t m = q / p.N;
  const int o = (int)(q - m * p.N);
  const float* a = static_cast<const float*>(p.a) + m * p.K;
  const float* w = static_cast<const float*>(p.w) + (int64_t)o * p.K;
  float acc = 0.f;
  for (int k = lane; k < p.K; k += 64) acc += a[k] * w[k];
  acc = xor_sum<1>(acc);
  if (lane == 0) {
    const float b = p.bias ? static_cast<const float*>(p.bias)[o] : 0.f;
    p.prob[q] = logistic(acc + b);
  }
}

}  // namespace

hipError_t launch_head_out(const HeadOutArgs& a, bool bf16, hipStream_t stream, int64_t* workgroups) {
  const int64_t pairs = a.M * a.N;
  const int64_t blocks = (pairs + kWavesPerBlock - 1) / kWavesPerBlock;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(head_out_bf16_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(head_out_f32_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wk
