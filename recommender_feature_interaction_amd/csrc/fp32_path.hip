// fp32 variants of the Wukong layer kernels (plain VALU FMA, fp32 throughout).
//
// Same layer as the bf16 path (Wukong paper, section 2.2, xdnf.cn repost):
// FMB compress Z = Phi X, interaction F = X Z^T, LN over vec(F); LCB rows
// Lc = W_L X finished with the residual LayerNorm; an MLP Linear; the FMB
// rows' residual LayerNorm lives in resid_ln.hip.  These serve small fp32
// layers, where launch latency dominates, so they favour simplicity: one
// workgroup per example holding X, Z, F and Lc in LDS.
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

constexpr int kF32Threads = 256;
constexpr size_t kF32MaxLds = 64 * 1024;

size_t fmb_lcb_f32_lds(int n, int d, int k, int n_l) {
  return (size_t)(n * d + k * d + n * k + n_l * d) * sizeof(float);
}

__device__ float block_sum(float v, float* red) {
  v = xor_sum<1>(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kF32Threads) void fmb_lcb_f32_kernel(FmbLcbF32Args p) {
  extern __shared__ __align__(16) float fs[];
  __shared__ float red[kF32Threads / 64];
  const int n = p.n, d = p.d, k = p.k, n_l = p.n_l, n_f = p.n_f;
  float* X = fs;                // [n][d]
  float* Z = X + n * d;         // [k][d]
  float* F = Z + k * d;         // [n][k]
  float* L = F + n * k;         // [n_l][d]
  const int64_t b = blockIdx.x;
  const float* xb = p.x + b * (int64_t)n * d;
  const int tid = threadIdx.x;
  for (int i = tid; i < n * d; i += blockDim.x) X[i] = xb[i];
  __syncthreads();
  // Z = Phi X and Lc = W_L X
  for (int i = tid; i < (k + n_l) * d; i += blockDim.x) {
    const int z = i / d, e = i % d;
    const float* wr = z < k ? p.phi + (int64_t)z * n : p.w_l + (int64_t)(z - k) * n;
    float s = 0.f;
    for (int m = 0; m < n; ++m) s = fmaf(wr[m], X[m * d + e], s);
    if (z < k) Z[z * d + e] = s; else L[(z - k) * d + e] = s;
  }
  __syncthreads();
  // F = X Z^T
  float ls = 0.f;
  for (int i = tid; i < n * k; i += blockDim.x) {
    const int m = i / k, j = i % k;
    float s = 0.f;
    for (int e = 0; e < d; ++e) s = fmaf(X[m * d + e], Z[j * d + e], s);
    F[i] = s;
    ls += s;
  }
  const float inv_nk = 1.0f / (float)(n * k);
  const float mean = block_sum(ls, red) * inv_nk;  // block_sum syncs, so F is complete
  float lq = 0.f;
  for (int i = tid; i < n * k; i += blockDim.x) {
    const float dv = F[i] - mean;
    lq += dv * dv;
  }
  const float rstd = rsqrtf(block_sum(lq, red) * inv_nk + p.eps);
  float* fnb = p.fn + b * (int64_t)n * k;
  for (int i = tid; i < n * k; i += blockDim.x) {
    const float gm = p.fm_gamma ? p.fm_gamma[i] : 1.f, bt = p.fm_beta ? p.fm_beta[i] : 0.f;
    fnb[i] = (F[i] - mean) * rstd * gm + bt;
  }
  // LCB rows of Y: one wave per row
  const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int i = wave; i < n_l; i += nw) {
    const int row = n_f + i;
    float s = 0.f;
    for (int e = lane; e < d; e += 64) s += L[i * d + e] + X[row * d + e];
    s = xor_sum<1>(s);
    const float mu = s / (float)d;
    float q = 0.f;
    for (int e = lane; e < d; e += 64) {
      const float dv = L[i * d + e] + X[row * d + e] - mu;
      q += dv * dv;
    }
    q = xor_sum<1>(q);
    const float rs = rsqrtf(q / (float)d + p.eps);
    float* yr = p.y + (b * n + row) * (int64_t)d;
    for (int e = lane; e < d; e += 64) {
      const float gm = p.out_gamma ? p.out_gamma[e] : 1.f, bt = p.out_beta ? p.out_beta[e] : 0.f;
      yr[e] = (L[i * d + e] + X[row * d + e] - mu) * rs * gm + bt;
    }
  }
}

// C = act(A W^T + bias): 64x64 tiles, 256 threads with 4x4 outputs each.
__global__ __launch_bounds__(256) void linear_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                         const float* __restrict__ bias, float* __restrict__ C,
                                                         int64_t M, int N, int K, int relu) {
  __shared__ float sA[16][65];
  __shared__ float sW[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * 256, r = idx >> 4, c = idx & 15;
      sA[c][r] = (m0 + r < M && k0 + c < K) ? A[(m0 + r) * K + k0 + c] : 0.f;
      sW[c][r] = (n0 + r < N && k0 + c < K) ? W[(int64_t)(n0 + r) * K + k0 + c] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) w[j] = sW[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j] + (bias ? bias[n] : 0.f);
      if (relu) v = fmaxf(v, 0.f);
      C[m * N + n] = v;
    }
  }
}

}  // namespace

bool fmb_lcb_f32_supported(int n, int d, int k, int n_l) {
  return n > 0 && d > 0 && k > 0 && n_l > 0 && fmb_lcb_f32_lds(n, d, k, n_l) <= kF32MaxLds;
}

hipError_t launch_fmb_lcb_f32(const FmbLcbF32Args& a, int64_t batch, hipStream_t stream,
                              int64_t* workgroups) {
  if (!fmb_lcb_f32_supported(a.n, a.d, a.k, a.n_l)) return hipErrorInvalidValue;
  if (workgroups) *workgroups = batch;
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(fmb_lcb_f32_kernel, dim3((unsigned)batch), dim3(kF32Threads),
                     fmb_lcb_f32_lds(a.n, a.d, a.k, a.n_l), stream, a);
  return hipGetLastError();
}

hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t stream, int64_t* workgroups) {
  const int64_t gy = (a.M + 63) / 64;
  const int gx = (a.N + 63) / 64;
  if (workgroups) *workgroups = gy * gx;
  if (gy == 0 || gx == 0) return hipSuccess;
  hipLaunchKernelGGL(linear_f32_kernel, dim3(gx, (unsigned)gy), dim3(256), 0, stream,
                     static_cast<const float*>(a.a), static_cast<const float*>(a.w),
                     static_cast<const float*>(a.bias), static_cast<float*>(a.c), a.M, a.N, a.K, a.act == kActRelu ? 1 : 0);
  return hipGetLastError();
}

}  // namespace wk
