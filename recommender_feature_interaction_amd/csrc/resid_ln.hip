// FMB rows of a Wukong layer's output: Y[b, r] = LN_d(M[b, r] + X[b, r]), r < n_F.
//
// Wukong paper, section 2.2 (xdnf.cn repost): the FMB and LCB outputs are
// concatenated, the residual is added and a LayerNorm is applied.  The LCB
// rows are finished inside the FMB+LCB kernel; this kernel finishes the FMB
// rows once the MLP has produced M = reshape(h_T, n_F x d).
//
// Memory-bound: per row it reads d values of M and of X and writes d values
// of Y.  A row of d bf16 is d/8 16-byte vectors; LPR lanes share a row
// (LPR = the largest power of two <= 8 dividing d/8) and each lane holds VPL
// vectors, lane j of the row taking vectors j, j + LPR, ...  Row statistics
// are a log2(LPR)-step xor-shuffle; the row stays in registers between the
// mean, the variance and the output pass.
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

struct ResidLnKArgs {
  const uint16_t* m;
  const uint16_t* x;
  const uint16_t* gamma;
  const uint16_t* beta;
  uint16_t* y;
  int64_t rows;  // batch * n_f
  int n, n_f;
  float eps;
};

template <int VPL, int LPR>
__global__ __launch_bounds__(256) void resid_ln_bf16_kernel(ResidLnKArgs p) {
  constexpr int D = 8 * VPL * LPR;
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  const int lr = lane % LPR;
  const bool valid = g < p.rows;
  const int64_t gg = valid ? g : 0;
  const int64_t b = gg / p.n_f;
  const int r = (int)(gg - b * p.n_f);
  const uint16_t* mrow = p.m + gg * D;
  const uint16_t* xrow = p.x + (b * p.n + r) * (int64_t)D;
  uint16_t* yrow = p.y + (b * p.n + r) * (int64_t)D;

  float v[VPL][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = (lr + LPR * i) * 8;
    u32x4 mv = u32x4{0u, 0u, 0u, 0u}, xv = u32x4{0u, 0u, 0u, 0u};
    if (valid) {
      mv = *reinterpret_cast<const u32x4*>(mrow + e);
      xv = *reinterpret_cast<const u32x4*>(xrow + e);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[i][2 * h] = bf16lo(mv[h]) + bf16lo(xv[h]);
      v[i][2 * h + 1] = bf16hi(mv[h]) + bf16hi(xv[h]);
      s += v[i][2 * h] + v[i][2 * h + 1];
    }
  }
  s = group_sum<LPR>(s);
  const float inv_d = 1.0f / (float)D;
  const float mean = s * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float dv = v[i][t] - mean;
      q += dv * dv;
    }
  q = group_sum<LPR>(q);
  const float rstd = rsqrtf(q * inv_d + p.eps);
  if (!valid) return;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = (lr + LPR * i) * 8;
    float gm[8], bt[8];
    if (p.gamma) {
      const u32x4 g4 = *reinterpret_cast<const u32x4*>(p.gamma + e);
#pragma unroll
      for (int h = 0; h < 4; ++h) { gm[2 * h] = bf16lo(g4[h]); gm[2 * h + 1] = bf16hi(g4[h]); }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) gm[t] = 1.f;
    }
    if (p.beta) {
      const u32x4 b4 = *reinterpret_cast<const u32x4*>(p.beta + e);
#pragma unroll
      for (int h = 0; h < 4; ++h) { bt[2 * h] = bf16lo(b4[h]); bt[2 * h + 1] = bf16hi(b4[h]); }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) bt[t] = 0.f;
    }
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = pack_bf16x2((v[i][2 * h] - mean) * rstd * gm[2 * h] + bt[2 * h],
                         (v[i][2 * h + 1] - mean) * rstd * gm[2 * h + 1] + bt[2 * h + 1]);
    *reinterpret_cast<u32x4*>(yrow + e) = o;
  }
}

struct ResidVariant {
  int vpl, lpr;
  void (*kernel)(ResidLnKArgs);
};

#define WK_RES_VARIANT(VPL, LPR) ResidVariant{VPL, LPR, resid_ln_bf16_kernel<VPL, LPR>}

const ResidVariant kResVariants[] = {
    WK_RES_VARIANT(1, 1), WK_RES_VARIANT(1, 2), WK_RES_VARIANT(3, 1), WK_RES_VARIANT(1, 4),
    WK_RES_VARIANT(5, 1), WK_RES_VARIANT(3, 2), WK_RES_VARIANT(7, 1), WK_RES_VARIANT(1, 8),
    WK_RES_VARIANT(5, 2), WK_RES_VARIANT(3, 4), WK_RES_VARIANT(2, 8), WK_RES_VARIANT(5, 4),
    WK_RES_VARIANT(3, 8), WK_RES_VARIANT(4, 8), WK_RES_VARIANT(5, 8), WK_RES_VARIANT(6, 8),
    WK_RES_VARIANT(8, 8),
};

const ResidVariant* pick_res(int d) {
  if (d <= 0 || d % 8 != 0) return nullptr;
  const int v = d / 8;
  int lpr = 1;
  while (lpr < 8 && v % (lpr * 2) == 0) lpr *= 2;
  const int vpl = v / lpr;
  for (const auto& r : kResVariants)
    if (r.vpl == vpl && r.lpr == lpr) return &r;
  return nullptr;
}

// fp32: one wave per row, lanes stride over d.
__global__ __launch_bounds__(256) void resid_ln_f32_kernel(const float* m, const float* x, const float* gamma,
                                                           const float* beta, float* y, int64_t rows, int n,
                                                           int n_f, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= rows) return;  // wave-uniform
  const int64_t b = g / n_f;
  const int r = (int)(g - b * n_f);
  const float* mr = m + g * d;
  const float* xr = x + (b * n + r) * (int64_t)d;
  float* yr = y + (b * n + r) * (int64_t)d;
  float s = 0.f;
  for (int e = lane; e < d; e += 64) s += mr[e] + xr[e];
  s = group_sum_v<64>(s);
  const float mean = s / (float)d;
  float q = 0.f;
  for (int e = lane; e < d; e += 64) {
    const float dv = mr[e] + xr[e] - mean;
    q += dv * dv;
  }
  q = group_sum_v<64>(q);
  const float rstd = rsqrtf(q / (float)d + eps);
  for (int e = lane; e < d; e += 64) {
    const float gm = gamma ? gamma[e] : 1.f, bt = beta ? beta[e] : 0.f;
    yr[e] = (mr[e] + xr[e] - mean) * rstd * gm + bt;
  }
}

}  // namespace

bool resid_ln_bf16_supported(int d) { return pick_res(d) != nullptr; }

hipError_t launch_resid_ln_bf16(const ResidLnArgs& a, hipStream_t stream, int64_t* workgroups) {
  const ResidVariant* v = pick_res(a.d);
  if (!v) return hipErrorInvalidValue;
  ResidLnKArgs k;
  k.m = static_cast<const uint16_t*>(a.m);
  k.x = static_cast<const uint16_t*>(a.x);
  k.gamma = static_cast<const uint16_t*>(a.gamma);
  k.beta = static_cast<const uint16_t*>(a.beta);
  k.y = static_cast<uint16_t*>(a.y);
  k.rows = a.batch * a.n_f;
  k.n = a.n;
  k.n_f = a.n_f;
  k.eps = a.eps;
  const int64_t rows_per_block = 4 * (64 / v->lpr);
  const int64_t blocks = (k.rows + rows_per_block - 1) / rows_per_block;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_resid_ln_f32(const ResidLnArgs& a, hipStream_t stream, int64_t* workgroups) {
  const int64_t rows = a.batch * a.n_f;
  const int64_t blocks = (rows + 3) / 4;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(resid_ln_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const float*>(a.m), static_cast<const float*>(a.x),
                     static_cast<const float*>(a.gamma), static_cast<const float*>(a.beta),
                     static_cast<float*>(a.y), rows, a.n, a.n_f, a.d, a.eps);
  return hipGetLastError();
}

}  // namespace wk
