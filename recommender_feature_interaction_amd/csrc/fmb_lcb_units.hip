// FMB + LCB for embedding units of width d = 8 (bf16, fp32 accumulation).
//
// Wukong paper, section 2.1: a feature's embedding is cut into 8-wide units
// and each unit takes part in the interaction as a feature of its own, so a
// layer sees n units of width d = 8 per example.  Section 2.2 defines the
// layer: [Z_b; Lc_b] = [Phi; W_L] X_b, F_b = X_b Z_b^T, Fn_b = LN(vec F_b),
// and the LCB rows of the output Y_b[n_F + i] = LN_d(Lc_b[i] + X_b[n_F + i]).
//
// With d = 8 an example's X_b is n x 16 bytes, too narrow for the per-example
// MFMA tiles of the other FMB+LCB kernels, and [Phi; W_L] (k + n_L rows of n)
// is far too large to stream per example.  So the left multiply becomes one
// GEMM over the whole batch:
//   1. units_transpose_kernel: Xt[b][e][j] = X[b][j][e] (the GEMM's operand,
//      K = n contiguous);
//   2. the bf16 DMA GEMM C'[r][(b, e)] = sum_j [Phi; W_L][r][j] Xt[(b, e)][j]
//      (units_gemm_kernel): its epilogue writes Z_b in fp32 and finishes the
//      LCB rows of Y (Lc in fp32 + residual, LayerNorm over the 8 values);
//   3. units_epilogue_kernel, a group of examples per workgroup: Z_b rounded
//      to bf16 (the MFMA operand precision of the other kernels) as a register
//      operand; F_b^T = Z_b X_b^T on the MFMA 32 rows at a time, the
//      statistics merged by Chan's parallel-variance formula (count, mean, sum
//      of squared deviations) and reduced over the workgroup; then a second
//      pass that recomputes each block and writes Fn with the FMB LayerNorm's
//      gamma / beta.
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

constexpr int UD = 8;        // unit width
constexpr int UE = 4;        // examples per workgroup in the epilogue
constexpr int UT = 256;      // threads per epilogue workgroup
constexpr int UKMAX = 32;    // largest k (Z rows fill one 32-row MFMA operand)

// Xt[b][e][j] = X[b][j][e]; two rows j, j + 1 per thread so each store is 4 bytes.
__global__ __launch_bounds__(256) void units_transpose_kernel(const uint16_t* x, uint16_t* xt, int64_t batch, int n) {
  const int half = n / 2;
  const int64_t total = batch * half;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = q / half;
    const int j = 2 * (int)(q - b * half);
    const u32x4 r0 = *reinterpret_cast<const u32x4*>(x + (b * n + j) * UD);
    const u32x4 r1 = *reinterpret_cast<const u32x4*>(x + (b * n + j + 1) * UD);
    uint32_t* out = reinterpret_cast<uint32_t*>(xt + b * n * UD + j);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      out[(2 * t) * (n / 2)] = pack_lo(r0[t], r1[t]);      // e = 2t
      out[(2 * t + 1) * (n / 2)] = pack_hi(r0[t], r1[t]);  // e = 2t + 1
    }
  }
}

struct UnitsArgs {
  const uint16_t* x;
  const float* z;            // [B][k][8]
  const uint16_t* fm_gamma;  // [n k] or null
  const uint16_t* fm_beta;
  uint16_t* fn;              // [B][n k]
  int n, k;
  float eps;
};

// Merge (count, mean, M2) of two disjoint sets (Chan, Golub, LeVeque).
__device__ __forceinline__ void chan_merge(float& cnt, float& mean, float& m2, float cb, float mb, float m2b) {
  const float tot = cnt + cb;
  if (cb == 0.f) return;
  if (cnt == 0.f) {
    cnt = cb;
    mean = mb;
    m2 = m2b;
    return;
  }
  const float delta = mb - mean;
  mean += delta * (cb / tot);
  m2 += m2b + delta * delta * (cnt * cb / tot);
  cnt = tot;
}

// F^T blocks on the MFMA: D = Z X^T over 32 rows m at a time with
// v_mfma_f32_32x32x16_bf16, the 8-wide contraction padded to 16 with zeros
// (lanes 32..63 supply zero operands).  Lane l then holds rows m = l % 32 and
// j = 8 (r / 4) + 4 (l / 32) + r % 4 of F, r = 0..15: chunks of 4 consecutive
// j, so the LayerNorm's gamma / beta and Fn move in 8-byte pieces.
__global__ __launch_bounds__(UT) void units_epilogue_kernel(UnitsArgs p, int64_t batch) {
  __shared__ float wred[UE][UT / 64][3];
  __shared__ float stat[UE][2];  // mean, rstd of F per example
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int n = p.n, k = p.k;
  const float inv_nk = 1.0f / (float)(n * k);
  const int64_t groups = (batch + UE - 1) / UE;
  for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
    const int64_t b0 = g * UE;
    const int ne = (int)(batch - b0 < UE ? batch - b0 : UE);
    // Z operands: lane l < 32 holds Z[l][0..7] rounded to bf16 (zero for l >= k)
    u32x4 zop[UE];
#pragma unroll
    for (int ex = 0; ex < UE; ++ex) {
      zop[ex] = u32x4{0u, 0u, 0u, 0u};
      if (ex < ne && h == 0 && l32 < k) {
        const f32x4* cz = reinterpret_cast<const f32x4*>(p.z + ((b0 + ex) * (int64_t)k + l32) * UD);
        const f32x4 z0 = cz[0], z1 = cz[1];
        zop[ex] = u32x4{pack_bf16x2(z0[0], z0[1]), pack_bf16x2(z0[2], z0[3]), pack_bf16x2(z1[0], z1[1]),
                        pack_bf16x2(z1[2], z1[3])};
      }
    }
    auto x_row = [&](int ex, int m) {  // lanes 0..31: X row m; lanes 32..63: zero (the padding)
      u32x4 xop = u32x4{0u, 0u, 0u, 0u};
      if (h == 0 && m < n) xop = *reinterpret_cast<const u32x4*>(p.x + ((b0 + ex) * n + m) * UD);
      return xop;
    };
    auto f_block = [&](int ex, const u32x4& xop) {  // this lane's 16 values of rows m .. m + 31 of F^T
      f32x16 zero;
#pragma unroll
      for (int r = 0; r < 16; ++r) zero[r] = 0.f;
      return mfma32x32x16(zop[ex], xop, zero);
    };
    // pass 1: statistics (count, mean, M2) per example
    float cnt[UE], mu[UE], m2[UE];
#pragma unroll
    for (int ex = 0; ex < UE; ++ex) cnt[ex] = mu[ex] = m2[ex] = 0.f;
    // The next block's loads are issued before this block's stores: the
    // vector-memory counter retires in order, so a load issued after a store
    // would also wait for the store to complete.
    u32x4 xc[UE], xn[UE];
    auto load_x = [&](int m, u32x4 (&xs)[UE]) {
#pragma unroll
      for (int ex = 0; ex < UE; ++ex) xs[ex] = ex < ne ? x_row(ex, m) : u32x4{0u, 0u, 0u, 0u};
    };
    if (wave * 32 < n) load_x(wave * 32 + l32, xc);
    for (int m0 = wave * 32; m0 < n; m0 += UT / 2) {
      const int m = m0 + l32;
      if (m0 + UT / 2 < n) load_x(m0 + UT / 2 + l32, xn);
#pragma unroll
      for (int ex = 0; ex < UE; ++ex) {
        if (ex >= ne) break;
        const u32x4 xop = xc[ex];
        const f32x16 d = f_block(ex, xop);
        float s = 0.f, c = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = m < n && 8 * (r >> 2) + 4 * h + (r & 3) < k;
          s += ok ? d[r] : 0.f;
          c += ok ? 1.f : 0.f;
        }
        const float lm = c > 0.f ? s / c : 0.f;
        float q = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = m < n && 8 * (r >> 2) + 4 * h + (r & 3) < k;
          q += ok ? (d[r] - lm) * (d[r] - lm) : 0.f;
        }
        chan_merge(cnt[ex], mu[ex], m2[ex], c, lm, q);
      }
#pragma unroll
      for (int ex = 0; ex < UE; ++ex) xc[ex] = xn[ex];
    }
#pragma unroll
    for (int ex = 0; ex < UE; ++ex) {
      for (int off = 1; off < 64; off <<= 1) {
        const float cb = __shfl_xor(cnt[ex], off, 64), mb = __shfl_xor(mu[ex], off, 64),
                    m2b = __shfl_xor(m2[ex], off, 64);
        chan_merge(cnt[ex], mu[ex], m2[ex], cb, mb, m2b);
      }
      if (lane == 0) {
        wred[ex][wave][0] = cnt[ex];
        wred[ex][wave][1] = mu[ex];
        wred[ex][wave][2] = m2[ex];
      }
    }
    __syncthreads();
    if (tid < UE) {
      float c0 = 0.f, mm = 0.f, s0 = 0.f;
      for (int w = 0; w < UT / 64; ++w) chan_merge(c0, mm, s0, wred[tid][w][0], wred[tid][w][1], wred[tid][w][2]);
      stat[tid][0] = mm;
      stat[tid][1] = rsqrtf(s0 * inv_nk + p.eps);
    }
    __syncthreads();
    // pass 2: recompute each block, FMB LayerNorm with gamma / beta, Fn in bf16
    // (the next block's X rows and gamma / beta requested before this block's stores)
    u32x2 gc[4], bc[4], gn[4], bn[4];
    auto load_gb = [&](int m, u32x2 (&gv)[4], u32x2 (&bv)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j0 = 8 * c + 4 * h;
        const bool ok = m < n && j0 < k;  // k % 4 == 0: all of j0 .. j0 + 3 valid
        const int64_t off = (int64_t)m * k + j0;
        gv[c] = ok && p.fm_gamma ? *reinterpret_cast<const u32x2*>(p.fm_gamma + off) : u32x2{0x3f803f80u, 0x3f803f80u};
        bv[c] = ok && p.fm_beta ? *reinterpret_cast<const u32x2*>(p.fm_beta + off) : u32x2{0u, 0u};
      }
    };
    if (wave * 32 < n) {
      load_x(wave * 32 + l32, xc);
      load_gb(wave * 32 + l32, gc, bc);
    }
    for (int m0 = wave * 32; m0 < n; m0 += UT / 2) {
      const int m = m0 + l32;
      if (m0 + UT / 2 < n) {
        load_x(m0 + UT / 2 + l32, xn);
        load_gb(m0 + UT / 2 + l32, gn, bn);
      }
#pragma unroll
      for (int ex = 0; ex < UE; ++ex) {
        if (ex >= ne) break;
        const f32x16 d = f_block(ex, xc[ex]);
        const float mean = stat[ex][0], rstd = stat[ex][1];
        uint16_t* out = p.fn + (b0 + ex) * (int64_t)n * k + (int64_t)m * k;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j0 = 8 * c + 4 * h;
          if (m < n && j0 < k) {
            u32x2 o;
            o[0] = pack_bf16x2((d[4 * c] - mean) * rstd * bf16lo(gc[c][0]) + bf16lo(bc[c][0]),
                               (d[4 * c + 1] - mean) * rstd * bf16hi(gc[c][0]) + bf16hi(bc[c][0]));
            o[1] = pack_bf16x2((d[4 * c + 2] - mean) * rstd * bf16lo(gc[c][1]) + bf16lo(bc[c][1]),
                               (d[4 * c + 3] - mean) * rstd * bf16hi(gc[c][1]) + bf16hi(bc[c][1]));
            *reinterpret_cast<u32x2*>(out + j0) = o;
          }
        }
      }
#pragma unroll
      for (int ex = 0; ex < UE; ++ex) xc[ex] = xn[ex];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gc[c] = gn[c];
        bc[c] = bn[c];
      }
    }
    __syncthreads();  // wred and stat are reused by the next group
  }
}

}  // namespace

bool fmb_lcb_units_supported(int n, int d, int k, int n_l) {
  return d == UD && n > 0 && n % 64 == 0 && k > 0 && k % 4 == 0 && k <= UKMAX && n_l > 0 && (k + n_l) % 8 == 0;
}

size_t fmb_lcb_units_workspace(int64_t batch, int n, int k, int n_l) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al((size_t)batch * n * UD * 2) + al((size_t)(k + n_l) * n * 2) + al((size_t)batch * k * UD * 4);
}

hipError_t launch_fmb_lcb_units(const FmbLcbArgs& a, int64_t batch, void* scratch, hipStream_t stream,
                                int64_t* workgroups) {
  if (!fmb_lcb_units_supported(a.n, a.d, a.k, a.n_l)) return hipErrorInvalidValue;
  if (workgroups) *workgroups = 0;
  if (batch == 0) return hipSuccess;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* base = static_cast<char*>(scratch);
  uint16_t* xt = reinterpret_cast<uint16_t*>(base);
  uint16_t* wcat = reinterpret_cast<uint16_t*>(base + al((size_t)batch * a.n * UD * 2));
  float* z = reinterpret_cast<float*>(base + al((size_t)batch * a.n * UD * 2) + al((size_t)(a.k + a.n_l) * a.n * 2));
  // [Phi; W_L] as one [k + n_l, n] operand
  hipError_t e = hipMemcpyAsync(wcat, a.phi, (size_t)a.k * a.n * 2, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(wcat + (size_t)a.k * a.n, a.w_l, (size_t)a.n_l * a.n * 2, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return e;
  int64_t tgrid = (batch * (a.n / 2) + 255) / 256;
  if (tgrid > 8192) tgrid = 8192;
  hipLaunchKernelGGL(units_transpose_kernel, dim3((unsigned)tgrid), dim3(256), 0, stream, a.x, xt, batch, a.n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  UnitsGemmArgs g;
  g.wcat = wcat;
  g.xt = xt;
  g.x = a.x;
  g.out_gamma = a.out_gamma;
  g.out_beta = a.out_beta;
  g.z = z;
  g.y = a.y;
  g.batch = batch;
  g.n = a.n;
  g.k = a.k;
  g.n_l = a.n_l;
  g.eps = a.eps;
  int64_t gw = 0;
  e = launch_units_gemm(g, stream, &gw);
  if (e != hipSuccess) return e;
  UnitsArgs u;
  u.x = a.x;
  u.z = z;
  u.fm_gamma = a.fm_gamma;
  u.fm_beta = a.fm_beta;
  u.fn = a.fn;
  u.n = a.n;
  u.k = a.k;
  u.eps = a.eps;
  const int64_t groups = (batch + UE - 1) / UE;
  const int64_t egrid = groups < 2048 ? groups : 2048;
  hipLaunchKernelGGL(units_epilogue_kernel, dim3((unsigned)egrid), dim3(UT), 0, stream, u, batch);
  if (workgroups) *workgroups = tgrid + gw + egrid;
  return hipGetLastError();
}

}  // namespace wk
