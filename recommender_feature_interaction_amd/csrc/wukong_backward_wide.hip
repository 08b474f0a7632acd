// Backward pass of one Wukong layer in bf16 for the wide layers (n of 256 to
// 720 embeddings), whose per-example working set does not fit the fused
// per-example kernels of wukong_backward.hip.  The chain rule is the same
// (Wukong paper, section 2.2: Z = Phi X, F = X Z^T, Fn = LN(vec F), the MLP to
// M, Lc = W_L X, Y = LN_d([M; Lc] + X)); the work is split so that every
// contraction with a weight shared by the batch runs as one batched GEMM:
//
//  bwd_rows_kernel, per row of every example: R = [M; Lc] + X from the
//    training forward's M and Lc (which it saved), the output LayerNorm's
//    input gradient dR = rstd (g - mean(g) - R_hat mean(g R_hat)), g = dY
//    gamma_out, stored in bf16 as dM (rows < n_F, the MLP's upstream gradient)
//    and as rows k .. k + n_L - 1 of G, the batch-major gradient matrix
//    [dZ; dLc] (element (row r, example b, column e) at G[r][b d + e]);
//    per-workgroup sums of dY R_hat and dY (gamma_out / beta_out gradients).
//  (the MLP's backward, on the GEMM kernels, gives d_Fn.)
//  bwd_fm_wide_kernel, per example with X, the saved Z and dF in LDS: F = X
//    Z^T with MFMA, the FM LayerNorm's statistics and input gradient dF
//    (bf16), dZ = dF^T X (bf16, to rows 0 .. k - 1 of G) and dXa = dR + dF Z
//    (fp32); per-workgroup sums of d_Fn F_hat and d_Fn (gamma_fm / beta_fm).
//  Then, on the GEMM kernels: d[Phi; W_L] = G X'^T with X' the batch-major
//  copy of X (split along the batch), and C = [Phi; W_L]^T G, from which
//  dx_final_kernel forms dX = bf16(dXa + C) (C is batch-major as well).
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define WW_LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4*)(p))

constexpr int kLdsMaxW = 160 * 1024;

__device__ __forceinline__ u32x4 row_frag(const uint16_t* base, int pitch, int r0, int c0, int li, int lg) {
  return *reinterpret_cast<const u32x4*>(base + (r0 + li) * pitch + c0 + 8 * lg);
}
// Rows r0 + 8 lg .. r0 + 8 lg + 7 of column c0 + li: lane (li, lg) addresses row
// r0 + 8 lg + li / 4, columns c0 + 4 (li % 4) ..; ds_read_b64_tr_b16 hands it
// rows + 0 .. 3 of column c0 + li, the second read (4 rows further) + 4 .. 7.
__device__ __forceinline__ u32x4 col_frag(const uint16_t* base, int pitch, int r0, int c0, int li, int lg) {
  const uint16_t* p0 = base + (r0 + 8 * lg + (li >> 2)) * pitch + c0 + 4 * (li & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WW_LDS_I16X4(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WW_LDS_I16X4(p0 + 4 * pitch));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

__device__ __forceinline__ float bf(uint16_t v) { return bf16_to_f32(v); }

// ---------------------------------------------------------------- rows
// LPR lanes per row, VPL 16-byte vectors per lane (D = 8 LPR VPL), vector v of
// lane i covering elements 8 (v LPR + i) ..
constexpr int kRowThreads = 256;

template <int D, int LPR>
__global__ __launch_bounds__(kRowThreads) void bwd_rows_kernel(BwdRowsArgs p) {
  constexpr int VPL = D / 8 / LPR;
  constexpr int RPI = kRowThreads / LPR;  // rows per workgroup iteration
  static_assert(VPL * LPR * 8 == D, "row split");
  __shared__ float red[kRowThreads / 64][2 * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR;
  const int n = p.n, n_f = p.n_f, k = p.k;
  const int64_t rows = p.batch * n;
  float dg[VPL][8], db[VPL][8], gam[VPL][8];
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      dg[v][t] = 0.f;
      db[v][t] = 0.f;
      const int e = 8 * (v * LPR + li) + t;
      gam[v][t] = p.gamma ? bf(static_cast<const uint16_t*>(p.gamma)[e]) : 1.f;
    }
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* DY = static_cast<const uint16_t*>(p.dy);
  const uint16_t* M = static_cast<const uint16_t*>(p.m);
  const float* LC = p.lc;
  uint16_t* DM = static_cast<uint16_t*>(p.dm);
  uint16_t* G = static_cast<uint16_t*>(p.g);
  const float inv_d = 1.0f / (float)D;
  for (int64_t row = (int64_t)blockIdx.x * RPI + tid / LPR; row < rows; row += (int64_t)gridDim.x * RPI) {
    const int64_t b = row / n;
    const int r = (int)(row - b * n);
    float R[VPL][8], gy[VPL][8];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e0 = 8 * (v * LPR + li);
      const u32x4 xv = *reinterpret_cast<const u32x4*>(X + row * D + e0);
      const u32x4 yv = *reinterpret_cast<const u32x4*>(DY + row * D + e0);
      float base[8];
      if (r < n_f) {
        const u32x4 mv = *reinterpret_cast<const u32x4*>(M + (b * n_f + r) * D + e0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          base[2 * t] = bf16lo(mv[t]);
          base[2 * t + 1] = bf16hi(mv[t]);
        }
      } else {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(LC + (b * p.n_l + (r - n_f)) * D + e0);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(LC + (b * p.n_l + (r - n_f)) * D + e0 + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          base[t] = l0[t];
          base[4 + t] = l1[t];
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        R[v][2 * t] = base[2 * t] + bf16lo(xv[t]);
        R[v][2 * t + 1] = base[2 * t + 1] + bf16hi(xv[t]);
        gy[v][2 * t] = bf16lo(yv[t]);
        gy[v][2 * t + 1] = bf16hi(yv[t]);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int t = 0; t < 8; ++t) s += R[v][t];
    const float mean = group_sum<LPR>(s) * inv_d;
    float q = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float dv = R[v][t] - mean;
        q += dv * dv;
      }
    const float rstd = rsqrtf(group_sum<LPR>(q) * inv_d + p.eps);
    float sg = 0.f, sgr = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float rh = (R[v][t] - mean) * rstd;
        const float g = gy[v][t] * gam[v][t];
        R[v][t] = rh;
        sg += g;
        sgr += g * rh;
        dg[v][t] += gy[v][t] * rh;
        db[v][t] += gy[v][t];
      }
    const float mg = group_sum<LPR>(sg) * inv_d, mgr = group_sum<LPR>(sgr) * inv_d;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e0 = 8 * (v * LPR + li);
      u32x4 o;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a0 = rstd * (gy[v][2 * t] * gam[v][2 * t] - mg - R[v][2 * t] * mgr);
        const float a1 = rstd * (gy[v][2 * t + 1] * gam[v][2 * t + 1] - mg - R[v][2 * t + 1] * mgr);
        o[t] = pack_bf16x2(a0, a1);
      }
      if (r < n_f) *reinterpret_cast<u32x4*>(DM + (b * n_f + r) * D + e0) = o;
      else *reinterpret_cast<u32x4*>(G + (int64_t)(k + r - n_f) * p.ldg + b * D + e0) = o;
    }
  }
  // per-workgroup sums: lanes with the same li share elements; across the wave by
  // xor-shuffles over the row index, across the waves in LDS
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float a = dg[v][t], c = db[v][t];
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) {
        a += __shfl_xor(a, m, kWave);
        c += __shfl_xor(c, m, kWave);
      }
      if (lane < LPR) {
        const int e = 8 * (v * LPR + li) + t;
        red[wave][e] = a;
        red[wave][D + e] = c;
      }
    }
  __syncthreads();
  for (int i = tid; i < 2 * D; i += kRowThreads) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kRowThreads / 64; ++w) s += red[w][i];
    p.part[(int64_t)blockIdx.x * 2 * D + i] = s;
  }
}

// ---------------------------------------------------------------- FM part, per example
constexpr int kFmWaves = 8;
constexpr int kFmThreads = kFmWaves * 64;

struct FmLds {
  int np, kp, xp, fp;  // rows of X and dF (n rounded up to 32), k rounded up to 32, pitches (u16)
  size_t xs, zs, fs, red, bytes;
};
__host__ __device__ inline FmLds fm_lds(int n, int d, int k) {
  FmLds L;
  L.np = (n + 31) / 32 * 32;
  L.kp = (k + 31) / 32 * 32;
  L.xp = d + 8;
  L.fp = L.kp + 8;
  L.xs = 0;
  L.zs = L.xs + (size_t)L.np * L.xp * 2;
  L.fs = L.zs + (size_t)L.kp * L.xp * 2;
  L.red = L.fs + (size_t)L.np * L.fp * 2;
  L.bytes = L.red + 4 * kFmWaves * sizeof(float);
  return L;
}

// D: embedding width; MPW: 16-row tiles of F per wave (ceil(n / 128)); KJ: 16-column tiles of k.
template <int D, int MPW, int KJ>
__global__ __launch_bounds__(kFmThreads) void bwd_fm_wide_kernel(BwdFmWideArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int n = p.n, k = p.k, n_f = p.n_f;
  const FmLds L = fm_lds(n, D, k);
  uint16_t* Xs = reinterpret_cast<uint16_t*>(smem + L.xs);
  uint16_t* Zs = reinterpret_cast<uint16_t*>(smem + L.zs);
  uint16_t* Fs = reinterpret_cast<uint16_t*>(smem + L.fs);
  float* red = reinterpret_cast<float*>(smem + L.red);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int XP = L.xp, FP = L.fp, NP = L.np, KP = L.kp;
  const int nk = n * k;
  // zero once: the padding rows of X, Z and dF and the padding columns of dF
  for (int i = tid; i < (int)(L.red / 2); i += kFmThreads) reinterpret_cast<uint16_t*>(smem)[i] = 0;
  __syncthreads();
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* Z = static_cast<const uint16_t*>(p.z);
  const uint16_t* DFN = static_cast<const uint16_t*>(p.dfn);
  const uint16_t* GAM = static_cast<const uint16_t*>(p.fm_gamma);
  const uint16_t* DM = static_cast<const uint16_t*>(p.dm);
  uint16_t* G = static_cast<uint16_t*>(p.g);
  float* part = p.part + (int64_t)blockIdx.x * 2 * nk;
  const float inv_nk = 1.0f / (float)nk;
  bool first = true;
  for (int64_t b = blockIdx.x; b < p.batch; b += gridDim.x) {
    // X and Z of the example into LDS (rows < n and < k; the padding stays zero)
    for (int c = tid; c < n * (D / 8); c += kFmThreads) {
      const int r = c / (D / 8), e = (c - r * (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Xs + r * XP + e) = *reinterpret_cast<const u32x4*>(X + (b * n + r) * D + e);
    }
    for (int c = tid; c < k * (D / 8); c += kFmThreads) {
      const int r = c / (D / 8), e = (c - r * (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Zs + r * XP + e) = *reinterpret_cast<const u32x4*>(Z + (b * k + r) * D + e);
    }
    __syncthreads();
    // F^T tiles: lane holds F[m = 16 mt + li][j = 16 jt + 4 lg + t]
    f32x4 facc[MPW][KJ];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int mt = wave + kFmWaves * i;
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        facc[i][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (16 * mt < n && 16 * jt < k) {  // wave-uniform
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks)
            facc[i][jt] = mfma16x16x32(row_frag(Zs, XP, 16 * jt, 32 * ks, li, lg),
                                       row_frag(Xs, XP, 16 * mt, 32 * ks, li, lg), facc[i][jt]);
        }
      }
    }
    auto valid = [&](int i, int jt) {
      const int m = 16 * (wave + kFmWaves * i) + li, j = 16 * jt + 4 * lg;
      return m < n && j < k;  // k % 4 == 0: the lane's 4 values are all valid or all not
    };
    // the FM LayerNorm's statistics over the n k values of the example
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MPW; ++i)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt)
        if (valid(i, jt)) s += (facc[i][jt][0] + facc[i][jt][1]) + (facc[i][jt][2] + facc[i][jt][3]);
    s = group_sum_v<64>(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kFmWaves; ++w) tot += red[w];
    const float mean = tot * inv_nk;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < MPW; ++i)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt)
        if (valid(i, jt))
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float dv = facc[i][jt][t] - mean;
            q += dv * dv;
          }
    q = group_sum_v<64>(q);
    if (lane == 0) red[kFmWaves + wave] = q;
    __syncthreads();
    float qt = 0.f;
#pragma unroll
    for (int w = 0; w < kFmWaves; ++w) qt += red[kFmWaves + w];
    const float rstd = rsqrtf(qt * inv_nk + p.eps);
    // d_Fn gamma_fm, and its two means
    u32x2 dfv[MPW][KJ];
    float sq = 0.f, sqf = 0.f;
#pragma unroll
    for (int i = 0; i < MPW; ++i)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        dfv[i][jt] = u32x2{0u, 0u};
        if (valid(i, jt)) {
          const int m = 16 * (wave + kFmWaves * i) + li, j = 16 * jt + 4 * lg;
          const u32x2 dv = *reinterpret_cast<const u32x2*>(DFN + b * nk + m * k + j);
          const u32x2 gv = GAM ? *reinterpret_cast<const u32x2*>(GAM + m * k + j) : u32x2{0x3f803f80u, 0x3f803f80u};
          dfv[i][jt] = dv;
          const float d4[4] = {bf16lo(dv[0]), bf16hi(dv[0]), bf16lo(dv[1]), bf16hi(dv[1])};
          const float g4[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float fh = (facc[i][jt][t] - mean) * rstd;
            const float qq = d4[t] * g4[t];
            facc[i][jt][t] = fh;  // from here on F_hat
            sq += qq;
            sqf += qq * fh;
          }
        }
      }
    sq = group_sum_v<64>(sq);
    sqf = group_sum_v<64>(sqf);
    if (lane == 0) {
      red[2 * kFmWaves + wave] = sq;
      red[3 * kFmWaves + wave] = sqf;
    }
    __syncthreads();
    float mq = 0.f, mqf = 0.f;
#pragma unroll
    for (int w = 0; w < kFmWaves; ++w) {
      mq += red[2 * kFmWaves + w];
      mqf += red[3 * kFmWaves + w];
    }
    mq *= inv_nk;
    mqf *= inv_nk;
    // dF = rstd (q - mean(q) - F_hat mean(q F_hat)) in bf16 to LDS; the gamma_fm / beta_fm
    // sums of this workgroup's examples (each (m, j) belongs to one lane of the workgroup)
#pragma unroll
    for (int i = 0; i < MPW; ++i)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt)
        if (valid(i, jt)) {
          const int m = 16 * (wave + kFmWaves * i) + li, j = 16 * jt + 4 * lg;
          const u32x2 dv = dfv[i][jt];
          const u32x2 gv = GAM ? *reinterpret_cast<const u32x2*>(GAM + m * k + j) : u32x2{0x3f803f80u, 0x3f803f80u};
          const float d4[4] = {bf16lo(dv[0]), bf16hi(dv[0]), bf16lo(dv[1]), bf16hi(dv[1])};
          const float g4[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
          float o[4];
          f32x4 pg, pb;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float fh = facc[i][jt][t];
            o[t] = rstd * (d4[t] * g4[t] - mq - fh * mqf);
            pg[t] = d4[t] * fh;
            pb[t] = d4[t];
          }
          *reinterpret_cast<u32x2*>(Fs + m * FP + j) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          f32x4* pgp = reinterpret_cast<f32x4*>(part + m * k + j);
          f32x4* pbp = reinterpret_cast<f32x4*>(part + nk + m * k + j);
          if (!first) {
            pg += *pgp;
            pb += *pbp;
          }
          *pgp = pg;
          *pbp = pb;
        }
    __syncthreads();
    // dZ = dF^T X: tiles (jt, et), lane holds dZ[16 jt + 4 lg + t][16 et + li]
    for (int tq = wave; tq < KJ * (D / 16); tq += kFmWaves) {
      const int jt = tq / (D / 16), et = tq - jt * (D / 16);
      if (16 * jt >= k) continue;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int m0 = 0; m0 < NP; m0 += 32)
        acc = mfma16x16x32(col_frag(Fs, FP, m0, 16 * jt, li, lg), col_frag(Xs, XP, m0, 16 * et, li, lg), acc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = 16 * jt + 4 * lg + t;
        if (j < k) G[(int64_t)j * p.ldg + b * D + 16 * et + li] = (uint16_t)f32_to_bf16(acc[t]);
      }
    }
    // dXa = dR + dF Z: tiles (mt, et), lane holds [16 mt + 4 lg + t][16 et + li]
    for (int tq = wave; tq < (NP / 16) * (D / 16); tq += kFmWaves) {
      const int mt = tq / (D / 16), et = tq - mt * (D / 16);
      if (16 * mt >= n) continue;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < KP; j0 += 32)
        acc = mfma16x16x32(row_frag(Fs, FP, 16 * mt, j0, li, lg), col_frag(Zs, XP, j0, 16 * et, li, lg), acc);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = 16 * mt + 4 * lg + t, e = 16 * et + li;
        if (m < n) {
          const uint16_t dr = m < n_f ? DM[(b * n_f + m) * D + e] : G[(int64_t)(k + m - n_f) * p.ldg + b * D + e];
          p.dxa[(b * n + m) * D + e] = acc[t] + bf(dr);
        }
      }
    }
    __syncthreads();  // LDS reused by the next example
    first = false;
  }
  if (first) {  // no example: the sums are zero
    for (int i = tid; i < 2 * nk; i += kFmThreads) part[i] = 0.f;
  }
}

// dst[r][b D + e] = src[b][r][e] (b < B), zero for columns B D .. ld - 1.
__global__ __launch_bounds__(256) void to_batch_major_kernel(const uint16_t* src, int64_t batch, int R, int D, int64_t ld,
                                                            uint16_t* dst) {
  const int64_t per_row = ld / 8;
  const int64_t total = (int64_t)R * per_row;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int r = (int)(q / per_row);
    const int64_t c = (q - (int64_t)r * per_row) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (c < batch * D) {
      const int64_t b = c / D;
      const int e = (int)(c - b * D);
      v = *reinterpret_cast<const u32x4*>(src + (b * R + r) * D + e);
    }
    *reinterpret_cast<u32x4*>(dst + (int64_t)r * ld + c) = v;
  }
}

// zero columns c0 .. ld - 1 of rows 0 .. R - 1 ((ld - c0) % 8 == 0)
__global__ __launch_bounds__(256) void zero_cols_kernel(uint16_t* p, int R, int64_t ld, int64_t c0) {
  const int64_t per_row = (ld - c0) / 8;
  const int64_t total = (int64_t)R * per_row;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int r = (int)(q / per_row);
    const int64_t c = c0 + (q - (int64_t)r * per_row) * 8;
    *reinterpret_cast<u32x4*>(p + (int64_t)r * ld + c) = u32x4{0u, 0u, 0u, 0u};
  }
}

// dX[b][j][e] = bf16(dXa[b][j][e] + C[j][b D + e]), 4 elements per thread
__global__ __launch_bounds__(256) void dx_final_kernel(const float* dxa, const float* c, int64_t ldc, int64_t batch,
                                                      int n, int D, uint16_t* dx) {
  const int64_t total = batch * n * D / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t i = q * 4;
    const int64_t row = i / D;
    const int e = (int)(i - row * D);
    const int64_t b = row / n;
    const int j = (int)(row - b * n);
    const f32x4 a = *reinterpret_cast<const f32x4*>(dxa + i);
    const f32x4 g = *reinterpret_cast<const f32x4*>(c + (int64_t)j * ldc + b * D + e);
    *reinterpret_cast<u32x2*>(dx + i) = u32x2{pack_bf16x2(a[0] + g[0], a[1] + g[1]), pack_bf16x2(a[2] + g[2], a[3] + g[3])};
  }
}

template <class K>
hipError_t allow_lds_w(K* kern) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMaxW);
}

struct FmVariant {
  int d, mpw, kj;
  void (*kernel)(BwdFmWideArgs);
};
const FmVariant kFmVariants[] = {
    {160, 2, 4, bwd_fm_wide_kernel<160, 2, 4>},  // n <= 256, k <= 64 at d = 160
    {32, 6, 2, bwd_fm_wide_kernel<32, 6, 2>},    // n <= 768, k <= 32 at d = 32
    {64, 3, 2, bwd_fm_wide_kernel<64, 3, 2>},    // n <= 384, k <= 32 at d = 64
};

const FmVariant* pick_fm(int n, int d, int k) {
  for (const auto& v : kFmVariants) {
    if (v.d != d || (n + 15) / 16 > kFmWaves * v.mpw || (k + 15) / 16 > v.kj) continue;
    if (fm_lds(n, d, k).bytes > (size_t)kLdsMaxW) continue;
    return &v;
  }
  return nullptr;
}

int rows_lpr(int d) {
  const int c = d / 8;
  for (int l = 8; l >= 1; l >>= 1)
    if (c % l == 0) return l;
  return 1;
}

}  // namespace

bool wukong_bwd_wide_supported(int n, int d, int k, int n_l) {
  (void)n_l;
  return d % 8 == 0 && k % 4 == 0 && (d == 32 || d == 64 || d == 160) && pick_fm(n, d, k) != nullptr;
}

hipError_t launch_bwd_rows(const BwdRowsArgs& a, int grid, hipStream_t stream, int64_t* workgroups) {
  if (workgroups) *workgroups = grid;
  if (grid <= 0) return hipSuccess;
  const int lpr = rows_lpr(a.d);
  switch (a.d * 16 + lpr) {
    case 32 * 16 + 4: hipLaunchKernelGGL((bwd_rows_kernel<32, 4>), dim3(grid), dim3(kRowThreads), 0, stream, a); break;
    case 64 * 16 + 8: hipLaunchKernelGGL((bwd_rows_kernel<64, 8>), dim3(grid), dim3(kRowThreads), 0, stream, a); break;
    case 160 * 16 + 4: hipLaunchKernelGGL((bwd_rows_kernel<160, 4>), dim3(grid), dim3(kRowThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_fm_wide(const BwdFmWideArgs& a, int grid, hipStream_t stream, int64_t* workgroups) {
  const FmVariant* v = pick_fm(a.n, a.d, a.k);
  if (!v || a.k % 4 != 0) return hipErrorInvalidValue;
  if (workgroups) *workgroups = grid;
  if (grid <= 0) return hipSuccess;
  const hipError_t e = allow_lds_w(v->kernel);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v->kernel, dim3(grid), dim3(kFmThreads), fm_lds(a.n, a.d, a.k).bytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_to_batch_major(const void* src, int64_t batch, int R, int D, int64_t ld, void* dst,
                                 hipStream_t stream) {
  if (D % 8 || ld % 8 || ld < batch * D) return hipErrorInvalidValue;
  int64_t grid = ((int64_t)R * (ld / 8) + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(to_batch_major_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), batch, R, D, ld, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_zero_cols(void* p, int R, int64_t ld, int64_t c0, hipStream_t stream) {
  if ((ld - c0) % 8 || c0 % 8) return hipErrorInvalidValue;
  int64_t grid = ((int64_t)R * ((ld - c0) / 8) + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_cols_kernel, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<uint16_t*>(p), R, ld, c0);
  return hipGetLastError();
}

hipError_t launch_dx_final(const float* dxa, const float* c, int64_t ldc, int64_t batch, int n, int D, void* dx,
                           hipStream_t stream, int64_t* workgroups) {
  if (D % 4) return hipErrorInvalidValue;
  int64_t grid = (batch * n * D / 4 + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (workgroups) *workgroups = grid;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(dx_final_kernel, dim3((unsigned)grid), dim3(256), 0, stream, dxa, c, ldc, batch, n, D,
                     static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

}  // namespace wk
