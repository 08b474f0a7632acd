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
//  bwd_fm_wide_kernel, per example, X streamed through LDS in row chunks (twice)
//    with the saved Z in LDS: F = X Z^T with MFMA, the FM LayerNorm's statistics
//    and input gradient dF (bf16), dZ = dF^T X (bf16, to rows 0 .. k - 1 of G)
//    and dXa = dR + dF Z (fp32); per-workgroup sums of d_Fn F_hat and d_Fn
//    (gamma_fm / beta_fm).
//  Then, on the GEMM kernels: d[Phi; W_L] = G X'^T with X' the batch-major
//  copy of X (split along the batch), and C = [Phi; W_L]^T G, whose epilogue
//  forms dX = bf16(dXa + C) (C's columns are (example, embedding) pairs).
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

// Rows of X walk through LDS in chunks of kChunk (one 16-row tile per wave), twice per
// example: pass 1 forms F chunk by chunk and gathers the FM LayerNorm's sums (Chan's
// parallel combination for the variance), pass 2 forms F again, dF, dZ += dF^T X and
// dR + dF Z for the chunk.  So any n fits; LDS holds Z, one chunk of X and of dF.
constexpr int kChunk = 16 * kFmWaves;

struct FmLds {
  int kp, xp, fp;  // k rounded up to 32, pitches (u16) of the X / Z rows and of the dF rows
  size_t zs, xs, fs, red, sums, bytes;
};
__host__ __device__ inline FmLds fm_lds(int n, int d, int k, bool sums_in_lds = false) {
  FmLds L;
  L.kp = (k + 31) / 32 * 32;
  L.xp = d + 8;
  L.fp = L.kp + 8;
  L.zs = 0;
  L.xs = L.zs + (size_t)L.kp * L.xp * 2;
  L.fs = L.xs + (size_t)kChunk * L.xp * 2;
  L.red = L.fs + (size_t)kChunk * L.fp * 2;
  L.sums = L.red + 8 * kFmWaves * sizeof(float);
  L.bytes = L.sums + (sums_in_lds ? (size_t)2 * n * k * sizeof(float) : 0);
  return L;
}

// D: embedding width; KJ: 16-column tiles of k; DZW: dZ tiles (of KJ x D/16) per wave.
// The workgroup's gamma_fm / beta_fm sums over its examples (each lane owns the same
// (m, j) in every example): NCH > 0: at most NCH row chunks, the sums in registers;
// NCH = -1: in LDS after the other arrays (fm_lds(.., true)); NCH = 0: read-modify-
// written in the workgroup's plane in global memory.
template <int D, int KJ, int NCH>
__global__ __launch_bounds__(kFmThreads) void bwd_fm_wide_kernel(BwdFmWideArgs p) {
  constexpr int ET = D / 16;
  constexpr int DZW = (KJ * ET + kFmWaves - 1) / kFmWaves;
  extern __shared__ __align__(16) unsigned char smem[];
  const int n = p.n, k = p.k, n_f = p.n_f;
  const FmLds L = fm_lds(n, D, k, NCH < 0);
  uint16_t* Zs = reinterpret_cast<uint16_t*>(smem + L.zs);
  uint16_t* Xs = reinterpret_cast<uint16_t*>(smem + L.xs);
  uint16_t* Fs = reinterpret_cast<uint16_t*>(smem + L.fs);
  float* red = reinterpret_cast<float*>(smem + L.red);
  float* Ss = reinterpret_cast<float*>(smem + L.sums);  // NCH < 0: the gamma_fm / beta_fm sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int XP = L.xp, FP = L.fp, KP = L.kp;
  const int nk = n * k;
  const int chunks = (n + kChunk - 1) / kChunk;
  // zero once: the padding rows of Z and the padding columns of dF stay zero (and the sums start at 0)
  for (int i = tid; i < (int)(L.bytes / 2); i += kFmThreads) reinterpret_cast<uint16_t*>(smem)[i] = 0;
  __syncthreads();
  const uint16_t* X = static_cast<const uint16_t*>(p.x);
  const uint16_t* Z = static_cast<const uint16_t*>(p.z);
  const uint16_t* DFN = static_cast<const uint16_t*>(p.dfn);
  const uint16_t* GAM = static_cast<const uint16_t*>(p.fm_gamma);
  const uint16_t* DM = static_cast<const uint16_t*>(p.dm);
  uint16_t* G = static_cast<uint16_t*>(p.g);
  float* part = p.part + (int64_t)blockIdx.x * 2 * nk;
  const float fnk = (float)nk;
  bool first = true;
  constexpr int NC = NCH > 0 ? NCH : 1;
  f32x4 psg[NC][KJ], psb[NC][KJ];  // used when NCH > 0
  if constexpr (NCH > 0) {
#pragma unroll
    for (int ch = 0; ch < NC; ++ch)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) psg[ch][jt] = psb[ch][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // X rows c0 .. c0 + kChunk - 1 of example b into Xs (rows past n as zero)
  auto load_chunk = [&](int64_t b, int c0) {
    for (int c = tid; c < kChunk * (D / 8); c += kFmThreads) {
      const int r = c / (D / 8), e = (c - r * (D / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (c0 + r < n) v = *reinterpret_cast<const u32x4*>(X + (b * n + c0 + r) * D + e);
      *reinterpret_cast<u32x4*>(Xs + r * XP + e) = v;
    }
  };
  // this wave's F tile row of the chunk: lane holds F[m = c0 + 16 wave + li][j = 16 jt + 4 lg + t]
  auto f_tiles = [&](f32x4 (&f)[KJ]) {
#pragma unroll
    for (int jt = 0; jt < KJ; ++jt) {
      f[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (16 * jt >= k) continue;  // uniform: columns past k
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        f[jt] = mfma16x16x32(row_frag(Zs, XP, 16 * jt, 32 * ks, li, lg), row_frag(Xs, XP, 16 * wave, 32 * ks, li, lg),
                             f[jt]);
    }
  };
  for (int64_t b = blockIdx.x; b < p.batch; b += gridDim.x) {
    __syncthreads();  // the previous example's reads of Z are done
    for (int c = tid; c < k * (D / 8); c += kFmThreads) {
      const int r = c / (D / 8), e = (c - r * (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Zs + r * XP + e) = *reinterpret_cast<const u32x4*>(Z + (b * k + r) * D + e);
    }
    // ---- pass 1: per-lane count, mean and M2 of F (Chan), and the sums of q = d_Fn gamma_fm and q F
    float cnt = 0.f, mu = 0.f, m2 = 0.f, sq = 0.f, sqf = 0.f;
    for (int ch = 0; ch < chunks; ++ch) {
      const int c0 = ch * kChunk;
      __syncthreads();  // the previous chunk's (and example's) reads are done
      load_chunk(b, c0);
      __syncthreads();
      f32x4 f[KJ];
      f_tiles(f);
      const int m = c0 + 16 * wave + li;
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        const int j = 16 * jt + 4 * lg;
        if (m < n && j < k) {  // k % 4 == 0: the lane's 4 values are all valid or all not
          const u32x2 dv = *reinterpret_cast<const u32x2*>(DFN + b * nk + m * k + j);
          const u32x2 gv = GAM ? *reinterpret_cast<const u32x2*>(GAM + m * k + j) : u32x2{0x3f803f80u, 0x3f803f80u};
          const float d4[4] = {bf16lo(dv[0]), bf16hi(dv[0]), bf16lo(dv[1]), bf16hi(dv[1])};
          const float g4[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float v = f[jt][t];
            cnt += 1.f;
            const float dl = v - mu;
            mu += dl / cnt;
            m2 += dl * (v - mu);
            const float q = d4[t] * g4[t];
            sq += q;
            sqf += q * v;
          }
        }
      }
    }
    // combine (count, mean, M2) over the lanes of the wave, then over the waves
    auto chan = [&](float& c1, float& m1, float& s1, float c2, float mean2, float s2) {
      const float c = c1 + c2;
      if (c > 0.f) {
        const float dl = mean2 - m1;
        m1 += dl * (c2 / c);
        s1 += s2 + dl * dl * (c1 * c2 / c);
      }
      c1 = c;
    };
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float c2 = __shfl_xor(cnt, off, kWave), mean2 = __shfl_xor(mu, off, kWave), s2 = __shfl_xor(m2, off, kWave);
      chan(cnt, mu, m2, c2, mean2, s2);
    }
    sq = group_sum_v<64>(sq);
    sqf = group_sum_v<64>(sqf);
    if (lane == 0) {
      red[wave] = cnt;
      red[kFmWaves + wave] = mu;
      red[2 * kFmWaves + wave] = m2;
      red[3 * kFmWaves + wave] = sq;
      red[4 * kFmWaves + wave] = sqf;
    }
    __syncthreads();
    float tc = 0.f, tmu = 0.f, tm2 = 0.f, tq = 0.f, tqf = 0.f;
#pragma unroll
    for (int w = 0; w < kFmWaves; ++w) {
      chan(tc, tmu, tm2, red[w], red[kFmWaves + w], red[2 * kFmWaves + w]);
      tq += red[3 * kFmWaves + w];
      tqf += red[4 * kFmWaves + w];
    }
    const float rstd = rsqrtf(tm2 / fnk + p.eps);
    const float mq = tq / fnk;                         // mean of q
    const float mqf = rstd * (tqf - tmu * tq) / fnk;   // mean of q F_hat
    // ---- pass 2: F again, dF (bf16) to LDS, dZ += dF^T X, dR + dF Z
    f32x4 dz[DZW];
#pragma unroll
    for (int i = 0; i < DZW; ++i) dz[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto pass2 = [&](int ch, f32x4 (&pgs)[KJ], f32x4 (&pbs)[KJ]) {
      const int c0 = ch * kChunk;
      __syncthreads();
      load_chunk(b, c0);
      __syncthreads();
      f32x4 f[KJ];
      f_tiles(f);
      const int m = c0 + 16 * wave + li;
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        const int j = 16 * jt + 4 * lg;
        u32x2 o = u32x2{0u, 0u};
        if (m < n && j < k) {
          const u32x2 dv = *reinterpret_cast<const u32x2*>(DFN + b * nk + m * k + j);
          const u32x2 gv = GAM ? *reinterpret_cast<const u32x2*>(GAM + m * k + j) : u32x2{0x3f803f80u, 0x3f803f80u};
          const float d4[4] = {bf16lo(dv[0]), bf16hi(dv[0]), bf16lo(dv[1]), bf16hi(dv[1])};
          const float g4[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
          float df[4];
          f32x4 pg, pb;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float fh = (f[jt][t] - tmu) * rstd;
            df[t] = rstd * (d4[t] * g4[t] - mq - fh * mqf);
            pg[t] = d4[t] * fh;
            pb[t] = d4[t];
          }
          o = u32x2{pack_bf16x2(df[0], df[1]), pack_bf16x2(df[2], df[3])};
          // this workgroup's gamma_fm / beta_fm sums: each (m, j) belongs to one lane
          if constexpr (NCH > 0) {
            pgs[jt] += pg;
            pbs[jt] += pb;
          } else if constexpr (NCH < 0) {
            f32x4* sg = reinterpret_cast<f32x4*>(Ss + m * k + j);
            f32x4* sb = reinterpret_cast<f32x4*>(Ss + nk + m * k + j);
            *sg += pg;
            *sb += pb;
          } else {
            f32x4* pgp = reinterpret_cast<f32x4*>(part + m * k + j);
            f32x4* pbp = reinterpret_cast<f32x4*>(part + nk + m * k + j);
            if (!first) {
              pg += *pgp;
              pb += *pbp;
            }
            *pgp = pg;
            *pbp = pb;
          }
        }
        if (j < KP) *reinterpret_cast<u32x2*>(Fs + (16 * wave + li) * FP + j) = o;  // rows past n: zero
      }
      __syncthreads();
      // dZ tiles (jt, et) owned by this wave: + dF_chunk^T X_chunk over the chunk's rows
#pragma unroll
      for (int i = 0; i < DZW; ++i) {
        const int tq2 = wave + kFmWaves * i;
        if (tq2 < KJ * ET && 16 * (tq2 / ET) < k) {  // wave-uniform
          const int jt = tq2 / ET, et = tq2 - jt * ET;
#pragma unroll
          for (int m0 = 0; m0 < kChunk; m0 += 32)
            dz[i] = mfma16x16x32(col_frag(Fs, FP, m0, 16 * jt, li, lg), col_frag(Xs, XP, m0, 16 * et, li, lg), dz[i]);
        }
      }
      // dR + dF Z for the chunk's rows: tiles (this wave's row tile, et)
      if (c0 + 16 * wave < n) {  // wave-uniform
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int j0 = 0; j0 < KP; j0 += 32)
            acc = mfma16x16x32(row_frag(Fs, FP, 16 * wave, j0, li, lg), col_frag(Zs, XP, j0, 16 * et, li, lg), acc);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int mm = c0 + 16 * wave + 4 * lg + t, e = 16 * et + li;
            if (mm < n) {
              const uint16_t dr =
                  mm < n_f ? DM[(b * n_f + mm) * D + e] : G[(int64_t)(k + mm - n_f) * p.ldg + b * D + e];
              p.dxa[(b * n + mm) * D + e] = acc[t] + bf(dr);
            }
          }
        }
      }
    };
    if constexpr (NCH > 0) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
        if (ch < chunks) pass2(ch, psg[ch], psb[ch]);
    } else {
      f32x4 unused[KJ];
      for (int ch = 0; ch < chunks; ++ch) pass2(ch, unused, unused);
    }
    // dZ (bf16) to its rows of G: lane holds dZ[16 jt + 4 lg + t][16 et + li]
#pragma unroll
    for (int i = 0; i < DZW; ++i) {
      const int tq2 = wave + kFmWaves * i;
      if (tq2 < KJ * ET) {
        const int jt = tq2 / ET, et = tq2 - jt * ET;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = 16 * jt + 4 * lg + t;
          if (j < k) G[(int64_t)j * p.ldg + b * D + 16 * et + li] = (uint16_t)f32_to_bf16(dz[i][t]);
        }
      }
    }
    first = false;
  }
  if constexpr (NCH > 0) {  // the register sums to the plane (zero if the workgroup had no example)
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int m = ch * kChunk + 16 * wave + li;
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        const int j = 16 * jt + 4 * lg;
        if (ch < chunks && m < n && j < k) {
          *reinterpret_cast<f32x4*>(part + m * k + j) = psg[ch][jt];
          *reinterpret_cast<f32x4*>(part + nk + m * k + j) = psb[ch][jt];
        }
      }
    }
  } else if constexpr (NCH < 0) {
    __syncthreads();
    for (int i = tid; i < 2 * nk; i += kFmThreads) part[i] = Ss[i];
  } else if (first) {  // no example: the sums are zero
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

template <class K>
hipError_t allow_lds_w(K* kern) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMaxW);
}

struct FmVariant {
  int d, kj, nch;
  void (*kernel)(BwdFmWideArgs);
};
const FmVariant kFmVariants[] = {
    {160, 3, 2, bwd_fm_wide_kernel<160, 3, 2>},    // d = 160, k <= 48, n <= 256: sums in registers
    {160, 3, 0, bwd_fm_wide_kernel<160, 3, 0>},    // d = 160, k <= 48
    {160, 6, 0, bwd_fm_wide_kernel<160, 6, 0>},    // d = 160, k <= 96
    {32, 2, -1, bwd_fm_wide_kernel<32, 2, -1>},    // d = 32, k <= 32: sums in LDS when they fit
    {32, 2, 0, bwd_fm_wide_kernel<32, 2, 0>},      // d = 32, k <= 32
    {64, 2, -1, bwd_fm_wide_kernel<64, 2, -1>},    // d = 64, k <= 32: sums in LDS when they fit
    {64, 2, 0, bwd_fm_wide_kernel<64, 2, 0>},      // d = 64, k <= 32
};

const FmVariant* pick_fm(int n, int d, int k) {
  for (const auto& v : kFmVariants) {
    if (v.d != d || (k + 15) / 16 > v.kj) continue;
    if (v.nch > 0 && (n + kChunk - 1) / kChunk > v.nch) continue;
    if (fm_lds(n, d, k, v.nch < 0).bytes > (size_t)kLdsMaxW) continue;
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
  hipLaunchKernelGGL(v->kernel, dim3(grid), dim3(kFmThreads), fm_lds(a.n, a.d, a.k, v->nch < 0).bytes, stream, a);
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


}  // namespace wk
