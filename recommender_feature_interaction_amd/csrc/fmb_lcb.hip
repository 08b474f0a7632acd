// FMB + LCB kernel of the Wukong layer (bf16 storage, fp32 accumulation).
//
// One workgroup per example b.  Wukong paper, section 2.2 (xdnf.cn repost):
// the FMB compresses the n embeddings to k before interacting them, and the
// LCB multiplies X by W_L; both act on the same X, so one pass over X_b
// serves both:
//
//   phase 1   [Z; Lc] = [Phi; W_L] X_b           ((k + n_L) x d, MFMA)
//             X_b is streamed through LDS in chunks of MC rows, transposed
//             on the way in so that the contraction index m is contiguous
//             for the MFMA operand; the weight rows [Phi; W_L] are read
//             straight from global memory (they are shared by every example
//             and stay resident in L2).  Wave w owns the 16-row tiles
//             w, w + NW, ... of [Phi; W_L] across the whole width d.
//   LCB rows  Y_b[n_F + i] = LN_d(Lc[i] + X_b[n_F + i]) finished in
//             registers: a row's d values sit in the 4 lanes l, l^16, l^32,
//             l^48 of one wave, so its statistics are two xor-shuffles.
//   phase 2   F_b = X_b Z_b^T (n x k, MFMA): Z_b (bf16) goes through LDS,
//             X_b rows are re-read from global memory (an L2 hit) in the
//             natural layout, which is the operand layout this product needs.
//   LN(F)     mean and variance over all n*k values (wave shuffles + LDS),
//             then Fn_b = bf16(LN(vec(F_b))) written row-major.
//
// MFMA used: v_mfma_f32_16x16x32_bf16 (16-row tiles keep the padding of the
// irregular k, n_L and n small).
#include <atomic>
#include <mutex>

#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

template <int ET, int NW, int ZW, int MW, int KW, int MC>
__global__ __launch_bounds__(NW * 64) void fmb_lcb_bf16_kernel(FmbLcbArgs p) {
  constexpr int D = 16 * ET;
  constexpr int XT_LD = MC + 8;          // LDS row pitch of X^T (u16), padded against bank conflicts
  constexpr int DZ = (D + 31) / 32 * 32; // d rounded up to the 32-wide K step of phase 2
  constexpr int Z_LD = DZ + 8;
  constexpr int NT = NW * 64;
  constexpr int MB = MC / 8;
  constexpr int EB = D / 8;
  constexpr int NBLK = MB * EB;          // 8x8 transpose blocks per chunk
  constexpr int BPT = (NBLK + NT - 1) / NT;
  constexpr int KS = MC / 32;
  constexpr bool EB_FAST = (EB < 8);     // narrow rows: let consecutive lanes walk along a row

  extern __shared__ __align__(16) uint16_t smem[];
  __shared__ float red[2 * NW];
  uint16_t* XT = smem;
  uint16_t* Zs = smem;  // reused once phase 1 is done

  const int n = p.n, k = p.k, n_l = p.n_l, n_f = p.n_f;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const uint16_t* xb = p.x + b * (int64_t)n * D;
  const int ZT = (k + n_l + 15) >> 4;

  // ------------------------------------------------------------- phase 1
  const uint16_t* wrow[ZW];
#pragma unroll
  for (int zi = 0; zi < ZW; ++zi) {
    const int zt = wave + zi * NW;
    const int z = zt * 16 + li;
    const uint16_t* r = nullptr;
    if (zt < ZT) {
      if (z < k)
        r = p.phi + (int64_t)z * n;
      else if (z < k + n_l)
        r = p.w_l + (int64_t)(z - k) * n;
    }
    wrow[zi] = r;
  }
  f32x4 acc[ZW][ET];
#pragma unroll
  for (int zi = 0; zi < ZW; ++zi)
#pragma unroll
    for (int et = 0; et < ET; ++et) acc[zi][et] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xr[BPT][8];
  auto load_chunk = [&](int m0) {
#pragma unroll
    for (int bi = 0; bi < BPT; ++bi) {
      const int blk = tid + bi * NT;
      const int mb = EB_FAST ? blk / EB : blk % MB;
      const int eb = EB_FAST ? blk % EB : blk / MB;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int m = m0 + mb * 8 + r;
        if (blk < NBLK && m < n)
          xr[bi][r] = *reinterpret_cast<const u32x4*>(xb + (int64_t)m * D + eb * 8);
        else
          xr[bi][r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int bi = 0; bi < BPT; ++bi) {
      const int blk = tid + bi * NT;
      if (blk < NBLK) {
        const int mb = EB_FAST ? blk / EB : blk % MB;
        const int eb = EB_FAST ? blk % EB : blk / MB;
        // 8x8 transpose: output row e = 8eb + c holds the 8 values of column c.
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = xr[bi][2 * q][c >> 1];
            const uint32_t hi = xr[bi][2 * q + 1][c >> 1];
            o[q] = (c & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
          }
          *reinterpret_cast<u32x4*>(XT + (eb * 8 + c) * XT_LD + mb * 8) = o;
        }
      }
    }
  };

  const int nchunks = (n + MC - 1) / MC;
  load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    const int m0 = c * MC;
    u32x4 wf[ZW][KS];
#pragma unroll
    for (int zi = 0; zi < ZW; ++zi)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int mk = m0 + ks * 32 + lg * 8;
        if (wrow[zi] != nullptr && mk < n)
          wf[zi][ks] = *reinterpret_cast<const u32x4*>(wrow[zi] + mk);
        else
          wf[zi][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    lds_barrier();  // everyone is done reading the previous chunk
    store_chunk();
    if (c + 1 < nchunks) load_chunk(m0 + MC);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (m0 + ks * 32 < n) {
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(XT + (et * 16 + li) * XT_LD + ks * 32 + lg * 8);
#pragma unroll
          for (int zi = 0; zi < ZW; ++zi)
            if (wave + zi * NW < ZT) acc[zi][et] = mfma16x16x32(a, wf[zi][ks], acc[zi][et]);
        }
      }
    }
  }
  lds_barrier();  // X^T no longer needed: its LDS becomes Z

  // Z rows -> LDS as bf16 (the phase-2 operand); padding rows/columns are zero.
  for (int i = tid; i < 16 * KW * Z_LD / 8; i += NT)
    reinterpret_cast<u32x4*>(Zs)[i] = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();

  const uint16_t* og = p.out_gamma;
  const uint16_t* ob = p.out_beta;
  const float inv_d = 1.0f / static_cast<float>(D);
#pragma unroll
  for (int zi = 0; zi < ZW; ++zi) {
    const int zt = wave + zi * NW;
    if (zt >= ZT) continue;  // wave-uniform
    const int z = zt * 16 + li;
    if (z < k) {
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[zi][et][0], acc[zi][et][1]);
        v[1] = pack_bf16x2(acc[zi][et][2], acc[zi][et][3]);
        *reinterpret_cast<u32x2*>(Zs + z * Z_LD + et * 16 + lg * 4) = v;
      }
    }
    // LCB rows of this tile: Y[n_F + i] = LN_d(Lc[i] + X[n_F + i])
    if (zt * 16 + 15 >= k && zt * 16 < k + n_l) {  // wave-uniform
      const bool is_l = (z >= k) && (z < k + n_l);
      const int row = n_f + (z - k);
      float v[ET][4];
      float s = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        u32x2 xv = u32x2{0u, 0u};
        if (is_l) xv = *reinterpret_cast<const u32x2*>(xb + (int64_t)row * D + et * 16 + lg * 4);
        v[et][0] = acc[zi][et][0] + bf16lo(xv[0]);
        v[et][1] = acc[zi][et][1] + bf16hi(xv[0]);
        v[et][2] = acc[zi][et][2] + bf16lo(xv[1]);
        v[et][3] = acc[zi][et][3] + bf16hi(xv[1]);
        s += (v[et][0] + v[et][1]) + (v[et][2] + v[et][3]);
      }
      s = xor_sum<16>(s);
      const float mean = s * inv_d;
      float q = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float dv = v[et][t] - mean;
          q += dv * dv;
        }
      q = xor_sum<16>(q);
      const float rstd = rsqrtf(q * inv_d + p.eps);
      if (is_l) {
        uint16_t* yrow = p.y + (b * n + row) * (int64_t)D;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + lg * 4;
          float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
          if (og) {
            const u32x2 g2 = *reinterpret_cast<const u32x2*>(og + e);
            gm[0] = bf16lo(g2[0]); gm[1] = bf16hi(g2[0]); gm[2] = bf16lo(g2[1]); gm[3] = bf16hi(g2[1]);
          }
          if (ob) {
            const u32x2 b2 = *reinterpret_cast<const u32x2*>(ob + e);
            bt[0] = bf16lo(b2[0]); bt[1] = bf16hi(b2[0]); bt[2] = bf16lo(b2[1]); bt[3] = bf16hi(b2[1]);
          }
          u32x2 o;
          o[0] = pack_bf16x2((v[et][0] - mean) * rstd * gm[0] + bt[0], (v[et][1] - mean) * rstd * gm[1] + bt[1]);
          o[1] = pack_bf16x2((v[et][2] - mean) * rstd * gm[2] + bt[2], (v[et][3] - mean) * rstd * gm[3] + bt[3]);
          *reinterpret_cast<u32x2*>(yrow + e) = o;
        }
      }
    }
  }
  lds_barrier();  // Z complete in LDS

  // ------------------------------------------------------------- phase 2
  const int MT = (n + 15) >> 4;
  const int KT = (k + 15) >> 4;
  f32x4 facc[MW][KW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int jt = 0; jt < KW; ++jt) facc[mi][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    const int mt = wave + mi * NW;
    if (mt < MT) {  // wave-uniform
      const int m = mt * 16 + li;
#pragma unroll
      for (int ks = 0; ks < DZ / 32; ++ks) {
        const int e0 = ks * 32 + lg * 8;
        u32x4 xf = u32x4{0u, 0u, 0u, 0u};
        if (m < n && e0 < D) xf = *reinterpret_cast<const u32x4*>(xb + (int64_t)m * D + e0);
#pragma unroll
        for (int jt = 0; jt < KW; ++jt) {
          if (jt < KT) {
            const u32x4 zf = *reinterpret_cast<const u32x4*>(Zs + (jt * 16 + li) * Z_LD + e0);
            facc[mi][jt] = mfma16x16x32(zf, xf, facc[mi][jt]);
          }
        }
      }
    }
  }

  // LN over the n*k values of F (facc[mi][jt][t] = F[16mt + li][16jt + 4lg + t])
  float s = 0.f;
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int jt = 0; jt < KW; ++jt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = (wave + mi * NW) * 16 + li;
        const int j = jt * 16 + lg * 4 + t;
        if (m < n && j < k) s += facc[mi][jt][t];
      }
  s = group_sum_v<64>(s);
  if (lane == 0) red[wave] = s;
  lds_barrier();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += red[w];
  const float inv_nk = 1.0f / static_cast<float>(n * k);
  const float mean = tot * inv_nk;
  float q = 0.f;
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int jt = 0; jt < KW; ++jt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = (wave + mi * NW) * 16 + li;
        const int j = jt * 16 + lg * 4 + t;
        if (m < n && j < k) {
          const float dv = facc[mi][jt][t] - mean;
          q += dv * dv;
        }
      }
  q = group_sum_v<64>(q);
  if (lane == 0) red[NW + wave] = q;
  lds_barrier();
  float qt = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) qt += red[NW + w];
  const float rstd = rsqrtf(qt * inv_nk + p.eps);

  uint16_t* fnb = p.fn + b * (int64_t)n * k;
#pragma unroll
  for (int mi = 0; mi < MW; ++mi)
#pragma unroll
    for (int jt = 0; jt < KW; ++jt) {
      const int m = (wave + mi * NW) * 16 + li;
      const int j0 = jt * 16 + lg * 4;
      if (m < n && j0 < k) {  // k % 4 == 0: the 4 values j0..j0+3 are all valid
        const int idx = m * k + j0;
        float gm[4] = {1.f, 1.f, 1.f, 1.f}, bt[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.fm_gamma) {
          const u32x2 g2 = *reinterpret_cast<const u32x2*>(p.fm_gamma + idx);
          gm[0] = bf16lo(g2[0]); gm[1] = bf16hi(g2[0]); gm[2] = bf16lo(g2[1]); gm[3] = bf16hi(g2[1]);
        }
        if (p.fm_beta) {
          const u32x2 b2 = *reinterpret_cast<const u32x2*>(p.fm_beta + idx);
          bt[0] = bf16lo(b2[0]); bt[1] = bf16hi(b2[0]); bt[2] = bf16lo(b2[1]); bt[3] = bf16hi(b2[1]);
        }
        const f32x4 f = facc[mi][jt];
        u32x2 o;
        o[0] = pack_bf16x2((f[0] - mean) * rstd * gm[0] + bt[0], (f[1] - mean) * rstd * gm[1] + bt[1]);
        o[1] = pack_bf16x2((f[2] - mean) * rstd * gm[2] + bt[2], (f[3] - mean) * rstd * gm[3] + bt[3]);
        *reinterpret_cast<u32x2*>(fnb + idx) = o;
      }
    }
}

// ---------------------------------------------------------------------------
// Resident variant: X_b lives in LDS in its natural row-major layout (row pitch
// Q 16-byte chunks, Q = d/8 + 1 odd, which spreads 16 consecutive rows over all
// banks), and each workgroup walks several examples.  The next example's X is
// loaded into registers while the current one is computed, then written to LDS
// between examples, so the HBM stream never waits on the compute.
//   phase 1  the K-major operand X^T (rows e, contraction m) is read with
//            ds_read_b64_tr_b16: in each 16-lane group, lane i receives value
//            i%4 of the 8-byte rows addressed by lanes 4k + i/4 (k = 0..3), so
//            if lane s points at X[m + s/4][e0 + 4(s%4)] lane i gets
//            X[m + k][e0 + i]: two such reads give the 8 consecutive m a
//            16x16x32 operand needs.
//   phase 2  X rows are read as 16-byte vectors from the same LDS copy.
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define WK_LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4*)(p))

__device__ __forceinline__ u32x4 tr_operand(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WK_LDS_I16X4(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WK_LDS_I16X4(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

template <int ET, int NW, int ZW, int MW, int KW, int NMAX, bool WL>
__global__ __launch_bounds__(NW * 64, 2) void fmb_lcb_resident_kernel(FmbLcbArgs p, int64_t batch) {
  constexpr int D = 16 * ET;
  constexpr int EB = D / 8;              // 16-byte chunks per row
  constexpr int Q = EB + 1;              // LDS row pitch in chunks (odd)
  constexpr int P = Q * 8;               // LDS row pitch in u16
  constexpr int NROWS = (NMAX + 31) / 32 * 32;
  constexpr int DZ = (D + 31) / 32 * 32;
  constexpr int Z_LD = DZ + 8;
  constexpr int NT = NW * 64;
  constexpr int CPT = (NMAX * EB + NT - 1) / NT;  // X chunks per thread
  constexpr int WP = NROWS + 8;          // LDS pitch of the [Phi; W_L] rows (u16); WP/8 is odd
  extern __shared__ __align__(16) uint16_t smem[];
  __shared__ float red[2 * NW];
  uint16_t* Xs = smem;                   // [NROWS][P]
  uint16_t* Zs = smem + NROWS * P;       // [16 KW][Z_LD]
  uint16_t* Gs = Zs + 16 * KW * Z_LD;    // out LayerNorm gamma [D] then beta [D] (bf16)
  uint16_t* Ws = Gs + 2 * D;             // [16 ZT][WP] when WL

  const int n = p.n, k = p.k, n_l = p.n_l, n_f = p.n_f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int ZT = (k + n_l + 15) >> 4;
  const int MT = (n + 15) >> 4;
  const int KT = (k + 15) >> 4;
  const int nchunks = n * EB;

  // rows n .. NROWS-1 stay zero: the last 32-row K step and 16-row m tile read them
  for (int i = n * Q + tid; i < NROWS * Q; i += NT) reinterpret_cast<u32x4*>(Xs)[i] = u32x4{0u, 0u, 0u, 0u};

  const uint16_t* wrow[ZW];
#pragma unroll
  for (int zi = 0; zi < ZW; ++zi) {
    const int zt = wave + zi * NW;
    const int z = zt * 16 + li;
    const uint16_t* r = nullptr;
    if (zt < ZT) {
      if (z < k)
        r = p.phi + (int64_t)z * n;
      else if (z < k + n_l)
        r = p.w_l + (int64_t)(z - k) * n;
    }
    wrow[zi] = r;
  }
  // the output LayerNorm's gamma / beta are the same for every example: stage them once
  // (a global load inside the example loop would wait for the in-flight X prefetch)
  for (int i = tid; i < 2 * D; i += NT) {
    const uint16_t* src = i < D ? p.out_gamma : p.out_beta;
    Gs[i] = src ? src[i < D ? i : i - D] : (uint16_t)(i < D ? 0x3f80u : 0u);
  }
  if constexpr (WL) {
    // [Phi; W_L] is the same for every example: stage it once, zero-padded to 16-row tiles and NROWS columns
    const int rows = ZT * 16, cpr = WP / 8;
    for (int i = tid; i < rows * cpr; i += NT) {
      const int z = i / cpr, c = (i - z * cpr) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (c < n) {
        if (z < k)
          v = *reinterpret_cast<const u32x4*>(p.phi + (int64_t)z * n + c);
        else if (z < k + n_l)
          v = *reinterpret_cast<const u32x4*>(p.w_l + (int64_t)(z - k) * n + c);
      }
      *reinterpret_cast<u32x4*>(Ws + z * WP + c) = v;
    }
  }

  u32x4 xr[CPT];
  auto load_x = [&](int64_t b) {
    const uint16_t* xb = p.x + b * (int64_t)n * D;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + c * NT;
      xr[c] = q < nchunks ? *reinterpret_cast<const u32x4*>(xb + (int64_t)q * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + c * NT;
      if (q < nchunks) {
        const int row = q / EB, ch = q - row * EB;
        *reinterpret_cast<u32x4*>(Xs + row * P + ch * 8) = xr[c];
      }
    }
  };

  // the FMB LayerNorm's gamma / beta at this lane's F positions, packed bf16 pairs: the same for every
  // example, so loaded once (a global load in the example loop would wait for older stores)
  constexpr bool PRE = MW * KW <= 4;  // enough registers to keep them
  constexpr int PMW = PRE ? MW : 1, PKW = PRE ? KW : 1;
  uint32_t fgam[PMW][PKW][2], fbet[PMW][PKW][2];
#pragma unroll
  for (int mi = 0; mi < PMW; ++mi)
#pragma unroll
    for (int jt = 0; jt < PKW; ++jt) {
      const int m = (wave + mi * NW) * 16 + li;
      const int j0 = jt * 16 + lg * 4;
      u32x2 g2 = u32x2{0x3f803f80u, 0x3f803f80u}, b2 = u32x2{0u, 0u};
      if (m < n && j0 < k) {
        if (p.fm_gamma) g2 = *reinterpret_cast<const u32x2*>(p.fm_gamma + m * k + j0);
        if (p.fm_beta) b2 = *reinterpret_cast<const u32x2*>(p.fm_beta + m * k + j0);
      }
      fgam[mi][jt][0] = g2[0]; fgam[mi][jt][1] = g2[1];
      fbet[mi][jt][0] = b2[0]; fbet[mi][jt][1] = b2[1];
    }

  int64_t b = blockIdx.x;
  if (b >= batch) return;
  load_x(b);
  store_x();
  lds_barrier();
  // the next example's X is always loaded right after the previous one was written to LDS, so the
  // loads are older than every store of the example in between and waiting for them never waits
  // for those stores
  if (b + gridDim.x < batch) load_x(b + gridDim.x);
  const float inv_d = 1.0f / static_cast<float>(D);
  const float inv_nk = 1.0f / static_cast<float>(n * k);
  for (; b < batch; b += gridDim.x) {
    const int64_t bn = b + gridDim.x;

    // ---- phase 1: [Z; Lc]^T = X^T [Phi; W_L]^T, K = m in steps of 32
    f32x4 acc[ZW][ET];
#pragma unroll
    for (int zi = 0; zi < ZW; ++zi)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[zi][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operand addresses: lane (group lg, s = li) points at row m0 + 8 lg + s/4, column e0 + 4 (s%4)
    const uint16_t* xa = Xs + (8 * lg + (li >> 2)) * P + 4 * (li & 3);
    if constexpr (WL) {
      const uint16_t* wl_base = Ws + (wave * 16 + li) * WP + lg * 8;
      for (int m0 = 0; m0 < n; m0 += 32) {
        u32x4 wf[ZW];
#pragma unroll
        for (int zi = 0; zi < ZW; ++zi)
          if (wave + zi * NW < ZT) wf[zi] = *reinterpret_cast<const u32x4*>(wl_base + zi * NW * 16 * WP + m0);
        const uint16_t* xr0 = xa + m0 * P;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const u32x4 a = tr_operand(xr0 + et * 16, xr0 + 4 * P + et * 16);
#pragma unroll
          for (int zi = 0; zi < ZW; ++zi)
            if (wave + zi * NW < ZT) acc[zi][et] = mfma16x16x32(a, wf[zi], acc[zi][et]);
        }
      }
    } else {
      u32x4 wf[ZW], wn[ZW];
      auto load_w = [&](u32x4* dst, int m0) {
#pragma unroll
        for (int zi = 0; zi < ZW; ++zi) {
          const int mk = m0 + lg * 8;
          dst[zi] = (wrow[zi] != nullptr && mk < n) ? *reinterpret_cast<const u32x4*>(wrow[zi] + mk)
                                                    : u32x4{0u, 0u, 0u, 0u};
        }
      };
      load_w(wf, 0);
      for (int m0 = 0; m0 < n; m0 += 32) {
        if (m0 + 32 < n) load_w(wn, m0 + 32);
        const uint16_t* xr0 = xa + m0 * P;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const u32x4 a = tr_operand(xr0 + et * 16, xr0 + 4 * P + et * 16);
#pragma unroll
          for (int zi = 0; zi < ZW; ++zi)
            if (wave + zi * NW < ZT) acc[zi][et] = mfma16x16x32(a, wf[zi], acc[zi][et]);
        }
#pragma unroll
        for (int zi = 0; zi < ZW; ++zi) wf[zi] = wn[zi];
      }
    }

    // ---- Z -> LDS (bf16, zero padding), LCB rows of Y
    for (int i = tid; i < 16 * KW * Z_LD / 8; i += NT) reinterpret_cast<u32x4*>(Zs)[i] = u32x4{0u, 0u, 0u, 0u};
    lds_barrier();
#pragma unroll
    for (int zi = 0; zi < ZW; ++zi) {
      const int zt = wave + zi * NW;
      if (zt >= ZT) continue;  // wave-uniform
      const int z = zt * 16 + li;
      if (z < k) {
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          u32x2 v;
          v[0] = pack_bf16x2(acc[zi][et][0], acc[zi][et][1]);
          v[1] = pack_bf16x2(acc[zi][et][2], acc[zi][et][3]);
          *reinterpret_cast<u32x2*>(Zs + z * Z_LD + et * 16 + lg * 4) = v;
        }
      }
      if (zt * 16 + 15 >= k && zt * 16 < k + n_l) {  // wave-uniform
        const bool is_l = (z >= k) && (z < k + n_l);
        const int row = n_f + (z - k);
        float v[ET][4];
        float sm = 0.f;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          u32x2 xv = u32x2{0u, 0u};
          if (is_l) xv = *reinterpret_cast<const u32x2*>(Xs + row * P + et * 16 + lg * 4);
          v[et][0] = acc[zi][et][0] + bf16lo(xv[0]);
          v[et][1] = acc[zi][et][1] + bf16hi(xv[0]);
          v[et][2] = acc[zi][et][2] + bf16lo(xv[1]);
          v[et][3] = acc[zi][et][3] + bf16hi(xv[1]);
          sm += (v[et][0] + v[et][1]) + (v[et][2] + v[et][3]);
        }
        sm = xor_sum<16>(sm);
        const float mean = sm * inv_d;
        float q = 0.f;
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float dv = v[et][t] - mean;
            q += dv * dv;
          }
        q = xor_sum<16>(q);
        const float rstd = rsqrtf(q * inv_d + p.eps);
        if (is_l) {
          uint16_t* yrow = p.y + (b * n + row) * (int64_t)D;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const int e = et * 16 + lg * 4;
            const u32x2 g2 = *reinterpret_cast<const u32x2*>(Gs + e);
            const u32x2 b2 = *reinterpret_cast<const u32x2*>(Gs + D + e);
            const float gm[4] = {bf16lo(g2[0]), bf16hi(g2[0]), bf16lo(g2[1]), bf16hi(g2[1])};
            const float bt[4] = {bf16lo(b2[0]), bf16hi(b2[0]), bf16lo(b2[1]), bf16hi(b2[1])};
            u32x2 o;
            o[0] = pack_bf16x2((v[et][0] - mean) * rstd * gm[0] + bt[0], (v[et][1] - mean) * rstd * gm[1] + bt[1]);
            o[1] = pack_bf16x2((v[et][2] - mean) * rstd * gm[2] + bt[2], (v[et][3] - mean) * rstd * gm[3] + bt[3]);
            *reinterpret_cast<u32x2*>(yrow + e) = o;
          }
        }
      }
    }
    lds_barrier();  // Z complete

    // ---- phase 2: F^T = Z X^T (rows j of Z, contraction e), X rows from LDS
    f32x4 facc[MW][KW];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int jt = 0; jt < KW; ++jt) facc[mi][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
      const int mt = wave + mi * NW;
      if (mt < MT) {  // wave-uniform
        const int m = mt * 16 + li;
#pragma unroll
        for (int ks = 0; ks < DZ / 32; ++ks) {
          const int e0 = ks * 32 + lg * 8;
          u32x4 xf = u32x4{0u, 0u, 0u, 0u};
          if (e0 < D) xf = *reinterpret_cast<const u32x4*>(Xs + m * P + e0);
#pragma unroll
          for (int jt = 0; jt < KW; ++jt) {
            if (jt < KT) {
              const u32x4 zf = *reinterpret_cast<const u32x4*>(Zs + (jt * 16 + li) * Z_LD + e0);
              facc[mi][jt] = mfma16x16x32(zf, xf, facc[mi][jt]);
            }
          }
        }
      }
    }
    float sm = 0.f;
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int jt = 0; jt < KW; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = (wave + mi * NW) * 16 + li;
          const int j = jt * 16 + lg * 4 + t;
          if (m < n && j < k) sm += facc[mi][jt][t];
        }
    sm = group_sum_v<64>(sm);
    if (lane == 0) red[wave] = sm;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[w];
    const float mean = tot * inv_nk;
    float q = 0.f;
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int jt = 0; jt < KW; ++jt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = (wave + mi * NW) * 16 + li;
          const int j = jt * 16 + lg * 4 + t;
          if (m < n && j < k) {
            const float dv = facc[mi][jt][t] - mean;
            q += dv * dv;
          }
        }
    q = group_sum_v<64>(q);
    if (lane == 0) red[NW + wave] = q;
    lds_barrier();  // also: every wave is done reading Xs and Zs of this example
    float qt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) qt += red[NW + w];
    const float rstd = rsqrtf(qt * inv_nk + p.eps);
    uint16_t* fnb = p.fn + b * (int64_t)n * k;
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int jt = 0; jt < KW; ++jt) {
        const int m = (wave + mi * NW) * 16 + li;
        const int j0 = jt * 16 + lg * 4;
        if (m < n && j0 < k) {
          const int idx = m * k + j0;
          u32x2 g2, b2;
          if constexpr (PRE) {
            g2 = u32x2{fgam[PRE ? mi : 0][PRE ? jt : 0][0], fgam[PRE ? mi : 0][PRE ? jt : 0][1]};
            b2 = u32x2{fbet[PRE ? mi : 0][PRE ? jt : 0][0], fbet[PRE ? mi : 0][PRE ? jt : 0][1]};
          } else {
            g2 = p.fm_gamma ? *reinterpret_cast<const u32x2*>(p.fm_gamma + idx) : u32x2{0x3f803f80u, 0x3f803f80u};
            b2 = p.fm_beta ? *reinterpret_cast<const u32x2*>(p.fm_beta + idx) : u32x2{0u, 0u};
          }
          const float gm[4] = {bf16lo(g2[0]), bf16hi(g2[0]), bf16lo(g2[1]), bf16hi(g2[1])};
          const float bt[4] = {bf16lo(b2[0]), bf16hi(b2[0]), bf16lo(b2[1]), bf16hi(b2[1])};
          const f32x4 f = facc[mi][jt];
          u32x2 o;
          o[0] = pack_bf16x2((f[0] - mean) * rstd * gm[0] + bt[0], (f[1] - mean) * rstd * gm[1] + bt[1]);
          o[1] = pack_bf16x2((f[2] - mean) * rstd * gm[2] + bt[2], (f[3] - mean) * rstd * gm[3] + bt[3]);
          *reinterpret_cast<u32x2*>(fnb + idx) = o;
        }
      }
    if (bn < batch) {
      store_x();  // the barrier above guarantees nobody still reads this example's X
      lds_barrier();
      if (bn + gridDim.x < batch) load_x(bn + gridDim.x);
    }
  }
}

// LDS bytes: X, Z and (when staged) the [Phi; W_L] tiles of zt_rows rows
template <int ET, int NW, int ZW, int MW, int KW, int NMAX, bool WL>
size_t resident_lds_bytes(int zt_rows) {
  constexpr int D = 16 * ET;
  constexpr int Q = D / 8 + 1;
  constexpr int NROWS = (NMAX + 31) / 32 * 32;
  constexpr int DZ = (D + 31) / 32 * 32;
  const size_t w = WL ? (size_t)zt_rows * (NROWS + 8) * 2 : 0;
  return (size_t)NROWS * Q * 16 + (size_t)16 * KW * (DZ + 8) * 2 + (size_t)4 * D + w;
}

struct ResidentVariant {
  int et, nw, zw, mw, kw, nmax, per_cu;
  bool wl;
  void (*kernel)(FmbLcbArgs, int64_t);
  size_t (*lds)(int);
};

#define WK_RES_FMB(ET, NW, ZW, MW, KW, NMAX, WL, PER_CU)                                           \
  ResidentVariant {                                                                               \
    ET, NW, ZW, MW, KW, NMAX, PER_CU, WL, fmb_lcb_resident_kernel<ET, NW, ZW, MW, KW, NMAX, WL>,  \
        resident_lds_bytes<ET, NW, ZW, MW, KW, NMAX, WL>                                          \
  }

const ResidentVariant kResident[] = {
    WK_RES_FMB(10, 4, 2, 2, 2, 128, true, 2),    // n=128, d=160, k=32, n_L=64: [Phi; W_L] staged in LDS
    WK_RES_FMB(2, 8, 3, 6, 2, 720, false, 2),    // n=720, d=32,  k=24, n_L=360
    WK_RES_FMB(10, 8, 2, 2, 3, 256, false, 1),   // n=256, d=160, k=48, n_L=128
};

const ResidentVariant* pick_resident(int n, int d, int k, int n_l) {
  if (d % 16 != 0) return nullptr;
  const int et = d / 16;
  const int zt = (k + n_l + 15) / 16, mt = (n + 15) / 16, kt = (k + 15) / 16;
  for (const auto& v : kResident) {
    if (v.et != et || n > v.nmax) continue;
    if ((zt + v.nw - 1) / v.nw > v.zw) continue;
    if ((mt + v.nw - 1) / v.nw > v.mw) continue;
    if (kt > v.kw) continue;
    return &v;
  }
  return nullptr;
}

template <int ET, int NW, int ZW, int MW, int KW, int MC>
size_t lds_bytes() {
  constexpr int D = 16 * ET;
  constexpr int DZ = (D + 31) / 32 * 32;
  const size_t xt = (size_t)D * (MC + 8) * 2;
  const size_t zs = (size_t)16 * KW * (DZ + 8) * 2;
  return xt > zs ? xt : zs;
}

struct FmbLcbVariant {
  int et, nw, zw, mw, kw, mc;
  void (*kernel)(FmbLcbArgs);
  size_t lds;
};

#define WK_FMB_VARIANT(ET, NW, ZW, MW, KW, MC)                                   \
  FmbLcbVariant {                                                                \
    ET, NW, ZW, MW, KW, MC, fmb_lcb_bf16_kernel<ET, NW, ZW, MW, KW, MC>,         \
        lds_bytes<ET, NW, ZW, MW, KW, MC>()                                      \
  }

// Tight variants for the measured shapes first, then general fallbacks.
const FmbLcbVariant kVariants[] = {
    WK_FMB_VARIANT(10, 4, 2, 2, 2, 64),   // n=128, d=160, k=32, n_L=64
    WK_FMB_VARIANT(10, 4, 3, 4, 3, 64),   // n=256, d=160, k=48, n_L=128
    WK_FMB_VARIANT(10, 8, 3, 4, 6, 64),   // n=512, d=160, k=96, n_L=256
    WK_FMB_VARIANT(2, 8, 3, 6, 2, 256),   // n=720, d=32,  k=24, n_L=360
    WK_FMB_VARIANT(1, 4, 4, 8, 4, 256),   // general fallbacks: d = 16
    WK_FMB_VARIANT(2, 4, 4, 8, 4, 256),   // d = 32
    WK_FMB_VARIANT(3, 4, 4, 8, 4, 128),   // d = 48
    WK_FMB_VARIANT(4, 4, 4, 8, 4, 128),   // d = 64
    WK_FMB_VARIANT(5, 4, 4, 8, 4, 128),   // d = 80
    WK_FMB_VARIANT(8, 4, 3, 8, 4, 64),    // d = 128
    WK_FMB_VARIANT(10, 4, 3, 8, 4, 64),   // d = 160
    WK_FMB_VARIANT(10, 8, 3, 4, 8, 64),   // d = 160, larger n / k
};

const FmbLcbVariant* pick(int n, int d, int k, int n_l) {
  if (d % 16 != 0) return nullptr;
  const int et = d / 16;
  const int zt = (k + n_l + 15) / 16, mt = (n + 15) / 16, kt = (k + 15) / 16;
  for (const auto& v : kVariants) {
    if (v.et != et) continue;
    if ((zt + v.nw - 1) / v.nw > v.zw) continue;
    if ((mt + v.nw - 1) / v.nw > v.mw) continue;
    if (kt > v.kw) continue;
    return &v;
  }
  return nullptr;
}

}  // namespace

bool fmb_lcb_bf16_supported(int n, int d, int k, int n_l) {
  return fmb_lcb_stream_supported(n, d, k, n_l) || pick_resident(n, d, k, n_l) != nullptr ||
         pick(n, d, k, n_l) != nullptr;
}

size_t fmb_lcb_bf16_pack_bytes(int n, int d, int k, int n_l, bool train) {
  // the same choice as launch_fmb_lcb_bf16: only the streamed kernel reads packed weights
  const ResidentVariant* res = pick_resident(n, d, k, n_l);
  if (train || !(res && res->wl)) return fmb_lcb_stream_pack_bytes(n, d, k, n_l);
  return 0;
}

bool fmb_lcb_kblocked_fn_supported(int n, int d, int k, int n_l) {
  const ResidentVariant* res = pick_resident(n, d, k, n_l);
  return !(res && res->wl) && fmb_lcb_stream_supported(n, d, k, n_l) && (n * k) % 64 == 0;
}

hipError_t launch_fmb_lcb_bf16(const FmbLcbArgs& a, int64_t batch, hipStream_t stream,
                               int64_t* workgroups) {
  if (a.fn_kblock_rows > 0) {  // K-blocked Fn: the plain forward's streamed kernel only
    if (a.z_out != nullptr || !fmb_lcb_kblocked_fn_supported(a.n, a.d, a.k, a.n_l) ||
        a.fn_kblock_rows % 256 != 0 || a.fn_kblock_rows < batch ||
        a.fn_kblock_rows * (int64_t)a.n * a.k * 2 >= ((int64_t)1 << 31))
      return hipErrorInvalidValue;
    return launch_fmb_lcb_stream(a, batch, stream, workgroups);
  }
  // Order: the resident kernel when [Phi; W_L] fits in its LDS next to X (the
  // weights are then read once per workgroup), else the streamed kernel (X
  // and the weights through an LDS ring, several examples per workgroup),
  // else the resident or chunked kernels.
  if (a.z_out != nullptr || a.lc_out != nullptr) {  // the training outputs: streamed kernel only
    if (!fmb_lcb_stream_supported(a.n, a.d, a.k, a.n_l)) return hipErrorInvalidValue;
    return launch_fmb_lcb_stream(a, batch, stream, workgroups);
  }
  const ResidentVariant* res = pick_resident(a.n, a.d, a.k, a.n_l);
  if (!(res && res->wl) && fmb_lcb_stream_supported(a.n, a.d, a.k, a.n_l))
    return launch_fmb_lcb_stream(a, batch, stream, workgroups);
  if (const ResidentVariant* r = res) {
    const int64_t grid = batch < (int64_t)256 * r->per_cu ? batch : (int64_t)256 * r->per_cu;
    if (workgroups) *workgroups = grid;
    if (batch == 0) return hipSuccess;
    // the dynamic LDS size depends on the shape: raise the kernel's limit when a larger one is needed
    static std::atomic<size_t> attr_set[sizeof(kResident) / sizeof(kResident[0])];
    const size_t vi = (size_t)(r - kResident);
    const size_t lds = r->lds(((a.k + a.n_l + 15) / 16) * 16);
    if (lds > attr_set[vi].load()) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(r->kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set[vi].store(lds);
    }
    hipLaunchKernelGGL(r->kernel, dim3((unsigned)grid), dim3(r->nw * 64), lds, stream, a, batch);
    return hipGetLastError();
  }
  const FmbLcbVariant* v = pick(a.n, a.d, a.k, a.n_l);
  if (!v) return hipErrorInvalidValue;
  if (workgroups) *workgroups = batch;
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)batch), dim3(v->nw * 64), v->lds, stream, a);
  return hipGetLastError();
}

}  // namespace wk
