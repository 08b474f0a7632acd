// WHALE's attention-based fusion step: the cross-branch attention, the FFN
// as one kernel, and a row LayerNorm for the unfused FFN (bf16, fp32
// accumulation).  The Fusion MLP's Linear (and the unfused FFN's Linears)
// run on the MLP GEMM kernels.
//
// WHALE technical summaries, section 2.1: the Wukong module's interaction
// representation H_w is the query and the HSTU module's behaviour
// representation H_s (the whole sequence of L positions) gives the keys and
// the values; section 2.2: keys and values are one shared tensor (K = V),
// which halves the attention's memory traffic.  Per example:
//   A = softmax(H_w H_s^T / sqrt(d)) H_s,   C = [H_w, A]   (n x 2d)
//
// whale_attention_kernel: one workgroup of 4 waves per (example, 128
// queries), 32 queries per wave.  Key tiles of 32 positions x d (64 at d = 64,
// 128 at d = 32) are DMA'd
// (buffer_load ... lds) into a ring of 4 LDS slots, 3 tiles ahead; each tile
// is read twice from LDS, as K (rows, for S^T = K Q^T) and as V (transposed
// reads, for O^T += V^T P^T): the shared K = V is loaded once.  Both products
// are computed transposed on v_mfma_f32_16x16x32_bf16, so a lane (li, lg)
// holds scores of one query (li) at keys 16 kk + 4 lg + t: over the tile's two
// key blocks, 8 keys, which in bf16 are exactly its B operand of the P V
// product when V^T's rows are read in the same key order -- P stays in
// registers.  The softmax is the online form (running maximum per query, O
// rescaled when it grows), in base 2 with the 1/sqrt(d) scale folded into the
// exponent; the 4 lanes of a query combine maxima with two xor-shuffles per
// key tile and keep partial sums that are combined once at the end.
// Positions past L read as zero through the buffer resource and are masked
// to -inf.
#include <math.h>

#include <type_traits>

#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define WF_LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4*)(p))
#define WF_LDSV(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int AW = 4;    // waves per workgroup
constexpr int AQ = 32;   // queries per wave (two 16-row tiles)
// 16-position key blocks per step: more at small d, where a step's products are short
// and the per-step maxima, barrier and waits would otherwise dominate
__host__ __device__ constexpr int attn_kb(int d) { return d <= 32 ? 8 : (d <= 64 ? 4 : 2); }

constexpr int vm_enc(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Eight consecutive rows r0 .. r0 + 7 of a row-major [*, D] LDS tile at one
// column, as one MFMA operand: in each 16-lane group, ds_read_b64_tr_b16 hands
// lane i value i % 4 of the 8-byte rows addressed by lanes 4k + i / 4, so lanes
// pointing at row 8 g + s / 4, column c0 + 4 (s % 4) receive rows 8 g .. 8 g + 3
// of column c0 + s; the second read covers rows 8 g + 4 .. 8 g + 7.
__device__ __forceinline__ u32x4 tr_rows8(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WF_LDS_I16X4(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WF_LDS_I16X4(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

struct AttnArgs {
  const uint16_t* hw;   // [B, n, D]
  const uint16_t* hs;   // [B, L, D]
  const uint16_t* w_f;  // [D, 2D]: the Fusion MLP's Linear
  const uint16_t* b_f;  // [D] or null
  uint16_t* q;          // [B, n, D]: Q = [H_w, A] W_f^T + b_f
  int64_t batch;
  int n, L;
  float scale_log2;     // log2(e) / sqrt(D)
};

template <int D>
__global__ __launch_bounds__(AW * 64, 2) void whale_attention_kernel(AttnArgs p) {
  constexpr int KB = attn_kb(D);            // 16-position key blocks per step
  constexpr int AKT = 16 * KB;              // sequence positions per step
  constexpr int DC = D / 32;                // 32-wide chunks of the Q K^T contraction
  constexpr int DT = D / 16;                // 16-wide output column tiles
  constexpr int TILE = AKT * D;             // u16 per key tile
  constexpr int INS = TILE * 2 / 1024;      // 1 KB DMA instructions per tile
  constexpr int INS_HI = (INS + AW - 1) / AW, INS_LO = INS / AW, R = INS % AW;
  static_assert(D % 32 == 0 && INS * 1024 == TILE * 2 && KB % 2 == 0, "D must be a multiple of 32");
  // the ring continues past the key tiles with W_f: a W_f step holds AKT / 2 of its rows
  // (all 2D columns, TILE u16 like a key tile), i.e. JPS 16-row output blocks of Q
  constexpr int NJ = D / 16, JPS = AKT / 32, NWS = (NJ + JPS - 1) / JPS;
  constexpr int WU = D / 4;                 // 16-byte units of a W_f row
  __shared__ __align__(16) uint16_t s0[TILE], s1[TILE], s2[TILE], s3[TILE];
  __shared__ __align__(16) uint16_t sbf[D];
  uint16_t* const slot[4] = {s0, s1, s2, s3};  // indexed with compile-time numbers only

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int n = p.n, L = p.L;
  const int qchunks = (n + AW * AQ - 1) / (AW * AQ);
  const int64_t b = blockIdx.x / qchunks;
  const int q0 = (int)(blockIdx.x - b * qchunks) * (AW * AQ) + wave * AQ;
  const int T = (L + AKT - 1) / AKT;
  const int TT = T + NWS;  // steps: key tiles, then W_f
  const float scale = p.scale_log2;
  for (int i = tid; i < D; i += AW * 64) sbf[i] = p.b_f ? p.b_f[i] : (uint16_t)0;

  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.hs + b * (int64_t)L * D), (short)0, L * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rwf =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.w_f, (short)0, 4 * D * D, 0x00020000);
  auto dma = [&](uint16_t* dst, int step) {
    if (step < T) {  // key tile: contiguous
#pragma unroll
      for (int q = 0; q < INS_HI; ++q) {
        const int i = wave + q * AW;  // wave-uniform
        if (i < INS) {
          const uint32_t vo = (uint32_t)step * (TILE * 2) + (uint32_t)(i * 1024 + lane * 16);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, WF_LDSV(dst + i * 512), 16, vo, 0, 0, 0);
        }
      }
    } else {  // W_f rows, 16-byte unit u of row r at LDS unit u ^ (r % 8); rows past D read zero
#pragma unroll
      for (int q = 0; q < INS_HI; ++q) {
        const int i = wave + q * AW;
        if (i < INS) {
          const int pos = i * 64 + lane, r = pos / WU, pu = pos - r * WU;
          const uint32_t vo = (uint32_t)(((step - T) * (AKT / 2) + r) * (4 * D) + (pu ^ (r & 7)) * 16);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rwf, WF_LDSV(dst + i * 512), 16, vo, 0, 0, 0);
        }
      }
    }
  };

  // queries of this wave as MFMA B operands: query q0 + 16 qt + li, columns 32 c + 8 lg ..
  u32x4 qf[2][DC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q0 + qt * 16 + li;
#pragma unroll
    for (int c = 0; c < DC; ++c)
      qf[qt][c] = q < n ? *reinterpret_cast<const u32x4*>(p.hw + (b * n + q) * D + c * 32 + lg * 8)
                        : u32x4{0u, 0u, 0u, 0u};
  }

#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (u < TT) dma(slot[u], u);

  // O^T: o[qt][dt][t] = O[query q0 + 16 qt + li][column 16 dt + 4 lg + t]; per query
  // (qt) the running maximum (scaled, base 2) and this lane's part of the sum
  f32x4 o[2][DT];
  float mrow[2], lrow[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrow[qt] = -INFINITY;
    lrow[qt] = 0.f;
  }
  // V^T operand lanes: key rows 4 lg + li / 4 (and 16 further), column 4 (li % 4)
  const int xa = (4 * lg + (li >> 2)) * D + 4 * (li & 3);

  // step t's copies landed (up to two newer steps may be in flight), for every wave
  auto step_begin = [&](uint16_t* next, int t) {
    const int newer = (TT - 1 - t < 2) ? TT - 1 - t : 2;  // DMA steps issued after step t
    if (newer <= 0) {
      __builtin_amdgcn_s_waitcnt(vm_enc(0));
    } else if (newer == 1) {
      if (wave < R) __builtin_amdgcn_s_waitcnt(vm_enc(INS_HI));
      else __builtin_amdgcn_s_waitcnt(vm_enc(INS_LO));
    } else {
      if (wave < R) __builtin_amdgcn_s_waitcnt(vm_enc(2 * INS_HI));
      else __builtin_amdgcn_s_waitcnt(vm_enc(2 * INS_LO));
    }
    ring_barrier();  // not lds_barrier: its fence would also wait for the two newer steps' DMA
    if (t + 3 < TT) dma(next, t + 3);
  };
  auto step = [&](const uint16_t* kt, uint16_t* next, int t) {
    step_begin(next, t);
    // S^T = K Q^T: sc[qt][kk][t] = S[query 16 qt + li][key 16 kk + 4 lg + t]
    f32x4 sc[2][KB];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) sc[qt][kk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + (kk * 16 + li) * D + c * 32 + lg * 8);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) sc[qt][kk] = mfma16x16x32(kf, qf[qt][c], sc[qt][kk]);
      }
    }
    // online softmax per query; P^T in bf16 as the B operand of V^T P^T: in K step ks,
    // key slots 0..3 = keys 32 ks + 4 lg + t, 4..7 = keys 32 ks + 16 + 4 lg + t
    u32x4 pf[2][KB / 2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (t == T - 1) {  // only the last key tile can reach past L
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t * AKT + kk * 16 + 4 * lg + r >= L) sc[qt][kk][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[qt][kk][0], sc[qt][kk][1]), fmaxf(sc[qt][kk][2], sc[qt][kk][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mnew = fmaxf(mrow[qt], mx * scale);
      // v_exp_f32 directly: no denormal range handling (results below 2^-126 flush to 0,
      // against a maximum term of 1); exp2(-inf) = 0 for the first step's alpha
      const float alpha = __builtin_amdgcn_exp2f(mrow[qt] - mnew);
      float e[KB][4];
      float sm = 0.f;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[kk][r] = __builtin_amdgcn_exp2f(fmaf(sc[qt][kk][r], scale, -mnew));
          sm += e[kk][r];
        }
      lrow[qt] = fmaf(lrow[qt], alpha, sm);
      // rescale O only when some query's running maximum grew (alpha is exactly 1 otherwise)
      if (__builtin_amdgcn_ballot_w64(mnew != mrow[qt]) != 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= alpha;
      }
      mrow[qt] = mnew;
#pragma unroll
      for (int ks = 0; ks < KB / 2; ++ks)
        pf[qt][ks] = u32x4{pack_bf16x2(e[2 * ks][0], e[2 * ks][1]), pack_bf16x2(e[2 * ks][2], e[2 * ks][3]),
                           pack_bf16x2(e[2 * ks + 1][0], e[2 * ks + 1][1]),
                           pack_bf16x2(e[2 * ks + 1][2], e[2 * ks + 1][3])};
    }
    // O^T += V^T P^T, V = the same key tile read transposed in the slot order
#pragma unroll
    for (int ks = 0; ks < KB / 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vk = kt + ks * 32 * D + xa + dt * 16;
        const u32x4 vf = tr_rows8(vk, vk + 16 * D);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[qt][dt] = mfma16x16x32(vf, pf[qt][ks], o[qt][dt]);
      }
  };
  // The Fusion MLP's Linear on [H_w, A]: Q^T = W_f [H_w, A]^T + b_f, with the C^T
  // operand in registers: H_w as loaded (qf), A = O / l rounded to bf16 in the
  // slot order of O^T (K step ks: columns 32 ks + 4 lg + t, then 32 ks + 16 + 4 lg + t),
  // which the W_f reads of A's half follow (two 8-byte pieces).
  u32x4 aop[2][DC];
  auto wf_step = [&](const uint16_t* wt, uint16_t* next, int t) {
    step_begin(next, t);
    const int w = t - T;
#pragma unroll
    for (int jj = 0; jj < JPS; ++jj) {
      const int jb = w * JPS + jj;
      if (jb < NJ) {  // uniform
        const int r = jj * 16 + li;  // W_f row 16 jb + li within the step
        const uint16_t* wr = wt + r * (2 * D);
        const int sw = r & 7;
        const u32x2 bb = *reinterpret_cast<const u32x2*>(sbf + jb * 16 + lg * 4);
        f32x4 qa[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) qa[qt] = f32x4{bf16lo(bb[0]), bf16hi(bb[0]), bf16lo(bb[1]), bf16hi(bb[1])};
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) {  // H_w half: columns 32 ks + 8 lg ..
          const u32x4 a = *reinterpret_cast<const u32x4*>(wr + (((ks * 4 + lg) ^ sw) * 8));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) qa[qt] = mfma16x16x32(a, qf[qt][ks], qa[qt]);
        }
#pragma unroll
        for (int ks = 0; ks < DC; ++ks) {  // A half: columns D + 32 ks + 4 lg .. and D + 32 ks + 16 + 4 lg ..
          const int u0 = D / 8 + ks * 4 + (lg >> 1), h = (lg & 1) * 4;
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(wr + ((u0 ^ sw) * 8) + h);
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(wr + (((u0 + 2) ^ sw) * 8) + h);
          const u32x4 a = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) qa[qt] = mfma16x16x32(a, aop[qt][ks], qa[qt]);
        }
        // Q[query 16 qt + li][16 jb + 4 lg + t]
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int q = q0 + qt * 16 + li;
          if (q < n)
            *reinterpret_cast<u32x2*>(p.q + (b * n + q) * D + jb * 16 + lg * 4) =
                u32x2{pack_bf16x2(qa[qt][0], qa[qt][1]), pack_bf16x2(qa[qt][2], qa[qt][3])};
        }
      }
    }
  };
  for (int t0 = 0; t0 < T; t0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // unrolled: every slot is a known object at each step
      if (t0 + u >= T) break;
      step(slot[u], slot[(u + 3) & 3], t0 + u);
    }
  }
  // A from O^T and the row sums (O is dead after this)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float l = lrow[qt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float inv = 1.0f / l;
#pragma unroll
    for (int ks = 0; ks < DC; ++ks) {
      const f32x4 v0 = o[qt][2 * ks], v1 = o[qt][2 * ks + 1];
      aop[qt][ks] = u32x4{pack_bf16x2(v0[0] * inv, v0[1] * inv), pack_bf16x2(v0[2] * inv, v0[3] * inv),
                          pack_bf16x2(v1[0] * inv, v1[1] * inv), pack_bf16x2(v1[2] * inv, v1[3] * inv)};
    }
  }
  // the W_f steps T .. TT - 1 continue the ring: step t in slot t % 4, the phase T % 4 a
  // compile-time constant in each branch
  auto wf_loop = [&](auto phase) {
    constexpr int P = decltype(phase)::value;
    for (int t0 = T; t0 < TT; t0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + u >= TT) break;
        wf_step(slot[(P + u) & 3], slot[(P + u + 3) & 3], t0 + u);
      }
    }
  };
  switch (T & 3) {
    case 0: wf_loop(std::integral_constant<int, 0>{}); break;
    case 1: wf_loop(std::integral_constant<int, 1>{}); break;
    case 2: wf_loop(std::integral_constant<int, 2>{}); break;
    default: wf_loop(std::integral_constant<int, 3>{}); break;
  }
}

// y[r] = LN(x[r]) * gamma + beta over rows of d (d % 8 == 0, d <= 512): G lanes
// per row (the power of two >= d / 8), 64 / G rows per wave, 8 values per lane.
template <int G>
__global__ __launch_bounds__(256) void row_ln_bf16_kernel(const uint16_t* x, uint16_t* y, int64_t rows, int d,
                                                           const uint16_t* gamma, const uint16_t* beta, float eps) {
  constexpr int RPW = 64 / G;  // rows per wave
  const int lane = threadIdx.x & 63, sub = lane % G;
  const int64_t r = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / G;
  const bool on = r < rows && sub * 8 < d;
  float v[8];
  const u32x4 xv = on ? *reinterpret_cast<const u32x4*>(x + r * d + sub * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[2 * t] = bf16lo(xv[t]);
    v[2 * t + 1] = bf16hi(xv[t]);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += v[e];
  s = group_sum<G>(s);
  const float mean = s / (float)d;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) q += on ? (v[e] - mean) * (v[e] - mean) : 0.f;
  q = group_sum<G>(q);
  const float rstd = rsqrtf(q / (float)d + eps);
  if (!on) return;
  const u32x4 g = gamma ? *reinterpret_cast<const u32x4*>(gamma + sub * 8)
                        : u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const u32x4 bt = beta ? *reinterpret_cast<const u32x4*>(beta + sub * 8) : u32x4{0u, 0u, 0u, 0u};
  u32x4 o;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    o[t] = pack_bf16x2((v[2 * t] - mean) * rstd * bf16lo(g[t]) + bf16lo(bt[t]),
                       (v[2 * t + 1] - mean) * rstd * bf16hi(g[t]) + bf16hi(bt[t]));
  *reinterpret_cast<u32x4*>(y + r * d + sub * 8) = o;
}

// ---- The fusion step's FFN in one kernel (WHALE section 2.2, pre-norm
// shared-gate SwiGLU with its residual):
//   H_f = Q + (silu(U) * U) W_down^T + b_down,   U = LN_d(Q) W_up^T + b_up.
// A workgroup of W waves takes W x 32 rows (32 per wave) and walks d_ff in
// chunks of 32: the chunk's 32 rows of W_up and 32 columns of W_down are
// DMA'd (buffer_load ... lds) into one of two LDS stages while the other
// stage is consumed, so silu(U) * U never leaves registers and the hidden
// width costs no HBM traffic.  Register layouts, lane = (l16, lg), lg = lane / 16:
//  * LN(Q) is the B operand of U^T = W_up LN(Q)^T: the lane holds row l16,
//    columns 32 ks + 8 lg .. + 7 (one 16-byte load of Q per K step).
//  * A-operand row i of U block fb is the chunk's W_up row 8 (i / 4) + 4 fb +
//    i % 4, so output lane (l16, lg) receives row l16's U at chunk columns
//    8 lg + 4 fb + t: over its two blocks, 8 consecutive columns, which is
//    the B operand of H^T = W_down G^T for the chunk's K step as it stands.
//  * H^T: the lane holds row l16, columns 16 jb + 4 lg + t; the bias, the
//    residual Q (reloaded in this layout) and the stores are 8 bytes a lane.
// The LDS copies are XOR-swizzled in 16-byte units so the 16-row fragment
// reads spread over the banks.  Rows past the end read as zero and their
// stores are dropped (buffer resources end at the last row).
struct FfnKArgs {
  const uint16_t* q;
  const uint16_t* gamma;
  const uint16_t* beta;
  const uint16_t* w_up;
  const uint16_t* b_up;
  const uint16_t* w_down;
  const uint16_t* b_down;
  uint16_t* out;
  int64_t rows;
  int F;
  float eps;
};

constexpr int FRB = 2;          // 16-row blocks per wave
constexpr int FC = 32;          // d_ff columns per chunk
constexpr int kFfnMaxF = 4096;  // b_up is staged in LDS whole

// 16-byte unit swizzle of a W_up chunk row (C units a row): within groups of 8
// units when C % 8 == 0, else of 4
template <int C>
__device__ __forceinline__ int up_swz(int row) {
  return C % 8 == 0 ? ((row & 3) | ((row >> 1) & 4)) : (((row >> 1) & 1) | ((row >> 2) & 2));
}
__device__ __forceinline__ int down_swz(int j) { return (j >> 1) & 3; }

template <int D, int W>
__global__ __launch_bounds__(W * 64) void fusion_ffn_kernel(FfnKArgs p) {
  constexpr int KS = D / 32, JB = D / 16, C16 = D / 8;
  constexpr int SU = FC * D, SD = D * FC;      // u16 of a stage's W_up and W_down parts
  constexpr int NIU = SU / 512, NI = (SU + SD) / 512;  // 1 KB DMA instructions per chunk
  constexpr int ROWS = W * FRB * 16;
  static_assert(D % 32 == 0 && SU % 512 == 0, "whole K steps and DMA instructions");
  constexpr int HI = (NI + W - 1) / W, LO = NI / W, R = NI % W;  // a wave's DMA instructions per chunk
  __shared__ __align__(16) uint16_t wu0[SU], wd0[SD], wu1[SU], wd1[SD], wu2[SU], wd2[SD];
  __shared__ __align__(16) uint16_t sbu[kFfnMaxF];
  __shared__ __align__(16) uint16_t sg[D], sbt[D], sbd[D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int F = p.F, NC = F / FC;

  const __amdgpu_buffer_rsrc_t rwu = __builtin_amdgcn_make_buffer_rsrc((void*)p.w_up, (short)0, F * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rwd =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.w_down, (short)0, D * F * 2, 0x00020000);
  auto dma = [&](uint16_t* su, uint16_t* sd, int c) {
    for (int i = wave; i < NI; i += W) {  // wave-uniform
      const int u = (i < NIU ? i : i - NIU) * 64 + lane;  // 16-byte unit of the part
      if (i < NIU) {
        const int row = u / C16, pu = u - row * C16;
        const uint32_t vo = (uint32_t)(((c * FC + row) * D + (pu ^ up_swz<C16>(row)) * 8) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rwu, WF_LDSV(su + i * 512), 16, vo, 0, 0, 0);
      } else {
        const int j = u >> 2, pu = u & 3;
        const uint32_t vo = (uint32_t)((j * F + c * FC + (pu ^ down_swz(j)) * 8) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rwd, WF_LDSV(sd + (i - NIU) * 512), 16, vo, 0, 0, 0);
      }
    }
  };
  dma(wu0, wd0, 0);
  if (NC > 1) dma(wu1, wd1, 1);
  for (int i = tid; i < F; i += W * 64) sbu[i] = p.b_up ? p.b_up[i] : (uint16_t)0;
  for (int i = tid; i < D; i += W * 64) {
    sg[i] = p.gamma ? p.gamma[i] : (uint16_t)0x3f80u;
    sbt[i] = p.beta ? p.beta[i] : (uint16_t)0;
    sbd[i] = p.b_down ? p.b_down[i] : (uint16_t)0;
  }

  // this workgroup's rows: Q in the B-operand layout
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const int nrows = (int)min<int64_t>(ROWS, p.rows - r0);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + r0 * D), (short)0, nrows * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.out + r0 * D), (short)0, nrows * D * 2, 0x00020000);
  const int wrow = wave * FRB * 16;
  u32x4 qn[FRB][KS];
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qn[rb][ks] = __builtin_amdgcn_raw_buffer_load_b128(
          rq, (uint32_t)(((wrow + rb * 16 + l16) * D + ks * 32 + lg * 8) * 2), 0, 0);
  __syncthreads();  // the staged constants (and chunk 0, which the wait inside covers)

  // LN(Q) per row: the row's D values sit in the 4 lanes l16 + 16 lg
  const float inv_d = 1.0f / static_cast<float>(D);
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) {
    float v[KS][8];
    float sm = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[ks][2 * e] = bf16lo(qn[rb][ks][e]);
        v[ks][2 * e + 1] = bf16hi(qn[rb][ks][e]);
        sm += v[ks][2 * e] + v[ks][2 * e + 1];
      }
    sm += __shfl_xor(sm, 16, kWave);
    sm += __shfl_xor(sm, 32, kWave);
    const float mean = sm * inv_d;
    float q = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) q += (v[ks][e] - mean) * (v[ks][e] - mean);
    q += __shfl_xor(q, 16, kWave);
    q += __shfl_xor(q, 32, kWave);
    const float rstd = rsqrtf(q * inv_d + p.eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(sg + ks * 32 + lg * 8);
      const u32x4 b = *reinterpret_cast<const u32x4*>(sbt + ks * 32 + lg * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qn[rb][ks][e] = pack_bf16x2((v[ks][2 * e] - mean) * rstd * bf16lo(g[e]) + bf16lo(b[e]),
                                    (v[ks][2 * e + 1] - mean) * rstd * bf16hi(g[e]) + bf16hi(b[e]));
    }
  }

  f32x4 oacc[JB][FRB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb) oacc[jb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the W_up rows this lane supplies as A-operand row l16 of blocks 0 and 1
  const int urow0 = 8 * (l16 >> 2) + (l16 & 3), urow1 = urow0 + 4;
  // chunk c reads stage c % 3 and sends chunk c + 2 to stage (c + 2) % 3, last read by chunk c - 1
  auto chunk = [&](const uint16_t* su, const uint16_t* sd, uint16_t* nu, uint16_t* nd, int c) {
    if (c + 2 < NC) dma(nu, nd, c + 2);
    // U starts from its bias: chunk columns 8 lg + 4 fb + t
    const u32x4 bu = *reinterpret_cast<const u32x4*>(sbu + c * FC + lg * 8);
    f32x4 uacc[2][FRB];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb)
        uacc[fb][rb] = f32x4{bf16lo(bu[2 * fb]), bf16hi(bu[2 * fb]), bf16lo(bu[2 * fb + 1]), bf16hi(bu[2 * fb + 1])};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cu = ks * 4 + lg;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(su + (urow0 * C16 + (cu ^ up_swz<C16>(urow0))) * 8);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(su + (urow1 * C16 + (cu ^ up_swz<C16>(urow1))) * 8);
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb) {
        uacc[0][rb] = mfma16x16x32(a0, qn[rb][ks], uacc[0][rb]);
        uacc[1][rb] = mfma16x16x32(a1, qn[rb][ks], uacc[1][rb]);
      }
    }
    // the W_down fragments, requested before the gate so their latency hides under it
    u32x4 wdf[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = jb * 16 + l16;
      wdf[jb] = *reinterpret_cast<const u32x4*>(sd + (j * 4 + (lg ^ down_swz(j))) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);  // keeps the scheduler from sinking them to their use
    // G = silu(U) * U in bf16: the B operand of the W_down product
    u32x4 gop[FRB];
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const f32x4 u = uacc[fb][rb];
        gop[rb][2 * fb] = pack_bf16x2(silu_gate(u[0]), silu_gate(u[1]));
        gop[rb][2 * fb + 1] = pack_bf16x2(silu_gate(u[2]), silu_gate(u[3]));
      }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb) oacc[jb][rb] = mfma16x16x32(wdf[jb], gop[rb], oacc[jb][rb]);
    // this wave's copies of chunk c + 1 have landed (those of chunk c + 2 may be in flight),
    // then every wave's, and every wave is done with this stage
    if (c + 2 < NC) {
      if (wave < R) __builtin_amdgcn_s_waitcnt(vm_enc(HI));
      else __builtin_amdgcn_s_waitcnt(vm_enc(LO));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_enc(0));
    }
    ring_barrier();  // not lds_barrier: its fence would also wait for chunk c + 2's DMA
  };
  for (int c = 0; c < NC; c += 3) {
    chunk(wu0, wd0, wu2, wd2, c);
    if (c + 1 < NC) chunk(wu1, wd1, wu0, wd0, c + 1);
    if (c + 2 < NC) chunk(wu2, wd2, wu1, wd1, c + 2);
  }

  // H_f = Q + H + b_down, Q reloaded in the H^T layout
  u32x2 qr[JB][FRB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
      qr[jb][rb] = __builtin_amdgcn_raw_buffer_load_b64(
          rq, (uint32_t)(((wrow + rb * 16 + l16) * D + jb * 16 + lg * 4) * 2), 0, 0);
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const u32x2 bd = *reinterpret_cast<const u32x2*>(sbd + jb * 16 + lg * 4);
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb) {
      const f32x4 h = oacc[jb][rb];
      const u32x2 r = qr[jb][rb];
      u32x2 o;
      o[0] = pack_bf16x2(h[0] + bf16lo(bd[0]) + bf16lo(r[0]), h[1] + bf16hi(bd[0]) + bf16hi(r[0]));
      o[1] = pack_bf16x2(h[2] + bf16lo(bd[1]) + bf16lo(r[1]), h[3] + bf16hi(bd[1]) + bf16hi(r[1]));
      __builtin_amdgcn_raw_buffer_store_b64(o, ro, (uint32_t)(((wrow + rb * 16 + l16) * D + jb * 16 + lg * 4) * 2),
                                            0, 0);
    }
  }
}

}  // namespace

bool fusion_ffn_supported(int d, int d_ff) {
  return (d == 32 || d == 64 || d == 96 || d == 128 || d == 160) && d_ff >= FC && d_ff % FC == 0 &&
         d_ff <= kFfnMaxF;
}

hipError_t launch_fusion_ffn(const FusionFfnArgs& a, hipStream_t stream, int64_t* workgroups) {
  if (!fusion_ffn_supported(a.d, a.d_ff) || a.rows < 0) return hipErrorInvalidValue;
  constexpr int W = 8;
  FfnKArgs k;
  k.q = static_cast<const uint16_t*>(a.q);
  k.gamma = static_cast<const uint16_t*>(a.gamma);
  k.beta = static_cast<const uint16_t*>(a.beta);
  k.w_up = static_cast<const uint16_t*>(a.w_up);
  k.b_up = static_cast<const uint16_t*>(a.b_up);
  k.w_down = static_cast<const uint16_t*>(a.w_down);
  k.b_down = static_cast<const uint16_t*>(a.b_down);
  k.out = static_cast<uint16_t*>(a.out);
  k.rows = a.rows;
  k.F = a.d_ff;
  k.eps = a.eps;
  const int64_t blocks = (a.rows + W * FRB * 16 - 1) / (W * FRB * 16);
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(W * 64);
  switch (a.d) {
    case 32: hipLaunchKernelGGL((fusion_ffn_kernel<32, W>), grid, block, 0, stream, k); break;
    case 64: hipLaunchKernelGGL((fusion_ffn_kernel<64, W>), grid, block, 0, stream, k); break;
    case 96: hipLaunchKernelGGL((fusion_ffn_kernel<96, W>), grid, block, 0, stream, k); break;
    case 128: hipLaunchKernelGGL((fusion_ffn_kernel<128, W>), grid, block, 0, stream, k); break;
    default: hipLaunchKernelGGL((fusion_ffn_kernel<160, W>), grid, block, 0, stream, k); break;
  }
  return hipGetLastError();
}

bool whale_attention_supported(int n, int d, int L) {
  return n > 0 && n % 16 == 0 && L > 0 && (d == 32 || d == 64 || d == 96 || d == 128 || d == 160) &&
         (int64_t)L * d * 2 < ((int64_t)1 << 31);
}

hipError_t launch_whale_attention(const void* hw, const void* hs, const void* w_f, const void* b_f, void* q,
                                  int64_t batch, int n, int d, int L, hipStream_t stream, int64_t* workgroups) {
  if (!whale_attention_supported(n, d, L) || w_f == nullptr) return hipErrorInvalidValue;
  AttnArgs a;
  a.hw = static_cast<const uint16_t*>(hw);
  a.hs = static_cast<const uint16_t*>(hs);
  a.w_f = static_cast<const uint16_t*>(w_f);
  a.b_f = static_cast<const uint16_t*>(b_f);
  a.q = static_cast<uint16_t*>(q);
  a.batch = batch;
  a.n = n;
  a.L = L;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  const int64_t qchunks = (n + AW * AQ - 1) / (AW * AQ);
  const int64_t blocks = batch * qchunks;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(AW * 64);
  switch (d) {
    case 32: hipLaunchKernelGGL(whale_attention_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(whale_attention_kernel<64>, grid, block, 0, stream, a); break;
    case 96: hipLaunchKernelGGL(whale_attention_kernel<96>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(whale_attention_kernel<128>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(whale_attention_kernel<160>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_row_ln_bf16(const void* x, void* y, int64_t rows, int d, const void* gamma, const void* beta,
                              float eps, hipStream_t stream, int64_t* workgroups) {
  if (d <= 0 || d % 8 != 0 || d > 512) return hipErrorInvalidValue;
  int g = 1;
  while (g * 8 < d) g *= 2;
  const int64_t rows_per_block = 4 * (64 / g);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* ys = static_cast<uint16_t*>(y);
  const auto* gs = static_cast<const uint16_t*>(gamma);
  const auto* bs = static_cast<const uint16_t*>(beta);
  const dim3 grid((unsigned)blocks), block(256);
  switch (g) {
    case 1: hipLaunchKernelGGL(row_ln_bf16_kernel<1>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    case 2: hipLaunchKernelGGL(row_ln_bf16_kernel<2>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    case 4: hipLaunchKernelGGL(row_ln_bf16_kernel<4>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    case 8: hipLaunchKernelGGL(row_ln_bf16_kernel<8>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    case 16: hipLaunchKernelGGL(row_ln_bf16_kernel<16>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    case 32: hipLaunchKernelGGL(row_ln_bf16_kernel<32>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
    default: hipLaunchKernelGGL(row_ln_bf16_kernel<64>, grid, block, 0, stream, xs, ys, rows, d, gs, bs, eps); break;
  }
  return hipGetLastError();
}

}  // namespace wk
