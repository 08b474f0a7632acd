// Backward pass of one Wukong layer in bf16 (fp32 accumulation): the two
// per-example kernels around the MLP's backward, and the transpose and
// reduction kernels the MLP's weight gradients use.
//
// The forward (Wukong paper, section 2.2, xdnf.cn repost): Z = Phi X,
// F = X Z^T, Fn = LN(vec F), MLP -> M, Lc = W_L X, Y = LN_d([M; Lc] + X).
// Its gradients, by the chain rule through those steps in reverse:
//
//  bwd_out_kernel (before the MLP's backward), per example: recompute Lc with
//    MFMA (W_L and X in LDS), R = [M; Lc] + X row by row, and the output
//    LayerNorm's input gradient
//        dR = rstd (g - mean(g) - R_hat mean(g R_hat)),   g = dY gamma_out,
//    stored in bf16 as dM (rows < n_F, the MLP's upstream gradient) and dLc;
//    per-workgroup sums of dY R_hat and dY (gamma_out / beta_out gradients).
//  bwd_fmb_kernel (after the MLP's backward has produced d_Fn), per example:
//    recompute Z = Phi X and F = X Z^T with MFMA, the FM LayerNorm's
//    statistics, dF = rstd (q - mean(q) - F_tilde mean(q F_tilde)) with
//    q = d_Fn gamma_fm, dZ = dF^T X, and
//        dX = dR + [dF | Phi^T | W_L^T] [Z; dZ; dLc]      (one MFMA product)
//    plus per-workgroup sums of dZ X^T (d_Phi), dLc X^T (d_W_L), d_Fn F_tilde
//    and d_Fn (gamma_fm / beta_fm gradients).
//
// One workgroup of 8 waves walks examples blockIdx.x, + gridDim.x, ... and
// keeps the weight-gradient sums of its examples in registers; the host then
// adds the per-workgroup planes in a fixed order (launch_sum_planes), so every
// result is independent of timing.  An example's inputs are fetched into
// registers one example ahead (all of a thread's 16-byte loads together) and
// written to LDS at the top of the next iteration; barriers are LDS-only, so
// those loads stay in flight through the compute phases.  Nothing else reads
// global memory inside the example loop: a load issued behind the prefetch
// would wait for it (the vector-memory counter retires in order), which is
// why W_L's operands are held in registers.  X of one example, the LDS copies of Phi
// and W_L and the per-example operands all live in LDS (up to 160 KB per
// workgroup on gfx950): the shapes this covers are those whose LDS plan and
// per-wave tile counts fit (wukong_bwd_supported).
//
// MFMA operands (v_mfma_f32_16x16x32_bf16, lane l = 16 lg + li): row_op reads
// the 8 consecutive columns 8 lg .. of row li of a row-major LDS array (an
// operand whose contraction index runs along rows of the array), tr_op uses
// ds_read_b64_tr_b16 to read 8 consecutive rows 8 lg .. at column li (an
// operand whose contraction index runs down the array's columns).  Padding
// rows and columns of every LDS array are zero, so contraction lengths round
// up to 32 freely.
#include <math.h>

#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define WB_LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4*)(p))

constexpr int BW = 8;            // waves per workgroup
constexpr int BT = BW * kWave;   // threads per workgroup
constexpr int kLdsMax = 160 * 1024;
// bwd_fmb_kernel holds at most QF F tiles, QP d_Phi tiles and QL d_W_L tiles
// (16 x 16) per wave in registers across its examples.
constexpr int kQF = 2, kQP = 2, kQL = 4;

__host__ __device__ constexpr int up16(int v) { return (v + 15) / 16 * 16; }
__host__ __device__ constexpr int up32(int v) { return (v + 31) / 32 * 32; }

__device__ __forceinline__ u32x4 row_op(const uint16_t* base, int pitch, int r0, int c0, int li, int lg) {
  return *reinterpret_cast<const u32x4*>(base + (r0 + li) * pitch + c0 + 8 * lg);
}

// Lane (li, lg) addresses row r0 + 8 lg + li / 4, columns c0 + 4 (li % 4) ..;
// the transposing read hands it rows r0 + 8 lg .. + 3 of column c0 + li, and
// the second read (4 rows further) rows + 4 .. + 7.
__device__ __forceinline__ u32x4 tr_op(const uint16_t* base, int pitch, int r0, int c0, int li, int lg) {
  const uint16_t* p0 = base + (r0 + 8 * lg + (li >> 2)) * pitch + c0 + 4 * (li & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WB_LDS_I16X4(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WB_LDS_I16X4(p0 + 4 * pitch));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

__device__ __forceinline__ uint16_t to_bf16(float v) { return (uint16_t)f32_to_bf16(v); }

// Sum of one value per thread over the workgroup; every thread gets it.  red
// holds 2 slots of BW floats used alternately (slot = 0, 1, 0, ...), so one
// LDS-only barrier per call is enough: a slot is rewritten two calls later,
// after every thread has passed the barrier of the call in between.
__device__ __forceinline__ float block_sum(float v, float* red, int slot) {
  v = group_sum_v<64>(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* r = red + slot * BW;
  if (lane == 0) r[wave] = v;
  lds_barrier();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < BW; ++w) s += r[w];
  return s;
}

// Two sums at once (red holds 2 slots of 2 BW floats).
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red, int slot) {
  a = group_sum_v<64>(a);
  b = group_sum_v<64>(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* r = red + slot * 2 * BW;
  if (lane == 0) {
    r[wave] = a;
    r[BW + wave] = b;
  }
  lds_barrier();
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int w = 0; w < BW; ++w) {
    sa += r[w];
    sb += r[BW + w];
  }
  a = sa;
  b = sb;
}

__device__ __forceinline__ void zero_lds(uint16_t* base, int bytes) {
  for (int i = threadIdx.x * 16; i < bytes; i += BT * 16)
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + i) = u32x4{0u, 0u, 0u, 0u};
}

// rows [0, rows) x cols [0, cols) of a row-major global bf16 matrix (cols % 8 == 0) into LDS at pitch
__device__ __forceinline__ void load_rows(uint16_t* dst, int pitch, const uint16_t* src, int rows, int cols) {
  const int c8 = cols / 8;
  for (int q = threadIdx.x; q < rows * c8; q += BT) {
    const int r = q / c8, c = (q - r * c8) * 8;
    *reinterpret_cast<u32x4*>(dst + r * pitch + c) = *reinterpret_cast<const u32x4*>(src + (int64_t)r * cols + c);
  }
}

// Row-major global rows [rows, c8 * 8] -> LDS at word offset `off`, pitch
// `pitch`.  Thread t moves chunk t % c8 of rows t / c8 + i * (BT / c8),
// i < MAXC; all its 16-byte loads are issued before the first LDS write, so
// an example's loads are in flight together.  The thread index goes through
// an opaque copy so the offsets are recomputed per call, not hoisted out of
// the example loop (where they would hold registers through every phase).
__host__ __device__ constexpr bool stage_fits(int rows, int c8, int maxc) {
  return c8 <= BT && rows <= maxc * (BT / c8);
}

template <int MAXC>
__device__ __forceinline__ void stage_rows(uint16_t* smem_base, int off, int pitch, const uint16_t* src, int rows,
                                           int c8) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int rpp = BT / c8, r0 = tid / c8, c = (tid - r0 * c8) * 8;
  const bool act = r0 < rpp;
  u32x4 reg[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int r = r0 + i * rpp;
    if (act && r < rows) reg[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * c8 * 8 + c);
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int r = r0 + i * rpp;
    if (act && r < rows) *reinterpret_cast<u32x4*>(smem_base + off + r * pitch + c) = reg[i];
  }
}

// stage_rows in two halves, so the loads can be issued one example ahead:
// fetch_rows puts a thread's chunks in registers, put_rows writes them to LDS.
template <int MAXC>
__device__ __forceinline__ void fetch_rows(u32x4 (&reg)[MAXC], const uint16_t* src, int rows, int c8) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int rpp = BT / c8, r0 = tid / c8, c = (tid - r0 * c8) * 8;
  const bool act = r0 < rpp;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int r = r0 + i * rpp;
    if (act && r < rows) reg[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * c8 * 8 + c);
  }
}

template <int MAXC>
__device__ __forceinline__ void put_rows(const u32x4 (&reg)[MAXC], uint16_t* smem_base, int off, int pitch, int rows,
                                         int c8) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int rpp = BT / c8, r0 = tid / c8, c = (tid - r0 * c8) * 8;
  const bool act = r0 < rpp;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int r = r0 + i * rpp;
    if (act && r < rows) *reinterpret_cast<u32x4*>(smem_base + off + r * pitch + c) = reg[i];
  }
}

// ---------------------------------------------------------------- LDS plans
constexpr int kMaxXChunks = 6;  // 16-byte chunks of X per thread and example
constexpr int kMaxRChunks = 3;  // ... of dLc, and of the FMB rows of dR
constexpr int kMaxFChunks = 2;  // ... of d_Fn (as rows of 4 chunks)
constexpr int kMaxKa = 256;     // the dX product's contraction 2 k + n_l, padded
constexpr int kLcK = 8;         // K steps of W_L X held as registers (n <= 256)

struct OutPlan {  // bwd_out_kernel
  int n32, pd, nlp, g;
  int xs, ys, ms, ls, bytes;  // byte offsets: X, dY, M (bf16, pitch pd), Lc (fp32, pitch d)
};

__host__ __device__ inline int pow2_at_least(int v) {
  int g = 1;
  while (g < v) g <<= 1;
  return g;
}

__host__ __device__ inline OutPlan out_plan(int n, int d, int n_l) {
  OutPlan p;
  p.n32 = up32(n);
  p.pd = up32(d) + 8;
  p.nlp = up16(n_l);
  p.g = pow2_at_least((d + 7) / 8);
  p.xs = 0;
  p.ys = p.xs + p.n32 * p.pd * 2;
  p.ms = p.ys + n * p.pd * 2;
  p.ls = p.ms + (n - n_l) * p.pd * 2;
  const int ls_bytes = p.nlp * d * 4, red_bytes = BW * 2 * d * 4;  // the sums reuse Lc's LDS at the end
  p.bytes = p.ls + (ls_bytes > red_bytes ? ls_bytes : red_bytes);
  return p;
}

struct FmbPlan {  // bwd_fmb_kernel
  int n16, n32, dp, pd, pn, kp, nlp, ka;
  int xs, as, bs, dms, dfs, red, bytes;
};

__host__ __device__ inline FmbPlan fmb_plan(int n, int d, int k, int n_l) {
  FmbPlan p;
  p.n16 = up16(n);
  p.n32 = up32(n);
  p.dp = up32(d);
  p.pd = p.dp + 8;
  p.pn = p.n32 + 8;
  p.kp = up16(k);
  p.nlp = up16(n_l);
  p.ka = up32(2 * p.kp + p.nlp);
  p.xs = 0;
  p.as = p.xs + p.n32 * p.pd * 2;
  p.bs = p.as + p.ka * p.pn * 2;
  p.dms = p.bs + p.ka * p.pd * 2;
  p.dfs = p.dms + (n - n_l) * p.pd * 2;
  p.red = p.dfs + (n * k * 2 + 15) / 16 * 16;
  p.bytes = p.red + 6 * BW * 4;  // block_sum's 2 slots, block_sum2's 2 slots of 2
  return p;
}

// ---------------------------------------------------------------- phase A
struct BwdOutKArgs {
  const uint16_t* x;      // [B, n, d]
  const uint16_t* m;      // [B, n_f, d]
  const uint16_t* dy;     // [B, n, d]
  const uint16_t* w_l;    // [n_l, n]
  const uint16_t* gamma;  // [d] or null
  uint16_t* dm;           // [B, n_f, d]
  uint16_t* dlc;          // [B, n_l, d]
  float* part;            // [gridDim.x, 2 d]
  int64_t batch;
  int n, d, n_f, n_l;
  float eps;
};

template <int G>
__global__ __launch_bounds__(BT) void bwd_out_kernel(BwdOutKArgs p) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int n = p.n, d = p.d, n_f = p.n_f, n_l = p.n_l, d8 = d / 8;
  const OutPlan pl = out_plan(n, d, n_l);
  uint16_t* Xs = smem + pl.xs / 2;
  const uint16_t* Ys = smem + pl.ys / 2;
  const uint16_t* Ms = smem + pl.ms / 2;
  float* Ls = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + pl.ls);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  constexpr int RPW = kWave / G;  // rows per wave and pass
  const int grp = lane / G, c = (lane % G) * 8;
  const bool col_ok = c < d;
  const int row0 = wave * RPW + grp, rstep = BW * RPW;

  zero_lds(smem, pl.ys);  // X's padding rows and columns stay zero
  __syncthreads();

  float gam[8], pg[8], pb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    gam[j] = (p.gamma != nullptr && col_ok) ? bf16_to_f32(p.gamma[c + j]) : 1.f;
    pg[j] = 0.f;
    pb[j] = 0.f;
  }
  const int dt = d / 16, tiles = (pl.nlp / 16) * dt;
  const float inv_d = 1.f / (float)d;
  // W_L as MFMA A operands, loaded once: wave w computes Lc row block w % rb_n
  // for the column blocks w / rb_n, + wpr, ...  (when every row block has a
  // wave and n <= 32 kLcK; otherwise each tile reads W_L from L2).  Loads of
  // W_L inside the example loop would queue behind the next example's
  // prefetch on the in-order vector-memory counter.
  const int rb_n = pl.nlp / 16;
  const bool cached = rb_n <= BW && pl.n32 <= 32 * kLcK;
  const int wpr = cached ? BW / rb_n : 1, my_rb = wave % rb_n, my_slot = wave / rb_n;
  u32x4 wa[kLcK];
#pragma unroll
  for (int kk = 0; kk < kLcK; ++kk) {
    const int wr = my_rb * 16 + li, kc = kk * 32 + 8 * lg;
    wa[kk] = (cached && kk * 32 < pl.n32 && wr < n_l && kc < n) ? *reinterpret_cast<const u32x4*>(p.w_l + wr * n + kc)
                                                               : u32x4{0u, 0u, 0u, 0u};
  }

  // X, dY and M of an example in one burst of loads, issued one example ahead
  u32x4 gx[kMaxXChunks], gy[kMaxXChunks], gm[kMaxRChunks];
  auto fetch_example = [&](int64_t e) {
    fetch_rows(gx, p.x + e * n * d, n, d8);
    fetch_rows(gy, p.dy + e * n * d, n, d8);
    fetch_rows(gm, p.m + e * n_f * d, n_f, d8);
  };
  if ((int64_t)blockIdx.x < p.batch) fetch_example(blockIdx.x);
  for (int64_t b = blockIdx.x; b < p.batch; b += gridDim.x) {
    put_rows(gx, smem, pl.xs / 2, pl.pd, n, d8);
    put_rows(gy, smem, pl.ys / 2, pl.pd, n, d8);
    put_rows(gm, smem, pl.ms / 2, pl.pd, n_f, d8);
    lds_barrier();
    {
      const int64_t nb = b + gridDim.x;
      if (nb < p.batch) fetch_example(nb);
    }
    // Lc = W_L X -> Ls (fp32)
    if (cached) {
      if (my_slot < wpr) {
        for (int cb = my_slot; cb < dt; cb += wpr) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < kLcK; ++kk)
            if (kk * 32 < pl.n32) acc = mfma16x16x32(wa[kk], tr_op(Xs, pl.pd, kk * 32, cb * 16, li, lg), acc);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = my_rb * 16 + 4 * lg + q;
            if (r < n_l) Ls[r * d + cb * 16 + li] = acc[q];
          }
        }
      }
    } else {
      for (int t = wave; t < tiles; t += BW) {
        const int rb = t / dt, cb = t - rb * dt;
        const int wr = rb * 16 + li;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < pl.n32; k0 += 32) {
          const int kc = k0 + 8 * lg;
          const u32x4 a = (wr < n_l && kc < n) ? *reinterpret_cast<const u32x4*>(p.w_l + wr * n + kc)
                                               : u32x4{0u, 0u, 0u, 0u};
          acc = mfma16x16x32(a, tr_op(Xs, pl.pd, k0, cb * 16, li, lg), acc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rb * 16 + 4 * lg + q;
          if (r < n_l) Ls[r * d + cb * 16 + li] = acc[q];
        }
      }
    }
    lds_barrier();
    // rows: R = [M; Lc] + X, LayerNorm backward (all operands in LDS)
    for (int r = row0; r < n; r += rstep) {  // uniform over the lane group
      float R[8], dyv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) R[e] = dyv[e] = 0.f;
      if (col_ok) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(Xs + r * pl.pd + c);
        const u32x4 yv = *reinterpret_cast<const u32x4*>(Ys + r * pl.pd + c);
        if (r < n_f) {
          const u32x4 mv = *reinterpret_cast<const u32x4*>(Ms + r * pl.pd + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            R[2 * e] = bf16lo(mv[e]) + bf16lo(xv[e]);
            R[2 * e + 1] = bf16hi(mv[e]) + bf16hi(xv[e]);
          }
        } else {
          const float* lr = Ls + (r - n_f) * d + c;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            R[2 * e] = lr[2 * e] + bf16lo(xv[e]);
            R[2 * e + 1] = lr[2 * e + 1] + bf16hi(xv[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dyv[2 * e] = bf16lo(yv[e]);
          dyv[2 * e + 1] = bf16hi(yv[e]);
        }
      }
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += R[e];
      const float mean = group_sum_v<G>(s) * inv_d;
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = col_ok ? R[e] - mean : 0.f;
        v += t * t;
      }
      const float rstd = rsqrtf(group_sum_v<G>(v) * inv_d + p.eps);
      float s1 = 0.f, s2 = 0.f, rh[8], g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rh[e] = (R[e] - mean) * rstd;
        g[e] = dyv[e] * gam[e];
        s1 += g[e];
        s2 += g[e] * rh[e];
      }
      const float m1 = group_sum_v<G>(s1) * inv_d, m2 = group_sum_v<G>(s2) * inv_d;
      if (col_ok) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(rstd * (g[2 * e] - m1 - rh[2 * e] * m2), rstd * (g[2 * e + 1] - m1 - rh[2 * e + 1] * m2));
        uint16_t* dst = r < n_f ? p.dm + (b * n_f + r) * d + c : p.dlc + (b * n_l + (r - n_f)) * d + c;
        *reinterpret_cast<u32x4*>(dst) = o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pg[e] += dyv[e] * rh[e];
          pb[e] += dyv[e];
        }
      }
    }
    lds_barrier();
  }
  // per-workgroup sums: lanes sharing columns (one per row group), then waves in order
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int mk = G; mk < kWave; mk <<= 1) {
      pg[j] += __shfl_xor(pg[j], mk, kWave);
      pb[j] += __shfl_xor(pb[j], mk, kWave);
    }
  }
  float* red = Ls;
  if (lane < G && col_ok) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      red[(wave * 2) * d + c + j] = pg[j];
      red[(wave * 2 + 1) * d + c + j] = pb[j];
    }
  }
  __syncthreads();
  for (int j = tid; j < 2 * d; j += BT) {
    const int which = j / d, e = j - which * d;
    float s = 0.f;
    for (int w = 0; w < BW; ++w) s += red[(w * 2 + which) * d + e];
    p.part[(int64_t)blockIdx.x * 2 * d + j] = s;
  }
}

// ---------------------------------------------------------------- phase B
struct BwdFmbKArgs {
  const uint16_t* x;         // [B, n, d]
  const uint16_t* dfn;       // [B, n k]
  const uint16_t* dm;        // [B, n_f, d]
  const uint16_t* dlc;       // [B, n_l, d]
  const uint16_t* phi;       // [k, n]
  const uint16_t* w_l;       // [n_l, n]
  const uint16_t* fm_gamma;  // [n k] or null
  uint16_t* dx;              // [B, n, d]
  float* part;               // [gridDim.x, k n + n_l n + 2 n k]
  int64_t batch;
  int n, d, k, n_f, n_l;
  float eps;
};

template <int QF, int QP, int QL>
__global__ __launch_bounds__(BT) void bwd_fmb_kernel(BwdFmbKArgs p) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int n = p.n, d = p.d, k = p.k, n_f = p.n_f, n_l = p.n_l;
  const FmbPlan pl = fmb_plan(n, d, k, n_l);
  uint16_t* Xs = smem + pl.xs / 2;    // X; after the weight sums, the dX tile staging
  uint16_t* As = smem + pl.as / 2;    // rows [0,kp) dF^T, [kp,2kp) Phi, [2kp,2kp+nlp) W_L
  uint16_t* Bs = smem + pl.bs / 2;    // rows [0,kp) Z, [kp,2kp) dZ, [2kp,2kp+nlp) dLc
  uint16_t* DMs = smem + pl.dms / 2;  // dR rows < n_f
  uint16_t* DFs = smem + pl.dfs / 2;  // d_Fn
  float* red = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + pl.red);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int kp = pl.kp, nk = n * k, d8 = d / 8;
  const int ib_n = pl.n16 / 16, jb_n = kp / 16, cb_n = d / 16;
  const int tilesF = ib_n * jb_n, tilesP = jb_n * ib_n, tilesL = (pl.nlp / 16) * ib_n;
  const float inv_nk = 1.f / (float)nk;

  zero_lds(smem, pl.red);
  __syncthreads();
  load_rows(As + kp * pl.pn, pl.pn, p.phi, k, n);
  load_rows(As + 2 * kp * pl.pn, pl.pn, p.w_l, n_l, n);

  f32x4 accP[QP], accL[QL], pgam[QF], pbet[QF], gfm[QF];
#pragma unroll
  for (int q = 0; q < QP; ++q) accP[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < QL; ++q) accL[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // gamma_fm at this lane's F positions (the same for every example)
#pragma unroll
  for (int q = 0; q < QF; ++q) {
    pgam[q] = pbet[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    gfm[q] = f32x4{1.f, 1.f, 1.f, 1.f};
    const int t = wave + q * BW;
    if (t < tilesF && p.fm_gamma != nullptr) {
      const int ib = t / jb_n, jb = t - ib * jb_n;
      const int j = jb * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * lg + r;
        if (i < n && j < k) gfm[q][r] = bf16_to_f32(p.fm_gamma[i * k + j]);
      }
    }
  }

  int slot = 0, slot2 = 0;
  float* red2 = red + 2 * BW;
  // an example's inputs: X, dLc, the FMB rows of dR, d_Fn; fetched one example
  // ahead (during the previous example's dX phase) and written to LDS here
  u32x4 gx[kMaxXChunks], gl[kMaxRChunks], gm[kMaxRChunks], gf[kMaxFChunks];
  auto fetch_example = [&](int64_t e) {
    fetch_rows(gx, p.x + e * n * d, n, d8);
    fetch_rows(gl, p.dlc + e * n_l * d, n_l, d8);
    fetch_rows(gm, p.dm + e * n_f * d, n_f, d8);
    fetch_rows(gf, p.dfn + e * nk, nk / 32, 4);
  };
  if ((int64_t)blockIdx.x < p.batch) fetch_example(blockIdx.x);
  for (int64_t b = blockIdx.x; b < p.batch; b += gridDim.x) {
    put_rows(gx, smem, pl.xs / 2, pl.pd, n, d8);
    put_rows(gl, smem, pl.bs / 2 + 2 * kp * pl.pd, pl.pd, n_l, d8);
    put_rows(gm, smem, pl.dms / 2, pl.pd, n_f, d8);
    put_rows(gf, smem, pl.dfs / 2, 32, nk / 32, 4);
    lds_barrier();
    // Z = Phi X -> Bs rows [0, kp)
    for (int t = wave; t < jb_n * cb_n; t += BW) {
      const int rb = t / cb_n, cb = t - rb * cb_n;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < pl.n32; k0 += 32)
        acc = mfma16x16x32(row_op(As, pl.pn, kp + rb * 16, k0, li, lg), tr_op(Xs, pl.pd, k0, cb * 16, li, lg), acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[(rb * 16 + 4 * lg + q) * pl.pd + cb * 16 + li] = to_bf16(acc[q]);
    }
    lds_barrier();
    // F = X Z^T, this wave's tiles in registers
    f32x4 F[QF];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < QF; ++q) {
      F[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = wave + q * BW;
      if (t < tilesF) {
        const int ib = t / jb_n, jb = t - ib * jb_n;
        for (int k0 = 0; k0 < pl.dp; k0 += 32)
          F[q] = mfma16x16x32(row_op(Xs, pl.pd, ib * 16, k0, li, lg), row_op(Bs, pl.pd, jb * 16, k0, li, lg), F[q]);
        // padded rows / columns of F are exactly 0 and add nothing
#pragma unroll
        for (int r = 0; r < 4; ++r) s += F[q][r];
      }
    }
    const float mean = block_sum(s, red, slot) * inv_nk;
    slot ^= 1;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < QF; ++q) {
      const int t = wave + q * BW;
      if (t < tilesF) {
        const int ib = t / jb_n, jb = t - ib * jb_n;
        const int j = jb * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = ib * 16 + 4 * lg + r;
          const float e = (i < n && j < k) ? F[q][r] - mean : 0.f;
          v += e * e;
        }
      }
    }
    const float rstd = rsqrtf(block_sum(v, red, slot) * inv_nk + p.eps);
    slot ^= 1;
    // F -> F_tilde; means of q = d_Fn gamma_fm and of q F_tilde
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QF; ++q) {
      const int t = wave + q * BW;
      if (t < tilesF) {
        const int ib = t / jb_n, jb = t - ib * jb_n;
        const int j = jb * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = ib * 16 + 4 * lg + r;
          if (i < n && j < k) {
            const float g = bf16_to_f32(DFs[i * k + j]) * gfm[q][r];
            const float ft = (F[q][r] - mean) * rstd;
            F[q][r] = ft;
            s1 += g;
            s2 += g * ft;
          } else {
            F[q][r] = 0.f;
          }
        }
      }
    }
    block_sum2(s1, s2, red2, slot2);
    slot2 ^= 1;
    s1 *= inv_nk;
    s2 *= inv_nk;
    // dF^T -> As rows [0, kp) (zeros at padding), FM LayerNorm parameter sums
#pragma unroll
    for (int q = 0; q < QF; ++q) {
      const int t = wave + q * BW;
      if (t < tilesF) {
        const int ib = t / jb_n, jb = t - ib * jb_n;
        const int j = jb * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = ib * 16 + 4 * lg + r;
          float df = 0.f;
          if (i < n && j < k) {
            const float gn = bf16_to_f32(DFs[i * k + j]);
            df = rstd * (gn * gfm[q][r] - s1 - F[q][r] * s2);
            pgam[q][r] += gn * F[q][r];
            pbet[q][r] += gn;
          }
          As[j * pl.pn + i] = to_bf16(df);
        }
      }
    }
    lds_barrier();
    // dZ = dF^T X -> Bs rows [kp, 2kp)
    for (int t = wave; t < jb_n * cb_n; t += BW) {
      const int rb = t / cb_n, cb = t - rb * cb_n;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < pl.n32; k0 += 32)
        acc = mfma16x16x32(row_op(As, pl.pn, rb * 16, k0, li, lg), tr_op(Xs, pl.pd, k0, cb * 16, li, lg), acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[(kp + rb * 16 + 4 * lg + q) * pl.pd + cb * 16 + li] = to_bf16(acc[q]);
    }
    lds_barrier();
    // d_Phi += dZ X^T, d_W_L += dLc X^T
#pragma unroll
    for (int q = 0; q < QP; ++q) {
      const int t = wave + q * BW;
      if (t < tilesP) {
        const int rb = t / ib_n, ib = t - rb * ib_n;
        for (int k0 = 0; k0 < pl.dp; k0 += 32)
          accP[q] = mfma16x16x32(row_op(Bs, pl.pd, kp + rb * 16, k0, li, lg), row_op(Xs, pl.pd, ib * 16, k0, li, lg),
                                 accP[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      const int t = wave + q * BW;
      if (t < tilesL) {
        const int rb = t / ib_n, ib = t - rb * ib_n;
        for (int k0 = 0; k0 < pl.dp; k0 += 32)
          accL[q] = mfma16x16x32(row_op(Bs, pl.pd, 2 * kp + rb * 16, k0, li, lg),
                                 row_op(Xs, pl.pd, ib * 16, k0, li, lg), accL[q]);
      }
    }
    lds_barrier();  // X no longer read: its LDS takes the dX tiles
    {
      const int64_t nb = b + gridDim.x;
      if (nb < p.batch) fetch_example(nb);
    }
    // dX = dR + [dF | Phi^T | W_L^T] [Z; dZ; dLc] -> Xs (bf16); a wave owns
    // 16-row blocks and keeps their A operands for every column tile
    for (int ib = wave; ib < ib_n; ib += BW) {
      u32x4 af[kMaxKa / 32];
#pragma unroll
      for (int kk = 0; kk < kMaxKa / 32; ++kk)
        if (kk * 32 < pl.ka) af[kk] = tr_op(As, pl.pn, kk * 32, ib * 16, li, lg);
      for (int cb = 0; cb < cb_n; ++cb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kMaxKa / 32; ++kk)
          if (kk * 32 < pl.ka) acc = mfma16x16x32(af[kk], tr_op(Bs, pl.pd, kk * 32, cb * 16, li, lg), acc);
        const int e = cb * 16 + li;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = ib * 16 + 4 * lg + q;
          if (i < n) {
            const float res =
                i < n_f ? bf16_to_f32(DMs[i * pl.pd + e]) : bf16_to_f32(Bs[(2 * kp + i - n_f) * pl.pd + e]);
            Xs[i * pl.pd + e] = to_bf16(acc[q] + res);
          }
        }
      }
    }
    lds_barrier();
    uint16_t* dxb = p.dx + b * n * d;
    for (int q = tid; q < n * d8; q += BT) {
      const int r = q / d8, c = (q - r * d8) * 8;
      *reinterpret_cast<u32x4*>(dxb + r * d + c) = *reinterpret_cast<const u32x4*>(Xs + r * pl.pd + c);
    }
    lds_barrier();
  }
  // this workgroup's plane: d_Phi [k, n], d_W_L [n_l, n], d_gamma_fm [n k], d_beta_fm [n k]
  float* out = p.part + (int64_t)blockIdx.x * (k * n + n_l * n + 2 * nk);
#pragma unroll
  for (int q = 0; q < QP; ++q) {
    const int t = wave + q * BW;
    if (t < tilesP) {
      const int rb = t / ib_n, ib = t - rb * ib_n;
      const int i = ib * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = rb * 16 + 4 * lg + r;
        if (j < k && i < n) out[j * n + i] = accP[q][r];
      }
    }
  }
  out += k * n;
#pragma unroll
  for (int q = 0; q < QL; ++q) {
    const int t = wave + q * BW;
    if (t < tilesL) {
      const int rb = t / ib_n, ib = t - rb * ib_n;
      const int i = ib * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = rb * 16 + 4 * lg + r;
        if (j < n_l && i < n) out[j * n + i] = accL[q][r];
      }
    }
  }
  out += n_l * n;
#pragma unroll
  for (int q = 0; q < QF; ++q) {
    const int t = wave + q * BW;
    if (t < tilesF) {
      const int ib = t / jb_n, jb = t - ib * jb_n;
      const int j = jb * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * lg + r;
        if (i < n && j < k) {
          out[i * k + j] = pgam[q][r];
          out[nk + i * k + j] = pbet[q][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- transposes and sums
// at[c][r] = a[r][c] for r < R and 0 for R <= r < Rp (Rp % 8 == 0); when
// colpart is set, colpart[tile row][c] = sum of the tile's 64 rows of column c.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* a, int64_t R, int C, int64_t Rp,
                                                             uint16_t* at, float* colpart) {
  __shared__ __align__(16) uint16_t t[64][72];
  const int c0 = blockIdx.x * 64;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int rr = q >> 3, cc = (q & 7) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r0 + rr < R && c0 + cc < C) v = *reinterpret_cast<const u32x4*>(a + (r0 + rr) * C + c0 + cc);
    *reinterpret_cast<u32x4*>(&t[rr][cc]) = v;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int oc = q >> 3, rr = (q & 7) * 8;
    uint32_t w[4];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t lo = t[rr + 2 * j][oc], hi = t[rr + 2 * j + 1][oc];
      w[j] = (uint32_t)lo | ((uint32_t)hi << 16);
      s += bf16_to_f32(lo) + bf16_to_f32(hi);
    }
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 4, kWave);
    if (c0 + oc < C) {
      if (r0 + rr < Rp) *reinterpret_cast<u32x4*>(at + (int64_t)(c0 + oc) * Rp + r0 + rr) = u32x4{w[0], w[1], w[2], w[3]};
      if (colpart != nullptr && (q & 7) == 0) colpart[(int64_t)blockIdx.y * C + c0 + oc] = s;
    }
  }
}

__global__ __launch_bounds__(256) void sum_planes_kernel(const float* part, int planes, int64_t stride, int64_t len,
                                                         float* out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < len; i += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int q = 0; q < planes; ++q) s += part[(int64_t)q * stride + i];
    out[i] = s;
  }
}

// 32 columns per workgroup; thread (column c, slice s) adds planes s, s + 8,
// ... in order, then the 8 slices are added in order s = 0 .. 7.
__global__ __launch_bounds__(256) void sum_many_planes_kernel(const float* part, int planes, int64_t stride,
                                                              int64_t len, float* out) {
  __shared__ float red[8][33];
  const int c = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int64_t col = (int64_t)blockIdx.x * 32 + c;
  float v = 0.f;
  if (col < len) {
#pragma unroll 4
    for (int q = sl; q < planes; q += 8) v += part[(int64_t)q * stride + col];
  }
  red[sl][c] = v;
  __syncthreads();
  if (sl == 0 && col < len) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i][c];
    out[col] = s;
  }
}

// Several plane sums in one launch: segment i covers workgroups first[i] ..
// first[i + 1] - 1, 32 columns each, summed exactly as sum_many_planes_kernel.
struct PlaneSegsK {
  PlaneSeg seg[kMaxPlaneSegs];
  int64_t first[kMaxPlaneSegs + 1];
  int nseg, planes;
};
__global__ __launch_bounds__(256) void sum_planes_multi_kernel(PlaneSegsK a) {
  __shared__ float red[8][33];
  int i = 0;
  while (i + 1 < a.nseg && (int64_t)blockIdx.x >= a.first[i + 1]) ++i;  // uniform
  const PlaneSeg sg = a.seg[i];
  const int c = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int64_t col = ((int64_t)blockIdx.x - a.first[i]) * 32 + c;
  float v = 0.f;
  if (col < sg.len) {
#pragma unroll 4
    for (int q = sl; q < a.planes; q += 8) v += sg.part[(int64_t)q * sg.stride + col];
  }
  red[sl][c] = v;
  __syncthreads();
  if (sl == 0 && col < sg.len) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += red[k][c];
    sg.out[col] = t;
  }
}

int workgroups_for(int64_t batch) { return (int)(batch < 256 ? batch : 256); }

// Lets a kernel take the whole 160 KB of LDS as dynamic shared memory (a host-side attribute, set per launch).
template <class K>
hipError_t allow_lds(K* kern) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
}

}  // namespace

// ---------------------------------------------------------------- host side
namespace {
bool fmb_tiles_fit(const FmbPlan& f) {
  const int ib = f.n16 / 16;
  return ib * (f.kp / 16) <= kQF * BW && (f.kp / 16) * ib <= kQP * BW && (f.nlp / 16) * ib <= kQL * BW;
}
}  // namespace

namespace {
// The shapes bwd_out_kernel takes: its LDS plan, X staging and LayerNorm rows fit.
bool out_supported(int n, int d, int n_l) {
  if (n <= 0 || d <= 0 || n_l <= 0 || n_l >= n || d % 16 || n % 8 || d > 512) return false;
  const OutPlan a = out_plan(n, d, n_l);
  return a.bytes <= kLdsMax && stage_fits(n, d / 8, kMaxXChunks) && stage_fits(n - n_l, d / 8, kMaxRChunks);
}

// The shapes bwd_fmb_kernel takes: its LDS plan, staging and register tiles fit.
bool fmb_supported(int n, int d, int k, int n_l) {
  if (n <= 0 || d <= 0 || k <= 0 || n_l <= 0 || n_l >= n || d % 16 || n % 8) return false;
  const FmbPlan f = fmb_plan(n, d, k, n_l);
  if (f.bytes > kLdsMax || f.ka > kMaxKa) return false;
  if (!stage_fits(n, d / 8, kMaxXChunks) || !stage_fits(n - n_l, d / 8, kMaxRChunks) ||
      !stage_fits(n_l, d / 8, kMaxRChunks) || (n * k) % 32 || !stage_fits(n * k / 32, 4, kMaxFChunks))
    return false;
  return fmb_tiles_fit(f);
}
}  // namespace

bool wukong_bwd_supported(int n, int d, int k, int n_l) { return out_supported(n, d, n_l) && fmb_supported(n, d, k, n_l); }

int wukong_bwd_workgroups(int64_t batch) { return workgroups_for(batch); }

size_t wukong_bwd_out_part_floats(int d) { return (size_t)2 * d; }
size_t wukong_bwd_fmb_part_floats(int n, int k, int n_l) { return (size_t)k * n + (size_t)n_l * n + 2 * (size_t)n * k; }

hipError_t launch_bwd_out(const BwdOutArgs& a, hipStream_t stream, int64_t* workgroups) {
  if (!out_supported(a.n, a.d, a.n_l)) return hipErrorInvalidValue;
  const int grid = workgroups_for(a.batch);
  if (workgroups) *workgroups = grid;
  if (grid == 0) return hipSuccess;
  BwdOutKArgs k;
  k.x = static_cast<const uint16_t*>(a.x);
  k.m = static_cast<const uint16_t*>(a.m);
  k.dy = static_cast<const uint16_t*>(a.dy);
  k.w_l = static_cast<const uint16_t*>(a.w_l);
  k.gamma = static_cast<const uint16_t*>(a.gamma);
  k.dm = static_cast<uint16_t*>(a.dm);
  k.dlc = static_cast<uint16_t*>(a.dlc);
  k.part = a.part;
  k.batch = a.batch;
  k.n = a.n;
  k.d = a.d;
  k.n_f = a.n - a.n_l;
  k.n_l = a.n_l;
  k.eps = a.eps;
  const OutPlan pl = out_plan(a.n, a.d, a.n_l);
  void (*kern)(BwdOutKArgs) = nullptr;
  switch (pl.g) {
    case 2: kern = bwd_out_kernel<2>; break;
    case 4: kern = bwd_out_kernel<4>; break;
    case 8: kern = bwd_out_kernel<8>; break;
    case 16: kern = bwd_out_kernel<16>; break;
    case 32: kern = bwd_out_kernel<32>; break;
    case 64: kern = bwd_out_kernel<64>; break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = allow_lds(kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(BT), pl.bytes, stream, k);
  return hipGetLastError();
}

hipError_t launch_bwd_fmb(const BwdFmbArgs& a, hipStream_t stream, int64_t* workgroups) {
  if (!fmb_supported(a.n, a.d, a.k, a.n_l)) return hipErrorInvalidValue;
  const int grid = workgroups_for(a.batch);
  if (workgroups) *workgroups = grid;
  if (grid == 0) return hipSuccess;
  BwdFmbKArgs k;
  k.x = static_cast<const uint16_t*>(a.x);
  k.dfn = static_cast<const uint16_t*>(a.dfn);
  k.dm = static_cast<const uint16_t*>(a.dm);
  k.dlc = static_cast<const uint16_t*>(a.dlc);
  k.phi = static_cast<const uint16_t*>(a.phi);
  k.w_l = static_cast<const uint16_t*>(a.w_l);
  k.fm_gamma = static_cast<const uint16_t*>(a.fm_gamma);
  k.dx = static_cast<uint16_t*>(a.dx);
  k.part = a.part;
  k.batch = a.batch;
  k.n = a.n;
  k.d = a.d;
  k.k = a.k;
  k.n_f = a.n - a.n_l;
  k.n_l = a.n_l;
  k.eps = a.eps;
  const FmbPlan pl = fmb_plan(a.n, a.d, a.k, a.n_l);
  void (*kern)(BwdFmbKArgs) = bwd_fmb_kernel<kQF, kQP, kQL>;
  const hipError_t e = allow_lds(kern);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(BT), pl.bytes, stream, k);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* a, int64_t R, int C, int64_t Rp, void* at, float* colpart,
                                 hipStream_t stream, int64_t* workgroups) {
  if (R < 0 || C <= 0 || C % 8 || Rp < R || Rp % 8) return hipErrorInvalidValue;
  const int64_t gy = (Rp + 63) / 64;
  if (gy > 65535) return hipErrorInvalidValue;
  const unsigned gx = (unsigned)((C + 63) / 64);
  if (workgroups) *workgroups = (int64_t)gx * gy;
  if (gy == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(gx, (unsigned)gy), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a), R, C, Rp, static_cast<uint16_t*>(at), colpart);
  return hipGetLastError();
}

hipError_t launch_sum_planes_strided(const float* part, int planes, int64_t stride, int64_t len, float* out,
                                     hipStream_t stream) {
  if (planes < 1 || len < 0 || stride < len) return hipErrorInvalidValue;
  if (len == 0) return hipSuccess;
  if (planes > 8) {  // many planes: 8 threads per column, each over every 8th plane
    const int64_t grid = (len + 31) / 32;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sum_many_planes_kernel, dim3((unsigned)grid), dim3(256), 0, stream, part, planes, stride, len,
                       out);
    return hipGetLastError();
  }
  int64_t grid = (len + 255) / 256;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(sum_planes_kernel, dim3((unsigned)grid), dim3(256), 0, stream, part, planes, stride, len, out);
  return hipGetLastError();
}

hipError_t launch_sum_planes_multi(const PlaneSeg* segs, int nseg, int planes, hipStream_t stream,
                                   int64_t* workgroups) {
  if (nseg < 0 || nseg > kMaxPlaneSegs || planes < 1) return hipErrorInvalidValue;
  PlaneSegsK a;
  a.nseg = 0;
  a.planes = planes;
  int64_t blocks = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].len < 0 || segs[i].stride < segs[i].len) return hipErrorInvalidValue;
    if (segs[i].len == 0 || segs[i].out == nullptr) continue;
    a.seg[a.nseg] = segs[i];
    a.first[a.nseg] = blocks;
    blocks += (segs[i].len + 31) / 32;
    ++a.nseg;
  }
  a.first[a.nseg] = blocks;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sum_planes_multi_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sum_planes(const float* part, int planes, int64_t len, float* out, hipStream_t stream) {
  return launch_sum_planes_strided(part, planes, len, len, out, stream);
}

}  // namespace wk
