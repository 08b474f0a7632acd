// FMB-MLP Linear on bf16 MFMA: C[M, N] = act(A[M, K] W[N, K]^T + bias[N]),
// and the last Linear fused with the layer output stage (linear_ln_kernel).
//
// The FMB's MLP (Wukong paper, section 2.2; its depth and widths are the
// "MLP" scaling knob of section 2.3) is where nearly all of a Wukong layer's
// FLOPs go, so this is a plain dense contraction on bf16 MFMA with fp32
// accumulation.  A is the activation (row-major, K contiguous) and W keeps
// torch.nn.Linear's [out, in] layout, so both operands are K-contiguous and
// land in LDS the same way: rows of 64 bf16 (128 B) whose 16-byte chunk c of
// row r is stored at c ^ ((r >> 1) & 7), which keeps the DMA writes and the
// 16-row MFMA fragment reads free of bank conflicts.  Each wave computes
// W_tile x A_tile^T, i.e. the transposed tile, so a lane ends up holding 4
// consecutive output columns of one row and stores 8 bytes at a time.
//
// Tile order: the hardware deals workgroup i to XCD i % 8; the logical tile
// index is remapped so each XCD gets a contiguous run of tiles, walked in
// groups of 8 tile-rows so that neighbouring tiles share A and W panels in
// that XCD's L2.
//
// Kernels:
//  * linear_dma_kernel (K % 64 == 0, the fast path): v_mfma_f32_16x16x32_bf16,
//    operands moved global -> LDS by buffer_load ... lds (no staging
//    registers), two static LDS stages so the next K tile streams in while the
//    current one is consumed.  Each workgroup's buffer resources start at its
//    tile's first row and end at the last valid row, so rows past M or N read
//    as zero.  Barriers are LDS-scoped (they do not wait for global loads).
//  * linear_ln_kernel: the same main loop on 256 x 320 tiles, whose epilogue
//    is the layer's output stage for the FMB rows (bias, residual, LayerNorm).
//  * linear_bf16_kernel (any K % 8 == 0): 32x32x16 MFMA, register-staged
//    loads with per-element bounds checks.
#include <mutex>

#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

struct LinearKArgs {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* bias;
  uint16_t* c;
  int64_t M;
  int N, K;
  int act;                // LinearAct
  const uint16_t* res;    // [M, N] added after the activation (kActReluMask: the mask), or null
  int tiles_m, tiles_n;
  int64_t a_kb_rows = 0;  // > 0: A is K-blocked (see LinearArgs::a_kblock_rows)
};

// The residual input: added after the activation, or, for kActReluMask, the
// mask source (outputs where it is not positive become 0).
__device__ __forceinline__ float apply_res(float v, float r, int act) {
  if (act == kActReluMask) return r > 0.f ? v : 0.f;
  return v + r;
}

__device__ __forceinline__ float apply_act(float v, int act) {
  if (act == kActRelu) return fmaxf(v, 0.f);
  if (act == kActSiluGate) return silu_gate(v);
  return v;
}

struct LinearLnKArgs {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* bias;
  const uint16_t* x;      // residual: row m at x + m * ld
  const uint16_t* gamma;  // [D] or null
  const uint16_t* beta;   // [D] or null
  uint16_t* y;            // row m at y + m * ld
  uint16_t* m_out;        // the bf16 GEMM output M, row m at m_out + m * N (MOUT kernels only)
  int64_t M;
  int N, K;
  int64_t ld;
  float eps;
  int tiles_m, tiles_n;
};

constexpr int kBK = 64;

#define WK_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) alone, and lgkmcnt(0) alone
constexpr int vm_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int lgkm_wait0() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }

__device__ __forceinline__ int swz(int row, int ch) { return row * kBK + ((ch ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ void tile_origin_at(int bid, int nblk, int tiles_m, int tiles_n, int BM, int BN,
                                               int64_t& m0, int& n0) {
  const int full = nblk & ~7;
  int logical = bid;
  if (bid < full) logical = (bid & 7) * (full >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_g = logical - group * per_group;
  m0 = (int64_t)(first_m + in_g % gsz) * BM;
  n0 = (in_g / gsz) * BN;
}
__device__ __forceinline__ void tile_origin(int tiles_m, int tiles_n, int BM, int BN, int64_t& m0, int& n0) {
  tile_origin_at(blockIdx.x, gridDim.x, tiles_m, tiles_n, BM, BN, m0, n0);
}


// The K loop of the DMA kernels: acc[i][j] (lane (l16, lg)) ends holding
// C[m0 + wm WTM + 16 j + l16][n0 + wn WTN + 16 i + 4 lg + t], t = 0..3.
// MFMA / VMEM interleave for the scheduler: MPER MFMAs, then one VMEM read, N times.
template <int N, int MPER>
__device__ __forceinline__ void interleave_mfma_vmem() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPER, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    interleave_mfma_vmem<N - 1, MPER>();
  }
}

// SPREAD: the next stage's DMA is issued between the first half-step's MFMAs
// instead of in one burst, and the stage loop has no branch (K % 128 == 0;
// the DMA issued after the last stage reads the rows' next 64 columns or
// zeros past the resource and lands in a stage nobody reads).
// a_kb_rows > 0: A is K-blocked, element (m, c) at ((c / 64) a_kb_rows + m) 64 + c % 64
// (a_kb_rows >= every row a tile reads, K % 64 == 0): a tile's 64-column step of A is
// then one contiguous run of BM x 128 bytes instead of BM rows K x 2 bytes apart.
// PRIO: the wave raises its issue priority while it issues a stage's MFMAs (s_setprio),
// so the SIMD's other wave's fragment reads and copies do not interleave with them
// (measured: the plain Linears 1-6 % faster; the Linear with the output LayerNorm
// 1-3 % slower, so it keeps the default).
template <int BM, int BN, int WGM, int WGN, bool SPREAD = false, bool PRIO = false>
__device__ __forceinline__ void dma_mainloop(const uint16_t* a_base, const uint16_t* w_base, int64_t M, int N,
                                             int K, int64_t m0, int n0, uint16_t* sA0, uint16_t* sW0,
                                             uint16_t* sA1, uint16_t* sW1,
                                             f32x4 (&acc)[BN / WGN / 16][BM / WGM / 16], int kbeg = 0,
                                             int klen = -1, int64_t a_kb_rows = 0) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int A_INS = BM / 8 / NW, W_INS = BN / 8 / NW;  // 1 KB (8 rows) DMA instructions per wave
  static_assert(A_INS * NW * 8 == BM && W_INS * NW * 8 == BN, "tile / wave mismatch");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int rows_a = (int)min<int64_t>(BM, M - m0), rows_w = min(BN, N - n0);
  const bool akb = a_kb_rows > 0;  // uniform
  // K-blocked A: the resource runs from the tile's first row of block 0 to the end of the
  // array; rows past M hold whatever the producer left there and only feed output rows
  // that are never stored
  // (readfirstlane: the compiler cannot tell the select is uniform, and a resource it takes
  // for divergent turns every DMA into a loop over lanes)
  const int a_bytes = __builtin_amdgcn_readfirstlane(
      akb ? (int)min<int64_t>((a_kb_rows * K - m0 * kBK) * 2, 0x7fffffff) : rows_a * K * 2);
  const int a_row = __builtin_amdgcn_readfirstlane(akb ? kBK : K);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a_base + m0 * a_row), (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w_base + (int64_t)n0 * K), (short)0, rows_w * K * 2, 0x00020000);
  // A DMA instruction writes 64 lanes x 16 B = 8 LDS rows; lane -> row lane/8,
  // LDS chunk lane%8, which holds global chunk (lane%8) ^ swizzle(row).  The
  // swizzle of row 8b + r is (4(b & 1) + r/2) & 7: two lane offsets suffice.
  const int lrow = lane >> 3, lpos = lane & 7;
  const uint32_t voff0 = (uint32_t)(lrow * K + ((lpos ^ (lrow >> 1)) << 3)) * 2u;
  const uint32_t voff1 = (uint32_t)(lrow * K + ((lpos ^ (4 + (lrow >> 1))) << 3)) * 2u;
  const uint32_t blk_bytes = (uint32_t)(16 * K);
  // A's rows are a_row elements apart: K, or 64 when K-blocked
  const uint32_t avoff0 = (uint32_t)(lrow * a_row + ((lpos ^ (lrow >> 1)) << 3)) * 2u;
  const uint32_t avoff1 = (uint32_t)(lrow * a_row + ((lpos ^ (4 + (lrow >> 1))) << 3)) * 2u;
  const uint32_t ablk_bytes = (uint32_t)(16 * a_row);
  // A K range that ends in half a step (K % 64 == 32, never K-blocked): in the last step the
  // lanes of columns 32..63 read zero (an offset past every record count)
  // instead of the next row's first columns.
  const int kspan = klen < 0 ? K : klen;
  const bool hi0 = (lpos ^ (lrow >> 1)) >= 4, hi1 = (lpos ^ (4 + (lrow >> 1))) >= 4;
  const uint32_t voff0t = hi0 ? 0x80000000u : voff0, voff1t = hi1 ? 0x80000000u : voff1;
  const uint32_t avoff0t = hi0 ? 0x80000000u : avoff0, avoff1t = hi1 ? 0x80000000u : avoff1;
  auto dma = [&](uint16_t* sa, uint16_t* sw, int k0) {
    const bool half = k0 + kBK > kspan;  // uniform
    const uint32_t v0 = half ? voff0t : voff0, v1 = half ? voff1t : voff1;
    const uint32_t a0 = half ? avoff0t : avoff0, a1 = half ? avoff1t : avoff1;
    // A's step offset (uniform): columns kbeg + k0 of a row, or block (kbeg + k0) / 64
    const int a_soff = akb ? (int)(((kbeg + k0) / kBK) * a_kb_rows * (kBK * 2)) : (kbeg + k0) * 2;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int blk = wave * A_INS + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, WK_LDS(sa + blk * 512), 16, ((blk & 1) ? a1 : a0) + blk * ablk_bytes,
                                               a_soff, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < W_INS; ++i) {
      const int blk = wave * W_INS + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, WK_LDS(sw + blk * 512), 16,
                                               ((blk & 1) ? v1 : v0) + blk * blk_bytes, (kbeg + k0) * 2, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int l16 = lane & 15, lg = lane >> 4;
  // W_tile x A_tile^T: the transposed tile, so a lane holds 4 consecutive output columns
  auto compute = [&](const uint16_t* a, const uint16_t* w) {
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int ch = ks * 4 + lg;
      u32x4 wf[NB], af[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) wf[i] = *reinterpret_cast<const u32x4*>(w + swz(wn * WTN + i * 16 + l16, ch));
#pragma unroll
      for (int j = 0; j < MB; ++j) af[j] = *reinterpret_cast<const u32x4*>(a + swz(wm * WTM + j * 16 + l16, ch));
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma16x16x32(wf[i], af[j], acc[i][j]);
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  };
  // columns kbeg .. kbeg + klen of K (all of them by default); the resources
  // still span whole rows.  A last half step (K % 64 == 32) is zero-padded.
  const int KT = (kspan + kBK - 1) / kBK;
  dma(sA0, sW0, 0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  lds_barrier();
  if constexpr (SPREAD) {
    constexpr int INS = A_INS + W_INS, MPER = NB * MB / INS;
    static_assert(MPER * INS <= NB * MB, "at least one MFMA per DMA instruction");
    auto stage = [&](const uint16_t* a, const uint16_t* w, uint16_t* na, uint16_t* nw, int nk0) {
      u32x4 wf[NB], af[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i) wf[i] = *reinterpret_cast<const u32x4*>(w + swz(wn * WTN + i * 16 + l16, lg));
#pragma unroll
      for (int j = 0; j < MB; ++j) af[j] = *reinterpret_cast<const u32x4*>(a + swz(wm * WTM + j * 16 + l16, lg));
      dma(na, nw, nk0);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma16x16x32(wf[i], af[j], acc[i][j]);
      __builtin_amdgcn_sched_group_barrier(0x100, NB + MB, 0);  // the fragment reads first
      interleave_mfma_vmem<INS, MPER>();
      __builtin_amdgcn_sched_group_barrier(0x008, NB * MB - MPER * INS, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) wf[i] = *reinterpret_cast<const u32x4*>(w + swz(wn * WTN + i * 16 + l16, 4 + lg));
#pragma unroll
      for (int j = 0; j < MB; ++j) af[j] = *reinterpret_cast<const u32x4*>(a + swz(wm * WTM + j * 16 + l16, 4 + lg));
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = mfma16x16x32(wf[i], af[j], acc[i][j]);
    };
    for (int kt = 0; kt < KT; kt += 2) {
      stage(sA0, sW0, sA1, sW1, (kt + 1) * kBK);
      __builtin_amdgcn_s_waitcnt(0x0070);
      lds_barrier();
      stage(sA1, sW1, sA0, sW0, (kt + 2) * kBK);
      __builtin_amdgcn_s_waitcnt(0x0070);
      lds_barrier();
    }
    return;
  }
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + 1 < KT) dma(sA1, sW1, (kt + 1) * kBK);
    compute(sA0, sW0);
    __builtin_amdgcn_s_waitcnt(0x0070);
    lds_barrier();
    if (kt + 1 < KT) {
      if (kt + 2 < KT) dma(sA0, sW0, (kt + 2) * kBK);
      compute(sA1, sW1);
      __builtin_amdgcn_s_waitcnt(0x0070);
      lds_barrier();
    }
  }
}

template <int BM, int BN, int WGM, int WGN, bool SPREAD>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_dma_kernel(LinearKArgs p) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0;
  int n0;
  tile_origin(p.tiles_m, p.tiles_n, BM, BN, m0, n0);
  const int64_t M = p.M;
  const int N = p.N;
  f32x4 acc[NB][MB];
  dma_mainloop<BM, BN, WGM, WGN, SPREAD, true>(p.a, p.w, M, N, p.K, m0, n0, sA0, sW0, sA1, sW1, acc, 0, -1,
                                               p.a_kb_rows);
  const uint16_t* bias = p.bias;
  const uint16_t* res = p.res;
  // The residual (or mask) values are all requested before the first store:
  // as far as the compiler knows a store to C may alias them, so a load
  // placed after a store would wait out its whole latency on its own.
  u32x2 rv[NB][MB];
  if (res != nullptr) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int n = n0 + wn * WTN + i * 16 + lg * 4;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int64_t m = m0 + wm * WTM + j * 16 + l16;
        rv[i][j] = (m < M && n < N) ? *reinterpret_cast<const u32x2*>(res + m * N + n) : u32x2{0u, 0u};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + wn * WTN + i * 16 + lg * 4;
    float bb[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias != nullptr && n < N) {
      const u32x2 b2 = *reinterpret_cast<const u32x2*>(bias + n);
      bb[0] = bf16lo(b2[0]); bb[1] = bf16hi(b2[0]); bb[2] = bf16lo(b2[1]); bb[3] = bf16hi(b2[1]);
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int64_t m = m0 + wm * WTM + j * 16 + l16;
      if (m < M && n < N) {
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = apply_act(acc[i][j][t] + bb[t], p.act);
        if (res != nullptr) {
          const u32x2 r2 = rv[i][j];
          v[0] = apply_res(v[0], bf16lo(r2[0]), p.act);
          v[1] = apply_res(v[1], bf16hi(r2[0]), p.act);
          v[2] = apply_res(v[2], bf16lo(r2[1]), p.act);
          v[3] = apply_res(v[3], bf16hi(r2[1]), p.act);
        }
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(p.c + m * N + n) = o;
      }
    }
  }
}

// The FMB MLP's last Linear with the layer's output stage fused into its
// epilogue (Wukong paper, section 2.2: the FMB output reshaped to n_F x d,
// concatenated with the LCB output, residual added, LayerNorm per embedding).
// GEMM column c of example m is embedding row c / D, element c % D, which sits
// at y + m ld + c because the FMB rows come first in the layer output.  A wave
// covers WTN = 160 columns, a whole number of embedding rows, and a lane holds
// 4 consecutive columns of one row for each 16-column block, so one embedding
// row is D/16 blocks x 4 columns x the 4 lanes l16 + 16 lg: its LayerNorm
// statistics are a sum over registers and two xor-shuffles.  M is rounded to
// bf16 before the residual is added, as the unfused path stores it.
// Split-K: a grid of tiles x splits; split s accumulates columns
// [s K/splits, (s + 1) K/splits) of K and writes its fp32 partial sums to
// part[s][m][n] (no bias, no activation).  splitk_reduce_kernel then adds the
// partials in the fixed order s = 0, 1, .. (the result does not depend on
// timing), the bias and the ReLU, and rounds to bf16.  For Linears whose tiles
// alone leave CUs idle (few rows, long K: the prediction head's first Linear).
template <int BM, int BN, int WGM, int WGN, bool SPREAD>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_splitk_kernel(LinearKArgs p, float* part, int splits) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int l16 = lane & 15, lg = lane >> 4;
  const int ntiles = p.tiles_m * p.tiles_n;
  const int split = (int)blockIdx.x / ntiles, tile = (int)blockIdx.x - split * ntiles;
  int64_t m0;
  int n0;
  tile_origin_at(tile, ntiles, p.tiles_m, p.tiles_n, BM, BN, m0, n0);
  const int64_t M = p.M;
  const int N = p.N;
  const int klen = p.K / splits;
  f32x4 acc[NB][MB];
  dma_mainloop<BM, BN, WGM, WGN, SPREAD>(p.a, p.w, M, N, p.K, m0, n0, sA0, sW0, sA1, sW1, acc, split * klen, klen);
  float* ps = part + (int64_t)split * M * N;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + wn * WTN + i * 16 + lg * 4;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int64_t m = m0 + wm * WTM + j * 16 + l16;
      if (m < M && n < N) *reinterpret_cast<f32x4*>(ps + m * N + n) = acc[i][j];
    }
  }
}

// dX[b][m][e] = bf16(dXa[b][m][e] + C[m][b D + e]) with C = A W^T (M rows, N = B D
// columns, batch-major): a product whose columns are (example, embedding) pairs,
// added to an fp32 tensor of the example-major layout and stored in bf16.  The
// wide-layer backward forms dX this way, without writing C.  A lane's 4
// consecutive columns lie in one example (D % 4 == 0).
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_dx_kernel(LinearKArgs p, const float* dxa, uint16_t* dx,
                                                                 int D) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0;
  int n0;
  tile_origin(p.tiles_m, p.tiles_n, BM, BN, m0, n0);
  const int64_t M = p.M;
  const int N = p.N;
  f32x4 acc[NB][MB];
  dma_mainloop<BM, BN, WGM, WGN, false>(p.a, p.w, M, N, p.K, m0, n0, sA0, sW0, sA1, sW1, acc);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + wn * WTN + i * 16 + lg * 4;
    const int b = n / D, e = n - b * D;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int64_t m = m0 + wm * WTM + j * 16 + l16;
      if (m < M && n < N) {
        const int64_t o = ((int64_t)b * M + m) * D + e;
        const f32x4 a = *reinterpret_cast<const f32x4*>(dxa + o);
        const f32x4 v = acc[i][j];
        *reinterpret_cast<u32x2*>(dx + o) =
            u32x2{pack_bf16x2(v[0] + a[0], v[1] + a[1]), pack_bf16x2(v[2] + a[2], v[3] + a[3])};
      }
    }
  }
}

// C = bf16(act(sum_s part[s] + bias) + res), 8 consecutive columns per thread (N % 8 == 0).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits, int64_t M, int N,
                                                            const uint16_t* bias, int act, const uint16_t* res,
                                                            uint16_t* c) {
  const int64_t total = M * N / 8;
  const int64_t plane = M * N;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q * 8;
    const int n = (int)(e % N);
    f32x4 lo = *reinterpret_cast<const f32x4*>(part + e);
    f32x4 hi = *reinterpret_cast<const f32x4*>(part + e + 4);
    for (int sp = 1; sp < splits; ++sp) {
      lo += *reinterpret_cast<const f32x4*>(part + sp * plane + e);
      hi += *reinterpret_cast<const f32x4*>(part + sp * plane + e + 4);
    }
    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (bias != nullptr) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(bias + n);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[2 * t] += bf16lo(b[t]);
        v[2 * t + 1] += bf16hi(b[t]);
      }
    }
    u32x4 rr = u32x4{0u, 0u, 0u, 0u};
    if (res != nullptr) rr = *reinterpret_cast<const u32x4*>(res + e);
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = apply_act(v[2 * t], act), x1 = apply_act(v[2 * t + 1], act);
      if (res != nullptr) {
        x0 = apply_res(x0, bf16lo(rr[t]), act);
        x1 = apply_res(x1, bf16hi(rr[t]), act);
      }
      o[t] = pack_bf16x2(x0, x1);
    }
    *reinterpret_cast<u32x4*>(c + e) = o;
  }
}

// MOUT: the epilogue also stores M = bf16(A W^T + bias) (the training forward
// keeps it for the backward): block j's values go out right after block j's
// wait, so every later wait counts those NB stores as well.
// One 256 x 320 tile (workgroup bid of nblk working on p) of the fused last Linear.
template <int BM, int BN, int WGM, int WGN, int D, bool MOUT>
__device__ __forceinline__ void linear_ln_tile(const LinearLnKArgs& p, int bid, int nblk) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int GI = D / 16;    // 16-column blocks per embedding row
  constexpr int NG = WTN / D;   // embedding rows per wave and example
  constexpr int NW = WGM * WGN;
  constexpr int RES = 16 * WTN;        // u16 of one wave's 16-row residual block
  constexpr int RES_INS = RES * 2 / 1024;  // 1 KB DMA instructions per block
  static_assert(D % 16 == 0 && WTN % D == 0, "a wave must cover whole embedding rows");
  static_assert(RES_INS * 1024 == RES * 2 && NW * RES <= BN * kBK, "residual blocks fit a W stage");
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  __shared__ __align__(16) uint16_t Es[BN + 2 * D];  // bias of the tile's columns, then gamma, beta
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0;
  int n0;
  tile_origin_at(bid, nblk, p.tiles_m, p.tiles_n, BM, BN, m0, n0);
  const int64_t M = p.M;
  const int N = p.N;
  // epilogue constants staged before the main loop (whose first wait covers these loads), so the
  // epilogue issues no global loads besides its residual DMA
  for (int i = threadIdx.x; i < BN + 2 * D; i += NW * 64) {
    uint16_t v;
    if (i < BN) v = (p.bias && n0 + i < N) ? p.bias[n0 + i] : (uint16_t)0;
    else if (i < BN + D) v = p.gamma ? p.gamma[i - BN] : (uint16_t)0x3f80u;
    else v = p.beta ? p.beta[i - BN - D] : (uint16_t)0;
    Es[i] = v;
  }
  f32x4 acc[NB][MB];
  dma_mainloop<BM, BN, WGM, WGN>(p.a, p.w, M, N, p.K, m0, n0, sA0, sW0, sA1, sW1, acc);

  // Residual rows: each wave DMAs its own 16-row x WTN-column blocks (block j: tile rows
  // wm WTM + 16 j ..) into a private slice of the now idle W stages, two blocks ahead, so
  // the loads overlap the LayerNorms.  Rows past M read as zero and their stores are
  // dropped (buffer resources end at row M).
  const int rows = (int)min<int64_t>(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.x + m0 * p.ld), (short)0, (int)(rows * p.ld * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ry =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.y + m0 * p.ld), (short)0, (int)(rows * p.ld * 2), 0x00020000);
  const int cw = n0 + wn * WTN;  // first column of this wave
  uint16_t* const slot[2] = {sW0 + wave * RES, sW1 + wave * RES};
  auto dma_res = [&](int j, uint16_t* dst) {
#pragma unroll
    for (int q = 0; q < RES_INS; ++q) {
      const int u = q * 64 + lane;  // 16-byte unit of the block
      const int r = u / (WTN / 8), ch = u - r * (WTN / 8);
      const uint32_t vo = (uint32_t)(((int64_t)(wm * WTM + j * 16 + r) * p.ld + cw + ch * 8) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, WK_LDS(dst + q * 512), 16, vo, 0, 0, 0);
    }
  };
  if (cw < N) {  // wave-uniform
    dma_res(0, slot[0]);
    if (MB > 1) dma_res(1, slot[1]);
  }
  // M = bf16(acc + bias), in place
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const u32x2 b2 = *reinterpret_cast<const u32x2*>(Es + wn * WTN + i * 16 + lg * 4);
    const float bb[4] = {bf16lo(b2[0]), bf16hi(b2[0]), bf16lo(b2[1]), bf16hi(b2[1])};
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const uint32_t h0 = pack_bf16x2(acc[i][j][0] + bb[0], acc[i][j][1] + bb[1]);
      const uint32_t h1 = pack_bf16x2(acc[i][j][2] + bb[2], acc[i][j][3] + bb[3]);
      acc[i][j] = f32x4{bf16lo(h0), bf16hi(h0), bf16lo(h1), bf16hi(h1)};
    }
  }
  if (cw >= N) return;  // wave-uniform: this wave's columns are all past N
  const float inv_d = 1.0f / static_cast<float>(D);
  constexpr int ST = NG * GI;         // Y stores per row block
  constexpr int SM = MOUT ? NB : 0;   // M stores per row block
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(MOUT ? p.m_out + m0 * N : p.y), (short)0, MOUT ? (int)(rows * (int64_t)N * 2) : 0, 0x00020000);
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    // block j must have landed; younger: block j+1's DMA (if issued before it) and the
    // stores of block j-1 and block j+1's DMA (issued after)
    if (j == 0) {
      if (MB > 1) __builtin_amdgcn_s_waitcnt(vm_wait(RES_INS)); else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    } else if (j + 1 < MB) {
      __builtin_amdgcn_s_waitcnt(vm_wait(SM + ST + RES_INS));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait(SM + ST));
    }
    if (MOUT) {  // M of this row block, before the residual is added in place
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int n = cw + i * 16 + lg * 4;
        const f32x4 r = acc[i][j];
        const u32x2 o{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        const uint32_t off = n < N ? (uint32_t)(((int64_t)(wm * WTM + j * 16 + l16) * N + n) * 2) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b64(o, rm, off, 0, 0);
      }
    }
    const uint16_t* res = slot[j & 1] + l16 * WTN + lg * 4;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float sm = 0.f;
#pragma unroll
      for (int ii = 0; ii < GI; ++ii) {
        const u32x2 xv = *reinterpret_cast<const u32x2*>(res + g * D + ii * 16);
        f32x4& r = acc[g * GI + ii][j];
        r[0] += bf16lo(xv[0]);
        r[1] += bf16hi(xv[0]);
        r[2] += bf16lo(xv[1]);
        r[3] += bf16hi(xv[1]);
        sm += (r[0] + r[1]) + (r[2] + r[3]);
      }
      sm += __shfl_xor(sm, 16, kWave);
      sm += __shfl_xor(sm, 32, kWave);
      const float mean = sm * inv_d;
      float q = 0.f;
#pragma unroll
      for (int ii = 0; ii < GI; ++ii)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float dv = acc[g * GI + ii][j][t] - mean;
          q += dv * dv;
        }
      q += __shfl_xor(q, 16, kWave);
      q += __shfl_xor(q, 32, kWave);
      const float rstd = rsqrtf(q * inv_d + p.eps);
      const int c0 = cw + g * D;
      // columns past N belong to no embedding row of this layer: offset past the resource
      const uint32_t yoff = c0 < N ? (uint32_t)(((int64_t)(wm * WTM + j * 16 + l16) * p.ld + c0) * 2) : 0x80000000u;
#pragma unroll
      for (int ii = 0; ii < GI; ++ii) {
        const int e = ii * 16 + lg * 4;
        const u32x2 g2 = *reinterpret_cast<const u32x2*>(Es + BN + e);
        const u32x2 e2 = *reinterpret_cast<const u32x2*>(Es + BN + D + e);
        const f32x4 r = acc[g * GI + ii][j];
        u32x2 o;
        o[0] = pack_bf16x2((r[0] - mean) * rstd * bf16lo(g2[0]) + bf16lo(e2[0]),
                           (r[1] - mean) * rstd * bf16hi(g2[0]) + bf16hi(e2[0]));
        o[1] = pack_bf16x2((r[2] - mean) * rstd * bf16lo(g2[1]) + bf16lo(e2[1]),
                           (r[3] - mean) * rstd * bf16hi(g2[1]) + bf16hi(e2[1]));
        __builtin_amdgcn_raw_buffer_store_b64(o, ry, yoff + e * 2, 0, 0);
      }
    }
    if (j + 2 < MB) {
      // this wave's reads of the slot are done before the DMA reuses it
      __builtin_amdgcn_s_waitcnt(lgkm_wait0());
      dma_res(j + 2, slot[j & 1]);
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int D, bool MOUT>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_ln_kernel(LinearLnKArgs p) {
  linear_ln_tile<BM, BN, WGM, WGN, D, MOUT>(p, blockIdx.x, gridDim.x);
}

// Several fused last Linears of the same D in one launch (the experts of a
// mixture): group i takes workgroups first[i] .. first[i + 1] - 1.
struct LinearLnGroupKArgs {
  LinearLnKArgs a[kMaxLnGroup];
  int first[kMaxLnGroup + 1];
  int n;
};
template <int BM, int BN, int WGM, int WGN, int D>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_ln_group_kernel(LinearLnGroupKArgs g) {
  int i = 0;
  while (i + 1 < g.n && (int)blockIdx.x >= g.first[i + 1]) ++i;  // uniform
  linear_ln_tile<BM, BN, WGM, WGN, D, false>(g.a[i], (int)blockIdx.x - g.first[i], g.first[i + 1] - g.first[i]);
}

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_bf16_kernel(LinearKArgs p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MBK = WTM / 32, NBK = WTN / 32;
  constexpr int A_PER = BM * 8 / NT, W_PER = BN * 8 / NT;
  static_assert(A_PER * NT == BM * 8 && W_PER * NT == BN * 8, "tile / thread mismatch");

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sA = smem;                 // [2][BM * 64]
  uint16_t* sW = smem + 2 * BM * kBK;  // [2][BN * 64]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;

  // ---- tile index: XCD-contiguous, grouped along M
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int full = nblk & ~7;
  int logical = bid;
  if (bid < full) logical = (bid & 7) * (full >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GM;
  const int gsz = min(p.tiles_m - first_m, GM);
  const int in_g = logical - group * per_group;
  const int tm = first_m + in_g % gsz;
  const int tn = in_g / gsz;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const int64_t M = p.M;
  const int N = p.N, K = p.K;
  const uint16_t* __restrict__ A = p.a;
  const uint16_t* __restrict__ W = p.w;

  u32x4 ra[A_PER], rw[W_PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int id = tid + i * NT;
      const int row = id >> 3, ch = id & 7;
      const int64_t gm = m0 + row;
      const int gk = k0 + ch * 8;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4*>(A + gm * K + gk) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
      const int id = tid + i * NT;
      const int row = id >> 3, ch = id & 7;
      const int gn = n0 + row;
      const int gk = k0 + ch * 8;
      rw[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4*>(W + (int64_t)gn * K + gk) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
    uint16_t* a = sA + buf * BM * kBK;
    uint16_t* w = sW + buf * BN * kBK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int id = tid + i * NT;
      *reinterpret_cast<u32x4*>(a + swz(id >> 3, id & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
      const int id = tid + i * NT;
      *reinterpret_cast<u32x4*>(w + swz(id >> 3, id & 7)) = rw[i];
    }
  };

  f32x16 acc[NBK][MBK];
#pragma unroll
  for (int i = 0; i < NBK; ++i)
#pragma unroll
    for (int j = 0; j < MBK; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  const int lr = lane & 31, lh = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load((kt + 1) * kBK);
    const uint16_t* a = sA + buf * BM * kBK;
    const uint16_t* w = sW + buf * BN * kBK;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = ks * 2 + lh;
      u32x4 wf[NBK], af[MBK];
#pragma unroll
      for (int i = 0; i < NBK; ++i) wf[i] = *reinterpret_cast<const u32x4*>(w + swz(wn * WTN + i * 32 + lr, ch));
#pragma unroll
      for (int j = 0; j < MBK; ++j) af[j] = *reinterpret_cast<const u32x4*>(a + swz(wm * WTM + j * 32 + lr, ch));
#pragma unroll
      for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < MBK; ++j) acc[i][j] = mfma32x32x16(wf[i], af[j], acc[i][j]);
    }
    if (kt + 1 < KT) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m][n..n+3] for each (i, j, q)
  const uint16_t* bias = p.bias;
#pragma unroll
  for (int i = 0; i < NBK; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * WTN + i * 32 + q * 8 + lh * 4;
      float bb[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias != nullptr && n < N) {
        const u32x2 b2 = *reinterpret_cast<const u32x2*>(bias + n);
        bb[0] = bf16lo(b2[0]); bb[1] = bf16hi(b2[0]); bb[2] = bf16lo(b2[1]); bb[3] = bf16hi(b2[1]);
      }
#pragma unroll
      for (int j = 0; j < MBK; ++j) {
        const int64_t m = m0 + wm * WTM + j * 32 + lr;
        if (m < M && n < N) {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = apply_act(acc[i][j][q * 4 + t] + bb[t], p.act);
          if (p.res != nullptr) {
            const u32x2 r2 = *reinterpret_cast<const u32x2*>(p.res + m * N + n);
            v[0] = apply_res(v[0], bf16lo(r2[0]), p.act);
            v[1] = apply_res(v[1], bf16hi(r2[0]), p.act);
            v[2] = apply_res(v[2], bf16lo(r2[1]), p.act);
            v[3] = apply_res(v[3], bf16hi(r2[1]), p.act);
          }
          u32x2 o;
          o[0] = pack_bf16x2(v[0], v[1]);
          o[1] = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(p.c + m * N + n) = o;
        }
      }
    }
  }
}

struct LinearVariant {
  int bm, bn, occupancy;
  float eff;  // relative per-FLOP speed measured on the MLP shapes, used only to rank variants
  void (*kernel)(LinearKArgs);
  size_t dyn_lds;  // dynamic LDS bytes (the DMA kernels use static LDS)
  int threads;
  int kmod;        // K must be a multiple of this (32 or 128: DMA kernels; 8: register-staged)
};

#define WK_DMA_VARIANT(BM, BN, WGM, WGN, OCC, EFF, SPREAD)                                              \
  LinearVariant {                                                                                     \
    BM, BN, OCC, EFF, linear_dma_kernel<BM, BN, WGM, WGN, SPREAD>, 0, WGM * WGN * 64, SPREAD ? 128 : 32 \
  }
#define WK_LIN_VARIANT(BM, BN, WGM, WGN, OCC, EFF)                                                   \
  LinearVariant {                                                                                    \
    BM, BN, OCC, EFF, linear_bf16_kernel<BM, BN, WGM, WGN>, (size_t)2 * (BM + BN) * kBK * 2, WGM * WGN * 64, \
        8                                                                                            \
  }

const LinearVariant kLinVariants[] = {
    WK_DMA_VARIANT(256, 256, 2, 4, 1, 1.00f, false),
    WK_DMA_VARIANT(256, 128, 2, 4, 1, 0.78f, false),
    WK_DMA_VARIANT(128, 128, 2, 2, 2, 0.84f, true),   // DMA spread over the MFMAs: ~5 % over the burst form
    WK_DMA_VARIANT(128, 128, 2, 2, 2, 0.80f, false),
    WK_LIN_VARIANT(256, 256, 2, 2, 1, 0.55f),
    WK_LIN_VARIANT(256, 128, 2, 2, 1, 0.50f),
    WK_LIN_VARIANT(128, 128, 2, 2, 2, 0.45f),
};
constexpr int kNumLinVariants = sizeof(kLinVariants) / sizeof(kLinVariants[0]);

constexpr int kNumCU = 256;

const LinearVariant* pick_linear(int64_t M, int N, int K) {
  const bool k32 = (K % 32) == 0;
  const LinearVariant* best = nullptr;
  double best_cost = 0;
  for (const auto& v : kLinVariants) {
    // the DMA family when K % 32 == 0 (the spread form needs K % 128 == 0), else the fallbacks
    if ((v.kmod >= 32) != k32 || K % v.kmod != 0) continue;
    const double tiles = (double)((M + v.bm - 1) / v.bm) * (double)((N + v.bn - 1) / v.bn);
    const double slots = (double)kNumCU * v.occupancy;
    const double rounds = (tiles + slots - 1) / slots;
    const double cost = (double)(int64_t)rounds * v.occupancy * (double)v.bm * v.bn / v.eff;
    if (!best || cost < best_cost) {
      best = &v;
      best_cost = cost;
    }
  }
  return best;
}

// Fused Linear + output LayerNorm: 256 x 320 tiles, 8 waves of 64 rows x 160
// columns; 160 must be a whole number of embedding rows.
struct LinearLnVariant {
  int d;
  void (*kernel)(LinearLnKArgs);
  void (*kernel_m)(LinearLnKArgs);  // also stores M
  void (*group)(LinearLnGroupKArgs);
};
#define WK_LN_VARIANT(D)                                                                                       \
  LinearLnVariant {                                                                                            \
    D, linear_ln_kernel<256, 320, 4, 2, D, false>, linear_ln_kernel<256, 320, 4, 2, D, true>,                  \
        linear_ln_group_kernel<256, 320, 4, 2, D>                                                              \
  }
const LinearLnVariant kLnVariants[] = {WK_LN_VARIANT(16), WK_LN_VARIANT(32), WK_LN_VARIANT(80),
                                       WK_LN_VARIANT(160)};
constexpr int kLnBM = 256, kLnBN = 320, kLnThreads = 512;

const LinearLnVariant* pick_linear_ln(int d) {
  for (const auto& v : kLnVariants)
    if (v.d == d) return &v;
  return nullptr;
}

// Embedding units of width 8 (Wukong paper, section 2.1: each 8-wide unit
// takes part in the interaction as a feature of its own), the left multiply of
// the layer (section 2.2) over the whole batch: C'[r][(b, e)] =
// sum_j [Phi; W_L][r][j] X_b[j][e], rows r of [Phi; W_L] against the columns
// (example, element) of the transposed X.  A lane holds 4 consecutive
// elements e0 .. e0 + 3 (e0 = 0 or 4) of one example and row, and lane ^ 16
// the other 4, so the epilogue finishes everything that needs only this
// product: Z_b rows (r < k) go out in fp32, [b][r][e], for the interaction;
// the LCB rows (r = k + i) get the residual X_b[n_F + i], the LayerNorm over
// their 8 values (one xor-shuffle per statistic) and go out as Y_b[n_F + i].
struct UnitsGemmKArgs {
  const uint16_t* wcat;      // [k + n_l][n] (the A operand)
  const uint16_t* xt;        // [B 8][n]: xt[(b, e)][j] = X[b][j][e] (the W operand)
  const uint16_t* x;         // [B][n][8]
  const uint16_t* out_gamma; // [8] or null
  const uint16_t* out_beta;
  float* z;                  // [B][k][8]
  uint16_t* y;               // [B][n][8]: rows n_f .. n - 1 written
  int64_t M;                 // k + n_l
  int N, K;                  // B 8, n
  int k, n_f, n_l;
  float eps;
  int tiles_m, tiles_n;
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void units_gemm_kernel(UnitsGemmKArgs p) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int UD = 8;
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0;
  int n0;
  tile_origin(p.tiles_m, p.tiles_n, BM, BN, m0, n0);
  f32x4 acc[NB][MB];
  dma_mainloop<BM, BN, WGM, WGN, false>(p.wcat, p.xt, p.M, p.N, p.K, m0, n0, sA0, sW0, sA1, sW1, acc);
  const int k = p.k, n = p.K, n_f = p.n_f, n_l = p.n_l;
  const int e0 = (4 * lg) & (UD - 1);  // every column block starts at a multiple of 16
  float og[4], ob[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    og[t] = p.out_gamma ? bf16_to_f32(p.out_gamma[e0 + t]) : 1.f;
    ob[t] = p.out_beta ? bf16_to_f32(p.out_beta[e0 + t]) : 0.f;
  }
  // the residual elements of the LCB rows, all requested before the first store
  u32x2 rv[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = n0 + wn * WTN + i * 16 + lg * 4;
    const int64_t b = q >> 3;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int r = (int)(m0 + wm * WTM + j * 16 + l16);
      const bool lcb = r >= k && r < k + n_l && q < p.N;
      rv[i][j] = lcb ? *reinterpret_cast<const u32x2*>(p.x + ((b * n + n_f + r - k) * UD + e0)) : u32x2{0u, 0u};
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = n0 + wn * WTN + i * 16 + lg * 4;
    const int64_t b = q >> 3;
    const bool qv = q < p.N;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int r = (int)(m0 + wm * WTM + j * 16 + l16);
      const f32x4 a = acc[i][j];
      if (r < k && qv) *reinterpret_cast<f32x4*>(p.z + (b * k + r) * UD + e0) = a;
      const u32x2 x2 = rv[i][j];
      float v[4] = {a[0] + bf16lo(x2[0]), a[1] + bf16hi(x2[0]), a[2] + bf16lo(x2[1]), a[3] + bf16hi(x2[1])};
      // every lane takes part in the shuffles; only the LCB rows are stored
      float sm = (v[0] + v[1]) + (v[2] + v[3]);
      sm += __shfl_xor(sm, 16, kWave);
      const float mean = sm * (1.0f / UD);
      float sq = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) sq += (v[t] - mean) * (v[t] - mean);
      sq += __shfl_xor(sq, 16, kWave);
      const float rstd = rsqrtf(sq * (1.0f / UD) + p.eps);
      if (r >= k && r < k + n_l && qv) {
        u32x2 o;
        o[0] = pack_bf16x2((v[0] - mean) * rstd * og[0] + ob[0], (v[1] - mean) * rstd * og[1] + ob[1]);
        o[1] = pack_bf16x2((v[2] - mean) * rstd * og[2] + ob[2], (v[3] - mean) * rstd * og[3] + ob[3]);
        *reinterpret_cast<u32x2*>(p.y + (b * n + n_f + r - k) * UD + e0) = o;
      }
    }
  }
}

}  // namespace

bool units_gemm_supported(int64_t batch, int n, int k, int n_l) {
  return batch > 0 && batch * 8 <= 0x7fffffff && n > 0 && n % kBK == 0 && k > 0 && k % 4 == 0 && n_l > 0 &&
         n_l % 4 == 0 && n_l <= n;
}

hipError_t launch_units_gemm(const UnitsGemmArgs& a, hipStream_t stream, int64_t* workgroups) {
  if (!units_gemm_supported(a.batch, a.n, a.k, a.n_l) || !a.wcat || !a.xt || !a.x || !a.z || !a.y)
    return hipErrorInvalidValue;
  UnitsGemmKArgs k;
  k.wcat = static_cast<const uint16_t*>(a.wcat);
  k.xt = static_cast<const uint16_t*>(a.xt);
  k.x = static_cast<const uint16_t*>(a.x);
  k.out_gamma = static_cast<const uint16_t*>(a.out_gamma);
  k.out_beta = static_cast<const uint16_t*>(a.out_beta);
  k.z = a.z;
  k.y = static_cast<uint16_t*>(a.y);
  k.M = a.k + a.n_l;
  k.N = (int)(a.batch * 8);
  k.K = a.n;
  k.k = a.k;
  k.n_f = a.n - a.n_l;
  k.n_l = a.n_l;
  k.eps = a.eps;
  k.tiles_m = (int)((k.M + 255) / 256);
  k.tiles_n = (k.N + 255) / 256;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n;
  if (workgroups) *workgroups = blocks;
  hipLaunchKernelGGL((units_gemm_kernel<256, 256, 2, 4>), dim3((unsigned)blocks), dim3(512), 0, stream, k);
  return hipGetLastError();
}

bool linear_ln_bf16_supported(int64_t M, int N, int K, int d) {
  return M > 0 && K > 0 && K % kBK == 0 && d > 0 && N % d == 0 && N > 0 && pick_linear_ln(d) != nullptr;
}

namespace {
LinearLnKArgs ln_kargs(const LinearLnArgs& a) {
  LinearLnKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = static_cast<const uint16_t*>(a.bias);
  k.x = static_cast<const uint16_t*>(a.x);
  k.gamma = static_cast<const uint16_t*>(a.gamma);
  k.beta = static_cast<const uint16_t*>(a.beta);
  k.y = static_cast<uint16_t*>(a.y);
  k.m_out = static_cast<uint16_t*>(a.m_out);
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.ld = a.ld;
  k.eps = a.eps;
  k.tiles_m = (int)((a.M + kLnBM - 1) / kLnBM);
  k.tiles_n = (a.N + kLnBN - 1) / kLnBN;
  return k;
}
}  // namespace

hipError_t launch_linear_ln_bf16_group(const LinearLnArgs* a, int n, hipStream_t stream, int64_t* workgroups) {
  if (n < 1 || n > kMaxLnGroup) return hipErrorInvalidValue;
  const LinearLnVariant* v = pick_linear_ln(a[0].d);
  if (!v) return hipErrorInvalidValue;
  LinearLnGroupKArgs g;
  g.n = n;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (a[i].d != a[0].d || a[i].m_out != nullptr || !linear_ln_bf16_supported(a[i].M, a[i].N, a[i].K, a[i].d))
      return hipErrorInvalidValue;
    g.a[i] = ln_kargs(a[i]);
    g.first[i] = (int)blocks;
    blocks += (int64_t)g.a[i].tiles_m * g.a[i].tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  }
  g.first[n] = (int)blocks;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(v->group, dim3((unsigned)blocks), dim3(kLnThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_linear_ln_bf16(const LinearLnArgs& a, hipStream_t stream, int64_t* workgroups) {
  const LinearLnVariant* v = pick_linear_ln(a.d);
  if (!v || !linear_ln_bf16_supported(a.M, a.N, a.K, a.d)) return hipErrorInvalidValue;
  LinearLnKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = static_cast<const uint16_t*>(a.bias);
  k.x = static_cast<const uint16_t*>(a.x);
  k.gamma = static_cast<const uint16_t*>(a.gamma);
  k.beta = static_cast<const uint16_t*>(a.beta);
  k.y = static_cast<uint16_t*>(a.y);
  k.m_out = static_cast<uint16_t*>(a.m_out);
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.ld = a.ld;
  k.eps = a.eps;
  k.tiles_m = (int)((a.M + kLnBM - 1) / kLnBM);
  k.tiles_n = (a.N + kLnBN - 1) / kLnBN;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(a.m_out ? v->kernel_m : v->kernel, dim3((unsigned)blocks), dim3(kLnThreads), 0, stream, k);
  return hipGetLastError();
}

// Split-K on 128 x 128 tiles (two workgroups per CU) when the unsplit tiling
// leaves workgroup slots empty: splits double while the tiles do not fill
// every slot, the split length stays a multiple of 128 (the spread main loop)
// and at least 2048 long.  1 = no split.
constexpr int kSplitBM = 128, kSplitBN = 128, kSplitOcc = 2, kMaxSplits = 8;

int linear_bf16_splits(int64_t M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || N % 8 != 0) return 1;
  const LinearVariant* v = pick_linear(M, N, K);
  if (!v) return 1;
  const double tiles_v = (double)((M + v->bm - 1) / v->bm) * (double)((N + v->bn - 1) / v->bn);
  if (tiles_v >= (double)kNumCU * v->occupancy) return 1;
  const double tiles = (double)((M + kSplitBM - 1) / kSplitBM) * (double)((N + kSplitBN - 1) / kSplitBN);
  int sp = 1;
  while (sp < kMaxSplits && tiles * sp < (double)kNumCU * kSplitOcc && K % (2 * sp * 128) == 0 &&
         K / (2 * sp) >= 2048)
    sp *= 2;
  return sp;
}

size_t linear_bf16_split_bytes(int64_t M, int N, int K) {
  const int sp = linear_bf16_splits(M, N, K);
  return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_linear_bf16_splitk(const LinearArgs& a, float* partial, hipStream_t stream, int64_t* workgroups) {
  const int sp = linear_bf16_splits(a.M, a.N, a.K);
  if (sp <= 1 || partial == nullptr) return hipErrorInvalidValue;
  LinearKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = static_cast<const uint16_t*>(a.bias);
  k.c = static_cast<uint16_t*>(a.c);
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.act = a.act;
  k.res = static_cast<const uint16_t*>(a.res);
  k.tiles_m = (int)((a.M + kSplitBM - 1) / kSplitBM);
  k.tiles_n = (a.N + kSplitBN - 1) / kSplitBN;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n * sp;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (workgroups) *workgroups = blocks;
  hipLaunchKernelGGL((linear_splitk_kernel<kSplitBM, kSplitBN, 2, 2, true>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, k, partial, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t groups8 = a.M * a.N / 8;
  int64_t grid = (groups8 + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partial, sp, a.M, a.N,
                     static_cast<const uint16_t*>(a.bias), a.act, static_cast<const uint16_t*>(a.res),
                     static_cast<uint16_t*>(a.c));
  return hipGetLastError();
}

// C (fp32, row-major [M, N]) = A W^T on 256 x 256 tiles with no bias or
// activation: the split kernel with one split writes its sums straight to C.
bool linear_bf16_f32out_supported(int64_t M, int N, int K) {
  return M > 0 && N > 0 && K > 0 && K % kBK == 0 && N % 8 == 0;
}

hipError_t launch_linear_bf16_f32out(const LinearArgs& a, float* c, hipStream_t stream, int64_t* workgroups) {
  if (!linear_bf16_f32out_supported(a.M, a.N, a.K) || c == nullptr) return hipErrorInvalidValue;
  LinearKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = nullptr;
  k.c = nullptr;
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.act = kActNone;
  k.res = nullptr;
  k.tiles_m = (int)((a.M + 255) / 256);
  k.tiles_n = (a.N + 255) / 256;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (workgroups) *workgroups = blocks;
  hipLaunchKernelGGL((linear_splitk_kernel<256, 256, 2, 4, false>), dim3((unsigned)blocks), dim3(512), 0, stream, k, c,
                     1);
  return hipGetLastError();
}

bool linear_bf16_dx_supported(int64_t M, int N, int K, int D) {
  return M > 0 && N > 0 && K > 0 && K % kBK == 0 && D > 0 && D % 4 == 0 && N % D == 0;
}

hipError_t launch_linear_bf16_dx(const LinearArgs& a, const float* dxa, void* dx, int D, hipStream_t stream,
                                 int64_t* workgroups) {
  if (!linear_bf16_dx_supported(a.M, a.N, a.K, D) || dxa == nullptr || dx == nullptr) return hipErrorInvalidValue;
  LinearKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = nullptr;
  k.c = nullptr;
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.act = kActNone;
  k.res = nullptr;
  k.tiles_m = (int)((a.M + 255) / 256);
  k.tiles_n = (a.N + 255) / 256;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (workgroups) *workgroups = blocks;
  hipLaunchKernelGGL((linear_dx_kernel<256, 256, 2, 4>), dim3((unsigned)blocks), dim3(512), 0, stream, k, dxa,
                     static_cast<uint16_t*>(dx), D);
  return hipGetLastError();
}

// Split-K form of the fp32-output product for shapes whose 256 x 256 tiles
// leave CUs idle: splits double while tiles x splits < CUs, each split keeps
// a multiple of 64 of K and at least 1024 of it.
int linear_bf16_f32out_splits_max(int64_t M, int N, int K, int max_splits) {
  if (!linear_bf16_f32out_supported(M, N, K)) return 1;
  const double tiles = (double)((M + 255) / 256) * (double)((N + 255) / 256);
  int sp = 1;
  while (sp < max_splits && tiles * sp < (double)kNumCU && K % (2 * sp * kBK) == 0 && K / (2 * sp) >= 1024) sp *= 2;
  return sp;
}
int linear_bf16_f32out_splits(int64_t M, int N, int K) { return linear_bf16_f32out_splits_max(M, N, K, kMaxSplits); }

size_t linear_bf16_f32out_split_bytes_max(int64_t M, int N, int K, int max_splits) {
  const int sp = linear_bf16_f32out_splits_max(M, N, K, max_splits);
  return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * sizeof(float) : 0;
}
size_t linear_bf16_f32out_split_bytes(int64_t M, int N, int K) {
  return linear_bf16_f32out_split_bytes_max(M, N, K, kMaxSplits);
}

hipError_t launch_linear_bf16_f32out_split(const LinearArgs& a, float* c, float* partial, hipStream_t stream,
                                           int64_t* workgroups) {
  return launch_linear_bf16_f32out_split_max(a, c, partial, kMaxSplits, stream, workgroups);
}

hipError_t launch_linear_bf16_f32out_split_max(const LinearArgs& a, float* c, float* partial, int max_splits,
                                               hipStream_t stream, int64_t* workgroups) {
  const int sp = linear_bf16_f32out_splits_max(a.M, a.N, a.K, max_splits);
  if (sp <= 1) return launch_linear_bf16_f32out(a, c, stream, workgroups);
  if (c == nullptr || partial == nullptr) return hipErrorInvalidValue;
  LinearKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = nullptr;
  k.c = nullptr;
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.act = kActNone;
  k.res = nullptr;
  k.tiles_m = (int)((a.M + 255) / 256);
  k.tiles_n = (a.N + 255) / 256;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n * sp;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (workgroups) *workgroups = blocks;
  hipLaunchKernelGGL((linear_splitk_kernel<256, 256, 2, 4, false>), dim3((unsigned)blocks), dim3(512), 0, stream, k,
                     partial, sp);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_planes(partial, sp, a.M * (int64_t)a.N, c, stream);
}

bool linear_bf16_supported(int64_t M, int N, int K) {
  return M > 0 && N > 0 && K > 0 && (K % 8) == 0 && (N % 8) == 0;
}

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream, int64_t* workgroups) {
  const LinearVariant* v = pick_linear(a.M, a.N, a.K);
  if (a.a_kblock_rows > 0) {  // K-blocked A: the DMA kernels only, every row of every tile inside the array
    if (a.K % kBK != 0 || v->kmod < 32 || a.a_kblock_rows % 256 != 0 || a.a_kblock_rows < a.M ||
        a.a_kblock_rows * (int64_t)a.K * 2 >= ((int64_t)1 << 31))
      return hipErrorInvalidValue;
  }
  LinearKArgs k;
  k.a_kb_rows = a.a_kblock_rows;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = static_cast<const uint16_t*>(a.bias);
  k.c = static_cast<uint16_t*>(a.c);
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.act = a.act;
  k.res = static_cast<const uint16_t*>(a.res);
  k.tiles_m = (int)((a.M + v->bm - 1) / v->bm);
  k.tiles_n = (a.N + v->bn - 1) / v->bn;
  const int64_t blocks = (int64_t)k.tiles_m * k.tiles_n;
  if (workgroups) *workgroups = blocks;
  if (blocks == 0) return hipSuccess;
  static std::once_flag attr_once[kNumLinVariants];
  static hipError_t attr_err[kNumLinVariants];
  const size_t vi = (size_t)(v - kLinVariants);
  std::call_once(attr_once[vi], [&] {
    attr_err[vi] = v->dyn_lds == 0 ? hipSuccess
                                   : hipFuncSetAttribute(reinterpret_cast<const void*>(v->kernel),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)v->dyn_lds);
  });
  if (attr_err[vi] != hipSuccess) return attr_err[vi];
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)blocks), dim3(v->threads), v->dyn_lds, stream, k);
  return hipGetLastError();
}

}  // namespace wk
