// FMB-MLP Linear on bf16 MFMA: C[M, N] = act(A[M, K] W[N, K]^T + bias[N]).
//
// The FMB's MLP (Wukong paper, section 2.2; its depth and widths are the
// "MLP" scaling knob of section 2.3) is where nearly all of a Wukong layer's
// FLOPs go, so this is a plain dense contraction on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.  A is the activation (row-major, K contiguous) and
// W keeps torch.nn.Linear's [out, in] layout, so both operands are
// K-contiguous and land in LDS the same way.
//
// Tiling: a BM x BN output tile per workgroup of WGM x WGN waves, K in steps
// of 64.  Global -> registers -> LDS double buffer: the next K tile's loads
// are in flight while the current one feeds the MFMAs.  LDS rows are 128 B
// (64 bf16); the 16-byte chunk c of row r is stored at c ^ ((r >> 1) & 7),
// which keeps both the row-wise stores and the 32-row MFMA fragment reads
// free of bank conflicts.  Each wave computes W_tile x A_tile^T, i.e. the
// transposed tile, so a lane ends up holding 4 consecutive output columns of
// one row: the epilogue adds the bias, applies ReLU, rounds to bf16 and
// stores 8 bytes per lane.
//
// Tile order: the hardware deals workgroup i to XCD i % 8; the logical tile
// index is remapped so each XCD gets a contiguous run of tiles, walked in
// groups of 8 tile-rows so that neighbouring tiles share A and W panels in
// that XCD's L2.
//
// Two kernels share this structure:
//  * linear_dma_kernel (K % 64 == 0, the fast path): v_mfma_f32_16x16x32_bf16,
//    operands moved global -> LDS by buffer_load ... lds (no staging
//    registers), two static LDS stages so the next K tile streams in while the
//    current one is consumed.  Each workgroup's buffer resources start at its
//    tile's first row and end at the last valid row, so rows past M or N read
//    as zero.  Barriers are LDS-scoped (they do not wait for global loads).
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
  int relu;
  int tiles_m, tiles_n;
};

constexpr int kBK = 64;

__device__ __forceinline__ int swz(int row, int ch) { return row * kBK + ((ch ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ void tile_origin(const LinearKArgs& p, int BM, int BN, int64_t& m0, int& n0) {
  const int nblk = gridDim.x, bid = blockIdx.x, full = nblk & ~7;
  int logical = bid;
  if (bid < full) logical = (bid & 7) * (full >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GM;
  const int gsz = min(p.tiles_m - first_m, GM);
  const int in_g = logical - group * per_group;
  m0 = (int64_t)(first_m + in_g % gsz) * BM;
  n0 = (in_g / gsz) * BN;
}

#define WK_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void linear_dma_kernel(LinearKArgs p) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int A_INS = BM / 8 / NW, W_INS = BN / 8 / NW;  // 1 KB (8 rows) DMA instructions per wave
  static_assert(A_INS * NW * 8 == BM && W_INS * NW * 8 == BN, "tile / wave mismatch");
  __shared__ __align__(16) uint16_t sA0[BM * kBK], sW0[BN * kBK], sA1[BM * kBK], sW1[BN * kBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  int64_t m0;
  int n0;
  tile_origin(p, BM, BN, m0, n0);
  const int64_t M = p.M;
  const int N = p.N, K = p.K;
  const int rows_a = (int)min<int64_t>(BM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + m0 * K), (short)0, rows_a * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (int64_t)n0 * K), (short)0, rows_w * K * 2, 0x00020000);
  // A DMA instruction writes 64 lanes x 16 B = 8 LDS rows; lane -> row lane/8,
  // LDS chunk lane%8, which holds global chunk (lane%8) ^ swizzle(row).  The
  // swizzle of row 8b + r is (4(b & 1) + r/2) & 7: two lane offsets suffice.
  const int lrow = lane >> 3, lpos = lane & 7;
  const uint32_t voff0 = (uint32_t)(lrow * K + ((lpos ^ (lrow >> 1)) << 3)) * 2u;
  const uint32_t voff1 = (uint32_t)(lrow * K + ((lpos ^ (4 + (lrow >> 1))) << 3)) * 2u;
  const uint32_t blk_bytes = (uint32_t)(16 * K);
  auto dma = [&](uint16_t* sa, uint16_t* sw, int k0) {
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int blk = wave * A_INS + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, WK_LDS(sa + blk * 512), 16,
                                               ((blk & 1) ? voff1 : voff0) + blk * blk_bytes, k0 * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < W_INS; ++i) {
      const int blk = wave * W_INS + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, WK_LDS(sw + blk * 512), 16,
                                               ((blk & 1) ? voff1 : voff0) + blk * blk_bytes, k0 * 2, 0, 0);
    }
  };
  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int l16 = lane & 15, lg = lane >> 4;
  // W_tile x A_tile^T: lane (l16, lg) ends with C[m0 + .. + l16][n .. n + 3]
  auto compute = [&](const uint16_t* a, const uint16_t* w) {
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
  };
  const int KT = K / kBK;
  dma(sA0, sW0, 0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  lds_barrier();
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
  const uint16_t* bias = p.bias;
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
        for (int t = 0; t < 4; ++t) {
          v[t] = acc[i][j][t] + bb[t];
          if (p.relu) v[t] = fmaxf(v[t], 0.f);
        }
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(p.c + m * N + n) = o;
      }
    }
  }
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
          for (int t = 0; t < 4; ++t) {
            v[t] = acc[i][j][q * 4 + t] + bb[t];
            if (p.relu) v[t] = fmaxf(v[t], 0.f);
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
  bool needs_k64;
};

#define WK_DMA_VARIANT(BM, BN, WGM, WGN, OCC, EFF) \
  LinearVariant { BM, BN, OCC, EFF, linear_dma_kernel<BM, BN, WGM, WGN>, 0, WGM * WGN * 64, true }
#define WK_LIN_VARIANT(BM, BN, WGM, WGN, OCC, EFF)                                                   \
  LinearVariant {                                                                                    \
    BM, BN, OCC, EFF, linear_bf16_kernel<BM, BN, WGM, WGN>, (size_t)2 * (BM + BN) * kBK * 2, WGM * WGN * 64, \
        false                                                                                        \
  }

const LinearVariant kLinVariants[] = {
    WK_DMA_VARIANT(256, 256, 2, 4, 1, 1.00f),
    WK_DMA_VARIANT(256, 128, 2, 4, 1, 0.78f),
    WK_DMA_VARIANT(128, 128, 2, 2, 2, 0.80f),
    WK_LIN_VARIANT(256, 256, 2, 2, 1, 0.55f),
    WK_LIN_VARIANT(256, 128, 2, 2, 1, 0.50f),
    WK_LIN_VARIANT(128, 128, 2, 2, 2, 0.45f),
};
constexpr int kNumLinVariants = sizeof(kLinVariants) / sizeof(kLinVariants[0]);

constexpr int kNumCU = 256;

const LinearVariant* pick_linear(int64_t M, int N, int K) {
  const bool k64 = (K % kBK) == 0;
  const LinearVariant* best = nullptr;
  double best_cost = 0;
  for (const auto& v : kLinVariants) {
    if (v.needs_k64 != k64) continue;
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

}  // namespace

bool linear_bf16_supported(int64_t M, int N, int K) {
  return M > 0 && N > 0 && K > 0 && (K % 8) == 0 && (N % 8) == 0;
}

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream, int64_t* workgroups) {
  const LinearVariant* v = pick_linear(a.M, a.N, a.K);
  LinearKArgs k;
  k.a = static_cast<const uint16_t*>(a.a);
  k.w = static_cast<const uint16_t*>(a.w);
  k.bias = static_cast<const uint16_t*>(a.bias);
  k.c = static_cast<uint16_t*>(a.c);
  k.M = a.M;
  k.N = a.N;
  k.K = a.K;
  k.relu = a.relu;
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
