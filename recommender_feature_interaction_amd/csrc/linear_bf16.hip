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
  float eff;  // relative per-FLOP speed, used only to rank the variants
  void (*kernel)(LinearKArgs);
  size_t lds;
  int threads;
};

#define WK_LIN_VARIANT(BM, BN, WGM, WGN, OCC, EFF)                                       \
  LinearVariant {                                                                        \
    BM, BN, OCC, EFF, linear_bf16_kernel<BM, BN, WGM, WGN>, (size_t)2 * (BM + BN) * kBK * 2, \
        WGM * WGN * 64                                                                   \
  }

const LinearVariant kLinVariants[] = {
    WK_LIN_VARIANT(256, 256, 2, 2, 1, 1.00f),
    WK_LIN_VARIANT(256, 128, 2, 2, 1, 0.92f),
    WK_LIN_VARIANT(128, 128, 2, 2, 2, 0.80f),
};

constexpr int kNumCU = 256;

const LinearVariant* pick_linear(int64_t M, int N) {
  const LinearVariant* best = nullptr;
  double best_cost = 0;
  for (const auto& v : kLinVariants) {
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
  const LinearVariant* v = pick_linear(a.M, a.N);
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
  static std::once_flag attr_once[sizeof(kLinVariants) / sizeof(kLinVariants[0])];
  static hipError_t attr_err[sizeof(kLinVariants) / sizeof(kLinVariants[0])];
  const size_t vi = (size_t)(v - kLinVariants);
  std::call_once(attr_once[vi], [&] {
    attr_err[vi] = hipFuncSetAttribute(reinterpret_cast<const void*>(v->kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)v->lds);
  });
  if (attr_err[vi] != hipSuccess) return attr_err[vi];
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)blocks), dim3(v->threads), v->lds, stream, k);
  return hipGetLastError();
}

}  // namespace wk
