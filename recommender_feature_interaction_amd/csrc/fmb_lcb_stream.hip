// FMB + LCB, streamed through LDS (bf16, fp32 accumulation).
//
// Computes, per example b (Wukong paper, section 2.2: the FMB's compress and
// interact steps and the LCB, which share the left factor X_b):
//   [Z_b; Lc_b] = [Phi; W_L] X_b           Z_b is k x d, Lc_b is n_L x d
//   Y_b[n_F + i] = LN_d(Lc_b[i] + X_b[n_F + i])   the LCB rows of the output
//   F_b = X_b Z_b^T,  Fn_b = LN_{n k}(vec(F_b))   the FMB-MLP input
//
// Work split: a workgroup of 8 waves takes a group of E consecutive examples
// at a time (persistent grid).  Phase 1 is a GEMM over K = n in steps of 32
// rows: each step's [Phi; W_L] columns and X rows (for all E examples) are
// copied global -> LDS by buffer_load ... lds into a ring of S slots (3 or
// 4), S - 1 steps ahead, so the weights are read once per E examples and the
// HBM stream of X runs ahead of the MFMAs.  Phi occupies the first ceil(k/16)
// 16-row tiles and W_L the following ones (a tile never mixes the two, so a
// DMA instruction has one source; the padding rows read as zero).  The
// MFMA computes the transposed tile [Z; Lc]^T = X^T [Phi; W_L]^T: the X^T
// operand comes from the row-major X rows with ds_read_b64_tr_b16 (in each
// 16-lane group, lane i receives value i%4 of the 8-byte rows addressed by
// lanes 4k + i/4, so lanes pointing at X[m + s/4][e0 + 4(s%4)] hand lane i
// X[m + k][e0 + i]), and a lane ends up with 4 consecutive embedding
// elements of one output row, so the LCB LayerNorm is a register sum and two
// xor-shuffles.  Z goes to LDS as bf16 (the MFMA operand of phase 2).
//
// Phase 2, per example: F^T = Z X^T with the X rows read again from global
// memory (they were streamed moments before, so they come from L2 or the
// last-level cache), the n k statistics reduced across the waves in LDS, and
// Fn written with the FMB LayerNorm's gamma / beta.  The first S - 1 steps
// of the next group's DMA are issued before phase 2 starts.
#include "wk_device.h"
#include "wk_kernels.h"

namespace wk {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define WK_LDS_I16X4(p) ((__attribute__((address_space(3))) i16x4*)(p))
#define WK_LDSV(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ u32x4 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WK_LDS_I16X4(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WK_LDS_I16X4(p1));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

constexpr int KC = 32;                  // X rows (= [Phi; W_L] columns) per step
constexpr int NWAVE = 8;
constexpr int NTHREAD = NWAVE * 64;
constexpr uint32_t kOOB = 0x80000000u;  // a voffset past every record count: the lane reads zero

// s_waitcnt vmcnt(n) immediate (gfx9 encoding; expcnt and lgkmcnt not waited for), n <= 63
constexpr int vm_enc(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

struct StreamShape {
  int zt;    // 16-row tiles of [Phi; W_L]: kz + ceil(n_l / 16)
  int kz;    // tiles holding Phi: ceil(k / 16)
  int steps; // ceil(n / KC)
  int e;     // examples per group
};

// Row pitch (u16) of the Z rows kept in LDS for phase 2: D rounded up to 32,
// plus 8 (zero padding).
__host__ __device__ constexpr int zs_pitch(int d) { return (d + 31) / 32 * 32 + 8; }

// GUARD: a wave skips its weight tiles past the shape's ZT (operands read first, one test per
// tile); without it every wave computes all WZ * ZPW tiles, the ones past ZT reading zero tiles
// of the slot (needs ZTMAX >= WZ * ZPW), branch-free with each operand consumed as it is read.
template <int ET, int ZPW, int WZ, int WE, int EPW, int MPW, int KJ, int ZTMAX, int S, bool GUARD>
__global__ __launch_bounds__(NTHREAD, 2) void fmb_lcb_stream_kernel(FmbLcbArgs p, int64_t batch, StreamShape sh) {
  constexpr int D = 16 * ET;
  constexpr int E = WE * EPW;
  constexpr int ZP = zs_pitch(D);
  constexpr int DZ = (D + 31) / 32 * 32;
  constexpr int NKS = DZ / 32;                 // 32-wide K steps of phase 2
  constexpr bool GB_REG = MPW * KJ <= 12;      // FMB LayerNorm gamma / beta held in registers
  // DMA instructions per step: ZTP = ZTMAX 16-row weight tiles (tiles past the
  // shape's ZT read as zero) and X_INS for the X rows (1 KB each), dealt round
  // robin: waves below R issue INS_HI per step, the others INS_LO, so every
  // counter wait is a compile-time constant.
  constexpr int X_INS = E * D / 16;
  constexpr int ZTP = ZTMAX;  // >= the shape's ZT (host check); may exceed WZ * ZPW (padding tiles)
  constexpr int NINS = ZTP + X_INS;
  constexpr int INS_HI = (NINS + NWAVE - 1) / NWAVE, INS_LO = NINS / NWAVE, R = NINS % NWAVE;
  constexpr int SW = ZTP * 16 * KC;       // weight part of a ring slot (u16)
  constexpr int SX = E * KC * D;          // X part of a ring slot
  static_assert(WZ * WE == NWAVE, "8 waves");
  static_assert(S == 3 || S == 4, "ring of 3 or 4 slots");
  static_assert(GUARD || ZTMAX >= WZ * ZPW, "unguarded tiles must lie in the slot");
  static_assert(2 * ((ZTMAX + WE * EPW * ET + NWAVE - 1) / NWAVE) <= 63, "vmcnt range");
  // The ring slots are separate objects: the compiler then knows a DMA into
  // one slot does not alias reads of another and inserts no wait for it.
  __shared__ __align__(16) uint16_t w0[SW], w1[SW], w2[SW], w3[S > 3 ? SW : 8];
  __shared__ __align__(16) uint16_t x0[SX], x1[SX], x2[SX], x3[S > 3 ? SX : 8];
  uint16_t* const wslot[4] = {w0, w1, w2, w3};  // indexed only with compile-time slot numbers
  uint16_t* const xslot[4] = {x0, x1, x2, x3};
  __shared__ __align__(16) uint16_t Zs[E * KJ * 16 * ZP];
  __shared__ __align__(16) uint16_t Gs[2 * D];
  __shared__ float red[2 * NWAVE];

  const int n = p.n, k = p.k, n_l = p.n_l, n_f = p.n_f;
  const int ZT = sh.zt, KZ = sh.kz, STEPS = sh.steps;
  const int tid = threadIdx.x, lane = tid & 63, lane_id = lane;
  // wave-uniform (readfirstlane): the DMA loop, its buffer resources and the tile choices stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int wz = wave % WZ, we = wave / WZ;

  // output LayerNorm gamma / beta, and the zero padding columns of Zs (never written otherwise)
  for (int i = tid; i < 2 * D; i += NTHREAD) {
    const uint16_t* src = i < D ? p.out_gamma : p.out_beta;
    Gs[i] = src ? src[i < D ? i : i - D] : (uint16_t)(i < D ? 0x3f80u : 0u);
  }
  for (int i = tid; i < E * KJ * 16 * (ZP - D); i += NTHREAD) {
    const int row = i / (ZP - D), c = i - row * (ZP - D);
    Zs[(size_t)row * ZP + D + c] = 0;
  }

  // ---- DMA issue: instruction i of a step goes to wave i % 8; 0 .. ZTP-1 are
  // weight tiles, the rest X rows.
  const __amdgpu_buffer_rsrc_t rphi =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.phi, (short)0, k * n * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rwl =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.w_l, (short)0, n_l * n * 2, 0x00020000);
  auto dma_step = [&](const __amdgpu_buffer_rsrc_t& rx, uint16_t* sw, uint16_t* sx, int step) {
    const int k0 = step * KC;
    // The lane's offsets are recomputed at every step (a few VALU operations)
    // from an opaque copy of the lane index: hoisted out of the step loop they
    // would stay live through it, spill, and each reload's wait for the
    // vector-memory counter would also wait for the DMA in flight.
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int q = 0; q < INS_HI; ++q) {
      const int i = wave + q * NWAVE;  // wave-uniform
      if (i >= NINS) break;
      if (i < ZTP) {
        // weight tile i: row z = 16 i + lane / 4, columns k0 + 8 (lane % 4) .. + 7
        const int col = k0 + 8 * (lane & 3);
        const int r = 16 * i + (lane >> 2);
        uint16_t* dst = sw + i * 16 * KC;
        if (i < KZ) {
          const uint32_t vo = (r < k && col < n) ? (uint32_t)(r * n + col) * 2u : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rphi, WK_LDSV(dst), 16, vo, 0, 0, 0);
        } else {
          const int rl = r - 16 * KZ;
          const uint32_t vo = (rl < n_l && col < n) ? (uint32_t)(rl * n + col) * 2u : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rwl, WK_LDSV(dst), 16, vo, 0, 0, 0);
        }
      } else {
        const int j = i - ZTP;
        const int ex = j / (D / 16), bb = j - ex * (D / 16);
        const int o = bb * 512 + lane * 8;  // element offset within the example's KC x D rows
        const int row = o / D, col = o - row * D;
        uint16_t* dst = sx + ex * KC * D + bb * 512;
        const uint32_t vo = (k0 + row < n) ? (uint32_t)(((ex * n) + k0 + row) * D + col) * 2u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, WK_LDSV(dst), 16, vo, 0, 0, 0);
      }
    }
  };
  // per-group buffer resources: byte offsets stay 32-bit (one VGPR each) and
  // examples past the batch fall outside the record count (loads read zero,
  // stores are dropped)
  auto grp_rsrc = [&](const uint16_t* base, int64_t g, int per_ex) {
    const int64_t b0 = g * E;
    const int64_t rem = batch - b0;
    const int cnt = rem < E ? (int)rem : E;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + b0 * (int64_t)per_ex), (short)0, cnt * per_ex * 2,
                                             0x00020000);
  };
  auto x_rsrc = [&](int64_t g) {
    const int64_t b0 = g * E;
    const int64_t rem = batch - b0;
    const int cnt = rem < E ? (int)rem : E;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(p.x + b0 * (int64_t)n * D), (short)0, cnt * n * D * 2,
                                             0x00020000);
  };

  const int64_t groups = (batch + E - 1) / E;
  int64_t g = blockIdx.x;
  if (g >= groups) return;
  auto prologue = [&](int64_t grp) {  // steps 0 .. S-2 of a group into slots 0 .. S-2
    const __amdgpu_buffer_rsrc_t rx = x_rsrc(grp);
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
      if (u < STEPS) dma_step(rx, wslot[u], xslot[u], u);
  };
  prologue(g);
  const float inv_d = 1.0f / static_cast<float>(D);
  const float inv_nk = 1.0f / static_cast<float>(n * k);
  // X^T operand lanes: row 8 lg + li/4 (+4), column 4 (li % 4)
  const int xa = (8 * lg + (li >> 2)) * D + 4 * (li & 3);
  for (; g < groups; g += gridDim.x) {
    const int64_t gn = g + gridDim.x;
    const __amdgpu_buffer_rsrc_t rx = x_rsrc(g);
    // Lane coordinates re-derived through an opaque copy each group: the
    // per-lane offsets of the epilogue and phase 2 are then computed where they
    // are used instead of being hoisted out of this loop and kept live (spilled)
    // through phase 1.
    int lane_g = lane;
    asm volatile("" : "+v"(lane_g));
    const int li = lane_g & 15, lg = lane_g >> 4;
    // the FMB LayerNorm's gamma / beta at this lane's F positions (the same for
    // every example): loaded once per group when they fit in registers, else
    // once per example
    u32x2 fgam[MPW][KJ], fbet[MPW][KJ];
    const __amdgpu_buffer_rsrc_t rgam =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.fm_gamma, (short)0, p.fm_gamma ? n * k * 2 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rbet =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.fm_beta, (short)0, p.fm_beta ? n * k * 2 : 0, 0x00020000);
    const bool has_gamma = p.fm_gamma != nullptr;
    auto load_gb_row = [&](int mi, u32x2 (&gam)[KJ], u32x2 (&bet)[KJ]) {  // one 16-row block
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) {
        const int m = (wave + mi * NWAVE) * 16 + li;
        const int j0 = jt * 16 + lg * 4;
        const uint32_t off = (m < n && j0 < k) ? (uint32_t)(m * k + j0) * 2u : kOOB;
        gam[jt] = has_gamma ? __builtin_amdgcn_raw_buffer_load_b64(rgam, off, 0, 0) : u32x2{0x3f803f80u, 0x3f803f80u};
        bet[jt] = __builtin_amdgcn_raw_buffer_load_b64(rbet, off, 0, 0);  // zero when absent
      }
    };
    auto load_gb = [&]() {
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) load_gb_row(mi, fgam[mi], fbet[mi]);
    };

    // ---- phase 1: acc[zi][ex][et] = D[e][z] blocks of [Z; Lc]^T
    f32x4 acc[ZPW][EPW][ET];
#pragma unroll
    for (int zi = 0; zi < ZPW; ++zi)
#pragma unroll
      for (int ex = 0; ex < EPW; ++ex)
#pragma unroll
        for (int et = 0; et < ET; ++et) acc[zi][ex][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step t reads slot t % S and sends step t + S - 1 to slot (t + S - 1) % S
    auto step = [&](const uint16_t* sw, const uint16_t* sx, uint16_t* nw, uint16_t* nx, int t) {
      // step t must have landed; the (up to S - 2) steps issued after it may still be in flight
      const int newer = (STEPS - 1 - t < S - 2) ? STEPS - 1 - t : S - 2;
      if (newer <= 0) {
        __builtin_amdgcn_s_waitcnt(vm_enc(0));
      } else if (S > 3 && newer >= 2) {
        if (wave < R) __builtin_amdgcn_s_waitcnt(vm_enc(2 * INS_HI));
        else __builtin_amdgcn_s_waitcnt(vm_enc(2 * INS_LO));
      } else {
        if (wave < R) __builtin_amdgcn_s_waitcnt(vm_enc(INS_HI));
        else __builtin_amdgcn_s_waitcnt(vm_enc(INS_LO));
      }
      lds_barrier();
      if (t + S - 1 < STEPS) dma_step(rx, nw, nx, t + S - 1);
      if constexpr (GUARD) {
        // the step's X^T operands first, then one uniform test per weight tile
        u32x4 xo[EPW][ET];
#pragma unroll
        for (int ex = 0; ex < EPW; ++ex) {
          const uint16_t* xs = sx + (we * EPW + ex) * KC * D + xa;
#pragma unroll
          for (int et = 0; et < ET; ++et) xo[ex][et] = tr_pair(xs + et * 16, xs + 4 * D + et * 16);
        }
#pragma unroll
        for (int zi = 0; zi < ZPW; ++zi) {
          const int zt = wz * ZPW + zi;
          if (zt < ZT) {  // wave-uniform
            const u32x4 wf = *reinterpret_cast<const u32x4*>(sw + (zt * 16 + li) * KC + lg * 8);
#pragma unroll
            for (int ex = 0; ex < EPW; ++ex)
#pragma unroll
              for (int et = 0; et < ET; ++et) acc[zi][ex][et] = mfma16x16x32(xo[ex][et], wf, acc[zi][ex][et]);
          }
        }
      } else {
        u32x4 wf[ZPW];
#pragma unroll
        for (int zi = 0; zi < ZPW; ++zi)
          wf[zi] = *reinterpret_cast<const u32x4*>(sw + ((wz * ZPW + zi) * 16 + li) * KC + lg * 8);
#pragma unroll
        for (int ex = 0; ex < EPW; ++ex) {
          const uint16_t* xs = sx + (we * EPW + ex) * KC * D + xa;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const u32x4 a = tr_pair(xs + et * 16, xs + 4 * D + et * 16);
#pragma unroll
            for (int zi = 0; zi < ZPW; ++zi) acc[zi][ex][et] = mfma16x16x32(a, wf[zi], acc[zi][ex][et]);
          }
        }
      }
    };
    for (int t0 = 0; t0 < STEPS; t0 += S) {
#pragma unroll
      for (int u = 0; u < S; ++u) {  // unrolled: every slot is a known object at each step
        if (t0 + u >= STEPS) break;
        step(wslot[u], xslot[u], wslot[(u + S - 1) % S], xslot[(u + S - 1) % S], t0 + u);
      }
    }
    lds_barrier();  // every wave is done reading the ring
    if (gn < groups) prologue(gn);
    __builtin_amdgcn_sched_barrier(0);

    // ---- Z -> LDS, LCB rows of Y.  The residual rows are all requested first so
    // their latencies overlap.
    const __amdgpu_buffer_rsrc_t ry = grp_rsrc(p.y, g, n * D);
    u32x2 xres[ZPW][EPW][ET];
#pragma unroll
    for (int zi = 0; zi < ZPW; ++zi) {
      const int zt = wz * ZPW + zi;
      const int zl = zt * 16 + li - 16 * KZ;  // LCB output row (tiles >= KZ only)
#pragma unroll
      for (int ex = 0; ex < EPW; ++ex) {
        const bool valid = zt < ZT && zt >= KZ && zl < n_l;
        const uint32_t off = valid ? (uint32_t)(((we * EPW + ex) * n + n_f + zl) * D + lg * 4) * 2u : kOOB;
#pragma unroll
        for (int et = 0; et < ET; ++et) xres[zi][ex][et] = __builtin_amdgcn_raw_buffer_load_b64(rx, off + et * 32, 0, 0);
      }
    }
#pragma unroll
    for (int zi = 0; zi < ZPW; ++zi) {
      const int zt = wz * ZPW + zi;
      if (zt >= ZT) continue;  // wave-uniform
      const int z = zt * 16 + li;
      if (zt < KZ) {
#pragma unroll
        for (int ex = 0; ex < EPW; ++ex) {
          uint16_t* zrow = Zs + ((we * EPW + ex) * KJ * 16 + z) * ZP;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            u32x2 v;
            v[0] = pack_bf16x2(acc[zi][ex][et][0], acc[zi][ex][et][1]);
            v[1] = pack_bf16x2(acc[zi][ex][et][2], acc[zi][ex][et][3]);
            *reinterpret_cast<u32x2*>(zrow + et * 16 + lg * 4) = v;
          }
        }
      } else {
        const int zl = z - 16 * KZ;  // LCB output row
#pragma unroll
        for (int ex = 0; ex < EPW; ++ex) {
          const bool valid = zl < n_l;  // examples past the batch: dropped by the resource bound
          float v[ET][4];
          float sm = 0.f;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const u32x2 xv = xres[zi][ex][et];
            v[et][0] = acc[zi][ex][et][0] + bf16lo(xv[0]);
            v[et][1] = acc[zi][ex][et][1] + bf16hi(xv[0]);
            v[et][2] = acc[zi][ex][et][2] + bf16lo(xv[1]);
            v[et][3] = acc[zi][ex][et][3] + bf16hi(xv[1]);
            sm += (v[et][0] + v[et][1]) + (v[et][2] + v[et][3]);
          }
          sm += __shfl_xor(sm, 16, kWave);
          sm += __shfl_xor(sm, 32, kWave);
          const float mean = sm * inv_d;
          float q = 0.f;
#pragma unroll
          for (int et = 0; et < ET; ++et)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float dv = v[et][t] - mean;
              q += dv * dv;
            }
          q += __shfl_xor(q, 16, kWave);
          q += __shfl_xor(q, 32, kWave);
          const float rstd = rsqrtf(q * inv_d + p.eps);
          const uint32_t yoff = valid ? (uint32_t)(((we * EPW + ex) * n + n_f + zl) * D) * 2u : kOOB;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const int e = et * 16 + lg * 4;
            const u32x2 g2 = *reinterpret_cast<const u32x2*>(Gs + e);
            const u32x2 b2 = *reinterpret_cast<const u32x2*>(Gs + D + e);
            u32x2 o;
            o[0] = pack_bf16x2((v[et][0] - mean) * rstd * bf16lo(g2[0]) + bf16lo(b2[0]),
                               (v[et][1] - mean) * rstd * bf16hi(g2[0]) + bf16hi(b2[0]));
            o[1] = pack_bf16x2((v[et][2] - mean) * rstd * bf16lo(g2[1]) + bf16lo(b2[1]),
                               (v[et][3] - mean) * rstd * bf16hi(g2[1]) + bf16hi(b2[1]));
            __builtin_amdgcn_raw_buffer_store_b64(o, ry, yoff + e * 2, 0, 0);
          }
        }
      }
    }
    lds_barrier();  // Z complete
    // phases do not overlap in the schedule: keeps each one's registers to itself
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2, one example at a time: F^T = Z X^T, rows m of X from global
    // memory.  An example's X rows are requested together, and the next
    // example's while this one's statistics are reduced.
    const int MT = (n + 15) >> 4;
    const int KT = (k + 15) >> 4;
    u32x4 xf[MPW][NKS];
    auto load_x = [&](int ex) {  // example ex of the group
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) {
        const int m = (wave + mi * NWAVE) * 16 + li;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int e0 = ks * 32 + lg * 8;
          const uint32_t off = (m < n && e0 < D) ? (uint32_t)((ex * n + m) * D + e0) * 2u : kOOB;
          xf[mi][ks] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        }
      }
    };
    const __amdgpu_buffer_rsrc_t rfn = grp_rsrc(p.fn, g, n * k);
    load_x(0);
    if constexpr (GB_REG) load_gb();
    for (int ex = 0; ex < E; ++ex) {
      const int64_t b = g * E + ex;
      if (b >= batch) break;  // uniform over the workgroup
      const uint16_t* zs = Zs + ex * KJ * 16 * ZP;
      f32x4 facc[MPW][KJ];
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt) facc[mi][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) {
        if (wave + mi * NWAVE < MT) {  // wave-uniform
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int jt = 0; jt < KJ; ++jt)
              if (jt < KT) {
                const u32x4 zf = *reinterpret_cast<const u32x4*>(zs + (jt * 16 + li) * ZP + ks * 32 + lg * 8);
                facc[mi][jt] = mfma16x16x32(zf, xf[mi][ks], facc[mi][jt]);
              }
        }
      }
      if (ex + 1 < E && b + 1 < batch) load_x(ex + 1);
      // without room for every block's gamma / beta: two blocks' worth, the
      // next one requested while the current one is written
      u32x2 gA[KJ], bA[KJ], gB[KJ], bB[KJ];
      if constexpr (!GB_REG) load_gb_row(0, gA, bA);
      float sm = 0.f;
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int m = (wave + mi * NWAVE) * 16 + li;
            const int j = jt * 16 + lg * 4 + t;
            if (m < n && j < k) sm += facc[mi][jt][t];
          }
      sm = group_sum_v<64>(sm);
      if (lane == 0) red[wave] = sm;
      lds_barrier();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) tot += red[w];
      const float mean = tot * inv_nk;
      float q = 0.f;
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int m = (wave + mi * NWAVE) * 16 + li;
            const int j = jt * 16 + lg * 4 + t;
            if (m < n && j < k) {
              const float dv = facc[mi][jt][t] - mean;
              q += dv * dv;
            }
          }
      q = group_sum_v<64>(q);
      if (lane == 0) red[NWAVE + wave] = q;
      lds_barrier();
      float qt = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) qt += red[NWAVE + w];
      const float rstd = rsqrtf(qt * inv_nk + p.eps);
      auto fn_store = [&](int mi, const u32x2 (&gam)[KJ], const u32x2 (&bet)[KJ]) {
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt) {
          const int m = (wave + mi * NWAVE) * 16 + li;
          const int j0 = jt * 16 + lg * 4;
          if (m < n && j0 < k) {  // k % 4 == 0: the 4 values j0 .. j0+3 are all valid
            const u32x2 g2 = gam[jt], b2 = bet[jt];
            const f32x4 f = facc[mi][jt];
            u32x2 o;
            o[0] = pack_bf16x2((f[0] - mean) * rstd * bf16lo(g2[0]) + bf16lo(b2[0]),
                               (f[1] - mean) * rstd * bf16hi(g2[0]) + bf16hi(b2[0]));
            o[1] = pack_bf16x2((f[2] - mean) * rstd * bf16lo(g2[1]) + bf16lo(b2[1]),
                               (f[3] - mean) * rstd * bf16hi(g2[1]) + bf16hi(b2[1]));
            __builtin_amdgcn_raw_buffer_store_b64(o, rfn, (uint32_t)((ex * n + m) * k + j0) * 2u, 0, 0);
          }
        }
      };
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) {
        if constexpr (GB_REG) {
          fn_store(mi, fgam[mi], fbet[mi]);
        } else if (mi & 1) {
          if (mi + 1 < MPW) load_gb_row(mi + 1, gA, bA);
          fn_store(mi, gB, bB);
        } else {
          if (mi + 1 < MPW) load_gb_row(mi + 1, gB, bB);
          fn_store(mi, gA, bA);
        }
      }
    }
  }
}


struct StreamVariant {
  int et, zpw, wz, we, epw, mpw, kj, ztmax, s;
  void (*kernel)(FmbLcbArgs, int64_t, StreamShape);
};

#define WK_STREAM(ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, GUARD)                 \
  StreamVariant {                                                                 \
    ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S,                                      \
        fmb_lcb_stream_kernel<ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, GUARD>     \
  }

// LDS per variant (static): S x (ZTMAX 16 KC + E KC D) + E KJ 16 ZP + 2 D u16.
const StreamVariant kStream[] = {
    WK_STREAM(10, 3, 4, 2, 1, 2, 3, 12, 3, false),  // n<=256, d=160, k<=48, ZT<=12: 2 examples per group
    WK_STREAM(10, 3, 8, 1, 1, 4, 6, 24, 3, false),  // n<=512, d=160, k<=96, ZT<=24
    WK_STREAM(2, 4, 8, 1, 4, 6, 2, 25, 4, true),    // n<=768, d=32,  k<=32, ZT<=25: 4 examples per group
};

StreamShape stream_shape(const StreamVariant& v, int n, int k, int n_l) {
  StreamShape sh;
  sh.kz = (k + 15) / 16;
  sh.zt = sh.kz + (n_l + 15) / 16;
  sh.steps = (n + KC - 1) / KC;
  sh.e = v.we * v.epw;
  return sh;
}

const StreamVariant* pick_stream(int n, int d, int k, int n_l, StreamShape* out) {
  if (d % 16 != 0) return nullptr;
  for (const auto& v : kStream) {
    if (16 * v.et != d) continue;
    const StreamShape sh = stream_shape(v, n, k, n_l);
    if (sh.zt > v.ztmax || sh.zt > v.wz * v.zpw) continue;  // DMA'd tiles and tiles with an owner wave
    if (sh.kz > v.kj) continue;
    if ((n + 15) / 16 > NWAVE * v.mpw) continue;

    // 32-bit byte offsets within one group's X and within the weights
    if ((int64_t)sh.e * n * d * 2 >= (int64_t)1 << 31 || (int64_t)(k + n_l) * n * 2 >= (int64_t)1 << 31) continue;
    if (out) *out = sh;
    return &v;
  }
  return nullptr;
}

}  // namespace

bool fmb_lcb_stream_supported(int n, int d, int k, int n_l) { return pick_stream(n, d, k, n_l, nullptr) != nullptr; }

hipError_t launch_fmb_lcb_stream(const FmbLcbArgs& a, int64_t batch, hipStream_t stream, int64_t* workgroups) {
  StreamShape sh;
  const StreamVariant* v = pick_stream(a.n, a.d, a.k, a.n_l, &sh);
  if (!v) return hipErrorInvalidValue;
  const int64_t groups = (batch + sh.e - 1) / sh.e;
  const int64_t grid = groups < 256 ? groups : 256;
  if (workgroups) *workgroups = grid;
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)grid), dim3(NTHREAD), 0, stream, a, batch, sh);
  return hipGetLastError();
}

}  // namespace wk
