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
// 16-row tiles and W_L the following ones.  A pack kernel first rearranges
// [Phi; W_L] into the ring's own order (step, tile, 16 rows x 32 columns,
// zero padded), so each weight DMA instruction copies 1 KB of consecutive
// bytes instead of 16 row pieces of 64 bytes (half an L2 line each).  The
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
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
  int ztp;   // weight tiles per step in the packed weights and in a ring slot (the variant's ZTMAX >= zt)
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
// TRAIN: the training forward also stores Z (bf16, as the interaction uses it) and Lc (fp32, as
// the LCB rows' LayerNorm uses it) for the backward.
// CONTIG: [Phi; W_L] rows are packed without padding between Phi and W_L (row z < k is Phi's,
// z - k W_L's), so a tile may hold both kinds; a lane's row kind is decided per lane.
template <int ET, int ZPW, int WZ, int WE, int EPW, int MPW, int KJ, int ZTMAX, int S, bool GUARD, bool CONTIG,
          bool TRAIN>
__global__ __launch_bounds__(NTHREAD, 2) void fmb_lcb_stream_kernel(FmbLcbArgs p, int64_t batch, StreamShape sh) {
  constexpr int D = 16 * ET;
  constexpr int E = WE * EPW;
  constexpr int ZP = zs_pitch(D);
  constexpr int DZ = (D + 31) / 32 * 32;
  constexpr int NKS = DZ / 32;                 // 32-wide K steps of phase 2
  constexpr bool GB_REG = MPW * KJ <= 12;      // FMB LayerNorm gamma / beta held in registers
  // DMA instructions per step: ZTP = ZTMAX 16-row weight tiles of 1 KB (the
  // packed weights hold ZTP tiles per step; those past the shape's ZT are
  // zero) and X_INS for the X rows (1 KB each).  Weight tile i = 8 q + wave
  // goes out in round q, then X instruction j = 8 q + wave: every wave issues
  // the same code, and only the last round of each kind is partial (waves
  // below RW, RX).  A wave's copies per step are C0 + (wave < RW) + (wave < RX).
  constexpr int X_INS = E * D / 16;
  constexpr int ZTP = ZTMAX;  // >= the shape's ZT (host check); may exceed WZ * ZPW (padding tiles)
  constexpr int WQ = (ZTP + NWAVE - 1) / NWAVE, XQ = (X_INS + NWAVE - 1) / NWAVE;
  constexpr int RW = ZTP % NWAVE, RX = X_INS % NWAVE;
  constexpr int C0 = ZTP / NWAVE + X_INS / NWAVE;
  constexpr int SW = ZTP * 16 * KC;       // weight part of a ring slot (u16)
  constexpr int SX = E * KC * D;          // X part of a ring slot
  static_assert(WZ * WE == NWAVE, "8 waves");
  static_assert(S == 3 || S == 4, "ring of 3 or 4 slots");
  static_assert(GUARD || ZTMAX >= WZ * ZPW, "unguarded tiles must lie in the slot");
  static_assert(2 * (WQ + XQ) <= 63, "vmcnt range");
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
  if constexpr (CONTIG) {  // Z rows k .. 16 KJ - 1 stay zero (their tile rows are W_L's)
    for (int i = tid; i < E * KJ * 16 * D; i += NTHREAD) {
      const int row = i / D, c = i - row * D;
      if (row % (KJ * 16) >= p.k) Zs[(size_t)row * ZP + c] = 0;
    }
  }

  // ---- DMA issue.  The packed weights: step t, tile i at byte (t ZTP + i) 1024.
  const __amdgpu_buffer_rsrc_t rpk =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.wpack, (short)0, STEPS * ZTP * 1024, 0x00020000);
  const bool ragged = n % KC != 0;  // the last step has rows past n, which read as zero
  auto dma_step = [&](const __amdgpu_buffer_rsrc_t& rx, uint16_t* sw, uint16_t* sx, int step) {
    const int k0 = step * KC;
    // The lane's offsets are recomputed at every step (a few VALU operations)
    // from an opaque copy of the lane index: hoisted out of the step loop they
    // would stay live through it, spill, and each reload's wait for the
    // vector-memory counter would also wait for the DMA in flight.
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const uint32_t l16 = (uint32_t)lane * 16u;
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int i = q * NWAVE + wave;  // wave-uniform
      if (RW != 0 && q == WQ - 1 && i >= ZTP) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rpk, WK_LDSV(sw + i * 16 * KC), 16,
                                               l16 + (uint32_t)((step * ZTP + i) * 1024), 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int j = q * NWAVE + wave;  // wave-uniform
      if (RX != 0 && q == XQ - 1 && j >= X_INS) break;
      const int ex = j / (D / 16), bb = j - ex * (D / 16);
      // elements bb 512 + 8 lane .. + 7 of the example's KC x D block of rows k0 ..
      uint32_t vo = l16 + (uint32_t)(((ex * n + k0) * D + bb * 512) * 2);
      if (ragged && k0 + KC > n && k0 + (bb * 512 + lane * 8) / D >= n) vo = kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, WK_LDSV(sx + ex * KC * D + bb * 512), 16, vo, 0, 0, 0);
    }
  };
  // wait until this wave's copies of a step have landed while the `newer` (0 .. 2)
  // steps issued after it may still be in flight
  const int extra = (wave < RW ? 1 : 0) + (wave < RX ? 1 : 0);  // wave-uniform
  auto wait_copies = [&](int newer) {
    if (newer <= 0) {
      __builtin_amdgcn_s_waitcnt(vm_enc(0));
    } else if (newer == 1) {
      if (extra == 0) __builtin_amdgcn_s_waitcnt(vm_enc(C0));
      else if (extra == 1) __builtin_amdgcn_s_waitcnt(vm_enc(C0 + 1));
      else __builtin_amdgcn_s_waitcnt(vm_enc(C0 + 2));
    } else {
      if (extra == 0) __builtin_amdgcn_s_waitcnt(vm_enc(2 * C0));
      else if (extra == 1) __builtin_amdgcn_s_waitcnt(vm_enc(2 * C0 + 2));
      else __builtin_amdgcn_s_waitcnt(vm_enc(2 * C0 + 4));
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
      wait_copies((STEPS - 1 - t < S - 2) ? STEPS - 1 - t : S - 2);
      ring_barrier();
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
    __amdgpu_buffer_rsrc_t rz = ry, rlc = ry;
    if constexpr (TRAIN) {
      rz = grp_rsrc(p.z_out, g, k * D);
      const int64_t b0 = g * E;
      const int cnt = batch - b0 < E ? (int)(batch - b0) : E;
      rlc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.lc_out + b0 * (int64_t)n_l * D), (short)0,
                                              cnt * n_l * D * 4, 0x00020000);
    }
    // lane row kinds: Z row z < k (CONTIG) or tile < KZ; else LCB output row zl
    auto is_z = [&](int zt, int z) { return CONTIG ? z < k : zt < KZ; };
    auto lcb_row = [&](int z) { return CONTIG ? z - k : z - 16 * KZ; };
    // the residual rows X[n_f + zl] of one example, requested one example ahead
    auto load_res = [&](int ex, u32x2 (&xr)[ZPW][ET]) {
#pragma unroll
      for (int zi = 0; zi < ZPW; ++zi) {
        const int zt = wz * ZPW + zi;
        const int z = zt * 16 + li, zl = lcb_row(z);
        const bool valid = zt < ZT && !is_z(zt, z) && zl < n_l;
        const uint32_t off = valid ? (uint32_t)(((we * EPW + ex) * n + n_f + zl) * D + lg * 4) * 2u : kOOB;
#pragma unroll
        for (int et = 0; et < ET; ++et) xr[zi][et] = __builtin_amdgcn_raw_buffer_load_b64(rx, off + et * 32, 0, 0);
      }
    };
    u32x2 xres[2][ZPW][ET];
    load_res(0, xres[0]);
#pragma unroll
    for (int ex = 0; ex < EPW; ++ex) {
      if (ex + 1 < EPW) load_res(ex + 1, xres[(ex + 1) & 1]);
#pragma unroll
      for (int zi = 0; zi < ZPW; ++zi) {
        const int zt = wz * ZPW + zi;
        if (zt >= ZT) continue;  // wave-uniform
        const int z = zt * 16 + li;
        if (is_z(zt, z)) {  // uniform unless CONTIG (then the 4 lanes of a row agree)
          uint16_t* zrow = Zs + ((we * EPW + ex) * KJ * 16 + z) * ZP;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            u32x2 v;
            v[0] = pack_bf16x2(acc[zi][ex][et][0], acc[zi][ex][et][1]);
            v[1] = pack_bf16x2(acc[zi][ex][et][2], acc[zi][ex][et][3]);
            *reinterpret_cast<u32x2*>(zrow + et * 16 + lg * 4) = v;
            if constexpr (TRAIN) {
              const uint32_t zoff = z < k ? (uint32_t)(((we * EPW + ex) * k + z) * D + et * 16 + lg * 4) * 2u : kOOB;
              __builtin_amdgcn_raw_buffer_store_b64(v, rz, zoff, 0, 0);
            }
          }
        } else {
          const int zl = lcb_row(z);  // LCB output row
          const bool valid = zl < n_l;  // examples past the batch: dropped by the resource bound
          if constexpr (TRAIN) {
            const uint32_t loff = valid ? (uint32_t)(((we * EPW + ex) * n_l + zl) * D + lg * 4) * 4u : kOOB;
#pragma unroll
            for (int et = 0; et < ET; ++et)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[zi][ex][et]), rlc,
                                                     loff + et * 64, 0, 0);
          }
          float v[ET][4];
          float sm = 0.f;
#pragma unroll
          for (int et = 0; et < ET; ++et) {
            const u32x2 xv = xres[ex & 1][zi][et];
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
    // Fn row-major per group, or K-blocked over the whole batch (64-column blocks of
    // fn_kblock_rows rows: the first Linear's A operand; the host keeps it below 2 GB)
    const uint32_t fkb = (uint32_t)p.fn_kblock_rows;
    const __amdgpu_buffer_rsrc_t rfn =
        fkb ? __builtin_amdgcn_make_buffer_rsrc((void*)p.fn, (short)0, (int)(fkb * (uint32_t)(n * k) * 2u), 0x00020000)
            : grp_rsrc(p.fn, g, n * k);
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
            const uint32_t c = (uint32_t)(m * k + j0);  // 4-aligned: the 4 values share a 64-column block
            const uint32_t off = fkb ? (((c >> 6) * fkb + (uint32_t)b) * 64u + (c & 63u)) * 2u
                                     : (uint32_t)((ex * n + m) * k + j0) * 2u;
            __builtin_amdgcn_raw_buffer_store_b64(o, rfn, off, 0, 0);
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


// FMB + LCB with [Phi; W_L] held in registers and X streamed in 32-column
// chunks (bf16, fp32 accumulation; the plain forward).
//
// The interaction is a sum over embedding columns: with Z_b = Phi X_b,
// F_b = X_b Z_b^T = sum_c X_b[:, c] Z_b[:, c]^T over column blocks c, and
// Z_b[:, c] = Phi X_b[:, c] needs only the same columns of X_b (Wukong paper,
// section 2.2: compress, then interact).  The LCB rows Lc_b = W_L X_b split by
// columns the same way.  So one pass over X, chunk by chunk, finishes
// everything an example needs while the chunk is in LDS: [Z; Lc][:, c], the
// residual X_b[n_F + i][c] added to the LCB columns, Z[:, c] rounded to bf16
// into LDS, and F_b += X_b[:, c] Z_b[:, c]^T.  X is read from HBM exactly once
// per layer (the two-phase kernel reads it twice when a group's X does not
// stay in L2 between its phases).
//
// Work split: a persistent workgroup of 4 waves (one per SIMD) takes one
// example at a time.  The weights are the same for every example, so each
// wave keeps its MFMA operand fragments of [Phi; W_L] in registers for the
// whole kernel: its Phi tile (wave < ceil(k / 16)) and W_L tiles wave and
// wave + 4, all n columns (the n = 256 layer: 96 registers).  LDS then holds
// only the X ring: NCH = d / 32 chunks of n rows x 32 columns (16 KB) per
// example in NCH slots, each chunk requested NCH - 1 chunks ahead (the next
// example's first chunks are in flight during this one's epilogue).  Phase A
// of a chunk multiplies its two 16-column tiles (the X^T operand, read with
// ds_read_b64_tr_b16) by the wave's weight tiles over K = n; phase B adds
// Z_c X_c^T to the wave's F^T blocks (rows wave + 4 mi of X).  A wave keeps
// its two LCB row tiles of every chunk in registers until the example's
// LayerNorm over d.
template <int N, int D, int MPW, int KJ>
__global__ __launch_bounds__(256, 1) void fmb_lcb_dchunk_kernel(FmbLcbArgs p, int64_t batch, StreamShape sh) {
  constexpr int NW = 4;                 // waves
  constexpr int CW = 32;                // chunk width (embedding columns)
  constexpr int NCH = D / CW;           // chunks per example = ring slots
  constexpr int S = NCH;
  constexpr int STEPS = N / KC;         // K steps of phase A
  constexpr int MT = N / 16;            // 16-row blocks of X
  constexpr int CX = N / 16 / NW;       // chunk DMA instructions per wave (1 KB = 16 rows x 32 columns)
  constexpr int ZP = CW + 8;            // Zs row pitch (u16)
  constexpr int SX = N * CW;            // ring slot (u16)
  // stores a wave issues per example: the LCB rows (2 tiles x NCH x 2) and Fn (MPW x KJ)
  constexpr int STORES = 2 * NCH * 2 + MPW * KJ;
  static_assert(D % CW == 0 && N % (16 * NW) == 0 && MT == NW * MPW, "shape");
  static_assert(S >= 3 && S <= 5, "ring slots");
  static_assert((S - 2) * CX + STORES <= 63, "vmcnt range");
  __shared__ __align__(16) uint16_t x0[SX], x1[SX], x2[SX], x3[S > 3 ? SX : 8], x4[S > 4 ? SX : 8];
  // a select rather than a table of pointers: a table with a constant initialiser may be
  // placed in constant memory, and a pointer loaded from there is taken to be global
  auto xslot = [&](int i) -> uint16_t* { return i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : i == 3 ? x3 : x4; };
  __shared__ __align__(16) uint16_t Zs[KJ * 16 * ZP];
  __shared__ __align__(16) float GsF[2 * D];  // the output LayerNorm's gamma, then beta (fp32)
  __shared__ __align__(16) uint16_t Gfm[2 * N * 16 * KJ];  // the FMB LayerNorm's gamma, then beta ([n k] each)
  __shared__ float red[2 * NW];

  const int k = p.k, n_f = p.n_f;
  const int KZ = sh.kz, ZTP = sh.ztp;
  const int KT = (k + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t first = blockIdx.x;
  if (first >= batch) return;
  const int64_t stride = gridDim.x;

  for (int i = tid; i < 2 * D; i += 256) {
    const uint16_t* src = i < D ? p.out_gamma : p.out_beta;
    GsF[i] = src ? bf16_to_f32(src[i < D ? i : i - D]) : (i < D ? 1.f : 0.f);
  }
  for (int i = tid; i < KJ * 16 * ZP; i += 256) Zs[i] = 0;  // rows past 16 KZ stay zero
  {  // the FMB LayerNorm's gamma / beta into LDS, 16 bytes per lane, all loads issued together
    const int nkg = N * k / 8;  // k % 16 == 0
    const __amdgpu_buffer_rsrc_t rgam =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.fm_gamma, (short)0, p.fm_gamma ? N * k * 2 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rbet =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.fm_beta, (short)0, p.fm_beta ? N * k * 2 : 0, 0x00020000);
    constexpr int GR = (N * KJ * 16 / 8 + 255) / 256;
    u32x4 gv[GR], bv[GR];
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      const uint32_t off = (uint32_t)(tid + r * 256) * 16u;
      gv[r] = p.fm_gamma ? __builtin_amdgcn_raw_buffer_load_b128(rgam, off, 0, 0)
                         : u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
      bv[r] = __builtin_amdgcn_raw_buffer_load_b128(rbet, off, 0, 0);  // zero when absent
    }
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      const int i = tid + r * 256;
      if (i < nkg) {
        *reinterpret_cast<u32x4*>(Gfm + i * 8) = gv[r];
        *reinterpret_cast<u32x4*>(Gfm + N * k + i * 8) = bv[r];
      }
    }
  }

  // ---- chunk c of example b into a slot: row r of the chunk at r CW, lane l of
  // instruction j holding row 16 j + l / 4, columns 8 (l % 4) .. + 7.  An example
  // past the batch gets a resource of no records: its lanes read nothing and the
  // slot it lands in is never consumed; issuing it anyway keeps the count of copies
  // in flight the same at every chunk.
  // The copies are written as inline asm: the compiler then does not track them, and
  // inserts no wait for them before LDS reads it cannot prove disjoint from the slot
  // being filled (it loses track of which slot a read addresses).  Every wait for them
  // is explicit (vmcnt before the chunk's barrier), and the asm's memory clobber keeps
  // LDS accesses from moving across an issue.
  const uint32_t xlane = (uint32_t)(((lane >> 2) * D + (lane & 3) * 8) * 2);
  auto dma_chunk = [&](uint16_t* sx, int64_t b, int c) {
    const bool in = b < batch;  // uniform
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(in ? p.x + b * (int64_t)N * D : p.x), (short)0, in ? N * D * 2 : 0, 0x00020000);
#pragma unroll
    for (int q = 0; q < CX; ++q) {
      const int j = q * NW + wave;
      const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(WK_LDSV(sx + j * 512));
      // s_nop 4: the hazard recogniser does not look inside asm, and the offset, resource or
      // M0 may have just been written by a vector instruction (v_readlane), which a vector
      // memory instruction may only read five wait states later
      asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                   :
                   : "v"(xlane), "s"(rx), "s"(__builtin_amdgcn_readfirstlane((16 * j * D + CW * c) * 2)),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                   : "memory");
    }
  };
  // ---- the weight fragments, from the packed [Phi; W_L] (step t, tile i: 1 KB at
  // (t ZTP + i) 1024; lane 4 r + g of it holds row 16 i + r, columns 32 t + 8 g ..):
  // lane (li, lg) takes row li, columns 8 lg .. of each step
  u32x4 wz[STEPS], wlc[2][STEPS];
  {
    const __amdgpu_buffer_rsrc_t rpk =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.wpack, (short)0, STEPS * ZTP * 1024, 0x00020000);
    const uint32_t lo = (uint32_t)(4 * li + lg) * 16u;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const uint32_t zo = wave < KZ ? (uint32_t)((t * ZTP + wave) * 1024) + lo : kOOB;
      wz[t] = __builtin_amdgcn_raw_buffer_load_b128(rpk, zo, 0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        wlc[i][t] = __builtin_amdgcn_raw_buffer_load_b128(rpk, (uint32_t)((t * ZTP + KZ + wave + NW * i) * 1024) + lo,
                                                           0, 0);
    }
  }
  // the first example's chunks 0 .. S - 2 (after the register loads, which the first wait covers)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) dma_chunk(xslot(s), first, s);

  const float inv_d = 1.0f / static_cast<float>(D);
  const float inv_nk = 1.0f / static_cast<float>(N * k);
  const int xa = (8 * lg + (li >> 2)) * CW + 4 * (li & 3);  // X^T operand lanes (ds_read_b64_tr_b16)
  const uint32_t fkb = (uint32_t)p.fn_kblock_rows;
  const bool has_z = wave < KZ;  // wave-uniform

  // The output stage of an example (the LCB rows' LayerNorm and Y stores, the FMB
  // LayerNorm and Fn stores) is software-pipelined into the next example's first two
  // chunks: its statistics are reduced at the end of the example (the FMB sums go to
  // `red`, published by the next chunk's barrier), and its 32 normalise-and-store
  // units are spread over those chunks' K steps (the Fn blocks and the first LCB tile
  // in chunk 0, the second LCB tile in chunk 1), where the vector ALU work and the
  // stores fill issue slots between MFMAs.  Before the first example the units run on
  // zeros with resources of no records (the stores are dropped), so every example's
  // first two chunks issue the same stores.
  f32x4 plc[2][NCH][2];  // the previous example's LCB rows (Lc + residual)
  f32x4 pfacc[MPW][KJ];  // and its F^T blocks
  float pmean[2] = {0.f, 0.f}, prstd[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NCH; ++c) plc[i][c][0] = plc[i][c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
    for (int jt = 0; jt < KJ; ++jt) pfacc[mi][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (lane == 0) red[wave] = red[NW + wave] = 0.f;
  int64_t pb = first;  // the previous example
  bool live = false;   // uniform: there is a previous example
  constexpr int UNITS = 2 * NCH * 2 + MPW * KJ;  // = STORES
  static_assert(UNITS == STORES, "one store per unit");
  constexpr int U0 = MPW * KJ + 2 * NCH, U1 = 2 * NCH;  // units (stores) in chunks 0 and 1
  static_assert(U0 + U1 == UNITS, "every unit scheduled");

  // resources of the previous example's outputs (no records before the first example)
  auto out_rsrc = [&](__amdgpu_buffer_rsrc_t& ry, __amdgpu_buffer_rsrc_t& rfn) {
    ry = __builtin_amdgcn_make_buffer_rsrc((void*)(p.y + pb * (int64_t)N * D), (short)0, live ? N * D * 2 : 0,
                                           0x00020000);
    // (assembled from uniform values: the compiler cannot tell the select is uniform, and a
    // resource it takes for divergent turns every store into a loop over lanes)
    const uint64_t fbase = reinterpret_cast<uint64_t>(fkb ? p.fn : p.fn + pb * (int64_t)N * k);
    const uint64_t fb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(fbase >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)fbase);
    const int frec = !live ? 0 : fkb ? (int)(fkb * (uint32_t)(N * k) * 2u) : N * k * 2;
    rfn = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(fb), (short)0,
                                            __builtin_amdgcn_readfirstlane(frec), 0x00020000);
  };
  // unit u < 2 NCH 2: LCB tile i, chunk c, half et of the previous example; else its Fn block
  auto out_unit = [&](int u, const __amdgpu_buffer_rsrc_t& ry, const __amdgpu_buffer_rsrc_t& rfn, float fm_mean,
                      float fm_rstd) {
    if (u < 2 * NCH * 2) {
      const int i = u / (2 * NCH), c = (u / 2) % NCH, et = u % 2;
      const int zl = (wave + NW * i) * 16 + li;
      const int e = c * CW + et * 16 + lg * 4;
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(GsF + e);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(GsF + D + e);
      const f32x4 v = plc[i][c][et];
      const float mean = pmean[i], rstd = prstd[i];
      u32x2 o;
      o[0] = pack_bf16x2((v[0] - mean) * rstd * g4[0] + b4[0], (v[1] - mean) * rstd * g4[1] + b4[1]);
      o[1] = pack_bf16x2((v[2] - mean) * rstd * g4[2] + b4[2], (v[3] - mean) * rstd * g4[3] + b4[3]);
      __builtin_amdgcn_raw_buffer_store_b64(o, ry, (uint32_t)(((n_f + zl) * D + e) * 2), 0, 0);
    } else {
      const int q = u - 2 * NCH * 2, mi = q / KJ, jt = q % KJ;
      const int m = (wave + mi * NW) * 16 + li;
      const int j0 = jt * 16 + lg * 4;  // k % 4 == 0: the 4 values j0 .. j0+3 are all valid or all not
      const int gi = j0 < k ? m * k + j0 : 0;
      const u32x2 g2 = *reinterpret_cast<const u32x2*>(Gfm + gi);
      const u32x2 b2 = *reinterpret_cast<const u32x2*>(Gfm + N * k + gi);
      const f32x4 f = pfacc[mi][jt];
      u32x2 o;
      o[0] = pack_bf16x2((f[0] - fm_mean) * fm_rstd * bf16lo(g2[0]) + bf16lo(b2[0]),
                         (f[1] - fm_mean) * fm_rstd * bf16hi(g2[0]) + bf16hi(b2[0]));
      o[1] = pack_bf16x2((f[2] - fm_mean) * fm_rstd * bf16lo(g2[1]) + bf16lo(b2[1]),
                         (f[3] - fm_mean) * fm_rstd * bf16hi(g2[1]) + bf16hi(b2[1]));
      // every lane stores (those past k to an offset past the record count), so each
      // unit is exactly one store
      const uint32_t cc = (uint32_t)(m * k + j0);  // 4-aligned: the 4 values share a 64-column block
      const uint32_t off = j0 >= k ? kOOB : fkb ? (((cc >> 6) * fkb + (uint32_t)pb) * 64u + (cc & 63u)) * 2u : cc * 2u;
      __builtin_amdgcn_raw_buffer_store_b64(o, rfn, off, 0, 0);
    }
  };
  // the FMB LayerNorm statistics of the previous example, from every wave's sums
  auto fm_stats = [&](float& mean, float& rstd) {
    mean = ((red[0] + red[1]) + (red[2] + red[3])) * inv_nk;
    const float ex2 = ((red[NW] + red[NW + 1]) + (red[NW + 2] + red[NW + 3])) * inv_nk;
    rstd = rsqrtf(fmaxf(ex2 - mean * mean, 0.f) + p.eps);
  };

  for (int64_t b = first; b < batch; b += stride) {
    f32x4 lc[2][NCH][2];  // LCB row tiles: lane holds e = 32 c + 16 et + 4 lg + t, row 16 (wave + 4 i) + li
    f32x4 facc[MPW][KJ];  // F^T blocks: lane holds j = 16 jt + 4 lg + t, m = 16 (wave + 4 mi) + li
#pragma unroll
    for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) facc[mi][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint16_t* sx = xslot(c);
      // chunk c landed.  Newer operations: the copies of the S - 2 chunks after it, and the
      // previous example's stores issued after its copy: U0 in chunk 0 (after the copies of
      // chunks 1 .. 3, before chunk 4's) and U1 in chunk 1 (after chunk 4's copy)
      if (c == 1) __builtin_amdgcn_s_waitcnt(vm_enc((S - 2) * CX + U0));
      else if (c == 2 || c == 3) __builtin_amdgcn_s_waitcnt(vm_enc((S - 2) * CX + U0 + U1));
      else if (c == 4) __builtin_amdgcn_s_waitcnt(vm_enc((S - 2) * CX + U1));
      else __builtin_amdgcn_s_waitcnt(vm_enc((S - 2) * CX));
      ring_barrier();  // the chunk landed for every wave; slot c - 1 and Zs are free
      __amdgpu_buffer_rsrc_t ry, rfn;
      float fm_mean = 0.f, fm_rstd = 0.f;
      if (c <= 1) out_rsrc(ry, rfn);
      if (c == 0) fm_stats(fm_mean, fm_rstd);
      // phase A: [Z; Lc]^T[:, chunk] = X_c^T [Phi; W_L]^T, the LCB accumulators starting
      // from the residual rows X[n_F + i][chunk] (so no vector ALU touches them before the
      // LayerNorm)
      f32x4 za[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int zl = (wave + NW * i) * 16 + li;  // < n_l (every W_L tile is full)
        const uint16_t* xr = sx + (n_f + zl) * CW + lg * 4;
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          const u32x2 xv = *reinterpret_cast<const u32x2*>(xr + et * 16);
          lc[i][c][et] = f32x4{bf16lo(xv[0]), bf16hi(xv[0]), bf16lo(xv[1]), bf16hi(xv[1])};
        }
      }
      // the next step's X^T operands are requested before this step's MFMAs
      u32x4 xn0 = tr_pair(sx + xa, sx + xa + 4 * CW), xn1 = tr_pair(sx + xa + 16, sx + xa + 4 * CW + 16);
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const u32x4 xo0 = xn0, xo1 = xn1;
        if (t + 1 < STEPS) {
          const uint16_t* xs = sx + (t + 1) * KC * CW + xa;
          xn0 = tr_pair(xs, xs + 4 * CW);
          xn1 = tr_pair(xs + 16, xs + 4 * CW + 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          lc[i][c][0] = mfma16x16x32(xo0, wlc[i][t], lc[i][c][0]);
          lc[i][c][1] = mfma16x16x32(xo1, wlc[i][t], lc[i][c][1]);
        }
        // (waves past the Phi tiles hold zero fragments: no branch in the MFMA stream)
        za[0] = mfma16x16x32(xo0, wz[t], za[0]);
        za[1] = mfma16x16x32(xo1, wz[t], za[1]);
        // the previous example's output units: in chunk 0 its Fn blocks and first LCB tile
        // (U0), in chunk 1 its second LCB tile (U1), spread over the K steps
        if (c == 0) {
#pragma unroll
          for (int v = t * U0 / STEPS; v < (t + 1) * U0 / STEPS; ++v)
            out_unit(v < MPW * KJ ? 2 * NCH * 2 + v : v - MPW * KJ, ry, rfn, fm_mean, fm_rstd);
        } else if (c == 1) {
#pragma unroll
          for (int v = t * U1 / STEPS; v < (t + 1) * U1 / STEPS; ++v) out_unit(2 * NCH + v, ry, rfn, fm_mean, fm_rstd);
        }
      }
      // Z columns to LDS (bf16, the interaction's operand)
      if (has_z) {
        uint16_t* zrow = Zs + (wave * 16 + li) * ZP + lg * 4;
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          u32x2 v;
          v[0] = pack_bf16x2(za[et][0], za[et][1]);
          v[1] = pack_bf16x2(za[et][2], za[et][3]);
          *reinterpret_cast<u32x2*>(zrow + et * 16) = v;
        }
      }
      // phase B's X rows are requested before the barrier (the chunk itself is complete)
      u32x4 xf4[MPW];
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
        xf4[mi] = *reinterpret_cast<const u32x4*>(sx + ((wave + mi * NW) * 16 + li) * CW + lg * 8);
      ring_barrier();  // Z columns of the chunk complete
      // phase B: F^T += Z_c X_c^T
      u32x4 zf[KJ];
#pragma unroll
      for (int jt = 0; jt < KJ; ++jt) zf[jt] = *reinterpret_cast<const u32x4*>(Zs + (jt * 16 + li) * ZP + lg * 8);
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) {
        const u32x4 xf = xf4[mi];
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt)
          if (jt < KT) facc[mi][jt] = mfma16x16x32(zf[jt], xf, facc[mi][jt]);
      }
      // chunk c + S - 1 of the sequence into the slot chunk c - 1 left (every wave passed
      // this chunk's barrier, so none still reads it): this example's last chunk when
      // c == 0, else the next example's chunk c - 1.  Issued after this chunk's LDS
      // reads, which then need no wait for it.
      if (c == 0) dma_chunk(xslot(S - 1), b, S - 1);
      else dma_chunk(xslot(c - 1), b + stride, c - 1);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- end of the example: its LayerNorm statistics; the normalisation and the stores
    // run in the next example's first chunk (or after the loop)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // one pass: the sum and the sum of squares (fp32; the rows are O(1) LayerNorm inputs)
      float sm = 0.f, sq = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int et = 0; et < 2; ++et)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            sm += lc[i][c][et][t];
            sq += lc[i][c][et][t] * lc[i][c][et][t];
          }
      sm += __shfl_xor(sm, 16, kWave);
      sq += __shfl_xor(sq, 16, kWave);
      sm += __shfl_xor(sm, 32, kWave);
      sq += __shfl_xor(sq, 32, kWave);
      pmean[i] = sm * inv_d;
      prstd[i] = rsqrtf(fmaxf(sq * inv_d - pmean[i] * pmean[i], 0.f) + p.eps);
#pragma unroll
      for (int c = 0; c < NCH; ++c) plc[i][c][0] = lc[i][c][0], plc[i][c][1] = lc[i][c][1];
    }
    {  // the FMB LayerNorm over vec(F): each wave's sum and sum of squares (fp32)
      float sm = 0.f, sq = 0.f;
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (jt * 16 + lg * 4 + t < k) {
              sm += facc[mi][jt][t];
              sq += facc[mi][jt][t] * facc[mi][jt][t];
            }
      sm = group_sum_v<64>(sm);
      sq = group_sum_v<64>(sq);
      // (every wave read the previous example's sums in this example's first chunk,
      // before that chunk's second barrier)
      if (lane == 0) {
        red[wave] = sm;
        red[NW + wave] = sq;
      }
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
        for (int jt = 0; jt < KJ; ++jt) pfacc[mi][jt] = facc[mi][jt];
    }
    pb = b;
    live = true;
  }
  // the last example's output stage
  ring_barrier();  // its FMB sums
  {
    __amdgpu_buffer_rsrc_t ry, rfn;
    float fm_mean, fm_rstd;
    out_rsrc(ry, rfn);
    fm_stats(fm_mean, fm_rstd);
#pragma unroll
    for (int u = 0; u < UNITS; ++u) out_unit(u, ry, rfn, fm_mean, fm_rstd);
  }
  __builtin_amdgcn_s_waitcnt(vm_enc(0));  // the copies issued past the last example
}

// [Phi; W_L] in the ring's order: 16-byte chunk c = (t ZTP + i) 64 + l holds
// row 16 i + l / 4 of [Phi (padded to KZ tiles, or not at all when contig); W_L],
// columns 32 t + 8 (l % 4) .. + 7, zero outside the matrices and in the tiles past ZT.
__global__ __launch_bounds__(256) void pack_stream_weights_kernel(const uint16_t* __restrict__ phi,
                                                                  const uint16_t* __restrict__ w_l,
                                                                  uint16_t* __restrict__ out, int n, int k, int n_l,
                                                                  int kz, int zt, int ztp, int steps, int contig) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= steps * ztp * 64) return;
  const int l = c & 63, ti = c >> 6;
  const int i = ti % ztp, t = ti / ztp;
  const int r = 16 * i + (l >> 2), col = KC * t + 8 * (l & 3);
  const uint16_t* src = phi;
  int row = r, rows = k;
  if (contig ? r >= k : i >= kz) {
    src = w_l;
    row = contig ? r - k : r - 16 * kz;
    rows = i < zt ? n_l : 0;  // tiles past zt: zero padding
  }
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (row < rows && col + e < n) ? src[(int64_t)row * n + col + e] : (uint16_t)0;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
  *reinterpret_cast<u32x4*>(out + (int64_t)c * 8) = o;
}

struct StreamVariant {
  int et, zpw, wz, we, epw, mpw, kj, ztmax, s;
  bool contig;
  void (*kernel)(FmbLcbArgs, int64_t, StreamShape);
  void (*kernel_train)(FmbLcbArgs, int64_t, StreamShape);  // also stores Z and Lc
};

#define WK_STREAM(ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, GUARD, CONTIG)                       \
  StreamVariant {                                                                               \
    ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, CONTIG,                                            \
        fmb_lcb_stream_kernel<ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, GUARD, CONTIG, false>,   \
        fmb_lcb_stream_kernel<ET, ZPW, WZ, WE, EPW, MPW, KJ, ZTMAX, S, GUARD, CONTIG, true>     \
  }

// LDS per variant (static): S x (ZTMAX 16 KC + E KC D) + E KJ 16 ZP + 2 D u16.
const StreamVariant kStream[] = {
    WK_STREAM(10, 3, 4, 2, 1, 2, 3, 12, 3, false, false),  // n<=256, d=160, k<=48, ZT<=12: 2 examples per group
    WK_STREAM(10, 3, 8, 1, 1, 4, 6, 24, 3, false, false),  // n<=512, d=160, k<=96, ZT<=24
    // n<=768, d=32, k<=32, k+n_l<=384 (24 contiguous tiles, 3 per wave): 8 examples per group
    WK_STREAM(2, 3, 8, 1, 8, 6, 2, 24, 3, false, true),
    WK_STREAM(2, 4, 8, 1, 4, 6, 2, 25, 4, true, false),    // n<=768, d=32,  k<=32, ZT<=25: 4 examples per group
};

StreamShape stream_shape(const StreamVariant& v, int n, int k, int n_l) {
  StreamShape sh;
  sh.kz = v.contig ? 0 : (k + 15) / 16;
  sh.zt = v.contig ? (k + n_l + 15) / 16 : sh.kz + (n_l + 15) / 16;
  sh.steps = (n + KC - 1) / KC;
  sh.e = v.we * v.epw;
  sh.ztp = v.ztmax;
  return sh;
}

const StreamVariant* pick_stream(int n, int d, int k, int n_l, StreamShape* out) {
  if (d % 16 != 0) return nullptr;
  for (const auto& v : kStream) {
    if (16 * v.et != d) continue;
    const StreamShape sh = stream_shape(v, n, k, n_l);
    if (sh.zt > v.ztmax || sh.zt > v.wz * v.zpw) continue;  // DMA'd tiles and tiles with an owner wave
    if ((k + 15) / 16 > v.kj) continue;
    if ((n + 15) / 16 > NWAVE * v.mpw) continue;

    // 32-bit byte offsets within one group's X and within the weights
    if ((int64_t)sh.e * n * d * 2 >= (int64_t)1 << 31 || (int64_t)(k + n_l) * n * 2 >= (int64_t)1 << 31) continue;
    if (out) *out = sh;
    return &v;
  }
  return nullptr;
}

// The d-chunked kernel (weights in registers) serves the plain forward of the
// n = 256, d = 160 layer with n_l = 128 (8 full W_L tiles, two per wave) and
// k <= 48, k % 16 == 0 (at most 3 Phi tiles, whole ones), packed by the
// n <= 256 streamed variant (Phi padded to whole tiles).
bool dchunk_fits(const StreamVariant& v, const StreamShape& sh, int n, int d, int k, int n_l) {
  return n == 256 && d == 160 && n_l == 128 && k <= 48 && k % 16 == 0 && !v.contig && sh.kz == k / 16 &&
         sh.zt == sh.kz + 8 && sh.steps == 8 && sh.ztp >= sh.zt;
}

}  // namespace

bool fmb_lcb_stream_supported(int n, int d, int k, int n_l) { return pick_stream(n, d, k, n_l, nullptr) != nullptr; }

size_t fmb_lcb_stream_pack_bytes(int n, int d, int k, int n_l) {
  StreamShape sh;
  if (!pick_stream(n, d, k, n_l, &sh)) return 0;
  return (size_t)sh.steps * sh.ztp * 1024;
}

hipError_t launch_fmb_lcb_stream(const FmbLcbArgs& a, int64_t batch, hipStream_t stream, int64_t* workgroups) {
  StreamShape sh;
  const StreamVariant* v = pick_stream(a.n, a.d, a.k, a.n_l, &sh);
  if (!v) return hipErrorInvalidValue;
  const int64_t groups = (batch + sh.e - 1) / sh.e;
  const int64_t grid = groups < 256 ? groups : 256;
  if (workgroups) *workgroups = grid;
  if ((a.z_out == nullptr) != (a.lc_out == nullptr)) return hipErrorInvalidValue;
  if (a.wpack == nullptr || (reinterpret_cast<uintptr_t>(a.wpack) & 15) != 0) return hipErrorInvalidValue;
  if (batch == 0) return hipSuccess;
  const int chunks = sh.steps * sh.ztp * 64;
  hipLaunchKernelGGL(pack_stream_weights_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, a.phi,
                     a.w_l, a.wpack, a.n, a.k, a.n_l, sh.kz, sh.zt, sh.ztp, sh.steps, v->contig ? 1 : 0);
  if (a.z_out == nullptr && dchunk_fits(*v, sh, a.n, a.d, a.k, a.n_l)) {
    const int64_t g = batch < 256 ? batch : 256;
    if (workgroups) *workgroups = g;
    hipLaunchKernelGGL((fmb_lcb_dchunk_kernel<256, 160, 4, 3>), dim3((unsigned)g), dim3(256), 0, stream, a, batch,
                       sh);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(a.z_out ? v->kernel_train : v->kernel, dim3((unsigned)grid), dim3(NTHREAD), 0, stream, a, batch,
                     sh);
  return hipGetLastError();
}

}  // namespace wk
