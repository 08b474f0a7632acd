// Internal launcher interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wk {

// FMB + LCB (see fmb_lcb.hip / fmb_lcb_f32.hip).  Element type: uint16_t
// bf16 bits for the bf16 kernel, float for the fp32 kernel (void* here).
struct FmbLcbArgs {
  const uint16_t* x;         // [B, n, d]
  const uint16_t* phi;       // [k, n]
  const uint16_t* w_l;       // [n_l, n]
  const uint16_t* fm_gamma;  // [n*k] or null
  const uint16_t* fm_beta;   // [n*k] or null
  const uint16_t* out_gamma; // [d] or null
  const uint16_t* out_beta;  // [d] or null
  uint16_t* fn;              // [B, n*k]
  uint16_t* y;               // [B, n, d]: rows n_f..n-1 are written
  int n, d, k, n_f, n_l;
  float eps;
  // training forward of the wide layers (streamed kernel only; both or neither):
  uint16_t* z_out = nullptr;  // [B, k, d] Z = bf16(Phi X), as the interaction uses it
  float* lc_out = nullptr;    // [B, n_l, d] Lc = W_L X in fp32, as the LCB rows' LayerNorm uses it
  // scratch for [Phi; W_L] rearranged into the streamed kernel's 1 KB step tiles
  // (fmb_lcb_bf16_pack_bytes(); needed when that is non-zero)
  uint16_t* wpack = nullptr;
  // > 0 (streamed kernel only): Fn is written K-blocked, element (b, c) at
  // ((c / 64) fn_kblock_rows + b) 64 + c % 64, the first Linear's A operand in
  // the layout LinearArgs::a_kblock_rows describes
  int64_t fn_kblock_rows = 0;
};
// Whether launch_fmb_lcb_bf16 can write Fn K-blocked for this shape (the plain forward).
bool fmb_lcb_kblocked_fn_supported(int n, int d, int k, int n_l);
bool fmb_lcb_bf16_supported(int n, int d, int k, int n_l);
// Streamed variant (fmb_lcb_stream.hip): several examples per workgroup, the
// weights and X rows DMA'd through an LDS ring.  Used first when it supports
// the shape.
bool fmb_lcb_stream_supported(int n, int d, int k, int n_l);
hipError_t launch_fmb_lcb_stream(const FmbLcbArgs& a, int64_t batch, hipStream_t stream, int64_t* workgroups);
// Bytes of the rearranged weights the streamed kernel reads (0 when the shape takes another kernel).
size_t fmb_lcb_stream_pack_bytes(int n, int d, int k, int n_l);
// Scratch (FmbLcbArgs::wpack) launch_fmb_lcb_bf16 needs for this shape; train: the Z / Lc outputs are set.
size_t fmb_lcb_bf16_pack_bytes(int n, int d, int k, int n_l, bool train);
hipError_t launch_fmb_lcb_bf16(const FmbLcbArgs& a, int64_t batch, hipStream_t stream,
                               int64_t* workgroups);
// WHALE fusion step (whale_fusion.hip): shared K = V cross-attention followed
// by the Fusion MLP's Linear, writing Q = [H_w, A] W_f^T + b_f ([B, n, d] bf16),
// n % 16 == 0, d in {32, 64, 96, 128, 160}; and a row LayerNorm (d % 8 == 0,
// d <= 512).
bool whale_attention_supported(int n, int d, int L);
hipError_t launch_whale_attention(const void* hw, const void* hs, const void* w_f, const void* b_f, void* q,
                                  int64_t batch, int n, int d, int L, hipStream_t stream, int64_t* workgroups);
hipError_t launch_row_ln_bf16(const void* x, void* y, int64_t rows, int d, const void* gamma, const void* beta,
                              float eps, hipStream_t stream, int64_t* workgroups);
// The fusion step's FFN as one kernel: out = q + (silu(U) * U) w_down^T + b_down,
// U = LN_d(q; gamma, beta) w_up^T + b_up, rows of d (bf16; gamma, beta and the
// biases may be null).  d in {32, 64, 96, 128, 160}, d_ff % 32 == 0, d_ff <= 4096.
struct FusionFfnArgs {
  const void* q;       // [rows, d]: the FFN input and its residual
  const void* gamma;   // [d]
  const void* beta;    // [d]
  const void* w_up;    // [d_ff, d]
  const void* b_up;    // [d_ff]
  const void* w_down;  // [d, d_ff]
  const void* b_down;  // [d]
  void* out;           // [rows, d]
  int64_t rows;
  int d, d_ff;
  float eps;
};
bool fusion_ffn_supported(int d, int d_ff);
hipError_t launch_fusion_ffn(const FusionFfnArgs& a, hipStream_t stream, int64_t* workgroups);
// Units of width d = 8 (fmb_lcb_units.hip): transpose, one batched GEMM whose
// epilogue finishes the LCB rows, and an epilogue kernel for the FMB rows; needs
// fmb_lcb_units_workspace() bytes
// of scratch (16-byte aligned), n % 64 == 0, k % 4 == 0, k <= 32,
// (k + n_l) % 8 == 0.
// The units' batched product with the LCB rows finished in its epilogue
// (linear_bf16.hip): Z (fp32, [B][k][8]) and Y's LCB rows (rows n - n_l ..)
// from the transposed X; n % 64 == 0, k % 4 == 0, n_l % 4 == 0.
struct UnitsGemmArgs {
  const void* wcat;  // [k + n_l][n] bf16
  const void* xt;    // [B 8][n] bf16, xt[(b, e)][j] = X[b][j][e]
  const void* x;     // [B][n][8] bf16
  const void* out_gamma;
  const void* out_beta;
  float* z;
  void* y;
  int64_t batch;
  int n, k, n_l;
  float eps;
};
bool units_gemm_supported(int64_t batch, int n, int k, int n_l);
hipError_t launch_units_gemm(const UnitsGemmArgs& a, hipStream_t stream, int64_t* workgroups);
bool fmb_lcb_units_supported(int n, int d, int k, int n_l);
size_t fmb_lcb_units_workspace(int64_t batch, int n, int k, int n_l);
hipError_t launch_fmb_lcb_units(const FmbLcbArgs& a, int64_t batch, void* scratch, hipStream_t stream,
                                int64_t* workgroups);

struct FmbLcbF32Args {
  const float* x;
  const float* phi;
  const float* w_l;
  const float* fm_gamma;
  const float* fm_beta;
  const float* out_gamma;
  const float* out_beta;
  float* fn;
  float* y;
  int n, d, k, n_f, n_l;
  float eps;
};
bool fmb_lcb_f32_supported(int n, int d, int k, int n_l);
hipError_t launch_fmb_lcb_f32(const FmbLcbF32Args& a, int64_t batch, hipStream_t stream,
                              int64_t* workgroups);

// One FMB-MLP Linear: C[M, N] = act(A[M, K] W[N, K]^T + bias[N]).
// Activation applied after the bias: none, ReLU, or the shared-gate SwiGLU
// u * silu(u) (gate and up projection are one matrix).  bf16 kernels take
// all three; the fp32 kernel takes none and ReLU.
// kActReluMask is the ReLU's backward: no activation, and `res` is the
// forward activation whose non-positive entries zero the output.
enum LinearAct { kActNone = 0, kActRelu = 1, kActSiluGate = 2, kActReluMask = 3 };
struct LinearArgs {
  const void* a;
  const void* w;
  const void* bias;  // or null
  void* c;
  int64_t M;
  int N, K;
  int act;
  const void* res = nullptr;  // bf16 only: [M, N] added after the activation (the mask for kActReluMask), or null
  // bf16 launch_linear_bf16 only, K % 64 == 0: > 0 when A is K-blocked, element (m, c) at
  // ((c / 64) a_kblock_rows + m) 64 + c % 64 (a_kblock_rows: a multiple of 256, >= M)
  int64_t a_kblock_rows = 0;
};
bool linear_bf16_supported(int64_t M, int N, int K);
hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream, int64_t* workgroups);
hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t stream, int64_t* workgroups);
// Split-K form of the bf16 Linear for shapes whose tiles leave CUs idle:
// linear_bf16_splits() = number of K splits (1: use launch_linear_bf16),
// linear_bf16_split_bytes() = the fp32 partial-sum buffer it needs (0 if none);
// the launch runs the split GEMM and the reduction (bias, ReLU, bf16).
int linear_bf16_splits(int64_t M, int N, int K);
size_t linear_bf16_split_bytes(int64_t M, int N, int K);
hipError_t launch_linear_bf16_splitk(const LinearArgs& a, float* partial, hipStream_t stream, int64_t* workgroups);
// C = A W^T in fp32 (no bias, no activation), K % 64 == 0, N % 8 == 0.
bool linear_bf16_f32out_supported(int64_t M, int N, int K);
hipError_t launch_linear_bf16_f32out(const LinearArgs& a, float* c, hipStream_t stream, int64_t* workgroups);
// dX[b][m][e] = bf16(dXa[b][m][e] + C[m][b D + e]) for C = A W^T on 256 x 256 tiles
// (C's columns are (example, embedding) pairs; K % 64 == 0, D % 4 == 0, N % D == 0).
bool linear_bf16_dx_supported(int64_t M, int N, int K, int D);
hipError_t launch_linear_bf16_dx(const LinearArgs& a, const float* dxa, void* dx, int D, hipStream_t stream,
                                 int64_t* workgroups);
// The same with K split when the tiles leave CUs idle: the fp32 partials
// (linear_bf16_f32out_split_bytes(), 0 when unsplit) are summed in split order.
int linear_bf16_f32out_splits(int64_t M, int N, int K);
size_t linear_bf16_f32out_split_bytes(int64_t M, int N, int K);
hipError_t launch_linear_bf16_f32out_split(const LinearArgs& a, float* c, float* partial, hipStream_t stream,
                                           int64_t* workgroups);
// out[j] = sum over p = 0, 1, .. planes-1 of part[p * len + j], in that order (fp32).
hipError_t launch_sum_planes(const float* part, int planes, int64_t len, float* out, hipStream_t stream);
// out[j] = sum over p of part[p * stride + j], j < len <= stride.
hipError_t launch_sum_planes_strided(const float* part, int planes, int64_t stride, int64_t len, float* out,
                                     hipStream_t stream);
// Up to kMaxPlaneSegs such sums over the same number of planes in one launch;
// segments with a null out are skipped.  Each column adds planes q = s, s + 8, ..
// for slices s = 0 .. 7, then the slices in order (with at most 8 planes this is
// plane order).
struct PlaneSeg {
  const float* part;
  float* out;
  int64_t stride, len;
};
constexpr int kMaxPlaneSegs = 8;
hipError_t launch_sum_planes_multi(const PlaneSeg* segs, int nseg, int planes, hipStream_t stream,
                                   int64_t* workgroups);

// The last Linear with the FMB rows' output stage fused in (bf16):
// Y[b, r] = LN_d(bf16(A[b] W^T + bias)[r d .. r d + d) + X[b, r]) for r < n_f,
// with X and Y rows of example b at b * ld (ld = n * d).  N = n_f * d.
struct LinearLnArgs {
  const void* a;
  const void* w;
  const void* bias;   // or null
  const void* x;      // [B, n, d]
  const void* gamma;  // [d] or null
  const void* beta;   // [d] or null
  void* y;            // [B, n, d]: rows 0..n_f-1 are written
  int64_t M;
  int N, K, d;
  int64_t ld;
  float eps;
  void* m_out = nullptr;  // or [M, N]: also store M = bf16(A W^T + bias) (kept for the backward)
};
bool linear_ln_bf16_supported(int64_t M, int N, int K, int d);
hipError_t launch_linear_ln_bf16(const LinearLnArgs& a, hipStream_t stream, int64_t* workgroups);
// Up to kMaxLnGroup of them (same d, no m_out) as one launch: the tiles of all
// groups fill the GPU together (the experts of a mixture, each with few tiles).
constexpr int kMaxLnGroup = 4;
hipError_t launch_linear_ln_bf16_group(const LinearLnArgs* a, int n, hipStream_t stream, int64_t* workgroups);

// FMB rows of the layer output: Y[b, r] = LN_d(M[b, r] + X[b, r]) for r < n_f.
struct ResidLnArgs {
  const void* m;  // [B, n_f, d]
  const void* x;  // [B, n, d]
  const void* gamma;
  const void* beta;
  void* y;        // [B, n, d]
  int64_t batch;
  int n, d, n_f;
  float eps;
};
bool resid_ln_bf16_supported(int d);
hipError_t launch_resid_ln_bf16(const ResidLnArgs& a, hipStream_t stream, int64_t* workgroups);
hipError_t launch_resid_ln_f32(const ResidLnArgs& a, hipStream_t stream, int64_t* workgroups);

// Backward pass of one bf16 layer (wukong_backward.hip).  The per-example
// kernels need wukong_bwd_supported(n, d, k, n_l); each launches
// wukong_bwd_workgroups(batch) workgroups and writes one fp32 plane of weight
// gradient sums per workgroup into `part` (launch_sum_planes adds them).
bool wukong_bwd_supported(int n, int d, int k, int n_l);
int wukong_bwd_workgroups(int64_t batch);
size_t wukong_bwd_out_part_floats(int d);                   // [2 d]: sum dY R_hat, sum dY
size_t wukong_bwd_fmb_part_floats(int n, int k, int n_l);   // [k n + n_l n + 2 n k]
struct BwdOutArgs {
  const void* x;      // [B, n, d]
  const void* m;      // [B, n_f, d] the forward's M
  const void* dy;     // [B, n, d]
  const void* w_l;    // [n_l, n]
  const void* gamma;  // [d] output LayerNorm scale, or null
  void* dm;           // [B, n_f, d] out: dR rows < n_f
  void* dlc;          // [B, n_l, d] out: dR rows >= n_f
  float* part;        // [workgroups, 2 d]
  int64_t batch;
  int n, d, n_l;
  float eps;
};
hipError_t launch_bwd_out(const BwdOutArgs& a, hipStream_t stream, int64_t* workgroups);
struct BwdFmbArgs {
  const void* x;         // [B, n, d]
  const void* dfn;       // [B, n k] gradient of the normalised interaction
  const void* dm;        // [B, n_f, d]
  const void* dlc;       // [B, n_l, d]
  const void* phi;       // [k, n]
  const void* w_l;       // [n_l, n]
  const void* fm_gamma;  // [n k] or null
  void* dx;              // [B, n, d] out
  float* part;           // [workgroups, k n + n_l n + 2 n k]
  int64_t batch;
  int n, d, k, n_l;
  float eps;
};
hipError_t launch_bwd_fmb(const BwdFmbArgs& a, hipStream_t stream, int64_t* workgroups);
// Backward of the wide layers (wukong_backward_wide.hip): n of 256 .. 720 at
// d = 160 (k <= 64), 32 (k <= 32) or 64, with the per-example gradient
// matrix G = [dZ; dLc] kept batch-major ([k + n_l, ldg], example b's
// columns b d .. b d + d - 1) so the weight products run as GEMMs.
bool wukong_bwd_wide_supported(int n, int d, int k, int n_l);
struct BwdRowsArgs {
  const void* x;      // [B, n, d]
  const void* m;      // [B, n_f, d] the forward's M (bf16)
  const float* lc;    // [B, n_l, d] the forward's Lc (fp32)
  const void* dy;     // [B, n, d]
  const void* gamma;  // [d] or null
  void* dm;           // [B, n_f, d] out: dR rows < n_f
  void* g;            // out: dR rows >= n_f at rows k .. of G
  int64_t ldg;
  float* part;        // [workgroups, 2 d]: sum dY R_hat, sum dY
  int64_t batch;
  int n, d, k, n_f, n_l;
  float eps;
};
hipError_t launch_bwd_rows(const BwdRowsArgs& a, int grid, hipStream_t stream, int64_t* workgroups);
struct BwdFmWideArgs {
  const void* x;         // [B, n, d]
  const void* z;         // [B, k, d] the forward's Z (bf16)
  const void* dfn;       // [B, n k]
  const void* fm_gamma;  // [n k] or null
  const void* dm;        // [B, n_f, d] dR rows < n_f
  void* g;               // in: dR rows >= n_f at rows k .. of G; out: dZ at rows 0 .. k-1
  int64_t ldg;
  float* dxa;            // [B, n, d] out: dR + dF Z
  float* part;           // [workgroups, 2 n k]: sum d_Fn F_hat, sum d_Fn
  int64_t batch;
  int n, d, k, n_f;
  float eps;
};
hipError_t launch_bwd_fm_wide(const BwdFmWideArgs& a, int grid, hipStream_t stream, int64_t* workgroups);
// dst[r][b D + e] = src[b][r][e] for b < batch, zero for columns batch D .. ld - 1
hipError_t launch_to_batch_major(const void* src, int64_t batch, int R, int D, int64_t ld, void* dst,
                                 hipStream_t stream);
hipError_t launch_zero_cols(void* p, int R, int64_t ld, int64_t c0, hipStream_t stream);
// The fp32-output product split along K into as many as max_splits parts (summed in split order).
int linear_bf16_f32out_splits_max(int64_t M, int N, int K, int max_splits);
size_t linear_bf16_f32out_split_bytes_max(int64_t M, int N, int K, int max_splits);
hipError_t launch_linear_bf16_f32out_split_max(const LinearArgs& a, float* c, float* partial, int max_splits,
                                               hipStream_t stream, int64_t* workgroups);
// at[c][r] = a[r][c] (a: [R, C] bf16, C % 8 == 0), zero for R <= r < Rp
// (Rp % 8 == 0); colpart (or null) gets ceil(Rp / 64) planes of per-64-row
// column sums, [plane][C] fp32.
hipError_t launch_transpose_bf16(const void* a, int64_t R, int C, int64_t Rp, void* at, float* colpart,
                                 hipStream_t stream, int64_t* workgroups);

// The prediction head's last Linear + logistic function (head.hip):
// prob[m, o] = 1 / (1 + exp(-(A[m] . W[o] + bias[o]))), fp32 out.
struct HeadOutArgs {
  const void* a;     // [M, K] bf16 or fp32
  const void* w;     // [N, K]
  const void* bias;  // [N] or null
  float* prob;       // [M, N]
  int64_t M;
  int N, K;          // bf16: K % 8 == 0
};
hipError_t launch_head_out(const HeadOutArgs& a, bool bf16, hipStream_t stream, int64_t* workgroups);

}  // namespace wk
