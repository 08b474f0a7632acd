// C ABI of libwukong (declared in include/wukong.h): argument checks,
// workspace planning and the launch sequence of a Wukong layer and stack.
//
// Per layer (Wukong paper, section 2.2, xdnf.cn repost), on one stream:
//   1. FMB+LCB kernel: X -> Fn (workspace) and the LCB rows of Y
//   2. one MLP Linear per FMB-MLP layer: Fn -> h_1 -> ... -> M, bias + ReLU
//      fused, no ReLU after the last
//   3. rows 0..n_F-1 of Y = LayerNorm(M + X).  In bf16, when d divides 160
//      and the last Linear's K is a multiple of 64, this stage is the last
//      Linear's epilogue and M never leaves registers; otherwise M goes to
//      the workspace and a residual LayerNorm kernel follows.
// A stack (section 2.3: l layers) chains layers through two ping-pong
// buffers in the workspace; the last layer writes y.  No host sync anywhere.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <algorithm>
#include <vector>

#include "wk_kernels.h"
#include "wukong.h"

struct wk_trace {
  int device = 0;
  int capacity = 0;
  int count = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int32_t> kind, layer, index;
  std::vector<int64_t> wgs;
};

namespace {

constexpr int kMaxLinear = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t esize(int32_t dtype) { return dtype == WK_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return an > 0 && bn > 0 && x < y + bn && y < x + an;
}

// expert = true: one expert of a mixture-of-experts layer, whose FMB and LCB
// rows are a share of the layer's n output rows (n_f + n_l < n allowed).
int32_t check_desc(const wk_layer_desc* d, bool expert = false) {
  if (!d) return WK_ERR_INVALID_ARG;
  if (d->n <= 0 || d->d <= 0 || d->k <= 0 || d->n_f <= 0 || d->n_l <= 0) return WK_ERR_INVALID_ARG;
  if (d->num_linear < 1 || d->num_linear > kMaxLinear || !d->mlp_dims) return WK_ERR_INVALID_ARG;
  if (!(d->ln_eps >= 0.0f) || !std::isfinite(d->ln_eps)) return WK_ERR_INVALID_ARG;
  if (d->dtype != WK_F32 && d->dtype != WK_BF16) return WK_ERR_INVALID_ARG;
  for (int t = 0; t <= d->num_linear; ++t)
    if (d->mlp_dims[t] <= 0) return WK_ERR_INVALID_ARG;
  const int64_t nk = (int64_t)d->n * d->k, nfd = (int64_t)d->n_f * d->d;
  if (nk > INT32_MAX || nfd > INT32_MAX) return WK_ERR_INVALID_ARG;
  if (d->mlp_dims[0] != nk || d->mlp_dims[d->num_linear] != nfd) return WK_ERR_INVALID_ARG;
  // The residual adds X row by row, so the concatenation must have n rows.
  if (expert ? d->n_f + d->n_l > d->n : d->n_f + d->n_l != d->n) return WK_ERR_UNSUPPORTED;
  // the unit-width FMB+LCB step writes the LCB rows up to row n
  if (expert && d->dtype == WK_BF16 && d->d % 16 != 0) return WK_ERR_UNSUPPORTED;
  if (d->dtype == WK_BF16) {
    const bool units = wk::fmb_lcb_units_supported(d->n, d->d, d->k, d->n_l);
    if ((d->d % 16 && !units) || d->n % 8 || d->k % 4) return WK_ERR_UNSUPPORTED;
    for (int t = 0; t <= d->num_linear; ++t)
      if (d->mlp_dims[t] % 8) return WK_ERR_UNSUPPORTED;
    if (!units && !wk::fmb_lcb_bf16_supported(d->n, d->d, d->k, d->n_l)) return WK_ERR_UNSUPPORTED;
    if (!wk::resid_ln_bf16_supported(d->d)) return WK_ERR_UNSUPPORTED;
  } else {
    if (!wk::fmb_lcb_f32_supported(d->n, d->d, d->k, d->n_l)) return WK_ERR_UNSUPPORTED;
  }
  return WK_OK;
}

struct LayerPlan {
  size_t fn = 0, h[2] = {0, 0}, m = 0, units = 0, wpack = 0, bytes = 0;
  int64_t fn_kb = 0;  // > 0: Fn K-blocked with this many rows per 64-column block (first Linear's A)
  int num_hidden_bufs = 0;
  bool keep_hidden = false;  // h_{t+1} goes to hid[t] (the training forward keeps them all)
  size_t hid[kMaxLinear] = {};
  bool fused_out = false;  // last Linear writes the FMB rows of Y itself; no M buffer
  bool use_units = false;  // d = 8: the FMB+LCB step runs as transpose + batched GEMM + epilogue
  bool save_zl = false;    // training forward of a wide layer: the FMB+LCB step also keeps Z and Lc
  size_t z = 0, lc = 0;
};

// Units of width 8 (bf16) take the batched-GEMM form of the FMB+LCB step.
bool units_path(const wk_layer_desc& d) {
  return d.dtype == WK_BF16 && d.d % 16 != 0 && wk::fmb_lcb_units_supported(d.n, d.d, d.k, d.n_l);
}

// Whether the last Linear carries the residual LayerNorm in its epilogue.
bool fuse_output_ln(const wk_layer_desc& d) {
  return d.dtype == WK_BF16 &&
         wk::linear_ln_bf16_supported(1, d.mlp_dims[d.num_linear], d.mlp_dims[d.num_linear - 1], d.d);
}

// Largest batch the launch geometry handles (one workgroup per example in the
// FMB+LCB kernel; grid dimensions are 32-bit).
constexpr int64_t kMaxBatch = (int64_t)1 << 30;

// The plain bf16 forward writes Fn K-blocked when the streamed FMB+LCB kernel
// produces it and the first Linear (a plain GEMM) reads it with a long K: each
// of the GEMM's 64-column steps of A is then one contiguous run instead of rows
// n k x 2 bytes apart.
int64_t fn_kblock_rows(const wk_layer_desc& d, int64_t batch) {
  const int64_t nk = (int64_t)d.n * d.k;
  const int unfused = fuse_output_ln(d) ? d.num_linear - 1 : d.num_linear;
  if (d.dtype != WK_BF16 || units_path(d) || unfused < 1 || nk < 8192) return 0;
  if (!wk::fmb_lcb_kblocked_fn_supported(d.n, d.d, d.k, d.n_l)) return 0;
  const int64_t rows = (batch + 255) / 256 * 256;
  return rows * nk * 2 < ((int64_t)1 << 31) ? rows : 0;
}

LayerPlan plan_layer(const wk_layer_desc& d, int64_t batch) {
  LayerPlan p;
  const size_t es = esize(d.dtype);
  const size_t B = (size_t)batch;
  size_t off = 0;
  p.fn = off;
  p.fn_kb = fn_kblock_rows(d, batch);
  off += align_up((p.fn_kb ? (size_t)p.fn_kb : B) * d.n * d.k * es);
  int64_t maxhid = 0;
  for (int t = 1; t < d.num_linear; ++t) maxhid = d.mlp_dims[t] > maxhid ? d.mlp_dims[t] : maxhid;
  p.num_hidden_bufs = d.num_linear >= 3 ? 2 : (d.num_linear == 2 ? 1 : 0);
  for (int i = 0; i < p.num_hidden_bufs; ++i) {
    p.h[i] = off;
    off += align_up(B * (size_t)maxhid * es);
  }
  p.fused_out = fuse_output_ln(d);
  if (!p.fused_out) {
    p.m = off;
    off += align_up(B * (size_t)d.n_f * d.d * es);
  }
  p.use_units = units_path(d);
  if (p.use_units) {  // transposed X, [Phi; W_L], fp32 Z (dead once Fn and the LCB rows are written)
    p.units = off;
    off += align_up(wk::fmb_lcb_units_workspace(batch, d.n, d.k, d.n_l));
  }
  if (d.dtype == WK_BF16 && !p.use_units) {  // [Phi; W_L] in the streamed kernel's tile order
    const size_t pk = wk::fmb_lcb_bf16_pack_bytes(d.n, d.d, d.k, d.n_l, false);
    if (pk) {
      p.wpack = off;
      off += align_up(pk);
    }
  }
  p.bytes = off;
  return p;
}

int32_t check_weights(const wk_layer_desc& d, const wk_layer_weights* w) {
  if (!w || !w->phi || !w->w_l || !w->mlp_w) return WK_ERR_INVALID_ARG;
  const void* opt[] = {w->fm_ln_gamma, w->fm_ln_beta, w->out_ln_gamma, w->out_ln_beta};
  if (!aligned16(w->phi) || !aligned16(w->w_l)) return WK_ERR_INVALID_ARG;
  for (const void* p : opt)
    if (p && !aligned16(p)) return WK_ERR_INVALID_ARG;
  for (int t = 0; t < d.num_linear; ++t) {
    if (!w->mlp_w[t] || !aligned16(w->mlp_w[t])) return WK_ERR_INVALID_ARG;
    if (w->mlp_b && w->mlp_b[t] && !aligned16(w->mlp_b[t])) return WK_ERR_INVALID_ARG;
  }
  return WK_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? WK_OK : WK_ERR_HIP; }

struct Launch {
  wk_trace* trace;
  hipStream_t stream;
  template <class F>
  int32_t operator()(int kind, int layer, int index, F&& fn) {
    int64_t wgs = 0;
    if (trace && trace->count < trace->capacity) {
      const int i = trace->count;
      if (hipEventRecord(trace->start[i], stream) != hipSuccess) return WK_ERR_HIP;
      const hipError_t e = fn(&wgs);
      if (e != hipSuccess) return WK_ERR_HIP;
      if (hipEventRecord(trace->stop[i], stream) != hipSuccess) return WK_ERR_HIP;
      trace->kind[i] = kind;
      trace->layer[i] = layer;
      trace->index[i] = index;
      trace->wgs[i] = wgs;
      trace->count = i + 1;
      return WK_OK;
    }
    return hip_status(fn(&wgs));
  }
};

// Where a layer's output rows go: its FMB rows start at row fmb_row0 and its
// LCB rows at lcb_row0 of each example's n rows (the residual reads the same
// rows of X); the output LayerNorm's gamma / beta.  A plain layer has
// fmb_row0 = 0, lcb_row0 = n_f and its own gamma / beta; an expert of a
// mixture-of-experts layer has its share of the rows and the layer's.
struct RowMap {
  int fmb_row0, lcb_row0;
  const void* out_gamma;
  const void* out_beta;
};

// Launches one layer; all arguments already checked.
// With defer_last (fused last Linear only), the last Linear's arguments are
// returned there instead of launched (the mixture launches its experts' together).
int32_t run_layer(const wk_layer_desc& d, const wk_layer_weights& w, int64_t batch, const void* x,
                  void* y, char* scratch, const LayerPlan& plan, Launch& launch, int layer_idx,
                  const RowMap* rows = nullptr, wk::LinearLnArgs* defer_last = nullptr) {
  const bool bf = d.dtype == WK_BF16;
  char* fn = scratch + plan.fn;
  char* mbuf = scratch + plan.m;
  const RowMap rm = rows ? *rows : RowMap{0, d.n_f, w.out_ln_gamma, w.out_ln_beta};
  const size_t fmb_off = (size_t)rm.fmb_row0 * d.d * esize(d.dtype);
  const void* x_f = static_cast<const char*>(x) + fmb_off;
  void* y_f = static_cast<char*>(y) + fmb_off;
  int32_t st;
  if (bf) {
    wk::FmbLcbArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.phi = static_cast<const uint16_t*>(w.phi);
    a.w_l = static_cast<const uint16_t*>(w.w_l);
    a.fm_gamma = static_cast<const uint16_t*>(w.fm_ln_gamma);
    a.fm_beta = static_cast<const uint16_t*>(w.fm_ln_beta);
    a.out_gamma = static_cast<const uint16_t*>(rm.out_gamma);
    a.out_beta = static_cast<const uint16_t*>(rm.out_beta);
    a.fn = reinterpret_cast<uint16_t*>(fn);
    a.y = static_cast<uint16_t*>(y);
    if (plan.save_zl) {
      a.z_out = reinterpret_cast<uint16_t*>(scratch + plan.z);
      a.lc_out = reinterpret_cast<float*>(scratch + plan.lc);
    }
    if (plan.wpack) a.wpack = reinterpret_cast<uint16_t*>(scratch + plan.wpack);
    a.fn_kblock_rows = plan.fn_kb;
    a.n = d.n; a.d = d.d; a.k = d.k; a.n_f = rm.lcb_row0; a.n_l = d.n_l; a.eps = d.ln_eps;
    if (plan.use_units) {
      void* us = scratch + plan.units;
      st = launch(WK_KERNEL_FMB_LCB, layer_idx, 0,
                  [&](int64_t* g) { return wk::launch_fmb_lcb_units(a, batch, us, launch.stream, g); });
    } else {
      st = launch(WK_KERNEL_FMB_LCB, layer_idx, 0,
                  [&](int64_t* g) { return wk::launch_fmb_lcb_bf16(a, batch, launch.stream, g); });
    }
  } else {
    wk::FmbLcbF32Args a;
    a.x = static_cast<const float*>(x);
    a.phi = static_cast<const float*>(w.phi);
    a.w_l = static_cast<const float*>(w.w_l);
    a.fm_gamma = static_cast<const float*>(w.fm_ln_gamma);
    a.fm_beta = static_cast<const float*>(w.fm_ln_beta);
    a.out_gamma = static_cast<const float*>(rm.out_gamma);
    a.out_beta = static_cast<const float*>(rm.out_beta);
    a.fn = reinterpret_cast<float*>(fn);
    a.y = static_cast<float*>(y);
    a.n = d.n; a.d = d.d; a.k = d.k; a.n_f = rm.lcb_row0; a.n_l = d.n_l; a.eps = d.ln_eps;
    st = launch(WK_KERNEL_FMB_LCB, layer_idx, 0,
                [&](int64_t* g) { return wk::launch_fmb_lcb_f32(a, batch, launch.stream, g); });
  }
  if (st != WK_OK) return st;

  const void* in = fn;
  const int unfused = plan.fused_out ? d.num_linear - 1 : d.num_linear;
  for (int t = 0; t < unfused; ++t) {
    const bool last = t == d.num_linear - 1;
    void* out = last ? static_cast<void*>(mbuf)
                     : static_cast<void*>(scratch + (plan.keep_hidden ? plan.hid[t] : plan.h[t % 2]));
    wk::LinearArgs a;
    a.a = in;
    a.w = w.mlp_w[t];
    a.bias = w.mlp_b ? w.mlp_b[t] : nullptr;
    a.c = out;
    a.M = batch;
    a.N = d.mlp_dims[t + 1];
    a.K = d.mlp_dims[t];
    a.act = last ? wk::kActNone : wk::kActRelu;
    if (t == 0) a.a_kblock_rows = plan.fn_kb;
    st = launch(WK_KERNEL_MLP_LINEAR, layer_idx, t, [&](int64_t* g) {
      return bf ? wk::launch_linear_bf16(a, launch.stream, g) : wk::launch_linear_f32(a, launch.stream, g);
    });
    if (st != WK_OK) return st;
    in = out;
  }

  if (plan.fused_out) {
    const int t = d.num_linear - 1;
    wk::LinearLnArgs a;
    a.a = in;
    a.w = w.mlp_w[t];
    a.bias = w.mlp_b ? w.mlp_b[t] : nullptr;
    a.x = x_f;
    a.gamma = rm.out_gamma;
    a.beta = rm.out_beta;
    a.y = y_f;
    a.M = batch;
    a.N = d.mlp_dims[t + 1];
    a.K = d.mlp_dims[t];
    a.d = d.d;
    a.ld = (int64_t)d.n * d.d;
    a.eps = d.ln_eps;
    a.m_out = plan.keep_hidden ? static_cast<void*>(mbuf) : nullptr;  // the training forward keeps M
    if (defer_last) {
      *defer_last = a;
      return WK_OK;
    }
    return launch(WK_KERNEL_MLP_LINEAR, layer_idx, t,
                  [&](int64_t* g) { return wk::launch_linear_ln_bf16(a, launch.stream, g); });
  }

  wk::ResidLnArgs r;
  r.m = mbuf;
  r.x = x_f;
  r.gamma = rm.out_gamma;
  r.beta = rm.out_beta;
  r.y = y_f;
  r.batch = batch;
  r.n = d.n;
  r.d = d.d;
  r.n_f = d.n_f;
  r.eps = d.ln_eps;
  return launch(WK_KERNEL_RESIDUAL_LN, layer_idx, 0, [&](int64_t* g) {
    return bf ? wk::launch_resid_ln_bf16(r, launch.stream, g) : wk::launch_resid_ln_f32(r, launch.stream, g);
  });
}

struct StackPlan {
  size_t scratch_bytes = 0, ping[2] = {0, 0}, bytes = 0;
};

int32_t check_stack(int32_t l, const wk_layer_desc* descs, int64_t batch, StackPlan* sp) {
  if (l < 1 || !descs) return WK_ERR_INVALID_ARG;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  for (int i = 0; i < l; ++i) {
    const int32_t st = check_desc(&descs[i]);
    if (st != WK_OK) return st;
    if (descs[i].n != descs[0].n || descs[i].d != descs[0].d || descs[i].dtype != descs[0].dtype)
      return WK_ERR_INVALID_ARG;
  }
  StackPlan p;
  for (int i = 0; i < l; ++i) {
    const size_t b = plan_layer(descs[i], batch).bytes;
    p.scratch_bytes = b > p.scratch_bytes ? b : p.scratch_bytes;
  }
  const size_t act = align_up((size_t)batch * descs[0].n * descs[0].d * esize(descs[0].dtype));
  size_t off = p.scratch_bytes;
  const int nping = l >= 3 ? 2 : (l == 2 ? 1 : 0);
  for (int i = 0; i < nping; ++i) {
    p.ping[i] = off;
    off += act;
  }
  p.bytes = off;
  if (sp) *sp = p;
  return WK_OK;
}

int32_t stack_forward(int32_t l, const wk_layer_desc* descs, const wk_layer_weights* weights,
                      int64_t batch, const void* x, void* y, void* ws, size_t ws_bytes, void* stream,
                      wk_trace* trace) {
  StackPlan sp;
  int32_t st = check_stack(l, descs, batch, &sp);
  if (st != WK_OK) return st;
  if (!weights) return WK_ERR_INVALID_ARG;
  for (int i = 0; i < l; ++i) {
    st = check_weights(descs[i], &weights[i]);
    if (st != WK_OK) return st;
  }
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * descs[0].n * descs[0].d * esize(descs[0].dtype);
  if (!x || !y || !aligned16(x) || !aligned16(y)) return WK_ERR_INVALID_ARG;
  if (overlap(x, act, y, act)) return WK_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return WK_ERR_INVALID_ARG;
  if (ws_bytes < sp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(ws, sp.bytes, x, act) || overlap(ws, sp.bytes, y, act)) return WK_ERR_INVALID_ARG;

  char* base = static_cast<char*>(ws);
  Launch launch{trace, static_cast<hipStream_t>(stream)};
  for (int i = 0; i < l; ++i) {
    const void* in = i == 0 ? x : static_cast<const void*>(base + sp.ping[(i - 1) % 2]);
    void* out = i == l - 1 ? y : static_cast<void*>(base + sp.ping[i % 2]);
    const LayerPlan lp = plan_layer(descs[i], batch);
    st = run_layer(descs[i], weights[i], batch, in, out, base, lp, launch, i);
    if (st != WK_OK) return st;
  }
  return WK_OK;
}

// ---- prediction head (top MLP): hidden Linears on the MLP GEMMs (+ReLU), the
// last Linear + logistic function on the dot-product kernel.
int32_t check_head_desc(const wk_head_desc* d) {
  if (!d || d->num_linear < 1 || d->num_linear > kMaxLinear || !d->dims) return WK_ERR_INVALID_ARG;
  if (d->dtype != WK_F32 && d->dtype != WK_BF16) return WK_ERR_INVALID_ARG;
  for (int t = 0; t <= d->num_linear; ++t)
    if (d->dims[t] <= 0) return WK_ERR_INVALID_ARG;
  if (d->dtype == WK_BF16) {
    for (int t = 0; t < d->num_linear; ++t)
      if (d->dims[t] % 8) return WK_ERR_UNSUPPORTED;  // GEMM widths and the last Linear's 16-byte loads
  }
  return WK_OK;
}

struct HeadPlan {
  size_t h[2] = {0, 0}, part = 0, bytes = 0;
};

// Workspace: two ping-pong buffers of the widest hidden layer, then (bf16) the
// fp32 partial sums of the largest split-K hidden Linear.
HeadPlan plan_head(const wk_head_desc& d, int64_t batch) {
  HeadPlan p;
  int64_t maxhid = 0;
  size_t part = 0;
  for (int t = 1; t < d.num_linear; ++t) {
    maxhid = d.dims[t] > maxhid ? d.dims[t] : maxhid;
    if (d.dtype == WK_BF16) {
      const size_t pb = wk::linear_bf16_split_bytes(batch, d.dims[t], d.dims[t - 1]);
      part = pb > part ? pb : part;
    }
  }
  const size_t buf = align_up((size_t)batch * (size_t)maxhid * esize(d.dtype));
  p.h[0] = 0;
  p.h[1] = buf;
  p.part = d.num_linear > 1 ? 2 * buf : 0;
  p.bytes = p.part + align_up(part);
  if (p.bytes == 0) p.bytes = kAlign;
  return p;
}

int32_t head_forward(const wk_head_desc* d, const wk_head_weights* w, int64_t batch, const void* y, float* prob,
                     void* ws, size_t ws_bytes, void* stream, wk_trace* trace) {
  int32_t st = check_head_desc(d);
  if (st != WK_OK) return st;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  if (!w || !w->w) return WK_ERR_INVALID_ARG;
  const int T = d->num_linear;
  for (int t = 0; t < T; ++t) {
    if (!w->w[t] || !aligned16(w->w[t])) return WK_ERR_INVALID_ARG;
    if (w->b && w->b[t] && !aligned16(w->b[t])) return WK_ERR_INVALID_ARG;
  }
  if (batch == 0) return WK_OK;
  const HeadPlan hp = plan_head(*d, batch);
  const size_t es = esize(d->dtype);
  const size_t in_bytes = (size_t)batch * d->dims[0] * es;
  const size_t out_bytes = (size_t)batch * d->dims[T] * sizeof(float);
  if (!y || !prob || !aligned16(y) || (reinterpret_cast<uintptr_t>(prob) & 3u)) return WK_ERR_INVALID_ARG;
  if (overlap(y, in_bytes, prob, out_bytes)) return WK_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return WK_ERR_INVALID_ARG;
  if (ws_bytes < hp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(ws, hp.bytes, y, in_bytes) || overlap(ws, hp.bytes, prob, out_bytes)) return WK_ERR_INVALID_ARG;

  const bool bf = d->dtype == WK_BF16;
  char* base = static_cast<char*>(ws);
  Launch launch{trace, static_cast<hipStream_t>(stream)};
  const void* in = y;
  for (int t = 0; t + 1 < T; ++t) {
    void* out = base + hp.h[t % 2];
    wk::LinearArgs a;
    a.a = in;
    a.w = w->w[t];
    a.bias = w->b ? w->b[t] : nullptr;
    a.c = out;
    a.M = batch;
    a.N = d->dims[t + 1];
    a.K = d->dims[t];
    a.act = wk::kActRelu;
    const bool split = bf && wk::linear_bf16_splits(a.M, a.N, a.K) > 1;
    float* part = reinterpret_cast<float*>(base + hp.part);
    st = launch(WK_KERNEL_HEAD_LINEAR, 0, t, [&](int64_t* g) {
      if (split) return wk::launch_linear_bf16_splitk(a, part, launch.stream, g);
      return bf ? wk::launch_linear_bf16(a, launch.stream, g) : wk::launch_linear_f32(a, launch.stream, g);
    });
    if (st != WK_OK) return st;
    in = out;
  }
  wk::HeadOutArgs o;
  o.a = in;
  o.w = w->w[T - 1];
  o.bias = w->b ? w->b[T - 1] : nullptr;
  o.prob = prob;
  o.M = batch;
  o.N = d->dims[T];
  o.K = d->dims[T - 1];
  return launch(WK_KERNEL_HEAD_OUT, 0, 0, [&](int64_t* g) { return wk::launch_head_out(o, bf, launch.stream, g); });
}

// ---- WHALE fusion step: attention with the Fusion Linear in the same kernel, then the
// FFN as one kernel (or, for d_ff % 32 != 0, a row LayerNorm and two Linears on the MLP GEMMs).
int32_t check_fusion_desc(const wk_fusion_desc* d) {
  if (!d || d->n <= 0 || d->d <= 0 || d->L <= 0 || d->d_ff <= 0) return WK_ERR_INVALID_ARG;
  if (!(d->ln_eps >= 0.0f) || !std::isfinite(d->ln_eps)) return WK_ERR_INVALID_ARG;
  if (d->dtype != WK_F32 && d->dtype != WK_BF16) return WK_ERR_INVALID_ARG;
  if (d->dtype != WK_BF16) return WK_ERR_UNSUPPORTED;
  if (!wk::whale_attention_supported(d->n, d->d, d->L) || d->d_ff % 8) return WK_ERR_UNSUPPORTED;
  return WK_OK;
}

struct FusionPlan {
  size_t q = 0, qn = 0, g = 0, bytes = 0;
  bool fused_ffn = false;  // LayerNorm + FFN + residual as one kernel: no LN(Q) or G buffers
};

FusionPlan plan_fusion(const wk_fusion_desc& d, int64_t batch) {
  FusionPlan p;
  const size_t rows = (size_t)batch * d.n;
  p.fused_ffn = wk::fusion_ffn_supported(d.d, d.d_ff);
  p.q = 0;
  p.bytes = p.q + align_up(rows * d.d * 2);
  if (!p.fused_ffn) {
    p.qn = p.bytes;
    p.g = p.qn + align_up(rows * d.d * 2);
    p.bytes = p.g + align_up(rows * d.d_ff * 2);
  }
  if (p.bytes == 0) p.bytes = kAlign;
  return p;
}

int32_t fusion_forward(const wk_fusion_desc* d, const wk_fusion_weights* w, int64_t batch, const void* hw,
                       const void* hs, void* hf, void* ws, size_t ws_bytes, void* stream, wk_trace* trace) {
  int32_t st = check_fusion_desc(d);
  if (st != WK_OK) return st;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  if (!w || !w->w_f || !w->w_up || !w->w_down) return WK_ERR_INVALID_ARG;
  const void* ptrs[] = {w->w_f, w->b_f, w->ln_gamma, w->ln_beta, w->w_up, w->b_up, w->w_down, w->b_down};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return WK_ERR_INVALID_ARG;
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * d->n * d->d * 2, seq = (size_t)batch * d->L * d->d * 2;
  if (!hw || !hs || !hf || !aligned16(hw) || !aligned16(hs) || !aligned16(hf)) return WK_ERR_INVALID_ARG;
  if (overlap(hw, act, hf, act) || overlap(hs, seq, hf, act)) return WK_ERR_INVALID_ARG;
  const FusionPlan fp = plan_fusion(*d, batch);
  if (!ws || !aligned16(ws)) return WK_ERR_INVALID_ARG;
  if (ws_bytes < fp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(ws, fp.bytes, hw, act) || overlap(ws, fp.bytes, hs, seq) || overlap(ws, fp.bytes, hf, act))
    return WK_ERR_INVALID_ARG;

  char* base = static_cast<char*>(ws);
  void* q = base + fp.q;
  void* qn = base + fp.qn;
  void* g = base + fp.g;
  const int64_t rows = batch * d->n;
  Launch launch{trace, static_cast<hipStream_t>(stream)};
  st = launch(WK_KERNEL_FUSION_ATTN, 0, 0, [&](int64_t* wg) {
    return wk::launch_whale_attention(hw, hs, w->w_f, w->b_f, q, batch, d->n, d->d, d->L, launch.stream, wg);
  });
  if (st != WK_OK) return st;
  auto linear = [&](int index, const void* a, const void* wt, const void* bias, void* out, int N, int K, int act_kind,
                    const void* res) {
    wk::LinearArgs la;
    la.a = a;
    la.w = wt;
    la.bias = bias;
    la.c = out;
    la.M = rows;
    la.N = N;
    la.K = K;
    la.act = act_kind;
    la.res = res;
    return launch(WK_KERNEL_FUSION_LINEAR, 0, index,
                  [&](int64_t* wg) { return wk::launch_linear_bf16(la, launch.stream, wg); });
  };
  if (fp.fused_ffn) {
    wk::FusionFfnArgs fa;
    fa.q = q;
    fa.gamma = w->ln_gamma;
    fa.beta = w->ln_beta;
    fa.w_up = w->w_up;
    fa.b_up = w->b_up;
    fa.w_down = w->w_down;
    fa.b_down = w->b_down;
    fa.out = hf;
    fa.rows = rows;
    fa.d = d->d;
    fa.d_ff = d->d_ff;
    fa.eps = d->ln_eps;
    return launch(WK_KERNEL_FUSION_FFN, 0, 0,
                  [&](int64_t* wg) { return wk::launch_fusion_ffn(fa, launch.stream, wg); });
  }
  st = launch(WK_KERNEL_FUSION_LN, 0, 0, [&](int64_t* wg) {
    return wk::launch_row_ln_bf16(q, qn, rows, d->d, w->ln_gamma, w->ln_beta, d->ln_eps, launch.stream, wg);
  });
  if (st != WK_OK) return st;
  st = linear(1, qn, w->w_up, w->b_up, g, d->d_ff, d->d, wk::kActSiluGate, nullptr);
  if (st != WK_OK) return st;
  return linear(2, g, w->w_down, w->b_down, hf, d->d, d->d_ff, wk::kActNone, q);
}

// ---- mixture of experts: several Wukong modules in one layer, each writing
// its share of the output rows (FMB rows of every expert first, then LCB rows).
constexpr int kMaxExperts = 64;

// Whether the experts' last Linears run as grouped launches: all of them
// carry the output LayerNorm.  Each expert then keeps a workspace of its own
// (its last hidden activation lives until the grouped launch).
bool moe_grouped(const wk_moe_desc* m) {
  if (m->num_experts < 2) return false;
  for (int e = 0; e < m->num_experts; ++e)
    if (!fuse_output_ln(m->experts[e])) return false;
  return true;
}

int32_t check_moe(const wk_moe_desc* m, int64_t batch, size_t* bytes) {
  if (!m || !m->experts || m->num_experts < 1 || m->num_experts > kMaxExperts) return WK_ERR_INVALID_ARG;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  const wk_layer_desc& e0 = m->experts[0];
  int64_t rows = 0;
  size_t need = 0, sum = 0;
  for (int e = 0; e < m->num_experts; ++e) {
    const wk_layer_desc& d = m->experts[e];
    const int32_t st = check_desc(&d, true);
    if (st != WK_OK) return st;
    if (d.n != e0.n || d.d != e0.d || d.dtype != e0.dtype || d.ln_eps != e0.ln_eps) return WK_ERR_INVALID_ARG;
    rows += (int64_t)d.n_f + d.n_l;
    const size_t b = plan_layer(d, batch).bytes;
    need = b > need ? b : need;
    sum += align_up(b);
  }
  if (rows != e0.n) return WK_ERR_UNSUPPORTED;  // the residual needs n output rows
  if (moe_grouped(m)) need = sum;
  if (bytes) *bytes = need ? need : kAlign;
  return WK_OK;
}

int32_t moe_forward(const wk_moe_desc* m, const wk_layer_weights* weights, const void* out_gamma,
                    const void* out_beta, int64_t batch, const void* x, void* y, void* ws, size_t ws_bytes,
                    void* stream, wk_trace* trace) {
  size_t need = 0;
  int32_t st = check_moe(m, batch, &need);
  if (st != WK_OK) return st;
  if (!weights) return WK_ERR_INVALID_ARG;
  for (int e = 0; e < m->num_experts; ++e) {
    st = check_weights(m->experts[e], &weights[e]);
    if (st != WK_OK) return st;
  }
  if ((out_gamma && !aligned16(out_gamma)) || (out_beta && !aligned16(out_beta))) return WK_ERR_INVALID_ARG;
  if (batch == 0) return WK_OK;
  const wk_layer_desc& e0 = m->experts[0];
  const size_t act = (size_t)batch * e0.n * e0.d * esize(e0.dtype);
  if (!x || !y || !aligned16(x) || !aligned16(y)) return WK_ERR_INVALID_ARG;
  if (overlap(x, act, y, act)) return WK_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return WK_ERR_INVALID_ARG;
  if (ws_bytes < need) return WK_ERR_WORKSPACE;
  if (overlap(ws, need, x, act) || overlap(ws, need, y, act)) return WK_ERR_INVALID_ARG;
  int n_f_total = 0;
  for (int e = 0; e < m->num_experts; ++e) n_f_total += m->experts[e].n_f;
  Launch launch{trace, static_cast<hipStream_t>(stream)};
  const bool grouped = moe_grouped(m);
  std::vector<wk::LinearLnArgs> last(grouped ? m->num_experts : 0);
  int fmb_row = 0, lcb_row = n_f_total;
  size_t off = 0;
  for (int e = 0; e < m->num_experts; ++e) {
    const wk_layer_desc& d = m->experts[e];
    const RowMap rm{fmb_row, lcb_row, out_gamma, out_beta};
    const LayerPlan pl = plan_layer(d, batch);
    st = run_layer(d, weights[e], batch, x, y, static_cast<char*>(ws) + off, pl, launch, e, &rm,
                   grouped ? &last[e] : nullptr);
    if (st != WK_OK) return st;
    if (grouped) off += align_up(pl.bytes);
    fmb_row += d.n_f;
    lcb_row += d.n_l;
  }
  // the experts' last Linears (with the output LayerNorm of their FMB rows), kMaxLnGroup per
  // launch, recorded as layer num_experts
  for (int c0 = 0; c0 < (int)last.size(); c0 += wk::kMaxLnGroup) {
    const int cnt = std::min<int>(wk::kMaxLnGroup, (int)last.size() - c0);
    st = launch(WK_KERNEL_MLP_LINEAR, m->num_experts, c0 / wk::kMaxLnGroup, [&](int64_t* g) {
      return wk::launch_linear_ln_bf16_group(last.data() + c0, cnt, launch.stream, g);
    });
    if (st != WK_OK) return st;
  }
  return WK_OK;
}

// ---- backward of one bf16 layer.
// Wide layers (n of 256 .. 720) take the backward of wukong_backward_wide.hip,
// whose training forward also keeps Z and Lc (streamed FMB+LCB kernel).
bool wide_backward(const wk_layer_desc& d) {
  return !wk::wukong_bwd_supported(d.n, d.d, d.k, d.n_l) && wk::wukong_bwd_wide_supported(d.n, d.d, d.k, d.n_l) &&
         wk::fmb_lcb_stream_supported(d.n, d.d, d.k, d.n_l);
}

int32_t check_backward_desc(const wk_layer_desc* d) {
  const int32_t st = check_desc(d);
  if (st != WK_OK) return st;
  if (d->dtype != WK_BF16) return WK_ERR_UNSUPPORTED;
  if (!wk::wukong_bwd_supported(d->n, d->d, d->k, d->n_l) && !wide_backward(*d)) return WK_ERR_UNSUPPORTED;
  return WK_OK;
}

// Saved activations of the training forward: Fn, h_1 .. h_{T-1}, M (and for a
// wide layer Z in bf16 and Lc in fp32).
LayerPlan plan_saved(const wk_layer_desc& d, int64_t batch) {
  LayerPlan p;
  const size_t B = (size_t)batch;
  size_t off = 0;
  p.fn = off;
  off += align_up(B * d.n * d.k * 2);
  p.keep_hidden = true;
  for (int t = 0; t + 1 < d.num_linear; ++t) {
    p.hid[t] = off;
    off += align_up(B * (size_t)d.mlp_dims[t + 1] * 2);
  }
  p.m = off;
  off += align_up(B * (size_t)d.n_f * d.d * 2);
  if (wide_backward(d)) {
    p.save_zl = true;
    p.z = off;
    off += align_up(B * (size_t)d.k * d.d * 2);
    p.lc = off;
    off += align_up(B * (size_t)d.n_l * d.d * 4);
  }
  if (const size_t pk = wk::fmb_lcb_bf16_pack_bytes(d.n, d.d, d.k, d.n_l, p.save_zl)) {
    p.wpack = off;  // scratch of the FMB+LCB step (rearranged [Phi; W_L]), not a saved activation
    off += align_up(pk);
  }
  p.bytes = off;
  p.fused_out = fuse_output_ln(d);  // the fused last Linear stores M for the backward as well
  return p;
}

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }

struct BackwardPlan {
  size_t dm = 0, dlc = 0, g[2] = {0, 0}, dfn = 0, gt = 0, at = 0, wt = 0, colpart = 0, split = 0, part_out = 0,
         part_fmb = 0, bytes = 0;
  // wide layers: G = [dZ; dLc] batch-major [kc, ldg], its transpose [ldg, kcp], X batch-major
  // [n, ldg], [Phi; W_L] and its transpose, dR + dF Z (fp32), split partials
  bool wide = false;
  int64_t ldg = 0;
  int kc = 0, kcp = 0;
  size_t gm = 0, gmt = 0, xb = 0, wcat = 0, wcatt = 0, dxa = 0, wsplit = 0;
};
constexpr int kWideWgradSplits = 256;

BackwardPlan plan_backward(const wk_layer_desc& d, int64_t batch) {
  BackwardPlan p;
  const size_t B = (size_t)batch, Bp = (size_t)pad64(batch);
  const int T = d.num_linear;
  size_t maxhid = 0, maxw = 0, maxsplit = 0, maxdim = 0;
  for (int t = 0; t < T; ++t) {
    const size_t mi = (size_t)d.mlp_dims[t], mo = (size_t)d.mlp_dims[t + 1];
    if (t > 0) maxhid = mi > maxhid ? mi : maxhid;
    maxw = mi * mo > maxw ? mi * mo : maxw;
    maxdim = mi > maxdim ? mi : maxdim;
    maxdim = mo > maxdim ? mo : maxdim;
    const size_t sb = wk::linear_bf16_f32out_split_bytes((int64_t)mo, (int)mi, (int64_t)Bp);
    maxsplit = sb > maxsplit ? sb : maxsplit;
  }
  const size_t wg = (size_t)wk::wukong_bwd_workgroups(batch);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p.dm = take(B * d.n_f * d.d * 2);
  if (!wide_backward(d)) p.dlc = take(B * d.n_l * d.d * 2);  // a wide layer keeps dLc in G
  p.g[0] = take(B * maxhid * 2);
  p.g[1] = take(B * maxhid * 2);
  p.dfn = take(B * d.n * d.k * 2);
  p.gt = take(maxdim * Bp * 2);
  p.at = take(maxdim * Bp * 2);
  p.wt = take(maxw * 2);
  p.colpart = take((Bp / 64) * maxdim * 4);
  p.split = take(maxsplit);
  p.part_out = take(wg * wk::wukong_bwd_out_part_floats(d.d) * 4);
  if (wide_backward(d)) {
    p.wide = true;
    p.ldg = (int64_t)(B * d.d + 63) / 64 * 64;
    p.kc = d.k + d.n_l;
    p.kcp = (p.kc + 63) / 64 * 64;
    const size_t L = (size_t)p.ldg;
    p.part_fmb = take(wg * 2 * (size_t)d.n * d.k * 4);
    p.gm = take((size_t)p.kc * L * 2);
    p.gmt = take(L * p.kcp * 2);
    p.xb = take((size_t)d.n * L * 2);
    p.wcat = take((size_t)p.kc * d.n * 2);
    p.wcatt = take((size_t)d.n * p.kcp * 2);
    p.dxa = take(B * d.n * d.d * 4);
    const size_t s1 = wk::linear_bf16_f32out_split_bytes_max(d.k, d.n, (int)p.ldg, kWideWgradSplits);
    const size_t s2 = wk::linear_bf16_f32out_split_bytes_max(d.n_l, d.n, (int)p.ldg, kWideWgradSplits);
    p.wsplit = take(s1 > s2 ? s1 : s2);
  } else {
    p.part_fmb = take(wg * wk::wukong_bwd_fmb_part_floats(d.n, d.k, d.n_l) * 4);
  }
  p.bytes = off;
  return p;
}

int32_t layer_forward_train(const wk_layer_desc* d, const wk_layer_weights* w, int64_t batch, const void* x, void* y,
                            void* saved, size_t saved_bytes, void* stream) {
  int32_t st = check_backward_desc(d);
  if (st != WK_OK) return st;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  st = check_weights(*d, w);
  if (st != WK_OK) return st;
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * d->n * d->d * 2;
  const LayerPlan sp = plan_saved(*d, batch);
  if (!x || !y || !saved || !aligned16(x) || !aligned16(y) || !aligned16(saved)) return WK_ERR_INVALID_ARG;
  if (saved_bytes < sp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(x, act, y, act) || overlap(saved, sp.bytes, x, act) || overlap(saved, sp.bytes, y, act))
    return WK_ERR_INVALID_ARG;
  Launch launch{nullptr, static_cast<hipStream_t>(stream)};
  return run_layer(*d, *w, batch, x, y, static_cast<char*>(saved), sp, launch, 0);
}

// Backward of a wide layer (wukong_backward_wide.hip): output rows, the MLP,
// the FM part per example, then the products with [Phi; W_L] as GEMMs over the
// batch-major gradient matrix G = [dZ; dLc].
template <class MlpBackward>
int32_t layer_backward_wide(const wk_layer_desc* d, const wk_layer_weights* w, int64_t batch, const void* x,
                            const char* sbase, const LayerPlan& sv, const void* dy, void* dx, const wk_layer_grads* gr,
                            char* base, const BackwardPlan& bp, Launch& launch, int layer_idx, MlpBackward& mlp_backward) {
  hipStream_t s = launch.stream;
  const int T = d->num_linear;
  const int wg = wk::wukong_bwd_workgroups(batch);
  const int64_t L = bp.ldg;
  const int n = d->n, D = d->d, k = d->k;
  void* G = base + bp.gm;
  float* part_out = reinterpret_cast<float*>(base + bp.part_out);
  float* part_fm = reinterpret_cast<float*>(base + bp.part_fmb);
  int32_t st;
  if (L > batch * D) {  // the padding columns of G take part in the weight products: zero
    st = hip_status(wk::launch_zero_cols(G, bp.kc, L, batch * D, s));
    if (st != WK_OK) return st;
  }
  wk::BwdRowsArgs ra;
  ra.x = x;
  ra.m = sbase + sv.m;
  ra.lc = reinterpret_cast<const float*>(sbase + sv.lc);
  ra.dy = dy;
  ra.gamma = w->out_ln_gamma;
  ra.dm = base + bp.dm;
  ra.g = G;
  ra.ldg = L;
  ra.part = part_out;
  ra.batch = batch;
  ra.n = n;
  ra.d = D;
  ra.k = k;
  ra.n_f = d->n_f;
  ra.n_l = d->n_l;
  ra.eps = d->ln_eps;
  st = launch(WK_KERNEL_BWD_OUT, layer_idx, 0, [&](int64_t* g) { return wk::launch_bwd_rows(ra, wg, s, g); });
  if (st != WK_OK) return st;
  st = mlp_backward();
  if (st != WK_OK) return st;
  wk::BwdFmWideArgs fa;
  fa.x = x;
  fa.z = sbase + sv.z;
  fa.dfn = base + bp.dfn;
  fa.fm_gamma = w->fm_ln_gamma;
  fa.dm = base + bp.dm;
  fa.g = G;
  fa.ldg = L;
  fa.dxa = reinterpret_cast<float*>(base + bp.dxa);
  fa.part = part_fm;
  fa.batch = batch;
  fa.n = n;
  fa.d = D;
  fa.k = k;
  fa.n_f = d->n_f;
  fa.eps = d->ln_eps;
  st = launch(WK_KERNEL_BWD_FMB, layer_idx, 0, [&](int64_t* g) { return wk::launch_bwd_fm_wide(fa, wg, s, g); });
  if (st != WK_OK) return st;
  // X batch-major, then d[Phi; W_L] = G X'^T split along the batch
  void* xb = base + bp.xb;
  st = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * T, [&](int64_t* g) {
    *g = 1;
    return wk::launch_to_batch_major(x, batch, n, D, L, xb, s);
  });
  if (st != WK_OK) return st;
  float* wsplit = reinterpret_cast<float*>(base + bp.wsplit);
  for (int part = 0; part < 2; ++part) {
    wk::LinearArgs wa;
    wa.a = static_cast<char*>(G) + (part ? (size_t)k * L * 2 : 0);
    wa.w = xb;
    wa.bias = nullptr;
    wa.c = nullptr;
    wa.M = part ? d->n_l : k;
    wa.N = n;
    wa.K = (int)L;
    wa.act = wk::kActNone;
    float* out = part ? gr->w_l : gr->phi;
    st = launch(WK_KERNEL_BWD_WGRAD, layer_idx, T + part, [&](int64_t* g) {
      return wk::launch_linear_bf16_f32out_split_max(wa, out, wsplit, kWideWgradSplits, s, g);
    });
    if (st != WK_OK) return st;
  }
  // C = [Phi; W_L]^T G (batch-major, fp32), then dX = bf16(dR + dF Z + C)
  void* wcat = base + bp.wcat;
  void* wcatt = base + bp.wcatt;
  void* gmt = base + bp.gmt;
  if (hipMemcpyAsync(wcat, w->phi, (size_t)k * n * 2, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(static_cast<char*>(wcat) + (size_t)k * n * 2, w->w_l, (size_t)d->n_l * n * 2,
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    return WK_ERR_HIP;
  st = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * T + 1, [&](int64_t* g) {
    return wk::launch_transpose_bf16(wcat, bp.kc, n, bp.kcp, wcatt, nullptr, s, g);
  });
  if (st != WK_OK) return st;
  st = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * T + 2, [&](int64_t* g) {
    return wk::launch_transpose_bf16(G, bp.kc, (int)L, bp.kcp, gmt, nullptr, s, g);
  });
  if (st != WK_OK) return st;
  wk::LinearArgs ca;
  ca.a = wcatt;
  ca.w = gmt;
  ca.bias = nullptr;
  ca.c = nullptr;
  ca.M = n;
  ca.N = (int)L;
  ca.K = bp.kcp;
  ca.act = wk::kActNone;
  // dX = bf16(dR + dF Z + [Phi; W_L]^T G): the product's epilogue adds the fp32 sum
  // of the other terms and stores dX (its columns past B d, the padding of G, are dropped)
  ca.N = (int)(batch * D);
  st = launch(WK_KERNEL_BWD_DGRAD, layer_idx, T, [&](int64_t* g) {
    return wk::launch_linear_bf16_dx(ca, reinterpret_cast<const float*>(base + bp.dxa), dx, D, s, g);
  });
  if (st != WK_OK) return st;
  const int64_t nk = (int64_t)n * k;
  const wk::PlaneSeg segs[4] = {{part_out, gr->out_ln_gamma, 2 * D, D},
                                {part_out + D, gr->out_ln_beta, 2 * D, D},
                                {part_fm, gr->fm_ln_gamma, 2 * nk, nk},
                                {part_fm + nk, gr->fm_ln_beta, 2 * nk, nk}};
  return launch(WK_KERNEL_BWD_REDUCE, layer_idx, 0,
                [&](int64_t* g) { return wk::launch_sum_planes_multi(segs, 4, wg, s, g); });
}

int32_t layer_backward(const wk_layer_desc* d, const wk_layer_weights* w, int64_t batch, const void* x,
                       const void* saved, const void* dy, void* dx, const wk_layer_grads* gr, void* ws,
                       size_t ws_bytes, void* stream, wk_trace* trace, int layer_idx = 0) {
  int32_t st = check_backward_desc(d);
  if (st != WK_OK) return st;
  if (batch < 0 || batch > kMaxBatch) return WK_ERR_INVALID_ARG;
  st = check_weights(*d, w);
  if (st != WK_OK) return st;
  const int T = d->num_linear;
  if (!gr || !gr->phi || !gr->w_l || !gr->mlp_w) return WK_ERR_INVALID_ARG;
  for (int t = 0; t < T; ++t)
    if (!gr->mlp_w[t]) return WK_ERR_INVALID_ARG;
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * d->n * d->d * 2;
  const LayerPlan sv = plan_saved(*d, batch);
  const BackwardPlan bp = plan_backward(*d, batch);
  if (bp.wide && bp.ldg > INT32_MAX) return WK_ERR_UNSUPPORTED;  // GEMM K and N are 32-bit
  if (!x || !saved || !dy || !dx) return WK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(saved) || !aligned16(dy) || !aligned16(dx)) return WK_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return WK_ERR_INVALID_ARG;
  if (ws_bytes < bp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(dx, act, x, act) || overlap(dx, act, dy, act) || overlap(dx, act, saved, sv.bytes) ||
      overlap(dx, act, ws, bp.bytes) || overlap(ws, bp.bytes, x, act) || overlap(ws, bp.bytes, dy, act) ||
      overlap(ws, bp.bytes, saved, sv.bytes))
    return WK_ERR_INVALID_ARG;

  char* base = static_cast<char*>(ws);
  const char* sbase = static_cast<const char*>(saved);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Launch launch{trace, s};
  const int64_t Bp = pad64(batch);
  const int wg = wk::wukong_bwd_workgroups(batch);
  void* dm = base + bp.dm;
  void* dlc = base + bp.dlc;
  float* part_out = reinterpret_cast<float*>(base + bp.part_out);
  float* part_fmb = reinterpret_cast<float*>(base + bp.part_fmb);
  const int64_t po = (int64_t)wk::wukong_bwd_out_part_floats(d->d);  // summed with the FMB planes at the end

  // MLP, last Linear first: g_{t+1} -> dW_t, db_t, g_t; the first g is dM, the last d_Fn
  auto mlp_backward = [&]() -> int32_t {
    const void* g_next = dm;
    void* gt = base + bp.gt;
    void* at = base + bp.at;
    void* wt = base + bp.wt;
    float* colpart = reinterpret_cast<float*>(base + bp.colpart);
    float* split = reinterpret_cast<float*>(base + bp.split);
    for (int t = T - 1; t >= 0; --t) {
      const int mi = d->mlp_dims[t], mo = d->mlp_dims[t + 1];
      const void* a_t =
          t == 0 ? static_cast<const void*>(sbase + sv.fn) : static_cast<const void*>(sbase + sv.hid[t - 1]);
      float* db = gr->mlp_b ? gr->mlp_b[t] : nullptr;
      int32_t r = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * t, [&](int64_t* g) {
        return wk::launch_transpose_bf16(g_next, batch, mo, Bp, gt, db ? colpart : nullptr, s, g);
      });
      if (r != WK_OK) return r;
      if (db) {
        r = launch(WK_KERNEL_BWD_REDUCE, layer_idx, 2 + t, [&](int64_t* g) {
          *g = 1;
          return wk::launch_sum_planes(colpart, (int)(Bp / 64), mo, db, s);
        });
        if (r != WK_OK) return r;
      }
      r = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * t + 1, [&](int64_t* g) {
        return wk::launch_transpose_bf16(a_t, batch, mi, Bp, at, nullptr, s, g);
      });
      if (r != WK_OK) return r;
      wk::LinearArgs wa;
      wa.a = gt;
      wa.w = at;
      wa.bias = nullptr;
      wa.c = nullptr;
      wa.M = mo;
      wa.N = mi;
      wa.K = (int)Bp;
      wa.act = wk::kActNone;
      r = launch(WK_KERNEL_BWD_WGRAD, layer_idx, t, [&](int64_t* g) {
        return wk::launch_linear_bf16_f32out_split(wa, gr->mlp_w[t], split, s, g);
      });
      if (r != WK_OK) return r;
      r = launch(WK_KERNEL_BWD_TRANSPOSE, layer_idx, 3 * t + 2, [&](int64_t* g) {
        return wk::launch_transpose_bf16(w->mlp_w[t], mo, mi, mo, wt, nullptr, s, g);
      });
      if (r != WK_OK) return r;
      void* g_out = t == 0 ? static_cast<void*>(base + bp.dfn) : static_cast<void*>(base + bp.g[t % 2]);
      wk::LinearArgs da;
      da.a = g_next;
      da.w = wt;
      da.bias = nullptr;
      da.c = g_out;
      da.M = batch;
      da.N = mi;
      da.K = mo;
      da.act = t == 0 ? wk::kActNone : wk::kActReluMask;
      da.res = t == 0 ? nullptr : a_t;
      r = launch(WK_KERNEL_BWD_DGRAD, layer_idx, t, [&](int64_t* g) { return wk::launch_linear_bf16(da, s, g); });
      if (r != WK_OK) return r;
      g_next = g_out;
    }
    return WK_OK;
  };

  if (bp.wide) return layer_backward_wide(d, w, batch, x, sbase, sv, dy, dx, gr, base, bp, launch, layer_idx,
                                          mlp_backward);

  // output LayerNorm + LCB rows: dR -> dM, dLc
  wk::BwdOutArgs oa;
  oa.x = x;
  oa.m = sbase + sv.m;
  oa.dy = dy;
  oa.w_l = w->w_l;
  oa.gamma = w->out_ln_gamma;
  oa.dm = dm;
  oa.dlc = dlc;
  oa.part = part_out;
  oa.batch = batch;
  oa.n = d->n;
  oa.d = d->d;
  oa.n_l = d->n_l;
  oa.eps = d->ln_eps;
  st = launch(WK_KERNEL_BWD_OUT, layer_idx, 0, [&](int64_t* g) { return wk::launch_bwd_out(oa, s, g); });
  if (st != WK_OK) return st;
  st = mlp_backward();
  if (st != WK_OK) return st;

  // FM LayerNorm, interaction, compression: dX and the FMB / LCB weight sums
  wk::BwdFmbArgs fa;
  fa.x = x;
  fa.dfn = base + bp.dfn;
  fa.dm = dm;
  fa.dlc = dlc;
  fa.phi = w->phi;
  fa.w_l = w->w_l;
  fa.fm_gamma = w->fm_ln_gamma;
  fa.dx = dx;
  fa.part = part_fmb;
  fa.batch = batch;
  fa.n = d->n;
  fa.d = d->d;
  fa.k = d->k;
  fa.n_l = d->n_l;
  fa.eps = d->ln_eps;
  st = launch(WK_KERNEL_BWD_FMB, layer_idx, 0, [&](int64_t* g) { return wk::launch_bwd_fmb(fa, s, g); });
  if (st != WK_OK) return st;
  // the output LayerNorm's gamma / beta and the FMB / LCB weight gradients: one launch of plane sums
  const int64_t pf = (int64_t)wk::wukong_bwd_fmb_part_floats(d->n, d->k, d->n_l);
  const int64_t kn = (int64_t)d->k * d->n, ln = (int64_t)d->n_l * d->n, nk = (int64_t)d->n * d->k;
  const wk::PlaneSeg segs[6] = {{part_out, gr->out_ln_gamma, po, d->d},
                                {part_out + d->d, gr->out_ln_beta, po, d->d},
                                {part_fmb, gr->phi, pf, kn},
                                {part_fmb + kn, gr->w_l, pf, ln},
                                {part_fmb + kn + ln, gr->fm_ln_gamma, pf, nk},
                                {part_fmb + kn + ln + nk, gr->fm_ln_beta, pf, nk}};
  return launch(WK_KERNEL_BWD_REDUCE, layer_idx, 0,
                [&](int64_t* g) { return wk::launch_sum_planes_multi(segs, 6, wg, s, g); });
}

// ---- training a stack: per layer, its input (layers after the first) and its
// saved activations; the backward runs the layers last to first.
struct StackTrainPlan {
  std::vector<size_t> in, sv;
  size_t bytes = 0;
};

int32_t check_stack_train(int32_t l, const wk_layer_desc* descs, int64_t batch, StackTrainPlan* out,
                          size_t* bwd_bytes) {
  int32_t st = check_stack(l, descs, batch, nullptr);
  if (st != WK_OK) return st;
  for (int i = 0; i < l; ++i) {
    st = check_backward_desc(&descs[i]);
    if (st != WK_OK) return st;
  }
  const size_t act = align_up((size_t)batch * descs[0].n * descs[0].d * 2);
  StackTrainPlan p;
  size_t off = 0, bw = 0;
  for (int i = 0; i < l; ++i) {
    p.in.push_back(off);
    if (i > 0) off += act;
    p.sv.push_back(off);
    off += plan_saved(descs[i], batch).bytes;
    const size_t b = plan_backward(descs[i], batch).bytes;
    bw = b > bw ? b : bw;
  }
  p.bytes = off ? off : kAlign;
  if (out) *out = p;
  if (bwd_bytes) *bwd_bytes = 2 * act + bw;  // two gradient ping-pong buffers, then one layer's workspace
  return WK_OK;
}

int32_t stack_forward_train(int32_t l, const wk_layer_desc* descs, const wk_layer_weights* weights, int64_t batch,
                            const void* x, void* y, void* saved, size_t saved_bytes, void* stream) {
  StackTrainPlan sp;
  int32_t st = check_stack_train(l, descs, batch, &sp, nullptr);
  if (st != WK_OK) return st;
  if (!weights) return WK_ERR_INVALID_ARG;
  for (int i = 0; i < l; ++i) {
    st = check_weights(descs[i], &weights[i]);
    if (st != WK_OK) return st;
  }
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * descs[0].n * descs[0].d * 2;
  if (!x || !y || !saved || !aligned16(x) || !aligned16(y) || !aligned16(saved)) return WK_ERR_INVALID_ARG;
  if (saved_bytes < sp.bytes) return WK_ERR_WORKSPACE;
  if (overlap(x, act, y, act) || overlap(saved, sp.bytes, x, act) || overlap(saved, sp.bytes, y, act))
    return WK_ERR_INVALID_ARG;
  char* base = static_cast<char*>(saved);
  Launch launch{nullptr, static_cast<hipStream_t>(stream)};
  for (int i = 0; i < l; ++i) {
    const void* in = i == 0 ? x : static_cast<const void*>(base + sp.in[i]);
    void* out = i == l - 1 ? y : static_cast<void*>(base + sp.in[i + 1]);
    st = run_layer(descs[i], weights[i], batch, in, out, base + sp.sv[i], plan_saved(descs[i], batch), launch, i);
    if (st != WK_OK) return st;
  }
  return WK_OK;
}

int32_t stack_backward(int32_t l, const wk_layer_desc* descs, const wk_layer_weights* weights, int64_t batch,
                       const void* x, const void* saved, const void* dy, void* dx, const wk_layer_grads* grads,
                       void* ws, size_t ws_bytes, void* stream, wk_trace* trace) {
  StackTrainPlan sp;
  size_t need = 0;
  int32_t st = check_stack_train(l, descs, batch, &sp, &need);
  if (st != WK_OK) return st;
  if (!weights || !grads) return WK_ERR_INVALID_ARG;
  // everything the per-layer calls would check, up front: nothing is launched on an error
  for (int i = 0; i < l; ++i) {
    st = check_weights(descs[i], &weights[i]);
    if (st != WK_OK) return st;
    const wk_layer_grads& gr = grads[i];
    if (!gr.phi || !gr.w_l || !gr.mlp_w) return WK_ERR_INVALID_ARG;
    for (int t = 0; t < descs[i].num_linear; ++t)
      if (!gr.mlp_w[t]) return WK_ERR_INVALID_ARG;
  }
  if (batch == 0) return WK_OK;
  const size_t act = (size_t)batch * descs[0].n * descs[0].d * 2;
  if (!x || !saved || !dy || !dx || !ws) return WK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(saved) || !aligned16(dy) || !aligned16(dx) || !aligned16(ws))
    return WK_ERR_INVALID_ARG;
  if (ws_bytes < need) return WK_ERR_WORKSPACE;
  if (overlap(ws, need, x, act) || overlap(ws, need, dy, act) || overlap(ws, need, dx, act) ||
      overlap(ws, need, saved, sp.bytes) || overlap(dx, act, x, act) || overlap(dx, act, dy, act) ||
      overlap(dx, act, saved, sp.bytes))
    return WK_ERR_INVALID_ARG;
  char* base = static_cast<char*>(ws);
  const size_t act_al = align_up(act);
  void* g[2] = {base, base + act_al};
  char* lws = base + 2 * act_al;
  const size_t lws_bytes = ws_bytes - 2 * act_al;
  const char* sb = static_cast<const char*>(saved);
  for (int i = l - 1; i >= 0; --i) {
    const void* xi = i == 0 ? x : static_cast<const void*>(sb + sp.in[i]);
    const void* dyi = i == l - 1 ? dy : static_cast<const void*>(g[(i + 1) % 2]);
    void* dxi = i == 0 ? dx : g[i % 2];
    st = layer_backward(&descs[i], &weights[i], batch, xi, sb + sp.sv[i], dyi, dxi, &grads[i], lws, lws_bytes,
                        stream, trace, i);
    if (st != WK_OK) return st;
  }
  return WK_OK;
}

}  // namespace

// ---- The layer forward without any allocation: its workspace is a file-scope
// device array (one copy per GPU, held until the process ends).  In host code
// `scratch` names a host-side stand-in, so its device address is looked up
// once per device with hipGetSymbolAddress and only that address is used.
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // the maximum workspace of wukong_layer_forward_noalloc
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return WK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WK_OK;
}

}  // namespace

extern "C" {

int32_t wukong_abi_version(void) { return WUKONG_ABI_VERSION; }

const char* wukong_status_string(int32_t s) {
  switch (s) {
    case WK_OK: return "WK_OK: success";
    case WK_ERR_INVALID_ARG: return "WK_ERR_INVALID_ARG: null, misaligned or overlapping pointer, or inconsistent dimensions";
    case WK_ERR_UNSUPPORTED: return "WK_ERR_UNSUPPORTED: shape or dtype outside the compiled kernel set (or n_F + n_L != n)";
    case WK_ERR_WORKSPACE: return "WK_ERR_WORKSPACE: workspace smaller than the required size";
    case WK_ERR_HIP: return "WK_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown wukong status";
  }
}

size_t wukong_layer_workspace_size(const wk_layer_desc* desc, int64_t batch) {
  StackPlan sp;
  if (check_stack(1, desc, batch, &sp) != WK_OK) return 0;
  return sp.bytes;
}

int32_t wukong_layer_workspace_layout(const wk_layer_desc* desc, int64_t batch, wk_workspace_layout* out) {
  if (!out) return WK_ERR_INVALID_ARG;
  const int32_t st = check_stack(1, desc, batch, nullptr);
  if (st != WK_OK) return st;
  const LayerPlan p = plan_layer(*desc, batch);
  out->fn = (int64_t)p.fn;
  out->fn_kblock_rows = p.fn_kb;
  out->m = p.fused_out ? -1 : (int64_t)p.m;
  out->num_hidden = desc->num_linear - 1;
  for (int i = 0; i < 8; ++i) out->hidden[i] = -1;
  for (int t = 1; t < desc->num_linear && t <= 8; ++t) {
    const bool survives = t >= desc->num_linear - 2;  // only the last two hidden outputs survive
    out->hidden[t - 1] = survives ? (int64_t)p.h[(t - 1) % 2] : -1;
  }
  return WK_OK;
}

int32_t wukong_layer_forward(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                             const void* x, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return stack_forward(1, desc, weights, batch, x, y, workspace, workspace_bytes, stream, nullptr);
}

size_t wukong_layer_forward_noalloc_max_workspace(void) { return kScratchBytes; }

int32_t wukong_layer_forward_noalloc(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                                     const void* x, void* y, void* stream) {
  StackPlan sp;
  const int32_t st = check_stack(1, desc, batch, &sp);
  if (st != WK_OK) return st;
  if (sp.bytes > kScratchBytes) return WK_ERR_WORKSPACE;  // the layer needs more than the static workspace
  void* ws = nullptr;
  const int32_t sst = scratch_of_current_device(&ws);
  if (sst != WK_OK) return sst;
  return stack_forward(1, desc, weights, batch, x, y, ws, kScratchBytes, stream, nullptr);
}

size_t wukong_stack_workspace_size(int32_t num_layers, const wk_layer_desc* descs, int64_t batch) {
  StackPlan sp;
  if (check_stack(num_layers, descs, batch, &sp) != WK_OK) return 0;
  return sp.bytes;
}

int32_t wukong_stack_forward(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                             int64_t batch, const void* x, void* y, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return stack_forward(num_layers, descs, weights, batch, x, y, workspace, workspace_bytes, stream, nullptr);
}

int32_t wukong_stack_forward_traced(int32_t num_layers, const wk_layer_desc* descs,
                                    const wk_layer_weights* weights, int64_t batch, const void* x, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream, wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return stack_forward(num_layers, descs, weights, batch, x, y, workspace, workspace_bytes, stream, trace);
}

int32_t wukong_trace_create(int32_t capacity, wk_trace** out) {
  if (!out || capacity <= 0 || capacity > (1 << 20)) return WK_ERR_INVALID_ARG;
  wk_trace* t = new (std::nothrow) wk_trace;
  if (!t) return WK_ERR_INVALID_ARG;
  if (hipGetDevice(&t->device) != hipSuccess) {
    delete t;
    return WK_ERR_HIP;
  }
  t->capacity = capacity;
  t->start.assign(capacity, nullptr);
  t->stop.assign(capacity, nullptr);
  t->kind.assign(capacity, 0);
  t->layer.assign(capacity, 0);
  t->index.assign(capacity, 0);
  t->wgs.assign(capacity, 0);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&t->start[i]) != hipSuccess || hipEventCreate(&t->stop[i]) != hipSuccess) {
      wukong_trace_destroy(t);
      return WK_ERR_HIP;
    }
  }
  *out = t;
  return WK_OK;
}

int32_t wukong_trace_destroy(wk_trace* t) {
  if (!t) return WK_ERR_INVALID_ARG;
  for (hipEvent_t e : t->start)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->stop)
    if (e) (void)hipEventDestroy(e);
  delete t;
  return WK_OK;
}

int32_t wukong_trace_reset(wk_trace* t) {
  if (!t) return WK_ERR_INVALID_ARG;
  t->count = 0;
  return WK_OK;
}

int32_t wukong_trace_count(const wk_trace* t) { return t ? t->count : -1; }

int32_t wukong_trace_get(wk_trace* t, int32_t i, int32_t* kind, int32_t* layer, int32_t* index,
                         int64_t* workgroups, float* ms) {
  if (!t || i < 0 || i >= t->count) return WK_ERR_INVALID_ARG;
  if (kind) *kind = t->kind[i];
  if (layer) *layer = t->layer[i];
  if (index) *index = t->index[i];
  if (workgroups) *workgroups = t->wgs[i];
  if (ms) {
    if (hipEventSynchronize(t->stop[i]) != hipSuccess) return WK_ERR_HIP;
    if (hipEventElapsedTime(ms, t->start[i], t->stop[i]) != hipSuccess) return WK_ERR_HIP;
  }
  return WK_OK;
}

}  // extern "C"

extern "C" {

size_t wukong_head_workspace_size(const wk_head_desc* desc, int64_t batch) {
  if (check_head_desc(desc) != WK_OK || batch < 0 || batch > kMaxBatch) return 0;
  return plan_head(*desc, batch).bytes;
}

int32_t wukong_head_forward(const wk_head_desc* desc, const wk_head_weights* weights, int64_t batch, const void* y,
                            float* prob, void* workspace, size_t workspace_bytes, void* stream) {
  return head_forward(desc, weights, batch, y, prob, workspace, workspace_bytes, stream, nullptr);
}

size_t wukong_fusion_workspace_size(const wk_fusion_desc* desc, int64_t batch) {
  if (check_fusion_desc(desc) != WK_OK || batch < 0 || batch > kMaxBatch) return 0;
  return plan_fusion(*desc, batch).bytes;
}

int32_t wukong_fusion_forward(const wk_fusion_desc* desc, const wk_fusion_weights* weights, int64_t batch,
                              const void* hw, const void* hs, void* hf, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return fusion_forward(desc, weights, batch, hw, hs, hf, workspace, workspace_bytes, stream, nullptr);
}

int32_t wukong_fusion_forward_traced(const wk_fusion_desc* desc, const wk_fusion_weights* weights, int64_t batch,
                                     const void* hw, const void* hs, void* hf, void* workspace,
                                     size_t workspace_bytes, void* stream, wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return fusion_forward(desc, weights, batch, hw, hs, hf, workspace, workspace_bytes, stream, trace);
}

size_t wukong_moe_layer_workspace_size(const wk_moe_desc* desc, int64_t batch) {
  size_t b = 0;
  return check_moe(desc, batch, &b) == WK_OK ? b : 0;
}

int32_t wukong_moe_layer_forward(const wk_moe_desc* desc, const wk_layer_weights* experts, const void* out_ln_gamma,
                                 const void* out_ln_beta, int64_t batch, const void* x, void* y, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return moe_forward(desc, experts, out_ln_gamma, out_ln_beta, batch, x, y, workspace, workspace_bytes, stream,
                     nullptr);
}

int32_t wukong_moe_layer_forward_traced(const wk_moe_desc* desc, const wk_layer_weights* experts,
                                        const void* out_ln_gamma, const void* out_ln_beta, int64_t batch,
                                        const void* x, void* y, void* workspace, size_t workspace_bytes,
                                        void* stream, wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return moe_forward(desc, experts, out_ln_gamma, out_ln_beta, batch, x, y, workspace, workspace_bytes, stream,
                     trace);
}

size_t wukong_layer_saved_size(const wk_layer_desc* desc, int64_t batch) {
  if (check_backward_desc(desc) != WK_OK || batch < 0 || batch > kMaxBatch) return 0;
  const size_t b = plan_saved(*desc, batch).bytes;
  return b ? b : kAlign;
}

int32_t wukong_layer_forward_train(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                                   const void* x, void* y, void* saved, size_t saved_bytes, void* stream) {
  return layer_forward_train(desc, weights, batch, x, y, saved, saved_bytes, stream);
}

size_t wukong_stack_saved_size(int32_t num_layers, const wk_layer_desc* descs, int64_t batch) {
  StackTrainPlan sp;
  return check_stack_train(num_layers, descs, batch, &sp, nullptr) == WK_OK ? sp.bytes : 0;
}

int32_t wukong_stack_forward_train(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                                   int64_t batch, const void* x, void* y, void* saved, size_t saved_bytes,
                                   void* stream) {
  return stack_forward_train(num_layers, descs, weights, batch, x, y, saved, saved_bytes, stream);
}

size_t wukong_stack_backward_workspace_size(int32_t num_layers, const wk_layer_desc* descs, int64_t batch) {
  size_t b = 0;
  return check_stack_train(num_layers, descs, batch, nullptr, &b) == WK_OK ? b : 0;
}

int32_t wukong_stack_backward(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                              int64_t batch, const void* x, const void* saved, const void* dy, void* dx,
                              const wk_layer_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
  return stack_backward(num_layers, descs, weights, batch, x, saved, dy, dx, grads, workspace, workspace_bytes,
                        stream, nullptr);
}

int32_t wukong_stack_backward_traced(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                                     int64_t batch, const void* x, const void* saved, const void* dy, void* dx,
                                     const wk_layer_grads* grads, void* workspace, size_t workspace_bytes,
                                     void* stream, wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return stack_backward(num_layers, descs, weights, batch, x, saved, dy, dx, grads, workspace, workspace_bytes,
                        stream, trace);
}

size_t wukong_layer_backward_workspace_size(const wk_layer_desc* desc, int64_t batch) {
  if (check_backward_desc(desc) != WK_OK || batch < 0 || batch > kMaxBatch) return 0;
  const BackwardPlan bp = plan_backward(*desc, batch);
  if (bp.wide && bp.ldg > INT32_MAX) return 0;
  return bp.bytes ? bp.bytes : kAlign;
}

int32_t wukong_layer_backward(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                              const void* x, const void* saved, const void* dy, void* dx,
                              const wk_layer_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
  return layer_backward(desc, weights, batch, x, saved, dy, dx, grads, workspace, workspace_bytes, stream, nullptr);
}

int32_t wukong_layer_backward_traced(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                                     const void* x, const void* saved, const void* dy, void* dx,
                                     const wk_layer_grads* grads, void* workspace, size_t workspace_bytes,
                                     void* stream, wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return layer_backward(desc, weights, batch, x, saved, dy, dx, grads, workspace, workspace_bytes, stream, trace);
}

int32_t wukong_head_forward_traced(const wk_head_desc* desc, const wk_head_weights* weights, int64_t batch,
                                   const void* y, float* prob, void* workspace, size_t workspace_bytes, void* stream,
                                   wk_trace* trace) {
  if (!trace) return WK_ERR_INVALID_ARG;
  return head_forward(desc, weights, batch, y, prob, workspace, workspace_bytes, stream, trace);
}

}  // extern "C"
