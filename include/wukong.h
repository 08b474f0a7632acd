/*
 * wukong.h -- C ABI of libwukong: forward pass of the stacked Wukong
 * interaction layer on one AMD Instinct MI355X (gfx950).
 *
 * The operation (Wukong paper, section 2.2 "Wukong", as summarised on the
 * xdnf.cn repost of the Zhihu article; the page's equations were lost in
 * extraction, so this follows its prose):  a Wukong layer runs a
 * Factorization Machine Block (FMB) and a Linear Compress Block (LCB) side by
 * side on one example's feature matrix X (n embeddings of width d), then
 * concatenates their outputs, adds the residual X and applies a LayerNorm.
 * The FMB "first compresses the number of features to k, then computes the
 * interaction" and ends in an MLP whose output is an n_F x d matrix; the LCB
 * is a weight matrix W_L mapping the n input embeddings to n_L outputs.
 * Section 2.3 of the same page lists the scaling knobs: the number of layers
 * l, n_F, n_L, k and the MLP's depth and widths.  WHALE's non-sequential
 * branch (WHALE summary, section 2.1 "Wukong module") applies the same
 * stacked FMB + LCB layer by layer, which is why a single layer is exposed
 * as well as the stack.
 *
 * Per example and layer, with row-major tensors:
 *   Z  = Phi X                (k x d)      Phi is a learned [k, n] weight
 *   F  = X Z^T                (n x k)      = (X X^T) Phi^T, the compressed FM
 *   Fn = LN(vec(F); gamma_fm, beta_fm)     over all n*k values, row-major
 *   h_t = ReLU(W_t h_{t-1} + b_t), t < T;  h_T = W_T h_{T-1} + b_T;  h_0 = Fn
 *   M  = reshape(h_T, n_F x d)             row-major
 *   Lc = W_L X                (n_L x d)
 *   Y[r] = LN([M; Lc][r] + X[r]; gamma_out, beta_out)   each row over d
 * LayerNorm uses the biased variance and the caller's epsilon.  n_F + n_L
 * must equal n (the residual adds X row by row).
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, last dimension contiguous, in device
 *     memory, owned by the caller.  The library never allocates device
 *     memory, frees it or keeps a pointer past the call.
 *   - Every tensor of a layer has the layer's dtype (WK_F32 or WK_BF16).
 *     WK_BF16 layers compute with fp32 accumulation and fp32 LayerNorm
 *     statistics; the tensors they store in bf16 are Z (as a product
 *     operand), Fn, every h_t, M and Y.  Lc is not rounded: the LCB rows of
 *     Y are finished from fp32 values.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting.  Nothing synchronises with the
 *     host.  A fault inside a kernel surfaces at the caller's next sync.
 *   - All arguments are checked before anything is launched: a call that
 *     returns an error has launched nothing.
 *   - Device pointers must be 16-byte aligned.  x and y must not overlap
 *     each other or the workspace.
 *   - Calls are thread-safe; concurrent calls need distinct workspaces and
 *     outputs.
 */
#ifndef WUKONG_H_
#define WUKONG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WUKONG_ABI_VERSION 2

typedef enum {
  WK_OK = 0,
  WK_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad dimension, aliasing */
  WK_ERR_UNSUPPORTED = 2, /* valid request outside the compiled kernel set   */
  WK_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_size     */
  WK_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed      */
} wk_status;

typedef enum { WK_F32 = 0, WK_BF16 = 1 } wk_dtype;

/* Shape of one layer.  mlp_dims is a HOST array of num_linear + 1 widths
 * [n*k, m_1, ..., n_f*d]; the FMB MLP has num_linear Linear layers.
 * WK_BF16 additionally needs d % 16 == 0, n % 8 == 0, k % 4 == 0 and every
 * MLP width % 8 == 0 (else WK_ERR_UNSUPPORTED).  ln_eps >= 0 is the
 * LayerNorm epsilon of both LayerNorms (1e-5 is the usual value). */
typedef struct {
  int32_t n, d, k, n_f, n_l;
  int32_t num_linear;
  const int32_t* mlp_dims;
  float ln_eps;
  int32_t dtype; /* wk_dtype */
} wk_layer_desc;

/* Device pointers to one layer's parameters (layer dtype, row-major).
 * mlp_w and mlp_b are HOST arrays of num_linear device pointers;
 * W_t is [m_t, m_{t-1}] (output-major, as torch.nn.Linear stores it) and
 * b_t is [m_t].  mlp_b itself, any of its entries, and any gamma/beta may
 * be NULL, meaning a zero bias, gamma = 1 or beta = 0. */
typedef struct {
  const void* phi;          /* [k, n]   */
  const void* w_l;          /* [n_l, n] */
  const void* fm_ln_gamma;  /* [n*k]    */
  const void* fm_ln_beta;   /* [n*k]    */
  const void* const* mlp_w; /* host array [num_linear] of device [m_t, m_{t-1}] */
  const void* const* mlp_b; /* host array [num_linear] of device [m_t], or NULL */
  const void* out_ln_gamma; /* [d]      */
  const void* out_ln_beta;  /* [d]      */
} wk_layer_weights;

/* Version of this header the library was built from (WUKONG_ABI_VERSION). */
int32_t wukong_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* wukong_status_string(int32_t status);

/* Bytes of device workspace wukong_layer_forward needs for `batch`
 * examples, or 0 if desc is invalid or unsupported.  Besides the
 * intermediates it holds, for the wider bf16 layers (n of 256 and more), a
 * copy of [Phi; W_L] rearranged into the tile order the FMB+LCB kernel
 * streams, rewritten at every call. */
size_t wukong_layer_workspace_size(const wk_layer_desc* desc, int64_t batch);

/* One Wukong layer: y[b] = layer(x[b]) for b < batch.
 *   x [batch, n, d] and y [batch, n, d] in the layer dtype.
 *   workspace: device scratch of at least wukong_layer_workspace_size bytes;
 *   its contents on return are the layer's intermediates laid out as
 *   wukong_layer_workspace_layout describes.  batch == 0 is a no-op. */
int32_t wukong_layer_forward(const wk_layer_desc* desc, const wk_layer_weights* weights,
                             int64_t batch, const void* x, void* y, void* workspace,
                             size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): wukong_layer_forward
 * with its workspace taken from a static device array of the library
 * (wukong_layer_forward_noalloc_max_workspace() bytes, 64 MiB, one copy per GPU,
 * held until the process ends).  The caller passes x and y as for
 * wukong_layer_forward; the call allocates and frees nothing.  Returns
 * WK_ERR_WORKSPACE, launching nothing, when wukong_layer_workspace_size(desc,
 * batch) exceeds that size (the d = 160, n = 128 layer fits up to a batch of
 * about 5400 examples), WK_ERR_HIP if the array's device address cannot be
 * obtained, else as wukong_layer_forward.  Every call on one GPU uses the same
 * array: calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race on it and must not be made.  The array keeps
 * the last call's intermediates; nothing in it needs clearing between calls. */
int32_t wukong_layer_forward_noalloc(const wk_layer_desc* desc, const wk_layer_weights* weights,
                                     int64_t batch, const void* x, void* y, void* stream);
size_t wukong_layer_forward_noalloc_max_workspace(void);

/* Byte offsets, within a layer's workspace, of the intermediates a
 * wukong_layer_forward call leaves there (for per-kernel checks):
 *   fn      [batch, n*k]       the normalised interaction Fn
 *   hidden  [batch, m_t] for t = 1..num_linear-1: hidden[t-1]; the hidden
 *           activations alternate between two buffers, so only the last two
 *           survive (offset -1 marks an overwritten one)
 *   m       [batch, n_f*d]     the last MLP output M, or -1 when the last
 *           Linear applies the residual LayerNorm in its own epilogue (bf16
 *           layers with d in {16, 32, 80, 160} and a last-Linear input width
 *           that is a multiple of 64): then M is never stored
 *   fn_kblock_rows  0 when Fn is row-major as above; R > 0 when it is stored
 *           K-blocked for the first Linear: element (b, c) at
 *           ((c / 64) R + b) 64 + c % 64, R = batch rounded up to a multiple
 *           of 256 (bf16 layers of n >= 256 whose first Linear has
 *           n*k >= 8192 inputs: the Linear's 64-column steps of Fn are then
 *           contiguous; rows b >= batch hold no data)
 * Returns WK_OK, or an error as wukong_layer_forward would for desc/batch. */
typedef struct {
  int64_t fn;
  int64_t m;
  int32_t num_hidden;
  int64_t hidden[8]; /* first min(num_hidden, 8) entries are meaningful */
  int64_t fn_kblock_rows;
} wk_workspace_layout;
int32_t wukong_layer_workspace_layout(const wk_layer_desc* desc, int64_t batch,
                                      wk_workspace_layout* out);

/* Bytes of workspace wukong_stack_forward needs (0 if invalid). */
size_t wukong_stack_workspace_size(int32_t num_layers, const wk_layer_desc* descs,
                                   int64_t batch);

/* l stacked Wukong layers: layer i reads layer i-1's output (Wukong paper,
 * section 2.3: l is the depth of the interaction stack).  descs and weights
 * are HOST arrays of num_layers entries; every layer must keep n and d
 * (n_F + n_L = n) and share one dtype.  x [batch, n, d] in, y [batch, n, d]
 * out; intermediate layer outputs live in the workspace. */
int32_t wukong_stack_forward(int32_t num_layers, const wk_layer_desc* descs,
                             const wk_layer_weights* weights, int64_t batch, const void* x,
                             void* y, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- tracing
 * Per-kernel timing for benchmarks: a trace owns a pool of HIP events.
 * wukong_stack_forward_traced behaves exactly like wukong_stack_forward and
 * additionally records an event before and after each kernel it launches
 * (on `stream`).  Records are appended until the pool is full; later
 * launches go unrecorded.  Kernel kinds: */
enum {
  WK_KERNEL_FMB_LCB = 1,    /* compress + interaction + LN(F) + LCB rows of Y */
  WK_KERNEL_MLP_LINEAR = 2, /* one FMB-MLP Linear (+bias, +ReLU)             */
  WK_KERNEL_RESIDUAL_LN = 3, /* FMB rows of Y: LN(M + X)                     */
  WK_KERNEL_HEAD_LINEAR = 4,  /* one hidden Linear of the prediction head     */
  WK_KERNEL_HEAD_OUT = 5,     /* the head's last Linear + logistic function   */
  WK_KERNEL_FUSION_ATTN = 6,  /* WHALE fusion: shared K = V cross-attention and the Fusion Linear */
  WK_KERNEL_FUSION_LINEAR = 7, /* fusion, unfused FFN: SwiGLU up (index 1), down (2) */
  WK_KERNEL_FUSION_LN = 8,    /* fusion: the pre-norm LayerNorm               */
  WK_KERNEL_BWD_OUT = 9,      /* backward: output LayerNorm + LCB rows (dR)   */
  WK_KERNEL_BWD_TRANSPOSE = 10, /* backward: bf16 transpose of Linear t's output gradient
                                 (index 3t), input (3t + 1) or weight (3t + 2) */
  WK_KERNEL_BWD_WGRAD = 11,   /* backward: dW_t (index t)                     */
  WK_KERNEL_BWD_DGRAD = 12,   /* backward: gradient of the Linear's input (t) */
  WK_KERNEL_BWD_FMB = 13,     /* backward: FM LayerNorm, interaction, dX      */
  WK_KERNEL_BWD_REDUCE = 14,  /* backward: per-workgroup / per-split sums: index 0
                                 gamma_out, beta_out, Phi, W_L, gamma_fm, beta_fm (one
                                 launch); 2 + t the bias of Linear t */
  WK_KERNEL_FUSION_FFN = 15   /* fusion: pre-norm LayerNorm + SwiGLU FFN + residual in one kernel */
};
typedef struct wk_trace wk_trace;
/* Creates a trace able to hold `capacity` launch records (creates HIP events
 * on the current device). */
int32_t wukong_trace_create(int32_t capacity, wk_trace** out);
int32_t wukong_trace_destroy(wk_trace* trace);
/* Forgets all records (events are reused). */
int32_t wukong_trace_reset(wk_trace* trace);
int32_t wukong_trace_count(const wk_trace* trace);
/* Record i: kernel kind, layer index, index within the layer (the Linear
 * number for WK_KERNEL_MLP_LINEAR, else 0), launch geometry (workgroups)
 * and elapsed milliseconds.  Waits for record i's stop event. */
int32_t wukong_trace_get(wk_trace* trace, int32_t i, int32_t* kind, int32_t* layer,
                         int32_t* index, int64_t* workgroups, float* ms);
int32_t wukong_stack_forward_traced(int32_t num_layers, const wk_layer_desc* descs,
                                    const wk_layer_weights* weights, int64_t batch,
                                    const void* x, void* y, void* workspace,
                                    size_t workspace_bytes, void* stream, wk_trace* trace);

/* ---- Prediction head (top MLP) -------------------------------------------
 * Wukong paper, section 2.2 (xdnf.cn repost): after the Wukong layers have
 * done the feature interaction, an MLP produces the prediction.  The page
 * gives no sizes; this head reads a layer output Y [batch, n, d] flattened
 * row-major (feature r*d + e), applies Linear + ReLU for every Linear but the
 * last, and writes the logistic function of the last Linear's output:
 *   prob[b, o] = 1 / (1 + exp(-(W_T h_{T-1}[b] + b_T)[o])).
 * bf16 heads keep the hidden activations in bf16 (as the layer's MLP does)
 * and accumulate in fp32; the probabilities are always fp32. */
typedef struct {
  int32_t num_linear;   /* T >= 1 Linear layers                                 */
  const int32_t* dims;  /* host array, length T+1: [n*d, m_1, ..., m_T]         */
  int32_t dtype;        /* WK_F32 or WK_BF16 (Y, weights, hidden activations)   */
} wk_head_desc;         /* bf16: dims[0..T-1] % 8 == 0; m_T >= 1 is free         */

typedef struct {
  const void* const* w; /* host array of T device pointers, W_t is [m_t, m_{t-1}] */
  const void* const* b; /* host array of T device pointers [m_t] (NULL entries or
                           a NULL array: no bias)                                  */
} wk_head_weights;

/* Workspace bytes for wukong_head_forward: two ping-pong buffers of the widest
 * hidden layer, plus (bf16) fp32 partial sums for a hidden Linear whose batch
 * is too small to fill the GPU, which is then split along K (the splits are
 * summed in a fixed order, so results do not depend on timing).  0 for an
 * invalid or unsupported desc; 256 for T == 1. */
size_t wukong_head_workspace_size(const wk_head_desc* desc, int64_t batch);

/* prob [batch, m_T] fp32 (device) from y [batch, dims[0]] (device, the layer
 * output).  Same conventions as wukong_layer_forward: device pointers 16-byte
 * aligned (prob 4-byte), arguments checked before any launch, asynchronous on
 * `stream`, no allocation; y, prob and the workspace must not overlap. */
int32_t wukong_head_forward(const wk_head_desc* desc, const wk_head_weights* weights, int64_t batch,
                            const void* y, float* prob, void* workspace, size_t workspace_bytes,
                            void* stream);
/* As wukong_head_forward, recording one event pair per launch into `trace`
 * (kinds WK_KERNEL_HEAD_LINEAR with the Linear number, WK_KERNEL_HEAD_OUT). */
int32_t wukong_head_forward_traced(const wk_head_desc* desc, const wk_head_weights* weights, int64_t batch,
                                   const void* y, float* prob, void* workspace, size_t workspace_bytes,
                                   void* stream, wk_trace* trace);

/* ---- Wukong mixture of experts -------------------------------------------
 * Kunlun technical summary, section 2.3: the global interaction module runs
 * several Wukong modules side by side within one layer, spreading the
 * layer's computation over them.  The page gives no formula; reading taken
 * here: expert e is a whole Wukong module on the layer input X (its own Phi_e,
 * FM LayerNorm, MLP and W_L) producing n_f,e FMB rows and n_l,e LCB rows;
 * the layer output is
 *   Y = LN_d([M_1; ...; M_E; Lc_1; ...; Lc_E] + X; gamma_out, beta_out)
 * (FMB rows of every expert first, in expert order, then the LCB rows), with
 * sum_e (n_f,e + n_l,e) = n.  With one expert it is wukong_layer_forward.
 * The experts run one after another on the stream (the same kernels, grouped
 * launches), sharing one workspace. */
typedef struct {
  int32_t num_experts;           /* 1 .. 64                                           */
  const wk_layer_desc* experts;  /* host array [num_experts]: equal n, d, dtype and
                                    ln_eps; n_f / n_l are the expert's own row counts;
                                    bf16 experts need d % 16 == 0                      */
} wk_moe_desc;

/* Workspace bytes for wukong_moe_layer_forward, 0 if desc is invalid or
 * unsupported: the largest expert's layer workspace, or, when every expert's
 * last Linear carries the output LayerNorm (bf16, d in {16, 32, 80, 160}, its
 * input width a multiple of 64), the sum of the experts' (their last Linears
 * then run as grouped launches, recorded in a trace as layer = num_experts,
 * index = group; four experts per launch). */
size_t wukong_moe_layer_workspace_size(const wk_moe_desc* desc, int64_t batch);

/* y [batch, n, d] from x [batch, n, d].  experts: host array of num_experts
 * weight sets (their out_ln_gamma / out_ln_beta are ignored); out_ln_gamma /
 * out_ln_beta [d] (or NULL) are the layer's output LayerNorm.  Same
 * conventions as wukong_layer_forward. */
int32_t wukong_moe_layer_forward(const wk_moe_desc* desc, const wk_layer_weights* experts, const void* out_ln_gamma,
                                 const void* out_ln_beta, int64_t batch, const void* x, void* y, void* workspace,
                                 size_t workspace_bytes, void* stream);
/* As wukong_moe_layer_forward, recording one event pair per launch into
 * `trace` (the layer index of a record is the expert index). */
int32_t wukong_moe_layer_forward_traced(const wk_moe_desc* desc, const wk_layer_weights* experts,
                                        const void* out_ln_gamma, const void* out_ln_beta, int64_t batch,
                                        const void* x, void* y, void* workspace, size_t workspace_bytes,
                                        void* stream, wk_trace* trace);

/* ---- Backward pass of one layer ------------------------------------------
 * The pages train the stack end to end (Wukong paper, xdnf.cn repost,
 * section 3.2.1: the dense layers are trained with Adam; WHALE technical
 * summaries, section 2.2: bf16 dense backbone).  Given dY = dLoss/dY for a
 * layer's output, wukong_layer_backward returns dLoss/dX and every weight's
 * gradient by the chain rule through the forward above:
 *   dR     = LN_d backward of dY (R = [M; Lc] + X, per row)
 *   dM, dLc = the FMB and LCB rows of dR;   dX  = dR + W_L^T dLc + ...
 *   d_W_L  = sum_b dLc X^T
 *   g_T = vec(dM);  d_W_t = sum_b g_{t+1} a_t^T,  d_b_t = sum_b g_{t+1},
 *   g_t = (W_t^T g_{t+1}) * [h_t > 0]  (a_0 = Fn, a_t = h_t),  d_Fn = W_0^T g_1
 *   dF     = LN backward of d_Fn over the n*k values of F
 *   dZ = dF^T X;  dX += dF Z + Phi^T dZ;  d_Phi = sum_b dZ X^T
 *   d_gamma / d_beta of both LayerNorms: sums of d(out) * normalised(in) / d(out)
 * bf16 only.  The forward's Fn, h_t and M come from wukong_layer_forward_train.
 * Layers whose per-example working set fits one workgroup's LDS (X, [Phi; W_L]
 * and the operand panels; the n = 128, d = 160, k = 32, n_l = 64 layer does)
 * recompute Lc, Z and F from x.  Wider layers (n = 256 .. 768 where the
 * streamed forward kernel takes the shape: the layers of the n = 256 and
 * n = 512 stacks and the n = 720, d = 32 layer) also keep Z (bf16) and Lc
 * (fp32) from the training forward and recompute only F.  Stored in bf16: dR
 * (as dM and dLc), every g_t, d_Fn, dF and dZ (as product operands) and dX;
 * fp32 accumulation and LayerNorm statistics; weight gradients are fp32.
 * Other shapes, and d % 16 != 0: WK_ERR_UNSUPPORTED. */
typedef struct {       /* device pointers, fp32, overwritten (not accumulated)  */
  float* phi;          /* [k, n]                                               */
  float* w_l;          /* [n_l, n]                                             */
  float* fm_ln_gamma;  /* [n*k] or NULL (not computed)                         */
  float* fm_ln_beta;   /* [n*k] or NULL                                        */
  float* const* mlp_w; /* host array [num_linear] of device [m_t, m_{t-1}]     */
  float* const* mlp_b; /* host array [num_linear] of device [m_t] (NULL array or entries: not computed) */
  float* out_ln_gamma; /* [d] or NULL                                          */
  float* out_ln_beta;  /* [d] or NULL                                          */
} wk_layer_grads;

/* Bytes of the activations wukong_layer_forward_train saves for the backward:
 * Fn [batch, n*k], h_t [batch, m_t] for t = 1..num_linear-1 and M
 * [batch, n_f*d], in that order, each at a 256-byte-aligned offset; for the
 * wider layers (see wukong_layer_backward) also Z [batch, k, d] bf16 and Lc
 * [batch, n_l, d] fp32 after them, and last the scratch copy of [Phi; W_L]
 * the FMB+LCB kernel streams (not an activation; rewritten by each training
 * forward).  0 if desc is invalid or the backward does not support it. */
size_t wukong_layer_saved_size(const wk_layer_desc* desc, int64_t batch);

/* The forward of wukong_layer_forward that also keeps Fn, every h_t and M (and
 * for the wider layers Z and Lc) in `saved` (device, saved_bytes >=
 * wukong_layer_saved_size).  y equals the plain forward's within bf16
 * rounding (M is rounded to bf16 before the residual LayerNorm here).  x, y
 * and saved must not overlap. */
int32_t wukong_layer_forward_train(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                                   const void* x, void* y, void* saved, size_t saved_bytes, void* stream);

/* Workspace bytes for wukong_layer_backward (0 if unsupported). */
size_t wukong_layer_backward_workspace_size(const wk_layer_desc* desc, int64_t batch);

/* dx [batch, n, d] and the weight gradients from x (the layer input), saved
 * (written by wukong_layer_forward_train on the same x and weights) and dy
 * [batch, n, d].  grads->phi, grads->w_l and every grads->mlp_w[t] are
 * required.  Same conventions as wukong_layer_forward; dx must not overlap
 * x, dy, saved or the workspace.  batch == 0 launches nothing and leaves the
 * gradients untouched.  Every sum over the batch is taken in a fixed order,
 * so results do not depend on timing. */
int32_t wukong_layer_backward(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                              const void* x, const void* saved, const void* dy, void* dx,
                              const wk_layer_grads* grads, void* workspace, size_t workspace_bytes, void* stream);
/* As wukong_layer_backward, recording one event pair per launch into `trace`
 * (kinds WK_KERNEL_BWD_*). */
int32_t wukong_layer_backward_traced(const wk_layer_desc* desc, const wk_layer_weights* weights, int64_t batch,
                                     const void* x, const void* saved, const void* dy, void* dx,
                                     const wk_layer_grads* grads, void* workspace, size_t workspace_bytes,
                                     void* stream, wk_trace* trace);

/* Training a stack of num_layers layers (equal n, d; bf16; each layer as
 * wukong_layer_backward supports).  The saved buffer holds, per layer, its
 * input (for every layer after the first; the first one's is x) and its
 * wukong_layer_forward_train activations.  The backward runs the layers last
 * to first, each layer's dX being the previous layer's upstream gradient;
 * grads is a HOST array of num_layers gradient sets (layer order).  The
 * workspace holds two [batch, n, d] gradient buffers and one layer's backward
 * workspace.  Conventions as wukong_layer_backward; records of the traced
 * form carry the layer index. */
size_t wukong_stack_saved_size(int32_t num_layers, const wk_layer_desc* descs, int64_t batch);
int32_t wukong_stack_forward_train(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                                   int64_t batch, const void* x, void* y, void* saved, size_t saved_bytes,
                                   void* stream);
size_t wukong_stack_backward_workspace_size(int32_t num_layers, const wk_layer_desc* descs, int64_t batch);
int32_t wukong_stack_backward(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                              int64_t batch, const void* x, const void* saved, const void* dy, void* dx,
                              const wk_layer_grads* grads, void* workspace, size_t workspace_bytes, void* stream);
int32_t wukong_stack_backward_traced(int32_t num_layers, const wk_layer_desc* descs, const wk_layer_weights* weights,
                                     int64_t batch, const void* x, const void* saved, const void* dy, void* dx,
                                     const wk_layer_grads* grads, void* workspace, size_t workspace_bytes,
                                     void* stream, wk_trace* trace);

/* ---- WHALE fusion step ----------------------------------------------------
 * WHALE technical summaries, section 2.1 (attention-based fusion module) and
 * section 2.2 (shared key-value, shared-gate SwiGLU): the Wukong output H_w
 * is the query, the sequence branch's output H_s is both the keys and the
 * values (K = V), the attention output is concatenated with H_w, projected by
 * the Fusion MLP, and passed through a pre-norm SwiGLU FFN whose gate and up
 * projections are one matrix.  Per example (rows of H_w are query tokens):
 *   A   = softmax(H_w H_s^T / sqrt(d)) H_s               [n, d]
 *   Q   = [H_w, A] W_f^T + b_f                            [n, d]
 *   U   = LN_d(Q; gamma, beta) W_up^T + b_up              [n, d_ff]
 *   H_f = Q + (silu(U) * U) W_down^T + b_down             [n, d]
 * Readings: no separate Q/K/V projections, one head; the Fusion MLP is one
 * Linear 2d -> d.  bf16 only: A, Q, LN(Q), silu(U)*U and H_f are stored in bf16,
 * the softmax weights enter P V as bf16 (their sum stays fp32), fp32
 * accumulation throughout. */
typedef struct {
  int32_t n;            /* query tokens per example (rows of H_w), n % 16 == 0  */
  int32_t d;            /* width of H_w, H_s, H_f: 32, 64, 96, 128 or 160      */
  int32_t L;            /* positions of H_s per example, L >= 1                 */
  int32_t d_ff;         /* SwiGLU hidden width, d_ff % 8 == 0                   */
  float ln_eps;         /* pre-norm LayerNorm epsilon (biased variance)         */
  int32_t dtype;        /* WK_BF16                                              */
} wk_fusion_desc;

typedef struct {        /* device pointers, row-major, [out, in] weights          */
  const void* w_f;      /* [d, 2d]                                              */
  const void* b_f;      /* [d] or NULL                                          */
  const void* ln_gamma; /* [d] or NULL (= 1)                                    */
  const void* ln_beta;  /* [d] or NULL (= 0)                                    */
  const void* w_up;     /* [d_ff, d]: gate and up projection                    */
  const void* b_up;     /* [d_ff] or NULL                                       */
  const void* w_down;   /* [d, d_ff]                                            */
  const void* b_down;   /* [d] or NULL                                          */
} wk_fusion_weights;

/* Workspace bytes for wukong_fusion_forward, 0 for an invalid or unsupported
 * desc.  The workspace holds Q ([batch, n, d], at offset 0), which the
 * attention kernel writes (it applies the Fusion Linear to [H_w, A] on chip);
 * when d_ff % 32 != 0 or d_ff > 4096 the FFN runs as separate kernels and
 * LN(Q) and silu(U) * U follow at multiples of 256 bytes.  Otherwise the
 * LayerNorm, both FFN products and the residual are one kernel that keeps
 * silu(U) * U on chip. */
size_t wukong_fusion_workspace_size(const wk_fusion_desc* desc, int64_t batch);

/* hf [batch, n, d] (device) from hw [batch, n, d] and hs [batch, L, d]
 * (device).  Same conventions as wukong_layer_forward: 16-byte aligned device
 * pointers, arguments checked before any launch, asynchronous on `stream`, no
 * allocation; hw, hs, hf and the workspace must not overlap. */
int32_t wukong_fusion_forward(const wk_fusion_desc* desc, const wk_fusion_weights* weights, int64_t batch,
                              const void* hw, const void* hs, void* hf, void* workspace, size_t workspace_bytes,
                              void* stream);
/* As wukong_fusion_forward, recording one event pair per launch into `trace`. */
int32_t wukong_fusion_forward_traced(const wk_fusion_desc* desc, const wk_fusion_weights* weights, int64_t batch,
                                     const void* hw, const void* hs, void* hf, void* workspace,
                                     size_t workspace_bytes, void* stream, wk_trace* trace);

/* ---- Measurement aid ---------------------------------------------------------
 * The on-chip bf16 MFMA ceiling, reported by the benchmark beside the published
 * peak: `blocks` workgroups of 8 waves each run `iters` rounds of 16
 * v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 multiply-adds each) on operands that
 * change from one instruction to the next.  operands: device buffer of 16 KB
 * (16 x 64 lanes x 8 bf16, any values; the caller fills it), read-only;
 * sink: device buffer of blocks x 512 floats, written.  FLOPs of one call:
 * blocks x 8 x iters x 16 x 16384.  Asynchronous on `stream`.
 * Returns WK_ERR_INVALID_ARG for null buffers or non-positive sizes. */
int32_t wukong_probe_mfma_bf16(const void* operands, void* sink, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WUKONG_H_ */
