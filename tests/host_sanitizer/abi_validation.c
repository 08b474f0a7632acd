/* Host-only driver of the C ABI's argument validation and workspace planning,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
 * of wukong_abi.cpp (test_host_sanitizer.py).  Every call here either only
 * computes sizes or is rejected before any launch, so no GPU is needed.
 * Exit status: the number of failed expectations. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "wukong.h"

static int failures = 0;
#define EXPECT(cond, what)                                   \
  do {                                                       \
    if (!(cond)) {                                           \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
      ++failures;                                            \
    }                                                        \
  } while (0)

static wk_layer_desc layer(int32_t n, int32_t d, int32_t k, int32_t n_f, int32_t n_l, const int32_t* mlp,
                           int32_t num_linear, int32_t dtype) {
  wk_layer_desc L;
  L.n = n; L.d = d; L.k = k; L.n_f = n_f; L.n_l = n_l;
  L.num_linear = num_linear; L.mlp_dims = mlp; L.ln_eps = 1e-5f; L.dtype = dtype;
  return L;
}

int main(void) {
  EXPECT(wukong_abi_version() == WUKONG_ABI_VERSION, "abi version");
  for (int32_t s = -1; s <= 5; ++s) EXPECT(wukong_status_string(s) && strlen(wukong_status_string(s)) > 0, "status string");

  /* the five workloads' layer shapes */
  const int32_t m1[] = {4096, 2048, 10240};
  const int32_t m2[] = {12288, 4096, 4096, 20480};
  const int32_t m3[] = {49152, 8192, 8192, 40960};
  const int32_t m4[] = {17280, 1024, 11520};
  const int32_t m0[] = {64, 64, 128};
  wk_layer_desc c0 = layer(16, 16, 4, 8, 8, m0, 2, WK_F32);
  wk_layer_desc c1 = layer(128, 160, 32, 64, 64, m1, 2, WK_BF16);
  wk_layer_desc c2 = layer(256, 160, 48, 128, 128, m2, 3, WK_BF16);
  wk_layer_desc c3 = layer(512, 160, 96, 256, 256, m3, 3, WK_BF16);
  wk_layer_desc c4 = layer(720, 32, 24, 360, 360, m4, 2, WK_BF16);
  const wk_layer_desc* all[] = {&c0, &c1, &c2, &c3, &c4};
  const int64_t batches[] = {64, 4096, 16384, 2048, 8192};
  for (int i = 0; i < 5; ++i) {
    const size_t ws = wukong_layer_workspace_size(all[i], batches[i]);
    EXPECT(ws > 0, "valid layer has a workspace");
    EXPECT(wukong_layer_workspace_size(all[i], 0) >= 0, "empty batch plans");
    wk_workspace_layout lay;
    EXPECT(wukong_layer_workspace_layout(all[i], batches[i], &lay) == WK_OK, "layout");
    EXPECT(lay.fn >= 0 && (size_t)lay.fn < ws, "fn inside the workspace");
    EXPECT(wukong_layer_workspace_layout(all[i], batches[i], NULL) == WK_ERR_INVALID_ARG, "layout out NULL");
  }
  wk_layer_desc stack8[8];
  for (int i = 0; i < 8; ++i) stack8[i] = c2;
  EXPECT(wukong_stack_workspace_size(8, stack8, 16384) > wukong_layer_workspace_size(&c2, 16384),
         "stack needs its ping-pong buffers");
  EXPECT(wukong_stack_workspace_size(0, stack8, 16) == 0, "zero layers");
  EXPECT(wukong_stack_workspace_size(8, NULL, 16) == 0, "null descs");
  stack8[3].d = 32;  /* a layer whose width does not chain */
  EXPECT(wukong_stack_workspace_size(8, stack8, 16) == 0, "widths must chain");

  /* invalid descs: every size query returns 0 */
  const int32_t bad_first[] = {4095, 2048, 10240};
  const int32_t bad_last[] = {4096, 2048, 10000};
  const int32_t zero_mid[] = {4096, 0, 10240};
  wk_layer_desc bad[8];
  bad[0] = layer(128, 160, 32, 64, 64, bad_first, 2, WK_BF16);
  bad[1] = layer(128, 160, 32, 64, 64, bad_last, 2, WK_BF16);
  bad[2] = layer(128, 160, 32, 64, 64, zero_mid, 2, WK_BF16);
  bad[3] = layer(128, 160, 32, 64, 64, m1, 0, WK_BF16);
  bad[4] = layer(128, 160, 32, 64, 64, NULL, 2, WK_BF16);
  bad[5] = layer(128, 160, 32, 64, 63, m1, 2, WK_BF16);   /* n_f + n_l != n */
  bad[6] = layer(128, 160, 32, 64, 64, m1, 2, 7);         /* unknown dtype */
  bad[7] = layer(128, 160, 32, 64, 64, m1, 2, WK_BF16);
  bad[7].ln_eps = -1.0f;
  for (int i = 0; i < 8; ++i) {
    EXPECT(wukong_layer_workspace_size(&bad[i], 16) == 0, "invalid desc plans nothing");
    EXPECT(wukong_layer_saved_size(&bad[i], 16) == 0, "invalid desc saves nothing");
    EXPECT(wukong_layer_backward_workspace_size(&bad[i], 16) == 0, "invalid desc: no backward");
  }
  EXPECT(wukong_layer_workspace_size(NULL, 16) == 0, "null desc");
  EXPECT(wukong_layer_workspace_size(&c1, -1) == 0, "negative batch");
  EXPECT(wukong_layer_workspace_size(&c1, (int64_t)1 << 40) == 0, "absurd batch");

  /* calls rejected before any launch: distinct, far-apart, 256-byte aligned addresses that are
     never dereferenced (nothing is launched) */
  void* X = (void*)(uintptr_t)0x100000000ull;
  void* Y = (void*)(uintptr_t)0x200000000ull;
  void* WS = (void*)(uintptr_t)0x300000000ull;
  void* P = (void*)(uintptr_t)0x400000000ull;
  const void* ws_ptrs[3] = {P, P, P};
  wk_layer_weights w;
  memset(&w, 0, sizeof w);
  w.phi = P; w.w_l = P; w.mlp_w = ws_ptrs;
  const size_t need = wukong_layer_workspace_size(&c1, 4);
  EXPECT(wukong_layer_forward(NULL, &w, 4, X, Y, WS, need, NULL) == WK_ERR_INVALID_ARG, "null desc");
  EXPECT(wukong_layer_forward(&c1, NULL, 4, X, Y, WS, need, NULL) == WK_ERR_INVALID_ARG, "null weights");
  EXPECT(wukong_layer_forward(&c1, &w, 4, NULL, Y, WS, need, NULL) == WK_ERR_INVALID_ARG, "null x");
  EXPECT(wukong_layer_forward(&c1, &w, 4, (char*)X + 8, Y, WS, need, NULL) == WK_ERR_INVALID_ARG, "misaligned x");
  EXPECT(wukong_layer_forward(&c1, &w, 4, X, X, WS, need, NULL) == WK_ERR_INVALID_ARG, "x aliases y");
  EXPECT(wukong_layer_forward(&c1, &w, 4, X, Y, WS, need - 1, NULL) == WK_ERR_WORKSPACE, "workspace too small");
  EXPECT(wukong_layer_forward(&bad[5], &w, 4, X, Y, WS, need, NULL) != WK_OK, "invalid desc");
  EXPECT(wukong_layer_forward_noalloc(&bad[0], &w, 4, X, Y, NULL) == WK_ERR_INVALID_ARG, "no-alloc: invalid desc");
  EXPECT(wukong_layer_forward_noalloc(&c1, &w, 1 << 20, X, Y, NULL) == WK_ERR_WORKSPACE,
         "no-alloc: beyond the static workspace");
  EXPECT(wukong_layer_forward_noalloc_max_workspace() == ((size_t)64 << 20), "no-alloc limit");

  /* prediction head, fusion and mixture-of-experts planning */
  const int32_t hd[] = {40960, 1024, 256, 1};
  wk_head_desc h = {3, hd, WK_BF16};
  EXPECT(wukong_head_workspace_size(&h, 16384) > 0, "head");
  h.num_linear = 0;
  EXPECT(wukong_head_workspace_size(&h, 16) == 0, "head without Linears");
  wk_fusion_desc f = {128, 160, 1024, 640, 1e-5f, WK_BF16};
  EXPECT(wukong_fusion_workspace_size(&f, 4096) > 0, "fusion");
  f.n = 40;  /* n % 16 != 0 */
  EXPECT(wukong_fusion_workspace_size(&f, 16) == 0, "fusion: n % 16");
  f.n = 128; f.d = 48;
  EXPECT(wukong_fusion_workspace_size(&f, 16) == 0, "fusion: unsupported d");
  EXPECT(wukong_fusion_workspace_size(NULL, 16) == 0, "fusion: null desc");

  if (failures == 0) printf("abi_validation: all expectations met\n");
  return failures;
}
