"""C ABI checks that run without a GPU: the library loads, exports every
symbol include/wukong.h declares, sizes workspaces as documented, and rejects
bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import recommender_feature_interaction_amd as wk
from recommender_feature_interaction_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wukong.h")

pytestmark = pytest.mark.skipif(not os.path.exists(wk.library_path()), reason="libwukong.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wukong_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = wk.load_library()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(wk.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    lib = wk.load_library()
    assert lib.wukong_abi_version() == 2
    for s in range(5):
        assert wk.status_string(s).startswith(["WK_OK", "WK_ERR_INVALID_ARG", "WK_ERR_UNSUPPORTED",
                                               "WK_ERR_WORKSPACE", "WK_ERR_HIP"][s])
    assert "unknown" in wk.status_string(99)


C1 = wk.LayerSpec(128, 160, 32, 64, 64, (4096, 2048, 10240))
C2 = wk.LayerSpec(256, 160, 48, 128, 128, (12288, 4096, 4096, 20480))


def al(v):
    return (v + 255) // 256 * 256


def test_workspace_sizes_follow_layout():
    B = 4096
    # Fn + one hidden buffer; d = 160 and K = 2048: the last Linear writes Y itself, no M
    assert wk.layer_workspace_size(C1, B) == al(B * 4096 * 2) + al(B * 2048 * 2)
    lay = wk.workspace_layout(C1, B)
    assert lay["fn"] == 0 and lay["hidden"] == [al(B * 4096 * 2)]
    assert lay["m"] == -1
    # d = 48 does not divide the fused epilogue's 160 columns: M is stored
    d48 = wk.LayerSpec(96, 48, 20, 40, 56, (1920, 256, 1920))
    assert wk.layer_workspace_size(d48, B) == al(B * 1920 * 2) + al(B * 256 * 2) + al(B * 1920 * 2)
    assert wk.workspace_layout(d48, B)["m"] == al(B * 1920 * 2) + al(B * 256 * 2)
    # K of the last Linear not a multiple of 64: M is stored
    k72 = wk.LayerSpec(40, 32, 12, 16, 24, (480, 72, 512))
    assert wk.workspace_layout(k72, B)["m"] == al(B * 480 * 2) + al(B * 72 * 2)
    # Fn K-blocked for the first Linear (the batch rounded up to 256 rows per 64-column block), two
    # hidden ping-pong buffers, then [Phi; W_L] rearranged for the streamed FMB+LCB kernel
    # (n = 256: 8 steps of 32 columns x 12 tiles of 16 x 32 bf16)
    B = 100
    assert wk.layer_workspace_size(C2, B) == al(256 * 12288 * 2) + 2 * al(B * 4096 * 2) + al(8 * 12 * 1024)
    assert wk.workspace_layout(C2, B)["fn_kblock_rows"] == 256
    assert wk.workspace_layout(C1, B)["fn_kblock_rows"] == 0  # n = 128: the resident kernel, row-major Fn
    # stacks add ping-pong activation buffers
    scratch = wk.layer_workspace_size(C2, B)
    act = al(B * 256 * 160 * 2)
    assert wk.stack_workspace_size([C2], B) == scratch
    assert wk.stack_workspace_size([C2] * 2, B) == scratch + act
    assert wk.stack_workspace_size([C2] * 8, B) == scratch + 2 * act
    # units of width 8: + transposed X, [Phi; W_L] and the fp32 Z after the M buffer
    u = wk.LayerSpec(64, 8, 8, 32, 32, (512, 64, 256))
    B = 9
    assert wk.layer_workspace_size(u, B) == (al(B * 512 * 2) + al(B * 64 * 2) + al(B * 256 * 2)
                                             + al(al(B * 64 * 8 * 2) + al(40 * 64 * 2) + al(B * 8 * 8 * 4)))
    f32 = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128), dtype="f32")
    assert wk.layer_workspace_size(f32, 64) == al(64 * 64 * 4) + al(64 * 64 * 4) + al(64 * 128 * 4)


def _size(spec, batch=8):
    return wk.layer_workspace_size(spec, batch)


def test_invalid_and_unsupported_descs():
    assert _size(C1, -1) == 0
    assert _size(wk.LayerSpec(128, 160, 32, 64, 64, (4096, 2048, 10000))) == 0      # m_T != n_F*d
    assert _size(wk.LayerSpec(128, 160, 32, 64, 64, (4000, 2048, 10240))) == 0      # m_0 != n*k
    assert _size(wk.LayerSpec(128, 160, 32, 64, 32, (4096, 2048, 10240))) == 0      # n_F + n_L != n
    assert _size(wk.LayerSpec(128, 150, 32, 64, 64, (4096, 2048, 9600))) == 0       # bf16 needs d % 16
    assert _size(wk.LayerSpec(128, 150, 32, 64, 64, (4096, 2048, 9600), dtype="f32")) == 0  # f32 LDS limit
    assert _size(wk.LayerSpec(16, 24, 4, 8, 8, (64, 30, 192), dtype="f32")) > 0     # f32 takes any width
    # bf16 units of width 8 (the batched-GEMM form): n % 64, k % 4, k <= 32, (k + n_l) % 8
    assert _size(wk.LayerSpec(64, 8, 8, 32, 32, (512, 64, 256))) > 0
    assert _size(wk.LayerSpec(2880, 8, 24, 1440, 1440, (69120, 1024, 11520))) > 0
    assert _size(wk.LayerSpec(72, 8, 8, 36, 36, (576, 64, 288))) == 0              # n % 64
    assert _size(wk.LayerSpec(64, 8, 40, 32, 32, (2560, 64, 256))) == 0            # k > 32
    assert _size(wk.LayerSpec(64, 8, 12, 32, 32, (768, 64, 256))) == 0             # (k + n_l) % 8


def _call_forward(spec, batch, x, y, ws, ws_bytes, weights=None, desc=None):
    lib = wk.load_library()
    d, dims = spec.make_desc()
    if desc is not None:
        d = desc
    T = len(spec.mlp) - 1
    wptrs = (ctypes.c_void_p * T)(*[0x10000 * (t + 1) for t in range(T)])
    if weights is None:
        weights = _abi.wk_layer_weights(0x1000, 0x2000, None, None,
                                        ctypes.cast(wptrs, ctypes.POINTER(ctypes.c_void_p)), None, None, None)
    return lib.wukong_layer_forward(ctypes.byref(d), ctypes.byref(weights), batch, x, y, ws, ws_bytes, None)


def test_forward_argument_errors_launch_nothing():
    spec = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128), dtype="bf16")
    need = wk.layer_workspace_size(spec, 4)
    X, Y, WS = 0x100000, 0x200000, 0x300000
    assert _call_forward(spec, 4, X, Y, WS, need - 1) == _abi.WK_ERR_WORKSPACE
    assert _call_forward(spec, 4, None, Y, WS, need) == _abi.WK_ERR_INVALID_ARG
    assert _call_forward(spec, 4, X + 8, Y, WS, need) == _abi.WK_ERR_INVALID_ARG   # misaligned
    assert _call_forward(spec, 4, X, X + 256, WS, need) == _abi.WK_ERR_INVALID_ARG  # x / y overlap
    assert _call_forward(spec, 4, X, Y, X, need) == _abi.WK_ERR_INVALID_ARG       # workspace overlaps x
    assert _call_forward(spec, -1, X, Y, WS, need) == _abi.WK_ERR_INVALID_ARG
    assert _call_forward(spec, 0, None, None, None, 0) == _abi.WK_OK              # empty batch: no-op
    bad = _abi.wk_layer_weights(0x1000, None, None, None, None, None, None, None)
    assert _call_forward(spec, 4, X, Y, WS, need, weights=bad) == _abi.WK_ERR_INVALID_ARG
    d, dims = spec.make_desc()
    d.dtype = 7
    assert _call_forward(spec, 4, X, Y, WS, need, desc=d) == _abi.WK_ERR_INVALID_ARG
    d, dims = spec.make_desc()
    d.ln_eps = float("nan")
    assert _call_forward(spec, 4, X, Y, WS, need, desc=d) == _abi.WK_ERR_INVALID_ARG
    d, dims = spec.make_desc()
    d.n_l = 4
    assert _call_forward(spec, 4, X, Y, WS, need, desc=d) == _abi.WK_ERR_UNSUPPORTED


def test_stack_requires_matching_layers():
    lib = wk.load_library()
    a = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128))
    b = wk.LayerSpec(16, 32, 4, 8, 8, (64, 64, 256))
    pa, pb = a.make_desc(), b.make_desc()
    descs = (_abi.wk_layer_desc * 2)(pa[0], pb[0])
    assert lib.wukong_stack_workspace_size(2, descs, 4) == 0
    assert lib.wukong_stack_workspace_size(0, descs, 4) == 0


def _head_call(dims, batch, y, prob, ws, ws_bytes, dtype="bf16", w=None, b=None, desc=None):
    lib = wk.load_library()
    spec = wk.HeadSpec(tuple(dims), dtype)
    d, _dims = spec.make_desc()
    if desc is not None:
        d = desc
    T = len(dims) - 1
    wp = (ctypes.c_void_p * T)(*([0x10000 * (t + 1) for t in range(T)] if w is None else w))
    bp = None if b is None else (ctypes.c_void_p * T)(*b)
    hw = _abi.wk_head_weights(ctypes.cast(wp, ctypes.POINTER(ctypes.c_void_p)),
                              None if bp is None else ctypes.cast(bp, ctypes.POINTER(ctypes.c_void_p)))
    return lib.wukong_head_forward(ctypes.byref(d), ctypes.byref(hw), batch, y, prob, ws, ws_bytes, None)


def test_head_workspace_sizes():
    # two ping-pong buffers of the widest hidden layer; 256 bytes with no hidden layer
    assert wk.head_workspace_size(wk.HeadSpec((40960, 1024, 256, 1)), 16384) == 2 * al(16384 * 1024 * 2)
    # + fp32 partial sums when a hidden Linear is split along K (few rows, long K): 2 and 4 splits
    assert wk.head_workspace_size(wk.HeadSpec((20480, 1024, 256, 1)), 4096) == \
        2 * al(4096 * 1024 * 2) + 2 * 4096 * 1024 * 4
    assert wk.head_workspace_size(wk.HeadSpec((81920, 1024, 256, 1)), 2048) == \
        2 * al(2048 * 1024 * 2) + 4 * 2048 * 1024 * 4
    assert wk.head_workspace_size(wk.HeadSpec((4096, 72, 1)), 37) == 2 * al(37 * 72 * 2) + al(2 * 37 * 72 * 4)
    assert wk.head_workspace_size(wk.HeadSpec((4096, 72, 1), "f32"), 37) == 2 * al(37 * 72 * 4)  # no split
    assert wk.head_workspace_size(wk.HeadSpec((64, 24, 40, 3), "f32"), 10) == 2 * al(10 * 40 * 4)
    assert wk.head_workspace_size(wk.HeadSpec((64, 1)), 10) == 256
    assert wk.head_workspace_size(wk.HeadSpec((64, 12, 1)), 10) == 0          # bf16 hidden width % 8
    assert wk.head_workspace_size(wk.HeadSpec((60, 16, 1)), 10) == 0          # bf16 input width % 8
    assert wk.head_workspace_size(wk.HeadSpec((60, 12, 1), "f32"), 10) > 0    # f32 takes any width
    assert wk.head_workspace_size(wk.HeadSpec((64, 1)), -1) == 0


def test_head_argument_errors_launch_nothing():
    dims = (64, 32, 1)
    need = wk.head_workspace_size(wk.HeadSpec(dims), 4)
    Y, P, WS = 0x100000, 0x200000, 0x300000
    assert _head_call(dims, 4, Y, P, WS, need - 1) == _abi.WK_ERR_WORKSPACE
    assert _head_call(dims, 4, None, P, WS, need) == _abi.WK_ERR_INVALID_ARG
    assert _head_call(dims, 4, Y, None, WS, need) == _abi.WK_ERR_INVALID_ARG
    assert _head_call(dims, 4, Y + 8, P, WS, need) == _abi.WK_ERR_INVALID_ARG      # misaligned y
    assert _head_call(dims, 4, Y, P + 2, WS, need) == _abi.WK_ERR_INVALID_ARG      # misaligned prob
    assert _head_call(dims, 4, Y, Y + 64, WS, need) == _abi.WK_ERR_INVALID_ARG     # prob inside y
    assert _head_call(dims, 4, Y, P, Y, need) == _abi.WK_ERR_INVALID_ARG           # workspace overlaps y
    assert _head_call(dims, -1, Y, P, WS, need) == _abi.WK_ERR_INVALID_ARG
    assert _head_call(dims, 0, None, None, None, 0) == _abi.WK_OK                  # empty batch: no-op
    assert _head_call(dims, 4, Y, P, WS, need, w=[0x10000, None]) == _abi.WK_ERR_INVALID_ARG
    assert _head_call(dims, 4, Y, P, WS, need, b=[0x20008, None]) == _abi.WK_ERR_INVALID_ARG  # misaligned bias
    assert _head_call((64, 12, 1), 4, Y, P, WS, need) == _abi.WK_ERR_UNSUPPORTED
    d, _dims = wk.HeadSpec(dims).make_desc()
    d.dtype = 9
    assert _head_call(dims, 4, Y, P, WS, need, desc=d) == _abi.WK_ERR_INVALID_ARG
    d, _dims = wk.HeadSpec(dims).make_desc()
    d.num_linear = 0
    assert _head_call(dims, 4, Y, P, WS, need, desc=d) == _abi.WK_ERR_INVALID_ARG
    d, _dims = wk.HeadSpec((64, 0, 1)).make_desc()
    assert _head_call(dims, 4, Y, P, WS, need, desc=d) == _abi.WK_ERR_INVALID_ARG


def test_fusion_workspace_and_argument_errors():
    lib = wk.load_library()
    spec = wk.FusionSpec(128, 160, 1024, 640)
    B = 7
    rows = B * 128
    # d_ff % 32 == 0: LN, FFN and residual are one kernel, so only Q lives in the workspace
    assert wk.fusion_workspace_size(spec, B) == al(rows * 160 * 2)
    # otherwise LN(Q) and silu(U) * U follow
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 160, 1024, 200), B) == \
        2 * al(rows * 160 * 2) + al(rows * 200 * 2)
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 160, 1024, 4128), B) == \
        2 * al(rows * 160 * 2) + al(rows * 4128 * 2)
    assert wk.fusion_workspace_size(wk.FusionSpec(120, 160, 1024, 640), B) == 0   # n % 16
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 48, 1024, 640), B) == 0    # d not a compiled width
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 160, 0, 640), B) == 0      # L >= 1
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 160, 64, 644), B) == 0     # d_ff % 8
    assert wk.fusion_workspace_size(wk.FusionSpec(128, 160, 64, 640, dtype="f32"), B) == 0
    need = wk.fusion_workspace_size(spec, B)
    desc = spec.make_desc()
    good = _abi.wk_fusion_weights(0x10000, None, None, None, 0x20000, None, 0x30000, None)
    HW, HS, HF, WS = 0x1000000, 0x2000000, 0x9000000, 0x10000000

    def call(hw=HW, hs=HS, hf=HF, ws=WS, nbytes=need, weights=good, batch=B):
        return lib.wukong_fusion_forward(ctypes.byref(desc), ctypes.byref(weights), batch, hw, hs, hf, ws, nbytes,
                                         None)
    assert call(nbytes=need - 1) == _abi.WK_ERR_WORKSPACE
    assert call(hw=None) == _abi.WK_ERR_INVALID_ARG
    assert call(hs=HS + 8) == _abi.WK_ERR_INVALID_ARG                 # misaligned
    assert call(hf=HW + 256) == _abi.WK_ERR_INVALID_ARG               # output overlaps the queries
    assert call(ws=HS) == _abi.WK_ERR_INVALID_ARG                     # workspace overlaps the sequence
    assert call(batch=-1) == _abi.WK_ERR_INVALID_ARG
    assert call(hw=None, hs=None, hf=None, ws=None, nbytes=0, batch=0) == _abi.WK_OK
    assert call(weights=_abi.wk_fusion_weights(0x10000, None, None, None, None, None, 0x30000, None)) == \
        _abi.WK_ERR_INVALID_ARG
    assert call(weights=_abi.wk_fusion_weights(0x10000, 0x20008, None, None, 0x20000, None, 0x30000, None)) == \
        _abi.WK_ERR_INVALID_ARG                                       # misaligned bias


def test_backward_sizes_and_support():
    B = 4096
    # saved activations: Fn, h_1, M
    assert wk.layer_saved_size(C1, B) == al(B * 4096 * 2) + al(B * 2048 * 2) + al(B * 64 * 160 * 2)
    lay = wk.saved_layout(C1, B)
    assert lay == {"fn": 0, "hidden": [al(B * 4096 * 2)], "m": al(B * 4096 * 2) + al(B * 2048 * 2)}
    assert wk.layer_backward_workspace_size(C1, B) > wk.layer_saved_size(C1, B)
    # the n = 256 layer takes the wide-layer backward: the saved buffer also holds Z (bf16) and Lc (fp32)
    fn, h1, h2, m = al(B * 12288 * 2), al(B * 4096 * 2), al(B * 4096 * 2), al(B * 128 * 160 * 2)
    assert wk.layer_saved_size(C2, B) == (fn + h1 + h2 + m + al(B * 48 * 160 * 2) + al(B * 128 * 160 * 4)
                                          + al(8 * 12 * 1024))  # + the rearranged [Phi; W_L]
    assert wk.layer_backward_workspace_size(C2, B) > 0
    C3 = wk.LayerSpec(512, 160, 96, 256, 256, (49152, 8192, 8192, 40960))
    assert wk.layer_saved_size(C3, 2048) > 0 and wk.layer_backward_workspace_size(C3, 2048) > 0
    # fp32 layers: unsupported
    f32 = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128), dtype="f32")
    assert wk.layer_backward_workspace_size(f32, B) == 0
    assert wk.layer_backward_workspace_size(wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128)), 37) > 0


def test_backward_argument_errors_launch_nothing():
    lib = wk.load_library()
    spec = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128))
    B = 37
    desc, _dims = spec.make_desc()
    wp = (ctypes.c_void_p * 2)(0x40000, 0x50000)
    weights = _abi.wk_layer_weights(0x10000, 0x20000, None, None, ctypes.cast(wp, ctypes.POINTER(ctypes.c_void_p)),
                                    None, None, None)
    gw = (ctypes.c_void_p * 2)(0x60000, 0x70000)
    grads = _abi.wk_layer_grads(0x80000, 0x90000, None, None, ctypes.cast(gw, ctypes.POINTER(ctypes.c_void_p)),
                                None, None, None)
    need = wk.layer_backward_workspace_size(spec, B)
    saved_need = wk.layer_saved_size(spec, B)
    X, SV, DY, DX, WS = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x10000000

    def call(x=X, saved=SV, dy=DY, dx=DX, ws=WS, nbytes=need, g=grads, batch=B):
        return lib.wukong_layer_backward(ctypes.byref(desc), ctypes.byref(weights), batch, x, saved, dy, dx,
                                         ctypes.byref(g) if g is not None else None, ws, nbytes, None)
    assert call(nbytes=need - 1) == _abi.WK_ERR_WORKSPACE
    assert call(x=None) == _abi.WK_ERR_INVALID_ARG
    assert call(dy=DY + 8) == _abi.WK_ERR_INVALID_ARG                 # misaligned
    assert call(dx=X + 256) == _abi.WK_ERR_INVALID_ARG                # dx overlaps x
    assert call(ws=SV) == _abi.WK_ERR_INVALID_ARG                     # workspace overlaps saved
    assert call(g=None) == _abi.WK_ERR_INVALID_ARG
    nogw = (ctypes.c_void_p * 2)(0x60000, None)
    bad = _abi.wk_layer_grads(0x80000, 0x90000, None, None, ctypes.cast(nogw, ctypes.POINTER(ctypes.c_void_p)),
                              None, None, None)
    assert call(g=bad) == _abi.WK_ERR_INVALID_ARG                     # every d_W_t is required
    assert call(batch=-1) == _abi.WK_ERR_INVALID_ARG
    assert call(x=None, saved=None, dy=None, dx=None, ws=None, nbytes=0, batch=0) == _abi.WK_OK
    f32, _d2 = wk.LayerSpec(16, 16, 4, 8, 8, (64, 64, 128), dtype="f32").make_desc()
    assert lib.wukong_layer_backward(ctypes.byref(f32), ctypes.byref(weights), B, X, SV, DY, DX, ctypes.byref(grads),
                                     WS, need, None) == _abi.WK_ERR_UNSUPPORTED
    # the training forward
    Y = 0x5000000
    assert lib.wukong_layer_forward_train(ctypes.byref(desc), ctypes.byref(weights), B, X, Y, SV, saved_need - 1,
                                          None) == _abi.WK_ERR_WORKSPACE
    assert lib.wukong_layer_forward_train(ctypes.byref(desc), ctypes.byref(weights), B, X, X + 512, SV, saved_need,
                                          None) == _abi.WK_ERR_INVALID_ARG
    assert lib.wukong_layer_forward_train(ctypes.byref(desc), ctypes.byref(weights), 0, None, None, None, 0,
                                          None) == _abi.WK_OK


def test_moe_sizes_and_argument_errors():
    lib = wk.load_library()
    E = [wk.LayerSpec(128, 160, 32, 16, 16, (4096, 2048, 2560)) for _ in range(4)]
    B = 64
    # every expert carries the output LayerNorm in its last Linear, so those run as one grouped launch
    # and each expert keeps its own workspace (Fn [B, n k] and h_1 [B, 2048]) until then
    al = lambda v: (v + 255) // 256 * 256
    assert wk.moe_workspace_size(wk.MoeSpec(E), B) == 4 * (al(B * 4096 * 2) + al(B * 2048 * 2))
    # otherwise (K % 64 != 0: residual LayerNorm kernel) the experts share the largest one
    E2 = [wk.LayerSpec(128, 160, 32, 16, 16, (4096, 2016, 2560)) for _ in range(4)]
    one = wk.layer_workspace_size(wk.LayerSpec(128, 160, 32, 16, 112, (4096, 2016, 2560)), B)
    # that stand-in layer (n_l = 112) takes the streamed FMB+LCB kernel and so also holds its
    # rearranged [Phi; W_L] (4 steps x 12 tiles of 1 KB); the experts (n_l = 16) take the resident one
    assert wk.moe_workspace_size(wk.MoeSpec(E2), B) == one - al(4 * 12 * 1024)
    assert wk.moe_workspace_size(wk.MoeSpec(E[:3]), B) == 0         # rows must add up to n
    bad_d = E[:3] + [wk.LayerSpec(128, 80, 32, 16, 16, (4096, 2048, 1280))]
    assert wk.moe_workspace_size(wk.MoeSpec(bad_d), B) == 0         # equal d
    units = [wk.LayerSpec(64, 8, 4, 16, 16, (256, 128)) for _ in range(2)]
    assert wk.moe_workspace_size(wk.MoeSpec(units), B) == 0         # bf16 experts need d % 16 == 0
    spec = wk.MoeSpec(E)
    desc, _keep = spec.make_desc()
    wp = [(ctypes.c_void_p * 2)(0x40000 + 0x1000 * e, 0x80000 + 0x1000 * e) for e in range(4)]
    ws_arr = (_abi.wk_layer_weights * 4)(*[
        _abi.wk_layer_weights(0x10000, 0x20000, None, None, ctypes.cast(wp[e], ctypes.POINTER(ctypes.c_void_p)),
                              None, None, None) for e in range(4)])
    need = wk.moe_workspace_size(spec, B)
    X, Y, WS = 0x1000000, 0x2000000, 0x10000000

    def call(x=X, y=Y, ws=WS, nbytes=need, gamma=None, beta=None, batch=B):
        return lib.wukong_moe_layer_forward(ctypes.byref(desc), ws_arr, gamma, beta, batch, x, y, ws, nbytes, None)
    assert call(nbytes=need - 1) == _abi.WK_ERR_WORKSPACE
    assert call(x=None) == _abi.WK_ERR_INVALID_ARG
    assert call(y=X + 512) == _abi.WK_ERR_INVALID_ARG                 # output overlaps input
    assert call(gamma=0x30008) == _abi.WK_ERR_INVALID_ARG             # misaligned gamma
    assert call(batch=-1) == _abi.WK_ERR_INVALID_ARG
    assert call(x=None, y=None, ws=None, nbytes=0, batch=0) == _abi.WK_OK
    desc.num_experts = 0
    assert call() == _abi.WK_ERR_INVALID_ARG


def test_stack_training_sizes_and_argument_errors():
    lib = wk.load_library()
    sp = wk.LayerSpec(40, 32, 20, 16, 24, (800, 96, 512))
    B = 37
    act = al(B * 40 * 32 * 2)
    one = wk.layer_saved_size(sp, B)
    assert wk.stack_saved_size([sp, sp], B) == one + act + one       # layer 1's input between the two
    assert wk.stack_backward_workspace_size([sp, sp], B) == 2 * act + wk.layer_backward_workspace_size(sp, B)
    assert wk.stack_saved_size([C2, C2], B) > 0                       # n = 256: the wide-layer backward
    C3 = wk.LayerSpec(512, 160, 96, 256, 256, (49152, 8192, 8192, 40960))
    assert wk.stack_saved_size([C3, C3], B) > 0                       # n = 512: the wide-layer backward
    pairs = [sp.make_desc() for _ in range(2)]
    descs = (_abi.wk_layer_desc * 2)(*[p[0] for p in pairs])
    wp = (ctypes.c_void_p * 2)(0x40000, 0x50000)
    w1 = _abi.wk_layer_weights(0x10000, 0x20000, None, None, ctypes.cast(wp, ctypes.POINTER(ctypes.c_void_p)),
                               None, None, None)
    warr = (_abi.wk_layer_weights * 2)(w1, w1)
    gw = (ctypes.c_void_p * 2)(0x60000, 0x70000)
    g1 = _abi.wk_layer_grads(0x80000, 0x90000, None, None, ctypes.cast(gw, ctypes.POINTER(ctypes.c_void_p)),
                             None, None, None)
    gmiss = (ctypes.c_void_p * 2)(0x60000, None)
    g_bad = _abi.wk_layer_grads(0x80000, 0x90000, None, None, ctypes.cast(gmiss, ctypes.POINTER(ctypes.c_void_p)),
                                None, None, None)
    need = wk.stack_backward_workspace_size([sp, sp], B)
    X, SV, DY, DX, WS = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x10000000

    def call(grads=(g1, g1), dx=DX, nbytes=need, batch=B):
        garr = (_abi.wk_layer_grads * 2)(*grads)
        return lib.wukong_stack_backward(2, descs, warr, batch, X, SV, DY, dx, garr, WS, nbytes, None)
    assert call(nbytes=need - 1) == _abi.WK_ERR_WORKSPACE
    assert call(grads=(g1, g_bad)) == _abi.WK_ERR_INVALID_ARG        # checked before layer 1 launches anything
    assert call(dx=DX + 8) == _abi.WK_ERR_INVALID_ARG                 # misaligned dx, used by the last call only
    assert call(dx=X + 256) == _abi.WK_ERR_INVALID_ARG                # dx overlaps x
    assert call(batch=0) == _abi.WK_OK
    saved = wk.stack_saved_size([sp, sp], B)
    assert lib.wukong_stack_forward_train(2, descs, warr, B, X, 0x5000000, SV, saved - 1, None) == \
        _abi.WK_ERR_WORKSPACE
