"""ctypes binding of libwukong's C ABI (include/wukong.h).

Argument marshalling only: torch supplies device memory and the stream, every
step of the layer runs in the HIP kernels behind the C ABI.  There is no CPU
fallback: if libwukong.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwukong.so")
_lib = None

F32, BF16 = 0, 1
WK_OK, WK_ERR_INVALID_ARG, WK_ERR_UNSUPPORTED, WK_ERR_WORKSPACE, WK_ERR_HIP = 0, 1, 2, 3, 4
KERNEL_FMB_LCB, KERNEL_MLP_LINEAR, KERNEL_RESIDUAL_LN, KERNEL_HEAD_LINEAR, KERNEL_HEAD_OUT = 1, 2, 3, 4, 5
KERNEL_FUSION_ATTN, KERNEL_FUSION_LINEAR, KERNEL_FUSION_LN = 6, 7, 8
KERNEL_BWD_OUT, KERNEL_BWD_TRANSPOSE, KERNEL_BWD_WGRAD, KERNEL_BWD_DGRAD, KERNEL_BWD_FMB, KERNEL_BWD_REDUCE = \
    9, 10, 11, 12, 13, 14
KERNEL_FUSION_FFN = 15
KERNEL_NAMES = {KERNEL_FMB_LCB: "fmb_lcb", KERNEL_MLP_LINEAR: "mlp_linear", KERNEL_RESIDUAL_LN: "residual_ln",
                KERNEL_HEAD_LINEAR: "head_linear", KERNEL_HEAD_OUT: "head_out",
                KERNEL_FUSION_ATTN: "fusion_attention", KERNEL_FUSION_LINEAR: "fusion_linear",
                KERNEL_FUSION_LN: "fusion_ln", KERNEL_BWD_OUT: "bwd_out", KERNEL_BWD_TRANSPOSE: "bwd_transpose",
                KERNEL_BWD_WGRAD: "bwd_wgrad", KERNEL_BWD_DGRAD: "bwd_dgrad", KERNEL_BWD_FMB: "bwd_fmb",
                KERNEL_BWD_REDUCE: "bwd_reduce", KERNEL_FUSION_FFN: "fusion_ffn"}
ABI_VERSION = 2


class wk_layer_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("d", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_f", ctypes.c_int32), ("n_l", ctypes.c_int32), ("num_linear", ctypes.c_int32),
                ("mlp_dims", ctypes.POINTER(ctypes.c_int32)), ("ln_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class wk_layer_weights(ctypes.Structure):
    _fields_ = [("phi", ctypes.c_void_p), ("w_l", ctypes.c_void_p),
                ("fm_ln_gamma", ctypes.c_void_p), ("fm_ln_beta", ctypes.c_void_p),
                ("mlp_w", ctypes.POINTER(ctypes.c_void_p)), ("mlp_b", ctypes.POINTER(ctypes.c_void_p)),
                ("out_ln_gamma", ctypes.c_void_p), ("out_ln_beta", ctypes.c_void_p)]


class wk_head_desc(ctypes.Structure):
    _fields_ = [("num_linear", ctypes.c_int32), ("dims", ctypes.POINTER(ctypes.c_int32)), ("dtype", ctypes.c_int32)]


class wk_head_weights(ctypes.Structure):
    _fields_ = [("w", ctypes.POINTER(ctypes.c_void_p)), ("b", ctypes.POINTER(ctypes.c_void_p))]


class wk_fusion_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("d", ctypes.c_int32), ("L", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class wk_fusion_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("w_f", "b_f", "ln_gamma", "ln_beta", "w_up", "b_up", "w_down", "b_down")]


class wk_layer_grads(ctypes.Structure):
    _fields_ = [("phi", ctypes.c_void_p), ("w_l", ctypes.c_void_p),
                ("fm_ln_gamma", ctypes.c_void_p), ("fm_ln_beta", ctypes.c_void_p),
                ("mlp_w", ctypes.POINTER(ctypes.c_void_p)), ("mlp_b", ctypes.POINTER(ctypes.c_void_p)),
                ("out_ln_gamma", ctypes.c_void_p), ("out_ln_beta", ctypes.c_void_p)]


class wk_moe_desc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("experts", ctypes.POINTER(wk_layer_desc))]


class wk_workspace_layout(ctypes.Structure):
    _fields_ = [("fn", ctypes.c_int64), ("m", ctypes.c_int64), ("num_hidden", ctypes.c_int32),
                ("hidden", ctypes.c_int64 * 8), ("fn_kblock_rows", ctypes.c_int64)]


# (name, restype, argtypes) of every exported symbol
_SIGNATURES = [
    ("wukong_abi_version", ctypes.c_int32, []),
    ("wukong_status_string", ctypes.c_char_p, [ctypes.c_int32]),
    ("wukong_layer_workspace_size", ctypes.c_size_t, [ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_layer_workspace_layout", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.c_int64, ctypes.POINTER(wk_workspace_layout)]),
    ("wukong_layer_forward", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_stack_workspace_size", ctypes.c_size_t,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_stack_forward", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_trace_create", ctypes.c_int32, [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]),
    ("wukong_trace_destroy", ctypes.c_int32, [ctypes.c_void_p]),
    ("wukong_trace_reset", ctypes.c_int32, [ctypes.c_void_p]),
    ("wukong_trace_count", ctypes.c_int32, [ctypes.c_void_p]),
    ("wukong_trace_get", ctypes.c_int32,
     [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_float)]),
    ("wukong_stack_forward_traced", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_fusion_workspace_size", ctypes.c_size_t, [ctypes.POINTER(wk_fusion_desc), ctypes.c_int64]),
    ("wukong_fusion_forward", ctypes.c_int32,
     [ctypes.POINTER(wk_fusion_desc), ctypes.POINTER(wk_fusion_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_fusion_forward_traced", ctypes.c_int32,
     [ctypes.POINTER(wk_fusion_desc), ctypes.POINTER(wk_fusion_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_moe_layer_workspace_size", ctypes.c_size_t, [ctypes.POINTER(wk_moe_desc), ctypes.c_int64]),
    ("wukong_moe_layer_forward", ctypes.c_int32,
     [ctypes.POINTER(wk_moe_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_moe_layer_forward_traced", ctypes.c_int32,
     [ctypes.POINTER(wk_moe_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_void_p, ctypes.c_void_p,
      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
      ctypes.c_void_p]),
    ("wukong_layer_saved_size", ctypes.c_size_t, [ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_layer_forward_train", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_layer_backward_workspace_size", ctypes.c_size_t, [ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_layer_backward", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(wk_layer_grads), ctypes.c_void_p,
      ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_layer_backward_traced", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(wk_layer_grads), ctypes.c_void_p,
      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_stack_saved_size", ctypes.c_size_t, [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_stack_forward_train", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_stack_backward_workspace_size", ctypes.c_size_t,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.c_int64]),
    ("wukong_stack_backward", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(wk_layer_grads),
      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_stack_backward_traced", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(wk_layer_grads),
      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_head_workspace_size", ctypes.c_size_t, [ctypes.POINTER(wk_head_desc), ctypes.c_int64]),
    ("wukong_head_forward", ctypes.c_int32,
     [ctypes.POINTER(wk_head_desc), ctypes.POINTER(wk_head_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("wukong_head_forward_traced", ctypes.c_int32,
     [ctypes.POINTER(wk_head_desc), ctypes.POINTER(wk_head_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_layer_forward_noalloc", ctypes.c_int32,
     [ctypes.POINTER(wk_layer_desc), ctypes.POINTER(wk_layer_weights), ctypes.c_int64, ctypes.c_void_p,
      ctypes.c_void_p, ctypes.c_void_p]),
    ("wukong_layer_forward_noalloc_max_workspace", ctypes.c_size_t, []),
    ("wukong_probe_mfma_bf16", ctypes.c_int32,
     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
]
EXPORTED_SYMBOLS = tuple(s[0] for s in _SIGNATURES)


class WukongError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libwukong.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m recommender_feature_interaction_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.wukong_abi_version() != ABI_VERSION:
        raise RuntimeError("libwukong.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().wukong_status_string(status).decode()


def _check(status: int, where: str):
    if status != WK_OK:
        raise WukongError(status, where)


# ------------------------------------------------------------------ layers
@dataclass(frozen=True)
class LayerSpec:
    n: int
    d: int
    k: int
    n_f: int
    n_l: int
    mlp: Tuple[int, ...]
    eps: float = 1e-5
    dtype: str = "bf16"  # "bf16" or "f32"

    @property
    def wk_dtype(self) -> int:
        return BF16 if self.dtype == "bf16" else F32

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def make_desc(self) -> Tuple[wk_layer_desc, object]:
        dims = (ctypes.c_int32 * len(self.mlp))(*self.mlp)
        desc = wk_layer_desc(self.n, self.d, self.k, self.n_f, self.n_l, len(self.mlp) - 1,
                             ctypes.cast(dims, ctypes.POINTER(ctypes.c_int32)), self.eps, self.wk_dtype)
        return desc, dims


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def to_device(a, dtype: str, device) -> torch.Tensor:
    """Host array (float32, or uint16 bf16 bit patterns) or tensor -> contiguous device tensor."""
    if isinstance(a, torch.Tensor):
        want = torch.bfloat16 if dtype == "bf16" else torch.float32
        if a.dtype != want:
            raise TypeError(f"expected {want}, got {a.dtype}")
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 host data must be uint16 bit patterns")
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype != np.float32:
        raise TypeError("f32 host data must be float32")
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """One layer's parameters resident in device memory, plus its C descriptors."""

    def __init__(self, spec: LayerSpec, phi, w_l, mlp_w: Sequence, mlp_b: Optional[Sequence] = None,
                 fm_gamma=None, fm_beta=None, out_gamma=None, out_beta=None, device="cuda"):
        dt = spec.dtype
        T = len(spec.mlp) - 1
        if len(mlp_w) != T or (mlp_b is not None and len(mlp_b) != T):
            raise ValueError("mlp_w / mlp_b must have one entry per Linear")
        cv = lambda a: None if a is None else to_device(a, dt, device)  # noqa: E731
        self.spec = spec
        self.phi, self.w_l = cv(phi), cv(w_l)
        self.fm_gamma, self.fm_beta = cv(fm_gamma), cv(fm_beta)
        self.out_gamma, self.out_beta = cv(out_gamma), cv(out_beta)
        self.mlp_w = [cv(w) for w in mlp_w]
        self.mlp_b = None if mlp_b is None else [cv(b) for b in mlp_b]
        n, d, k = spec.n, spec.d, spec.k
        expect = [("phi", self.phi, (k, n)), ("w_l", self.w_l, (spec.n_l, n)),
                  ("fm_gamma", self.fm_gamma, (n * k,)), ("fm_beta", self.fm_beta, (n * k,)),
                  ("out_gamma", self.out_gamma, (d,)), ("out_beta", self.out_beta, (d,))]
        for t in range(T):
            expect.append((f"mlp_w[{t}]", self.mlp_w[t], (spec.mlp[t + 1], spec.mlp[t])))
            if self.mlp_b is not None:
                expect.append((f"mlp_b[{t}]", self.mlp_b[t], (spec.mlp[t + 1],)))
        for name, t, shape in expect:
            if t is not None and tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        self.desc, self._dims = spec.make_desc()
        self._w_ptrs = (ctypes.c_void_p * T)(*[w.data_ptr() for w in self.mlp_w])
        self._b_ptrs = None if self.mlp_b is None else (ctypes.c_void_p * T)(*[_ptr(b) for b in self.mlp_b])
        self.weights = wk_layer_weights(
            _ptr(self.phi), _ptr(self.w_l), _ptr(self.fm_gamma), _ptr(self.fm_beta),
            ctypes.cast(self._w_ptrs, ctypes.POINTER(ctypes.c_void_p)),
            None if self._b_ptrs is None else ctypes.cast(self._b_ptrs, ctypes.POINTER(ctypes.c_void_p)),
            _ptr(self.out_gamma), _ptr(self.out_beta))

    @classmethod
    def from_host(cls, spec: LayerSpec, hw, device="cuda") -> "DeviceLayer":
        """From an object with phi, w_l, fm_gamma, fm_beta, mlp_w, mlp_b, out_gamma, out_beta."""
        return cls(spec, hw.phi, hw.w_l, hw.mlp_w, hw.mlp_b, hw.fm_gamma, hw.fm_beta,
                   hw.out_gamma, hw.out_beta, device=device)

    def nbytes(self) -> int:
        ts = [self.phi, self.w_l, self.fm_gamma, self.fm_beta, self.out_gamma, self.out_beta, *self.mlp_w]
        ts += self.mlp_b or []
        return int(sum(t.numel() * t.element_size() for t in ts if t is not None))


def _stream_handle(stream, *tensors) -> Optional[int]:
    """The HIP stream to launch on.  When it is not the current stream, it first
    waits for the current stream's work (which includes making the tensors this
    call allocated), and every tensor the launches touch is marked as used on it,
    so the caching allocator does not hand their memory to other work before the
    launches have finished with it."""
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        return cur.cuda_stream
    stream.wait_stream(cur)
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            t.record_stream(stream)
    return stream.cuda_stream


def _descs(layers: Sequence[DeviceLayer]):
    descs = (wk_layer_desc * len(layers))(*[l.desc for l in layers])
    ws = (wk_layer_weights * len(layers))(*[l.weights for l in layers])
    return descs, ws


def layer_workspace_size(spec: LayerSpec, batch: int) -> int:
    desc, _dims = spec.make_desc()
    return int(load_library().wukong_layer_workspace_size(ctypes.byref(desc), batch))


def stack_workspace_size(specs: Sequence[LayerSpec], batch: int) -> int:
    pairs = [s.make_desc() for s in specs]
    descs = (wk_layer_desc * len(specs))(*[p[0] for p in pairs])
    return int(load_library().wukong_stack_workspace_size(len(specs), descs, batch))


def workspace_layout(spec: LayerSpec, batch: int) -> dict:
    desc, _dims = spec.make_desc()
    out = wk_workspace_layout()
    _check(load_library().wukong_layer_workspace_layout(ctypes.byref(desc), batch, ctypes.byref(out)),
           "wukong_layer_workspace_layout")
    return {"fn": out.fn, "m": out.m,
            "hidden": [out.hidden[i] for i in range(min(out.num_hidden, 8))],
            "fn_kblock_rows": out.fn_kblock_rows}


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _check_x(x: torch.Tensor, spec: LayerSpec) -> int:
    if not x.is_cuda or x.dtype != spec.torch_dtype or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous {spec.torch_dtype} CUDA tensor")
    if x.dim() != 3 or x.shape[1] != spec.n or x.shape[2] != spec.d:
        raise ValueError(f"x must be [batch, {spec.n}, {spec.d}], got {tuple(x.shape)}")
    return x.shape[0]


def layer_forward(x: torch.Tensor, layer: DeviceLayer, y: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One Wukong layer on x [batch, n, d]; returns y [batch, n, d]."""
    lib = load_library()
    B = _check_x(x, layer.spec)
    y = torch.empty_like(x) if y is None else y
    need = layer_workspace_size(layer.spec, B)
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    st = lib.wukong_layer_forward(ctypes.byref(layer.desc), ctypes.byref(layer.weights), B, x.data_ptr(),
                                  y.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream, x, y, workspace))
    _check(st, "wukong_layer_forward")
    return y


def layer_forward_noalloc(x: torch.Tensor, layer: DeviceLayer, y: torch.Tensor, stream=None) -> torch.Tensor:
    """One Wukong layer on x [batch, n, d] into the caller's y, with the library's static
    workspace (wukong_layer_forward_noalloc: nothing is allocated by the call or here)."""
    lib = load_library()
    B = _check_x(x, layer.spec)
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous() or not y.is_cuda:
        raise ValueError("y must be a contiguous CUDA tensor shaped like x")
    st = lib.wukong_layer_forward_noalloc(ctypes.byref(layer.desc), ctypes.byref(layer.weights), B, x.data_ptr(),
                                          y.data_ptr(), _stream_handle(stream, x, y))
    _check(st, "wukong_layer_forward_noalloc")
    return y


def noalloc_max_workspace() -> int:
    return int(load_library().wukong_layer_forward_noalloc_max_workspace())


# ------------------------------------------------------------------ mixture of experts
class MoeSpec:
    """A mixture-of-experts layer: one LayerSpec per expert (equal n, d, dtype, eps;
    n_f / n_l are the expert's own FMB / LCB row counts, adding up to n over the experts)."""

    def __init__(self, experts: Sequence[LayerSpec]):
        self.experts = tuple(experts)

    def make_desc(self):
        pairs = [e.make_desc() for e in self.experts]
        arr = (wk_layer_desc * len(pairs))(*[p[0] for p in pairs])
        desc = wk_moe_desc(len(pairs), ctypes.cast(arr, ctypes.POINTER(wk_layer_desc)))
        return desc, (arr, pairs)


class DeviceMoe:
    """Experts' parameters (DeviceLayer each) plus the layer's output LayerNorm, with the C descriptors."""

    def __init__(self, spec: MoeSpec, experts: Sequence[DeviceLayer], out_gamma=None, out_beta=None,
                 device="cuda"):
        if len(experts) != len(spec.experts):
            raise ValueError("one DeviceLayer per expert")
        dt = spec.experts[0].dtype
        self.spec = spec
        self.experts = list(experts)
        self.out_gamma = None if out_gamma is None else to_device(out_gamma, dt, device)
        self.out_beta = None if out_beta is None else to_device(out_beta, dt, device)
        self.desc, self._keep = spec.make_desc()
        self.weights = (wk_layer_weights * len(experts))(*[e.weights for e in experts])


def moe_workspace_size(spec: MoeSpec, batch: int) -> int:
    desc, _keep = spec.make_desc()
    return int(load_library().wukong_moe_layer_workspace_size(ctypes.byref(desc), batch))


def moe_forward(x: torch.Tensor, moe: DeviceMoe, y: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None, trace: "Trace" = None) -> torch.Tensor:
    """One mixture-of-experts layer on x [batch, n, d]; returns y [batch, n, d]."""
    lib = load_library()
    B = _check_x(x, moe.spec.experts[0])
    y = torch.empty_like(x) if y is None else y
    need = moe_workspace_size(moe.spec, B)
    if need == 0:
        raise WukongError(WK_ERR_UNSUPPORTED, "wukong_moe_layer_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    args = [ctypes.byref(moe.desc), moe.weights, _ptr(moe.out_gamma), _ptr(moe.out_beta), B, x.data_ptr(),
            y.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(stream, x, y, workspace)]
    if trace is None:
        _check(lib.wukong_moe_layer_forward(*args), "wukong_moe_layer_forward")
    else:
        _check(lib.wukong_moe_layer_forward_traced(*args, trace.handle), "wukong_moe_layer_forward_traced")
    return y


# ------------------------------------------------------------------ training: one layer's backward
def layer_saved_size(spec: LayerSpec, batch: int) -> int:
    desc, _dims = spec.make_desc()
    return int(load_library().wukong_layer_saved_size(ctypes.byref(desc), batch))


def layer_backward_workspace_size(spec: LayerSpec, batch: int) -> int:
    desc, _dims = spec.make_desc()
    return int(load_library().wukong_layer_backward_workspace_size(ctypes.byref(desc), batch))


def saved_layout(spec: LayerSpec, batch: int) -> dict:
    """Byte offsets of Fn, h_1 .. h_{T-1} and M in a training forward's saved buffer."""
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    off = 0
    out = {"fn": 0}
    off += al(batch * spec.n * spec.k * 2)
    out["hidden"] = []
    for t in range(1, len(spec.mlp) - 1):
        out["hidden"].append(off)
        off += al(batch * spec.mlp[t] * 2)
    out["m"] = off
    return out


def layer_forward_train(x: torch.Tensor, layer: DeviceLayer, y: Optional[torch.Tensor] = None,
                        saved: Optional[torch.Tensor] = None, stream=None):
    """Training forward of one bf16 layer: returns (y, saved), saved holding Fn, h_t and M."""
    lib = load_library()
    B = _check_x(x, layer.spec)
    y = torch.empty_like(x) if y is None else y
    need = layer_saved_size(layer.spec, B)
    if need == 0:
        raise WukongError(WK_ERR_UNSUPPORTED, "wukong_layer_saved_size")
    if saved is None:
        saved = alloc_workspace(need, x.device)
    st = lib.wukong_layer_forward_train(ctypes.byref(layer.desc), ctypes.byref(layer.weights), B, x.data_ptr(),
                                        y.data_ptr(), saved.data_ptr(), saved.numel() * saved.element_size(),
                                        _stream_handle(stream, x, y, saved))
    _check(st, "wukong_layer_forward_train")
    return y, saved


class LayerGrads:
    """fp32 device gradients of one layer's weights (the C ABI overwrites them).

    zero=True fills them with zeros: the gradients of an empty batch, for which
    the C ABI launches nothing."""

    def __init__(self, layer: DeviceLayer, affine: bool = True, bias: bool = True, zero: bool = False):
        spec = layer.spec
        dev = layer.phi.device
        alloc = torch.zeros if zero else torch.empty
        z = lambda *shape: alloc(*shape, dtype=torch.float32, device=dev)  # noqa: E731
        n, d, k = spec.n, spec.d, spec.k
        T = len(spec.mlp) - 1
        self.phi, self.w_l = z(k, n), z(spec.n_l, n)
        self.fm_gamma = z(n * k) if affine else None
        self.fm_beta = z(n * k) if affine else None
        self.out_gamma = z(d) if affine else None
        self.out_beta = z(d) if affine else None
        self.mlp_w = [z(spec.mlp[t + 1], spec.mlp[t]) for t in range(T)]
        self.mlp_b = [z(spec.mlp[t + 1]) for t in range(T)] if bias else None
        self._w = (ctypes.c_void_p * T)(*[w.data_ptr() for w in self.mlp_w])
        self._b = None if self.mlp_b is None else (ctypes.c_void_p * T)(*[b.data_ptr() for b in self.mlp_b])
        self.c = wk_layer_grads(
            _ptr(self.phi), _ptr(self.w_l), _ptr(self.fm_gamma), _ptr(self.fm_beta),
            ctypes.cast(self._w, ctypes.POINTER(ctypes.c_void_p)),
            None if self._b is None else ctypes.cast(self._b, ctypes.POINTER(ctypes.c_void_p)),
            _ptr(self.out_gamma), _ptr(self.out_beta))

    def as_dict(self) -> dict:
        return {"phi": self.phi, "w_l": self.w_l, "fm_gamma": self.fm_gamma, "fm_beta": self.fm_beta,
                "mlp_w": self.mlp_w, "mlp_b": self.mlp_b, "out_gamma": self.out_gamma, "out_beta": self.out_beta}

    def tensors(self) -> list:
        """Every gradient tensor (the backward writes all of them)."""
        ts = [self.phi, self.w_l, self.fm_gamma, self.fm_beta, self.out_gamma, self.out_beta, *self.mlp_w]
        return [t for t in ts + list(self.mlp_b or []) if t is not None]


def layer_backward(x: torch.Tensor, saved: torch.Tensor, dy: torch.Tensor, layer: DeviceLayer,
                   grads: Optional[LayerGrads] = None, dx: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None, trace: "Trace" = None):
    """Backward of one bf16 layer: returns (dx, grads) from x, the training forward's saved buffer and dy.

    With an empty batch, gradients allocated here are zero; grads passed in are left untouched."""
    lib = load_library()
    B = _check_x(x, layer.spec)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise ValueError("dy must be contiguous and shaped like x")
    grads = LayerGrads(layer, zero=B == 0) if grads is None else grads
    dx = torch.empty_like(x) if dx is None else dx
    need = layer_backward_workspace_size(layer.spec, B)
    if need == 0:
        raise WukongError(WK_ERR_UNSUPPORTED, "wukong_layer_backward_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    args = [ctypes.byref(layer.desc), ctypes.byref(layer.weights), B, x.data_ptr(), saved.data_ptr(),
            dy.data_ptr(), dx.data_ptr(), ctypes.byref(grads.c), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(),
            _stream_handle(stream, x, saved, dy, dx, workspace, *grads.tensors())]
    if trace is None:
        _check(lib.wukong_layer_backward(*args), "wukong_layer_backward")
    else:
        _check(lib.wukong_layer_backward_traced(*args, trace.handle), "wukong_layer_backward_traced")
    return dx, grads


def stack_saved_size(specs: Sequence[LayerSpec], batch: int) -> int:
    pairs = [sp.make_desc() for sp in specs]
    descs = (wk_layer_desc * len(specs))(*[p[0] for p in pairs])
    return int(load_library().wukong_stack_saved_size(len(specs), descs, batch))


def stack_backward_workspace_size(specs: Sequence[LayerSpec], batch: int) -> int:
    pairs = [sp.make_desc() for sp in specs]
    descs = (wk_layer_desc * len(specs))(*[p[0] for p in pairs])
    return int(load_library().wukong_stack_backward_workspace_size(len(specs), descs, batch))


def stack_forward_train(x: torch.Tensor, layers: Sequence[DeviceLayer], y: Optional[torch.Tensor] = None,
                        saved: Optional[torch.Tensor] = None, stream=None):
    """Training forward of a bf16 stack: returns (y, saved), saved holding every layer's input and activations."""
    lib = load_library()
    B = _check_x(x, layers[0].spec)
    y = torch.empty_like(x) if y is None else y
    need = stack_saved_size([l.spec for l in layers], B)
    if need == 0:
        raise WukongError(WK_ERR_UNSUPPORTED, "wukong_stack_saved_size")
    if saved is None:
        saved = alloc_workspace(need, x.device)
    descs, ws = _descs(layers)
    _check(lib.wukong_stack_forward_train(len(layers), descs, ws, B, x.data_ptr(), y.data_ptr(), saved.data_ptr(),
                                          saved.numel() * saved.element_size(), _stream_handle(stream, x, y, saved)),
           "wukong_stack_forward_train")
    return y, saved


def stack_backward(x: torch.Tensor, saved: torch.Tensor, dy: torch.Tensor, layers: Sequence[DeviceLayer],
                   grads: Optional[Sequence[LayerGrads]] = None, dx: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None, trace: "Trace" = None):
    """Backward of a bf16 stack: returns (dx, [LayerGrads per layer]).

    With an empty batch, gradients allocated here are zero; grads passed in are left untouched."""
    lib = load_library()
    B = _check_x(x, layers[0].spec)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise ValueError("dy must be contiguous and shaped like x")
    grads = [LayerGrads(l, zero=B == 0) for l in layers] if grads is None else list(grads)
    dx = torch.empty_like(x) if dx is None else dx
    need = stack_backward_workspace_size([l.spec for l in layers], B)
    if need == 0:
        raise WukongError(WK_ERR_UNSUPPORTED, "wukong_stack_backward_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    descs, ws = _descs(layers)
    garr = (wk_layer_grads * len(grads))(*[g.c for g in grads])
    args = [len(layers), descs, ws, B, x.data_ptr(), saved.data_ptr(), dy.data_ptr(), dx.data_ptr(), garr,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(stream, x, saved, dy, dx, workspace, *[t for g in grads for t in g.tensors()])]
    if trace is None:
        _check(lib.wukong_stack_backward(*args), "wukong_stack_backward")
    else:
        _check(lib.wukong_stack_backward_traced(*args, trace.handle), "wukong_stack_backward_traced")
    return dx, grads


class Trace:
    """Per-kernel HIP-event timing of stack_forward calls (see wukong_trace_*)."""

    def __init__(self, capacity: int = 4096):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.wukong_trace_create(capacity, ctypes.byref(h)), "wukong_trace_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def reset(self):
        _check(self._lib.wukong_trace_reset(self._h), "wukong_trace_reset")

    def records(self) -> List[dict]:
        out = []
        kind, layer, index = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        wgs, ms = ctypes.c_int64(), ctypes.c_float()
        for i in range(self._lib.wukong_trace_count(self._h)):
            _check(self._lib.wukong_trace_get(self._h, i, ctypes.byref(kind), ctypes.byref(layer),
                                              ctypes.byref(index), ctypes.byref(wgs), ctypes.byref(ms)),
                   "wukong_trace_get")
            out.append({"kernel": KERNEL_NAMES.get(kind.value, str(kind.value)), "layer": layer.value,
                        "index": index.value, "workgroups": wgs.value, "ms": ms.value})
        return out

    def close(self):
        if self._h is not None:
            self._lib.wukong_trace_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stack_forward(x: torch.Tensor, layers: Sequence[DeviceLayer], y: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  trace: Optional[Trace] = None) -> torch.Tensor:
    """l stacked Wukong layers on x [batch, n, d]; returns y [batch, n, d]."""
    lib = load_library()
    B = _check_x(x, layers[0].spec)
    y = torch.empty_like(x) if y is None else y
    descs, ws = _descs(layers)
    need = int(lib.wukong_stack_workspace_size(len(layers), descs, B))
    if workspace is None:
        workspace = alloc_workspace(need, x.device)
    args = (len(layers), descs, ws, B, x.data_ptr(), y.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(stream, x, y, workspace))
    if trace is None:
        st = lib.wukong_stack_forward(*args)
    else:
        st = lib.wukong_stack_forward_traced(*args, trace.handle)
    _check(st, "wukong_stack_forward")
    return y


# ------------------------------------------------------------------ prediction head
@dataclass(frozen=True)
class HeadSpec:
    """The top MLP after the stack: dims = (n*d, m_1, ..., m_T)."""
    dims: Tuple[int, ...]
    dtype: str = "bf16"

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def make_desc(self) -> Tuple[wk_head_desc, object]:
        dims = (ctypes.c_int32 * len(self.dims))(*self.dims)
        desc = wk_head_desc(len(self.dims) - 1, ctypes.cast(dims, ctypes.POINTER(ctypes.c_int32)),
                            BF16 if self.dtype == "bf16" else F32)
        return desc, dims


class DeviceHead:
    """The head's weights resident in device memory, plus its C descriptors."""

    def __init__(self, spec: HeadSpec, w: Sequence, b: Optional[Sequence] = None, device="cuda"):
        T = len(spec.dims) - 1
        if len(w) != T or (b is not None and len(b) != T):
            raise ValueError("w / b must have one entry per Linear")
        cv = lambda a: None if a is None else to_device(a, spec.dtype, device)  # noqa: E731
        self.spec = spec
        self.w = [cv(x) for x in w]
        self.b = None if b is None else [cv(x) for x in b]
        for t in range(T):
            if tuple(self.w[t].shape) != (spec.dims[t + 1], spec.dims[t]):
                raise ValueError(f"w[{t}] has shape {tuple(self.w[t].shape)}, expected "
                                 f"{(spec.dims[t + 1], spec.dims[t])}")
            if self.b is not None and self.b[t] is not None and tuple(self.b[t].shape) != (spec.dims[t + 1],):
                raise ValueError(f"b[{t}] has shape {tuple(self.b[t].shape)}")
        self.desc, self._dims = spec.make_desc()
        self._w_ptrs = (ctypes.c_void_p * T)(*[x.data_ptr() for x in self.w])
        self._b_ptrs = None if self.b is None else (ctypes.c_void_p * T)(*[_ptr(x) for x in self.b])
        self.weights = wk_head_weights(ctypes.cast(self._w_ptrs, ctypes.POINTER(ctypes.c_void_p)),
                                       None if self._b_ptrs is None
                                       else ctypes.cast(self._b_ptrs, ctypes.POINTER(ctypes.c_void_p)))


def head_workspace_size(spec: HeadSpec, batch: int) -> int:
    desc, _dims = spec.make_desc()
    return int(load_library().wukong_head_workspace_size(ctypes.byref(desc), batch))


def head_forward(y: torch.Tensor, head: DeviceHead, prob: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 trace: Optional[Trace] = None) -> torch.Tensor:
    """Prediction head on a layer output y [batch, n, d] (or [batch, n*d]); returns fp32 [batch, m_T]."""
    lib = load_library()
    spec = head.spec
    if not y.is_cuda or y.dtype != spec.torch_dtype or not y.is_contiguous():
        raise ValueError(f"y must be a contiguous {spec.torch_dtype} CUDA tensor")
    B = y.shape[0]
    if y.numel() != B * spec.dims[0]:
        raise ValueError(f"y must hold {spec.dims[0]} features per example")
    prob = torch.empty((B, spec.dims[-1]), dtype=torch.float32, device=y.device) if prob is None else prob
    need = head_workspace_size(spec, B)
    if workspace is None:
        workspace = alloc_workspace(need, y.device)
    args = (ctypes.byref(head.desc), ctypes.byref(head.weights), B, y.data_ptr(), prob.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(stream, y, prob, workspace))
    if trace is None:
        st = lib.wukong_head_forward(*args)
    else:
        st = lib.wukong_head_forward_traced(*args, trace.handle)
    _check(st, "wukong_head_forward")
    return prob


# ------------------------------------------------------------------ WHALE fusion step
@dataclass(frozen=True)
class FusionSpec:
    """WHALE's fusion step: n query tokens (rows of H_w) of width d, L sequence positions, SwiGLU width d_ff."""
    n: int
    d: int
    L: int
    d_ff: int
    ln_eps: float = 1e-5
    dtype: str = "bf16"

    def make_desc(self) -> wk_fusion_desc:
        return wk_fusion_desc(self.n, self.d, self.L, self.d_ff, self.ln_eps, BF16 if self.dtype == "bf16" else F32)


class DeviceFusion:
    """The fusion step's weights resident in device memory (None = absent bias / identity LN affine)."""

    def __init__(self, spec: FusionSpec, w_f, w_up, w_down, b_f=None, ln_gamma=None, ln_beta=None, b_up=None,
                 b_down=None, device="cuda"):
        cv = lambda a: None if a is None else to_device(a, spec.dtype, device)  # noqa: E731
        self.spec = spec
        self.w_f, self.w_up, self.w_down = cv(w_f), cv(w_up), cv(w_down)
        self.b_f, self.ln_gamma, self.ln_beta, self.b_up, self.b_down = (cv(b_f), cv(ln_gamma), cv(ln_beta),
                                                                          cv(b_up), cv(b_down))
        d, dff = spec.d, spec.d_ff
        for name, t, shape in (("w_f", self.w_f, (d, 2 * d)), ("w_up", self.w_up, (dff, d)),
                               ("w_down", self.w_down, (d, dff)), ("b_f", self.b_f, (d,)),
                               ("ln_gamma", self.ln_gamma, (d,)), ("ln_beta", self.ln_beta, (d,)),
                               ("b_up", self.b_up, (dff,)), ("b_down", self.b_down, (d,))):
            if t is not None and tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        self.desc = spec.make_desc()
        self.weights = wk_fusion_weights(*[_ptr(t) for t in (self.w_f, self.b_f, self.ln_gamma, self.ln_beta,
                                                              self.w_up, self.b_up, self.w_down, self.b_down)])


def fusion_workspace_size(spec: FusionSpec, batch: int) -> int:
    desc = spec.make_desc()
    return int(load_library().wukong_fusion_workspace_size(ctypes.byref(desc), batch))


def fusion_forward(hw: torch.Tensor, hs: torch.Tensor, fusion: DeviceFusion, hf: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   trace: Optional[Trace] = None) -> torch.Tensor:
    """H_f [batch, n, d] from the Wukong output hw [batch, n, d] and the sequence output hs [batch, L, d]."""
    lib = load_library()
    spec = fusion.spec
    for name, t, per in (("hw", hw, spec.n * spec.d), ("hs", hs, spec.L * spec.d)):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a bf16 CUDA tensor")
        if not t.is_contiguous() or t.numel() != t.shape[0] * per:
            raise ValueError(f"{name} must be contiguous with {per} elements per example")
    B = hw.shape[0]
    if hs.shape[0] != B:
        raise ValueError("hw and hs need the same batch")
    hf = torch.empty((B, spec.n, spec.d), dtype=torch.bfloat16, device=hw.device) if hf is None else hf
    if workspace is None:
        workspace = alloc_workspace(fusion_workspace_size(spec, B), hw.device)
    args = (ctypes.byref(fusion.desc), ctypes.byref(fusion.weights), B, hw.data_ptr(), hs.data_ptr(),
            hf.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(stream, hw, hs, hf, workspace))
    if trace is None:
        st = lib.wukong_fusion_forward(*args)
    else:
        st = lib.wukong_fusion_forward_traced(*args, trace.handle)
    _check(st, "wukong_fusion_forward")
    return hf


# ------------------------------------------------------------------ measurement aid
def probe_mfma_bf16(blocks: int = 1024, iters: int = 4000, reps: int = 3, device="cuda") -> float:
    """On-chip bf16 MFMA rate in TFLOP/s (wukong_probe_mfma_bf16): 8 waves per
    workgroup, operands that change between consecutive instructions."""
    lib = load_library()
    g = torch.Generator(device="cpu").manual_seed(7)
    ops = (torch.rand(16 * 64 * 8, generator=g) * 2 - 1).to(torch.bfloat16).to(device)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=device)
    st = torch.cuda.current_stream()
    _check(lib.wukong_probe_mfma_bf16(ops.data_ptr(), sink.data_ptr(), blocks, 8, st.cuda_stream), "probe")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        _check(lib.wukong_probe_mfma_bf16(ops.data_ptr(), sink.data_ptr(), blocks, iters, st.cuda_stream), "probe")
    e1.record(st)
    torch.cuda.synchronize()
    flops = reps * blocks * 8.0 * iters * 16 * 16384
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
