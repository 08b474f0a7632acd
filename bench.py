"""Throughput of the Wukong layer-stack forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config stack8_n256]
                    [--sections stack8_n512,smalld_n720,layer_d160]

A step is one forward pass of the whole stack (FMB+LCB kernel, every MLP
Linear, the residual LayerNorm of the FMB rows, for every layer) over one
batch of seeded synthetic input that is already resident in HBM.  The
headline workload is the 8-layer n = 256 stack (B = 16384, d = 160).  W
untimed warm-up steps, then K timed steps bracketed by device
synchronisation give `value`.  Each step is also timed between HIP events on
the launch stream ("step_ms_events": median, min, p90, mean), replayed from a
HIP graph, and timed with 512 MB written between steps (no input or weight
left in L2 or the last-level cache: "cold_cache_ms_per_step").  A pass with
HIP events recorded by the library around each kernel launch gives the
per-kernel durations and the kernel with the largest share of the step,
reported against its roofline.  "step_roofline_frac" is the sum over kernels
of max(FLOPs / peak, bytes / HBM bandwidth) divided by the measured step.

Two on-box ceilings are measured first: a 256 MiB device copy
("copy_gbps_measured") and the bf16 MFMA rate on changing operands
("mfma_tflops_measured", the library's probe kernel).

The other workloads (the n = 512 stack, the n = 720 small-d layer, the
d = 160 layer) are measured the same way in the same run and reported under
"workloads"; the n = 720 layer's "memory_bound_kernels" gives the
algorithmic bytes of FMB+LCB (and the residual LayerNorm where it runs) over
their time.  The prediction head and WHALE's fusion step are timed on the
headline's output; the training step (forward + backward of the layer or
the whole stack) on every workload; the fusion step and the
mixture-of-experts layer on the single-layer workloads.  None of
these is part of `value`.  The CPU oracle is timed on a bounded sample of the
headline workload on this host as a reference baseline (fp64, and the same
steps in fp32).

Prints one JSON line.

    python bench.py --copy-calibration BYTES

instead runs a plain device-to-device copy of BYTES bytes a few times (the
reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters) and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (AMD specification)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "Wukong stack fwd examples/sec; achieved TFLOP/s as % of bf16 MFMA peak"
PROFILE_DIR = os.path.join(ROOT, "profiles")
# sources whose SHA-256 (over their concatenation) a traffic record in profiles/ must match
KERNEL_SOURCES = {
    "fmb_lcb": ("fmb_lcb.hip", "fmb_lcb_stream.hip", "fmb_lcb_units.hip", "linear_bf16.hip"),
    "mlp_linear": ("linear_bf16.hip",),
    "residual_ln": ("resid_ln.hip",),
    "head_linear": ("linear_bf16.hip",),
    "head_out": ("head.hip",),
    "fusion_attention": ("whale_fusion.hip",),
    "fusion_linear": ("linear_bf16.hip",),
    "fusion_ln": ("whale_fusion.hip",),
    "fusion_ffn": ("whale_fusion.hip",),
    "bwd_out": ("wukong_backward.hip", "wukong_backward_wide.hip"),
    "bwd_fmb": ("wukong_backward.hip", "wukong_backward_wide.hip"),
    "bwd_transpose": ("wukong_backward.hip", "wukong_backward_wide.hip"),
    "bwd_reduce": ("wukong_backward.hip", "wukong_backward_wide.hip"),
    "bwd_wgrad": ("linear_bf16.hip",),
    "bwd_dgrad": ("linear_bf16.hip",),
}


def kernel_accounting(cfg, fused_layers=()):
    """Algorithmic FLOPs and HBM bytes per launch of each kernel of each layer.
    In the layers listed in `fused_layers` the last Linear applies the output
    LayerNorm itself: it reads the FMB rows of X and writes those of Y instead
    of writing M, and there is no residual LayerNorm kernel."""
    es = 2 if cfg.dtype == "bf16" else 4
    B = cfg.batch
    out = {}
    for li, s in enumerate(cfg.layers):
        n, d, k, n_f, n_l = s.n, s.d, s.k, s.n_f, s.n_l
        out[("fmb_lcb", li, 0)] = {
            "flops": B * (2 * (k + n_l) * n * d + 2 * n * d * k),
            # X in; Fn and the LCB rows of Y out; [Phi; W_L] once
            "bytes": B * (n * d + n * k + n_l * d) * es + (k + n_l) * n * es,
        }
        T = len(s.mlp) - 1
        for t, (a, b) in enumerate(zip(s.mlp[:-1], s.mlp[1:])):
            fused = li in fused_layers and t == T - 1
            out[("mlp_linear", li, t)] = {
                "flops": 2 * B * a * b,
                # A, W, bias in; C out (fused: also the FMB rows of X in, C is those of Y)
                "bytes": (B * a + a * b + B * b + b + (B * b if fused else 0)) * es,
                "shape": [B, b, a],
            }
        if li in fused_layers:
            continue
        out[("residual_ln", li, 0)] = {
            "flops": 0,
            # M and the FMB rows of X in, FMB rows of Y out
            "bytes": 3 * B * n_f * d * es,
        }
    return out


def head_accounting(dims, batch, es):
    """Algorithmic FLOPs and HBM bytes per launch of the prediction head's kernels."""
    out = {}
    T = len(dims) - 1
    for t, (a, b) in enumerate(zip(dims[:-1], dims[1:])):
        if t + 1 < T:  # hidden Linear + ReLU on the GEMM: A, W, bias in, C out
            out[("head_linear", 0, t)] = {"flops": 2 * batch * a * b,
                                          "bytes": (batch * a + a * b + b + batch * b) * es}
        else:  # last Linear + logistic: A, W, bias in, fp32 probabilities out
            out[("head_out", 0, 0)] = {"flops": 2 * batch * a * b,
                                       "bytes": (batch * a + a * b + b) * es + batch * b * 4}
    return out


def roofline_of(kernel, ac, avg_ms, dtype, workload, traffic_index=None):
    """Place one kernel against its roofline: MFMA (or fp32 ALU) when its
    arithmetic intensity is above the ridge point, HBM otherwise."""
    avg_s = avg_ms * 1e-3
    traffic = read_traffic(kernel["kernel"], kernel["index"], workload)
    label = f"{kernel['kernel']}[layer {kernel['layer']}, index {kernel['index']}]"
    if ac["flops"] > 0 and ac["flops"] / ac["bytes"] > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
        ach = ac["flops"] / avg_s / 1e12
        return {"bound": "mfma" if dtype == "bf16" else "alu", "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic, "kernel": label,
                "algorithmic_flops_per_launch": ac["flops"], "avg_ms": avg_ms}
    ach = ac["bytes"] / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic, "kernel": label,
            "algorithmic_bytes_per_launch": ac["bytes"], "avg_ms": avg_ms}


def summarize_trace(recs, acct, per_step_ms, steps):
    """Average each (kernel, layer, index) over the trace; return the rows and
    the dominant one (largest total time over kernels of one kind and index)."""
    agg = {}
    for r in recs:
        key = (r["kernel"], r["layer"], r["index"])
        a = agg.setdefault(key, {"ms": 0.0, "count": 0, "workgroups": r["workgroups"]})
        a["ms"] += r["ms"]
        a["count"] += 1
    kernels = []
    for key, a in agg.items():
        avg = a["ms"] / a["count"]
        ac = acct[key]
        kernels.append({"kernel": key[0], "layer": key[1], "index": key[2], "avg_ms": round(avg, 5),
                        "launches": a["count"], "workgroups": a["workgroups"],
                        "share_of_step": round(a["ms"] / steps / per_step_ms, 4),
                        "tflops": round(ac["flops"] / (avg * 1e-3) / 1e12, 2),
                        "gbps": round(ac["bytes"] / (avg * 1e-3) / 1e9, 1)})
    if not kernels:
        return kernels, None
    by_kind = {}
    for kr in kernels:
        by_kind.setdefault((kr["kernel"], kr["index"]), []).append(kr)
    best = max(by_kind.items(), key=lambda it: sum(k["avg_ms"] for k in it[1]))
    return kernels, best[1][0]


def backward_accounting(B, s, wide=False):
    """Algorithmic FLOPs and HBM bytes per launch of one bf16 layer's backward
    kernels (recomputed products included: they are work the kernels do).  wide:
    the wide layers' backward (output rows, FM part per example, [Phi; W_L]
    products as GEMMs over the batch-major gradient matrix G = [dZ; dLc])."""
    n, d, k, n_f, n_l = s.n, s.d, s.k, s.n_f, s.n_l
    Bp = (B + 63) // 64 * 64
    if not wide:
        out = {
            # X, M, dY in; dR (dM and dLc) out; W_L once.  Lc = W_L X recomputed.
            ("bwd_out", 0, 0): {"flops": B * 2 * n_l * n * d, "bytes": B * (3 * n * d + n_f * d) * 2 + n_l * n * 2},
            # X, d_Fn, dR in; dX out; [Phi; W_L] once.  Z, F recomputed; dZ, dX, d_Phi, d_W_L.
            ("bwd_fmb", 0, 0): {"flops": B * (2 * k * n * d * 4 + 2 * n * d * (2 * k + n_l) + 2 * n_l * n * d),
                                "bytes": B * (3 * n * d + n * k) * 2 + (k + n_l) * n * 2},
        }
    else:
        T = len(s.mlp) - 1
        kc, bd = k + n_l, B * d
        ldg = (bd + 63) // 64 * 64
        kcp = (kc + 63) // 64 * 64
        out = {
            # X, dY, M (bf16) and Lc (fp32) in; dR out (dM and the dLc rows of G)
            ("bwd_out", 0, 0): {"flops": 0, "bytes": B * ((3 * n * d + n_f * d) * 2 + n_l * d * 4)},
            # X, Z, d_Fn, dR in; dZ (bf16) and dR + dF Z (fp32) out; F recomputed, dZ = dF^T X, dF Z
            ("bwd_fmb", 0, 0): {"flops": B * 6 * n * k * d,
                                "bytes": B * ((2 * n * d + k * d + n * k + k * d) * 2 + n * d * 4)},
            ("bwd_transpose", 0, 3 * T): {"flops": 0, "bytes": 2 * B * n * d * 2},  # X batch-major
            ("bwd_transpose", 0, 3 * T + 1): {"flops": 0, "bytes": (kc * n + n * kcp) * 2},  # [Phi; W_L]^T
            ("bwd_transpose", 0, 3 * T + 2): {"flops": 0, "bytes": (kc * ldg + ldg * kcp) * 2},  # G^T
            ("bwd_wgrad", 0, T): {"flops": 2 * k * n * bd, "bytes": (k + n) * ldg * 2 + k * n * 4},  # d_Phi
            ("bwd_wgrad", 0, T + 1): {"flops": 2 * n_l * n * bd, "bytes": (n_l + n) * ldg * 2 + n_l * n * 4},
            # dX = bf16(dXa + [Phi; W_L]^T G): G^T and [Phi; W_L]^T in, dXa (fp32) in, dX out
            ("bwd_dgrad", 0, T): {"flops": 2 * n * kc * bd,
                                  "bytes": (ldg * kcp + n * kcp) * 2 + B * n * d * (4 + 2)},
        }
    out[("bwd_reduce", 0, 0)] = {"flops": 0, "bytes": 0}  # the LayerNorm and FMB / LCB weight sums
    for t, (a, b) in enumerate(zip(s.mlp[:-1], s.mlp[1:])):
        out[("bwd_transpose", 0, 3 * t)] = {"flops": 0, "bytes": (B * b + Bp * b) * 2}
        out[("bwd_transpose", 0, 3 * t + 1)] = {"flops": 0, "bytes": (B * a + Bp * a) * 2}
        out[("bwd_transpose", 0, 3 * t + 2)] = {"flops": 0, "bytes": 2 * a * b * 2}
        out[("bwd_wgrad", 0, t)] = {"flops": 2 * b * a * B, "bytes": (a + b) * Bp * 2 + a * b * 4}
        out[("bwd_dgrad", 0, t)] = {"flops": 2 * B * b * a,
                                    "bytes": (B * b + a * b + B * a + (B * a if t > 0 else 0)) * 2}
        out[("bwd_reduce", 0, 2 + t)] = {"flops": 0, "bytes": 0}
    return out


def measure_training(wk, ws, torch, cfg, layers, x, stream, steps, warmup, seed):
    """One training step of a bf16 layer or stack: the forward that keeps what
    the backward needs (every layer's input, Fn, h_t and M; Z and Lc for the
    wider layers), then the backward (dX and every weight gradient) for a
    seeded dY."""
    if cfg.dtype != "bf16":
        return None
    B = cfg.batch
    specs = [l.spec for l in layers]
    single = len(layers) == 1
    if single:
        need, saved_b = wk.layer_backward_workspace_size(specs[0], B), wk.layer_saved_size(specs[0], B)
    else:
        need, saved_b = wk.stack_backward_workspace_size(specs, B), wk.stack_saved_size(specs, B)
    if need == 0 or saved_b == 0:
        return None
    dy = wk.to_device(ws.make_upstream_grad(cfg, seed), "bf16", x.device)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    saved = wk.alloc_workspace(saved_b, x.device)
    bws = wk.alloc_workspace(need, x.device)
    grads = [wk.LayerGrads(l) for l in layers]

    def forward():
        if single:
            wk.layer_forward_train(x, layers[0], y=y, saved=saved, stream=stream)
        else:
            wk.stack_forward_train(x, layers, y=y, saved=saved, stream=stream)

    def backward(trace=None):
        if single:
            wk.layer_backward(x, saved, dy, layers[0], grads=grads[0], dx=dx, workspace=bws, stream=stream,
                              trace=trace)
        else:
            wk.stack_backward(x, saved, dy, layers, grads=grads, dx=dx, workspace=bws, stream=stream, trace=trace)

    for _ in range(warmup):
        forward()
        backward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        forward()
        backward()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        forward()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sum(5 * (len(s.mlp) - 1) + 16 for s in cfg.layers)
    trace = wk.Trace(capacity=per * steps + 8)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        backward(trace)
    torch.cuda.synchronize()
    bwd_ms = (time.perf_counter() - t1) * 1e3 / steps
    recs = trace.records()
    per_step = len(recs) // steps if steps else 0
    launch_order = [[r["kernel"], r["layer"], r["index"]] for r in recs[:per_step]]
    acct = {}
    for i, s in enumerate(cfg.layers):
        T = len(s.mlp) - 1
        wide = any(r["kernel"] == "bwd_wgrad" and r["layer"] == i and r["index"] == T for r in recs)
        for (kname, _, idx), v in backward_accounting(B, s, wide).items():
            acct[(kname, i, idx)] = v
    kernels, dom = summarize_trace(recs, acct, bwd_ms, steps)
    trace.close()
    roof = None
    if dom is not None:
        roof = roofline_of(dom, acct[(dom["kernel"], dom["layer"], dom["index"])], dom["avg_ms"], "bf16", cfg.name)
    fwd_flops = cfg.flops_per_example() * B
    bwd_flops = sum(a["flops"] for a in acct.values())
    return {"ms_per_step": round(ms, 4), "forward_train_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
            "examples_per_s": round(B / ms * 1e3, 1),
            # the usual training count: backward = 2 x forward
            "model_tflops": round(3 * fwd_flops / (ms * 1e-3) / 1e12, 2),
            "kernel_tflops": round((fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12, 2),
            "roofline": roof,
            "kernels": sorted(kernels, key=lambda k: (k["layer"], k["kernel"], k["index"])),
            "backward_launch_order": launch_order}


MOE_EXPERTS = 4  # experts of the measured mixture-of-experts layer


def moe_expert_shapes(s, E=MOE_EXPERTS):
    """E experts of a layer's width: each keeps the layer's k and hidden MLP
    widths and produces 1/E of its FMB and LCB rows."""
    if s.n_f % E or s.n_l % E:
        return None
    nf, nl = s.n_f // E, s.n_l // E
    return [(s.k, nf, nl, (s.n * s.k,) + tuple(s.mlp[1:-1]) + (nf * s.d,))] * E


def measure_moe(wk, ws, torch, cfg, x, stream, steps, warmup, seed):
    """A Wukong mixture-of-experts layer (the experts run as grouped launches of
    the layer kernels) on the workload's input, timed on its own."""
    if cfg.num_layers != 1:
        return None
    s = cfg.layers[0]
    shapes = moe_expert_shapes(s)
    if shapes is None:
        return None
    specs = [wk.LayerSpec(s.n, s.d, k, nf, nl, mlp, 1e-5, cfg.dtype) for k, nf, nl, mlp in shapes]
    spec = wk.MoeSpec(specs)
    need = wk.moe_workspace_size(spec, cfg.batch)
    if need == 0:
        return None
    experts = []
    for e, (k, nf, nl, mlp) in enumerate(shapes):
        h = ws.make_expert_weights(cfg.name + "/moe", e, s.n, s.d, k, nl, mlp, cfg.dtype, seed, "identity")
        experts.append(wk.DeviceLayer.from_host(specs[e], h, device=x.device))
    og, ob = ws.make_out_layernorm(cfg.name + "/moe", s.d, cfg.dtype, seed, "identity")
    moe = wk.DeviceMoe(spec, experts, og, ob, device=x.device)
    y = torch.empty_like(x)
    mws = wk.alloc_workspace(need, x.device)
    # the HIP runtime's first few dozen launches of the grouped kernel carry a one-off host cost
    # (about 1.3 ms a call, measured): warm up past it
    for _ in range(max(warmup, 64)):
        wk.moe_forward(x, moe, y=y, workspace=mws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wk.moe_forward(x, moe, y=y, workspace=mws, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = MOE_EXPERTS * (2 + len(s.mlp))
    trace = wk.Trace(capacity=per * steps + 8)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        wk.moe_forward(x, moe, y=y, workspace=mws, stream=stream, trace=trace)
    torch.cuda.synchronize()
    traced_ms = (time.perf_counter() - t1) * 1e3 / steps
    # per-expert accounting (trace layer index = expert), as kernel_accounting for a layer
    es = 2 if cfg.dtype == "bf16" else 4
    B = cfg.batch
    acct = {}
    for e, (k, nf, nl, mlp) in enumerate(shapes):
        acct[("fmb_lcb", e, 0)] = {"flops": B * (2 * (k + nl) * s.n * s.d + 2 * s.n * s.d * k),
                                   "bytes": B * (s.n * s.d + s.n * k + nl * s.d) * es + (k + nl) * s.n * es}
        # the last Linear carries the output LayerNorm for bf16, d in {16, 32, 80, 160}
        # and an input width that is a multiple of 64 (include/wukong.h)
        fused = cfg.dtype == "bf16" and s.d in (16, 32, 80, 160) and mlp[-2] % 64 == 0
        T = len(mlp) - 1
        for t, (a_, b_) in enumerate(zip(mlp[:-1], mlp[1:])):
            extra = B * b_ if (fused and t == T - 1) else 0
            acct[("mlp_linear", e, t)] = {"flops": 2 * B * a_ * b_, "bytes": (B * a_ + a_ * b_ + B * b_ + b_ + extra) * es}
        if not fused:
            acct[("residual_ln", e, 0)] = {"flops": 0, "bytes": 3 * B * nf * s.d * es}
    # when every expert's last Linear is fused, those run as one grouped launch recorded as
    # layer = number of experts: its work is the sum of theirs
    E = len(shapes)
    last = [acct[("mlp_linear", e, len(mlp) - 2)] for e, (_, _, _, mlp) in enumerate(shapes)]
    acct[("mlp_linear", E, 0)] = {"flops": sum(a["flops"] for a in last), "bytes": sum(a["bytes"] for a in last)}
    kernels, dom = summarize_trace(trace.records(), acct, traced_ms, steps)
    flops = sum(acct[(k["kernel"], k["layer"], k["index"])]["flops"] * k["launches"] / steps for k in kernels)
    trace.close()
    roof = None
    if dom is not None:
        # the experts' kernels share names with the layer's but not its shapes: no layer traffic file applies
        roof = roofline_of(dom, acct[(dom["kernel"], dom["layer"], dom["index"])], dom["avg_ms"], cfg.dtype,
                           f"{cfg.name}_moe")
    return {"experts": [{"k": k, "n_f": nf, "n_l": nl, "mlp": list(mlp)} for k, nf, nl, mlp in shapes],
            "ms_per_call": round(ms, 4), "examples_per_s": round(cfg.batch / ms * 1e3, 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "mfma_frac": round(flops / (ms * 1e-3) / 1e12 /
                                                                                PEAK_BF16_TFLOPS, 4),
            "roofline": roof, "kernels": sorted(kernels, key=lambda k: (k["layer"], k["kernel"], k["index"]))}


def optional_section(name, fn, *args):
    """Run one optional measurement; a failure is reported in its place instead
    of ending the run (the main result line must still be printed)."""
    try:
        return fn(*args)
    except Exception as e:  # noqa: BLE001
        print(f"# {name} section failed: {e}", file=sys.stderr, flush=True)
        return {"error": f"{type(e).__name__}: {e}"}


def measure_head(wk, ws, torch, cfg, y, stream, steps, warmup, seed):
    """The prediction head (top MLP + logistic function) on the stack's output,
    timed on its own: widths cfg.head_dims(), Xavier-uniform weights."""
    dims = cfg.head_dims()
    w, b = ws.make_head_weights(cfg.name, dims, cfg.dtype, seed, "identity")
    head = wk.DeviceHead(wk.HeadSpec(dims, cfg.dtype), w, b, device=y.device)
    prob = torch.empty((cfg.batch, dims[-1]), dtype=torch.float32, device=y.device)
    hws = wk.alloc_workspace(wk.head_workspace_size(head.spec, cfg.batch), y.device)
    for _ in range(warmup):
        wk.head_forward(y, head, prob=prob, workspace=hws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wk.head_forward(y, head, prob=prob, workspace=hws, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    trace = wk.Trace(capacity=len(dims) * steps + 8)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        wk.head_forward(y, head, prob=prob, workspace=hws, stream=stream, trace=trace)
    torch.cuda.synchronize()
    traced_ms = (time.perf_counter() - t1) * 1e3 / steps
    acct = head_accounting(dims, cfg.batch, 2 if cfg.dtype == "bf16" else 4)
    kernels, dom = summarize_trace(trace.records(), acct, traced_ms, steps)
    trace.close()
    roof = None
    if dom is not None:
        roof = roofline_of(dom, acct[(dom["kernel"], dom["layer"], dom["index"])], dom["avg_ms"], cfg.dtype,
                           cfg.name)
    flops = sum(2 * a * o for a, o in zip(dims[:-1], dims[1:])) * cfg.batch
    return {"dims": list(dims), "ms_per_call": round(ms, 4), "examples_per_s": round(cfg.batch / ms * 1e3, 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "roofline": roof,
            "kernels": sorted(kernels, key=lambda k: (k["kernel"] != "head_linear", k["index"]))}


FUSION_L = 1024  # sequence positions of H_s in the measured fusion step


def fusion_accounting(B, n, d, L, dff):
    """Algorithmic FLOPs and HBM bytes per launch of the fusion step's kernels (bf16)."""
    rows = B * n
    return {
        # S = Q K^T, O = P V and the Fusion Linear Q = [H_w, A] W_f^T + b_f in one kernel:
        # H_s (K = V) read once, H_w read, W_f and b_f read, Q written
        ("fusion_attention", 0, 0): {"flops": 4 * B * n * L * d + 2 * rows * 2 * d * d,
                                     "bytes": (B * L * d + B * n * d + 2 * d * d + d + rows * d) * 2},
        ("fusion_ln", 0, 0): {"flops": 0, "bytes": 2 * rows * d * 2},
        ("fusion_linear", 0, 1): {"flops": 2 * rows * d * dff, "bytes": (rows * d + dff * d + dff + rows * dff) * 2},
        ("fusion_linear", 0, 2): {"flops": 2 * rows * dff * d,
                                  "bytes": (rows * dff + d * dff + d + 2 * rows * d) * 2},
        # LN + both FFN products + residual in one kernel: Q read once, H_f written, silu(U) * U on chip
        ("fusion_ffn", 0, 0): {"flops": 4 * rows * d * dff,
                               "bytes": (2 * rows * d + 2 * dff * d + dff + 3 * d) * 2},
    }


def measure_fusion(wk, ws, torch, cfg, y, stream, steps, warmup, seed):
    """WHALE's fusion step on the stack's output as H_w, with a seeded H_s of
    FUSION_L positions and d_ff = 4d, timed on its own."""
    s = cfg.layers[-1]
    n, d, L, dff = s.n, s.d, FUSION_L, 4 * s.d
    spec = wk.FusionSpec(n, d, L, dff)
    if wk.fusion_workspace_size(spec, cfg.batch) == 0:
        return None
    w = ws.make_fusion_weights(cfg.name, d, dff, cfg.dtype, seed, "identity")
    fusion = wk.DeviceFusion(spec, w.w_f, w.w_up, w.w_down, w.b_f, w.gamma, w.beta, w.b_up, w.b_down, device=y.device)
    hs = wk.to_device(ws.make_sequence(cfg.name, cfg.batch, L, d, cfg.dtype, seed), cfg.dtype, y.device)
    hf = torch.empty_like(y)
    fws = wk.alloc_workspace(wk.fusion_workspace_size(spec, cfg.batch), y.device)
    for _ in range(warmup):
        wk.fusion_forward(y, hs, fusion, hf=hf, workspace=fws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wk.fusion_forward(y, hs, fusion, hf=hf, workspace=fws, stream=stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    trace = wk.Trace(capacity=5 * steps + 8)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        wk.fusion_forward(y, hs, fusion, hf=hf, workspace=fws, stream=stream, trace=trace)
    torch.cuda.synchronize()
    traced_ms = (time.perf_counter() - t1) * 1e3 / steps
    acct = fusion_accounting(cfg.batch, n, d, L, dff)
    kernels, dom = summarize_trace(trace.records(), acct, traced_ms, steps)
    trace.close()
    roof = None
    if dom is not None:
        roof = roofline_of(dom, acct[(dom["kernel"], dom["layer"], dom["index"])], dom["avg_ms"], cfg.dtype, cfg.name)
    # the kernels that ran (the accounting also lists the unfused FFN's)
    flops = sum(acct[(k["kernel"], k["layer"], k["index"])]["flops"] for k in kernels)
    return {"n": n, "d": d, "L": L, "d_ff": dff, "ms_per_call": round(ms, 4),
            "examples_per_s": round(cfg.batch / ms * 1e3, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "roofline": roof, "kernels": sorted(kernels, key=lambda k: (k["kernel"], k["index"]))}


def source_digest(name):
    h = hashlib.sha256()
    for src in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "recommender_feature_interaction_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(kernel, index, workload):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), or None
    when absent or when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{index}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256") != source_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(cfg, host_w, x, budget_s):
    """The oracle (as it stands) on the first examples of the batch, in chunks,
    until about budget_s seconds of host time are spent: pure fp64 (the parity
    reference), then the same steps in fp32 for about half that time."""
    import numpy as np

    import oracle

    def run(dtype, budget):
        chunk = 64 if cfg.num_layers == 1 else 4
        done, t0 = 0, time.perf_counter()
        while done < cfg.batch:
            m = min(chunk, cfg.batch - done)
            oracle.wukong_stack(x[done:done + m], host_w, storage=(), dtype=dtype)
            done += m
            if time.perf_counter() - t0 >= budget:
                break
        return done, time.perf_counter() - t0

    done, el = run(np.float64, budget_s)
    done32, el32 = run(np.float32, budget_s / 2)
    return {"value": round(done / el, 3), "unit": "examples/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {done} of {cfg.batch} examples of {cfg.name}, fp64 numpy oracle, "
                      f"{el:.1f} s on {os.cpu_count()} host CPUs",
            "value_f32": round(done32 / el32, 3),
            "sample_f32": f"first {done32} examples, the same oracle steps in fp32, {el32:.1f} s"}


# workloads measured in the same run as the headline, each reported as a section of its own
SECTIONS = ("stack8_n512", "smalld_n720", "layer_d160")


def stats_ms(v):
    import numpy as np

    a = np.sort(np.asarray(v, dtype=np.float64))
    return {"median": round(float(np.median(a)), 4), "min": round(float(a[0]), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4)}


def memory_bound_share(cfg, kernels, acct, copy_gbps):
    """Algorithmic bytes of the memory-bound kernels (FMB+LCB and the residual
    LayerNorm, or the fused last Linear's extra X / Y traffic is not counted
    here) over their measured time, as a fraction of HBM bandwidth."""
    names = ("fmb_lcb", "residual_ln")
    by = [k for k in kernels if k["kernel"] in names]
    if not by:
        return None
    nbytes = sum(acct[(k["kernel"], k["layer"], k["index"])]["bytes"] for k in by)
    ms = sum(k["avg_ms"] for k in by)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"kernels": sorted({k["kernel"] for k in by}), "algorithmic_bytes": nbytes, "ms": round(ms, 5),
            "gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "frac_of_measured_copy": round(gbps / copy_gbps, 4)}


def measure_workload(wk, ws, torch, name, args, dev, stream, copy_gbps, mfma_probe, extras=()):
    """One workload: the stack forward over its batch, timed as the headline is
    (wall clock over K steps, per-step events, HIP-graph replay, 512 MB flush
    between steps, per-kernel events), plus the optional sections in `extras`.
    Returns (result, host weights, host input)."""
    cfg = ws.get(name)
    t_gen = time.time()
    host_w = ws.make_stack_weights(cfg, args.seed, "identity")
    x_host = ws.make_input(cfg, args.seed)
    layers = [wk.DeviceLayer.from_host(wk.LayerSpec(s.n, s.d, s.k, s.n_f, s.n_l, tuple(s.mlp), 1e-5, cfg.dtype),
                                       h, device=dev) for s, h in zip(cfg.layers, host_w)]
    x = wk.to_device(x_host, cfg.dtype, dev)
    y = torch.empty_like(x)
    specs = [l.spec for l in layers]
    ws_t = wk.alloc_workspace(wk.stack_workspace_size(specs, cfg.batch), dev)
    torch.cuda.synchronize()
    print(f"# {cfg.name}: inputs ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def fwd(trace=None):
        wk.stack_forward(x, layers, y=y, workspace=ws_t, stream=stream, trace=trace)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    print(f"# {cfg.name}: timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # each step between HIP events on the launch stream (no synchronisation between steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        fwd()
        e1.record(stream)
    torch.cuda.synchronize()
    step_ms = stats_ms([e0.elapsed_time(e1) for e0, e1 in ev])

    # the same step captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                wk.stack_forward(x, layers, y=y, workspace=ws_t)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            wk.stack_forward(x, layers, y=y, workspace=ws_t)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg) * 1e3 / args.steps
        del graph

    # per-kernel pass: the library records HIP events around every launch on the launch stream
    kpl = sum(2 + len(s.mlp) - 1 for s in cfg.layers)  # launches per step (at most)
    kernels, dominant, traced_ms = [], None, None
    fused_layers = [li for li, sp in enumerate(specs) if wk.workspace_layout(sp, cfg.batch)["m"] < 0]
    acct = kernel_accounting(cfg, fused_layers)
    if not args.no_trace:
        trace = wk.Trace(capacity=kpl * args.steps + 16)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            fwd(trace)
        torch.cuda.synchronize()
        traced_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        kernels, dominant = summarize_trace(trace.records(), acct, traced_ms, args.steps)
        trace.close()
    roofline = None
    if dominant is not None:
        roofline = roofline_of(dominant, acct[(dominant["kernel"], dominant["layer"], dominant["index"])],
                               dominant["avg_ms"], cfg.dtype, cfg.name)
        if roofline["unit"] == "GB/s":
            roofline["frac_of_measured_copy"] = round(roofline["achieved"] / copy_gbps, 4)
        elif cfg.dtype == "bf16" and mfma_probe:
            roofline["frac_of_measured_mfma"] = round(roofline["achieved"] / mfma_probe, 4)

    # the same steps with 512 MB written between them (untimed), so no input or weight is
    # still in L2 or the 256 MB last-level cache when a step starts
    cold_ms = None
    if not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evc:
            flush.fill_(1)
            e0.record(stream)
            fwd()
            e1.record(stream)
        torch.cuda.synchronize()
        cold_ms = sum(e0.elapsed_time(e1) for e0, e1 in evc) / args.steps
        del flush

    # layer roofline fraction: sum over kernels of max(F/P, B/BW) against the measured step
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    ideal_ms = sum(1e3 * max(ac["flops"] / (peak * 1e12), ac["bytes"] / (PEAK_HBM_GBPS * 1e9))
                   for ac in acct.values())
    step_tflops = cfg.flops_per_example() * cfg.batch / (ms_per_step * 1e-3) / 1e12
    s0 = cfg.layers[0]
    res = {
        "workload": cfg.name, "global_batch": cfg.batch, "layers": cfg.num_layers, "n": s0.n, "d": s0.d,
        "k": s0.k, "n_f": s0.n_f, "n_l": s0.n_l, "mlp": list(s0.mlp), "dtype": cfg.dtype,
        "ms_per_step": round(ms_per_step, 4),
        "examples_per_s": round(cfg.batch / ms_per_step * 1e3, 1),
        "step_ms_events": step_ms,
        "traced_ms_per_step": None if traced_ms is None else round(traced_ms, 4),
        "step_tflops": round(step_tflops, 2),
        "step_mfma_frac": round(step_tflops / PEAK_BF16_TFLOPS, 4) if cfg.dtype == "bf16" else None,
        "step_mfma_frac_of_measured": (round(step_tflops / mfma_probe, 4)
                                       if cfg.dtype == "bf16" and mfma_probe else None),
        "step_roofline_frac": round(ideal_ms / ms_per_step, 4),
        "roofline": roofline,
        "cold_cache_ms_per_step": None if cold_ms is None else round(cold_ms, 4),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "memory_bound_kernels": memory_bound_share(cfg, kernels, acct, copy_gbps),
        "kernels": sorted(kernels, key=lambda k: (k["layer"], k["kernel"] != "fmb_lcb", k["kernel"], k["index"])),
    }
    if "head" in extras:
        res["head"] = optional_section("head", measure_head, wk, ws, torch, cfg, y, stream, args.steps,
                                       args.warmup, args.seed)
    if "fusion" in extras and cfg.dtype == "bf16":
        res["fusion"] = optional_section("fusion", measure_fusion, wk, ws, torch, cfg, y, stream, args.steps,
                                         args.warmup, args.seed)
    if "training" in extras:
        res["training"] = optional_section("training", measure_training, wk, ws, torch, cfg, layers, x, stream,
                                           args.steps, args.warmup, args.seed)
        if isinstance(res["training"], dict):
            res["training"].pop("backward_launch_order", None)  # for profiling runs (--only training) only
    if "moe" in extras and cfg.dtype == "bf16":
        res["moe"] = optional_section("moe", measure_moe, wk, ws, torch, cfg, x, stream, args.steps, args.warmup,
                                      args.seed)
    for key in ("head", "fusion", "training", "moe"):
        v = res.get(key)
        if v and "error" not in v:
            ms = v.get("ms_per_call", v.get("ms_per_step"))
            print(f"# {cfg.name} {key}: {ms:.3f} ms", file=sys.stderr, flush=True)
    del x, y, ws_t, layers
    torch.cuda.empty_cache()
    return res, host_w, x_host


def measure_copy(torch, dev, stream):
    """On-box copy bandwidth: a 256 MiB device-to-device copy (reads + writes)."""
    csrc = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        cdst.copy_(csrc)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    return 2 * (256 << 20) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="stack8_n256", help="the headline workload")
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated further workloads measured in the same run ('' for none)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--no-head", action="store_true", help="skip the prediction-head measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache (512 MB flush) step timing")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-fusion", action="store_true", help="skip the WHALE fusion-step measurement")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the training step (forward + backward of the layer or stack) measurement")
    ap.add_argument("--no-moe", action="store_true", help="skip the mixture-of-experts layer measurement")
    ap.add_argument("--only", choices=("fusion", "training", "moe"), default=None,
                    help="profiling aid: run the stack forward once, then time only this section and print it")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch

        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark measures one GPU only: the Wukong forward needs no "
                                   "collectives and every example is independent, so N GPUs would each run "
                                   "this same one-GPU workload on their share of the batch; run with --gpus 1"}))
        sys.exit(2)

    import torch

    import recommender_feature_interaction_amd as wk
    import wukong_synth as ws

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.only:
        cfg = ws.get(args.config)
        host_w = ws.make_stack_weights(cfg, args.seed, "identity")
        layers = [wk.DeviceLayer.from_host(wk.LayerSpec(s.n, s.d, s.k, s.n_f, s.n_l, tuple(s.mlp), 1e-5, cfg.dtype),
                                           h, device=dev) for s, h in zip(cfg.layers, host_w)]
        x = wk.to_device(ws.make_input(cfg, args.seed), cfg.dtype, dev)
        y = wk.stack_forward(x, layers, stream=stream)
        torch.cuda.synchronize()
        if args.only == "fusion":
            res = measure_fusion(wk, ws, torch, cfg, y, stream, args.steps, args.warmup, args.seed)
        elif args.only == "moe":
            res = measure_moe(wk, ws, torch, cfg, x, stream, args.steps, args.warmup, args.seed)
        else:
            res = measure_training(wk, ws, torch, cfg, layers, x, stream, args.steps, args.warmup, args.seed)
        print(json.dumps({"only": args.only, "config": {"workload": cfg.name, "global_batch": cfg.batch},
                          args.only: res}), flush=True)
        return

    copy_gbps = measure_copy(torch, dev, stream)
    mfma_probe = wk.probe_mfma_bf16()
    print(f"# copy {copy_gbps:.1f} GB/s, MFMA probe {mfma_probe:.1f} TFLOP/s", file=sys.stderr, flush=True)

    extras = [e for e, off in (("head", args.no_head), ("fusion", args.no_fusion), ("training", args.no_training))
              if not off]
    if ws.get(args.config).num_layers == 1 and not args.no_moe:
        extras.append("moe")
    head_res, host_w, x_host = measure_workload(wk, ws, torch, args.config, args, dev, stream, copy_gbps, mfma_probe,
                                                extras)
    cfg = ws.get(args.config)
    sections = {}
    for name in [s for s in args.sections.split(",") if s and s != args.config]:
        ex = [e for e, off in (("fusion", args.no_fusion), ("training", args.no_training)) if not off]
        if ws.get(name).num_layers == 1 and not args.no_moe:
            ex.append("moe")
        sections[name] = optional_section(name, lambda n=name, e=ex: measure_workload(
            wk, ws, torch, n, args, dev, stream, copy_gbps, mfma_probe, e)[0])

    h = head_res
    out = {
        "metric": METRIC,
        "value": round(cfg.batch * 1e3 / h["ms_per_step"], 1),
        "unit": "examples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) inputs, Xavier-uniform weights)",
        "config": {"workload": cfg.name, "global_batch": cfg.batch, "layers": cfg.num_layers, "n": h["n"],
                   "d": h["d"], "k": h["k"], "n_f": h["n_f"], "n_l": h["n_l"], "mlp": h["mlp"],
                   "parallelism": "single GPU"},
        "roofline": h["roofline"],
        "step_ms_events": h["step_ms_events"],
        "traced_ms_per_step": h["traced_ms_per_step"],
        "step_tflops": h["step_tflops"],
        "step_mfma_frac": h["step_mfma_frac"],
        "step_mfma_frac_of_measured": h["step_mfma_frac_of_measured"],
        "step_roofline_frac": h["step_roofline_frac"],
        "cold_cache_ms_per_step": h["cold_cache_ms_per_step"],
        "graph_ms_per_step": h["graph_ms_per_step"],
        "copy_gbps_measured": round(copy_gbps, 1),
        "mfma_tflops_measured": round(mfma_probe, 1),
        "mfma_frac_measured_of_peak": round(mfma_probe / PEAK_BF16_TFLOPS, 4),
        "memory_bound_kernels": h["memory_bound_kernels"],
        "kernels": h["kernels"],
        "head": h.get("head"),
        "fusion": h.get("fusion"),
        "training": h.get("training"),
        "moe": h.get("moe"),
        "workloads": sections,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, host_w, x_host, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
