"""Parity of the HIP path (through the C ABI) with the CPU oracle.

fp32 layers are compared with the pure fp64 oracle, bf16 layers with the
oracle run at the bf16 storage points the library documents (Z, Fn, h_t, M,
Y).  The gate (tests/_metrics.py): fp32 elementwise max relative error
<= 1e-4; bf16 normwise max relative error <= 2e-2 and rms <= 1e-2 at any
depth, plus elementwise <= 2e-2 for single layers and their intermediates.
"""
import numpy as np
import pytest
import torch

import oracle
import recommender_feature_interaction_amd as wk
import wukong_synth as ws
from _gpu_helpers import BF16_STORAGE, Run, check, host_f64, log, sample_indices, spec_of, storage_for, to_host
from _metrics import rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    wk.load_library()  # no fallback: a missing library fails here


def _ws_tensor(ws_t, off, count, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    es = 2 if dtype == "bf16" else 4
    return to_host(ws_t[off:off + count * es].view(tdt))


def _ws_fn(ws_t, lay, batch, nk, dtype):
    """Fn [batch, nk] from a layer workspace: row-major, or K-blocked (64-column blocks of
    fn_kblock_rows rows, as wk_workspace_layout documents) for the first Linear."""
    rows = lay["fn_kblock_rows"]
    if rows == 0:
        return _ws_tensor(ws_t, lay["fn"], batch * nk, dtype).reshape(batch, nk)
    assert nk % 64 == 0 and rows >= batch and rows % 256 == 0
    blocked = _ws_tensor(ws_t, lay["fn"], rows * nk, dtype).reshape(nk // 64, rows, 64)
    return np.ascontiguousarray(blocked.transpose(1, 0, 2)).reshape(rows, nk)[:batch]


def test_tiny_f32_full_batch():
    for affine in ("identity", "random"):
        r = Run(ws.TINY_F32, seed=0, affine=affine)
        log(f"tiny_f32 affine={affine}")
        y = host_f64(to_host(r.forward()))
        check("Y", y, r.oracle(), "f32")


# One layer of each workload (the 8-layer stacks' layer shapes included: n = 256
# with three Linears, and n = 512, whose FMB+LCB runs the streamed kernel with
# one example per group), at a batch the oracle finishes in seconds.
SINGLE = [(ws.TINY_F32, 64), (ws.LAYER_D160, 48), (ws.SMALLD_N720, 48), (ws.UNITS_N2880, 48),
          (ws.STACK8_N256.with_layers(1), 8), (ws.STACK8_N512.with_layers(1), 6)]


@pytest.mark.parametrize("cfg,B", SINGLE, ids=[c.name for c, _ in SINGLE])
def test_single_layer_intermediates(cfg, B):
    r = Run(cfg, seed=11, affine="random", batch=B)
    spec = spec_of(cfg.layers[0], cfg.dtype)
    wst = wk.alloc_workspace(wk.layer_workspace_size(spec, B))
    y = wk.layer_forward(r.xd, r.layers[0], workspace=wst)
    torch.cuda.synchronize()
    lay = wk.workspace_layout(spec, B)
    st = BF16_STORAGE if cfg.dtype == "bf16" else ()
    Y, it = oracle.wukong_layer(r.x, r.host_w[0], storage=st, intermediates=True)
    tol = cfg.dtype
    s = cfg.layers[0]
    fn = host_f64(_ws_fn(wst, lay, B, s.n * s.k, cfg.dtype))
    if lay["fn_kblock_rows"]:
        log(f"  Fn K-blocked ({lay['fn_kblock_rows']} rows per 64-column block)")
    check("Fn", fn, it["Fn"], tol)
    for t, off in enumerate(lay["hidden"]):
        if off >= 0:
            h = host_f64(_ws_tensor(wst, off, B * s.mlp[t + 1], cfg.dtype)).reshape(B, -1)
            check(f"h{t + 1}", h, it["h"][t], tol)
    if lay["m"] >= 0:
        m = host_f64(_ws_tensor(wst, lay["m"], B * s.n_f * s.d, cfg.dtype)).reshape(B, s.n_f, s.d)
        check("M", m, it["M"], tol)
    else:
        log("  M not stored: the last Linear applies the output LayerNorm itself")
    yh = host_f64(to_host(y))
    check("Y rows of FMB", yh[:, :s.n_f], Y[:, :s.n_f], tol)
    check("Y rows of LCB", yh[:, s.n_f:], Y[:, s.n_f:], tol)


# Ragged batches of the streamed FMB+LCB layers, whose Fn is K-blocked for the first Linear:
# B = 257 leaves 255 padding rows per 64-column block and a last group of one example (two per
# group at n = 256, four at n = 720); B = 259 a last group of three at n = 720.
RAGGED = [(ws.STACK8_N256.with_layers(1), 257), (ws.SMALLD_N720, 257), (ws.SMALLD_N720, 259)]


@pytest.mark.parametrize("cfg,B", RAGGED, ids=[f"{c.name}_B{b}" for c, b in RAGGED])
def test_ragged_batch_kblocked_fn(cfg, B):
    r = Run(cfg, seed=B, affine="random", batch=B)
    spec = spec_of(cfg.layers[0], cfg.dtype)
    lay = wk.workspace_layout(spec, B)
    assert lay["fn_kblock_rows"] == 512, lay
    wst = wk.alloc_workspace(wk.layer_workspace_size(spec, B))
    y = wk.layer_forward(r.xd, r.layers[0], workspace=wst)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 127, 255, 256] + list(range(257, B)))
    s = cfg.layers[0]
    Y, it = oracle.wukong_layer(r.x[idx], r.host_w[0], storage=BF16_STORAGE, intermediates=True)
    fn = host_f64(_ws_fn(wst, lay, B, s.n * s.k, cfg.dtype))[idx]
    check(f"Fn at examples {idx.tolist()}", fn, it["Fn"], "bf16")
    check(f"Y at examples {idx.tolist()}", host_f64(to_host(y))[idx], Y, "bf16")


def test_n256_layer_three_examples_per_workgroup():
    """The n = 256 layer's FMB+LCB kernel takes one example at a time per persistent
    workgroup and finishes each example's output stage during the next one's first
    chunk (the last example's after the loop).  At B = 515 workgroups 0..2 take three
    examples and the others two: the examples checked are first, middle and last ones
    of those sequences (Fn K-blocked over 768 rows, and Y)."""
    cfg, B = ws.STACK8_N256.with_layers(1), 515
    r = Run(cfg, seed=B, affine="random", batch=B)
    spec = spec_of(cfg.layers[0], cfg.dtype)
    lay = wk.workspace_layout(spec, B)
    assert lay["fn_kblock_rows"] == 768, lay
    wst = wk.alloc_workspace(wk.layer_workspace_size(spec, B))
    y = wk.layer_forward(r.xd, r.layers[0], workspace=wst)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 2, 3, 255, 256, 257, 258, 259, 511, 512, 513, 514])
    s = cfg.layers[0]
    Y, it = oracle.wukong_layer(r.x[idx], r.host_w[0], storage=BF16_STORAGE, intermediates=True)
    fn = host_f64(_ws_fn(wst, lay, B, s.n * s.k, cfg.dtype))[idx]
    check(f"Fn at examples {idx.tolist()}", fn, it["Fn"], "bf16")
    check(f"Y at examples {idx.tolist()}", host_f64(to_host(y))[idx], Y, "bf16")


@pytest.mark.parametrize("cfg,batch", [(ws.STACK8_N256, 6), (ws.STACK8_N512, 4)], ids=["stack8_n256", "stack8_n512"])
def test_stack_two_layers(cfg, batch):
    r = Run(cfg, seed=5, affine="random", num_layers=2, batch=batch)
    y = host_f64(to_host(r.forward()))
    check("Y (bf16-storage oracle)", y, r.oracle(), "bf16", elementwise=False)
    log(f"  vs pure fp64 oracle: elementwise {rel_err(y, r.oracle(storage=())):.3e} (reported)")


def _oracle_layer_bits(x_bits, host_w):
    """The oracle's bf16-storage output of one layer, as the bf16 bit patterns the GPU takes
    as the next layer's input (the stored Y is a bf16 value, so the conversion is exact)."""
    ref = oracle.wukong_layer(x_bits, host_w, storage=BF16_STORAGE)
    bits = ws.to_bf16_bits(ref.astype(np.float32))
    assert np.array_equal(ws.bf16_bits_to_f32(bits).astype(np.float64), ref), "oracle Y is not bf16-valued"
    return ref, bits


@pytest.mark.parametrize("cfg,batch", [(ws.STACK8_N256, 4), (ws.STACK8_N512, 3)], ids=["stack8_n256", "stack8_n512"])
def test_stack_teacher_forced_per_layer(cfg, batch):
    """Every layer of the 8-layer stacks, elementwise: layer i on the GPU takes the
    oracle's (bf16) output of layer i - 1 as its input, so each layer is gated at
    2e-2 elementwise on its own instead of inheriting the rounding flips of the
    layers below it (which only the normwise and rms views tolerate)."""
    r = Run(cfg, seed=7, affine="random", batch=batch)
    x_bits = r.x
    for i, layer in enumerate(r.layers):
        ref, nxt = _oracle_layer_bits(x_bits, r.host_w[i])
        y = wk.layer_forward(wk.to_device(x_bits, "bf16", "cuda"), layer)
        torch.cuda.synchronize()
        check(f"layer {i} Y (input: oracle layer {i - 1})", host_f64(to_host(y)), ref, "bf16")
        x_bits = nxt


def _custom(name, dtype, n, d, k, n_f, mlp, batch, layers=1):
    shape = ws.LayerShape(n, d, k, n_f, n - n_f, tuple(mlp))
    return ws.WukongConfig(name, dtype, batch, tuple([shape] * layers))


RAGGED = [
    _custom("ragged_n40_d32", "bf16", 40, 32, 12, 16, (480, 72, 512), 37),
    _custom("ragged_three_linear", "bf16", 24, 16, 8, 8, (192, 136, 64, 128), 5),
    _custom("ragged_d48", "bf16", 96, 48, 20, 40, (1920, 264, 1920), 3),
    _custom("ragged_one_linear", "bf16", 16, 64, 4, 8, (64, 512), 300),
    _custom("ragged_stack3", "bf16", 40, 32, 12, 16, (480, 72, 512), 9, layers=3),
    # the last Linear carries the residual LayerNorm: partial 256-row and 320-column tiles
    _custom("fused_d32_m300", "bf16", 40, 32, 12, 16, (480, 128, 512), 300),
    _custom("fused_d80", "bf16", 24, 80, 8, 10, (192, 64, 800), 7),
    _custom("fused_d16_one_linear", "bf16", 32, 16, 4, 12, (128, 192), 3),
    _custom("fused_d160_stack2", "bf16", 16, 160, 4, 8, (64, 128, 1280), 260, layers=2),
    # K % 128 == 0 on a ragged batch: the Linear whose DMA is spread over its MFMAs
    _custom("spread_k256_m37", "bf16", 32, 32, 8, 16, (256, 384, 512), 37),
    # K % 64 == 32: the DMA GEMM's last K step is half zero-padded (K = 160, 96)
    _custom("kstep_half_k160", "bf16", 40, 32, 4, 16, (160, 96, 512), 37),
    # the streamed FMB+LCB kernel: phase 2 pairs j tiles when k % 8 == 0 (16-byte LN loads / Fn stores)
    _custom("stream_d32_k20", "bf16", 64, 32, 20, 32, (1280, 64, 1024), 7),
    _custom("stream_d32_k24", "bf16", 48, 32, 24, 16, (1152, 136, 512), 9),
    _custom("stream_d160_k40", "bf16", 192, 160, 40, 96, (7680, 256, 15360), 5),
    _custom("stream_d160_k36", "bf16", 192, 160, 36, 96, (6912, 256, 15360), 3),
    # units of width 8: transpose + batched GEMM (fp32 out) + epilogue
    _custom("units_d8_n64", "bf16", 64, 8, 8, 32, (512, 64, 256), 9),
    _custom("units_d8_k24", "bf16", 128, 8, 24, 64, (3072, 128, 512), 37),
    _custom("units_d8_k32_stack2", "bf16", 192, 8, 32, 96, (6144, 136, 768), 6, layers=2),
    _custom("ragged_f32", "f32", 12, 24, 3, 5, (36, 20, 120), 9),
    _custom("ragged_f32_stack", "f32", 12, 24, 3, 5, (36, 20, 120), 4, layers=2),
]


@pytest.mark.parametrize("cfg", RAGGED, ids=lambda c: c.name)
def test_ragged_shapes(cfg):
    r = Run(cfg, seed=21, affine="random")
    y = host_f64(to_host(r.forward()))
    check("Y", y, r.oracle(), cfg.dtype, elementwise=cfg.num_layers == 1)


def test_determinism_and_batch_invariance():
    r = Run(ws.LAYER_D160, seed=3, affine="random", batch=64)
    y1 = to_host(r.forward())
    y2 = to_host(r.forward())
    assert np.array_equal(y1, y2), "two runs differ"
    sub = wk.stack_forward(r.xd[5:21].contiguous(), r.layers)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(sub), y1[5:21]), "a subset's rows differ from the full batch's"


@pytest.mark.parametrize("cfg,batch", [(ws.LAYER_D160, 64), (ws.STACK8_N256.with_layers(2), 6),
                                       (_custom("units_graph", "bf16", 128, 8, 24, 64, (3072, 128, 512), 11), 11)],
                         ids=["layer_d160", "stack2_n256", "units_d8"])
def test_graph_replay_matches_eager(cfg, batch):
    """A stack captured into a HIP graph and replayed several times, with other
    eager work between the replays, gives the eager result bit for bit."""
    r = Run(cfg, seed=12, affine="random", batch=batch)
    specs = [l.spec for l in r.layers]
    wst = wk.alloc_workspace(wk.stack_workspace_size(specs, batch))
    y_eager = to_host(wk.stack_forward(r.xd, r.layers, workspace=wst))
    torch.cuda.synchronize()
    yg = torch.empty_like(r.xd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wk.stack_forward(r.xd, r.layers, y=yg, workspace=wst)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wk.stack_forward(r.xd, r.layers, y=yg, workspace=wst)
    other = torch.empty_like(r.xd)
    for i in range(3):
        yg.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(yg), y_eager), f"replay {i} differs from the eager result"
        wk.stack_forward(r.xd, r.layers, y=other, workspace=wst)  # eager work between replays
        torch.cuda.synchronize()
    log(f"  {cfg.name}: 3 graph replays equal the eager output")


NULL_AFFINE = [ws.TINY_F32, ws.LAYER_D160, ws.SMALLD_N720,
               _custom("null_stream_d160", "bf16", 192, 160, 40, 96, (7680, 256, 15360), 3),
               _custom("null_units_d8", "bf16", 128, 8, 24, 64, (3072, 128, 512), 5),
               _custom("null_chunked_d48", "bf16", 96, 48, 20, 40, (1920, 264, 1920), 3)]


@pytest.mark.parametrize("cfg", NULL_AFFINE, ids=lambda c: c.name)
def test_null_optional_parameters(cfg):
    """NULL LayerNorm gamma / beta and MLP biases mean identity / zero (include/wukong.h)."""
    import dataclasses
    B = min(cfg.batch, 8)
    c = cfg.with_batch(B)
    host = ws.make_stack_weights(c, 31, "random")
    bare = [dataclasses.replace(h, fm_gamma=None, fm_beta=None, out_gamma=None, out_beta=None,
                                mlp_b=[None] * len(h.mlp_w)) for h in host]
    layers = [wk.DeviceLayer(spec_of(c.layers[i], c.dtype), h.phi, h.w_l, h.mlp_w) for i, h in enumerate(host)]
    x = ws.make_input(c, 31)
    y = wk.stack_forward(wk.to_device(x, c.dtype, "cuda"), layers)
    torch.cuda.synchronize()
    ref = oracle.wukong_stack(x, bare, storage=storage_for(c))
    check("Y (no gamma / beta / biases)", host_f64(to_host(y)), ref, c.dtype)


def test_empty_and_single_example():
    r = Run(ws.LAYER_D160, seed=4, affine="random", batch=1)
    y = host_f64(to_host(r.forward()))
    check("Y (batch 1)", y, r.oracle(), "bf16")
    x0 = r.xd[:0]
    y0 = wk.stack_forward(x0, r.layers)
    torch.cuda.synchronize()
    assert y0.shape == (0, 128, 160)


def test_large_magnitudes():
    """Per-feature scales up to 10 and an extra x100 on X: F grows by 1e4 and is still normalised."""
    r = Run(ws.SMALLD_N720, seed=8, affine="random", batch=16)
    x = ws.bf16_bits_to_f32(r.x) * np.float32(100.0)
    r.x = ws.to_bf16_bits(x)
    r.xd = wk.to_device(r.x, "bf16", "cuda")
    y = host_f64(to_host(r.forward()))
    check("Y (x100)", y, r.oracle(), "bf16")


FULL = [(ws.STACK8_N256, 4), (ws.STACK8_N512, 4), (ws.UNITS_N2880, 8)]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,count", FULL, ids=[c.name for c, _ in FULL])
def test_full_size_sampled(cfg, count):
    """Full batch and depth on the GPU (the benchmark's launch configuration);
    the oracle recomputes a sample of examples one by one."""
    r = Run(cfg, seed=cfg.batch % 97, affine="identity")
    y = r.forward()
    idx = sample_indices(cfg.batch, count, seed=1)
    got = host_f64(to_host(y[torch.as_tensor(idx, device=y.device)]))
    assert torch.isfinite(y.float()).all().item(), "non-finite values in the full output"
    del y
    ref = r.oracle(idx)
    check(f"Y at examples {idx.tolist()}", got, ref, "bf16", elementwise=cfg.num_layers == 1)
    log(f"  vs pure fp64 oracle: elementwise {rel_err(got, r.oracle(idx, storage=())):.3e} (reported)")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [ws.LAYER_D160, ws.SMALLD_N720], ids=lambda c: c.name)
def test_full_batch_every_example(cfg):
    """The single-layer workloads at their full batch (4096 and 8192 examples), in the
    benchmark's launch configuration, compared with the bf16-storage oracle on every
    example, elementwise: cross-example and tail-tile mistakes cannot hide in a sample."""
    r = Run(cfg, seed=cfg.batch % 89, affine="identity")
    got = host_f64(to_host(r.forward()))
    worst = {"elementwise": 0.0, "normwise": 0.0, "rms": 0.0}
    chunk = 1024
    for b0 in range(0, cfg.batch, chunk):
        ref = oracle.wukong_stack(r.x[b0:b0 + chunk], r.host_w, storage=BF16_STORAGE)
        e = check(f"Y examples {b0}..{b0 + len(ref) - 1}", got[b0:b0 + chunk], ref, "bf16")
        worst = {k: max(worst[k], e[k]) for k in worst}
    log(f"  all {cfg.batch} examples: worst {worst}")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,count", [(ws.STACK8_N256, 3), (ws.STACK8_N512, 3)], ids=["stack8_n256", "stack8_n512"])
def test_full_size_teacher_forced(cfg, count):
    """The 8-layer stacks at full batch, one layer call per layer (the launch
    configuration of the stack's own layers): before each layer, the rows of the
    sampled examples in its input are replaced by the oracle's output of the layer
    below, and those examples' outputs are gated elementwise against the oracle's
    layer on that same input."""
    r = Run(cfg, seed=cfg.batch % 97, affine="identity")
    idx = sample_indices(cfg.batch, count, seed=3)
    idx_d = torch.as_tensor(idx, device="cuda")
    spec = r.layers[0].spec
    wst = wk.alloc_workspace(wk.layer_workspace_size(spec, cfg.batch))
    cur, nxt = r.xd, torch.empty_like(r.xd)
    x_bits = r.x[idx]
    for i, layer in enumerate(r.layers):
        cur[idx_d] = wk.to_device(x_bits, "bf16", "cuda")
        wk.layer_forward(cur, layer, y=nxt, workspace=wst)
        torch.cuda.synchronize()
        assert torch.isfinite(nxt.float()).all().item(), f"layer {i}: non-finite values in the full output"
        ref, x_bits = _oracle_layer_bits(x_bits, r.host_w[i])
        check(f"layer {i} Y at examples {idx.tolist()}", host_f64(to_host(nxt[idx_d])), ref, "bf16")
        cur, nxt = nxt, cur


def test_side_stream_launch():
    """A call on a stream other than the current one: the binding orders it after the
    current stream's work and keeps the memory it allocated alive for that stream;
    the result equals the call on the current stream."""
    r = Run(ws.LAYER_D160, seed=13, affine="random", batch=16)
    y_ref = to_host(wk.stack_forward(r.xd, r.layers))
    side = torch.cuda.Stream()
    y = wk.stack_forward(r.xd, r.layers, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(y), y_ref)
