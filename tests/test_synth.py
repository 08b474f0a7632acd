"""The seeded generator and the workload table (host only)."""
import hashlib

import numpy as np
import pytest

import wukong_synth as ws


def test_config_shapes():
    for c in ws.CONFIGS:
        for s in c.layers:
            assert s.mlp[0] == s.n * s.k and s.mlp[-1] == s.n_f * s.d and s.n_f + s.n_l == s.n
    assert [c.num_layers for c in ws.CONFIGS] == [1, 1, 8, 8, 1]
    assert [c.batch for c in ws.CONFIGS] == [64, 4096, 16384, 2048, 8192]


def test_flops_per_example():
    # 2knd + 2ndk + 2 n_L n d + sum 2 m_{t-1} m_t, per layer
    assert ws.TINY_F32.flops_per_example() == 2 * 4 * 16 * 16 * 2 + 2 * 8 * 16 * 16 + 2 * (64 * 64 + 64 * 128)
    assert ws.LAYER_D160.flops_per_example() == 63_963_136
    assert ws.STACK8_N256.flops_per_example() == 8 * 320_339_968
    assert ws.STACK8_N512.flops_per_example() == 8 * 1_684_013_056
    assert ws.SMALLD_N720.flops_per_example() == 77_783_040


def test_bf16_bits_match_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000)).astype(np.float32)
    x[:64] = np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(64, dtype=np.float32)  # ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ws.to_bf16_bits(x), ref)
    assert np.array_equal(ws.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_deterministic_and_frozen():
    a = ws.make_input(ws.TINY_F32, seed=0)
    b = ws.make_input(ws.TINY_F32, seed=0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, ws.make_input(ws.TINY_F32, seed=1))
    w1 = ws.make_layer_weights("tiny_f32", 0, ws.TINY_F32.layers[0], "f32", 0)
    w2 = ws.make_layer_weights("tiny_f32", 0, ws.TINY_F32.layers[0], "f32", 0)
    assert all(np.array_equal(p, q) for p, q in zip(w1.mlp_w, w2.mlp_w))
    # Philox streams are platform-stable: freeze a digest of the first values
    h = hashlib.sha256(a[:2].tobytes()).hexdigest()[:16]
    assert h == FROZEN_TINY_X


FROZEN_TINY_X = "3d221ba0e40394f1"


def test_subset_regeneration():
    cfg = ws.LAYER_D160.with_batch(300)
    full = ws.make_input(cfg, seed=1)
    part = ws.make_input(cfg, seed=1, batch=37, first_example=101)
    assert np.array_equal(full[101:138], part)


def test_distributions():
    cfg = ws.LAYER_D160.with_batch(64)
    x = ws.bf16_bits_to_f32(ws.make_input(cfg, seed=2)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    s = cfg.layers[0]
    w = ws.make_layer_weights(cfg.name, 0, s, "bf16", 2)
    for W in w.mlp_w + [w.phi, w.w_l]:
        a = np.sqrt(6.0 / (W.shape[0] + W.shape[1]))
        v = ws.bf16_bits_to_f32(W)
        assert np.abs(v).max() <= a * (1 + 2 ** -8)
        assert abs(v.mean()) < 0.05 * a and abs(v.var() - a * a / 3) < 0.05 * a * a
    assert np.all(ws.bf16_bits_to_f32(w.out_gamma) == 1.0) and np.all(ws.bf16_bits_to_f32(w.mlp_b[0]) == 0.0)
    wr = ws.make_layer_weights(cfg.name, 0, s, "bf16", 2, affine="random")
    g = ws.bf16_bits_to_f32(wr.fm_gamma)
    assert g.min() >= 0.5 and g.max() <= 1.5 and g.std() > 0.2


def test_feature_scaled_units():
    cfg = ws.SMALLD_N720.with_batch(256)
    s = ws.feature_scales(cfg, seed=4)
    assert s.shape == (720,) and s.min() >= 0.1 and s.max() <= 10.0
    logs = np.log10(s)
    assert abs(logs.mean()) < 0.1 and abs(logs.var() - 1 / 3) < 0.05
    x = ws.bf16_bits_to_f32(ws.make_input(cfg, seed=4)).astype(np.float64)
    per_feature_std = x.std(axis=(0, 2))
    assert np.allclose(per_feature_std / s, 1.0, atol=0.1)
