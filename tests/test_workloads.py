"""Seeded input generators: determinism, independence, encodings (no GPU)."""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, get_config
from workloads import gen


def test_config_shapes():
    c1 = get_config("tinymlp_f32")
    assert c1.count == 12 and c1.total_numel() == 12 * 2048 * 512
    c4 = get_config("llama3_8b")
    assert c4.count == 224
    assert c4.total_numel() == 32 * (2 * 4096 * 4096 + 2 * 1024 * 4096 + 3 * 14336 * 4096)
    c5 = get_config("hybrid")
    assert c5.count == 432
    assert sum(m.numel < 100_000 for m in c5.matrices) == 96
    c2 = get_config("spectrum")
    assert c2.ns_only and c2.ns_steps == (3, 5, 7, 10)
    assert set(CONFIGS) == {"tinymlp_f32", "spectrum", "square4096", "llama3_8b", "hybrid"}


def test_streams_are_order_independent():
    cfg = get_config("tinymlp_f32")
    a = gen.draw_matrix(cfg, 5, gen.GRAD).values
    _ = gen.draw_matrix(cfg, 0, gen.GRAD)
    b = gen.draw_matrix(cfg, 5, gen.GRAD).values
    assert np.array_equal(a, b)
    assert not np.array_equal(a, gen.draw_matrix(cfg, 5, gen.WEIGHT).values)
    assert not np.array_equal(a, gen.draw_matrix(cfg, 6, gen.GRAD).values[: a.shape[0]])


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38], np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(gen.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_draw_values_are_exact():
    cfg = get_config("hybrid")
    d = gen.draw_matrix(cfg, 7, gen.GRAD)  # a_proj 2048 x 32, student-t
    assert d.dtype == "bf16" and d.bits.shape == (2048, 32)
    assert np.array_equal(gen.f32_to_bf16_bits(d.values), d.bits)


def test_haar_orthonormal():
    q = gen.haar_orthonormal(np.random.default_rng(1), 300, 40)
    assert np.abs(q.T @ q - np.eye(40)).max() < 1e-13


def test_spectrum_matrix():
    g, left, s, right = gen.spectrum_matrix(2, 0, 256, 1024)
    assert g.shape == (256, 1024) and s.min() >= 1e-3 and s.max() <= 1.0
    sv = np.linalg.svd(g, compute_uv=False)
    assert np.allclose(np.sort(sv), np.sort(s), rtol=1e-12, atol=1e-15)
    f32, b16 = gen.spectrum_copies(g)
    assert f32.bits is None and b16.bits is not None
    assert np.array_equal(gen.f32_to_bf16_bits(f32.values), b16.bits)


@pytest.mark.parametrize("key", ["tinymlp_f32", "square4096"])
def test_distribution_scale(key):
    cfg = get_config(key)
    d = gen.draw_matrix(cfg, 0, gen.GRAD)
    assert abs(float(d.values.std()) / cfg.grad_scale - 1.0) < 0.02
