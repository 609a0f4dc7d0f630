"""GPU parity of per-segment gradient clipping (dmuon_clip_grad_norm) against
the oracle: totals to fp32-accumulation accuracy, clipped gradients bit for bit
given the GPU's own total."""
import math

import numpy as np
import pytest
import torch

import oracle
import newton_schulz_08_amd as nsa
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits

from gpu_util import to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()


def _round(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32.astype(np.float32).astype(np.float64)
    return bf16_bits_to_f32(f32_to_bf16_bits(x32.astype(np.float32))).astype(np.float64)


def _expected_coef(max_norm: float, total_gpu: float) -> np.float32:
    """The coefficient as the kernel forms it: fp32, clamped at 1."""
    c = np.float32(max_norm) / (np.float32(total_gpu) + np.float32(1e-6))
    return np.float32(1.0) if c >= 1.0 else np.float32(c)


def _make(shapes, dtype, seed):
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for i, n in enumerate(shapes):
        v = (rng.standard_normal(n) * (0.5 + i)).astype(np.float32)
        if dtype == "bf16":
            v = bf16_bits_to_f32(f32_to_bf16_bits(v))
        host.append(v.astype(np.float64))
        t = torch.from_numpy(v).cuda()
        t = t if dtype == "f32" else t.to(torch.bfloat16)
        if i == 1:
            # an unaligned view: the tensor starts one element into a buffer
            big = torch.zeros(n + 1, dtype=t.dtype, device="cuda")
            big[1:] = t
            t = big[1:]
            assert t.data_ptr() % 16 != 0
        dev.append(t)
    return host, dev


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm_type", [2.0, 1.0, math.inf, 3.0])
def test_clip_matches_oracle(dtype, norm_type):
    shapes = [5000, 4097, 0, 3, 70000, 12288, 1]
    segs = [0, 0, 1, 2, 1, 2, 0]
    host, dev = _make(shapes, dtype, 7 + int(min(norm_type, 9)))
    _, want_t = oracle.clip_grad_norm_buckets(host, segs, [1.0, 1.0, 1.0], norm_type)
    # segment 0 and 2 clip, segment 1 does not
    max_norms = [want_t[0] * 0.25, want_t[1] * 4.0, want_t[2] * 0.5]
    want, want_t = oracle.clip_grad_norm_buckets(host, segs, max_norms, norm_type)
    totals = nsa.clip_grad_norm_(dev, max_norms, segs, norm_type)
    torch.cuda.synchronize()
    tg = totals.cpu().numpy().astype(np.float64)
    for s in range(3):
        if math.isinf(norm_type):
            assert tg[s] == want_t[s], (s, tg[s], want_t[s])
        else:
            assert abs(tg[s] - want_t[s]) <= 2e-6 * want_t[s], (s, tg[s], want_t[s])
    for i, (h, d, s) in enumerate(zip(host, dev, segs)):
        got = to_host_f64(d)
        coef = _expected_coef(max_norms[s], tg[s])
        expect = _round(h.astype(np.float32) * coef, dtype)
        assert np.array_equal(got, expect), f"tensor {i} (segment {s}) differs from round(g * coef)"
        if s == 1:
            assert np.array_equal(got, h), "an unclipped segment must be left unchanged"
        if h.size:
            assert np.allclose(got, want[i], rtol=4e-6 if dtype == "f32" else 8e-3, atol=0)


def test_clip_deterministic_and_large():
    rng = np.random.default_rng(3)
    g = torch.from_numpy((rng.standard_normal(48 * 1024 * 1024) * 1e-3).astype(np.float32)).cuda()
    a, b = g.clone().to(torch.bfloat16), g.clone().to(torch.bfloat16)
    ta = nsa.clip_grad_norm_([a], 0.01)
    tb = nsa.clip_grad_norm_([b], 0.01)
    torch.cuda.synchronize()
    assert torch.equal(ta, tb) and torch.equal(a, b)
    h = to_host_f64(g.to(torch.bfloat16))
    want = float(np.sqrt(np.sum(h * h)))
    assert abs(ta.item() - want) <= 2e-6 * want


def test_clip_nonfinite_total():
    g = torch.tensor([1.0, float("inf"), 2.0], device="cuda")
    h = torch.tensor([3.0, 4.0], device="cuda")
    t = nsa.clip_grad_norm_([g, h], [1.0, 10.0], [0, 1])
    torch.cuda.synchronize()
    assert math.isinf(t[0].item()) and t[1].item() == 5.0
    assert g[0].item() == 0.0 and g[2].item() == 0.0     # coef = 1 / inf = 0
    assert torch.equal(h, torch.tensor([3.0, 4.0], device="cuda"))
