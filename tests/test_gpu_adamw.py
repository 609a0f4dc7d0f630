"""GPU parity of the fused AdamW step (dmuon_adamw_step) against the oracle.

Each step is checked element by element from the GPU's own state before the
step: moments to a few fp32 roundings of their terms, fp32 parameters to a few
roundings of the decayed parameter and of the update, bf16 parameters to
round-to-nearest of that fp32 value."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import newton_schulz_08_amd as nsa
from newton_schulz_08_amd import _lib
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits

from gpu_util import to_host_f64, ulp

pytestmark = pytest.mark.gpu

U = 2.0 ** -24   # fp32 unit roundoff


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()


def f32(x: float) -> float:
    return float(np.float32(x))


def _bf16_round(v: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(v.astype(np.float32)))


def _device(v: np.ndarray, dtype, unaligned: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda().to(dtype)
    if unaligned:
        # the tensor starts one element into its buffer: the element-wise path
        big = torch.zeros(t.numel() + 1, dtype=dtype, device="cuda")
        big[1:] = t
        t = big[1:]
        assert t.data_ptr() % 16 != 0
    return t


def check_adamw(before, after, step, hp, dtype):
    """before/after: (p, g, m, v) host fp64 arrays; hp: (lr, b1, b2, eps, wd)."""
    p0, g, m0, v0 = before
    p1, m1, v1 = after
    lr, b1, b2, eps, wd = hp
    pe, me, ve = oracle.adamw_step(p0, g, m0, v0, step, lr, b1, b2, eps, wd)
    mterm = b1 * np.abs(m0) + (1 - b1) * np.abs(g)
    vterm = b2 * v0 + (1 - b2) * g * g
    assert np.all(np.abs(m1 - me) <= 5 * U * mterm), "exp_avg outside 5 roundings of its terms"
    assert np.all(np.abs(v1 - ve) <= 5 * U * vterm), "exp_avg_sq outside 5 roundings of its terms"
    step_size = lr / (1 - b1 ** step)
    denom = np.sqrt(ve) / np.sqrt(1 - b2 ** step) + eps
    e32 = 4 * U * (np.abs(p0) + np.abs(pe)) + step_size * 16 * U * (mterm + np.abs(me)) / denom
    if dtype == torch.float32:
        bound = e32
    else:
        bound = 0.5 * ulp(np.abs(pe) + e32, "bf16") + e32
    err = np.abs(p1 - pe)
    bad = err > bound * 1.0000001
    assert not bad.any(), f"{int(bad.sum())} parameters out of bound; worst excess {np.max(err / bound):.3f}x"


def _draw(numels, seed, dtype):
    """Parameters like an embedding (N(0, 0.02)) or a norm weight (near 1),
    gradients with exact zeros, and nonzero moments as after earlier steps."""
    rng = np.random.default_rng(seed)
    out = []
    for i, n in enumerate(numels):
        p = rng.standard_normal(n) * 0.02 if i % 2 == 0 else 1.0 + 0.1 * rng.standard_normal(n)
        g = rng.standard_normal(n) * (1e-3 * 10 ** (i % 4))
        g[rng.random(n) < 0.05] = 0.0
        m = rng.standard_normal(n) * 1e-3
        v = rng.random(n) * 1e-5
        p32 = p.astype(np.float32)
        g32 = g.astype(np.float32)
        if dtype == torch.bfloat16:
            p32, g32 = _bf16_round(p32), _bf16_round(g32)
        out.append((p32, g32, m.astype(np.float32), v.astype(np.float32)))
    return out


NUMELS = [0, 1, 3, 4095, 4096, 4097, 12289, 1000 * 64, 3 * 4096 + 5]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("hp", [(1e-3, 0.9, 0.999, 1e-8, 0.01), (3e-2, 0.8, 0.95, 1e-6, 0.1), (1e-2, 0.0, 0.0, 1e-8, 0.0)],
                         ids=["guide_defaults", "large_lr", "betas_zero"])
def test_adamw_matches_oracle(dtype, hp):
    hp = tuple(f32(x) for x in hp)
    drawn = _draw(NUMELS, 90, dtype)
    unaligned = {2, 5}
    P = [_device(d[0], dtype, i in unaligned) for i, d in enumerate(drawn)]
    G = [_device(d[1], dtype, i in unaligned) for i, d in enumerate(drawn)]
    M = [_device(d[2], torch.float32, i in unaligned) for i, d in enumerate(drawn)]
    V = [_device(d[3], torch.float32, False) for d in drawn]
    ws = nsa.alloc_workspace(nsa.adamw_step_workspace_bytes(NUMELS))
    for step in (1, 2, 7):
        before = [tuple(to_host_f64(t) for t in (P[i], G[i], M[i], V[i])) for i in range(len(NUMELS))]
        nsa.adamw_step_(P, G, M, V, step, *hp[:1], betas=hp[1:3], eps=hp[3], weight_decay=hp[4], workspace=ws)
        torch.cuda.synchronize()
        for i in range(len(NUMELS)):
            check_adamw(before[i], tuple(to_host_f64(t) for t in (P[i], M[i], V[i])), step, hp, dtype)


def test_adamw_zero_state_first_step_closed_form():
    """From zero moments the first step moves each element by lr g / (|g| + eps)
    after decay: the bias corrections cancel the (1 - beta) factors."""
    n = 3 * 4096 + 17
    rng = np.random.default_rng(91)
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g[:64] = 0.0
    lr, wd, eps = f32(1e-3), f32(0.01), f32(1e-8)
    P, G = torch.from_numpy(p).cuda(), torch.from_numpy(g).cuda()
    M, V = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    nsa.adamw_step_([P], [G], [M], [V], 1, lr, betas=(0.9, 0.999), eps=eps, weight_decay=wd)
    got = to_host_f64(P)
    g64 = g.astype(np.float64)
    want = p.astype(np.float64) * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
    assert np.all(np.abs(got - want) <= 8 * U * (np.abs(want) + lr))
    assert not to_host_f64(M)[:64].any() and not to_host_f64(V)[:64].any()


def test_adamw_class_counts_steps():
    """AdamWStep keeps zeroed fp32 moments and advances the step counter."""
    n = 5000
    rng = np.random.default_rng(92)
    p = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    p_ref = p.clone()
    opt = nsa.AdamWStep([p], [g], lr=1e-3, weight_decay=0.0)
    opt()
    opt()
    m, v = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    nsa.adamw_step_([p_ref], [g], [m], [v], 1, 1e-3, weight_decay=0.0)
    nsa.adamw_step_([p_ref], [g], [m], [v], 2, 1e-3, weight_decay=0.0)
    assert opt.step == 2
    assert torch.equal(p, p_ref) and torch.equal(opt.exp_avg[0], m) and torch.equal(opt.exp_avg_sq[0], v)


def test_adamw_empty_and_rejects_misaligned():
    nsa.adamw_step_([], [], [], [], 1)
    # a bf16 parameter at an odd byte address is refused on the host
    raw = torch.zeros(32, dtype=torch.uint8, device="cuda")
    lib = _lib.load()
    m = torch.zeros(8, device="cuda")
    v = torch.zeros(8, device="cuda")
    ws = nsa.alloc_workspace(nsa.adamw_step_workspace_bytes([8]))
    one = lambda ptr: (ctypes.c_void_p * 1)(ptr)  # noqa: E731
    st = lib.dmuon_adamw_step(1, one(raw.data_ptr() + 1), one(raw.data_ptr() + 16), one(m.data_ptr()),
                              one(v.data_ptr()), (ctypes.c_int64 * 1)(4), _lib.DMUON_BF16, 1, ctypes.c_float(1e-3),
                              ctypes.c_float(0.9), ctypes.c_float(0.999), ctypes.c_float(1e-8), ctypes.c_float(0.0),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == _lib.DMUON_ERR_INVALID_ARG and "aligned" in _lib.last_error()


# Llama-3-8B's non-matrix parameters: token embedding and output head
# (128256 x 4096 each) and 65 RMSNorm weights of 4096.
LLAMA3_8B_ADAMW = [128256 * 4096, 128256 * 4096] + [4096] * 65


def test_adamw_full_size_sampled():
    """The bench's workload, bf16 parameters, step 5 from nonzero moments;
    sampled elements of every tensor against the oracle."""
    torch.manual_seed(93)
    dt = torch.bfloat16
    P = [torch.randn(n, device="cuda").mul_(0.02).to(dt) for n in LLAMA3_8B_ADAMW]
    G = [torch.randn(n, device="cuda").mul_(1e-3).to(dt) for n in LLAMA3_8B_ADAMW]
    M = [torch.randn(n, device="cuda").mul_(1e-4) for n in LLAMA3_8B_ADAMW]
    V = [torch.rand(n, device="cuda").mul_(1e-6) for n in LLAMA3_8B_ADAMW]
    gen = torch.Generator(device="cpu").manual_seed(94)
    idx = [torch.cat([torch.tensor([0, n - 1]), torch.randint(0, n, (4096,), generator=gen)]).cuda()
           for n in LLAMA3_8B_ADAMW]
    before = [tuple(to_host_f64(t[ix]) for t in (P[i], G[i], M[i], V[i])) for i, ix in enumerate(idx)]
    hp = tuple(f32(x) for x in (1e-3, 0.9, 0.999, 1e-8, 0.01))
    nsa.adamw_step_(P, G, M, V, 5, hp[0], betas=hp[1:3], eps=hp[3], weight_decay=hp[4])
    torch.cuda.synchronize()
    for i, ix in enumerate(idx):
        check_adamw(before[i], tuple(to_host_f64(t[ix]) for t in (P[i], M[i], V[i])), 5, hp, dt)
