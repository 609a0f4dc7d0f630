"""dmuon_muon_step_noalloc against dmuon_muon_step, through the C ABI.

The allocation-free entry point runs the same kernels on the library's static
scratch instead of a caller workspace, so its results must equal the
workspace entry point's bitwise: two calls in a row on the same GPU, the
second with a smaller set (the scratch keeps the first call's contents), in
both dtypes.  A set larger than the scratch is rejected before anything runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import newton_schulz_08_amd as nsa
from newton_schulz_08_amd import _lib
from workloads import gen
from workloads.configs import MatrixSpec, SetConfig

from gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()


def _arrays(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _shapes(shapes):
    n = len(shapes)
    return (ctypes.c_int64 * n)(*[s[0] for s in shapes]), (ctypes.c_int64 * n)(*[s[1] for s in shapes])


def _inputs(shapes, dtype, cfg_id):
    cfg = SetConfig(key=f"noalloc{cfg_id}", cfg_id=cfg_id,
                    matrices=tuple(MatrixSpec(f"m{i}", r, c) for i, (r, c) in enumerate(shapes)),
                    dtype=dtype, grad_dist="normal", grad_scale=1.0, weight_scale=1.0)
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(len(shapes))]
    p = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(len(shapes))]
    b = [to_device(gen.draw_matrix(cfg, i, gen.MOMENTUM)) for i in range(len(shapes))]
    return g, p, b


def _step(lib, shapes, dtype, g, p, b, noalloc, stream):
    """One step on clones of p and b; returns (params, momentum, update, norms)."""
    p = [t.clone() for t in p]
    b = [t.clone() for t in b]
    u = [torch.full(s, float("nan"), device="cuda") for s in shapes]
    norms = torch.full((len(shapes),), float("nan"), device="cuda")
    rows, cols = _shapes(shapes)
    dt = nsa.dtype_code(p[0].dtype)
    common = (len(shapes), _arrays(p), _arrays(g), _arrays(b), rows, cols, dt, 5, None, ctypes.c_float(0.9), 1,
              ctypes.c_float(0.02), ctypes.c_float(0.01), _lib.DMUON_LR_SCALE_MOONLIGHT, None, _arrays(u),
              ctypes.c_void_p(norms.data_ptr()))
    if noalloc:
        st = lib.dmuon_muon_step_noalloc(*common, ctypes.c_void_p(stream))
    else:
        need = nsa.muon_step_workspace_bytes(shapes, p[0].dtype)
        assert need <= _lib.DMUON_NOALLOC_SCRATCH_BYTES, need
        ws = nsa.alloc_workspace(need)
        st = lib.dmuon_muon_step(*common, ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(stream))
    assert st == 0, _lib.last_error()
    torch.cuda.synchronize()
    return p, b, u, norms


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point(dtype):
    lib = nsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    # a larger set first, then a smaller one, so the second call runs on
    # scratch that still holds the first call's iterate, Gram and partials
    sets = [[(1024, 2048), (2048, 1024), (600, 1100), (40, 60), (512, 768)],
            [(512, 768), (300, 700), (30, 40)]]
    for k, shapes in enumerate(sets):
        print(f"[noalloc] {dtype} call {k}: {shapes}", flush=True)
        g, p, b = _inputs(shapes, dtype, 600 + 2 * k + (dtype == "bf16"))
        want = _step(lib, shapes, dtype, g, p, b, False, stream)
        got = _step(lib, shapes, dtype, g, p, b, True, stream)
        for i, s in enumerate(shapes):
            for name, x, y in zip(("params", "momentum", "update"), (want[0][i], want[1][i], want[2][i]),
                                  (got[0][i], got[1][i], got[2][i])):
                assert torch.isfinite(y).all(), (name, s)
                assert torch.equal(x, y), (dtype, k, name, s)
        assert torch.equal(want[3], got[3])


def test_noalloc_rejects_sets_beyond_its_scratch():
    lib = nsa.load()
    shapes = [(4096, 4096)] * 2    # 2 x (3 x 32 MB + 32 MB) of bf16 scratch
    need = nsa.muon_step_workspace_bytes(shapes, torch.bfloat16)
    assert need > _lib.DMUON_NOALLOC_SCRATCH_BYTES
    g = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    p = [torch.ones(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    b = [torch.zeros(s, device="cuda") for s in shapes]
    rows, cols = _shapes(shapes)
    st = lib.dmuon_muon_step_noalloc(2, _arrays(p), _arrays(g), _arrays(b), rows, cols, _lib.DMUON_BF16, 5, None,
                                     ctypes.c_float(0.95), 1, ctypes.c_float(0.02), ctypes.c_float(0.0), 0, None, None,
                                     None, None)
    assert st == _lib.DMUON_ERR_WORKSPACE
    assert "DMUON_NOALLOC_SCRATCH_BYTES" in _lib.last_error()
    torch.cuda.synchronize()
    assert all(torch.equal(t, torch.ones_like(t)) for t in p)
