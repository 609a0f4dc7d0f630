"""Stream capture: every compute entry point refuses a stream that is capturing
a graph, enqueues nothing, and leaves the library usable afterwards.

Each call uploads its descriptors from host memory that lives only for the
call, so a recorded copy would read freed memory when the graph is replayed;
the library refuses instead of recording it."""
import ctypes
import warnings

import pytest
import torch

import newton_schulz_08_amd as nsa
from newton_schulz_08_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()


def _status_under_capture(fn):
    """Run fn while torch captures a graph on its side stream; return the
    library's status (None if fn did not raise)."""
    g = torch.cuda.CUDAGraph()
    status = None
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")  # torch warns that the captured graph is empty
        with torch.cuda.graph(g):
            try:
                fn()
            except nsa.DmuonError as e:
                status = e.status
    torch.cuda.synchronize()
    return status


def test_every_entry_point_refuses_capture():
    torch.manual_seed(0)
    p = torch.randn(256, 512, device="cuda")
    g = torch.randn(256, 512, device="cuda")
    mom = torch.randn(256, 512, device="cuda")
    x = torch.randn(300, 512, device="cuda")
    out = torch.zeros_like(x)
    m = torch.randn(1000, device="cuda")
    v = torch.rand(1000, device="cuda")
    pa, ga = torch.randn(1000, device="cuda"), torch.randn(1000, device="cuda")
    before = [t.clone() for t in (p, g, mom, x, out, m, v, pa, ga)]

    step = nsa.MuonStep([p], [g], [mom], ns_steps=3)
    clipped = nsa.MuonStep([p], [g], [mom], ns_steps=3, clip_max_norm=0.5)
    lib = nsa.load()

    def noalloc():
        P = ctypes.c_void_p * 1
        rows, cols = (ctypes.c_int64 * 1)(256), (ctypes.c_int64 * 1)(512)
        st = lib.dmuon_muon_step_noalloc(1, P(p.data_ptr()), P(g.data_ptr()), P(mom.data_ptr()), rows, cols,
                                         _lib.DMUON_F32, 3, None, ctypes.c_float(0.95), 1, ctypes.c_float(0.02),
                                         ctypes.c_float(0.0), 0, None, None, None,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        _lib.check(st, "dmuon_muon_step_noalloc")
    ws_ns = nsa.alloc_workspace(nsa.ns_workspace_bytes([tuple(x.shape)], x.dtype))
    ws_clip = nsa.alloc_workspace(nsa.clip_grad_norm_workspace_bytes([ga.numel()]))
    ws_adam = nsa.alloc_workspace(nsa.adamw_step_workspace_bytes([pa.numel()]))
    torch.cuda.synchronize()

    calls = {
        "muon_step": lambda: step(),
        "muon_step_clipped": lambda: clipped(),
        "muon_step_noalloc": noalloc,
        "ns_batched": lambda: nsa.ns_batched([x], [out], ns_steps=3, workspace=ws_ns),
        "clip_grad_norm": lambda: nsa.clip_grad_norm_([ga], 0.5, workspace=ws_clip),
        "adamw_step": lambda: nsa.adamw_step_([pa], [ga], [m], [v], 1, workspace=ws_adam),
    }
    for name, fn in calls.items():
        assert _status_under_capture(fn) == _lib.DMUON_ERR_INVALID_ARG, name
        assert "capturing" in _lib.last_error(), name
    # nothing was enqueued
    for i, (t, b) in enumerate(zip((p, g, mom, x, out, m, v, pa, ga), before)):
        assert torch.equal(t, b), i
    # and the same calls still run eagerly afterwards
    step()
    nsa.ns_batched([x], [out], ns_steps=3, workspace=ws_ns)
    torch.cuda.synchronize()
    assert not torch.equal(p, before[0])
    assert torch.isfinite(out).all() and out.abs().sum() > 0
