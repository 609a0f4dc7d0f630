"""Full-size parity: each configured matrix set runs as one batched call, in
the launch configuration the benchmark times.  Matrices the oracle can afford
(all of the small sets, a sample of every shape in the large ones) are
compared with it one by one; properties that hold at any size are checked on
every matrix."""
import numpy as np
import pytest
import torch

import oracle
import newton_schulz_08_amd as nsa
from workloads import gen, get_config
from workloads.device import make_set

from gpu_util import (TOL, check_update_faithful, f32_mu, max_ulp_err_f32, rel_fro, to_device, to_host_f64,
                      worst_tile_error)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()


def run_set(key, sample, ns_steps):
    cfg = get_config(key)
    print(f"[fullsize] {key}: {cfg.count} matrices, ns_steps={ns_steps}, sampled {sample}", flush=True)
    data = make_set(cfg, host_indices=sample)
    upd = [torch.empty(g.shape, device="cuda") if i in data["host"] else None for i, g in enumerate(data["grads"])]
    norms = torch.empty(cfg.count, device="cuda")
    step = nsa.MuonStep(data["params"], data["grads"], data["momentum"], ns_steps=ns_steps, mu=cfg.momentum,
                        nesterov=cfg.nesterov, lr=cfg.lr, update_out=upd, norms_out=norms)
    step()
    torch.cuda.synchronize()
    # any size: momentum from zero equals the gradient exactly; parameters stay finite
    for i in range(cfg.count):
        assert torch.equal(data["momentum"][i], data["grads"][i].float()), f"momentum {i}"
        assert torch.isfinite(data["params"][i]).all(), f"params {i}"
    assert torch.isfinite(norms).all()
    mu32 = f32_mu(cfg.momentum)
    worst = 0.0
    for i in sample:
        dg, dw = data["host"][i]
        spec = cfg.matrices[i]
        pw, bw, uw, nw = oracle.muon_step([dw.as_f64()], [dg.as_f64()], [np.zeros((spec.rows, spec.cols))], mu32,
                                          cfg.nesterov, ns_steps, cfg.lr)
        u = to_host_f64(upd[i])
        if spec.numel < oracle.MIN_NS_NUMEL:
            assert max_ulp_err_f32(u, uw[0]) <= 1.0, spec.name
        else:
            err = rel_fro(u, uw[0])
            worst = max(worst, err)
            terr, tij = worst_tile_error(u, uw[0])
            print(f"[fullsize] {key} {spec.name} {spec.rows}x{spec.cols}: rel err {err:.3e}, worst 256x256 tile "
                  f"{tij} {terr:.3e}", flush=True)
            assert err <= TOL[cfg.dtype], (spec.name, err)
            assert terr <= TOL[cfg.dtype], (spec.name, tij, terr)
        check_update_faithful(to_host_f64(data["params"][i]), dw.as_f64(), u, cfg.lr, 1.0, cfg.dtype)
        assert abs(norms[i].item() - nw[0]) <= 1e-5 * nw[0]
    del data, step
    torch.cuda.empty_cache()
    return worst


@pytest.mark.timeout(900)
def test_tinymlp_f32_all_matrices():
    cfg = get_config("tinymlp_f32")
    run_set("tinymlp_f32", list(range(cfg.count)), 5)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ns_steps", [5, 10])
def test_square4096_sampled(ns_steps):
    run_set("square4096", [0, 37], ns_steps)


@pytest.mark.timeout(1200)
def test_llama3_8b_sampled():
    # q of layer 0, k of layer 1, gate (tall) of layer 5, down (wide) of layer 31
    run_set("llama3_8b", [0, 8, 39, 223], 5)


@pytest.mark.timeout(900)
def test_hybrid_sampled():
    # q, gate (tall), down (wide), a_proj and b_proj (elementwise route) of layer 0, up of layer 20,
    # b_proj of layer 47
    run_set("hybrid", [0, 4, 6, 7, 8, 185, 431], 5)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_spectrum_set_all_steps(dtype):
    """Spectrum-controlled set through ns_batched: every matrix against the
    oracle for k in {3, 5, 7, 10}, and the orthogonality error (wide side) must
    not increase with k."""
    cfg = get_config("spectrum")
    xs, ins = [], []
    for i, spec in enumerate(cfg.matrices):
        g64 = gen.spectrum_matrix(cfg.cfg_id, i, spec.rows, spec.cols)[0]
        f32, b16 = gen.spectrum_copies(g64)
        d = f32 if dtype == "f32" else b16
        ins.append(d)
        xs.append(to_device(d))
    errs = {}
    for k in cfg.ns_steps:
        outs = nsa.ns_batched(xs, ns_steps=k)
        torch.cuda.synchronize()
        worst = 0.0
        for i, (d, o) in enumerate(zip(ins, outs)):
            u = to_host_f64(o)
            want = oracle.newton_schulz(d.as_f64(), k)
            err = rel_fro(u, want)
            assert err <= TOL[dtype], (i, k, err)
            terr, tij = worst_tile_error(u, want)
            assert terr <= TOL[dtype], (i, k, tij, terr)
            worst = max(worst, err)
            errs.setdefault(i, []).append(oracle.orthogonality_error(u))
        print(f"spectrum set {dtype} k={k}: worst relative Frobenius error {worst:.3e}", flush=True)
    floor = 1e-5 if dtype == "f32" else 5e-2
    for i, e in errs.items():
        for a, b in zip(e, e[1:]):
            assert b <= a + floor, (i, e)


@pytest.mark.timeout(600)
def test_spectrum_flat_recurrence_on_gpu():
    """A flat spectrum of rank r must come out with every singular value equal
    to the scalar recurrence f(s) = 1.5 s - 0.5 s^3 applied k times to
    1 / (sqrt(r) + eps) (fp32 path)."""
    rng = np.random.default_rng(5)
    for r, n in ((256, 1024), (1024, 256)):
        q = gen.haar_orthonormal(rng, max(r, n), min(r, n))
        x = (q.T if r < n else q).astype(np.float32)          # r x n, semi-orthogonal
        dx = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        for k in (3, 5, 10):
            out = nsa.ns_batched([dx], ns_steps=k)[0]
            sv = np.linalg.svd(out.double().cpu().numpy(), compute_uv=False)
            s = 1.0 / (np.sqrt(min(r, n)) + 1e-7)
            for _ in range(k):
                s = 1.5 * s - 0.5 * s ** 3
            assert np.max(np.abs(sv - s)) < 1e-5, (r, n, k, sv.min(), sv.max(), s)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["llama3_8b", "hybrid"])
def test_every_matrix_independent_of_batch_order(key):
    """Every matrix of a full-size set, through every tile of the batched
    launches: the step must give bitwise the same update and parameters when
    the batch is passed in reverse order, which moves each matrix's tiles to
    other workgroups and tile-order rounds, and to other XCDs wherever a
    shape's tile count is not a multiple of 256 (every shape group of these
    sets has an even count, so no matrix keeps its place).  A tile that a
    launch skipped or computed twice at some position would differ; a fault
    tied to a tile's place within a round is left to the oracle comparisons
    of the sampled tests."""
    cfg = get_config(key)
    print(f"[fullsize] {key}: every matrix, forward and reversed batch order", flush=True)
    results = []
    for order in (list(range(cfg.count)), list(range(cfg.count))[::-1]):
        data = make_set(cfg)
        upd = [torch.empty(g.shape, device="cuda") for g in data["grads"]]

        def pick(xs):
            return [xs[i] for i in order]

        step = nsa.MuonStep(pick(data["params"]), pick(data["grads"]), pick(data["momentum"]),
                            ns_steps=cfg.ns_steps[0], mu=cfg.momentum, nesterov=cfg.nesterov, lr=cfg.lr,
                            update_out=pick(upd))
        step()
        torch.cuda.synchronize()
        results.append((upd, data["params"]))
        del data, step
    (u0, p0), (u1, p1) = results
    for i, spec in enumerate(cfg.matrices):
        assert torch.isfinite(u0[i]).all(), spec.name
        assert torch.equal(u0[i], u1[i]), (i, spec.name)
        assert torch.equal(p0[i], p1[i]), (i, spec.name)
    del results, u0, u1, p0, p1
    torch.cuda.empty_cache()
