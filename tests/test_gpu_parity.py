"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element on seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import newton_schulz_08_amd as nsa
from workloads import gen
from workloads.configs import MatrixSpec, SetConfig, get_config

from gpu_util import (TOL, TORCH_DT, check_update_faithful, f32_mu, gpu_lr_scale, max_ulp_err_f32, rel_fro,
                      to_device, to_host_f64, ulp, worst_tile_error)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsa.load()
    print("backend:", nsa.backend_info(), flush=True)


def _adhoc(shapes, dtype, cfg_id, grad_dist="normal", grad_scale=1.0):
    return SetConfig(key=f"adhoc{cfg_id}", cfg_id=cfg_id,
                     matrices=tuple(MatrixSpec(f"m{i}", r, c) for i, (r, c) in enumerate(shapes)),
                     dtype=dtype, grad_dist=grad_dist, grad_scale=grad_scale, weight_scale=1.0)


def run_muon(cfg, *, ns_steps=5, mu=0.95, nesterov=True, lr=0.02, lr_scale=None, nonzero_buf=False,
             with_update=True, weight_decay=0.0, moonlight=False, ns_coeffs=None, ns_backend="gram"):
    """One dmuon_muon_step over every matrix of cfg; returns host copies."""
    n = cfg.count
    g = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(n)]
    p = [gen.draw_matrix(cfg, i, gen.WEIGHT) for i in range(n)]
    b = [gen.draw_matrix(cfg, i, gen.MOMENTUM) if nonzero_buf else None for i in range(n)]
    dg = [to_device(x) for x in g]
    dp = [to_device(x) for x in p]
    db = [to_device(x) if x is not None else torch.zeros(x_.values.shape, dtype=torch.float32, device="cuda")
          for x, x_ in zip(b, g)]
    du = [torch.full(x.values.shape, float("nan"), dtype=torch.float32, device="cuda") for x in g] \
        if with_update else None
    norms = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    nsa.muon_step(dp, dg, db, ns_steps=ns_steps, mu=mu, nesterov=nesterov, lr=lr, lr_scale=lr_scale,
                  update_out=du, norms_out=norms, weight_decay=weight_decay,
                  lr_scale_mode="moonlight" if moonlight else "one", ns_coeffs=ns_coeffs, ns_backend=ns_backend)
    torch.cuda.synchronize()
    return dict(
        g=[x.as_f64() for x in g], p0=[x.as_f64() for x in p],
        b0=[x.as_f64() if x is not None else np.zeros(x_.values.shape) for x, x_ in zip(b, g)],
        p=[to_host_f64(t) for t in dp], b=[to_host_f64(t) for t in db],
        u=[to_host_f64(t) for t in du] if with_update else None,
        norms=norms.cpu().numpy().astype(np.float64))


def check_against_oracle(cfg, res, *, ns_steps=5, mu=0.95, nesterov=True, lr=0.02, lr_scale=None,
                         indices=None, weight_decay=0.0, moonlight=False, ns_coeffs=None):
    dtype = cfg.dtype
    mu32 = f32_mu(mu)
    indices = range(cfg.count) if indices is None else indices
    worst = 0.0
    for i in indices:
        spec = cfg.matrices[i]
        s = 1.0 if lr_scale is None else float(lr_scale[i])
        pw, bw, uw, nw = oracle.muon_step([res["p0"][i]], [res["g"][i]], [res["b0"][i]], mu32, nesterov,
                                          ns_steps, lr, [s], weight_decay=weight_decay, moonlight=moonlight,
                                          ns_coeffs=ns_coeffs)
        # momentum: one fused multiply-add in fp32 -> within one fp32 ulp
        e = max_ulp_err_f32(res["b"][i], bw[0])
        assert e <= 1.0, f"{spec.name}: momentum off by {e:.2f} ulp"
        assert abs(res["norms"][i] - nw[0]) <= 1e-5 * nw[0] + 1e-30, (spec.name, res["norms"][i], nw[0])
        if res["u"] is not None:
            u = res["u"][i]
            assert np.all(np.isfinite(u)), spec.name
            if spec.numel < oracle.MIN_NS_NUMEL:
                # U = fma(mu, buf', g) rounded once, from the GPU's own buf'
                y_exact = res["g"][i] + mu32 * res["b"][i] if nesterov else res["b"][i]
                eu = max_ulp_err_f32(u, y_exact)
                assert eu <= 1.0, f"{spec.name}: elementwise-route update off by {eu:.2f} ulp"
                # against the oracle: buf' rounding (<= 1 ulp) propagates through mu
                bound = mu32 * ulp(bw[0], "f32") + ulp(uw[0], "f32")
                assert np.all(np.abs(u - uw[0]) <= bound * 1.0000001), spec.name
            else:
                err = rel_fro(u, uw[0])
                worst = max(worst, err)
                assert err <= TOL[dtype], f"{spec.name} {spec.rows}x{spec.cols}: rel err {err:.3e} > {TOL[dtype]}"
                terr, tij = worst_tile_error(u, uw[0])
                assert terr <= TOL[dtype], f"{spec.name} {spec.rows}x{spec.cols}: tile {tij} rel err {terr:.3e}"
            check_update_faithful(res["p"][i], res["p0"][i], u, lr, gpu_lr_scale(s, spec.rows, spec.cols, moonlight),
                                  dtype, weight_decay)
    return worst


# ------------------------------------------------------------------ maximum dimension
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maximum_dimension(dtype):
    """A wide and a tall matrix at DMUON_MAX_DIM (65536) on their long side, with
    ragged short sides: the largest row pitches and operand offsets any call can
    produce."""
    cfg = _adhoc([(200, 65536), (65536, 300)], dtype, 71)
    res = run_muon(cfg, ns_steps=3)
    check_against_oracle(cfg, res, ns_steps=3)


# ------------------------------------------------------------------ small / ragged
RAGGED = [(600, 1100), (1100, 600), (300, 700), (257, 1000), (1000, 130), (250, 400), (3, 33333),
          (50, 70), (2048, 32), (512, 512)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_batch(dtype):
    cfg = _adhoc(RAGGED, dtype, 101 if dtype == "f32" else 102)
    res = run_muon(cfg)
    worst = check_against_oracle(cfg, res)
    print(f"ragged {dtype}: worst NS rel err {worst:.3e}", flush=True)


def _random_shapes(seed, n=24):
    """Seeded shapes across the cases the launch planner distinguishes: tiny and odd
    sizes, each side of the 256 tile and the 512 small-tile bounds, log-uniform
    sizes up to 1200 in both orientations (numel < 100000 takes the
    elementwise route)."""
    rng = np.random.default_rng(seed)
    edges = [255, 256, 257, 511, 512, 513]
    shapes = []
    for i in range(n):
        if i < 4:
            a, b = (int(x) for x in rng.integers(1, 41, size=2))
        elif i < 10:
            a, b = edges[i - 4], int(rng.integers(200, 1101))
        else:
            a, b = (int(x) for x in np.exp(rng.uniform(np.log(24.0), np.log(1200.0), size=2)).round())
        shapes.append((a, b) if rng.integers(2) else (b, a))
    return shapes


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_shapes(dtype):
    """One call over 24 seeded shapes of every kind at once (both routes, both
    orientations, ragged and tile-edge sizes); every matrix against the oracle."""
    shapes = _random_shapes(2024 if dtype == "f32" else 2025)
    print(f"random shapes {dtype}: {shapes}", flush=True)
    cfg = _adhoc(shapes, dtype, 140 + (dtype == "bf16"))
    res = run_muon(cfg, nonzero_buf=True)
    worst = check_against_oracle(cfg, res)
    print(f"random shapes {dtype}: worst NS rel err {worst:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("nesterov", [True, False])
def test_nonzero_momentum_and_lr_scale(dtype, nesterov):
    shapes = [(384, 640), (640, 384), (40, 60)]
    cfg = _adhoc(shapes, dtype, 110 + (dtype == "bf16") * 2 + nesterov)
    scale = [oracle.moonlight_lr_scale(r, c) for r, c in shapes]
    res = run_muon(cfg, nonzero_buf=True, nesterov=nesterov, lr_scale=scale, mu=0.9, lr=0.01)
    check_against_oracle(cfg, res, nesterov=nesterov, lr_scale=scale, mu=0.9, lr=0.01)


@pytest.mark.parametrize("steps", [0, 1, 2, 7])
def test_step_counts(steps):
    cfg = _adhoc([(512, 768), (768, 512)], "f32", 120 + steps)
    res = run_muon(cfg, ns_steps=steps)
    check_against_oracle(cfg, res, ns_steps=steps)


def test_worked_example_small_route(golden):
    fx = golden("momentum_worked_example.txt")
    for dt in (torch.float32, torch.bfloat16):
        for nesterov, tag in ((True, "nesterov"), (False, "plain")):
            t = lambda k, d=dt: torch.tensor(fx[k], dtype=d, device="cuda").reshape(2, 2)  # noqa: E731
            p, g, b = t("p0"), t("grad"), t("buf0", torch.float32)
            u = torch.empty(2, 2, dtype=torch.float32, device="cuda")
            nsa.muon_step([p], [g], [b], ns_steps=5, mu=fx["mu"][0], nesterov=nesterov, lr=fx["lr"][0],
                          update_out=[u])
            torch.cuda.synchronize()
            assert b.cpu().flatten().tolist() == fx["buf1"]
            assert u.cpu().flatten().tolist() == fx["y_" + tag]
            assert p.float().cpu().flatten().tolist() == fx["p1_" + tag]


def test_zero_gradient_gives_zero_update():
    for dt in (torch.float32, torch.bfloat16):
        g = torch.zeros(512, 1024, dtype=dt, device="cuda")
        p = torch.randn(512, 1024, device="cuda").to(dt)
        p0 = p.clone()
        b = torch.zeros(512, 1024, device="cuda")
        u = torch.full((512, 1024), float("nan"), device="cuda")
        norms = torch.full((1,), float("nan"), device="cuda")
        nsa.muon_step([p], [g], [b], update_out=[u], norms_out=norms)
        torch.cuda.synchronize()
        assert torch.equal(p, p0)
        assert torch.count_nonzero(u).item() == 0
        assert norms.item() == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rank_one_gradient(dtype):
    """A rank-one gradient u v^T: its normalised singular value is 1, a fixed
    point of every step of the cubic map, so U = u v^T / (|u| |v|)."""
    rng = np.random.default_rng(72)
    for rows, cols in ((384, 1000), (1000, 384)):
        uvec, vvec = rng.standard_normal(rows), rng.standard_normal(cols)
        g64 = np.outer(uvec, vvec)
        g = torch.from_numpy(g64.astype(np.float32)).cuda().to(TORCH_DT[dtype])
        gh = to_host_f64(g)                      # the exact input after rounding to dtype
        out = nsa.ns_batched([g], ns_steps=5)[0]
        want = oracle.newton_schulz(gh, 5)
        closed = g64 / (np.linalg.norm(uvec) * np.linalg.norm(vvec))
        got = to_host_f64(out)
        assert rel_fro(got, want) <= TOL[dtype]
        assert rel_fro(got, closed) <= TOL[dtype]


def test_nonfinite_matrix_does_not_leak():
    """A NaN in one matrix's gradient makes that matrix's update NaN (its norm is
    NaN) and leaves every other matrix of the batch exactly as when it runs alone."""
    cfg = _adhoc([(512, 768), (256, 1024)], "bf16", 73)
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(2)]
    p = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(2)]
    g[0][3, 5] = float("nan")
    pa = [t.clone() for t in p]
    u = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in p]
    nsa.muon_step(pa, g, [torch.zeros(t.shape, device="cuda") for t in p], update_out=u)
    pb = p[1].clone()
    ub = torch.zeros(pb.shape, dtype=torch.float32, device="cuda")
    nsa.muon_step([pb], [g[1]], [torch.zeros(pb.shape, device="cuda")], update_out=[ub])
    torch.cuda.synchronize()
    assert torch.isnan(u[0]).all()
    assert torch.equal(u[1], ub) and torch.equal(pa[1], pb)


def test_empty_batch_is_noop():
    assert nsa.ns_batched([]) == []
    lib = nsa.load()
    assert lib.dmuon_muon_step(0, None, None, None, None, None, 0, 5, None, 0.95, 1, 0.02, 0.0, 0, None, None, None,
                               None, 0, None) == 0


def test_route_boundary():
    # 99,999 elements -> elementwise; 100,000 -> Newton-Schulz
    cfg = _adhoc([(3, 33333), (250, 400), (400, 250)], "f32", 130)
    res = run_muon(cfg)
    check_against_oracle(cfg, res)
    u_small = res["u"][0]
    y = res["g"][0] * (1.0 + f32_mu(0.95))
    assert max_ulp_err_f32(u_small, y) <= 1.0


# ------------------------------------------------------------------ determinism / invariance
def test_bitwise_determinism_and_batch_invariance():
    shapes = [(512, 1024), (1024, 512), (256, 300)]
    cfg = _adhoc(shapes, "bf16", 140)
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(3)]
    p0 = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(3)]

    def once(idx):
        p = [p0[i].clone() for i in idx]
        b = [torch.zeros(shapes[i], device="cuda") for i in idx]
        u = [torch.empty(shapes[i], device="cuda") for i in idx]
        nsa.muon_step(p, [g[i] for i in idx], b, update_out=u)
        torch.cuda.synchronize()
        return p, b, u

    pa, ba, ua = once([0, 1, 2])
    pb, bb, ub = once([0, 1, 2])
    pc, bc, uc = once([2, 0])
    for x, y in zip(pa + ba + ua, pb + bb + ub):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x, y.view(torch.uint8)
                           if y.dtype == torch.bfloat16 else y)
    assert torch.equal(ua[2], uc[0]) and torch.equal(ua[0], uc[1])
    assert torch.equal(pa[2].view(torch.int16), pc[0].view(torch.int16))


def test_update_out_does_not_change_params():
    shapes = [(512, 768), (768, 512), (30, 40)]
    cfg = _adhoc(shapes, "bf16", 150)
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(3)]
    p0 = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(3)]
    outs = []
    for with_u in (False, True):
        p = [x.clone() for x in p0]
        b = [torch.zeros(s, device="cuda") for s in shapes]
        u = [torch.empty(s, device="cuda") for s in shapes] if with_u else None
        nsa.muon_step(p, g, b, update_out=u)
        torch.cuda.synchronize()
        outs.append(p)
    for x, y in zip(*outs):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_two_steps_nesterov():
    """Two consecutive steps from a zero buffer (distinguishes the Nesterov
    readings: the second step's input is G2 + mu (mu G1 + G2))."""
    shapes = [(512, 640), (640, 512)]
    cfg = _adhoc(shapes, "f32", 160)
    g1 = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(2)]
    g2 = [gen.draw_matrix(cfg, i, gen.GRAD2) for i in range(2)]
    p0 = [gen.draw_matrix(cfg, i, gen.WEIGHT) for i in range(2)]
    dp = [to_device(x) for x in p0]
    db = [torch.zeros(s, device="cuda") for s in shapes]
    du = [torch.empty(s, device="cuda") for s in shapes]
    step = nsa.MuonStep(dp, [to_device(x) for x in g1], db, update_out=du)
    step()
    dg2 = [to_device(x) for x in g2]
    step2 = nsa.MuonStep(dp, dg2, db, update_out=du, workspace=step.workspace)
    step2()
    torch.cuda.synchronize()
    mu = f32_mu(0.95)
    for i in range(2):
        pw, bw, uw, _ = oracle.muon_step([p0[i].as_f64()], [g1[i].as_f64()], [np.zeros(shapes[i])], mu, True, 5,
                                         0.02)
        pw, bw, uw, _ = oracle.muon_step(pw, [g2[i].as_f64()], bw, mu, True, 5, 0.02)
        assert rel_fro(to_host_f64(du[i]), uw[0]) <= TOL["f32"]
        assert max_ulp_err_f32(to_host_f64(db[i]), bw[0]) <= 2.0
        assert rel_fro(to_host_f64(dp[i]), pw[0]) < 1e-6


# ------------------------------------------------------------------ ns_batched
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ns_batched_ragged(dtype):
    shapes = [(300, 700), (700, 300), (40, 50), (256, 256), (520, 1030)]
    cfg = _adhoc(shapes, dtype, 170 + (dtype == "bf16"))
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    outs = nsa.ns_batched([to_device(x) for x in xs], ns_steps=5)
    torch.cuda.synchronize()
    for x, o, s in zip(xs, outs, shapes):
        err = rel_fro(to_host_f64(o), oracle.newton_schulz(x.as_f64(), 5))
        assert err <= TOL[dtype], (s, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ns_steps", [3, 7])
def test_ns_batched_random_shapes(dtype, ns_steps):
    """Newton-Schulz alone (every matrix orthogonalised, tiny ones included)
    over 24 seeded shapes in one call, each against the oracle."""
    shapes = _random_shapes(3000 + ns_steps + 10 * (dtype == "bf16"))
    cfg = _adhoc(shapes, dtype, 180 + ns_steps + 10 * (dtype == "bf16"))
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    outs = nsa.ns_batched([to_device(x) for x in xs], ns_steps=ns_steps)
    torch.cuda.synchronize()
    worst = 0.0
    for x, o, sh in zip(xs, outs, shapes):
        err = rel_fro(to_host_f64(o), oracle.newton_schulz(x.as_f64(), ns_steps))
        assert err <= TOL[dtype], (sh, err)
        worst = max(worst, err)
    print(f"ns_batched random shapes {dtype} k={ns_steps}: worst rel err {worst:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_gram_ablation_matches(dtype, monkeypatch):
    """DMUON_NS_KERNEL=gemm (every Gram tile, no mirror) gives the default
    path's result to rounding and meets the oracle tolerance."""
    shapes = [(520, 1030), (1030, 520), (768, 768)]
    cfg = _adhoc(shapes, dtype, 180 + (dtype == "bf16"))
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    ref = nsa.ns_batched([to_device(x) for x in xs], ns_steps=5)
    monkeypatch.setenv("DMUON_NS_KERNEL", "gemm")
    full = nsa.ns_batched([to_device(x) for x in xs], ns_steps=5)
    torch.cuda.synchronize()
    for x, r, f, s in zip(xs, ref, full, shapes):
        assert rel_fro(to_host_f64(f), to_host_f64(r)) <= TOL[dtype] / 10, s
        assert rel_fro(to_host_f64(f), oracle.newton_schulz(x.as_f64(), 5)) <= TOL[dtype], s


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_gram_runs_in_k_slices(dtype):
    """A matrix of at most two 256-tile rows has its Gram product cut into K
    slices and summed by a second launch (2 Gram launches per step; fp32 on
    128 x 128 tiles, in 2 slices when n' >= 1024); three tile rows or more
    take one.  Split and unsplit shapes in one batch, the
    square product of a three-term map, and the direct backend all meet the
    oracle."""
    shapes = [(300, 2100), (2100, 300), (256, 1024), (800, 1500)]
    cfg = _adhoc(shapes, dtype, 190 + (dtype == "bf16"))
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    steps = 4
    for split, launches in (([0, 1, 2], 2 * steps), ([3], steps)):
        nsa.profile_read()
        nsa.profile_enable(True)
        nsa.ns_batched([to_device(xs[i]) for i in split], ns_steps=steps)
        torch.cuda.synchronize()
        nsa.profile_enable(False)
        assert nsa.profile_read()["syrk"]["launches"] == launches, split
    for kw in ({}, {"ns_backend": "direct"}, {"ns_coeffs": QUINTIC_CLASSICAL}):
        outs = nsa.ns_batched([to_device(x) for x in xs], ns_steps=steps, **kw)
        torch.cuda.synchronize()
        for x, o, sh in zip(xs, outs, shapes):
            want = oracle.newton_schulz(x.as_f64(), steps, coeffs=kw.get("ns_coeffs"))
            assert rel_fro(to_host_f64(o), want) <= TOL[dtype], (kw, sh)


QUINTIC_FAST = (3.4445, -4.7750, 2.0315)
QUINTIC_CLASSICAL = (1.875, -1.25, 0.375)


def test_small_fp32_tiles():
    """fp32 matrices with m' <= 512 run on 128 x 128 tiles in launches of their
    own: m' of 256 and 512, both orientations, n' below 1024 (one Gram slice)
    and above (two), ragged edges, beside a shape group on 256 x 256 tiles in
    the same call.  The Muon step (the last Newton-Schulz step writing the
    caller's parameters in their own orientation, update_out, weight decay,
    Moonlight scale, non-zero momentum), the three-term square product and
    the direct backend all meet the oracle, whole matrix and per tile."""
    shapes = [(300, 900), (900, 300), (500, 2100), (2100, 500), (129, 1000), (250, 700), (700, 250), (513, 1500)]
    cfg = _adhoc(shapes, "f32", 250)
    print("[parity] small fp32 tiles", flush=True)
    nsa.profile_read()
    nsa.profile_enable(True)
    res = run_muon(cfg, nonzero_buf=True, weight_decay=0.1, moonlight=True)
    nsa.profile_enable(False)
    prof = nsa.profile_read()
    assert prof["ns_gemm"]["launches"] == 2 * 5          # a 128-tile and a 256-tile update table
    assert prof["syrk"]["launches"] == 3 * 5             # both Gram tables and the small tiles' slice sums
    check_against_oracle(cfg, res, weight_decay=0.1, moonlight=True)
    for kw in ({"ns_coeffs": QUINTIC_FAST}, {"ns_backend": "direct"}):
        res = run_muon(cfg, **kw)
        check_against_oracle(cfg, res, ns_coeffs=kw.get("ns_coeffs"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_weight_decay_and_moonlight_scale(dtype):
    """Decoupled decay and the 0.2*sqrt(max(m, n)) multiplier, on both routes."""
    shapes = [(384, 640), (640, 384), (40, 60), (2048, 32)]
    cfg = _adhoc(shapes, dtype, 190 + (dtype == "bf16"))
    scale = [1.0, 0.5, 2.0, 1.5]
    res = run_muon(cfg, nonzero_buf=True, weight_decay=0.1, lr_scale=scale, moonlight=True)
    check_against_oracle(cfg, res, weight_decay=0.1, lr_scale=scale, moonlight=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_custom_coefficients_ns_batched(dtype):
    """Odd-polynomial maps: two- and three-term, fixed and per-step, against the
    oracle; the direct backend gives the same result as the gram one."""
    shapes = [(520, 1030), (1030, 520), (256, 768), (300, 700)]
    cfg = _adhoc(shapes, dtype, 200 + (dtype == "bf16"))
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    dxs = [to_device(x) for x in xs]
    schedules = [(QUINTIC_FAST, 5), (QUINTIC_CLASSICAL, 5), ([QUINTIC_FAST] * 3 + [(1.5, -0.5)] * 2, 5),
                 ((1.6, -0.6), 4), ([(2.0, -1.5, 0.5), (1.5, -0.5, 0.0)], 2)]
    for coeffs, k in schedules:
        outs = nsa.ns_batched(dxs, ns_steps=k, ns_coeffs=coeffs)
        torch.cuda.synchronize()
        for x, o, sh in zip(xs, outs, shapes):
            err = rel_fro(to_host_f64(o), oracle.newton_schulz(x.as_f64(), k, coeffs))
            print(f"coeffs {coeffs if not isinstance(coeffs, list) else 'schedule'} k={k} {sh}: {err:.3e}", flush=True)
            assert err <= TOL[dtype], (coeffs, k, sh, err)
    gram = nsa.ns_batched(dxs, ns_steps=5, ns_coeffs=QUINTIC_FAST)
    direct = nsa.ns_batched(dxs, ns_steps=5, ns_coeffs=QUINTIC_FAST, ns_backend="direct")
    torch.cuda.synchronize()
    for g_, d_ in zip(gram, direct):
        assert rel_fro(to_host_f64(d_), to_host_f64(g_)) <= TOL[dtype] / 10


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_muon_step_quintic_with_decay(dtype):
    shapes = [(600, 1100), (1100, 600), (50, 70)]
    cfg = _adhoc(shapes, dtype, 210 + (dtype == "bf16"))
    res = run_muon(cfg, weight_decay=0.05, ns_coeffs=QUINTIC_FAST)
    check_against_oracle(cfg, res, weight_decay=0.05, ns_coeffs=QUINTIC_FAST)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_three_term_random_shapes(dtype):
    """The three-term map (the square launch B = c2 A A + c1 A, split into K
    slices for small matrices) with the classical quintic over 24 seeded
    shapes, every matrix against the oracle."""
    shapes = _random_shapes(4000 + (dtype == "bf16"))
    cfg = _adhoc(shapes, dtype, 230 + (dtype == "bf16"))
    res = run_muon(cfg, ns_coeffs=QUINTIC_CLASSICAL)
    worst = check_against_oracle(cfg, res, ns_coeffs=QUINTIC_CLASSICAL)
    print(f"three-term random shapes {dtype}: worst NS rel err {worst:.3e}", flush=True)


def test_ns_batched_in_place():
    x = torch.randn(384, 896, device="cuda")
    ref = nsa.ns_batched([x.clone()], ns_steps=5)[0]
    nsa.ns_batched([x], [x], ns_steps=5)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


def test_ns_rejects_bad_input():
    with pytest.raises(ValueError):
        nsa.ns_batched([torch.randn(16, device="cuda")])
    with pytest.raises(TypeError):
        nsa.ns_batched([torch.randn(16, 16, device="cuda", dtype=torch.float16)])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segments_of_whole_tile_rounds_and_a_tail(dtype):
    """Shape groups large enough that the contraction launches hand their
    tiles to the XCDs in whole rounds of 256 plus a ragged tail: five
    2560 x 2560 matrices (500 update tiles, 275 lower-triangle Gram tiles) and
    2560 x 5376 in both orientations (630 update tiles, 165 Gram tiles of
    K = 5376).  Every matrix against the oracle."""
    shapes = [(2560, 2560)] * 5 + [(5376, 2560), (2560, 5376), (5376, 2560)]
    cfg = _adhoc(shapes, dtype, 220 + (dtype == "bf16"))
    print(f"[parity] whole rounds + tail: {dtype} {shapes}", flush=True)
    res = run_muon(cfg)
    check_against_oracle(cfg, res)


# ------------------------------------------------------------------ scale, transpose, many shape groups
def _half_ulp_f32(x: float) -> float:
    return float(np.spacing(np.float32(x))) / 2.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_power_of_two_scaling(dtype):
    """Blog post, "常见错误" 1: Newton-Schulz needs the normalisation, or large
    norms blow up.  Gradients scaled by 2^k, k in {-40, -20, 0, 20, 40}, one
    Llama-3-8B k_proj shape (1024 x 4096) and one TinyMLP gate shape
    (2048 x 512, tall): every update meets the oracle.  Scaling by a power of
    two is exact in every fp32/bf16 operation of the path (no value leaves the
    normal range), so for every k at which the +1e-7 of the norm is below
    half an ulp of the norm (it then cannot change the rounded sum) the update
    and parameters must be bitwise the same.  That holds at k = 20 and 40 for
    both shapes, and at k = 0 where the norm is large enough."""
    shapes = [(1024, 4096), (2048, 512)]
    cfg = _adhoc(shapes, dtype, 230 + (dtype == "bf16"), grad_scale=1e-3 if dtype == "bf16" else 1.0)
    g = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(2)]
    p0 = [gen.draw_matrix(cfg, i, gen.WEIGHT) for i in range(2)]
    exact = {0: [], 1: []}   # per matrix: (k, update, params) where the epsilon is negligible
    for k in (0, -40, -20, 20, 40):
        dg = [to_device(x) * (2.0 ** k) for x in g]
        dp = [to_device(x) for x in p0]
        db = [torch.zeros(s, device="cuda") for s in shapes]
        du = [torch.empty(s, device="cuda") for s in shapes]
        norms = torch.empty(2, device="cuda")
        nsa.muon_step(dp, dg, db, update_out=du, norms_out=norms)
        torch.cuda.synchronize()
        nrm = norms.cpu().tolist()
        for i in range(2):
            gh = to_host_f64(dg[i])
            assert np.array_equal(gh, g[i].as_f64() * 2.0 ** k)      # the scaling itself was exact
            _, _, uw, nw = oracle.muon_step([p0[i].as_f64()], [gh], [np.zeros(shapes[i])], f32_mu(0.95), True, 5,
                                            0.02)
            u = to_host_f64(du[i])
            err = rel_fro(u, uw[0])
            print(f"[scale] {dtype} 2^{k} {shapes[i]}: norm {nrm[i]:.4e}, rel err {err:.3e}", flush=True)
            assert err <= TOL[dtype], (k, shapes[i], err)
            assert abs(nrm[i] - nw[0]) <= 1e-5 * nw[0]
            if 1e-7 < _half_ulp_f32(nrm[i]):
                exact[i].append((k, du[i], dp[i]))
    for i in range(2):
        ks = [k for k, _, _ in exact[i]]
        assert 20 in ks and 40 in ks, (shapes[i], ks)
        k0, u0, p0_ = exact[i][0]
        for k, u, pp in exact[i][1:]:
            assert torch.equal(u, u0), (shapes[i], k0, k)
            assert torch.equal(pp, p0_), (shapes[i], k0, k)


def test_norm_beyond_folded_range_gives_nan():
    """The 1/||Y|| scale is folded into the first Gram product, which needs
    ||Y||^2 and 1/||Y||^2 to be normal floats: ||Y|| < 2^63.  A matrix beyond
    that gets a NaN update (as a non-finite gradient does) instead of a
    silently wrong one, and the rest of its batch is bitwise unchanged."""
    shapes = [(512, 768), (768, 512)]
    cfg = _adhoc(shapes, "f32", 232)
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(2)]
    p = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(2)]
    g[0] = g[0] * 2.0 ** 60                      # ||Y|| ~ 1.95 * 627 * 2^60 > 2^63
    pa = [t.clone() for t in p]
    u = [torch.zeros(s, device="cuda") for s in shapes]
    norms = torch.empty(2, device="cuda")
    nsa.muon_step(pa, g, [torch.zeros(s, device="cuda") for s in shapes], update_out=u, norms_out=norms)
    pb = p[1].clone()
    ub = torch.zeros(shapes[1], device="cuda")
    nsa.muon_step([pb], [g[1]], [torch.zeros(shapes[1], device="cuda")], update_out=[ub])
    torch.cuda.synchronize()
    assert not norms[0].item() < 2.0 ** 63
    assert torch.isnan(u[0]).all()
    assert torch.equal(u[1], ub) and torch.equal(pa[1], pb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transpose_gives_bitwise_transposed_result(dtype):
    """Blog post, "代码实现": a matrix with more rows than columns is iterated
    as its transpose and transposed back, so NS(G^T) = NS(G)^T.  Both run on
    the same wide iterate here, and the norm is summed in one order over the
    wide orientation whatever the caller's layout, so the results are bitwise
    transposes of each other: through ns_batched, and through the Muon step
    (update, parameters, momentum, norm)."""
    shapes = [(300, 700), (520, 1030), (1024, 4096), (256, 2304)]
    cfg = _adhoc(shapes, dtype, 234 + (dtype == "bf16"))
    g = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(len(shapes))]
    gt = [x.t().contiguous() for x in g]
    outs = nsa.ns_batched(g, ns_steps=5)
    outs_t = nsa.ns_batched(gt, ns_steps=5)
    torch.cuda.synchronize()
    for x, o, ot, s in zip(g, outs, outs_t, shapes):
        assert torch.equal(ot, o.t()), s
        assert rel_fro(to_host_f64(o), oracle.newton_schulz(to_host_f64(x), 5)) <= TOL[dtype], s
    p = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(len(shapes))]
    res = []
    for gg, pp in ((g, p), (gt, [x.t().contiguous() for x in p])):
        pp = [x.clone() for x in pp]
        b = [torch.zeros(x.shape, device="cuda") for x in gg]
        u = [torch.empty(x.shape, device="cuda") for x in gg]
        norms = torch.empty(len(gg), device="cuda")
        nsa.muon_step(pp, gg, b, update_out=u, norms_out=norms)
        torch.cuda.synchronize()
        res.append((pp, b, u, norms))
    (p0, b0, u0, n0), (p1, b1, u1, n1) = res
    assert torch.equal(n0, n1)
    for i, s in enumerate(shapes):
        assert torch.equal(u1[i], u0[i].t()), s
        assert torch.equal(p1[i], p0[i].t()), s
        assert torch.equal(b1[i], b0[i].t()), s


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_more_than_sixteen_shape_groups(dtype):
    """One call with 21 distinct padded shapes (m', n') = (256 a, 256 b), both
    orientations, ragged: every contraction launch table holds at most 16
    shape groups, so each product runs as two launches with their own tile
    numbering and XCD mapping.  bf16: the 18 groups with m' <= 512 (every b
    has a slice count in 2..4) have their Gram cut into K slices, so split
    segments land in both Gram launches and the slice sums need two launches
    as well.  fp32: those 18 groups run on 128 x 128 tiles in tables of their
    own (16 + 2), the other 3 in one table, and the 14 small groups with
    n' >= 1024 are split (one slice-sum table).  Every matrix against the
    oracle."""
    shapes = []
    bs_split = (2, 3, 4, 6, 8, 9, 10, 12, 14)
    for a, bs in ((1, bs_split), (2, bs_split), (3, range(4, 7))):
        for b in bs:
            r, c = 256 * a - 5 * a, 256 * b - 11
            shapes.append((r, c) if (a + b) % 2 else (c, r))
    assert len({(-(-min(s) // 256), -(-max(s) // 256)) for s in shapes}) == 21
    cfg = _adhoc(shapes, dtype, 236 + (dtype == "bf16"))
    print(f"[parity] 21 shape groups, {dtype}", flush=True)
    nsa.profile_read()
    nsa.profile_enable(True)
    res = run_muon(cfg, ns_steps=5)
    nsa.profile_enable(False)
    prof = nsa.profile_read()
    gemm_tables = 2 if dtype == "bf16" else 3
    assert prof["ns_gemm"]["launches"] == gemm_tables * 5
    assert prof["syrk"]["launches"] == 4 * 5          # product and slice-sum tables, as above
    check_against_oracle(cfg, res, ns_steps=5)


def test_side_stream_allocations_outlive_the_call():
    """ns_batched and the one-shot muon_step allocate their workspace (and
    ns_batched its outputs) from the current stream's pool but run on the
    given stream.  A same-size block allocated and filled on the current
    stream right after each call must not be one of those blocks while the
    side stream still uses them: the results must still meet the oracle."""
    shapes = [(2048, 6144), (6144, 2048), (2048, 6144)]
    cfg = _adhoc(shapes, "bf16", 240, grad_scale=1e-3)
    xs = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    dx = [to_device(x) for x in xs]
    need = nsa.ns_workspace_bytes(shapes, torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = nsa.ns_batched(dx, ns_steps=5, stream=side)
    junk = torch.empty(need, dtype=torch.uint8, device="cuda")
    junk.fill_(0xFF)
    junk_outs = [torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda") for s in shapes]
    side.synchronize()
    torch.cuda.synchronize()
    for x, o, s in zip(xs, outs, shapes):
        assert rel_fro(to_host_f64(o), oracle.newton_schulz(x.as_f64(), 5)) <= TOL["bf16"], s
    del junk, junk_outs
    # the one-shot Muon step: its workspace is dropped on return
    p0 = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(len(shapes))]
    p = [t.clone() for t in p0]
    b = [torch.zeros(s, device="cuda") for s in shapes]
    u = [torch.empty(s, device="cuda") for s in shapes]
    need = nsa.muon_step_workspace_bytes(shapes, torch.bfloat16)
    torch.cuda.synchronize()
    nsa.muon_step(p, dx, b, update_out=u, stream=side)
    junk = torch.empty(need, dtype=torch.uint8, device="cuda")
    junk.fill_(0xFF)
    side.synchronize()
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        _, _, uw, _ = oracle.muon_step([to_host_f64(p0[i])], [xs[i].as_f64()], [np.zeros(s)], f32_mu(0.95), True, 5,
                                       0.02)
        assert rel_fro(to_host_f64(u[i]), uw[0]) <= TOL["bf16"], s


# ------------------------------------------------------------------ logging, checkpoint / resume
def test_dmuon_log_prints_each_new_plan_once(monkeypatch, capfd):
    """DMUON_LOG=1: a call prints its plan (dmuon_plan_summary's text) to
    stderr when the plan differs from the last one printed, so a training loop
    logs it once (the training guide's INFO summary, "日志与调试")."""
    shapes = [(333, 777), (777, 333)]
    x = [torch.randn(s, device="cuda") for s in shapes]
    monkeypatch.setenv("DMUON_LOG", "1")
    capfd.readouterr()
    nsa.ns_batched(x, ns_steps=3)
    nsa.ns_batched(x, ns_steps=3)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert err.count("dmuon plan:") == 1, err
    assert nsa.plan_summary(shapes, torch.float32, 3, muon=False) in err
    nsa.ns_batched(x[:1], ns_steps=3)
    torch.cuda.synchronize()
    assert capfd.readouterr().err.count("dmuon plan:") == 1
    monkeypatch.setenv("DMUON_LOG", "0")
    nsa.ns_batched(x, ns_steps=3)
    torch.cuda.synchronize()
    assert "dmuon plan:" not in capfd.readouterr().err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_checkpoint_resume_is_bitwise(dtype, tmp_path):
    """Training guide, "相关文档" (检查点: saving and loading training
    state).  The Muon state is the parameters and the momentum buffers; the
    library keeps nothing between calls.  One step, a checkpoint through
    torch.save, a load (weights_only) into fresh device tensors and a second
    step with a fresh workspace must give bitwise the parameters and momentum
    of two uninterrupted steps."""
    shapes = [(600, 1100), (1100, 600), (40, 60)]
    cfg = _adhoc(shapes, dtype, 250 + (dtype == "bf16"))
    g1 = [to_device(gen.draw_matrix(cfg, i, gen.GRAD)) for i in range(3)]
    g2 = [to_device(gen.draw_matrix(cfg, i, gen.GRAD2)) for i in range(3)]
    p0 = [to_device(gen.draw_matrix(cfg, i, gen.WEIGHT)) for i in range(3)]
    # uninterrupted
    pa = [t.clone() for t in p0]
    ba = [torch.zeros(s, device="cuda") for s in shapes]
    first = nsa.MuonStep(pa, g1, ba)
    first()
    nsa.MuonStep(pa, g2, ba, workspace=first.workspace)()
    # interrupted after the first step
    pb = [t.clone() for t in p0]
    bb = [torch.zeros(s, device="cuda") for s in shapes]
    nsa.MuonStep(pb, g1, bb)()
    torch.cuda.synchronize()
    path = tmp_path / "muon_state.pt"
    torch.save({"params": [t.cpu() for t in pb], "momentum": [t.cpu() for t in bb]}, path)
    del pb, bb
    state = torch.load(path, weights_only=True)
    pc = [t.cuda() for t in state["params"]]
    bc = [t.cuda() for t in state["momentum"]]
    nsa.MuonStep(pc, g2, bc)()
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        assert torch.equal(pc[i], pa[i]), s
        assert torch.equal(bc[i], ba[i]), s


# ------------------------------------------------------------------ clipping folded into the step
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm_type", [2.0, float("inf")])
def test_clipped_step_against_oracle(dtype, norm_type):
    """Training guide, "梯度裁剪": per-segment global p-norm clipping before
    momentum and Newton-Schulz, folded into the step (dmuon_muon_step_clipped).
    Against the oracle's clip_grad_norm_buckets followed by its muon_step:
    segment totals; momentum within one fp32 ulp of mu b + fl32(g coef) with
    the GPU's own coefficient; U within the tolerance (elementwise route: one
    ulp of the Nesterov input); parameters faithful.  Two segments clip, the
    third does not and must equal the plain step bitwise; the caller's
    gradients are not modified."""
    shapes = [(600, 1100), (1100, 600), (40, 60), (512, 768), (300, 400), (700, 300)]
    segments = [0, 0, 1, 1, 2, 2]
    cfg = _adhoc(shapes, dtype, 260 + (dtype == "bf16") + 2 * (norm_type == 2.0))
    g = [gen.draw_matrix(cfg, i, gen.GRAD) for i in range(len(shapes))]
    p0 = [gen.draw_matrix(cfg, i, gen.WEIGHT) for i in range(len(shapes))]
    b0 = [gen.draw_matrix(cfg, i, gen.MOMENTUM) for i in range(len(shapes))]
    g64 = [x.as_f64() for x in g]
    _, want_tot = oracle.clip_grad_norm_buckets(g64, segments, [1.0, 1.0, 1.0], norm_type)
    max_norm = [0.5 * want_tot[0], 0.1 * want_tot[1], 10.0 * want_tot[2]]
    clipped64, tot64 = oracle.clip_grad_norm_buckets(g64, segments, max_norm, norm_type)
    dg = [to_device(x) for x in g]
    dg_before = [t.clone() for t in dg]
    dp = [to_device(x) for x in p0]
    db = [to_device(x) for x in b0]
    du = [torch.full(x.values.shape, float("nan"), device="cuda") for x in g]
    totals = torch.full((3,), float("nan"), device="cuda")
    mu, lr = 0.9, 0.02
    nsa.MuonStep(dp, dg, db, mu=mu, lr=lr, update_out=du, clip_max_norm=max_norm, clip_segments=segments,
                 clip_norm_type=norm_type, clip_totals=totals)()
    # the plain step on the same inputs, for the unclipped segment
    pp = [to_device(x) for x in p0]
    bp = [to_device(x) for x in b0]
    up = [torch.full(x.values.shape, float("nan"), device="cuda") for x in g]
    nsa.MuonStep(pp, dg, bp, mu=mu, lr=lr, update_out=up)()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(dg, dg_before))
    tot = totals.cpu().numpy().astype(np.float64)
    for s in range(3):
        assert abs(tot[s] - tot64[s]) <= 2e-6 * tot64[s], (s, tot[s], tot64[s])
    mu32 = f32_mu(mu)
    for i, sh in enumerate(shapes):
        s = segments[i]
        coef = np.float32(max_norm[s]) / (np.float32(tot[s]) + np.float32(1e-6))
        coef = np.float32(1.0) if coef >= 1.0 else np.float32(coef)
        g32 = (g[i].values.astype(np.float32) if dtype == "f32" else g64[i].astype(np.float32)) * coef
        b_exact = mu32 * b0[i].as_f64() + g32.astype(np.float64)
        bg = to_host_f64(db[i])
        assert max_ulp_err_f32(bg, b_exact) <= 1.0, (sh, "momentum")
        u = to_host_f64(du[i])
        pw, _, uw, _ = oracle.muon_step([p0[i].as_f64()], [clipped64[i]], [b0[i].as_f64()], mu32, True, 5, lr)
        if sh[0] * sh[1] < oracle.MIN_NS_NUMEL:
            y = g32.astype(np.float64) + mu32 * bg
            assert max_ulp_err_f32(u, y) <= 1.0, (sh, "elementwise update")
        else:
            err = rel_fro(u, uw[0])
            assert err <= TOL[dtype], (sh, err)
        check_update_faithful(to_host_f64(dp[i]), p0[i].as_f64(), u, lr, 1.0, dtype)
        if s == 2:
            assert coef == 1.0
            assert torch.equal(du[i], up[i]) and torch.equal(dp[i], pp[i]) and torch.equal(db[i], bp[i]), sh
        else:
            assert coef < 1.0
