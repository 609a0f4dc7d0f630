#!/usr/bin/env python3
"""Benchmark: one batched Muon step over a Llama-3-8B-shaped matrix set on one
MI355X.

A step is one dmuon_muon_step call over all 224 projection matrices
(32 layers x q, k, v, o, gate, up, down): momentum + Nesterov + Frobenius norm,
5 Newton-Schulz iterations (Gram product + update product per iteration) and
the weight update.  Inputs are seeded synthetic tensors already resident in
HBM: bf16 gradients ~ N(0, 1e-3^2), bf16 weights ~ N(0, 1), fp32 momentum
starting at zero.

Prints one JSON line.  `value` is the whole step's algorithmic Newton-Schulz
throughput (TFLOP/s): per matrix and iteration m'(m'+1)n' for the
lower-triangle Gram product plus 2m'^2 n' + 3m'n' for the update product and
its epilogue (m' = min(rows, cols), n' = max(rows, cols)), divided by the
measured step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


NS_COEFFS = {
    "cubic": None,                              # the blog's map (1.5, -0.5)
    "quintic": (3.4445, -4.7750, 2.0315),       # a widely used fast quintic
    "classical": (1.875, -1.25, 0.375),         # (15 s - 10 s^3 + 3 s^5) / 8
}


def ns_flops(shapes, ns_steps, three_terms=False):
    """Algorithmic Newton-Schulz flops per step: the lower-triangle Gram product,
    for three-term maps the lower-triangle square c2 A A + c1 A, and the
    update product with its epilogue."""
    syrk = gemm = 0.0
    for r, c in shapes:
        if r * c < 100_000:
            continue
        m, n = float(min(r, c)), float(max(r, c))
        syrk += m * (m + 1.0) * n
        if three_terms:
            syrk += m * (m + 1.0) * m + 2.0 * m * m
        gemm += 2.0 * m * m * n + 3.0 * m * n
    return syrk * ns_steps, gemm * ns_steps


def cpu_baseline(cfg, sample_idx, ns_steps, mu, lr):
    """The fp64 oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    mats = []
    for i in sample_idx:
        g = gen.draw_matrix(cfg, i, gen.GRAD).as_f64()
        p = gen.draw_matrix(cfg, i, gen.WEIGHT).as_f64()
        mats.append((p, g, np.zeros_like(g)))
    t0 = time.perf_counter()
    for p, g, b in mats:
        oracle.muon_step([p], [g], [b], mu, True, ns_steps, lr)
    dt = time.perf_counter() - t0
    shapes = [(cfg.matrices[i].rows, cfg.matrices[i].cols) for i in sample_idx]
    s, g = ns_flops(shapes, ns_steps)
    desc = ", ".join(f"{cfg.matrices[i].name} {cfg.matrices[i].rows}x{cfg.matrices[i].cols}" for i in sample_idx)
    return {"value": (s + g) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one Muon step (k={ns_steps}) of {len(sample_idx)} matrices: {desc}; {dt:.2f} s wall, "
                      f"float64 NumPy oracle",
            "flop_count": "algorithmic: m'(m'+1)n' + 2m'^2 n' + 3m'n' per matrix and step, the count the GPU "
                          "figure uses (the oracle itself forms the full X X^T, the dense-equivalent count)",
            "value_dense_equivalent": dense_equivalent_flops(shapes, ns_steps) / dt / 1e12,
            "wall_s": dt, "per_config": cpu_baseline_small_sets(),
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_small_sets():
    """Wall time of the fp64 oracle over the two small sets in full: the
    TinyMLP set (one Muon step, k = 5) and the spectrum set (Newton-Schulz of
    all 32 matrices for k in {3, 5, 7, 10}, from its fp32 and its bf16 copy).
    Input generation is not timed."""
    import numpy as np
    import oracle
    from workloads import gen, get_config
    out = {}
    tiny = get_config("tinymlp_f32")
    mats = [(gen.draw_matrix(tiny, i, gen.WEIGHT).as_f64(), gen.draw_matrix(tiny, i, gen.GRAD).as_f64())
            for i in range(tiny.count)]
    mu = float(np.float32(tiny.momentum))
    t0 = time.perf_counter()
    for p, g in mats:
        oracle.muon_step([p], [g], [np.zeros_like(g)], mu, tiny.nesterov, 5, tiny.lr)
    dt = time.perf_counter() - t0
    shapes = [(m.rows, m.cols) for m in tiny.matrices]
    s, gf = ns_flops(shapes, 5)
    out["tinymlp_f32"] = {"what": f"one Muon step, k=5, all {tiny.count} matrices", "wall_s": dt,
                          "tflops": (s + gf) / dt / 1e12,
                          "tflops_dense_equivalent": dense_equivalent_flops(shapes, 5) / dt / 1e12}
    spec = get_config("spectrum")
    ins = []
    for i, m in enumerate(spec.matrices):
        f32, b16 = gen.spectrum_copies(gen.spectrum_matrix(spec.cfg_id, i, m.rows, m.cols)[0])
        ins += [f32.as_f64(), b16.as_f64()]
    t0 = time.perf_counter()
    for k in spec.ns_steps:
        for x in ins:
            oracle.newton_schulz(x, k)
    dt = time.perf_counter() - t0
    shapes = [(m.rows, m.cols) for m in spec.matrices] * 2
    flops = sum(sum(ns_flops(shapes, k)) for k in spec.ns_steps)
    dense = sum(dense_equivalent_flops(shapes, k) for k in spec.ns_steps)
    out["spectrum"] = {"what": f"Newton-Schulz of all {spec.count} matrices for k in {list(spec.ns_steps)}, "
                               "fp32 and bf16 copies", "wall_s": dt, "tflops": flops / dt / 1e12,
                       "tflops_dense_equivalent": dense / dt / 1e12}
    return out


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def dense_equivalent_flops(shapes, ns_steps):
    """What the same steps cost as two plain GEMMs each (4 m'^2 n' per matrix
    and step: the full X X^T and A X), the count the method avoids with the
    triangle; reported beside the algorithmic figure, never as % of peak."""
    total = 0.0
    for r, c in shapes:
        if r * c < 100_000:
            continue
        m, n = float(min(r, c)), float(max(r, c))
        total += 4.0 * m * m * n
    return total * ns_steps


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None when the
    MFMA kernel source has changed since the counters were taken (or no summary exists)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "llama3_8b_hbm_counters.md")
    src = os.path.join(ROOT, "newton_schulz_08_amd", "csrc", "kernels_mfma.hip")
    try:
        text = open(path).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    for m in re.finditer(r"traffic (\S+) bytes_per_launch=(\d+) source_sha256=([0-9a-f]{64})", text):
        if m.group(1) == kernel and m.group(3) == digest:
            return int(m.group(2))
    return None


def _smi_json(args, timeout=30):
    """amd-smi ... --json as a dict, or None (a child process; never raises)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", *args, "--json"], capture_output=True, text=True, timeout=timeout)
        d = json.loads(r.stdout)
        if isinstance(d, dict):
            d = d.get("gpu_data", [d])
        return d[0] if isinstance(d, list) and d else None
    except Exception:
        return None


def _mhz(v):
    """'2400 MHz' / '2400MHz' / {'value': 2400, ...} -> 2400.0, else None."""
    try:
        if isinstance(v, dict):
            return float(v["value"])
        return float(str(v).replace("MHz", "").strip())
    except (KeyError, TypeError, ValueError):
        return None


def gpu_static_info():
    """Product name, CU count and the highest graphics clock level, read with
    amd-smi before this process touches the GPU."""
    d = _smi_json(["static", "--asic", "--clock"])
    if not d:
        return {}
    asic, clk = d.get("asic", {}), d.get("clock", {})
    levels = (clk.get("sys") or {}).get("frequency_levels") or {}
    top = [m for m in (_mhz(v) for v in levels.values()) if m]
    return {"market_name": asic.get("market_name"), "num_compute_units": asic.get("num_compute_units"),
            "max_gfx_clock_mhz": max(top) if top else None}


def clock_sampler(path, parent):
    """Child-process loop: sample the graphics clocks (every XCD) and the power
    with amd-smi into `path`, one JSON line each, until the parent exits (or
    20 minutes pass)."""
    t_end = time.time() + 1200
    with open(path, "w") as f:
        while os.getppid() == parent and time.time() < t_end:
            t0 = time.time()
            d = _smi_json(["metric", "--clock", "--power"], timeout=20)
            rec = {"t0": t0, "t1": time.time()}
            if d:
                clk = d.get("clock") or {}
                rec["gfx_mhz"] = [m for k, v in sorted(clk.items()) if k.startswith("gfx_") and isinstance(v, dict)
                                  for m in [_mhz(v.get("clk"))] if m]
                rec["mem_mhz"] = [m for k, v in sorted(clk.items()) if k.startswith("mem") and isinstance(v, dict)
                                  for m in [_mhz(v.get("clk"))] if m]
                power = d.get("power") or {}
                rec["power_w"] = {k: float(v["value"]) for k, v in power.items()
                                  if isinstance(v, dict) and isinstance(v.get("value"), (int, float))}
            f.write(json.dumps(rec) + "\n")
            f.flush()
            time.sleep(0.2)


def start_clock_sampler():
    """Start clock_sampler in a child process (before the GPU is touched).
    Not under a profiler, which would follow the child."""
    import subprocess
    import tempfile
    if any(k.startswith("ROCPROF") for k in os.environ):
        return None
    fd, path = tempfile.mkstemp(prefix="bench_clock_", suffix=".jsonl")
    os.close(fd)
    proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--clock-sampler", path, str(os.getpid())],
                            stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return proc, path


def stop_clock_sampler(sampler, t0, t1):
    """Stop the sampler; summarise the samples taken wholly inside [t0, t1]."""
    if sampler is None:
        return None
    proc, path = sampler
    proc.terminate()
    try:
        proc.wait(timeout=10)
    except Exception:  # pragma: no cover
        proc.kill()
        proc.wait()
    recs = []
    try:
        with open(path) as f:
            recs = [json.loads(line) for line in f if line.strip()]
    except (OSError, ValueError):
        pass
    os.unlink(path)
    inside = [r for r in recs if r["t0"] >= t0 and r["t1"] <= t1 and r.get("gfx_mhz")]
    if not inside:
        return {"samples": 0}
    mean = [sum(r["gfx_mhz"]) / len(r["gfx_mhz"]) for r in inside]
    out = {"samples": len(inside), "gfx_clock_mhz_mean": sum(mean) / len(mean), "gfx_clock_mhz_min": min(mean),
           "gfx_clock_mhz_max": max(mean)}
    mem = [sum(r["mem_mhz"]) / len(r["mem_mhz"]) for r in inside if r.get("mem_mhz")]
    if mem:
        out.update({"mem_clock_mhz_mean": sum(mem) / len(mem), "mem_clock_mhz_min": min(mem),
                    "mem_clock_mhz_max": max(mem)})
    pw = [r.get("power_w", {}) for r in inside]
    for k in sorted(set().union(*pw)):
        vals = [p[k] for p in pw if k in p]
        out[f"{k}_w_mean"] = sum(vals) / len(vals)
    return out


def metadata(torch):
    meta = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "peaks": {"bf16_mfma_tflops": PEAK_TFLOPS["bf16"], "f32_mfma_tflops": PEAK_TFLOPS["f32"],
                      "hbm_gbs": PEAK_HBM_GBS}}
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    try:
        prop = torch.cuda.get_device_properties(0)
        meta["gpu"] = prop.name or None
        meta["gcn_arch"] = getattr(prop, "gcnArchName", None)
        meta["cus"] = prop.multi_processor_count
    except Exception:  # pragma: no cover
        pass
    return meta


def clip_bench(torch, nsa, grads, reps=5):
    """Per-segment gradient clipping over the whole gradient set (one segment
    per projection kind): an unclipped pass (read only) and a clipping pass
    (read, then read and write), timed by the library's kernel events."""
    kinds = sorted({g.shape for g in grads})
    segs = [kinds.index(g.shape) for g in grads]
    numel = sum(g.numel() for g in grads)
    eb = grads[0].element_size()
    ws = nsa.alloc_workspace(nsa.clip_grad_norm_workspace_bytes([g.numel() for g in grads], len(kinds)))
    out = {"tensors": len(grads), "segments": len(kinds), "elements": numel}
    for tag, max_norm, bytes_per in (("no_clip", 1e30, eb), ("clip", 0.0, 3 * eb)):
        nsa.clip_grad_norm_(grads, [max_norm] * len(kinds), segs, workspace=ws)
        torch.cuda.synchronize()
        nsa.profile_read()
        nsa.profile_enable(True)
        for _ in range(reps):
            nsa.clip_grad_norm_(grads, [max_norm] * len(kinds), segs, workspace=ws)
        torch.cuda.synchronize()
        nsa.profile_enable(False)
        st = nsa.profile_read().get("grad_clip")
        ms = st["total_ms"] / st["launches"]
        gbs = numel * bytes_per / (ms * 1e-3) / 1e9
        out[tag] = {"ms": ms, "algorithmic_bytes": numel * bytes_per, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    return out


def fused_clip_bench(torch, nsa, params, grads, moms, cfg, ns_steps, plain_step_ms, reps=3):
    """The Muon step with per-segment clipping folded in (one segment per
    projection kind, each clipped to half its norm): the clip's partials pass
    (timed by the library's kernel events) is its only extra work, one read of
    the gradients; the step itself reads the gradients as before, scaled on
    load."""
    kinds = sorted({g.shape for g in grads})
    segs = [kinds.index(g.shape) for g in grads]
    totals = torch.zeros(len(kinds), device="cuda")
    ws = nsa.alloc_workspace(nsa.clip_grad_norm_workspace_bytes([g.numel() for g in grads], len(kinds)))
    totals = nsa.clip_grad_norm_(grads, [3.0e38] * len(kinds), segs, workspace=ws)   # totals only: nothing clips
    max_norm = [0.5 * float(t) for t in totals.cpu()]
    del ws
    step = nsa.MuonStep(params, grads, moms, ns_steps=ns_steps, mu=cfg.momentum, nesterov=cfg.nesterov, lr=cfg.lr,
                        clip_max_norm=max_norm, clip_segments=segs)
    step()
    torch.cuda.synchronize()
    nsa.profile_read()
    nsa.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    nsa.profile_enable(False)
    st = nsa.profile_read().get("grad_clip")
    numel = sum(g.numel() for g in grads)
    clip_ms = st["total_ms"] / st["launches"]
    out = {"step_ms": ms, "plain_step_ms": plain_step_ms, "clip_ms": clip_ms,
           "clip_algorithmic_bytes": numel * grads[0].element_size(),
           "clip_gbs": numel * grads[0].element_size() / (clip_ms * 1e-3) / 1e9,
           "segments": len(kinds), "max_norm": "half of each segment's norm"}
    del step
    torch.cuda.empty_cache()
    return out


# Llama-3-8B's non-matrix parameters, which go to AdamW: token embedding and
# output head (128256 x 4096 each) and 65 RMSNorm weights of 4096.
ADAMW_SET = [128256 * 4096, 128256 * 4096] + [4096] * 65


def adamw_bench(torch, nsa, dtype, reps=10):
    """The fused AdamW step over the non-matrix parameter set, seeded synthetic
    values, timed by the library's kernel events.  Algorithmic bytes per
    element: parameters and gradients in `dtype`, fp32 moments; read p, g, m, v
    and write p, m, v."""
    gen = torch.Generator(device="cuda").manual_seed(7)
    eb = torch.empty((), dtype=dtype).element_size()
    P = [torch.randn(n, device="cuda", generator=gen).mul_(0.02).to(dtype) for n in ADAMW_SET]
    G = [torch.randn(n, device="cuda", generator=gen).mul_(1e-3).to(dtype) for n in ADAMW_SET]
    M = [torch.zeros(n, device="cuda") for n in ADAMW_SET]
    V = [torch.zeros(n, device="cuda") for n in ADAMW_SET]
    ws = nsa.alloc_workspace(nsa.adamw_step_workspace_bytes(ADAMW_SET))
    numel = sum(ADAMW_SET)
    bytes_per = 3 * eb + 16
    nsa.adamw_step_(P, G, M, V, 1, workspace=ws)
    torch.cuda.synchronize()
    nsa.profile_read()
    nsa.profile_enable(True)
    for t in range(reps):
        nsa.adamw_step_(P, G, M, V, 2 + t, workspace=ws)
    torch.cuda.synchronize()
    nsa.profile_enable(False)
    st = nsa.profile_read().get("adamw")
    ms = st["total_ms"] / st["launches"]
    gbs = numel * bytes_per / (ms * 1e-3) / 1e9
    out = {"tensors": len(ADAMW_SET), "elements": numel, "param_dtype": str(dtype).replace("torch.", ""),
           "hyper": "lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight_decay 0.01", "ms": ms,
           "algorithmic_bytes": numel * bytes_per, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    del P, G, M, V, ws
    torch.cuda.empty_cache()
    return out


def reference_gemm(torch, n=8192, reps=30):
    """Context only: torch.matmul (hipBLASLt) on an n^3 bf16 GEMM of random data on the same GPU, sustained
    over ~1 s, to show the practical power-limited MFMA rate next to the published peak."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    a = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    c = torch.matmul(a, b)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return {"what": f"torch.matmul bf16 {n}x{n}x{n}, random data (vendor library, context only)",
            "tflops": 2.0 * n ** 3 / dt / 1e12}


def main():
    if len(sys.argv) == 4 and sys.argv[1] == "--clock-sampler":
        clock_sampler(sys.argv[2], int(sys.argv[3]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--ns-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true", default=True)
    ap.add_argument("--no-reference-gemm", action="store_true",
                    help="skip timing the vendor library's bf16 GEMM on the same GPU (context only)")
    ap.add_argument("--ns-coeffs", choices=sorted(NS_COEFFS), default="cubic",
                    help="Newton-Schulz polynomial (default: the cubic 1.5, -0.5)")
    ap.add_argument("--weight-decay", type=float, default=0.0)
    ap.add_argument("--moonlight", action="store_true", help="scale lr by 0.2*sqrt(max(m, n)) per matrix")
    ap.add_argument("--no-clip-bench", action="store_true", help="skip timing per-segment gradient clipping")
    ap.add_argument("--no-adamw-bench", action="store_true",
                    help="skip timing the AdamW step over the non-matrix parameter set")
    ap.add_argument("--full-gram", action="store_true",
                    help="ablation: compute every Gram tile instead of the lower triangle plus its mirror")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="do not sample the GPU clock and power with amd-smi during the timed steps")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of GIB GiB (calibrates the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the batched step runs the whole "
              "matrix set on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    if args.full_gram:
        os.environ["DMUON_NS_KERNEL"] = "gemm"
    # amd-smi runs in child processes started before this process touches the GPU
    static_info = gpu_static_info() if args.copy_calibration <= 0 else {}
    sampler = start_clock_sampler() if args.copy_calibration <= 0 and not args.no_clock_sample else None
    import torch
    import newton_schulz_08_amd as nsa
    from workloads import get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 2**30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)                      # runtime copy kernel
        torch.mul(src, 1.0, out=dst)        # elementwise copy kernel
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return
    cfg = get_config(args.config)
    ns_steps = args.ns_steps if args.ns_steps is not None else cfg.ns_steps[0]
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[cfg.dtype]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_setup = time.perf_counter()
    from workloads.device import make_set
    data = make_set(cfg, device=dev)
    params, grads, moms = data["params"], data["grads"], data["momentum"]
    coeffs = NS_COEFFS[args.ns_coeffs]
    step = nsa.MuonStep(params, grads, moms, ns_steps=ns_steps, mu=cfg.momentum, nesterov=cfg.nesterov, lr=cfg.lr,
                        weight_decay=args.weight_decay, lr_scale_mode="moonlight" if args.moonlight else "one",
                        ns_coeffs=coeffs)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"[bench] {cfg.key}: {cfg.count} matrices, workspace {step.workspace_bytes / 2**30:.1f} GiB, "
          f"setup {setup_s:.1f} s", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    nsa.profile_read()
    if args.profile:
        nsa.profile_enable(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.time()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    w1 = time.time()
    clocks = stop_clock_sampler(sampler, w0, w1)
    nsa.profile_enable(False)
    kstats = nsa.profile_read() if args.profile else {}
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    import numpy as np
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    shapes = [(m.rows, m.cols) for m in cfg.matrices]
    syrk_f, gemm_f = ns_flops(shapes, ns_steps, coeffs is not None and len(coeffs) == 3)
    ns_total = syrk_f + gemm_f
    value = ns_total / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]

    kernels = {}
    for name, s in kstats.items():
        avg_ms = s["total_ms"] / max(s["launches"], 1)
        ent = {"launches": s["launches"], "avg_ms": avg_ms, "ms_per_step": s["total_ms"] / args.steps}
        if s["flops"] > 0:
            ent["tflops"] = s["flops"] / (s["total_ms"] * 1e-3) / 1e12
        if s["bytes"] > 0:
            ent["gbs"] = s["bytes"] / (s["total_ms"] * 1e-3) / 1e9
        kernels[name] = ent
    roofline = None
    # the dominant kernel: the contraction family with the most time in the timed steps
    fams = [k for k in ("ns_iter", "ns_gemm", "syrk") if k in kstats and kstats[k]["flops"] > 0]
    if fams:
        fam = max(fams, key=lambda k: kstats[k]["total_ms"])
        kname = f"{fam}_kernel<{'bf16' if cfg.dtype == 'bf16' else 'f32'}>"
        s = kstats[fam]
        achieved = s["flops"] / (s["total_ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": recorded_traffic(kname),
                    "per_launch_flops": s["flops"] / max(s["launches"], 1),
                    "avg_launch_ms": s["total_ms"] / max(s["launches"], 1)}
        top = static_info.get("max_gfx_clock_mhz")
        if clocks and clocks.get("samples") and top:
            # the published peak assumes the top clock; under this load the
            # chip holds its power limit at a lower one
            mhz = clocks["gfx_clock_mhz_mean"]
            roofline["at_timed_clock"] = {"gfx_clock_mhz": mhz, "peak": peak * mhz / top,
                                          "frac": achieved / (peak * mhz / top)}
    ns_kernel_ms = sum(kstats[k]["total_ms"] for k in ("syrk", "syrk_square", "ns_iter", "ns_gemm")
                       if k in kstats) / args.steps

    out = {
        "metric": "Muon step ms + NS TFLOP/s (% of MFMA peak), Llama-8B-shaped matrix set",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_events": {"median": float(np.median(step_ms)), "min": float(step_ms.min()),
                           "p90": float(np.percentile(step_ms, 90))},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.key}: {cfg.count} matrices "
                               f"({', '.join(sorted(set(f'{m.rows}x{m.cols}' for m in cfg.matrices)))}), "
                               f"{cfg.dtype} grads/params, fp32 momentum, ns_steps={ns_steps}, "
                               f"mu={cfg.momentum}, nesterov={cfg.nesterov}, lr={cfg.lr}",
                   "matrices": cfg.count, "ns_steps": ns_steps, "parallelism": "single-gpu",
                   "gram": "full (ablation)" if args.full_gram else "lower triangle + mirror",
                   "ns_coeffs": args.ns_coeffs if coeffs is None else f"{args.ns_coeffs} {coeffs}",
                   "weight_decay": args.weight_decay, "lr_scale": "moonlight" if args.moonlight else "one"},
        "ns_tflops_kernels": (ns_total / (ns_kernel_ms * 1e-3) / 1e12) if ns_kernel_ms > 0 else None,
        "ns_tflops_dense_equivalent": dense_equivalent_flops(shapes, ns_steps) / (ms_per_step * 1e-3) / 1e12,
        "pct_mfma_peak": 100.0 * value / peak,
        "roofline": roofline,
        "kernels": kernels,
        "backend": nsa.backend_info(),
        "meta": {**metadata(torch), **static_info, "timed_region_clocks": clocks},
    }
    if not args.no_clip_bench:
        del step
        torch.cuda.empty_cache()
        # before the in-place clipping pass below, which rescales the gradients
        fused = fused_clip_bench(torch, nsa, params, grads, moms, cfg, ns_steps, ms_per_step)
        out["grad_clip"] = clip_bench(torch, nsa, grads)
        out["grad_clip"]["fused_in_step"] = fused
    if not args.no_adamw_bench:
        out["adamw"] = adamw_bench(torch, nsa, torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    if not args.no_reference_gemm and cfg.dtype == "bf16":
        out["reference_gemm"] = reference_gemm(torch)
    if not args.no_cpu_baseline:
        import numpy as np
        # layer 0's q_proj (4096x4096), k_proj (1024x4096) and gate_proj (14336x4096): one of each shape
        sample = [0, 1, 4] if cfg.key == "llama3_8b" else [0]
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, sample, ns_steps, float(np.float32(cfg.momentum)), cfg.lr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
