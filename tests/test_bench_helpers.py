"""Host logic of bench.py: the algorithmic flop count, the counter-traffic
lookup and the amd-smi clock sampling, without a GPU."""
import json
import os
import time

import pytest

import bench


def test_ns_flops_counts_the_method_work():
    # a 300x1000 matrix (m' = 300, n' = 1000): lower-triangle Gram m'(m'+1)n',
    # update 2 m'^2 n' + 3 m'n'; a small matrix (numel < 100000) adds nothing
    syrk, gemm = bench.ns_flops([(300, 1000), (100, 999)], ns_steps=1)
    assert syrk == 300 * 301 * 1000
    assert gemm == 2 * 300 * 300 * 1000 + 3 * 300 * 1000
    # orientation does not matter, steps scale linearly
    assert bench.ns_flops([(1000, 300)], ns_steps=5) == (5 * syrk, 5 * gemm)
    # a three-term map adds the lower-triangle square m'(m'+1)m' + 2m'^2
    s3, g3 = bench.ns_flops([(300, 1000)], ns_steps=1, three_terms=True)
    assert s3 == syrk + 300 * 301 * 300 + 2 * 300 * 300 and g3 == gemm


def test_dense_equivalent_counts_two_full_products():
    assert bench.dense_equivalent_flops([(300, 1000), (100, 999)], ns_steps=2) == 2 * 4 * 300 * 300 * 1000
    # about 4/3 of the method's own count for a wide matrix
    syrk, gemm = bench.ns_flops([(4096, 14336)], 1)
    assert 1.3 < bench.dense_equivalent_flops([(4096, 14336)], 1) / (syrk + gemm) < 1.34


def test_cpu_model_is_a_string_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_recorded_traffic_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "newton_schulz_08_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "kernels_mfma.hip").write_bytes(b"kernel source\n")
    import hashlib
    digest = hashlib.sha256(b"kernel source\n").hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "llama3_8b_hbm_counters.md").write_text(
        f"    traffic k<bf16> bytes_per_launch=123 source_sha256={digest}\n"
        f"    traffic other bytes_per_launch=7 source_sha256={'0' * 64}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("k<bf16>") == 123
    assert bench.recorded_traffic("other") is None          # stale hash
    (src / "kernels_mfma.hip").write_bytes(b"kernel source, changed\n")
    assert bench.recorded_traffic("k<bf16>") is None


def test_committed_traffic_matches_the_current_source():
    # the committed counter summary must describe the kernel source in the tree
    assert bench.recorded_traffic("ns_gemm_kernel<bf16>") is not None


def test_mhz_parsing():
    assert bench._mhz("2400 MHz") == 2400.0
    assert bench._mhz("110MHz") == 110.0
    assert bench._mhz({"value": 1653, "unit": "MHz"}) == 1653.0
    assert bench._mhz("N/A") is None and bench._mhz(None) is None


def test_gpu_static_info(monkeypatch):
    fake = {"asic": {"market_name": "GPU X", "num_compute_units": 256},
            "clock": {"sys": {"frequency_levels": {"Level 0": "110 MHz", "Level 1": "500 MHz",
                                                   "Level 2": "2400 MHz"}}}}
    monkeypatch.setattr(bench, "_smi_json", lambda args, timeout=30: fake)
    assert bench.gpu_static_info() == {"market_name": "GPU X", "num_compute_units": 256, "max_gfx_clock_mhz": 2400.0}
    monkeypatch.setattr(bench, "_smi_json", lambda args, timeout=30: None)
    assert bench.gpu_static_info() == {}


class _DoneProc:
    def terminate(self):
        pass

    def wait(self, timeout=None):
        return 0


def test_clock_summary_keeps_samples_inside_the_timed_region(tmp_path):
    path = tmp_path / "samples.jsonl"
    recs = [
        {"t0": 0.5, "t1": 1.5, "gfx_mhz": [2400.0] * 8, "power_w": {"socket_power": 300.0}},   # straddles start
        {"t0": 2.0, "t1": 2.5, "gfx_mhz": [1600.0, 1700.0], "power_w": {"socket_power": 1300.0}},
        {"t0": 3.0, "t1": 3.5, "gfx_mhz": [1650.0, 1650.0], "power_w": {"socket_power": 1400.0}},
        {"t0": 4.0, "t1": 4.2},                                                                # amd-smi failed
        {"t0": 4.8, "t1": 5.5, "gfx_mhz": [2400.0], "power_w": {"socket_power": 200.0}},      # straddles end
    ]
    path.write_text("".join(json.dumps(r) + "\n" for r in recs))
    out = bench.stop_clock_sampler((_DoneProc(), str(path)), 1.0, 5.0)
    assert out["samples"] == 2
    assert out["gfx_clock_mhz_mean"] == pytest.approx(1650.0)
    assert out["gfx_clock_mhz_min"] == pytest.approx(1650.0) and out["gfx_clock_mhz_max"] == pytest.approx(1650.0)
    assert out["socket_power_w_mean"] == pytest.approx(1350.0)
    assert not path.exists()
    assert bench.stop_clock_sampler(None, 0.0, 1.0) is None


def test_sampler_child_exits_after_stop():
    # without a GPU amd-smi yields nothing, but the child must start, stop and clean up
    smp = bench.start_clock_sampler()
    if smp is None:
        pytest.skip("running under a profiler")
    proc, path = smp
    t0 = time.time()
    time.sleep(0.5)
    out = bench.stop_clock_sampler(smp, t0, time.time())
    assert proc.poll() is not None
    assert not os.path.exists(path)
    assert out["samples"] >= 0
