"""bench.py: the contract line (GPU) and the host logic behind its `traffic`
field (CPU): counter files from two rocprofv3 --pmc runs are scaled by the
known-size device copy and tagged with the attention kernel's source hash."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, kib in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_record_traffic_scales_by_the_copy_and_tags_the_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib_kib = (1 << 30) / 1024
    # the counters see half of the copy's reads and all of its writes
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [("__amd_rocclr_copyBuffer", gib_kib / 2),
                     ("void at::native::vectorized_elementwise_kernel<4, copy>", 123.0),
                     ("void sage::attn_fwd_kernel<128, false, false, false>(sage::AttnArgs)", 1000.0),
                     ("void sage::attn_fwd_kernel<128, false, false, false>(sage::AttnArgs)", 3000.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [("__amd_rocclr_copyBuffer", gib_kib),
                     ("void sage::attn_fwd_kernel<128, false, false, false>(sage::AttnArgs)", 500.0)])
    bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w"))
    e = json.load(open(tmp_path / "traffic.json"))["video_14b_720p/fp8"]
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)   # mean of the two dispatches
    assert e["write_bytes"] == pytest.approx(500.0 * 1024)
    assert e["bytes_per_launch"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
    assert e["source_hash"] == bench.attn_source_hash()


def test_record_traffic_of_the_quantization_pass_per_step(tmp_path, monkeypatch):
    """The quantization kernels of the same counter runs: their bytes summed
    per step (one quant_qk_kernel launch per step), scaled by the copy."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib_kib = (1 << 30) / 1024
    attn = "void sage::attn_fwd_kernel<128, false, false, 0, false>(sage::AttnArgs)"
    quant = [("void sage::kv_stats_kernel<128>(...)", 100.0), ("sage::k_mean_kernel", 1.0),
             ("void sage::quant_qk_kernel<128, false>(...)", 200.0),
             ("void sage::quant_v_fp8_kernel<128>(...)", 50.0)]
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [("__amd_rocclr_copyBuffer", gib_kib / 2), (attn, 10.0)] + quant + quant)
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [("__amd_rocclr_copyBuffer", gib_kib), (attn, 5.0)] + quant)
    bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w"))
    e = json.load(open(tmp_path / "traffic.json"))["video_14b_720p/fp8/quant"]
    assert e["fetch_bytes"] == pytest.approx(351.0 * 1024 * 2.0)  # two steps, mean
    assert e["write_bytes"] == pytest.approx(351.0 * 1024)
    assert e["bytes_per_step"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
    assert e["source_hash"] == bench.attn_source_hash(quant=True)


def test_record_traffic_refuses_runs_without_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _write_counters(tmp_path / "f", "FETCH_SIZE", [("void sage::attn_fwd_kernel<128>", 1.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [("void sage::attn_fwd_kernel<128>", 1.0)])
    with pytest.raises(SystemExit):
        bench.record_traffic("tiny", "fp8", str(tmp_path / "f"), str(tmp_path / "w"))


def test_record_traffic_of_the_mx_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib_kib = (1 << 30) / 1024
    rows = [("__amd_rocclr_copyBuffer", gib_kib),
            ("void sage::attn_fwd_kernel<128, false, false, 0, false>(sage::AttnArgs)", 9.0),
            ("void sage::attn_mx_kernel<128, false>(sage::AttnArgs)", 700.0)]
    _write_counters(tmp_path / "f", "FETCH_SIZE", rows)
    _write_counters(tmp_path / "w", "WRITE_SIZE", rows)
    bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w"), mx=True)
    data = json.load(open(tmp_path / "traffic.json"))
    assert list(data) == ["video_14b_720p/mxfp6"]
    e = data["video_14b_720p/mxfp6"]
    assert e["kernel"] == "attn_mx_kernel" and e["fetch_bytes"] == pytest.approx(700.0 * 1024)
    # the MXFP4 run of the same kernel goes under its own key
    bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w"),
                         mx="mxfp4")
    data = json.load(open(tmp_path / "traffic.json"))
    assert sorted(data) == ["video_14b_720p/mxfp4", "video_14b_720p/mxfp6"]


def test_record_traffic_of_the_backward_sums_its_kernels_per_call(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gib_kib = (1 << 30) / 1024
    call = [("_ZN4sage15bwd_prep_kernelILi128EEEvPKt", 10.0),
            ("void sage::bwd_t8_kernel<128>(signed char const*, int, signed char*)", 2.0),
            ("void sage::bwd_t8_kernel<128>(signed char const*, int, signed char*)", 3.0),
            ("void sage::bwd_dq_kernel<128, false>(sage::BwdArgs)", 100.0),
            ("void sage::bwd_dkdv_kernel<128, false, 1>(sage::BwdArgs)", 80.0),
            ("void sage::bwd_dkdv_kernel<128, false, 2>(sage::BwdArgs)", 120.0)]
    # the training forward and the copy are not part of a backward call; two calls
    rows = [("__amd_rocclr_copyBuffer", gib_kib),
            ("void sage::attn_fwd_kernel<128, false, false, 0, false>(sage::AttnArgs)", 50.0)]
    _write_counters(tmp_path / "f", "FETCH_SIZE", rows + call + call)
    _write_counters(tmp_path / "w", "WRITE_SIZE", rows + call + call)
    bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w"), bwd=True)
    e = json.load(open(tmp_path / "traffic.json"))["video_14b_720p/bwd"]
    assert e["fetch_bytes"] == pytest.approx(315.0 * 1024)
    assert e["write_bytes"] == pytest.approx(315.0 * 1024)
    assert e["source_hash"] == bench.attn_source_hash(bwd=True) != bench.attn_source_hash()
    # counters without a dQ sweep say nothing per call
    _write_counters(tmp_path / "w2", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib)] + call[:3])
    with pytest.raises(SystemExit):
        bench.record_traffic("video_14b_720p", "fp8", str(tmp_path / "f"), str(tmp_path / "w2"),
                             bwd=True)


@pytest.mark.parametrize("causal_name", ["tiny", "causal_prefill"])
def test_cpu_baseline_all_core_run(causal_name):
    """The all-core run: the same oracle on disjoint rows in threads; one
    thread reports the single-thread rate itself."""
    import synthetic_inputs as si

    wl = si.make(causal_name, B=1, H=1, N=600)
    one = bench.cpu_baseline(wl, "fp8", target_s=0.2, cores=1)
    assert one["cores"] == 1 and one["value"] == one["single_core_value"] > 0
    two = bench.cpu_baseline(wl, "fp8", target_s=0.2, cores=2, all_core_s=0.2)
    assert two["cores"] == 2 and two["value"] > 0 and two["single_core_value"] > 0
    assert "2 threads" in two["sample"]


def test_cpu_baseline_of_the_mx_path():
    import synthetic_inputs as si

    wl = si.make("tiny", N=300, H=1)
    r = bench.cpu_baseline(wl, "fp8", target_s=0.2, mx=True)
    assert r["value"] > 0 and r["kind"] == "oracle" and r["cores"] == bench.host_cores()
    assert "MXFP6" in r["sample"]
    r4 = bench.cpu_baseline(wl, "fp8", target_s=0.2, mx="mxfp4", cores=1)
    assert r4["value"] > 0 and "MXFP4" in r4["sample"]


def test_mx_refuses_the_other_variants():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mx", "--q-smooth"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "MX path" in r.stderr
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mx", "mxfp5"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "invalid choice" in r.stderr


def test_bwd_refuses_the_other_variants_and_samples_the_oracle():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--bwd", "--mx"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "backward" in r.stderr
    import synthetic_inputs as si

    wl = si.make("tiny", N=300, H=1)
    res = bench.cpu_baseline_bwd(wl)
    assert res["value"] > 0 and res["kind"] == "oracle" and "dQ" in res["sample"]
    assert res["cores"] == min(bench.host_cores(), 3)     # at most one thread per query block
    one = bench.cpu_baseline_bwd(wl, cores=1)
    assert one["cores"] == 1 and one["value"] == one["single_core_value"] > 0
    # the blended backward peak: 2d ops each at 5.0 POPS for four products, dP at 2.5
    assert bench.PEAK_TOPS["bwd"] == pytest.approx(10.0 / (8.0 / 5000.0 + 2.0 / 2500.0))


def test_algorithmic_ops_count():
    # 4 d ops per (query, key) pair: 2d for Q K^T, 2d for P V
    assert bench.attn_ops(1, 40, 75600, 128) == pytest.approx(1.1705e14, rel=1e-4)
    assert bench.attn_ops(2, 3, 5, 64) == 4 * 2 * 3 * 25 * 64


def test_visited_ops_closed_forms():
    import numpy as np

    import synthetic_inputs as si

    wl = si.make("tiny", N=300)
    full = np.ones((1, 2, 3, 3), np.uint8)
    assert bench.visited_ops(wl, full) == bench.attn_ops(1, 2, 300, 128)   # ragged tiles
    half = full.copy()
    half[:, :, :, 1] = 0                                                   # drop key tile 1
    assert bench.visited_ops(wl, half) == 4 * 128 * 2 * 300 * (300 - 128)
    wc = si.make("causal_prefill", B=1, H=1, N=300)
    m = bench.tile_mask_for(wc, 1.0)
    assert m.shape == (1, 1, 3, 3) and not np.triu(m[0, 0], 1).any()      # nothing above the diagonal
    assert bench.visited_ops(wc, m) == 4 * 128 * 300 * 301 / 2            # N (N + 1) / 2 pairs
    wl = si.make("tiny")
    m = bench.tile_mask_for(wl, 0.0)                                       # band + first tile only
    i, j = np.meshgrid(np.arange(8), np.arange(8), indexing="ij")
    assert np.array_equal(m[0, 0].astype(bool), (abs(i - j) <= 1) | (j == 0))


def test_source_hash_covers_the_kernel_sources():
    h = bench.attn_source_hash()
    assert len(h) == 16 and all(os.path.exists(f) for f in bench.ATTN_SOURCES)
    assert h == bench.attn_source_hash()
    assert all(os.path.exists(f) for f in bench.BWD_SOURCES)
    assert any(f.endswith("sage_bwd.hip") for f in bench.BWD_SOURCES)


def test_measured_peak_is_absent_without_the_microbenchmarks(monkeypatch):
    from quantized_attention_video_02_amd.microbench import __main__ as mb

    monkeypatch.setattr(mb, "LIB", os.path.join(ROOT, "no_such_libmb.so"))
    assert bench.measured_mfma_tops() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_line_keeps_the_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["value"] > 0
    rf = line["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 5000.0 and rf["unit"] == "TFLOP/s"
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["target_frac"] == 0.5 and rf["target_met"] == (rf["frac"] >= 0.5)
    from quantized_attention_video_02_amd.microbench import __main__ as mb

    if os.path.exists(mb.LIB):
        mp = rf["measured_peak"]
        assert 0 < mp["int8"] <= 5000 * 1.05 and 0 < mp["fp8"] <= 5000 * 1.05
        assert min(mp["int8"], mp["fp8"]) <= mp["blend"] <= max(mp["int8"], mp["fp8"])
        assert mp["frac"] == pytest.approx(rf["achieved"] / mp["blend"])
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and 1 <= cb["cores"] <= 16 and cb["single_core_value"] > 0
    assert line["config"]["workload"] == "tiny"


@pytest.mark.gpu
def test_mx_bench_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--mx",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    rf = line["roofline"]
    assert line["dtype"] == "mxfp6" and rf["kernel"] == "attn_mx_kernel"
    assert rf["peak"] == 10100.0 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert "MXFP6" in line["cpu_baseline"]["sample"]
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--mx",
                        "mxfp4", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["dtype"] == "mxfp4" and line["config"]["pv"] == "mxfp4"
    assert line["roofline"]["kernel"] == "attn_mx_kernel" and line["roofline"]["peak"] == 10100.0


@pytest.mark.gpu
def test_bwd_bench_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--bwd",
                        "--steps", "3", "--warmup", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    rf = line["roofline"]
    assert line["config"]["pass"] == "backward" and line["value"] > 0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert line["cpu_baseline"]["kind"] == "oracle"


@pytest.mark.gpu
def test_bench_shape_override_and_no_causal():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "causal_prefill",
                        "--shape", "1,2,1000", "--no-causal", "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cfg = line["config"]
    assert (cfg["B"], cfg["H"], cfg["N"], cfg["causal"]) == (1, 2, 1000, False)
    assert line["roofline"]["traffic"] is None
    assert "ops_counted" not in line["roofline"]
