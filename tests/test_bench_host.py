"""Host-side logic of bench.py (no GPU): the one-GPU guard, the per-step FLOP
count, and the rocprofv3 counter summary that feeds the roofline's traffic,
clock and MFMA-busy figures."""
import csv
import os

import pytest

import bench
import seeded_inputs as si


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name", ["prefill_bf16_s128k_p16", "gqa16_bf16_s8k_p8", "prefill_bf16_s1m_p8"])
@pytest.mark.parametrize("order", ["pass_kv", "pass_q"])
def test_ring_step_flops_cover_the_causal_triangle(name, order):
    w = si.WORKLOADS[name]
    steps = bench.ring_step_flops(w, order)
    assert len(steps) == w.n_chunks
    # S(S+1)/2 visible pairs at 4 * D * Hq FLOP each, split over the steps
    assert sum(steps) == pytest.approx(4.0 * w.D * w.Hq * w.B * w.Sq * (w.Sq + 1) / 2, rel=1e-12)
    assert sum(steps) == pytest.approx(w.flops(), rel=1e-12)
    # step 0 holds the P diagonal pairs (half a full pair each, plus the diagonal itself)
    C = w.chunk
    assert steps[0] == pytest.approx(w.n_chunks * 4.0 * w.D * w.Hq * w.B * C * (C + 1) / 2, rel=1e-12)


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=fields)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(fields, r)))


def test_counter_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    k, copy = "partial_bf16_fast_kernel<128, false>(args)", "vectorized_elementwise_kernel<MulFunctor>"
    gib_kib = (1 << 30) / 1024.0
    # the copy kernel's FETCH_SIZE reads half its true bytes (scale 2), WRITE_SIZE all of them
    _write_counters(tmp_path / "f", [(k, "FETCH_SIZE", 1000.0, 0, 1), (k, "FETCH_SIZE", 3000.0, 0, 1),
                                     (copy, "FETCH_SIZE", gib_kib / 2, 0, 1)])
    _write_counters(tmp_path / "w", [(k, "WRITE_SIZE", 500.0, 0, 1), (k, "WRITE_SIZE", 500.0, 0, 1),
                                     (copy, "WRITE_SIZE", gib_kib, 0, 1)])
    # 8 XCDs x 1.6 GHz over a 1 ms dispatch; the copy at 2.4 GHz
    _write_counters(tmp_path / "c", [(k, "GRBM_GUI_ACTIVE", 8 * 1.6e6, 0, 1_000_000),
                                     (copy, "GRBM_GUI_ACTIVE", 8 * 2.4e6, 0, 1_000_000)])
    assert bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "c")) == 0
    kv = dict(ln.split(":", 1) for ln in out.read_text().splitlines() if ":" in ln and not ln.startswith("#"))
    assert float(kv["copy_fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["copy_write_scale"]) == pytest.approx(1.0)
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(2000.0 * 1024 * 2.0)
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(500.0 * 1024)
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx(2000.0 * 2048 + 500.0 * 1024)
    assert float(kv["sclk_ghz_partial_kernel"]) == pytest.approx(1.6)
    assert float(kv["sclk_ghz_copy_kernel"]) == pytest.approx(2.4)
    # the bench reads it back only while the kernel source is the one the counters were taken on
    hbm, clk, _, _ = bench.read_pmc_summary()
    assert hbm == pytest.approx(2000.0 * 2048 + 500.0 * 1024) and clk == pytest.approx(1.6)
    out.write_text(out.read_text().replace(bench.kernel_hash(), "0" * 16))
    assert bench.read_pmc_summary() == (None, None, None, None)


def test_trace_summary_and_its_readback(tmp_path, monkeypatch):
    """The kernel-trace summary: average partial-kernel launch -> TFLOP/s and fraction of the dense
    peak, beside the plain bench line of the same machine; read back only for the same kernel sources."""
    import json
    out = tmp_path / "trace.txt"
    monkeypatch.setattr(bench, "TRACE_FILE", str(out))
    d = tmp_path / "tr"
    d.mkdir()
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow(["partial_bf16_fast_kernel<128, false>(args)", 96, 96 * 3.5e6, 3.5e6, 99.0, 1e6, 7e6, 1.0])
        wr.writerow(["decode_stream_kernel<128>(args)", 10, 3.3e6, 3.3e5, 1.0, 3e5, 4e5, 1.0])
    bj = tmp_path / "b.json"
    bj.write_text(json.dumps({"ms_per_step": 57.0, "value": 1234.5,
                              "roofline": {"avg_launch_ms": 3.45, "frac": 0.51, "machine": {"host": "hostA", "gpu_uuid": "u"}}}))
    assert bench.summarize_trace(str(d), str(bj)) == 0
    w = si.WORKLOADS["prefill_bf16_s128k_p16"]
    tv = bench.trace_values()
    assert tv["machine_host"] == "hostA"
    assert tv["partial_kernel_avg_ms"] == pytest.approx(3.5)
    assert tv["frac_profiled"] == pytest.approx(w.flops() / 16 / 3.5e-3 / 1e12 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert tv["trace_kernel_ms_per_step"] == pytest.approx(56.0)
    assert tv["bench_ms_per_step"] == pytest.approx(57.0)
    out.write_text(out.read_text().replace(bench.kernel_hash(), "0" * 16))
    assert bench.trace_values() == {}


def test_decode_summary_and_its_readback(tmp_path, monkeypatch):
    """The decode profile: trace averages of the decode kernel and of its merge (not the ring merge),
    their bytes per dispatch scaled by the copy kernel, read back only for the same kernel sources."""
    import json
    out = tmp_path / "decode.txt"
    monkeypatch.setattr(bench, "DECODE_FILE", str(out))
    d = tmp_path / "tr"
    d.mkdir()
    dk, mk, rk = "decode_stream_kernel(cpattn::DecodeLaunch, int)", "merge_kernel(cpattn::MergeLaunch)", \
        "ring_merge_kernel(cpattn::RingMergeLaunch)"
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow([dk, 44, 44 * 3.0e5, 3.0e5, 90.0, 1e5, 4e5, 1.0])
        wr.writerow([mk, 44, 44 * 1.0e4, 1.0e4, 5.0, 1e4, 2e4, 1.0])
        wr.writerow([rk, 4, 4 * 9.0e5, 9.0e5, 5.0, 1e5, 1e6, 1.0])
    copy = "vectorized_elementwise_kernel<MulFunctor>"
    gib_kib = (1 << 30) / 1024.0
    _write_counters(tmp_path / "f", [(dk, "FETCH_SIZE", 1000.0, 0, 1), (mk, "FETCH_SIZE", 10.0, 0, 1),
                                     (rk, "FETCH_SIZE", 9999.0, 0, 1), (copy, "FETCH_SIZE", gib_kib / 2, 0, 1)])
    _write_counters(tmp_path / "w", [(dk, "WRITE_SIZE", 40.0, 0, 1), (mk, "WRITE_SIZE", 4.0, 0, 1),
                                     (rk, "WRITE_SIZE", 9999.0, 0, 1), (copy, "WRITE_SIZE", gib_kib, 0, 1)])
    bj = tmp_path / "b.json"
    bj.write_text("[bench] log line\n" + json.dumps({"decode": {"ms": 0.31, "GB/s": 6900.0, "frac_hbm": 0.8625},
                                                     "machine": {"host": "hostB", "gpu_uuid": "u2"}}) + "\n")
    assert bench.summarize_decode(str(d), str(tmp_path / "f"), str(tmp_path / "w"), str(bj)) == 0
    nb = bench.decode_bytes(si.WORKLOADS[bench.DECODE])
    assert nb["total"] == nb["kernel"] + nb["merge"]
    assert nb["total"] == 2165972992  # 2 x 128 x 32768 x 128 x 2 B of K/V + Q + partials twice + O/LSE
    pv = bench.decode_profile_values()
    assert pv["machine_host"] == "hostB"
    assert pv["decode_kernel_avg_ms"] == pytest.approx(0.3)
    assert pv["merge_kernel_avg_ms"] == pytest.approx(0.01)
    assert pv["kernel_and_merge_GB/s"] == pytest.approx(nb["total"] / 0.31e-3 / 1e9, abs=0.1)
    assert pv["decode_kernel_fetch_bytes"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert pv["merge_kernel_hbm_bytes"] == pytest.approx(10.0 * 2048 + 4.0 * 1024)
    assert pv["bench_decode_ms"] == pytest.approx(0.31)
    out.write_text(out.read_text().replace(bench.kernel_hash(), "0" * 16))
    assert bench.decode_profile_values() == {}


def test_merge_summary_and_its_readback(tmp_path, monkeypatch):
    """The ring-merge profile: the trace average of ring_merge_kernel against the algorithmic bytes of
    the 128K ring's 136 slots read and 16 owners written, and its counted traffic."""
    import json
    out = tmp_path / "merge.txt"
    monkeypatch.setattr(bench, "MERGE_FILE", str(out))
    d = tmp_path / "tr"
    d.mkdir()
    rk = "void cpattn::ring_merge_kernel<128>(cpattn::RingMergeLaunch)"
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow([rk, 14, 14 * 1.9e6, 1.9e6, 40.0, 1.8e6, 2.0e6, 1.0])
        wr.writerow(["partial_bf16_fast_kernel<128, false>(args)", 16, 16 * 3.5e6, 3.5e6, 60.0, 1e6, 7e6, 1.0])
    copy = "vectorized_elementwise_kernel<MulFunctor>"
    gib_kib = (1 << 30) / 1024.0
    _write_counters(tmp_path / "f", [(rk, "FETCH_SIZE", 5000.0, 0, 1), (copy, "FETCH_SIZE", gib_kib / 2, 0, 1)])
    _write_counters(tmp_path / "w", [(rk, "WRITE_SIZE", 600.0, 0, 1), (copy, "WRITE_SIZE", gib_kib, 0, 1)])
    bj = tmp_path / "m.json"
    bj.write_text(json.dumps({"ring_merge": {"ms": 1.88, "GB/s": 5470.0, "frac_hbm": 0.684},
                              "machine": {"host": "hostC", "gpu_uuid": "u3"}}) + "\n")
    assert bench.summarize_merge(str(d), str(tmp_path / "f"), str(tmp_path / "w"), str(bj)) == 0
    w = si.WORKLOADS[bench.PREFILL]
    nb = bench.ring_merge_bytes(w)
    # 136 slots read + 16 owners written, 8192 rows x 16 heads x 129 floats each
    assert nb == (136 + 16) * 8192 * 16 * 129 * 4
    mv = bench.merge_profile_values()
    assert mv["machine_host"] == "hostC"
    assert mv["ring_merge_kernel_avg_ms"] == pytest.approx(1.9)
    assert mv["ring_merge_GB/s"] == pytest.approx(nb / 1.9e-3 / 1e9, abs=0.1)
    assert mv["ring_merge_kernel_hbm_bytes"] == pytest.approx(5000.0 * 2048 + 600.0 * 1024)
    assert mv["bench_merge_ms"] == pytest.approx(1.88)
    out.write_text(out.read_text().replace(bench.kernel_hash(), "0" * 16))
    assert bench.merge_profile_values() == {}


def test_committed_profiles_match_the_kernel_sources():
    """Every committed profile summary was taken on the kernel sources as they stand: a change to a
    kernel source without new profiles fails here (the bench would otherwise just drop the figures)."""
    names = ["partial_bf16_prefill_s128k_p16_trace.txt", "partial_bf16_prefill_s128k_p16_traffic.txt",
             "decode_stream_b128_kv32k_p8.txt", "ring_merge_s128k_p16.txt"]
    for name in names:
        path = os.path.join(bench.ROOT, "profiles", name)
        tags = [ln.split(":", 1)[1].strip() for ln in open(path) if ln.startswith("kernel_source_sha256_16:")]
        assert tags == [bench.kernel_hash()], f"{name} was taken on other kernel sources: {tags}"


def test_cpu_threads_respect_the_job_share(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_threads() == 1
    monkeypatch.setenv("OMP_NUM_THREADS", str(10 * n))
    assert bench.cpu_threads() == n
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads() == n
