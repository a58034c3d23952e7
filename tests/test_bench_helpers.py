"""bench.py's HBM-traffic record (CPU only): a recorded figure is reported
only while the kernel's sources hash to the recorded value and the record was
taken on the workload being run."""
import json

import bench


def test_recorded_traffic_tied_to_sources_and_workload(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    sha = bench._sources_sha("prefill_gemm")
    rec.write_text(json.dumps({"prefill_gemm": {"bytes_per_launch": 123, "sha256": sha,
                                                "workload": "w"}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic("prefill_gemm", "w") == 123
    assert bench.recorded_traffic("prefill_gemm", "other") is None
    assert bench.recorded_traffic("decode_ffn", "w") is None
    rec.write_text(json.dumps({"prefill_gemm": {"bytes_per_launch": 123, "sha256": "0" * 64,
                                                "workload": "w"}}))
    assert bench.recorded_traffic("prefill_gemm", "w") is None


def test_record_traffic_scales_counters(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE rows (KiB per dispatch) become bytes per
    launch with the calibrated factors, averaged over dispatches and summed
    over the kind's kernels."""
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    hdr = "Kernel_Name,Counter_Name,Counter_Value\n"
    f = tmp_path / "f"
    w = tmp_path / "w"
    f.mkdir()
    w.mkdir()
    (f / "p_counter_collection.csv").write_text(
        hdr + '"void moert::ffn_kernel<1, 1, 4, 2>(moert::FfnArgs)",FETCH_SIZE,100\n'
        '"void moert::ffn_kernel<1, 1, 4, 2>(moert::FfnArgs)",FETCH_SIZE,300\n'
        '"moert::plan_kernel<4>(x)",FETCH_SIZE,999\n')
    (w / "p_counter_collection.csv").write_text(
        hdr + '"void moert::ffn_kernel<1, 1, 4, 2>(moert::FfnArgs)",WRITE_SIZE,10\n')
    r = bench.record_traffic("decode_ffn", "wl", str(f), str(w))
    assert r["bytes_per_launch"] == round(200 * bench.FETCH_SCALE + 10 * bench.WRITE_SCALE)
    assert r["workload"] == "wl" and r["sha256"] == bench._sources_sha("decode_ffn")
