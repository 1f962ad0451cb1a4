"""Host-side logic of bench.py (no GPU): argument handling and the reading of
the committed hardware-counter summary."""
import os

import bench


def test_more_than_one_gpu_exits_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_recorded_traffic_sums_kernels_and_drops_stale_stages(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "w_hbm_traffic.txt").write_text(
        "# comment\n"
        "fetch_scale 2.0\n"
        "stage route kernel row_or_kernel src_sha good fetch_kib 1 write_kib 1 bytes 100\n"
        "stage route kernel materialize_kernel src_sha good fetch_kib 1 write_kib 1 bytes 250\n"
        "stage spmm_sparse kernel spmm_list_bf16_kernel src_sha stale fetch_kib 1 write_kib 1 bytes 7\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda stage: "good")
    t = bench.recorded_traffic("w")
    assert t["route"] == 350.0
    assert t["spmm_sparse"] is None  # sources changed since the counters were taken
    assert t["up_gemm_pack"] is None and t["fallback_gemm"] is None  # not recorded


def test_recorded_traffic_without_a_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert all(v is None for v in bench.recorded_traffic("nothing").values())


def test_stage_sources_exist():
    for stage, files in bench.STAGE_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(bench.ROOT, f)), (stage, f)
        assert len(bench.source_sha(stage)) == 16


def test_conversion_bytes_counts_h_twell_and_dense_rows_once():
    # 2 rows of d_ff 512 in bf16, T 256 (2 tiles), C 8, one dense row:
    # h 2*512*2 = 2048; TwELL 2 rows * 2 tiles * (8*2 + 8 + 1) = 100; dense row 512*2 = 1024
    assert bench.conversion_bytes(2, 512, 256, 8, 2, 1) == 2048 + 100 + 1024
    # no dense rows, fp32, T = C = 64: h 64*4, TwELL 1 tile * (64*4 + 64 + 1)
    assert bench.conversion_bytes(1, 64, 64, 64, 4, 0) == 256 + 321


def test_cpu_baseline_reports_affinity_cores_and_blas():
    from activation_sparse_transformer_amd.synth import CONFIGS, make_inputs

    cfg = CONFIGS["tiny_fp32"]
    r = bench.cpu_oracle_baseline(make_inputs(cfg), cfg, target_s=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["blas"]["build"]  # the BLAS NumPy was built against is named


def test_median_and_percentiles():
    assert bench.median([3.0, 1.0, 2.0, 100.0, 4.0]) == 3.0
    assert bench.percentile([1, 2, 3, 4, 5], 50) == 3.0
