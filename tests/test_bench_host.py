"""CPU checks of the benchmark's host-side arithmetic (no GPU): the algorithmic
byte count behind `value` and `roofline.achieved`, the two summaries that turn
rocprofv3 FETCH_SIZE / WRITE_SIZE runs into HBM bytes, the source-hash gate on
the committed traffic record, and the refusal of more than one GPU.

The counter files here are small synthetic CSVs with the columns rocprofv3
writes, so every expected number follows from the inputs by hand.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KIB = 1024
COPY_KIB = 256 * 1024  # one 256 MiB calibration copy, in KiB


def test_gemv_bytes_matches_the_format():
    # GSQ card, "Storage layout": [28672, 8192] -> 768 int32 words and 64 bf16 scales per row
    n, k = 28672, 8192
    words = n * 768 * 4
    scales = n * 64 * 2
    assert bench.gemv_bytes(n, k) == words + scales + 2 * k + 4 * n == 91_881_472
    # M activation rows and M output rows on top of the same weights
    assert bench.gemv_bytes(n, k, 16) - bench.gemv_bytes(n, k, 1) == 15 * (2 * k + 4 * n)


def _counter_csv(path, counter, rows):
    """rows: (kernel name, KiB per dispatch), one dispatch each."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_traffic_summary_scales_by_the_calibration_copies(tmp_path):
    kern = "void (anonymous namespace)::qgemv_mfma_kernel<16, 4, false>(unsigned short const*, GemvSegs)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half the bytes (factor 2), WRITE_SIZE the bytes (factor 1); a small copy
    # that is not one of the five 256 MiB calibration copies must be ignored
    fetch = [(copy, 16.0)] + [(copy, COPY_KIB / 2)] * 5 + [(kern, 40_000.0), (kern, 50_000.0)]
    write = [(copy, 16.0)] + [(copy, COPY_KIB)] * 5 + [(kern, 100.0), (kern, 124.0)]
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    rec = bench.traffic_from_counters(str(f), str(w), str(out))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == 2 * 45_000 * KIB
    assert rec["hbm_write_bytes_per_launch"] == 112 * KIB
    assert rec["dispatches_averaged"] == 2
    assert rec["algorithmic_bytes_per_launch"] == bench.gemv_bytes(28672, 8192)
    assert rec["traffic_over_algorithmic"] == pytest.approx((90_000 + 112) * KIB / bench.gemv_bytes(28672, 8192),
                                                           abs=1e-4)
    assert json.loads(out.read_text()) == rec


def test_case_traffic_sums_the_library_kernels_of_one_call(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    prep = "(anonymous namespace)::prep_x_slice_kernel(unsigned short const*, HIP_vector_type<unsigned int, 4u>*)"
    ring = "void (anonymous namespace)::qgemm_mr_kernel<8, 2, false>(HIP_vector_type<unsigned int, 4u> const*)"
    csum = "(anonymous namespace)::qgemm_chunk_sum_kernel(float const*, float*, long, int, long)"
    pack = "(anonymous namespace)::qpack_kernel(unsigned char const*, unsigned int*, long)"
    torch_fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >"
    fetch = ([(copy, COPY_KIB / 2)] * 5 + [(pack, 9e9), (torch_fill, 9e9)] +
             [(prep, 300.0), (prep, 300.0), (ring, 48_000.0), (ring, 48_000.0), (csum, 3_600.0), (csum, 3_600.0)])
    write = ([(copy, COPY_KIB)] * 5 + [(pack, 9e9), (torch_fill, 9e9)] +
             [(prep, 260.0), (prep, 260.0), (ring, 7_168.0), (ring, 7_168.0), (csum, 3_584.0), (csum, 3_584.0)])
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    rec = bench.case_traffic_from_counters("gate_proj:32", str(f), str(w))
    per = rec["per_kernel"]
    assert set(per) == {"prep_x_slice_kernel", "qgemm_mr_kernel<8, 2, false>", "qgemm_chunk_sum_kernel"}
    assert per["qgemm_mr_kernel<8, 2, false>"] == {"fetch_bytes": 96_000 * KIB, "write_bytes": 7_168 * KIB,
                                                   "dispatches": 2}
    total = (600 + 96_000 + 7_200 + 260 + 7_168 + 3_584) * KIB
    assert rec["hbm_bytes_per_call"] == total
    assert rec["algorithmic_bytes_per_call"] == bench.gemv_bytes(28672, 8192, 32)


def test_committed_traffic_is_used_only_for_its_own_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic() == 123
    rec["kernel_source_sha256_16"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_covers_every_library_source_and_the_build_flags(tmp_path, monkeypatch):
    src, build = tmp_path / "csrc", tmp_path / "_build.py"
    src.mkdir()
    for name in ("qw3.hip", "qw3_gemv.hip", "qw3_common.h"):
        (src / name).write_text("// %s\n" % name)
    (src / "notes.txt").write_text("not a source")
    build.write_text("UNITS = []\n")
    monkeypatch.setattr(bench, "KERNEL_SRC_DIR", str(src))
    monkeypatch.setattr(bench, "KERNEL_BUILD", str(build))
    h0 = bench.kernel_source_hash()
    (src / "notes.txt").write_text("still not a source")
    assert bench.kernel_source_hash() == h0
    for path in (src / "qw3_gemv.hip", src / "qw3_common.h", build):
        old = path.read_text()
        path.write_text(old + "// edited\n")
        assert bench.kernel_source_hash() != h0, path.name
        path.write_text(old)
        assert bench.kernel_source_hash() == h0
    (src / "qw3_extra.hip").write_text("// a new unit\n")
    assert bench.kernel_source_hash() != h0


def test_compact_summary_of_the_other_workloads():
    layer = {"gate_proj": {"us": 18.4, "GB/s": 4992.3, "bytes": 91881472, "us_stream_launches": 18.5},
             "k_proj": {"us": 4.56, "GB/s": 722.5, "bytes": 3297280, "us_stream_launches": 11.8}}
    lines = [{"workload": "Llama-3.1-70B decoder layer at B=1: q/o [8192, 8192], k/v [1024, 8192], gate/up "
                          "[28672, 8192], down [8192, 28672] (device time, graph replay)",
              "layer_bytes": 334725120, "layer_us": 84.528, "per_projection": {}},
             {"workload": "gate_proj [28672, 8192] M=16", "us": 27.708, "HBM_frac": 0.4234, "MFMA_frac": 0.1085},
             {"workload": "down_proj [8192, 28672] M=512", "us": 260.04, "HBM_frac": 0.0663, "MFMA_frac": 0.37}]
    layer_bytes, layer_ms, fused_ms = 334725120, 0.084528, 0.077332
    out = bench.compact_summary(layer, layer_ms, fused_ms, layer_bytes, lines)
    assert out["gate_proj_M1"] == {"us": 18.4, "frac": round(4992.3 / 8000, 4)}
    assert out["k_proj_M1"]["frac"] == round(722.5 / 8000, 4)
    assert out["layer_70b_M1"] == {"us": 84.528, "frac": round(layer_bytes / layer_ms / 1e6 / 8000, 4)}
    assert out["layer_70b_M1_fused"]["us"] == 77.332
    assert out["gate_proj_M16"] == {"us": 27.708, "frac": 0.4234}     # decode: the HBM fraction
    assert out["down_proj_M512"] == {"us": 260.04, "frac": 0.37}      # prefill: the MFMA fraction
    assert len(out) == 1 + 2 + 2 + 2  # unit, two projections, two layer figures, two calls
    # the full summary (7 projections, 2 layers, 10 batched/prefill calls) keeps the line short
    full = dict(out, **{"%s_M%d" % (nm, m): {"us": 123.456, "frac": 0.1234}
                        for nm in ("gate_proj", "down_proj") for m in (4, 8, 16, 32, 512)})
    full.update({"%s_M1" % nm: {"us": 12.345, "frac": 0.1234} for nm in bench.LAYER_ORDER})
    assert len(json.dumps(full)) < 1500
