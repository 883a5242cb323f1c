"""Host-side logic of bench.py: the kernel-code hash that keys the traffic record, and the
scaling of the rocprofv3 traffic counters by the calibration copy.  No GPU."""
import csv
import json
import os

import pytest

import bench


def test_source_hash_ignores_comments_and_blank_space():
    code = "int f(int x) {\n    return x + 1;  // add one\n}\n/* block\n comment */\n"
    same = "int f(int x) {   return x + 1; }\n// another comment\n\n"
    other = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench.source_hash(code) == bench.source_hash(same)
    assert bench.source_hash(code) != bench.source_hash(other)
    assert len(bench.source_hash(code)) == 16


def test_source_hash_of_the_kernel_files_is_stable():
    assert [os.path.basename(p) for p in bench.KERNEL_SOURCES] == ["mla_bf16.hip", "mla_internal.h",
                                                                  "mla_sparse.cpp"]
    text = "\n".join(open(p).read() for p in bench.KERNEL_SOURCES)
    assert bench.source_hash() == bench.source_hash(text)
    assert bench.source_hash(text + "\n// trailing note\n") == bench.source_hash(text)


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, value in rows:
            # two counter instances per dispatch, summed by the reader
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value / 2})


def test_write_traffic_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    mib = 256
    # the copy reads 256 MiB; FETCH_SIZE reports half of it (KiB), WRITE_SIZE all of it
    fetch_rows = [(1, "mla::attn_bf16(...)", 80000.0), (2, "mla::uv_bf16(...)", 26000.0),
                  (3, "mla::absorb_q_bf16(...)", 9800.0), (4, "mla::attn_bf16(...)", 80000.0)]
    fetch_rows += [(10 + i, "__amd_rocclr_copyBuffer", mib * 1024 / 2) for i in range(3)]
    write_rows = [(1, "mla::attn_bf16(...)", 33536.0), (2, "mla::uv_bf16(...)", 2048.0),
                  (3, "mla::absorb_q_bf16(...)", 9216.0)]
    write_rows += [(10 + i, "__amd_rocclr_copyBuffer", mib * 1024.0) for i in range(3)]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch_rows)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write_rows)
    bench.write_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), mib, "cmd")
    rec = json.loads(out.read_text())
    assert rec["read_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(80000.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(33536.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(80000.0 * 2048 + 33536.0 * 1024)
    assert rec["algorithmic_bytes_per_launch"] == 64 * 2048 * 1152
    assert rec["kernel_source_sha256_16"] == bench.source_hash()
    assert rec["FETCH_SIZE_kib_uv"] == pytest.approx(26000.0)
    # the whole call: the three kernels' counters, each scaled like the attention kernel's
    assert rec["step_bytes_per_call"] == pytest.approx((80000.0 + 26000.0 + 9800.0) * 2048
                                                       + (33536.0 + 2048.0 + 9216.0) * 1024)
    assert rec["algorithmic_step_bytes_per_call"] == bench.step_bytes(64, 2048)


def test_traffic_record_is_used_only_while_the_code_matches(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("int kernel() { return 1; }\n")
    rec_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(src),))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec_file))
    assert bench.traffic_from_profile() == (None, None)       # no record
    rec_file.write_text(json.dumps({"kernel_source_sha256_16": bench.source_hash(),
                                    "bytes_per_launch": 123.0, "step_bytes_per_call": 456.0}))
    assert bench.traffic_from_profile() == (123.0, 456.0)
    src.write_text("int kernel() { return 1; }  // comment edits keep the record\n")
    assert bench.traffic_from_profile() == (123.0, 456.0)
    src.write_text("int kernel() { return 2; }\n")
    assert bench.traffic_from_profile() == (None, None)       # the code changed


def test_step_bytes_and_flops():
    # headline call: 131,072 selected rows of 1,152 bytes, two 16 MiB weight matrices,
    # q_nope + q_pe in and the output out (320 bf16 per row and head), 4-byte indices
    assert bench.step_bytes(64, 2048) == 150_994_944 + 33_554_432 + 5_242_880 + 524_288
    assert bench.step_flops(64, 2048) == 131_072 * 2 * 128 * 1088 + 4 * 64 * 128 * 128 * 512


def test_every_benchmark_mode_has_its_function():
    # each mode flag dispatches to a function of the module; a missing one fails only at run time
    for name in ("bench_prefill", "prefill_measure", "bench_project", "bench_append", "bench_dequant",
                 "cpu_baseline", "write_traffic", "traffic_from_profile"):
        assert callable(getattr(bench, name, None)), name
