"""Host logic of bench.py, on the CPU: the algorithmic bytes and flops behind the roofline
figures, the rocprofv3 trace summary and counter-traffic arithmetic, and the refusal of
more than one GPU.  Nothing here touches a GPU or imports torch."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

H, I, E, K, S = 2048, 768, 256, 6, 1
SHP = (H, I, E, K, S)


def test_expert_bytes_follow_the_storage_formats():
    # bf16: three I x H matrices of 2-byte values
    assert bench.expert_bytes(0, H, I) == 3 * 768 * 2048 * 2 == 9_437_184
    # NVFP4: per matrix, one 4-bit code per weight, one E4M3 byte per 16 weights and one
    # fp32 tensor scale (the per-expert figure the pages' format gives: 2,654,220 B)
    assert bench.expert_bytes(1, H, I) == 3 * (768 * 2048 // 2 + 768 * 2048 // 16 + 4) == 2_654_220
    # INT4: one 4-bit code per weight and one bf16 scale per 128 weights
    assert bench.expert_bytes(2, H, I) == 3 * (768 * 2048 // 2 + 2 * 768 * 2048 // 128) == 2_433_024
    assert bench.expert_bytes(0, H, I) / bench.expert_bytes(1, H, I) == pytest.approx(3.556, abs=1e-3)


def test_single_token_layer_bytes():
    # 6 routed + 1 shared expert, the 2 MiB fp32 router matrix, one bf16 token in and out
    assert bench.algorithmic_bytes(0, SHP, 1, 6) == 68_165_632          # 68.17 MB
    assert bench.algorithmic_bytes(1, SHP, 1, 6) == 20_684_884          # 20.68 MB
    assert bench.algorithmic_bytes(0, SHP, 1, 6) / bench.algorithmic_bytes(1, SHP, 1, 6) > 3.2
    # the dense layer: the shared expert alone, no router
    dense = (H, 4096, 0, 0, 1)
    assert bench.algorithmic_bytes(0, dense, 1, 0) == 3 * 4096 * 2048 * 2 + 4 * 2048


def test_small_batch_bytes_grow_with_touched_experts_only():
    b8 = bench.algorithmic_bytes(0, SHP, 8, 44)
    b8_more = bench.algorithmic_bytes(0, SHP, 8, 45)
    assert b8_more - b8 == bench.expert_bytes(0, H, I)
    assert b8 == pytest.approx(429e6, rel=0.01)  # about 44 distinct routed experts + shared


def test_prefill_flops():
    f = bench.layer_flops(SHP, 8192)
    assert f == 2.0 * 8192 * 7 * 3 * 2048 * 768
    assert f / 1e9 == pytest.approx(541.17, abs=0.01)
    # floors at the published peaks: ~216 us of bf16 MFMA
    assert f / (bench.BF16_PEAK_TFLOPS * 1e12) * 1e6 == pytest.approx(216.5, abs=0.1)


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


KFIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _trace_rows():
    """A warm-up dispatch, the start marker, two timed layer calls of two kernels plus the
    status call's own copy, the end marker and a dispatch after it; rows out of time order."""
    t = []
    def k(name, start, dur):
        t.append({"Kernel_Name": name, "Start_Timestamp": start, "End_Timestamp": start + dur})
    k("void flint::(anonymous namespace)::decode1_kernel<0>(flint::D1Args)", 0, 50_000)
    k("flint::ws_status_kernel(unsigned int*, int*)", 100_000, 1_000)
    k("void flint::(anonymous namespace)::decode1_kernel<0>(flint::D1Args)", 102_000, 20_000)
    k("void flint::gemv_combine_kernel(int, int, int, int, float const*)", 123_000, 4_000)
    k("void flint::(anonymous namespace)::decode1_kernel<0>(flint::D1Args)", 128_000, 22_000)
    k("void flint::gemv_combine_kernel(int, int, int, int, float const*)", 151_000, 6_000)
    k("__amd_rocclr_copyBuffer", 158_000, 1_000)
    k("flint::ws_status_kernel(unsigned int*, int*)", 160_000, 1_000)
    k("void flint::(anonymous namespace)::decode1_kernel<0>(flint::D1Args)", 200_000, 90_000)
    return t[::-1]


def test_summarize_trace_counts_only_the_marked_window(tmp_path):
    p = tmp_path / "kernel_trace.csv"
    _write_csv(p, KFIELDS, _trace_rows())
    md = bench.summarize_trace(str(p), "title", "cmd")
    assert "Dispatches between the two ws_status_kernel markers (the timed trials only): 5, over 59.0 us." in md
    rows = {l.split("|")[1].strip(): l for l in md.splitlines() if l.startswith("| ") and not l.startswith("| kernel |")}
    dec = [c.strip() for c in rows["decode1_kernel<0>"].split("|")[2:7]]
    assert dec == ["2", "21.00", "20.00", "22.00", "79.25"]  # 42 of the window's 53 us of kernels
    comb = [c.strip() for c in rows["gemv_combine_kernel"].split("|")[2:7]]
    assert comb == ["2", "5.00", "4.00", "6.00", "18.87"]
    assert rows["__amd_rocclr_copyBuffer"].split("|")[2].strip() == "1"
    assert set(rows) == {"decode1_kernel<0>", "gemv_combine_kernel", "__amd_rocclr_copyBuffer"}


def test_summarize_trace_needs_two_markers(tmp_path):
    p = tmp_path / "kernel_trace.csv"
    _write_csv(p, KFIELDS, [r for r in _trace_rows() if not (r["Start_Timestamp"] == 160_000)])
    with pytest.raises(SystemExit):
        bench.summarize_trace(str(p), "title", "cmd")


CFIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp"]


def test_traffic_scaled_by_the_copy_calibration(tmp_path):
    # the plain 1 GiB copy reads 1.25 GiB and writes 1 GiB by its counters
    copy_f, copy_w = tmp_path / "cf.csv", tmp_path / "cw.csv"
    _write_csv(copy_f, CFIELDS, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                                  "Counter_Value": 1.25 * (1 << 20), "Start_Timestamp": 0}])
    _write_csv(copy_w, CFIELDS, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                                  "Counter_Value": float(1 << 20), "Start_Timestamp": 0}])
    mark = "flint::ws_status_kernel(unsigned int*, int*)"
    ka, kb = "void flint::ka(int)", "void flint::kb(int)"

    def run(ctr, vals):
        rows = [{"Kernel_Name": ka, "Counter_Name": ctr, "Counter_Value": 999999.0, "Start_Timestamp": 1},
                {"Kernel_Name": mark, "Counter_Name": ctr, "Counter_Value": 0.0, "Start_Timestamp": 10}]
        ts = 20
        for va, vb in vals:  # two layer calls: ka then kb
            rows.append({"Kernel_Name": ka, "Counter_Name": ctr, "Counter_Value": va, "Start_Timestamp": ts})
            rows.append({"Kernel_Name": kb, "Counter_Name": ctr, "Counter_Value": vb, "Start_Timestamp": ts + 1})
            ts += 10
        rows.append({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": ctr, "Counter_Value": 5.0,
                     "Start_Timestamp": ts})
        rows.append({"Kernel_Name": mark, "Counter_Name": ctr, "Counter_Value": 0.0, "Start_Timestamp": ts + 5})
        return rows

    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(f, CFIELDS, run("FETCH_SIZE", [(1000.0, 250.0), (1500.0, 250.0)]))
    _write_csv(w, CFIELDS, run("WRITE_SIZE", [(100.0, 20.0), (100.0, 20.0)]))
    out = bench.traffic_json(str(copy_f), str(copy_w), ["wl=%s,%s" % (f, w)])
    assert out["calibration"]["FETCH_SIZE"]["scale"] == pytest.approx(0.8)
    assert out["calibration"]["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    c = out["configs"]["wl"]
    assert c["layer_calls_counted"] == 2
    fetch = (1000 + 250 + 1500 + 250) * 0.8 * 1024
    write = (100 + 20 + 100 + 20) * 1024
    assert c["bytes_per_layer_call"] == int(round((fetch + write) / 2))
    assert c["per_kernel_bytes_per_layer_call"]["ka"]["FETCH_SIZE"] == int(round(2500 * 0.8 * 1024 / 2))
    assert out["csrc_sha256"] == bench.csrc_digest()


def test_counter_traffic_is_dropped_once_the_sources_change(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"csrc_sha256": bench.csrc_digest(),
                             "configs": {"decode_t1": {"bytes_per_layer_call": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic("decode_t1") == 123
    assert bench.measured_traffic("prefill") is None
    p.write_text(json.dumps({"csrc_sha256": "0" * 64, "configs": {"decode_t1": {"bytes_per_layer_call": 123}}}))
    assert bench.measured_traffic("decode_t1") is None


def test_committed_traffic_matches_the_current_sources():
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    if t["csrc_sha256"] != bench.csrc_digest():
        pytest.skip("the kernels changed since the committed counters were taken (bench reports traffic null)")
    for name in bench.DEFAULT_CONFIGS:
        assert name in t["configs"], name


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "nope"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "unknown workload" in r.stderr
