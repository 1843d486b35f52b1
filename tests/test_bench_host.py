"""bench.py host logic (no GPU): the algorithmic byte counts behind every
roofline figure, the rocprofv3 counter bookkeeping, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_match_the_workload_table():
    # Global workload (30720 x 7168, top-8 of 256): dispatch reads x and the
    # slots and writes K payload+scale rows; combine reads K BF16 rows, the
    # slots and gates, and writes y.  Counted by hand from the layouts.
    T, H, K, E, G = 30720, 7168, 8, 256, 56
    ab = bench.algorithmic_bytes(T, H, K, E)
    assert ab["dispatch"] == 2 * T * H + 4 * T * K + T * K * (H + 4 * G) == 2_258_042_880
    assert ab["combine"] == 2 * T * K * H + 8 * T * K + 2 * T * H == 3_965_583_360
    assert ab["combine_q8"] == T * K * (H + 4 * G) + 8 * T * K + 2 * T * H == 2_259_025_920
    assert ab["route"] == 4 * T * E + 12 * T * K == 34_406_400
    one = bench.algorithmic_bytes(1, H, K, E)
    assert (one["dispatch"], one["combine"], one["combine_q8"]) == (73_504, 129_088, 73_536)
    # Prefill with a shared expert (K = 9): 5,301,862,400 / 9,399,959,552 B.
    pf = bench.algorithmic_bytes(65536, H, 9, E)
    assert pf["dispatch"] == 5_301_862_400 and pf["combine"] == 9_399_959_552


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_rocprof_reads_stats_and_counters(tmp_path, capsys):
    _write_csv(str(tmp_path / "p" / "x_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [["combine_kernel<8, false, false, 4>", 10, 732500, 720000, 750000, 55.5]])
    _write_csv(str(tmp_path / "p" / "x_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["k", "FETCH_SIZE", 10.0], ["k", "FETCH_SIZE", 30.0]])
    out = tmp_path / "s.txt"
    bench.summarize_rocprof(str(tmp_path / "p"), str(out))
    text = out.read_text()
    assert "732.50" in text and "720.00" in text and "750.00" in text
    assert "    2                 20.0     FETCH_SIZE  k" in text


def test_record_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    tf = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    comb = "void moedc::(anonymous namespace)::combine_kernel<8, false, 16, 1>(moedc::CombineArgs)"
    comb_q8 = "void moedc::(anonymous namespace)::combine_kernel<8, true, 16, 1>(moedc::CombineArgs)"
    disp = "void moedc::(anonymous namespace)::dispatch_token_block<false, true>(moedc::DispatchArgs)"
    _write_csv(str(tmp_path / "f" / "f_counter_collection.csv"), hdr,
               [[comb, "FETCH_SIZE", 1000.0], [comb, "FETCH_SIZE", 1000.0],
                [comb_q8, "FETCH_SIZE", 7.0], [disp, "FETCH_SIZE", 300.0]])
    _write_csv(str(tmp_path / "w" / "w_counter_collection.csv"), hdr,
               [[comb, "WRITE_SIZE", 500.0], [comb_q8, "WRITE_SIZE", 9.0],
                [disp, "WRITE_SIZE", 100.0]])
    # A 4096-byte copy whose counters read 2 KiB fetched and 4 KiB written.
    _write_csv(str(tmp_path / "cf" / "c_counter_collection.csv"), hdr,
               [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 2.0]])
    _write_csv(str(tmp_path / "cw" / "c_counter_collection.csv"), hdr,
               [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 4.0]])
    dirs = [str(tmp_path / d) for d in ("f", "w", "cf", "cw")]
    bench.record_traffic("global", *dirs, 4096)
    d = json.loads(tf.read_text())
    g = d["global"]
    # BF16 combine only (the Q8 kernel is another row), scaled by the copy.
    assert g["combine"]["fetch_bytes"] == 1000 * 1024 * 2.0
    assert g["combine"]["write_bytes"] == 500 * 1024 * 1.0
    assert g["dispatch"]["bytes_per_launch"] == 300 * 1024 * 2.0 + 100 * 1024
    assert g["combine"]["source_sha"] == bench.source_sha(bench.KERNEL_SOURCES["combine"])
    assert "route" not in g
    # The recorded figure is served while the kernel source is unchanged...
    assert bench.measured_traffic("combine") == 1000 * 1024 * 2.0 + 500 * 1024
    # ...for the workload the counters were taken on only...
    assert bench.measured_traffic("combine", "prefill") is None
    # ...and a second workload's run is merged beside the first.
    bench.record_traffic("prefill", *dirs, 8192)
    d = json.loads(tf.read_text())
    assert set(d) == {"_about", "global", "prefill"}
    assert bench.measured_traffic("combine", "prefill") == 2 * (1000 * 1024 * 2.0 + 500 * 1024)
    # ...and withheld once the kernel changes.
    d["global"]["combine"]["source_sha"] = "0" * 16
    tf.write_text(json.dumps(d))
    assert bench.measured_traffic("combine") is None
    assert bench.measured_traffic("dispatch") == 300 * 1024 * 2.0 + 100 * 1024
    # Runs without combine and dispatch rows are an error, and nothing is written.
    tf.unlink()
    _write_csv(str(tmp_path / "e" / "e_counter_collection.csv"), hdr, [["other", "FETCH_SIZE", 1.0]])
    with pytest.raises(SystemExit):
        bench.record_traffic("global", str(tmp_path / "e"), *dirs[1:], 4096)
    assert not tf.exists()


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = 'int a = 1; // note\n/* block */ const char *s = "// kept"; float b = a / 2.0f;\n'
    (tmp_path / "k.hip").write_text(src)
    h = bench.source_sha("k.hip")
    (tmp_path / "k.hip").write_text(src.replace("note", "another note").replace("block", "x"))
    assert bench.source_sha("k.hip") == h            # comments only
    (tmp_path / "k.hip").write_text(src.replace('"// kept"', '"// changed"'))
    assert bench.source_sha("k.hip") != h            # a string literal is code
    (tmp_path / "k.hip").write_text(src.replace("a / 2.0f", "a * 2.0f"))
    assert bench.source_sha("k.hip") != h


def test_source_hash_covers_every_file_of_a_kernel(tmp_path, monkeypatch):
    """A record is keyed to the kernel's .hip file and the headers it
    includes: a code change in a header invalidates it too."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("int main_part = 1;\n")
    (tmp_path / "h.hpp").write_text("int helper = 2;\n")
    h = bench.source_sha(("k.hip", "h.hpp"))
    assert h != bench.source_sha("k.hip")
    (tmp_path / "h.hpp").write_text("int helper = 3;\n")
    assert bench.source_sha(("k.hip", "h.hpp")) != h
    for key, files in bench.KERNEL_SOURCES.items():
        assert "combine_moedc_route_amd/csrc/internal.hpp" in files, key
    assert "combine_moedc_route_amd/csrc/quant.hpp" in bench.KERNEL_SOURCES["dispatch"]


def test_summary_splits_a_kernel_launched_with_several_grid_sizes(tmp_path):
    """One kernel serving two batch sizes gets one row per launch shape."""
    name = "void moedc::(anonymous namespace)::dispatch_token_block<false, true>(moedc::DispatchArgs)"
    _write_csv(str(tmp_path / "p" / "b_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[name, 3, 1000.0, 4000.0, 430000.0, 100.0]])
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]
    _write_csv(str(tmp_path / "p" / "b_kernel_trace.csv"), hdr,
               [[name, 0, 430000, 27525120, 896], [name, 0, 4000, 86016, 896],
                [name, 0, 6000, 86016, 896]])
    bench.summarize_rocprof(str(tmp_path / "p"), str(tmp_path / "s.txt"))
    text = (tmp_path / "s.txt").read_text()
    assert "per launch shape" in text
    assert "     1     430.00     430.00     430.00   27525120   896" in text
    assert "     2       5.00       4.00       6.00      86016   896" in text


def test_trace_summary_decodes_records_and_overlap():
    """Synthetic dispatch trace records (include/moedc_trace.h layout): two
    tokens of two waves on two CUs, times in 10 ns ticks."""
    import numpy as np
    T, nw = 2, 2
    rec = np.zeros((T * nw, 8), np.uint64)
    hw_a = (np.uint64(3) << np.uint64(32)) | np.uint64(0x0500)   # XCC 3, CU bits 0x05
    hw_b = (np.uint64(1) << np.uint64(32)) | np.uint64(0x0A00)   # XCC 1, CU bits 0x0A
    #         start loaded scales quant issued done   (ticks)
    stamps = [[100, 200, 250, 260, 300, 400],   # token 0 wave 0, CU A
              [350, 450, 470, 480, 520, 600],   # token 0 wave 1, CU A: loads while wave 0 stores
              [100, 150, 160, 170, 180, 200],   # token 1 wave 0, CU B
              [900, 950, 960, 970, 980, 1000]]  # token 1 wave 1, CU B
    for i, st in enumerate(stamps):
        t, w = divmod(i, nw)
        rec[i, 0] = (np.uint64(t) << np.uint64(32)) | np.uint64(w)
        rec[i, 1] = hw_a if i < 2 else hw_b
        rec[i, 2:] = np.array(st, np.uint64)
    r = bench.trace_summary(rec, T, nw, sample_us=0.1)
    assert r["records_complete"] and r["stamps_monotone"]
    assert r["waves"] == 4 and r["cus"] == 2
    assert abs(r["span_us"] - 9.0) < 1e-9                        # (1000 - 100) ticks
    assert abs(r["phase_us"]["load"]["median_us"] - 0.75) < 1e-9  # loads 1.0, 1.0, 0.5, 0.5 us
    assert abs(r["phase_us"]["store complete"]["max_us"] - 1.0) < 1e-9
    # CU A at 3.5-4.0 us: wave 1 loading, wave 0 storing -> some overlap, but not everywhere
    assert 0 < r["frac_busy_cu_samples_loading_and_storing"] < 1
    # a record missing (zero stamps) or out of order is reported
    bad = rec.copy()
    bad[3, 2:] = 0
    assert not bench.trace_summary(bad, T, nw)["records_complete"]
    bad = rec.copy()
    bad[0, 4] = 150   # quantized before scales known
    assert not bench.trace_summary(bad, T, nw)["stamps_monotone"]


def test_parity_compares_route_slots_and_outputs():
    """bench.parity on a small synthetic case: equal outputs report exact
    and zero ulps; a changed slot byte, gate ulp or BF16 step is reported."""
    import numpy as np
    rng = np.random.default_rng(0)
    T, K, H, S, sd = 6, 2, 256, 20, 512
    slots = rng.choice(S, (T, K), replace=False).astype(np.int32)
    slots[0, 1] = -1
    r = {"topk_ids": rng.integers(0, 8, (T, K)).astype(np.int32), "slots": slots,
         "counts": np.arange(8, dtype=np.int32), "offsets": np.arange(9, dtype=np.int32),
         "dropped": 1, "topk_w": rng.random((T, K)).astype(np.float32)}
    dbuf = rng.integers(0, 256, (S, sd)).astype(np.uint8)
    y = rng.integers(0, 2 ** 16, (T, H)).astype(np.uint16)
    orc = {"route": r, "dbuf": dbuf, "y": y, "slot_stride": sd}
    gpu = {"topk_ids": r["topk_ids"].copy(), "slots": slots.copy(), "counts": r["counts"].copy(),
           "offsets": r["offsets"].copy(), "dropped": np.array([1], np.int32),
           "w": r["topk_w"].copy(), "dbuf": dbuf.reshape(-1).copy(), "y": y.copy()}
    p = bench.parity(gpu, orc)
    assert p["route_ids_slots_counts_exact"] and p["dispatch_slot_bytes_exact"]
    assert p["gates_max_ulp"] == 0 and p["combine_max_bf16_ulp"] == 0
    unused = np.setdiff1d(np.arange(S), slots[slots >= 0])[0]
    gpu["dbuf"][unused * sd] ^= 1            # a byte outside every occupied slot: not compared
    assert bench.parity(gpu, orc)["dispatch_slot_bytes_exact"]
    gpu["dbuf"][slots[2, 0] * sd + 5] ^= 1   # a payload byte of an occupied slot
    gpu["w"][1, 1] = np.nextafter(gpu["w"][1, 1], np.float32(2))
    gpu["y"][3, 7] += 1
    gpu["slots"][4, 0] = -1
    p = bench.parity(gpu, orc)
    assert not p["dispatch_slot_bytes_exact"] and not p["route_ids_slots_counts_exact"]
    assert p["gates_max_ulp"] == 1 and p["combine_max_bf16_ulp"] == 1
    assert p["combine_tokens_not_bit_identical"] == 1
