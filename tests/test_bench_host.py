"""bench.py's host logic on the CPU (no GPU, no kernel launch): the argument defaults, the
refusal of more than one GPU, the names of the counter summaries, the algorithmic bytes per
launch, and the counter parsing and copy calibration that give the roofline's ``traffic``."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_defaults():
    a = bench.parse_args([])
    assert a.workload == "qwen3_32b_like_decode" and a.gpus == 1
    assert (a.steps, a.warmup) == bench.DEFAULT_STEPS["qwen3_32b_like_decode"]
    assert a.counters == os.path.join(ROOT, "profiles", "hbm_counters.qwen3_32b_like_decode.json")
    assert not a.graph


@pytest.mark.parametrize("argv,tag", [
    ([], "qwen3_32b_like_decode"),
    (["--variant", "fused"], "qwen3_32b_like_decode.fused"),
    (["--workload", "prefill_chunk", "--variant", "plain"], "prefill_chunk.plain"),
    (["--workload", "prefill_chunk", "--k-block", "64"], "prefill_chunk.k64"),
    (["--k-bits", "2", "--v-bits", "2"], "qwen3_32b_like_decode.k2v2bit"),
    (["--workload", "small_batch_decode", "--variant", "fused", "--v-bits", "2"],
     "small_batch_decode.fused.k4v2bit"),
])
def test_counter_file_names(argv, tag):
    a = bench.parse_args(argv)
    assert bench.workload_tag(a) == tag
    assert os.path.basename(a.counters) == f"hbm_counters.{tag}.json"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr and r.stdout == ""


def _setup_stub(argv):
    s = bench.Setup.__new__(bench.Setup)          # the byte formulas only: no device set-up
    s.args = bench.parse_args(argv)
    return s


def test_algorithmic_bytes():
    s = _setup_stub([])
    # per (token, head): K and V codes 64 B each plus two fp16 (scale, zero) pairs
    assert s.kv_row_bytes() == 136
    # write: bf16 K and V in (2 x 256 B per head), the cache rows out, the int32 slot
    assert s.write_bytes(1, 8) == 5188 and s.write_bytes(256, 8) == 256 * 5188
    # decode of lengths 16 and 17 (3 pages of 16), Hkv 8, Hq 64: 33 tokens x 8 x 136,
    # bf16 q and fp32 out per query head, one page id per page, one length per sequence
    assert s.decode_bytes([16, 17], 8, 64, 16) == 33 * 1088 + 2 * 64 * (256 + 512) + 3 * 4 + 2 * 4
    s2 = _setup_stub(["--k-bits", "2", "--v-bits", "2"])
    assert s2.kv_row_bytes() == 72 and s2.write_bytes(1, 8) == 8 * (512 + 72) + 4


DEC = "kvrq::(anonymous namespace)::decode_balanced_kernel<128, 2, 0>(kvrq::DecodeArgs)"
SPLIT = "kvrq::(anonymous namespace)::decode_split_kernel<64, 2, false, 0>(kvrq::DecodeArgs)"
COPY = "kvrq::(anonymous namespace)::device_copy_kernel(HIP_vector_type<unsigned int, 4u>*, long)"


def _counter_dir(path, counter, rows):
    os.makedirs(os.path.join(path, "host", "1234"))
    with open(os.path.join(path, "host", "1234", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
        # another counter in the same file and a kernel that is not the library's: both ignored
        w.writerow({"Kernel_Name": DEC, "Counter_Name": "GRBM_COUNT", "Counter_Value": 7})
        w.writerow({"Kernel_Name": "at::native::fill_kernel", "Counter_Name": counter, "Counter_Value": 9e9})


def test_counters_to_traffic(tmp_path):
    fd, wd, out = str(tmp_path / "F"), str(tmp_path / "W"), str(tmp_path / "c.json")
    # a 1 GiB copy counts half its reads in FETCH_SIZE (factor 2) and all its writes
    _counter_dir(fd, "FETCH_SIZE", [(DEC, 1000), (DEC, 1002), (COPY, 524288), (SPLIT, 40)])
    _counter_dir(wd, "WRITE_SIZE", [(DEC, 500), (DEC, 502), (COPY, 1048576), (SPLIT, 10)])
    bench.parse_counter_dirs(fd, wd, out, profiled_args="--steps 5")
    c = json.load(open(out))
    assert c["kernel_hash"] == bench.kernel_source_hash()
    assert c["fetch_kib"][DEC] == {"mean": 1001.0, "dispatches": 2}
    assert c["write_kib"][DEC] == {"mean": 501.0, "dispatches": 2}
    assert not any("fill_kernel" in k for k in c["fetch_kib"])
    copy = 1 << 30
    t, note = bench.traffic_from_counters(out, ("decode_balanced_kernel", "decode_split_kernel"), copy)
    assert note == {"fetch_factor": 2.0, "write_factor": 1.0}
    assert t == 1001 * 1024 * 2 + 501 * 1024 * 1
    # the first listed symbol that the summary holds is the one reported
    t2, _ = bench.traffic_from_counters(out, ("decode_split_kernel", "decode_balanced_kernel"), copy)
    assert t2 == 40 * 1024 * 2 + 10 * 1024
    assert bench.traffic_from_counters(out, ("rotquant_write_kernel",), copy) == (None, "incomplete")
    assert bench.traffic_from_counters(str(tmp_path / "none.json"), ("x",), copy) == (None, None)
    c["kernel_hash"] = "0" * 16                       # counters taken on other kernel sources
    json.dump(c, open(out, "w"))
    assert bench.traffic_from_counters(out, ("decode_balanced_kernel",), copy) == (None, "stale")


def test_graph_replay_covers_decode_steps_only():
    a = bench.parse_args(["--workload", "prefill_chunk", "--graph"])
    r = bench.measure_graph(types.SimpleNamespace(), a, None)
    assert "skipped" in r
