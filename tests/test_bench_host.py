"""Host logic of bench.py (CPU only): the algorithmic byte counts the
roofline divides by, the counter calibration and span arithmetic on
synthetic rocprofv3 tables, the window summary, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import workloads as wl  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _table(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})
            # another counter in the same table is ignored
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": "GRBM_COUNT",
                        "Counter_Value": 1e9})


def test_headline_bytes():
    # 21504 rows of 168 blocks of 18 bytes, plus x (5376 floats) and y (21504 floats)
    assert bench.matvec_bytes(21504, 5376, 1) == 21504 * 168 * 18 + 4 * 5376 + 4 * 21504 == 65135616
    assert bench.matvec_bytes(6144, 2048, 1) == 6144 * 64 * 18 + 4 * (2048 + 6144) == 7110656
    # B rows of activations and outputs; Q8_0 blocks of 34 bytes
    assert bench.matvec_bytes(10, 64, 3, block_bytes=34) == 10 * 2 * 34 + 4 * 3 * (64 + 10)


def test_decode_step_bytes():
    # the bench's figure is the mean over the run's 16 steps of: every weight
    # byte, the Q8_0 table once (logits) plus the B gathered rows, every
    # visible key and value row of every layer plus the appended ones, logits
    def mean_step(m, kv_bytes=4):
        return sum(bench.decode_algorithmic_bytes(m, s, kv_bytes) for s in range(m.steps)) / m.steps
    assert abs(mean_step(wl.QWEN3_4B) / 1e9 - 7.3169) < 5e-4
    assert abs(mean_step(wl.GEMMA4_31B) / 1e9 - 20.998) < 5e-3
    # each later step reads one more key and value row per layer, kv head and
    # sequence, except in sliding-window layers whose window is full
    m = wl.QWEN3_4B
    per_key = sum(2 * ly.n_kv_heads * ly.head_dim * 4 for ly in m.layers) * m.batch
    assert bench.decode_algorithmic_bytes(m, 1) - bench.decode_algorithmic_bytes(m, 0) == per_key
    g = wl.GEMMA4_31B
    per_key_full = sum(2 * ly.n_kv_heads * ly.head_dim * 4 for ly in g.layers if not ly.window) * g.batch
    assert bench.decode_algorithmic_bytes(g, 1) - bench.decode_algorithmic_bytes(g, 0) == per_key_full
    # binary16 caches halve the cache part only
    q0, h0 = bench.decode_algorithmic_bytes(m, 0), bench.decode_algorithmic_bytes(m, 0, kv_bytes=2)
    n = m.start_pos + 1
    cache = sum(m.batch * ly.n_kv_heads * ly.head_dim * 4 * (2 * n + 2) for ly in m.layers)
    assert q0 - h0 == cache // 2


def test_summary_of_windows():
    s = bench.summarize([1.0, 3.0, 2.0, 2.0, 2.0])
    assert s["median_ms"] == 2.0 and s["min_ms"] == 1.0 and s["max_ms"] == 3.0 and s["windows"] == 5
    assert abs(s["cv"] - (0.4 ** 0.5) / 2.0) < 1e-4


def test_counter_calibration(tmp_path):
    # FETCH_SIZE reads half of a copy's bytes, WRITE_SIZE all of them
    gib_kib = bench.COPY_BYTES / 1024.0
    fetch = [("mv_b1_kernel<0, 3>", 32000.0), ("mv_b1_kernel<0, 3>", 32100.0), ("mv_b1_kernel<0, 3>", 32200.0),
             ("__amd_rocclr_copyBuffer", gib_kib / 2), ("__amd_rocclr_copyBuffer", gib_kib / 2),
             ("__amd_rocclr_copyBuffer", 1.0)]  # a small copy is not a calibration copy
    write = [("mv_b1_kernel<0, 3>", 100.0), ("mv_b1_kernel<0, 3>", 100.0), ("mv_b1_kernel<0, 3>", 100.0),
             ("__amd_rocclr_copyBuffer", gib_kib), ("__amd_rocclr_copyBuffer", gib_kib)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _table(f, "FETCH_SIZE", fetch)
    _table(w, "WRITE_SIZE", write)
    t = bench.pmc_traffic(str(f), str(w))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == round(32100.0 * 1024 * 2 + 100.0 * 1024)


def test_counter_span_between_markers(tmp_path):
    gib_kib = bench.COPY_BYTES / 1024.0
    # warm-up dispatch, marker, 2 units of 3 dispatches, marker, trailing dispatch
    fetch = [("attn_split_kernel", 999.0), ("__amd_rocclr_copyBuffer", gib_kib / 2)] + \
        [("attn_split_kernel", 100.0), ("attn_merge_kernel", 10.0), ("mv_b1_kernel", 50.0)] * 2 + \
        [("__amd_rocclr_copyBuffer", gib_kib / 2), ("argmax_part_kernel", 777.0)]
    write = [("attn_split_kernel", 999.0), ("__amd_rocclr_copyBuffer", gib_kib)] + \
        [("attn_split_kernel", 4.0), ("attn_merge_kernel", 1.0), ("mv_b1_kernel", 0.0)] * 2 + \
        [("__amd_rocclr_copyBuffer", gib_kib), ("argmax_part_kernel", 777.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _table(f, "FETCH_SIZE", fetch)
    _table(w, "WRITE_SIZE", write)
    t = bench.pmc_traffic_span(str(f), str(w), units=2)
    assert t["dispatches_per_unit"] == 3
    assert t["fetch_bytes_per_unit"] == round(160.0 * 1024 * 2)
    assert t["write_bytes_per_unit"] == round(5.0 * 1024)
    assert t["bytes_per_unit"] == t["fetch_bytes_per_unit"] + t["write_bytes_per_unit"]


def test_source_digest_tracks_the_kernels():
    a = bench.kernel_source_hash(("matvec.hip", "common.hpp"))
    assert a == bench.kernel_source_hash(("matvec.hip", "common.hpp"))
    assert a != bench.kernel_source_hash(("attention.hip",))
    assert "matvec.hip" in bench.all_sources() and "attention.hip" in bench.all_sources()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
