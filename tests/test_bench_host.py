"""Host-side checks of bench.py: the one-GPU contract, the counter summary's
arithmetic, and the FLOP / byte counts the reported rates divide by.  No GPU
is used."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_bsa_counts_by_hand():
    # 3 live tiles over 2 heads, B = 2, bs = 4, d = 8, bf16
    layout = np.zeros((2, 3, 3), dtype=np.int32)
    layout[0, 0, 0] = layout[0, 2, 1] = layout[1, 1, 2] = 1
    tiles, flops, nbytes = bench.bsa_counts(layout, B=2, bs=4, d=8)
    assert tiles == 6
    assert flops == 4 * 4 * 4 * 8 * 3 * 2
    q_o = 2 * 2 * 2 * 3 * 4 * 8 * 2          # read q and write out: B H S d, 2 bytes
    kv = 2 * 4 * 8 * 2 * 3 * 2                # K and V tile per live tile per batch item
    lse = 4 * 2 * 2 * 3 * 4                   # fp32 per query row
    assert nbytes == q_o + kv + lse


def test_topk_counts_by_hand():
    idx = np.array([[[0, 5, -1, 2], [-1, -1, -1, -1]]], dtype=np.int32)   # B1, M2, topk 4
    valid, flops, nbytes = bench.topk_counts(idx, H=3, d=16)
    assert valid == 3
    assert flops == 4 * 16 * 3 * 3
    assert nbytes == 3 * 16 * 2 + 2 * (2 * 3 * 16 * 2 + 4 * 4)


def test_percentiles():
    p = bench.percentiles([float(x) for x in range(1, 101)])
    assert p["median_ms"] == pytest.approx(50.5)
    assert p["p10_ms"] == pytest.approx(10.9)
    assert p["p90_ms"] == pytest.approx(90.1)


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_counters_scales_by_the_calibration_copy(tmp_path):
    fwd = "_ZN3bsa12_GLOBAL__N_118bsa_fwd_dma_kernelILi128ELi128ELi1ELi2ELb0ELb0ELb0ELb0ELb0EEEvPK"
    topk = "void topk_kernel<512, true>(bool _Accum const*, ...)"
    neg = "void at::native::neg_kernel_cuda(...)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # the copy reads and writes 1 GiB; FETCH_SIZE sees half of it, WRITE_SIZE all
    _write_counters(fetch, "FETCH_SIZE", [(neg, 524288.0), (fwd, 1000.0), (fwd, 3000.0), (topk, 10.0)])
    _write_counters(write, "WRITE_SIZE", [(neg, 1048576.0), (fwd, 500.0), (fwd, 500.0), (topk, 1.0)])
    out = tmp_path / "traffic.json"
    res = bench.summarize_counters(str(fetch), str(write), str(out))
    assert res["_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert res["_calibration"]["write_scale"] == pytest.approx(1.0)
    f = res["bsa_forward"]
    assert f["read_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)    # mean of the two launches
    assert f["write_bytes"] == pytest.approx(500.0 * 1024)
    assert f["bytes_per_launch"] == pytest.approx(f["read_bytes"] + f["write_bytes"])
    assert res["topk_sparse_attn"]["read_bytes"] == pytest.approx(10.0 * 1024 * 2.0)
    assert json.loads(out.read_text())["bsa_forward"]["source_sha"] == \
        bench.source_hash(bench.KERNEL_SOURCES["bsa_forward"])


def test_same_segment_tiles_by_hand():
    # bs 2, blocks of ids [0 0] [0 1] [1 1]: block 0 and block 2 share no segment
    seg = np.array([[0, 0, 0, 1, 1, 1]], dtype=np.int32)
    full = np.ones((1, 3, 3), dtype=np.int32)
    assert bench.same_segment_tiles(full, seg, 2) == 7
    lower = np.tril(np.ones((3, 3), dtype=np.int32))[None]
    assert bench.same_segment_tiles(lower, seg, 2) == 5
    # a cut last block takes the last id; two batch items add up: blocks
    # [0 0] [1 1] [2 2] overlap only themselves, a single segment everything
    seg2 = np.array([[0, 0, 1, 1, 2], [5, 5, 5, 5, 5]], dtype=np.int32)
    assert bench.same_segment_tiles(full, seg2, 2) == 3 + 9
