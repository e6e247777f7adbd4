"""Host-side pins of bench.py's algorithmic byte counts (the denominators of every GB/s and roofline
fraction it reports), against the per-workload figures worked out from the record layout:
80,896 B per quantised tile-head (2 x 32 KiB fp16 read, one 15,360 B k4v2 record written),
15,360 B per cached page-head read by decode, 512 B per fp16 tail token-head (K and V rows)."""
import numpy as np

import bench


def test_quantize_bytes_per_tile_head():
    R = 15360
    per = 2 * 128 * 128 * 2 + R
    assert per == 80896
    assert bench.Q_TILES * bench.Q_HKV * per == 331_350_016


def test_decode_bytes_bulk_and_long_context():
    R = 15360
    lens = np.full(32, 16384, np.int64)
    # 32 x 128 pages x 4 kv heads x 15,360 B, plus q and out (32 x 32 heads x 256 B each way)
    assert bench._decode_bytes(lens, 4, 32, R) == 32 * 128 * 4 * R + 32 * 32 * 512 == 252_182_528
    # 4 x 131072 tokens on 1 kv head, 8 query heads
    assert bench._decode_bytes(np.full(4, 131072, np.int64), 1, 8, R) == 4 * 1024 * R + 4 * 8 * 512
    # a tail of t tokens adds t x 512 B per kv head
    assert bench._decode_bytes(np.array([128 + 37]), 2, 4, R) == 2 * R + 37 * 2 * 512 + 4 * 512


def test_append_bytes_with_and_without_a_fill():
    R = 15360
    lens = np.array([5, 127, 300], np.int64)   # the second sequence's append fills a tile
    base = 3 * 4 * 4 * 256 + 3 * 8               # new K/V rows read, tail slots written, lengths
    assert bench._append_bytes(lens, 4, R) == base + 1 * 4 * (2 * 128 * 128 * 2 + R)
    assert bench._append_bytes(np.array([0, 1]), 2, R) == 2 * 2 * 4 * 256 + 2 * 8


def test_bench_refuses_more_than_one_gpu():
    """The method needs no cross-GPU exchange and only one GPU is measured: --gpus 2 exits with a
    message (status 2) before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
