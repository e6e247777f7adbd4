"""Host-side pins of bench.py's algorithmic byte counts (the denominators of every GB/s and roofline
fraction it reports), against the per-workload figures worked out from the record layout:
80,896 B per quantised tile-head (2 x 32 KiB fp16 read, one 15,360 B k4v2 record written),
15,360 B per cached page-head read by decode, 512 B per fp16 tail token-head (K and V rows)."""
import numpy as np
import pytest

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


def test_traffic_from_pmc_csv_scales_by_the_copy_and_adds_the_merge(tmp_path):
    """FETCH/WRITE KiB per dispatch -> bytes per launch: each counter scaled so that the plain copy reads
    the bytes it moves; the decode call is its page kernel plus its merge kernel (B 32 x 16K shape)."""
    import bench
    copy_mib = 4
    q_grid = bench.Q_TILES * bench.Q_HKV * 256
    d_grid = bench.D_B * bench.D_HKV * 256 * 17
    m_grid = bench.D_B * bench.D_HQ * 512
    rows = [("__amd_rocclr_copyBuffer", 1024, 2048.0, 4096.0),       # fetch counts half the copy's bytes
            ("quantize_tiles_kernel<4,2,1>", q_grid, 1000.0, 300.0),
            ("quantize_tiles_kernel<4,2,1>", q_grid, 1200.0, 300.0),
            ("quantize_tiles_kernel<4,2,1>", 4 * q_grid, 9999.0, 9999.0),  # the cache-building launch: ignored
            ("decode_kernel<4,2,8,1>", d_grid, 500.0, 20.0),
            ("decode_kernel<4,2,8,1>", 4 * 1 * 256 * 129, 7777.0, 7777.0),  # the long-context shape
            ("decode_merge_kernel", m_grid, 50.0, 4.0),
            ("decode_merge_kernel", 32 * 512, 8888.0, 8888.0)]
    paths = []
    for name, col in (("FETCH_SIZE", 2), ("WRITE_SIZE", 3)):
        p = tmp_path / f"{name}.csv"
        with open(p, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
            for i, r in enumerate(rows):
                f.write(f"{i},\"{r[0]}\",{r[1]},{name},{r[col]}\n")
        paths.append(str(p))
    out = bench.traffic_from_csv(paths[0], paths[1], copy_mib)
    ff = copy_mib * (1 << 20) / (2048.0 * 1024)
    wf = copy_mib * (1 << 20) / (4096.0 * 1024)
    assert out["factors"] == {"FETCH_SIZE": ff, "WRITE_SIZE": wf}
    assert out["kernels"]["quantize_tiles"] == round(1100.0 * 1024 * ff + 300.0 * 1024 * wf)
    assert out["kernels"]["decode_attention"] == round((500.0 + 50.0) * 1024 * ff + (20.0 + 4.0) * 1024 * wf)


@pytest.mark.gpu
def test_timing_events_bracket_device_work():
    """bench.py's fence-free HIP timing events run on torch's own HIP runtime and stream: an interval
    around a device copy is positive, grows with the work it brackets and stays within the host clock's
    time for the same work."""
    import time

    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    res = []
    for n in (1, 8):
        e0, e1 = bench.TimingEvent(), bench.TimingEvent()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(n):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        ms = e0.elapsed_time(e1)
        assert 0.0 < ms <= host_ms
        res.append(ms)
    assert res[1] > 2 * res[0]
