#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. kvarn_quantize_tiles   bulk quantise 1024 tiles x 4 kv heads (8 sequences x 16384 tokens, the
                            kv-head share of a Qwen3-32B-shaped layer at TP=2), k4v2 g128, pages permuted
  2. kvarn_append_token     one new token for each of 32 sequences x 4 kv heads (fp16 tail; a tail that
                            fills is quantised inline)
  3. kvarn_decode_attention decode for 32 sequences at 16384+ tokens, 32 query / 4 kv heads, over the
                            k4v2 paged cache plus the fp16 tails (two kernels: split-K partials over
                            the pages and the tail, then one merge per (sequence, query head))
Inputs are resident in HBM before the timed region.  Two copies of every input and cache are used
alternately, so each kernel's reads come from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line.  value = algorithmic bytes of the step / step time (GB/s); the per-kernel
numbers (quantize GB/s, decode tokens/s, fractions of the 8 TB/s HBM peak) are in "kernels", with
the decode also timed on its own (back-to-back calls over rotated cache copies), the long-context
serving loop (4 sequences x 128K tokens, 8 query / 1 kv head, append + decode per step, five cache
copies in turn; eager and HIP-graph replay) and the ragged continuous-batching step (64 sequences of
1K-32K tokens, k4v2 and k8v8 pools, append + decode per step), all after the timed steps.

--variants (a separate run, not the step): the same quantise and decode workloads in the grouped
formats k4v2 g64 / g32; chunked prefill (4 sequences, a 512-token chunk on top of 16384 cached
tokens, 32 query / 4 kv heads, k4v2 g128) against the fp16 MFMA peak; and the ragged step again; one
JSON line of its own.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0            # dense fp16 matrix-core peak of MI355X
FORMAT = "kvarn_k4v2_g128"

# workload sizes (see kv_cache_quantization_pipeline_amd/synth.py WORKLOADS)
Q_TILES, Q_HKV = 1024, 4                 # bulk quantise
D_B, D_CTX, D_HQ, D_HKV = 32, 16384, 32, 4  # decode


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=250,
                    help="untimed steps first (the step time settles after ~200 steps, ~45 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="wall seconds per oracle leg (quantise, decode) of the CPU baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for scaling PMC byte counters)")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the step: grouped formats (g64, g32) and chunked prefill, one JSON line")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no benchmark: turn the counter_collection.csv files of two rocprofv3 --pmc runs of "
                         "this script (FETCH_SIZE, then WRITE_SIZE; both with --copy-calibration-mib N) into "
                         "profiles/traffic.json")
    return ap.parse_args()


def source_hash():
    """Hash of the sources of the step's kernels (everything in csrc/ but the prefill kernel)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_quantization_pipeline_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "prefill.hip":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(src_hash):
    """HBM bytes per launch from committed rocprofv3 PMC runs, only if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != src_hash:
        return {}
    return t.get("kernels", {})


def traffic_from_csv(fetch_csv, write_csv, copy_mib):
    """HBM bytes per launch of the two timed kernels from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
    (KiB per dispatch), each scaled by the factor that maps the same counter of a plain copy of
    copy_mib MiB onto the bytes that copy moves."""
    import csv

    def per_dispatch(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = r["Dispatch_Id"]
                rows.setdefault(key, [r["Kernel_Name"], int(r["Grid_Size"]), 0.0])[2] += float(r["Counter_Value"])
        return list(rows.values())

    if copy_mib <= 0:
        raise SystemExit("--traffic-from needs --copy-calibration-mib N (the copy size of the profiled runs)")
    copy_bytes = copy_mib * (1 << 20)
    out = {"source_hash": source_hash(), "unit": "bytes per launch", "copy_calibration_bytes": copy_bytes,
           "kernels": {}, "factors": {}}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, counter)
        copies = [v for name, grid, v in rows if "copyBuffer" in name]
        if not copies:
            raise SystemExit(f"{path}: no copy kernel dispatch to calibrate against")
        factor = copy_bytes / (max(copies) * 1024.0)
        out["factors"][counter] = factor
        q_grid = Q_TILES * Q_HKV * 256
        quant = [v for name, grid, v in rows if "quantize_tiles_kernel" in name and grid == q_grid]
        # the step's decode call: the page kernel (grid: B x Hkv workgroups of 256 per split) and the merge
        # kernel (B x Hq workgroups of 512) of the B 32 x 16K shape
        per_split = D_B * D_HKV * 256
        dec = [v for name, grid, v in rows if "decode_kernel" in name and grid % per_split == 0 and grid > per_split]
        mrg = [v for name, grid, v in rows if "decode_merge_kernel" in name and grid == D_B * D_HQ * 512]
        if not quant or not dec or not mrg:
            raise SystemExit(f"{path}: missing quantize/decode dispatches")
        per.setdefault("quantize_tiles", 0.0)
        per["quantize_tiles"] += sum(quant) / len(quant) * 1024.0 * factor
        per.setdefault("decode_attention", 0.0)
        per["decode_attention"] += (sum(dec) / len(dec) + sum(mrg) / len(mrg)) * 1024.0 * factor
    out["kernels"] = {k: int(round(v)) for k, v in per.items()}
    return out


def write_traffic(fetch_csv, write_csv, copy_mib):
    out = traffic_from_csv(fetch_csv, write_csv, copy_mib)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model / stepping numbers (a
    virtualised host may name only the vendor's product line)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                k, _, v = line.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(k1, v1, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload: whole sequences of the
    bulk-quantise batch, then decode steps over oracle-quantised sequences of the decode shape."""
    import numpy as np

    import oracle
    from kv_cache_quantization_pipeline_amd import synth

    threads = oracle.threads_used(0)
    R = oracle.record_bytes(4, 2)
    # quantise leg: one sequence (128 tiles x 4 heads) at a time until `seconds` have passed
    q_bytes, q_time, q_seqs = 0, 0.0, 0
    kt = k1.reshape(-1, 128, Q_HKV, 128)
    vt = v1.reshape(-1, 128, Q_HKV, 128)
    cache = np.zeros(128 * Q_HKV * R, np.uint8)
    pages = np.arange(128, dtype=np.int32)
    while q_time < seconds and q_seqs < kt.shape[0] // 128:
        s0 = q_seqs * 128
        t0 = time.perf_counter()
        oracle.quantize_tiles(4, 2, 8, kt[s0:s0 + 128].view(np.uint16), vt[s0:s0 + 128].view(np.uint16), pages,
                              cache, Q_HKV * R, nthreads=threads)
        q_time += time.perf_counter() - t0
        q_bytes += 128 * Q_HKV * (2 * 128 * 128 * 2 + R)
        q_seqs += 1
    # decode leg: the sequence just quantised, decoded with 32 query heads, repeated until `seconds`
    q = synth.gen_q(2, 1, D_HQ)
    pt = pages[None, :]
    lens = np.array([128 * 128], np.int32)
    tail = np.zeros((1, Q_HKV, 128, 128), np.uint16)
    d_bytes, d_time, d_calls = 0, 0.0, 0
    while d_time < seconds:
        t0 = time.perf_counter()
        oracle.decode_attention(4, 2, q.view(np.uint16), cache, Q_HKV * R, pt, lens, tail, tail,
                                1 / math.sqrt(128), Q_HKV, nthreads=threads)
        d_time += time.perf_counter() - t0
        d_bytes += 128 * Q_HKV * R + 2 * D_HQ * 256
        d_calls += 1
    rate = (q_bytes + d_bytes) / (q_time + d_time) / 1e9
    # single-thread runs: the single-tile workload (1 kv head, 128 tokens, seed 0) and a 64-tile subset
    # of the bulk batch (64 tiles x 4 kv heads)
    k0, v0 = synth.gen_kv(0, 128, 1)
    c0 = np.zeros(R, np.uint8)
    t0 = time.perf_counter()
    oracle.quantize_tiles(4, 2, 8, synth.tiles_view(k0).view(np.uint16), synth.tiles_view(v0).view(np.uint16),
                          np.zeros(1, np.int32), c0, R, nthreads=1)
    t_single = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.quantize_tiles(4, 2, 8, np.ascontiguousarray(kt[:64]).view(np.uint16),
                          np.ascontiguousarray(vt[:64]).view(np.uint16), pages[:64], cache, Q_HKV * R, nthreads=1)
    t_sub = time.perf_counter() - t0
    sub_bytes = 64 * Q_HKV * (2 * 128 * 128 * 2 + R)
    return {"value": rate, "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": _cpu_model(),
            "single_thread": {"single_tile_quantize_ms": t_single * 1e3,
                              "bulk_64_tiles_quantize_s": t_sub, "bulk_64_tiles_quantize_GBps": sub_bytes / t_sub / 1e9},
            "sample": (f"{q_seqs} sequence(s) of 128 tiles x 4 kv heads quantised ({q_bytes / 1e6:.1f} MB, "
                       f"{q_time:.1f} s) + {d_calls} decode call(s) of 1 sequence x 16384 tokens x 32 query "
                       f"heads ({d_bytes / 1e6:.1f} MB, {d_time:.1f} s); fp64 oracle, {threads} threads"),
            "quantize_GBps": q_bytes / q_time / 1e9, "decode_tokens_per_s": d_calls / d_time}


# hipEventDisableSystemFence (hip_runtime_api.h): recording the event performs no system-scope fence
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP event used only for timing, with the two calls of torch.cuda.Event that this script uses
    (record() on the current stream, elapsed_time(end) in ms).  It is created with
    hipEventDisableSystemFence, so that recording it does not write back and invalidate the caches at
    system scope: in a rocprofv3 kernel trace an ordinary event between two launches leaves 5.6-5.8 us
    between them, this one 4.3-4.5 us (the marker packet's own processing), and an interval between two
    events spans about that much more than the launches it brackets.  Elapsed times are read after a
    device synchronisation.  The HIP runtime is the one already loaded by torch (found in this
    process's mappings), so the events and torch's streams belong to one runtime."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import torch
            torch.cuda.init()
            paths = set()
            with open("/proc/self/maps") as f:
                for line in f:
                    parts = line.split()
                    if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64.so"):
                        paths.add(os.path.realpath(parts[5]))
            if len(paths) != 1:
                raise RuntimeError(f"expected one loaded HIP runtime, found {sorted(paths)}")
            hip = ctypes.CDLL(paths.pop())
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for fn in (hip.hipEventCreateWithFlags, hip.hipEventRecord, hip.hipEventElapsedTime, hip.hipEventDestroy):
                fn.restype = ctypes.c_int
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self._h = ctypes.c_void_p()
        st = self._runtime().hipEventCreateWithFlags(ctypes.byref(self._h), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        import torch
        st = self._hip.hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        st = self._hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        try:
            if self._hip is not None and self._h:
                self._hip.hipEventDestroy(self._h)
        except Exception:
            pass


def _blocks_time(fn, per_block, blocks, warmup):
    """Median over `blocks` blocks of the mean time per call of `per_block` back-to-back calls, each
    block bracketed by one pair of HIP events on the launch stream (no event between the calls)."""
    import numpy as np
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(2)] for _ in range(blocks)]
    for b in range(blocks):
        ev[b][0].record()
        for i in range(per_block):
            fn(warmup + b * per_block + i)
        ev[b][1].record()
    torch.cuda.synchronize()
    return float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3 / per_block


def _events_time(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = TimingEvent()
    e1 = TimingEvent()
    e0.record()
    for i in range(steps):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def variants(args):
    """Grouped formats and chunked prefill, timed with HIP events on the launch stream."""
    import numpy as np
    import torch

    import kv_cache_quantization_pipeline_amd as kv
    from kv_cache_quantization_pipeline_amd import synth

    dev = torch.device("cuda:0")
    out = {"variants": "grouped formats and chunked prefill", "steps": args.steps, "warmup": args.warmup,
           "data": "synthetic", "results": {}}
    res = out["results"]
    # quantise: the bulk workload, two copies of the inputs
    w1 = synth.WORKLOADS["bulk_quantize_qwen3_32b_tp2"]
    k1, v1 = synth.gen_kv(w1["seed"], w1["batch"] * w1["ctx"], w1["n_kv_heads"])
    kd = [torch.from_numpy(synth.tiles_view(k1)).to(dev)]
    vd = [torch.from_numpy(synth.tiles_view(v1)).to(dev)]
    kd.append(kd[0].clone())
    vd.append(vd[0].clone())
    del k1, v1
    pages = torch.from_numpy(synth.gen_page_perm(w1["seed"], Q_TILES)).to(dev)
    for name in ("kvarn_k4v2_g64", "kvarn_k4v2_g32"):
        fmt = kv.format_parse(name)
        R = kv.record_bytes(fmt)
        caches = [torch.zeros(Q_TILES * Q_HKV * R, dtype=torch.uint8, device=dev) for _ in range(2)]
        t = _events_time(lambda i: kv.quantize_tiles(fmt, kd[i % 2], vd[i % 2], pages, caches[i % 2], Q_HKV * R),
                         args.steps, args.warmup)
        b = Q_TILES * Q_HKV * (2 * 128 * 128 * 2 + R)
        res[f"quantize_tiles {name}"] = {"us": t * 1e6, "bytes": b, "GBps": b / t / 1e9,
                                         "frac_hbm": b / t / 1e9 / HBM_PEAK_GBPS}
        del caches
    del kd, vd

    # decode: batch 32 x 16384 tokens, 32 query / 4 kv heads, two cache copies
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    pps = D_CTX // 128
    maxp = pps + 1
    n_pool = D_B * maxp
    pt = torch.from_numpy(np.ascontiguousarray(synth.gen_page_perm(2, n_pool).reshape(D_B, maxp))).to(dev)
    lens = torch.full((D_B,), D_CTX, dtype=torch.int32, device=dev)
    tk = torch.zeros(D_B, D_HKV, 128, 128, dtype=torch.float16, device=dev)
    tv = torch.zeros_like(tk)
    q = torch.from_numpy(synth.gen_q(2, D_B, D_HQ)).to(dev)
    o = torch.empty_like(q)
    sm = 1.0 / math.sqrt(128)
    for name in ("kvarn_k4v2_g64", "kvarn_k4v2_g32"):
        fmt = kv.format_parse(name)
        R = kv.record_bytes(fmt)
        caches = []
        for _ in range(2):
            c = torch.zeros(n_pool * D_HKV * R, dtype=torch.uint8, device=dev)
            for s0 in range(0, D_B, 8):
                kk = torch.randn(8 * pps, 128, D_HKV, 128, generator=g, device=dev).half()
                vv = torch.randn(8 * pps, 128, D_HKV, 128, generator=g, device=dev).half()
                kv.quantize_tiles(fmt, kk, vv, pt[s0:s0 + 8, :pps].reshape(-1).contiguous(), c, D_HKV * R)
            caches.append(c)
        ws = kv.decode_workspace(fmt, D_B, D_HQ, D_HKV, maxp, dev)
        t = _events_time(lambda i: kv.decode_attention(fmt, q, caches[i % 2], D_HKV * R, pt, lens, tk, tv, sm, o, ws,
                                                       D_HKV), args.steps, args.warmup)
        b = D_B * pps * D_HKV * R + D_B * D_HQ * 256 * 2
        res[f"decode_attention {name}"] = {"us": t * 1e6, "bytes": b, "GBps": b / t / 1e9,
                                           "frac_hbm": b / t / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": D_B / t}
        del caches

    # chunked prefill: 4 sequences, 16384 cached tokens + a 512-token chunk (its keys appended), k4v2 g128
    P_B, P_CTX, P_Q = 4, 16384, 512
    fmt = kv.format_parse(FORMAT)
    R = kv.record_bytes(fmt)
    L = P_CTX + P_Q
    full = L // 128
    n_pool = P_B * (full + 1)
    ptp = torch.from_numpy(np.ascontiguousarray(synth.gen_page_perm(5, n_pool).reshape(P_B, full + 1))).to(dev)
    cache = torch.zeros(n_pool * D_HKV * R, dtype=torch.uint8, device=dev)
    for s0 in range(P_B):
        kk = torch.randn(full, 128, D_HKV, 128, generator=g, device=dev).half()
        vv = torch.randn(full, 128, D_HKV, 128, generator=g, device=dev).half()
        kv.quantize_tiles(fmt, kk, vv, ptp[s0, :full].contiguous(), cache, D_HKV * R)
    plens = torch.full((P_B,), L, dtype=torch.int32, device=dev)
    qlens = torch.full((P_B,), P_Q, dtype=torch.int32, device=dev)
    ptk = torch.zeros(P_B, D_HKV, 128, 128, dtype=torch.float16, device=dev)
    ptv = torch.zeros_like(ptk)
    pq = torch.randn(P_B, P_Q, D_HQ, 128, generator=g, device=dev).half()
    po = torch.empty_like(pq)
    t = _events_time(lambda i: kv.prefill_attention(fmt, pq, qlens, cache, D_HKV * R, ptp, plens, ptk, ptv, sm, po,
                                                    D_HKV), args.steps, args.warmup)
    pairs = P_B * D_HQ * (P_Q * (L - P_Q) + P_Q * (P_Q + 1) // 2)   # (query, visible key) pairs
    flops = 4 * 128 * pairs                                          # QK and PV multiply-adds
    res["prefill_attention kvarn_k4v2_g128"] = {
        "us": t * 1e6, "workload": f"{P_B} seqs x ({P_CTX} cached + {P_Q}-token chunk), {D_HQ} q / {D_HKV} kv heads",
        "flops": flops, "TFLOPs": flops / t / 1e12, "frac_mfma_f16": flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "query_tokens_per_s": P_B * P_Q / t}
    del cache, ptk, ptv, pq, po
    res["decode_step ragged_mixed"] = ragged_mixed_steps(kv, synth, dev, args.steps)
    print(json.dumps(out), flush=True)


def _append_bytes(lens_before, n_kv_heads, R):
    """Algorithmic bytes of one append call: new K/V rows read, tail slots written, lengths read and
    written; a tile that fills is read (K and V, 128 x 128 fp16) and its record written."""
    n = len(lens_before)
    fills = int(((lens_before + 1) % 128 == 0).sum())
    return n * n_kv_heads * 4 * 256 + n * 8 + fills * n_kv_heads * (2 * 128 * 128 * 2 + R)


def _decode_bytes(lens, n_kv_heads, n_q_heads, R):
    """Algorithmic bytes of one decode call: full pages, fp16 tails (K and V rows), queries and outputs."""
    return int((lens // 128 * n_kv_heads * R).sum() + (lens % 128 * n_kv_heads * 512).sum()
               + len(lens) * n_q_heads * 256 * 2)


def long_context_steps(kv, synth, dev):
    """4 sequences x 131072 tokens, 8 query heads on 1 kv head, k4v2: 128 steps of append one token +
    decode per copy (the last append of each copy fills the tail and quantises it inline).  The cache
    is 63 MB, so five independent copies (315 MB) are used in turn and every read comes from HBM,
    not from the 256 MB Infinity Cache.  The calls are prepared (marshalled once), so that the host keeps
    ahead of the GPU.  Timed three ways: the eager loop by the host clock with no event between the
    launches; the same loop with events around every call (the append / decode split); and the steps
    captured as one HIP graph per copy, timed by replay.  The decode alone is also timed back-to-back
    over the copies."""
    import numpy as np
    import torch
    w = synth.WORKLOADS["decode_long_b4_ctx128k"]
    fmt = kv.format_parse(FORMAT)
    R = kv.record_bytes(fmt)
    B, hq, hkv, ctx = w["batch"], w["n_q_heads"], w["n_kv_heads"], w["ctx"]
    full, n_copies, n_steps = ctx // 128, 5, 128
    maxp = full + 1
    stride = hkv * R
    pt = torch.from_numpy(synth.gen_page_perm(w["seed"], B * maxp).reshape(B, maxp)).to(dev)
    dst = pt[:, :full].reshape(-1).contiguous()
    k, v = synth.gen_kv(w["seed"], B * full * 128, hkv)
    kd, vd = torch.from_numpy(synth.tiles_view(k)).to(dev), torch.from_numpy(synth.tiles_view(v)).to(dev)
    del k, v
    caches = []
    for _ in range(n_copies):
        c = torch.zeros(B * maxp * stride, dtype=torch.uint8, device=dev)
        kv.quantize_tiles(fmt, kd, vd, dst, c, stride)
        caches.append(c)
    del kd, vd
    rng = np.random.default_rng(w["seed"] + 7)
    knew = torch.from_numpy((rng.standard_normal((n_steps, B, hkv, 128)) * 1.5).astype(np.float16)).to(dev)
    vnew = torch.from_numpy((rng.standard_normal((n_steps, B, hkv, 128)) * 1.5).astype(np.float16)).to(dev)
    q = torch.from_numpy(synth.gen_q(w["seed"], B, hq)).to(dev)
    out = torch.empty(B, hq, 128, dtype=torch.float16, device=dev)
    lens = [torch.full((B,), ctx, dtype=torch.int32, device=dev) for _ in range(n_copies)]
    tails = [(torch.zeros(B, hkv, 128, 128, dtype=torch.float16, device=dev),
              torch.zeros(B, hkv, 128, 128, dtype=torch.float16, device=dev)) for _ in range(n_copies)]
    ws = kv.decode_workspace(fmt, B, hq, hkv, maxp, dev)
    sm = 1.0 / math.sqrt(128)

    # the calls marshalled once (the GPU work per call is a few microseconds, so the host must not
    # fall behind), and the events created beforehand
    apps = [[kv.prepare_append_token(fmt, knew[s], vnew[s], lens[c], tails[c][0], tails[c][1], pt, caches[c], stride)
             for c in range(n_copies)] for s in range(n_steps)]
    decs = [kv.prepare_decode_attention(fmt, q, caches[c], stride, pt, lens[c], tails[c][0], tails[c][1], sm, out, ws,
                                        hkv) for c in range(n_copies)]
    events = [[TimingEvent() for _ in range(3)] for _ in range(n_steps * n_copies)]

    def run(steps, record):
        ev = []
        for s in range(steps):
            for c in range(n_copies):
                e = events[s * n_copies + c]
                if record:
                    e[0].record()
                apps[s][c]()
                if record:
                    e[1].record()
                decs[c]()
                if record:
                    e[2].record()
                    ev.append(e)
        return ev

    def reset():
        torch.cuda.synchronize(dev)
        for c in range(n_copies):
            lens[c].fill_(ctx)
            tails[c][0].zero_()
            tails[c][1].zero_()
        torch.cuda.synchronize(dev)

    run(4, False)                                  # warm-up, then back to the starting state
    reset()
    # eager, no events between the launches: the step time by the host clock
    t0 = time.perf_counter()
    run(n_steps, False)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    assert lens[0].cpu().tolist() == [ctx + n_steps] * B
    n = n_steps * n_copies
    # the instrumented pass (events around every call): the append / decode split within the loop
    reset()
    ev = run(n_steps, True)
    torch.cuda.synchronize(dev)
    ta = sum(e[0].elapsed_time(e[1]) for e in ev) / n * 1e-3
    td_in = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    # decode alone, back-to-back over the five copies at 64 tail tokens (the loop's mean tail length)
    for c in range(n_copies):
        lens[c].fill_(ctx + 64)
    td_med = _blocks_time(lambda i: decs[i % n_copies](), 4 * n_copies, 5, n_copies)
    lb64 = np.full(B, ctx + 64, np.int64)
    b_dec64 = _decode_bytes(lb64, hkv, hq, R)
    b_app = b_dec = 0
    for s in range(n_steps):
        lb = np.full(B, ctx + s, np.int64)
        b_app += _append_bytes(lb, hkv, R)
        b_dec += _decode_bytes(lb + 1, hkv, hq, R)
    b_app, b_dec = b_app / n_steps, b_dec / n_steps
    step = elapsed / n

    # the same 128 steps per copy captured once as a HIP graph (append + decode, 256 launches) and
    # replayed, each copy reset to its starting state first; timed with events around each replay
    reset()
    graphs = []
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    for c in range(n_copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for s in range(n_steps):
                kv.append_token(fmt, knew[s], vnew[s], lens[c], tails[c][0], tails[c][1], pt, caches[c], stride)
                kv.decode_attention(fmt, q, caches[c], stride, pt, lens[c], tails[c][0], tails[c][1], sm, out, ws,
                                    hkv)
        graphs.append(g)
    torch.cuda.current_stream(dev).wait_stream(side)
    ge = [[TimingEvent() for _ in range(2)] for _ in range(n_copies)]
    reset()
    for c in range(n_copies):
        ge[c][0].record()
        graphs[c].replay()
        ge[c][1].record()
    torch.cuda.synchronize(dev)
    assert lens[0].cpu().tolist() == [ctx + n_steps] * B
    g_step = sum(e[0].elapsed_time(e[1]) for e in ge) * 1e-3 / (n_copies * n_steps)
    del graphs
    return {"workload": f"{B} seqs x {ctx}+ tokens, {hq} q / {hkv} kv heads, {FORMAT}, {n_steps} append + decode "
                        f"steps on each of {n_copies} cache copies (one tail fill per sequence per copy)",
            "us_per_step": step * 1e6, "tokens_per_s": B / step, "step_GBps": (b_app + b_dec) / step / 1e9,
            "step_frac_hbm": (b_app + b_dec) / step / 1e9 / HBM_PEAK_GBPS,
            "graph_us_per_step": g_step * 1e6, "graph_tokens_per_s": B / g_step,
            "graph_step_frac_hbm": (b_app + b_dec) / g_step / 1e9 / HBM_PEAK_GBPS,
            "decode_us": td_med * 1e6, "decode_bytes": b_dec64,
            "decode_GBps": b_dec64 / td_med / 1e9, "decode_frac_hbm": b_dec64 / td_med / 1e9 / HBM_PEAK_GBPS,
            "decode_tokens_per_s": B / td_med,
            "decode_note": ("decode alone at 131072 + 64 tokens, back-to-back over the five copies; median over "
                            "5 blocks of 20 calls of the mean per call"),
            "instrumented": {"append_us": ta * 1e6, "decode_us_median": td_in * 1e6, "append_bytes": b_app,
                             "decode_bytes": b_dec,
                             "note": "the loop again with events around every call (each event adds idle time)"}}


def ragged_mixed_steps(kv, synth, dev, steps):
    """64 sequences with lengths uniform in [1024, 32768], 32 query / 4 kv heads, each sequence k4v2 or
    k8v8 (one pool and one append + decode call per format).  Each step appends one token to every
    sequence (tiles that fill are quantised inline) and decodes; the step reads ~0.9 GB, well past the
    Infinity Cache.  Full pages are quantised beforehand from fp16 K/V ~ N(0, 1.5^2) drawn on the device
    (the kernels' time does not depend on the values)."""
    import numpy as np
    import torch
    w = synth.WORKLOADS["ragged_mixed_64seq"]
    B, hq, hkv = w["batch"], w["n_q_heads"], w["n_kv_heads"]
    lens0 = synth.gen_lengths(w["seed"], B, w["ctx_lo"], w["ctx_hi"]).astype(np.int64)
    fmts = synth.gen_formats(w["seed"], B)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w["seed"])
    q_all = synth.gen_q(w["seed"], B, hq)
    rng = np.random.default_rng(w["seed"] + 7)
    sm = 1.0 / math.sqrt(128)
    n_steps = max(1, min(steps, 100))
    pools = []
    for fi, name in enumerate(("kvarn_k4v2_g128", "kvarn_k8v8_g128")):
        idx = np.nonzero(fmts == fi)[0]
        if len(idx) == 0:
            continue
        fmt = kv.format_parse(name)
        R = kv.record_bytes(fmt)
        stride = hkv * R
        lens = lens0[idx]
        full = lens // 128
        maxp = int(full.max()) + 2
        n = len(idx)
        pt_h = synth.gen_page_perm(w["seed"] + fi, n * maxp).reshape(n, maxp)
        cache = torch.zeros(n * maxp * stride, dtype=torch.uint8, device=dev)
        dst = np.concatenate([pt_h[i, :full[i]] for i in range(n)]).astype(np.int32)
        for c0 in range(0, len(dst), 2048):
            m = min(2048, len(dst) - c0)
            kt = (torch.randn(m, 128, hkv, 128, generator=gen, device=dev) * 1.5).half()
            vt = (torch.randn(m, 128, hkv, 128, generator=gen, device=dev) * 1.5).half()
            kv.quantize_tiles(fmt, kt, vt, torch.from_numpy(dst[c0:c0 + m]).to(dev), cache, stride)
        tk = (torch.randn(n, hkv, 128, 128, generator=gen, device=dev) * 1.5).half()
        tv = (torch.randn(n, hkv, 128, 128, generator=gen, device=dev) * 1.5).half()
        knew = torch.from_numpy((rng.standard_normal((n_steps, n, hkv, 128)) * 1.5).astype(np.float16)).to(dev)
        vnew = torch.from_numpy((rng.standard_normal((n_steps, n, hkv, 128)) * 1.5).astype(np.float16)).to(dev)
        pools.append(dict(name=name, fmt=fmt, R=R, stride=stride, lens0=lens.copy(), cache=cache, tk=tk, tv=tv,
                          pt=torch.from_numpy(np.ascontiguousarray(pt_h)).to(dev), knew=knew, vnew=vnew,
                          lens=torch.from_numpy(lens.astype(np.int32)).to(dev),
                          q=torch.from_numpy(q_all[idx]).to(dev),
                          out=torch.empty(n, hq, 128, dtype=torch.float16, device=dev),
                          ws=kv.decode_workspace(fmt, n, hq, hkv, maxp, dev)))

    for p in pools:
        p["apps"] = [kv.prepare_append_token(p["fmt"], p["knew"][s], p["vnew"][s], p["lens"], p["tk"], p["tv"],
                                             p["pt"], p["cache"], p["stride"]) for s in range(n_steps)]
        p["dec"] = kv.prepare_decode_attention(p["fmt"], p["q"], p["cache"], p["stride"], p["pt"], p["lens"], p["tk"],
                                               p["tv"], sm, p["out"], p["ws"], hkv)

    def run(nst):
        for s in range(nst):
            for p in pools:
                p["apps"][s]()
                p["dec"]()

    run(1)                                         # warm-up, then back to the starting lengths
    torch.cuda.synchronize(dev)
    for p in pools:
        p["lens"].copy_(torch.from_numpy(p["lens0"].astype(np.int32)))
    torch.cuda.synchronize(dev)
    e0 = TimingEvent()
    e1 = TimingEvent()
    e0.record()
    run(n_steps)
    e1.record()
    torch.cuda.synchronize(dev)
    step = e0.elapsed_time(e1) * 1e-3 / n_steps
    total = fills = 0
    for p in pools:
        assert np.array_equal(p["lens"].cpu().numpy(), p["lens0"] + n_steps)
        for s in range(n_steps):
            lb = p["lens0"] + s
            total += _append_bytes(lb, hkv, p["R"]) + _decode_bytes(lb + 1, hkv, hq, p["R"])
            fills += int(((lb + 1) % 128 == 0).sum())
    per_step = total / n_steps
    return {"workload": (f"{B} seqs, lengths U[{w['ctx_lo']}, {w['ctx_hi']}] (seeded), {hq} q / {hkv} kv heads, "
                         f"formats " + " / ".join(f"{p['name']} x {len(p['lens0'])}" for p in pools)
                         + f", {n_steps} append + decode steps"),
            "us_per_step": step * 1e6, "bytes_per_step": per_step, "GBps": per_step / step / 1e9,
            "frac_hbm": per_step / step / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": B / step,
            "tile_fills": fills}


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.copy_calibration_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU; the method needs no cross-GPU exchange "
              "(kv heads and sequences shard independently), so runs with --gpus > 1 are not provided.",
              file=sys.stderr)
        sys.exit(2)
    if args.variants:
        variants(args)
        return

    import numpy as np
    import torch

    import kv_cache_quantization_pipeline_amd as kv
    from kv_cache_quantization_pipeline_amd import synth

    dev = torch.device("cuda:0")
    fmt = kv.format_parse(FORMAT)
    R = kv.record_bytes(fmt)
    t_prep = time.perf_counter()

    # ---- bulk quantise inputs (two copies) -------------------------------------------------
    w1 = synth.WORKLOADS["bulk_quantize_qwen3_32b_tp2"]
    k1, v1 = synth.gen_kv(w1["seed"], w1["batch"] * w1["ctx"], w1["n_kv_heads"])
    pages1 = torch.from_numpy(synth.gen_page_perm(w1["seed"], Q_TILES)).to(dev)
    k1d = [torch.from_numpy(synth.tiles_view(k1)).to(dev)]
    v1d = [torch.from_numpy(synth.tiles_view(v1)).to(dev)]
    k1d.append(k1d[0].clone())
    v1d.append(v1d[0].clone())
    stride1 = Q_HKV * R
    cache1 = [torch.zeros(Q_TILES * stride1, dtype=torch.uint8, device=dev) for _ in range(2)]

    # ---- decode cache: quantise the decode workload's K/V once (untimed), two copies ----------
    w2 = synth.WORKLOADS["decode_gqa8_b32_ctx16k"]
    pages_per_seq = D_CTX // 128
    # pages for tails that fill during the run: each copy takes (warmup + 2 steps + 1) // 2 appends
    # (the timed steps and the instrumented pass after them)
    extra = -(-((args.warmup + 2 * args.steps + 1) // 2) // 128) + 1
    max_pages = pages_per_seq + extra
    n_pool = D_B * max_pages
    perm2 = synth.gen_page_perm(w2["seed"], n_pool).reshape(D_B, max_pages)
    pt2 = torch.from_numpy(np.ascontiguousarray(perm2)).to(dev)
    stride2 = D_HKV * R
    k2, v2 = synth.gen_kv(w2["seed"], D_B * D_CTX, D_HKV)
    k2d = torch.from_numpy(synth.tiles_view(k2)).to(dev)
    v2d = torch.from_numpy(synth.tiles_view(v2)).to(dev)
    del k2, v2
    dst2 = torch.from_numpy(np.ascontiguousarray(perm2[:, :pages_per_seq]).reshape(-1)).to(dev)
    cache2 = []
    for _ in range(2):
        c = torch.zeros(n_pool * stride2, dtype=torch.uint8, device=dev)
        kv.quantize_tiles(fmt, k2d, v2d, dst2, c, stride2)
        cache2.append(c)
    del k2d, v2d
    rng = np.random.default_rng(w2["seed"] + 7)
    knew = torch.from_numpy((rng.standard_normal((D_B, D_HKV, 128)) * 1.5).astype(np.float16)).to(dev)
    vnew = torch.from_numpy((rng.standard_normal((D_B, D_HKV, 128)) * 1.5).astype(np.float16)).to(dev)
    lens2 = [torch.full((D_B,), D_CTX, dtype=torch.int32, device=dev) for _ in range(2)]
    tails = [(torch.zeros(D_B, D_HKV, 128, 128, dtype=torch.float16, device=dev),
              torch.zeros(D_B, D_HKV, 128, 128, dtype=torch.float16, device=dev)) for _ in range(2)]
    q2 = torch.from_numpy(synth.gen_q(w2["seed"], D_B, D_HQ)).to(dev)
    out2 = torch.empty(D_B, D_HQ, 128, dtype=torch.float16, device=dev)
    ws2 = kv.decode_workspace(fmt, D_B, D_HQ, D_HKV, max_pages, dev)
    sm = 1.0 / math.sqrt(128)
    torch.cuda.synchronize(dev)
    prep_s = time.perf_counter() - t_prep

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    # host-side mirror of the decode lengths, for the algorithmic byte count of each step
    host_lens = [np.full(D_B, D_CTX, np.int64) for _ in range(2)]

    def decode_bytes(lens):
        return _decode_bytes(lens, D_HKV, D_HQ, R)

    def append_bytes(lens_before):
        return _append_bytes(lens_before, D_HKV, R)

    quant_bytes = Q_TILES * Q_HKV * (2 * 128 * 128 * 2 + R)

    # events: None, "quantize" (around the quantise launch only) or "all" (between every launch).
    # Each event recorded between two launches leaves the GPU idle for a few microseconds, so only every
    # fifth timed step carries events, the two around the dominant kernel; the append / decode split
    # comes from an instrumented pass of the same step after the timed ones.
    def step(i, events, ev):
        c = i % 2
        e = [TimingEvent() for _ in range(4 if events == "all" else 2)] if events else None
        if events:
            e[0].record()
        kv.quantize_tiles(fmt, k1d[c], v1d[c], pages1, cache1[c], stride1)
        if events:
            e[1].record()
        kv.append_token(fmt, knew, vnew, lens2[c], tails[c][0], tails[c][1], pt2, cache2[c], stride2)
        if events == "all":
            e[2].record()
        kv.decode_attention(fmt, q2, cache2[c], stride2, pt2, lens2[c], tails[c][0], tails[c][1], sm, out2, ws2,
                            D_HKV)
        if events == "all":
            e[3].record()
        if events:
            ev.append(e)
        b_app = append_bytes(host_lens[c])
        host_lens[c] += 1
        return b_app, decode_bytes(host_lens[c])

    for i in range(args.warmup):
        step(i, None, None)
    torch.cuda.synchronize(dev)
    bytes_app = bytes_dec = 0
    ev_q = []
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        # the quantise of every fifth timed step between two events (each event idles the GPU ~4 us)
        ba, bd = step(i, "quantize" if (i - args.warmup) % 5 == 0 else None, ev_q)
        bytes_app += ba
        bytes_dec += bd
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    assert torch.isfinite(out2.float()).all().item()

    # the instrumented pass: the same steps with events between all launches (append / decode split)
    ev = []
    br_app = br_dec = 0
    t0 = time.perf_counter()
    for i in range(args.warmup + args.steps, args.warmup + 2 * args.steps):
        ba, bd = step(i, "all", ev)
        br_app += ba
        br_dec += bd
    torch.cuda.synchronize(dev)
    elapsed_br = time.perf_counter() - t0

    # isolated decode (the decode workload alone: batch 32 x 16384 tokens, no tail): back-to-back calls
    # on the two cache copies in turn, each bracketed by events on the launch stream; median per call
    for c in range(2):
        lens2[c].fill_(D_CTX)
    dec_calls = [kv.prepare_decode_attention(fmt, q2, cache2[c], stride2, pt2, lens2[c], tails[c][0], tails[c][1], sm,
                                             out2, ws2, D_HKV) for c in range(2)]
    t_iso = _blocks_time(lambda i: dec_calls[i % 2](), 8, 5, 4)
    iso_bytes = decode_bytes(np.full(D_B, D_CTX, np.int64))
    del dec_calls

    # the long-context serving loop (4 sequences x 128K tokens, 8 query heads on 1 kv head)
    long_ctx = long_context_steps(kv, synth, dev)
    # the ragged continuous-batching step (64 sequences of 1K-32K tokens in a k4v2 and a k8v8 pool)
    ragged = ragged_mixed_steps(kv, synth, dev, args.steps)

    # the "achievable" line: a plain device-to-device copy that moves as many bytes (read + write) as
    # one bulk quantise, two copies alternated like the step's inputs (outside the timed step)
    n_copy = quant_bytes // 2 // 256 * 256
    csrc = [torch.empty(n_copy, dtype=torch.uint8, device=dev).fill_(1) for _ in range(2)]
    cdst = [torch.empty_like(s) for s in csrc]
    t_copy = _events_time(lambda i: cdst[i % 2].copy_(csrc[i % 2]), 20, 3)
    del csrc, cdst

    tq = sum(e[0].elapsed_time(e[1]) for e in ev_q) / len(ev_q) * 1e-3
    ta = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev) * 1e-3
    td = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev) * 1e-3
    med = [float(np.median([e[0].elapsed_time(e[1]) for e in ev_q])) * 1e3] + \
          [float(np.median([e[i].elapsed_time(e[i + 1]) for e in ev])) * 1e3 for i in (1, 2)]
    step_s = elapsed / args.steps
    total_bytes = quant_bytes * args.steps + bytes_app + bytes_dec
    value = total_bytes / elapsed / 1e9
    dec_b = br_dec / args.steps
    app_b = br_app / args.steps
    instrumented_step_us = elapsed_br / args.steps * 1e6

    src_hash = source_hash()
    traffic = load_traffic(src_hash)
    kernels = {
        "quantize_tiles": {"GBps": quant_bytes / tq / 1e9, "frac_hbm": quant_bytes / tq / 1e9 / HBM_PEAK_GBPS,
                           "us": tq * 1e6, "us_median": med[0], "bytes": quant_bytes, "tile_heads": Q_TILES * Q_HKV},
        "append_token": {"us": ta * 1e6, "us_median": med[1], "bytes": app_b, "GBps": app_b / ta / 1e9,
                         "note": "from the instrumented pass of the step"},
        "decode_attention": {"GBps": dec_b / td / 1e9, "frac_hbm": dec_b / td / 1e9 / HBM_PEAK_GBPS,
                             "us": td * 1e6, "us_median": med[2], "bytes": dec_b, "tokens_per_s": D_B / td,
                             "note": ("page kernel (split-K partials) + merge kernel; one layer call, 1 token per "
                                      "sequence; from the instrumented pass of the step")},
        "step_instrumented": {"us_per_step": instrumented_step_us,
                              "note": ("the same steps with events between all launches, after the timed ones "
                                       "(the timed steps record events around the quantise only)")},
        "decode_attention_isolated": {
            "us_median": t_iso * 1e6, "bytes": iso_bytes, "GBps": iso_bytes / t_iso / 1e9,
            "frac_hbm": iso_bytes / t_iso / 1e9 / HBM_PEAK_GBPS, "tokens_per_s": D_B / t_iso,
            "note": ("decode alone: batch 32 x 16384 tokens (no tail), 32 q / 4 kv heads, k4v2; back-to-back calls "
                     "on two cache copies (page kernel + merge kernel), median over 5 blocks of 8 calls of the "
                     "mean per call")},
        "decode_long_context": long_ctx,
        "decode_step_ragged_mixed": ragged,
        "device_copy": {"us": t_copy * 1e6, "bytes": 2 * n_copy, "GBps": 2 * n_copy / t_copy / 1e9,
                        "frac_hbm": 2 * n_copy / t_copy / 1e9 / HBM_PEAK_GBPS,
                        "note": "plain device copy of the quantise's byte count (read + write): the achievable line"},
    }
    # the dominant kernel by median time; achieved = its algorithmic bytes per launch / median duration
    dom = "quantize_tiles" if med[0] >= med[2] else "decode_attention"
    dk = kernels[dom]
    t_dom = dk["us_median"] * 1e-6
    tr = traffic.get(dom)
    roofline = {"bound": "hbm", "achieved": dk["bytes"] / t_dom / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": dk["bytes"] / t_dom / 1e9 / HBM_PEAK_GBPS, "traffic": tr, "kernel": dom,
                "algorithmic_bytes_per_launch": dk["bytes"], "time": "median of per-launch HIP events"}

    result = {
        "metric": "quantize GB/s + quantized decode-attn tokens/s, % of HBM peak (k4v2 g128)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": ("bulk quantize 1024 tiles x 4 kv heads (8 seqs x 16384 tokens) + append 1 token "
                                "x 32 seqs + decode 32 seqs x 16384 ctx, 32 q / 4 kv heads, head_dim 128, "
                                "kvarn_k4v2_g128, block 128, 8 Sinkhorn iterations"),
                   "format": FORMAT, "quantize_tiles": Q_TILES, "kv_heads": Q_HKV, "decode_batch": D_B,
                   "decode_ctx": D_CTX, "q_heads": D_HQ, "parallelism": "single GPU"},
        "frac_hbm_step": value / HBM_PEAK_GBPS,
        "kernels": kernels,
        "roofline": roofline,
        "source_hash": src_hash,
        "prep_s": prep_s,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(k1, v1, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
