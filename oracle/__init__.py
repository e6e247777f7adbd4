"""ctypes wrapper of the fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py.  The product path (kv_cache_quantization_pipeline_amd)
never imports this package.  All arrays are numpy, host memory.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVARN_ORACLE_LIB selects another build of the same source (the sanitizer build of the CPU tests)
_LIB_PATH = os.environ.get("KVARN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

T = 128
D = 128


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_record_bytes.restype = ctypes.c_size_t
        L.oracle_record_bytes.argtypes = [i32, i32, i32]
        L.oracle_threads_used.restype = i32
        L.oracle_threads_used.argtypes = [i32]
        L.oracle_half_to_double.argtypes = [vp, vp, i64]
        L.oracle_double_to_half.argtypes = [vp, vp, i64]
        L.oracle_rotate.argtypes = [vp, vp, i32]
        L.oracle_sinkhorn.argtypes = [vp, i32, vp, vp, vp]
        L.oracle_rtn.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_quantize_tile_debug.restype = i32
        L.oracle_quantize_tile_debug.argtypes = [vp, i32, i32, i32] + [vp] * 10
        L.oracle_pack_record.restype = i32
        L.oracle_pack_record.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_unpack_record.restype = i32
        L.oracle_unpack_record.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_dequant_record.restype = i32
        L.oracle_dequant_record.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_quantize_tiles.restype = i32
        L.oracle_quantize_tiles.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i64, i32]
        L.oracle_append_token.restype = i32
        L.oracle_append_token.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i64,
                                          i32]
        L.oracle_decode_attention.restype = i32
        L.oracle_decode_attention.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, vp, i32, vp, vp, vp,
                                              dbl, vp, vp, i32]
        L.oracle_prefill_attention.restype = i32
        L.oracle_prefill_attention.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, i32, vp, vp,
                                               vp, dbl, vp, vp, i32]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def record_bytes(kb, vb, group=128):
    return int(lib().oracle_record_bytes(kb, vb, group))


def n_groups(group):
    return D // group


def split_scales(sc, group=128):
    """Scale block of a record (flat float32) -> (cK, s'K, m'K, cV, s'V, m'V); s'/m' are [ng][128]
    (group gi of token t at [gi][t]), squeezed to [128] when the group is the whole token."""
    ng = n_groups(group)
    hs = D * (1 + 2 * ng)
    sc = np.asarray(sc, np.float32).reshape(-1)
    assert sc.size == 2 * hs
    out = []
    for h in range(2):
        b = sc[h * hs:(h + 1) * hs]
        sp = b[D:D + ng * T].reshape(ng, T)
        mp = b[D + ng * T:].reshape(ng, T)
        out += [b[:D], sp[0] if ng == 1 else sp, mp[0] if ng == 1 else mp]
    return tuple(out)


def threads_used(n=0):
    return int(lib().oracle_threads_used(n))


def half_to_double(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_half_to_double(_p(h), _p(out), h.size)
    return out


def double_to_half(d):
    d = _c(d, np.float64)
    out = np.empty(d.shape, np.uint16)
    lib().oracle_double_to_half(_p(d), _p(out), d.size)
    return out


def rotate(x):
    """y = x Hn row by row (x: [rows, 128] float64)."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib().oracle_rotate(_p(x), _p(y), x.shape[0])
    return y


def sinkhorn(y, iters):
    """Log-space Sinkhorn on A = y*y (y: [128,128]) -> (u[128], v[128], col_dev[iters])."""
    y = _c(y, np.float64)
    u = np.empty(T)
    v = np.empty(D)
    dev = np.empty(max(iters, 1))
    lib().oracle_sinkhorn(_p(y), iters, _p(u), _p(v), _p(dev))
    return u, v, dev[:iters]


def rtn(z, bits):
    """Asymmetric RTN per row (one group = one row of n values) -> (mn[rows], s[rows], q[rows,n] uint8, tval)."""
    z = _c(z, np.float64)
    rows, n = z.shape
    mn = np.empty(rows)
    s = np.empty(rows)
    q = np.empty((rows, n), np.uint8)
    tv = np.empty((rows, n))
    lib().oracle_rtn(_p(z), rows, n, bits, _p(mn), _p(s), _p(q), _p(tv))
    return mn, s, q, tv


def quantize_tile_debug(x16, bits, iters=8, group=128):
    """One tile half (x16: [128,128] uint16 fp16 bits) with every intermediate.  s' and m' are
    [ng][128] (group-major), squeezed to [128] when the group is the whole token."""
    x16 = _c(x16, np.uint16)
    assert x16.shape == (T, D)
    ng = n_groups(group)
    out = dict(y=np.empty((T, D)), u=np.empty(T), v=np.empty(D), z=np.empty((T, D)), tval=np.empty((T, D)),
               q=np.empty((T, D), np.uint8), c=np.empty(D, np.float32), sp=np.empty((ng, T), np.float32),
               mp=np.empty((ng, T), np.float32), col_dev=np.empty(max(iters, 1)))
    rc = lib().oracle_quantize_tile_debug(_p(x16), bits, iters, group, *[_p(out[k]) for k in
                                          ("y", "u", "v", "z", "tval", "q", "c", "sp", "mp", "col_dev")])
    assert rc == 0
    out["col_dev"] = out["col_dev"][:iters]
    if ng == 1:
        out["sp"], out["mp"] = out["sp"][0], out["mp"][0]
    return out


def pack_record(kb, vb, qk, qv, scales, group=128):
    """scales: [2 (1 + 2 ng), 128] float32 rows cK, s'K[ng], m'K[ng], cV, s'V[ng], m'V[ng] (or flat)."""
    rec = np.empty(record_bytes(kb, vb, group), np.uint8)
    rc = lib().oracle_pack_record(kb, vb, group, _p(_c(qk, np.uint8)), _p(_c(qv, np.uint8)),
                                  _p(_c(scales, np.float32)), _p(rec))
    assert rc == 0
    return rec


def unpack_record(kb, vb, rec, group=128):
    """-> (qk [128,128], qv [128,128], scales [2 (1 + 2 ng), 128] float32; [6, 128] for g128)."""
    rec = _c(rec, np.uint8)
    qk = np.empty((T, D), np.uint8)
    qv = np.empty((T, D), np.uint8)
    sc = np.empty((2 * (1 + 2 * n_groups(group)), D), np.float32)
    rc = lib().oracle_unpack_record(kb, vb, group, _p(rec), _p(qk), _p(qv), _p(sc))
    assert rc == 0
    return qk, qv, sc


def dequant_record(kb, vb, rec, group=128):
    rec = _c(rec, np.uint8)
    k = np.empty((T, D))
    v = np.empty((T, D))
    rc = lib().oracle_dequant_record(kb, vb, group, _p(rec), _p(k), _p(v))
    assert rc == 0
    return k, v


def quantize_tiles(kb, vb, iters, k, v, dst_pages, cache, page_stride, nthreads=0, group=128):
    """k, v: uint16 [num_tiles,128,Hkv,128]; cache: uint8 pool (modified in place)."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    dst = _c(dst_pages, np.int32)
    assert cache.flags["C_CONTIGUOUS"] and cache.dtype == np.uint8
    rc = lib().oracle_quantize_tiles(kb, vb, iters, group, k.shape[0], k.shape[2], _p(k), _p(v), _p(dst),
                                     _p(cache), page_stride, nthreads)
    assert rc == 0


def append_token(kb, vb, iters, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache, page_stride,
                 nthreads=0, group=128):
    """All arrays host numpy; seq_lens, tail_k, tail_v, cache modified in place."""
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    pt = _c(page_table, np.int32)
    for a in (seq_lens, tail_k, tail_v, cache):
        assert a.flags["C_CONTIGUOUS"]
    rc = lib().oracle_append_token(kb, vb, iters, group, k_new.shape[0], k_new.shape[1], _p(k_new), _p(v_new),
                                   _p(seq_lens), _p(tail_k), _p(tail_v), _p(pt), pt.shape[1], _p(cache),
                                   page_stride, nthreads)
    assert rc == 0


def decode_attention(kb, vb, q, cache, page_stride, page_table, seq_lens, tail_k, tail_v, sm_scale,
                     num_kv_heads, nthreads=0, group=128):
    """q: uint16 [B,Hq,128] -> (out fp16 bits [B,Hq,128], out fp64)."""
    q = _c(q, np.uint16)
    cache = _c(cache, np.uint8)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    tk = _c(tail_k, np.uint16)
    tv = _c(tail_v, np.uint16)
    out = np.empty(q.shape, np.uint16)
    out64 = np.empty(q.shape, np.float64)
    rc = lib().oracle_decode_attention(kb, vb, group, q.shape[0], q.shape[1], num_kv_heads, _p(q), _p(cache),
                                       page_stride, _p(pt), pt.shape[1], _p(sl), _p(tk), _p(tv),
                                       float(sm_scale), _p(out), _p(out64), nthreads)
    assert rc == 0
    return out, out64


def prefill_attention(kb, vb, q, q_lens, cache, page_stride, page_table, seq_lens, tail_k, tail_v, sm_scale,
                      num_kv_heads, nthreads=0, group=128, out=None):
    """q: uint16 [B, max_q, Hq, 128]; query i of sequence s at position seq_lens[s] - q_lens[s] + i attends
    causally.  -> (out fp16 bits, out fp64), rows i >= q_lens[s] as given in `out` (zeros by default)."""
    q = _c(q, np.uint16)
    ql = _c(q_lens, np.int32)
    cache = _c(cache, np.uint8)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    tk = _c(tail_k, np.uint16)
    tv = _c(tail_v, np.uint16)
    o16 = np.zeros(q.shape, np.uint16) if out is None else np.array(out, np.uint16)
    o64 = np.zeros(q.shape, np.float64)
    rc = lib().oracle_prefill_attention(kb, vb, group, q.shape[0], q.shape[1], q.shape[2], num_kv_heads, _p(q),
                                        _p(ql), _p(cache), page_stride, _p(pt), pt.shape[1], _p(sl), _p(tk), _p(tv),
                                        float(sm_scale), _p(o16), _p(o64), nthreads)
    assert rc == 0
    return o16, o64

