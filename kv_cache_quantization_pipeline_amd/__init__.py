"""Python binding of libkvarn (KVarN KV-cache quantisation for MI355X / gfx950).

Argument marshalling only: every step of the method runs in the HIP kernels of
libkvarn.so, which this module loads with ctypes.  torch supplies device memory
and the current stream.  If the library has not been built this module raises
on first use; there is no CPU fallback.

Functions mirror include/libkvarn.h:
    format_parse, record_bytes, decode_workspace_bytes,
    quantize_tiles, append_token, decode_attention, prefill_attention,
    decode_attention_noalloc, PagePool (kvarn_page_pool_*)
plus decode_workspace (a workspace tensor for decode_attention) and
prepare_append_token / prepare_decode_attention (the same calls with their arguments marshalled
once, for serving loops whose kernels take a few microseconds).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVARN_LIB selects another build of the same sources (the host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("KVARN_LIB") or os.path.join(_HERE, "libkvarn.so")

KVARN_OK, KVARN_E_INVALID_ARG, KVARN_E_UNSUPPORTED, KVARN_E_HIP, KVARN_E_SCRATCH_LIMIT, KVARN_E_OUT_OF_PAGES = range(6)

# every C-ABI entry point declared in include/libkvarn.h
EXPORTS = (
    "kvarn_format_parse",
    "kvarn_format_check",
    "kvarn_record_bytes",
    "kvarn_decode_workspace_bytes",
    "kvarn_quantize_tiles",
    "kvarn_append_token",
    "kvarn_decode_attention",
    "kvarn_decode_attention_noalloc",
    "kvarn_decode_noalloc_max_workspace_bytes",
    "kvarn_prefill_attention",
    "kvarn_page_pool_create",
    "kvarn_page_pool_destroy",
    "kvarn_page_pool_num_free",
    "kvarn_page_pool_reserve",
    "kvarn_page_pool_release",
    "kvarn_status_string",
)


class KvarnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class Format(ctypes.Structure):
    """kvarn_format: bits, group and sizes of one kv-cache dtype."""
    _fields_ = [("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32)]

    def __repr__(self):
        return (f"Format(k{self.k_bits}v{self.v_bits}_g{self.group}, head_dim={self.head_dim}, "
                f"block={self.block_size}, iters={self.sinkhorn_iters})")


_lib = None


def lib():
    """The loaded libkvarn.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvarn.so not found at {LIB_PATH}; run __graft_entry__.build() "
                               "or python kv_cache_quantization_pipeline_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, flt = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        fp = ctypes.POINTER(Format)
        L.kvarn_format_parse.restype = i32
        L.kvarn_format_parse.argtypes = [ctypes.c_char_p, fp]
        L.kvarn_format_check.restype = i32
        L.kvarn_format_check.argtypes = [fp]
        L.kvarn_record_bytes.restype = sz
        L.kvarn_record_bytes.argtypes = [fp]
        L.kvarn_decode_workspace_bytes.restype = sz
        L.kvarn_decode_workspace_bytes.argtypes = [fp, i32, i32, i32, i32]
        L.kvarn_quantize_tiles.restype = i32
        L.kvarn_quantize_tiles.argtypes = [fp, i32, i32, vp, vp, vp, vp, i64, vp]
        L.kvarn_append_token.restype = i32
        L.kvarn_append_token.argtypes = [fp, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i64, vp]
        L.kvarn_decode_attention.restype = i32
        L.kvarn_decode_attention.argtypes = [fp, i32, i32, i32, vp, vp, i64, vp, i32, vp, vp, vp, flt, vp, vp, sz,
                                             vp]
        L.kvarn_decode_attention_noalloc.restype = i32
        L.kvarn_decode_attention_noalloc.argtypes = [fp, i32, i32, i32, vp, vp, i64, vp, i32, vp, vp, vp, flt, vp,
                                                     vp]
        L.kvarn_decode_noalloc_max_workspace_bytes.restype = sz
        L.kvarn_decode_noalloc_max_workspace_bytes.argtypes = []
        L.kvarn_prefill_attention.restype = i32
        L.kvarn_prefill_attention.argtypes = [fp, i32, i32, i32, i32, vp, vp, vp, i64, vp, i32, vp, vp, vp, flt, vp,
                                              vp]
        L.kvarn_page_pool_create.restype = i32
        L.kvarn_page_pool_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.kvarn_page_pool_destroy.restype = None
        L.kvarn_page_pool_destroy.argtypes = [vp]
        L.kvarn_page_pool_num_free.restype = i32
        L.kvarn_page_pool_num_free.argtypes = [vp]
        L.kvarn_page_pool_reserve.restype = i32
        L.kvarn_page_pool_reserve.argtypes = [vp, i32, vp, vp, i32, vp]
        L.kvarn_page_pool_release.restype = i32
        L.kvarn_page_pool_release.argtypes = [vp, vp, i32, vp]
        L.kvarn_status_string.restype = ctypes.c_char_p
        L.kvarn_status_string.argtypes = [i32]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvarn_status_string(status).decode()


def _check(status: int, what: str):
    if status != KVARN_OK:
        raise KvarnError(status, what)


def format_parse(name: str) -> Format:
    f = Format()
    _check(lib().kvarn_format_parse(name.encode(), ctypes.byref(f)), f"kvarn_format_parse({name!r})")
    return f


def record_bytes(fmt: Format) -> int:
    return int(lib().kvarn_record_bytes(ctypes.byref(fmt)))


def decode_workspace_bytes(fmt: Format, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                           max_pages_per_seq: int) -> int:
    return int(lib().kvarn_decode_workspace_bytes(ctypes.byref(fmt), num_seqs, num_q_heads, num_kv_heads,
                                                  max_pages_per_seq))


def decode_workspace(fmt: Format, num_seqs: int, num_q_heads: int, num_kv_heads: int, max_pages_per_seq: int,
                     device=None):
    """A device workspace for decode_attention at these sizes (its contents need no initialisation;
    the tensor can be reused by later calls on the same stream)."""
    import torch
    n = decode_workspace_bytes(fmt, num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq)
    if n == 0:
        raise ValueError("unsupported decode shape")
    return torch.empty(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def quantize_tiles(fmt: Format, k, v, dst_pages, cache, page_stride_bytes: int, stream=None):
    """k, v: fp16 [num_tiles, 128, Hkv, 128]; dst_pages: int32 [num_tiles]; cache: uint8 pool."""
    import torch
    _need(k, "k", torch.float16, 4)
    _need(v, "v", torch.float16, 4)
    _need(dst_pages, "dst_pages", torch.int32, 1)
    _need(cache, "cache", torch.uint8)
    if k.shape != v.shape or k.shape[1] != 128 or k.shape[3] != 128 or dst_pages.shape[0] != k.shape[0]:
        raise ValueError(f"bad shapes k {tuple(k.shape)} v {tuple(v.shape)} dst_pages {tuple(dst_pages.shape)}")
    st = lib().kvarn_quantize_tiles(ctypes.byref(fmt), k.shape[0], k.shape[2], _ptr(k), _ptr(v), _ptr(dst_pages),
                                    _ptr(cache), page_stride_bytes, _stream(stream))
    _check(st, "kvarn_quantize_tiles")


def _append_args(fmt, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache, page_stride_bytes, stream):
    import torch
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(tail_k, "tail_k", torch.float16, 4)
    _need(tail_v, "tail_v", torch.float16, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(cache, "cache", torch.uint8)
    B, hkv = k_new.shape[0], k_new.shape[1]
    if k_new.shape[2] != 128:
        raise ValueError(f"k_new must be [B, Hkv, 128] (head_dim 128), got {tuple(k_new.shape)}")
    if (v_new.shape != k_new.shape or tuple(tail_k.shape) != (B, hkv, 128, 128) or tail_v.shape != tail_k.shape
            or seq_lens.shape[0] != B or page_table.shape[0] != B):
        raise ValueError("inconsistent shapes for append_token")
    return (ctypes.byref(fmt), B, hkv, _ptr(k_new), _ptr(v_new), _ptr(seq_lens), _ptr(tail_k), _ptr(tail_v),
            _ptr(page_table), page_table.shape[1], _ptr(cache), page_stride_bytes, _stream(stream))


def append_token(fmt: Format, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache, page_stride_bytes: int,
                 stream=None):
    """k_new, v_new: fp16 [B, Hkv, 128]; seq_lens int32 [B] (incremented); tails fp16 [B, Hkv, 128, 128];
    page_table int32 [B, max_pages]."""
    args = _append_args(fmt, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache, page_stride_bytes, stream)
    _check(lib().kvarn_append_token(*args), "kvarn_append_token")


def _decode_args(fmt, q, cache, page_stride_bytes, page_table, seq_lens, tail_k, tail_v, sm_scale, out, workspace,
                 num_kv_heads, stream):
    import torch
    _need(q, "q", torch.float16, 3)
    _need(out, "out", torch.float16, 3)
    _need(cache, "cache", torch.uint8)
    _need(page_table, "page_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(tail_k, "tail_k", torch.float16, 4)
    _need(tail_v, "tail_v", torch.float16, 4)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    B, hq = q.shape[0], q.shape[1]
    if q.shape[2] != 128:
        raise ValueError(f"q must be [B, Hq, 128] (head_dim 128), got {tuple(q.shape)}")
    if out.shape != q.shape or seq_lens.shape[0] != B or page_table.shape[0] != B:
        raise ValueError("inconsistent shapes for decode_attention")
    if tuple(tail_k.shape) != (B, num_kv_heads, 128, 128) or tail_v.shape != tail_k.shape:
        raise ValueError(f"tails must be [B, Hkv, 128, 128], got {tuple(tail_k.shape)}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (ctypes.byref(fmt), B, hq, num_kv_heads, _ptr(q), _ptr(cache), page_stride_bytes, _ptr(page_table),
            page_table.shape[1], _ptr(seq_lens), _ptr(tail_k), _ptr(tail_v), float(sm_scale), _ptr(out),
            _ptr(workspace), ws_bytes, _stream(stream))


def decode_attention(fmt: Format, q, cache, page_stride_bytes: int, page_table, seq_lens, tail_k, tail_v,
                     sm_scale: float, out, workspace, num_kv_heads: int, stream=None):
    """q, out: fp16 [B, Hq, 128]; page_table int32 [B, max_pages]; seq_lens int32 [B];
    tails fp16 [B, Hkv, 128, 128]; workspace: device tensor of >= decode_workspace_bytes bytes (any
    contents, e.g. from decode_workspace)."""
    args = _decode_args(fmt, q, cache, page_stride_bytes, page_table, seq_lens, tail_k, tail_v, sm_scale, out,
                        workspace, num_kv_heads, stream)
    _check(lib().kvarn_decode_attention(*args), "kvarn_decode_attention")


def decode_attention_noalloc(fmt: Format, q, cache, page_stride_bytes: int, page_table, seq_lens, tail_k, tail_v,
                             sm_scale: float, out, num_kv_heads: int, stream=None):
    """decode_attention with the library's fixed per-GPU scratch instead of a caller workspace (for
    callers that cannot allocate); calls that may overlap on one GPU race."""
    args = _decode_args(fmt, q, cache, page_stride_bytes, page_table, seq_lens, tail_k, tail_v, sm_scale, out,
                        None, num_kv_heads, stream)
    args = args[:14] + args[16:]
    _check(lib().kvarn_decode_attention_noalloc(*args), "kvarn_decode_attention_noalloc")


def decode_noalloc_max_workspace_bytes() -> int:
    return int(lib().kvarn_decode_noalloc_max_workspace_bytes())


class PreparedCall:
    """One C-ABI call whose arguments were checked and marshalled once (the tensors it points to are
    held here).  Calling it only re-issues the call on the stream it was prepared for, for loops whose
    GPU work per call is a few microseconds and whose host time would otherwise dominate."""

    def __init__(self, fn, args, what, keep):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != KVARN_OK:
            raise KvarnError(st, self._what)


def prepare_append_token(fmt: Format, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache,
                         page_stride_bytes: int, stream=None) -> PreparedCall:
    """append_token with the same arguments, checked and marshalled once: returns a callable that
    issues it on the stream current now (or `stream`)."""
    args = _append_args(fmt, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache, page_stride_bytes, stream)
    return PreparedCall(lib().kvarn_append_token, args, "kvarn_append_token",
                        (fmt, k_new, v_new, seq_lens, tail_k, tail_v, page_table, cache))


def prepare_decode_attention(fmt: Format, q, cache, page_stride_bytes: int, page_table, seq_lens, tail_k, tail_v,
                             sm_scale: float, out, workspace, num_kv_heads: int, stream=None) -> PreparedCall:
    """decode_attention with the same arguments, checked and marshalled once: returns a callable
    that issues it on the stream current now (or `stream`)."""
    args = _decode_args(fmt, q, cache, page_stride_bytes, page_table, seq_lens, tail_k, tail_v, sm_scale, out,
                        workspace, num_kv_heads, stream)
    return PreparedCall(lib().kvarn_decode_attention, args, "kvarn_decode_attention",
                        (fmt, q, cache, page_table, seq_lens, tail_k, tail_v, out, workspace))


def prefill_attention(fmt: Format, q, q_lens, cache, page_stride_bytes: int, page_table, seq_lens, tail_k, tail_v,
                      sm_scale: float, out, num_kv_heads: int, stream=None):
    """q, out: fp16 [B, max_q, Hq, 128]; q_lens, seq_lens: int32 [B]; page_table int32 [B, max_pages];
    tails fp16 [B, Hkv, 128, 128].  The last q_lens[s] of the seq_lens[s] cached tokens are the queries."""
    import torch
    _need(q, "q", torch.float16, 4)
    _need(out, "out", torch.float16, 4)
    _need(q_lens, "q_lens", torch.int32, 1)
    _need(cache, "cache", torch.uint8)
    _need(page_table, "page_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(tail_k, "tail_k", torch.float16, 4)
    _need(tail_v, "tail_v", torch.float16, 4)
    B, max_q, hq = q.shape[0], q.shape[1], q.shape[2]
    if (out.shape != q.shape or q.shape[3] != 128 or q_lens.shape[0] != B or seq_lens.shape[0] != B
            or page_table.shape[0] != B):
        raise ValueError("inconsistent shapes for prefill_attention")
    if tuple(tail_k.shape) != (B, num_kv_heads, 128, 128) or tail_v.shape != tail_k.shape:
        raise ValueError(f"tails must be [B, Hkv, 128, 128], got {tuple(tail_k.shape)}")
    st = lib().kvarn_prefill_attention(ctypes.byref(fmt), B, max_q, hq, num_kv_heads, _ptr(q), _ptr(q_lens),
                                       _ptr(cache), page_stride_bytes, _ptr(page_table), page_table.shape[1],
                                       _ptr(seq_lens), _ptr(tail_k), _ptr(tail_v), float(sm_scale), _ptr(out),
                                       _stream(stream))
    _check(st, "kvarn_prefill_attention")



class PagePool:
    """kvarn_page_pool: host-side pool of 128-token cache pages.  Page tables and ownership counts are
    numpy int32 arrays on the host, filled in place (upload the table to the device afterwards)."""

    def __init__(self, num_pages: int):
        h = ctypes.c_void_p()
        _check(lib().kvarn_page_pool_create(num_pages, ctypes.byref(h)), "kvarn_page_pool_create")
        self._h = h
        self.num_pages = num_pages

    def close(self):
        if self._h is not None and self._h.value:
            lib().kvarn_page_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(lib().kvarn_page_pool_num_free(self._h))

    @staticmethod
    def _i32(a, name, ndim):
        import numpy as np
        if not isinstance(a, np.ndarray) or a.dtype != np.int32 or a.ndim != ndim or not a.flags.c_contiguous:
            raise ValueError(f"{name} must be a C-contiguous numpy int32 array with {ndim} dims")
        return a.ctypes.data_as(ctypes.c_void_p)

    def reserve(self, new_lens, page_table, num_owned):
        """new_lens int32 [B]; page_table int32 [B, max_pages] and num_owned int32 [B], both updated."""
        B = new_lens.shape[0] if hasattr(new_lens, "shape") else 0
        pl, pt, po = (self._i32(new_lens, "new_lens", 1), self._i32(page_table, "page_table", 2),
                      self._i32(num_owned, "num_owned", 1))
        if page_table.shape[0] != B or num_owned.shape[0] != B:
            raise ValueError("inconsistent batch sizes for reserve")
        _check(lib().kvarn_page_pool_reserve(self._h, B, pl, pt, page_table.shape[1], po), "kvarn_page_pool_reserve")

    def release(self, page_table_row, num_owned, s: int = 0):
        """Return sequence s's pages: page_table_row is the int32 [max_pages] row (or the [B, max_pages] table
        with row s), num_owned the int32 [B] counts; both updated."""
        row = page_table_row if page_table_row.ndim == 1 else page_table_row[s]
        self._i32(row, "page_table_row", 1)
        self._i32(num_owned, "num_owned", 1)
        if not 0 <= s < num_owned.shape[0]:
            raise ValueError("sequence index out of range")
        cnt = num_owned[s:s + 1]
        _check(lib().kvarn_page_pool_release(self._h, row.ctypes.data_as(ctypes.c_void_p), row.shape[0],
                                             cnt.ctypes.data_as(ctypes.c_void_p)), "kvarn_page_pool_release")
