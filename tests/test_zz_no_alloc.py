"""GPU test of kvarn_decode_attention_noalloc (the decode entry point that allocates nothing and
keeps its split partials in the library's fixed per-GPU scratch) against kvarn_decode_attention with
a caller workspace, through the C-ABI: two calls in a row, the second with fewer, shorter sequences,
each bit-identical to the workspace entry point on the same inputs (same kernels, same plan) and
within the decode tolerance of the oracle on the GPU's own cache bytes."""
import math

import numpy as np
import pytest

import oracle
from kv_cache_quantization_pipeline_amd import synth
from parity import DECODE_REL_L2, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_quantization_pipeline_amd as kv  # noqa: E402

DEV = "cuda"


def _case(lens, hkv, hq, seed, name="kvarn_k4v2_g128"):
    fmt = kv.format_parse(name)
    R = kv.record_bytes(fmt)
    stride = hkv * R
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    full = lens // 128
    max_pages = int(full.max()) + 1
    n_full = int(full.sum())
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_full + 1).astype(np.int32)
    pt = np.full((B, max_pages), perm[-1], np.int32)
    dst, c = [], 0
    for s in range(B):
        for p in range(full[s]):
            pt[s, p] = perm[c]
            dst.append(perm[c])
            c += 1
    k, v = synth.gen_kv(seed, max(n_full, 1) * 128, hkv)
    cache = torch.zeros((n_full + 1) * stride, dtype=torch.uint8, device=DEV)
    if n_full:
        kv.quantize_tiles(fmt, torch.from_numpy(np.ascontiguousarray(synth.tiles_view(k)[:n_full])).to(DEV),
                          torch.from_numpy(np.ascontiguousarray(synth.tiles_view(v)[:n_full])).to(DEV),
                          torch.from_numpy(np.asarray(dst, np.int32)).to(DEV), cache, stride)
    tk = (rng.standard_normal((B, hkv, 128, 128)) * 1.5).astype(np.float16)
    tv = (rng.standard_normal((B, hkv, 128, 128)) * 1.5).astype(np.float16)
    q = synth.gen_q(seed, B, hq)
    return dict(fmt=fmt, stride=stride, lens=lens, pt=pt, cache=cache, tk=tk, tv=tv, q=q, hkv=hkv, hq=hq, B=B)


def _run(c, noalloc):
    sm = 1.0 / math.sqrt(128)
    out = torch.full((c["B"], c["hq"], 128), float("nan"), dtype=torch.float16, device=DEV)
    args = (c["fmt"], torch.from_numpy(c["q"]).to(DEV), c["cache"], c["stride"], torch.from_numpy(c["pt"]).to(DEV),
            torch.from_numpy(c["lens"]).to(DEV), torch.from_numpy(c["tk"]).to(DEV), torch.from_numpy(c["tv"]).to(DEV),
            sm, out)
    if noalloc:
        kv.decode_attention_noalloc(*args, c["hkv"])
    else:
        ws = kv.decode_workspace(c["fmt"], c["B"], c["hq"], c["hkv"], c["pt"].shape[1], DEV)
        kv.decode_attention(*args, ws, c["hkv"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_oracle(c, got):
    host = c["cache"].cpu().numpy()
    _, ref = oracle.decode_attention(c["fmt"].k_bits, c["fmt"].v_bits, c["q"].view(np.uint16), host, c["stride"],
                                     c["pt"], c["lens"], c["tk"].view(np.uint16), c["tv"].view(np.uint16),
                                     1.0 / math.sqrt(128), c["hkv"], group=c["fmt"].group)
    for s in range(c["B"]):
        for h in range(c["hq"]):
            if c["lens"][s] == 0:
                assert np.all(got[s, h] == 0)
            else:
                assert rel_l2(got[s, h].astype(np.float64), ref[s, h]) <= DECODE_REL_L2, (s, h)


def test_noalloc_decode_matches_workspace_decode_twice():
    big = _case([3000, 129, 0, 1029, 640, 127, 2048 + 77], hkv=2, hq=16, seed=41)
    small = _case([300, 5, 128], hkv=1, hq=8, seed=42)
    need_big = kv.decode_workspace_bytes(big["fmt"], big["B"], big["hq"], big["hkv"], big["pt"].shape[1])
    need_small = kv.decode_workspace_bytes(small["fmt"], small["B"], small["hq"], small["hkv"], small["pt"].shape[1])
    assert need_small < need_big <= kv.decode_noalloc_max_workspace_bytes()
    print("case: 7 seqs x 16 q / 2 kv heads, then 3 seqs x 8 q / 1 kv head", flush=True)
    a = _run(big, noalloc=True)
    b = _run(small, noalloc=True)
    assert np.array_equal(a.view(np.uint16), _run(big, noalloc=False).view(np.uint16))
    assert np.array_equal(b.view(np.uint16), _run(small, noalloc=False).view(np.uint16))
    _check_oracle(big, a)
    _check_oracle(small, b)


def test_noalloc_decode_grouped_format():
    c = _case([1500, 64, 2 * 128], hkv=2, hq=4, seed=43, name="kvarn_k8v4_g64")
    print("case: kvarn_k8v4_g64, 3 seqs x 4 q / 2 kv heads", flush=True)
    got = _run(c, noalloc=True)
    assert np.array_equal(got.view(np.uint16), _run(c, noalloc=False).view(np.uint16))
    _check_oracle(c, got)
