"""Seeded random shapes against the oracle: the tile quantiser over formats, iteration counts, tile and
kv-head counts, magnitudes and token-scale spreads; append steps with pages from the host pool; decode
and chunked prefill over formats, query heads per kv head, kv-head counts, ragged lengths (page
boundaries, empty sequences, tails of every size) and page tables wider than the lengths need (so the
split counts, the tail-split mode and the merge shape vary from case to case).  Every case prints its
parameters before it runs."""
import numpy as np
import pytest

import oracle
from kv_cache_quantization_pipeline_amd import synth
from parity import assert_code_rate, check_record
from test_gpu_decode import Setup, _compare
from test_gpu_prefill import Prefill

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_quantization_pipeline_amd as kv  # noqa: E402

FORMATS = [f"kvarn_k{kb}v{vb}_g{g}" for g in (128, 64, 32) for kb in (2, 4, 8) for vb in (2, 4, 8)]
N_CASES = 60


def _case(i):
    rng = np.random.default_rng(1000 + i)
    name = FORMATS[rng.integers(len(FORMATS))]
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 3, 5]))
    B = int(rng.integers(1, 6))
    lens = []
    for _ in range(B):
        kind = rng.integers(4)
        if kind == 0:
            lens.append(int(rng.integers(0, 2600)))
        elif kind == 1:
            lens.append(int(rng.integers(0, 21)) * 128 + int(rng.choice([-1, 0, 1])))
        elif kind == 2:
            lens.append(int(rng.integers(0, 3)))
        else:
            lens.append(int(rng.integers(2000, 6000)))
    lens = [max(0, x) for x in lens]
    need = max(1, max(x // 128 for x in lens) + 1)
    # occasionally a page table far wider than the lengths need (more than 64 page splits in the
    # one-page-per-wave formats)
    extra = int(rng.choice([0, 3, 40, 300]))
    q_lens = [int(rng.integers(0, min(x, 96) + 1)) for x in lens]
    return name, G, hkv, lens, need + extra, q_lens, 2000 + i


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(i):
    name, G, hkv, lens, max_pages, _, seed = _case(i)
    print(f"case {i}: decode {name} G {G} hkv {hkv} lens {lens} max_pages {max_pages}", flush=True)
    st = Setup(name, lens, hkv=hkv, hq=hkv * G, seed=seed, max_pages=max_pages)
    _compare(st.run_gpu(), st.run_oracle(), st.lens)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill(i):
    name, G, hkv, lens, _, q_lens, seed = _case(i)
    lens = [min(x, 3000) for x in lens]           # bounds the oracle's causal attention
    q_lens = [min(q, x) for q, x in zip(q_lens, lens)]
    print(f"case {i}: prefill {name} G {G} hkv {hkv} lens {lens} q_lens {q_lens}", flush=True)
    st = Prefill(name, lens, q_lens, hkv=hkv, hq=hkv * G, seed=seed)
    st.compare(st.run_gpu(), st.run_oracle())


def _quant_case(i):
    rng = np.random.default_rng(3000 + i)
    name = FORMATS[rng.integers(len(FORMATS))]
    iters = int(rng.choice([8, 8, 8, 1, 3]))
    T = int(rng.integers(1, 7))
    hkv = int(rng.integers(1, 6))
    scale = float(2.0 ** rng.integers(-8, 8))
    spread = float(rng.choice([0.0, 0.5, 2.3]))       # log-normal token-scale spread (2.3: four decades)
    return name, iters, T, hkv, scale, spread, rng


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_quantize(i):
    """Random format, iteration count, tile and kv-head counts, magnitude (x 2^-8 .. 2^7), token-scale
    spread and outlier channels, with zero tokens and zero channels mixed in; tiles go to permuted
    pages of a canary-filled pool, and every record must match the oracle's (layout bit-exact,
    scales and codes to the parity criteria)."""
    name, iters, T, hkv, scale, spread, rng = _quant_case(i)
    print(f"case {i}: quantize {name} iters {iters} tiles {T} hkv {hkv} scale {scale} spread {spread}", flush=True)
    fmt = kv.format_parse(name)
    fmt.sinkhorn_iters = iters
    x = rng.standard_normal((2, T, 128, hkv, 128))
    x *= np.exp(spread * rng.standard_normal((2, T, 128, hkv, 1)))
    out_ch = rng.integers(0, 128, size=4)
    x[..., out_ch] *= 20.0
    x[:, :, rng.integers(0, 128, size=3)] = 0.0          # zero tokens
    x[..., rng.integers(0, 128, size=2)] = 0.0           # zero channels
    x = np.clip(x * scale, -60000.0, 60000.0).astype(np.float16)
    k16, v16 = x[0], x[1]
    R = kv.record_bytes(fmt)
    stride = hkv * R
    n_pool = T + 2
    pages = rng.permutation(n_pool)[:T].astype(np.int32)
    cache = torch.full((n_pool * stride,), 0xA5, dtype=torch.uint8, device="cuda")
    kv.quantize_tiles(fmt, torch.from_numpy(np.ascontiguousarray(k16)).to("cuda"),
                      torch.from_numpy(np.ascontiguousarray(v16)).to("cuda"), torch.from_numpy(pages).to("cuda"),
                      cache, stride)
    torch.cuda.synchronize()
    host = cache.cpu().numpy()
    used = np.zeros(n_pool, bool)
    used[pages] = True
    for p in np.nonzero(~used)[0]:
        assert np.all(host[p * stride:(p + 1) * stride] == 0xA5), f"page {p} (not a destination) was written"
    n_bad = 0
    for t in range(T):
        for h in range(hkv):
            off = int(pages[t]) * stride + h * R
            rk = oracle.quantize_tile_debug(np.ascontiguousarray(k16[t, :, h]).view(np.uint16), fmt.k_bits, iters,
                                            group=fmt.group)
            rv = oracle.quantize_tile_debug(np.ascontiguousarray(v16[t, :, h]).view(np.uint16), fmt.v_bits, iters,
                                            group=fmt.group)
            n_bad += check_record(host[off:off + R], fmt.k_bits, fmt.v_bits, rk, rv, f"tile {t} head {h}",
                                  group=fmt.group)
    assert_code_rate(n_bad, T * hkv * 2 * 128 * 128, f"case {i}")


@pytest.mark.parametrize("i", range(24))
def test_random_append_steps(i):
    """Random format, batch and kv heads, lengths near tile boundaries and 1-4 append steps per case,
    with pages handed out by the host pool (reserved up front for the lengths after the last step) into
    a canary-filled cache.  After the steps: lengths and fp16 tails equal the oracle's append bit for bit,
    every tile that filled is a record matching the oracle's quantiser, no other page was written, and
    decode over the result matches the oracle."""
    rng = np.random.default_rng(4000 + i)
    name = FORMATS[rng.integers(len(FORMATS))]
    B = int(rng.integers(1, 9))
    hkv = int(rng.integers(1, 6))
    G = int(rng.choice([1, 4, 8]))
    steps = int(rng.integers(1, 5))
    lens0 = np.array([int(rng.integers(0, 6)) * 128 + int(rng.choice([125, 126, 127, 0, 64]))
                      for _ in range(B)], np.int32)
    print(f"case {i}: append {name} B {B} hkv {hkv} G {G} steps {steps} lens {lens0.tolist()}", flush=True)
    fmt = kv.format_parse(name)
    R = kv.record_bytes(fmt)
    stride = hkv * R
    maxp = int((lens0.max() + steps) // 128) + 1
    n_pool = B * maxp + 2
    pool = kv.PagePool(n_pool)
    pt = np.full((B, maxp), -1, np.int32)
    owned = np.zeros(B, np.int32)
    pool.reserve(lens0 + steps, pt, owned)
    assert (owned == (lens0 + steps) // 128).all()
    pt[pt < 0] = n_pool - 1                       # a page no sequence owns; never written
    full0 = lens0 // 128
    # the initial full pages: random tiles quantised by the GPU (their bytes are what both sides read)
    tiles = [(s, p) for s in range(B) for p in range(full0[s])]
    cache = torch.full((n_pool * stride,), 0xA5, dtype=torch.uint8, device="cuda")
    if tiles:
        kt = (rng.standard_normal((len(tiles), 128, hkv, 128)) * 1.5).astype(np.float16)
        vt = (rng.standard_normal((len(tiles), 128, hkv, 128)) * 1.5).astype(np.float16)
        dst = np.array([pt[s, p] for s, p in tiles], np.int32)
        kv.quantize_tiles(fmt, torch.from_numpy(kt).to("cuda"), torch.from_numpy(vt).to("cuda"),
                          torch.from_numpy(dst).to("cuda"), cache, stride)
    tails_k = (rng.standard_normal((B, hkv, 128, 128)) * 1.5).astype(np.float16)
    tails_v = (rng.standard_normal((B, hkv, 128, 128)) * 1.5).astype(np.float16)
    torch.cuda.synchronize()
    cache0 = cache.cpu().numpy()
    # oracle state (its append quantises in fp64; only the tails and lengths are compared bit for bit)
    o_lens, o_tk, o_tv, o_cache = lens0.copy(), tails_k.view(np.uint16).copy(), tails_v.view(np.uint16).copy(), \
        cache0.copy()
    g_lens = torch.from_numpy(lens0.copy()).to("cuda")
    g_tk = torch.from_numpy(tails_k.copy()).to("cuda")
    g_tv = torch.from_numpy(tails_v.copy()).to("cuda")
    g_pt = torch.from_numpy(pt).to("cuda")
    filled = []                                    # (seq, page index, tail contents at the fill)
    for st in range(steps):
        k_new = (rng.standard_normal((B, hkv, 128)) * 1.5).astype(np.float16)
        v_new = (rng.standard_normal((B, hkv, 128)) * 1.5).astype(np.float16)
        before = o_lens.copy()
        oracle.append_token(fmt.k_bits, fmt.v_bits, 8, k_new.view(np.uint16), v_new.view(np.uint16), o_lens, o_tk,
                            o_tv, pt, o_cache, stride, group=fmt.group)
        for s in range(B):
            if (before[s] + 1) % 128 == 0:
                filled.append((s, int(before[s] // 128), o_tk.view(np.float16)[s].copy(),
                               o_tv.view(np.float16)[s].copy()))
        kv.append_token(fmt, torch.from_numpy(k_new).to("cuda"), torch.from_numpy(v_new).to("cuda"), g_lens, g_tk,
                        g_tv, g_pt, cache, stride)
    torch.cuda.synchronize()
    assert np.array_equal(g_lens.cpu().numpy(), o_lens)
    assert np.array_equal(g_tk.cpu().numpy().view(np.uint16), o_tk)
    assert np.array_equal(g_tv.cpu().numpy().view(np.uint16), o_tv)
    host = cache.cpu().numpy()
    touched = set()
    n_bad = 0
    for s, p, tk_s, tv_s in filled:
        page = int(pt[s, p])
        touched.add(page)
        for h in range(hkv):
            off = page * stride + h * R
            rk = oracle.quantize_tile_debug(np.ascontiguousarray(tk_s[h]).view(np.uint16), fmt.k_bits, 8,
                                            group=fmt.group)
            rv = oracle.quantize_tile_debug(np.ascontiguousarray(tv_s[h]).view(np.uint16), fmt.v_bits, 8,
                                            group=fmt.group)
            n_bad += check_record(host[off:off + R], fmt.k_bits, fmt.v_bits, rk, rv, f"seq {s} page {p} head {h}",
                                  group=fmt.group)
    assert_code_rate(n_bad, max(1, len(filled)) * hkv * 2 * 128 * 128, f"case {i}")
    for page in range(n_pool):
        if page not in touched:
            assert np.array_equal(host[page * stride:(page + 1) * stride], cache0[page * stride:(page + 1) * stride]), \
                f"page {page} changed without a fill"
    # decode over the GPU's own cache and tails
    q = synth.gen_q(5000 + i, B, hkv * G)
    out = torch.empty(B, hkv * G, 128, dtype=torch.float16, device="cuda")
    ws = kv.decode_workspace(fmt, B, hkv * G, hkv, maxp, "cuda")
    sm = 0.08838834764831845
    kv.decode_attention(fmt, torch.from_numpy(q).to("cuda"), cache, stride, g_pt, g_lens, g_tk, g_tv, sm, out, ws,
                        hkv)
    torch.cuda.synchronize()
    _, ref = oracle.decode_attention(fmt.k_bits, fmt.v_bits, q.view(np.uint16), host, stride, pt, o_lens,
                                     g_tk.cpu().numpy().view(np.uint16), g_tv.cpu().numpy().view(np.uint16), sm, hkv,
                                     group=fmt.group)
    _compare(out.cpu().numpy(), ref, o_lens)
    pool.close()
