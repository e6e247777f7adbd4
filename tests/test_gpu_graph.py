"""HIP-graph capture of a serving step: append one token + decode, captured once and replayed.

The long-context workload (4 sequences x 131072 cached tokens, 8 query heads on 1 kv head, k4v2) is
set up twice from the same seeded K/V: one state stepped eagerly, one by replaying a graph captured
from the same two calls.  Pages come from the host page pool, reserved ahead for the length after the
last replayed step (the graph never returns to the host for pages).  Every sequence starts with 37
tokens in its fp16 tail, so the 91st step fills a tile and quantises it inside the replay.  Between
replays the test writes the next token's q/k/v into the captured input buffers with ordinary eager
copies and synchronises; each replay's output must equal the eager step's bit for bit, and so must the
cache, the tails and the lengths at the end.  No call in the step issues a memset, so nothing in the
graph depends on memset nodes."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_quantization_pipeline_amd as kv  # noqa: E402
from kv_cache_quantization_pipeline_amd import synth  # noqa: E402

DEV = "cuda"
STEPS = 128


class State:
    def __init__(self, fmt, B, hq, hkv, maxp, cache, pt, lens, tk, tv):
        self.fmt, self.B, self.hq, self.hkv = fmt, B, hq, hkv
        self.stride = hkv * kv.record_bytes(fmt)
        self.cache, self.pt, self.lens, self.tk, self.tv = cache, pt, lens, tk, tv
        self.q = torch.zeros(B, hq, 128, dtype=torch.float16, device=DEV)
        self.k_new = torch.zeros(B, hkv, 128, dtype=torch.float16, device=DEV)
        self.v_new = torch.zeros_like(self.k_new)
        self.out = torch.zeros(B, hq, 128, dtype=torch.float16, device=DEV)
        self.ws = kv.decode_workspace(fmt, B, hq, hkv, maxp, DEV)

    def step(self):
        kv.append_token(self.fmt, self.k_new, self.v_new, self.lens, self.tk, self.tv, self.pt, self.cache,
                        self.stride)
        kv.decode_attention(self.fmt, self.q, self.cache, self.stride, self.pt, self.lens, self.tk, self.tv,
                            1.0 / math.sqrt(128), self.out, self.ws, self.hkv)


def test_graph_replay_of_append_and_decode_matches_eager():
    w = synth.WORKLOADS["decode_long_b4_ctx128k"]
    fmt = kv.format_parse("kvarn_k4v2_g128")
    B, hq, hkv, ctx = w["batch"], w["n_q_heads"], w["n_kv_heads"], w["ctx"]
    tail0 = 37
    print(f"case: graph replay B{B} ctx {ctx}+{tail0} hq {hq} hkv {hkv}, {STEPS} steps", flush=True)
    full0 = ctx // 128
    maxp = (ctx + tail0 + STEPS) // 128 + 1
    R = kv.record_bytes(fmt)
    stride = hkv * R

    # pages from the host pool: the initial full tiles, then every tile that fills in the replayed steps
    pool = kv.PagePool(B * maxp)
    pt_host = np.full((B, maxp), -1, np.int32)
    owned = np.zeros(B, np.int32)
    pool.reserve(np.full(B, ctx + tail0, np.int32), pt_host, owned)
    assert (owned == full0).all()
    init_pages = pt_host[:, :full0].copy()
    pool.reserve(np.full(B, ctx + tail0 + STEPS, np.int32), pt_host, owned)
    assert (owned == (ctx + tail0 + STEPS) // 128).all()
    assert pool.num_free == B * maxp - B * owned[0]

    g = torch.Generator(device=DEV)
    g.manual_seed(w["seed"])
    cache = torch.zeros(B * maxp * stride, dtype=torch.uint8, device=DEV)
    for s in range(B):
        kk = torch.randn(full0, 128, hkv, 128, generator=g, device=DEV).half()
        vv = torch.randn(full0, 128, hkv, 128, generator=g, device=DEV).half()
        kv.quantize_tiles(fmt, kk, vv, torch.from_numpy(init_pages[s].copy()).to(DEV), cache, stride)
    tk = torch.zeros(B, hkv, 128, 128, dtype=torch.float16, device=DEV)
    tv = torch.zeros_like(tk)
    tk[:, :, :tail0] = torch.randn(B, hkv, tail0, 128, generator=g, device=DEV).half()
    tv[:, :, :tail0] = torch.randn(B, hkv, tail0, 128, generator=g, device=DEV).half()
    lens = torch.full((B,), ctx + tail0, dtype=torch.int32, device=DEV)
    ptd = torch.from_numpy(pt_host).to(DEV)
    torch.cuda.synchronize()

    eager = State(fmt, B, hq, hkv, maxp, cache, ptd, lens, tk, tv)
    graphed = State(fmt, B, hq, hkv, maxp, cache.clone(), ptd.clone(), lens.clone(), tk.clone(), tv.clone())

    qs = torch.randn(STEPS, B, hq, 128, generator=g, device=DEV).half()
    ks = (torch.randn(STEPS, B, hkv, 128, generator=g, device=DEV) * 1.5).half()
    vs = (torch.randn(STEPS, B, hkv, 128, generator=g, device=DEV) * 1.5).half()

    # capture on a side stream (the calls issue on the capturing stream; nothing runs during capture)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            graphed.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(graphed.lens, eager.lens), "capture must not run the step"

    for i in range(STEPS):
        for st in (eager, graphed):
            st.q.copy_(qs[i])
            st.k_new.copy_(ks[i])
            st.v_new.copy_(vs[i])
        eager.step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed.out, eager.out), f"replay {i}: output differs from the eager step"
        assert torch.equal(graphed.lens, eager.lens), f"replay {i}: lengths differ"
    assert eager.lens.cpu().tolist() == [ctx + tail0 + STEPS] * B
    assert torch.equal(graphed.tk, eager.tk) and torch.equal(graphed.tv, eager.tv)
    assert torch.equal(graphed.cache, eager.cache)
    # the tile that filled at step 91 was written into the page the pool reserved for it
    filled = pt_host[:, full0]
    host = eager.cache.view(B * maxp, stride).cpu()
    for s in range(B):
        assert host[int(filled[s])].any(), f"seq {s}: filled tile's page {filled[s]} is empty"
    assert torch.isfinite(eager.out.float()).all()
