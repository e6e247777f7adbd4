"""GPU parity of chunked prefill attention (kvarn_prefill_attention) against the oracle attending
causally over the same (GPU-written) cache bytes and fp16 tails, through the C-ABI."""
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
SENTINEL = 0x7BFF   # fp16 65504: rows the call must not write keep it


class Prefill:
    """Pages quantised on the GPU, fp16 tails and a chunk of queries per sequence."""

    def __init__(self, name, lens, q_lens, hkv, hq, seed, max_q=None, pool_extra=2):
        self.fmt = kv.format_parse(name)
        self.lens = np.asarray(lens, np.int32)
        self.q_lens = np.asarray(q_lens, np.int32)
        self.B = len(lens)
        self.hkv, self.hq = hkv, hq
        self.max_q = int(max_q or max(1, int(self.q_lens.max())))
        self.R = kv.record_bytes(self.fmt)
        self.stride = hkv * self.R
        full = self.lens // 128
        self.max_pages = max(1, int(full.max()) + 1)
        n_full = int(full.sum())
        self.n_pool = n_full + pool_extra
        rng = np.random.default_rng(seed)
        perm = rng.permutation(self.n_pool).astype(np.int32)
        self.pt = np.full((self.B, self.max_pages), perm[-1], np.int32)
        k_all, v_all = synth.gen_kv(seed, max(n_full, 1) * 128, hkv)
        kt = synth.tiles_view(k_all)[:n_full]
        vt = synth.tiles_view(v_all)[:n_full]
        dst, c = [], 0
        for s in range(self.B):
            for p in range(full[s]):
                self.pt[s, p] = perm[c]
                dst.append(perm[c])
                c += 1
        self.cache = torch.zeros(self.n_pool * self.stride, dtype=torch.uint8, device=DEV)
        if n_full:
            kv.quantize_tiles(self.fmt, torch.from_numpy(np.ascontiguousarray(kt)).to(DEV),
                              torch.from_numpy(np.ascontiguousarray(vt)).to(DEV),
                              torch.from_numpy(np.asarray(dst, np.int32)).to(DEV), self.cache, self.stride)
        self.tail_k = (rng.standard_normal((self.B, hkv, 128, 128)) * 1.5).astype(np.float16)
        self.tail_v = (rng.standard_normal((self.B, hkv, 128, 128)) * 1.5).astype(np.float16)
        self.q = rng.standard_normal((self.B, self.max_q, hq, 128)).astype(np.float16)
        self.sm = 1.0 / math.sqrt(128)

    def run_gpu(self):
        out = torch.full((self.B, self.max_q, self.hq, 128), SENTINEL, dtype=torch.int16,
                         device=DEV).view(torch.float16)
        kv.prefill_attention(self.fmt, torch.from_numpy(self.q).to(DEV), torch.from_numpy(self.q_lens).to(DEV),
                             self.cache, self.stride, torch.from_numpy(self.pt).to(DEV),
                             torch.from_numpy(self.lens).to(DEV), torch.from_numpy(self.tail_k).to(DEV),
                             torch.from_numpy(self.tail_v).to(DEV), self.sm, out, self.hkv)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def run_oracle(self, seqs=None):
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        host = self.cache.cpu().numpy()
        _, o64 = oracle.prefill_attention(self.fmt.k_bits, self.fmt.v_bits, self.q[seqs].view(np.uint16),
                                          self.q_lens[seqs], host, self.stride, self.pt[seqs], self.lens[seqs],
                                          self.tail_k[seqs].view(np.uint16), self.tail_v[seqs].view(np.uint16),
                                          self.sm, self.hkv, group=self.fmt.group)
        return o64

    def compare(self, gpu, ref, seqs=None):
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        worst = 0.0
        for j, s in enumerate(seqs):
            n = self.q_lens[s]
            assert np.all(gpu[s, n:].view(np.uint16) == SENTINEL), f"seq {s}: rows past q_lens written"
            for i in range(n):
                for h in range(self.hq):
                    e = rel_l2(gpu[s, i, h].astype(np.float64), ref[j, i, h])
                    worst = max(worst, e)
                    assert e <= DECODE_REL_L2, f"seq {s} query {i} head {h}: rel L2 {e:.3g}"
        return worst


LENS = [326, 128, 5, 0, 1029, 640, 127, 256]
QLENS = [40, 128, 5, 0, 300, 64, 127, 1]     # chunk across page + tail, whole page, tail only, empty, ...


@pytest.mark.parametrize("name", [f"kvarn_k{kb}v{vb}_g128" for kb in (2, 4, 8) for vb in (2, 4, 8)])
@pytest.mark.parametrize("G", [1, 8, 16])
def test_prefill_ragged_small(name, G):
    st = Prefill(name, LENS, QLENS, hkv=2, hq=2 * G, seed=31)
    print(f"worst rel L2 {st.compare(st.run_gpu(), st.run_oracle()):.3g}")


GROUPED = [f"kvarn_k{kb}v{vb}_g{g}" for g in (64, 32) for kb, vb in ((4, 2), (2, 8), (8, 4), (8, 8))]


@pytest.mark.parametrize("name", GROUPED)
@pytest.mark.parametrize("G", [1, 8, 16])
def test_prefill_grouped_ragged_small(name, G):
    """Quantisation groups of 64 and 32 channels: per-group K dot products and scales, per-group V
    weights and zero points."""
    st = Prefill(name, LENS, QLENS, hkv=2, hq=2 * G, seed=35)
    print(f"worst rel L2 {st.compare(st.run_gpu(), st.run_oracle()):.3g}")


def test_prefill_grouped_long_context_sampled():
    lens = [4096 + 130, 4096 + 77]
    st = Prefill("kvarn_k4v2_g32", lens, [130, 77], hkv=2, hq=16, seed=36)
    st.compare(st.run_gpu(), st.run_oracle())


@pytest.mark.parametrize("G", [2, 4])
def test_prefill_gqa_k4v2(G):
    st = Prefill("kvarn_k4v2_g128", LENS, QLENS, hkv=3, hq=3 * G, seed=32, max_q=301)
    st.compare(st.run_gpu(), st.run_oracle())


def test_prefill_last_query_equals_decode():
    """The chunk's last query sees the whole sequence: the decode kernel's output for that query."""
    st = Prefill("kvarn_k4v2_g128", [1029, 326, 640], [77, 40, 64], hkv=2, hq=16, seed=33)
    pre = st.run_gpu()
    q_last = np.stack([st.q[s, st.q_lens[s] - 1] for s in range(st.B)])
    ws = kv.decode_workspace(st.fmt, st.B, st.hq, st.hkv, st.max_pages, DEV)
    dec = torch.empty(st.B, st.hq, 128, dtype=torch.float16, device=DEV)
    kv.decode_attention(st.fmt, torch.from_numpy(q_last).to(DEV), st.cache, st.stride,
                        torch.from_numpy(st.pt).to(DEV), torch.from_numpy(st.lens).to(DEV),
                        torch.from_numpy(st.tail_k).to(DEV), torch.from_numpy(st.tail_v).to(DEV), st.sm, dec, ws,
                        st.hkv)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    for s in range(st.B):
        for h in range(st.hq):
            assert rel_l2(pre[s, st.q_lens[s] - 1, h].astype(np.float64), dec[s, h].astype(np.float64)) <= 2e-3


def test_prefill_chunk_at_long_context_sampled():
    """A 256-token chunk at 8K context, 16 query / 2 kv heads (the rows of 8 blocks per kv head), on
    two sequences in full against the oracle."""
    lens = [8192 + 256, 8192 + 200]
    st = Prefill("kvarn_k4v2_g128", lens, [256, 200], hkv=2, hq=16, seed=34)
    out = st.run_gpu()
    assert np.all(np.isfinite(out[0, :256].astype(np.float32)))
    st.compare(out, st.run_oracle())
