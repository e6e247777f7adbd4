"""GPU parity at K/V magnitudes far from the synthetic N(0, 1) range: K and V scaled by 2^-8 and 2^7
(together and separately), and tiles whose per-token scales span four decades.  For each case the GPU
quantiser's records are checked against the oracle's (scales, codes, layout), then decode and chunked
prefill against the oracle attending over the GPU's own cache bytes, per (sequence, query head) or
(query row, head) at the decode tolerance.  Small V magnitudes with 8-bit codes put the softmax
weights p_t s'_t far below fp16's normal range unless the kernels rescale them, large ones near its
top; large K magnitudes give large logits."""
import math

import numpy as np
import pytest

import oracle
from kv_cache_quantization_pipeline_amd import synth
from parity import DECODE_REL_L2, assert_code_rate, check_record, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_quantization_pipeline_amd as kv  # noqa: E402

DEV = "cuda"
FP16_MAX = 65000.0


def _scaled(x16, scale, token_span, rng):
    """fp16 x [n_tok, Hkv, 128] times `scale`, and (token_span) times 10^(-2 + 4u) per token, u ~ U[0, 1];
    clipped into fp16's range."""
    x = x16.astype(np.float32) * np.float32(scale)
    if token_span:
        x *= (10.0 ** (-2.0 + 4.0 * rng.random((x.shape[0], x.shape[1], 1)))).astype(np.float32)
    return np.clip(x, -FP16_MAX, FP16_MAX).astype(np.float16)


class ScaledCache:
    def __init__(self, name, lens, hkv, hq, seed, ks, vs, token_span=False):
        self.fmt = kv.format_parse(name)
        self.lens = np.asarray(lens, np.int32)
        self.B, self.hkv, self.hq = len(lens), hkv, hq
        self.R = kv.record_bytes(self.fmt)
        self.stride = hkv * self.R
        full = self.lens // 128
        self.max_pages = int(full.max()) + 1
        n_full = int(full.sum())
        rng = np.random.default_rng(seed)
        perm = rng.permutation(n_full + 1).astype(np.int32)
        self.pt = np.full((self.B, self.max_pages), perm[-1], np.int32)
        k, v = synth.gen_kv(seed, n_full * 128, hkv)
        k, v = _scaled(k, ks, token_span, rng), _scaled(v, vs, token_span, rng)
        self.kt, self.vt = synth.tiles_view(k), synth.tiles_view(v)
        self.dst = []
        c = 0
        for s in range(self.B):
            for p in range(full[s]):
                self.pt[s, p] = perm[c]
                self.dst.append(perm[c])
                c += 1
        self.cache = torch.zeros((n_full + 1) * self.stride, dtype=torch.uint8, device=DEV)
        kv.quantize_tiles(self.fmt, torch.from_numpy(np.ascontiguousarray(self.kt)).to(DEV),
                          torch.from_numpy(np.ascontiguousarray(self.vt)).to(DEV),
                          torch.from_numpy(np.asarray(self.dst, np.int32)).to(DEV), self.cache, self.stride)
        tk = (rng.standard_normal((self.B * 128, hkv, 128)) * 1.5).astype(np.float16)
        tv = (rng.standard_normal((self.B * 128, hkv, 128)) * 1.5).astype(np.float16)
        self.tail_k = _scaled(tk, ks, token_span, rng).reshape(self.B, 128, hkv, 128).transpose(0, 2, 1, 3).copy()
        self.tail_v = _scaled(tv, vs, token_span, rng).reshape(self.B, 128, hkv, 128).transpose(0, 2, 1, 3).copy()
        self.q = synth.gen_q(seed, self.B, hq)
        self.sm = 1.0 / math.sqrt(128)
        torch.cuda.synchronize()
        self.host = self.cache.cpu().numpy()

    def check_records(self):
        n_bad = 0
        f = self.fmt
        for i, page in enumerate(self.dst):
            for h in range(self.hkv):
                rk = oracle.quantize_tile_debug(np.ascontiguousarray(self.kt[i, :, h, :]).view(np.uint16), f.k_bits,
                                                f.sinkhorn_iters, group=f.group)
                rv = oracle.quantize_tile_debug(np.ascontiguousarray(self.vt[i, :, h, :]).view(np.uint16), f.v_bits,
                                                f.sinkhorn_iters, group=f.group)
                off = int(page) * self.stride + h * self.R
                n_bad += check_record(self.host[off:off + self.R], f.k_bits, f.v_bits, rk, rv, f"tile {i} head {h}",
                                      group=f.group)
        assert_code_rate(n_bad, len(self.dst) * self.hkv * 2 * 128 * 128)

    def decode(self):
        out = torch.empty(self.B, self.hq, 128, dtype=torch.float16, device=DEV)
        ws = kv.decode_workspace(self.fmt, self.B, self.hq, self.hkv, self.max_pages, DEV)
        kv.decode_attention(self.fmt, torch.from_numpy(self.q).to(DEV), self.cache, self.stride,
                            torch.from_numpy(self.pt).to(DEV), torch.from_numpy(self.lens).to(DEV),
                            torch.from_numpy(self.tail_k).to(DEV), torch.from_numpy(self.tail_v).to(DEV), self.sm,
                            out, ws, self.hkv)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got.astype(np.float32)))
        _, ref = oracle.decode_attention(self.fmt.k_bits, self.fmt.v_bits, self.q.view(np.uint16), self.host,
                                         self.stride, self.pt, self.lens, self.tail_k.view(np.uint16),
                                         self.tail_v.view(np.uint16), self.sm, self.hkv, group=self.fmt.group)
        worst = 0.0
        for s in range(self.B):
            for h in range(self.hq):
                e = rel_l2(got[s, h].astype(np.float64), ref[s, h])
                worst = max(worst, e)
                assert e <= DECODE_REL_L2, f"decode seq {s} head {h}: rel L2 {e:.3g}"
        return worst

    def prefill(self, q_lens):
        q_lens = np.asarray(q_lens, np.int32)
        max_q = int(q_lens.max())
        rng = np.random.default_rng(7)
        q = rng.standard_normal((self.B, max_q, self.hq, 128)).astype(np.float16)
        out = torch.zeros(self.B, max_q, self.hq, 128, dtype=torch.float16, device=DEV)
        kv.prefill_attention(self.fmt, torch.from_numpy(q).to(DEV), torch.from_numpy(q_lens).to(DEV), self.cache,
                             self.stride, torch.from_numpy(self.pt).to(DEV), torch.from_numpy(self.lens).to(DEV),
                             torch.from_numpy(self.tail_k).to(DEV), torch.from_numpy(self.tail_v).to(DEV), self.sm,
                             out, self.hkv)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        _, ref = oracle.prefill_attention(self.fmt.k_bits, self.fmt.v_bits, q.view(np.uint16), q_lens, self.host,
                                          self.stride, self.pt, self.lens, self.tail_k.view(np.uint16),
                                          self.tail_v.view(np.uint16), self.sm, self.hkv, group=self.fmt.group)
        worst = 0.0
        for s in range(self.B):
            for i in range(q_lens[s]):
                for h in range(self.hq):
                    e = rel_l2(got[s, i, h].astype(np.float64), ref[s, i, h])
                    worst = max(worst, e)
                    assert e <= DECODE_REL_L2, f"prefill seq {s} query {i} head {h}: rel L2 {e:.3g}"
        return worst


CASES = [
    ("both x2^-8", 2.0 ** -8, 2.0 ** -8, False),
    ("both x2^7", 2.0 ** 7, 2.0 ** 7, False),
    ("V x2^-8", 1.0, 2.0 ** -8, False),
    ("K x2^-8, V x2^7", 2.0 ** -8, 2.0 ** 7, False),
    ("token scales over 1e-2..1e2", 1.0, 1.0, True),
]


@pytest.mark.parametrize("name", ["kvarn_k4v2_g128", "kvarn_k4v8_g128", "kvarn_k8v8_g128"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_quantize_decode_prefill_at_extreme_scales(name, case):
    _, ks, vs, span = case
    print(f"case: {name} {case[0]}", flush=True)
    c = ScaledCache(name, [1029, 300, 700 + 77], hkv=2, hq=16, seed=51, ks=ks, vs=vs, token_span=span)
    c.check_records()
    wd = c.decode()
    wp = c.prefill([40, 128, 77])
    print(f"{name} {case[0]}: decode worst rel L2 {wd:.3g}, prefill {wp:.3g}")
