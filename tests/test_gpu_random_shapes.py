"""Seeded random shapes: decode and chunked prefill against the oracle over formats, query heads per kv
head, kv-head counts, ragged lengths (page boundaries, empty sequences, tails of every size) and page
tables wider than the lengths need (so the split counts, the tail-split mode and the merge shape vary
from case to case).  Every case prints its parameters before it runs."""
import numpy as np
import pytest

from test_gpu_decode import Setup, _compare
from test_gpu_prefill import Prefill

pytestmark = pytest.mark.gpu

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
