"""The host-side 128-token page pool (kvarn_page_pool_*): page accounting, all-or-nothing batch
reservation, rejected releases, and a randomised run against a plain Python model of the same rules.
Host code only; runs without a GPU."""
import ctypes
import threading

import numpy as np
import pytest

import kv_cache_quantization_pipeline_amd as kv


def _state(pool, pt, own):
    return pool.num_free, pt.copy(), own.copy()


def test_create_rejects_bad_arguments_and_null_pool_calls():
    L = kv.lib()
    h = ctypes.c_void_p()
    assert L.kvarn_page_pool_create(-1, ctypes.byref(h)) == kv.KVARN_E_INVALID_ARG
    assert L.kvarn_page_pool_create(4, None) == kv.KVARN_E_INVALID_ARG
    assert L.kvarn_page_pool_num_free(None) == -1
    L.kvarn_page_pool_destroy(None)
    assert L.kvarn_page_pool_reserve(None, 1, None, None, 1, None) == kv.KVARN_E_INVALID_ARG
    own = ctypes.c_int32(0)
    assert L.kvarn_page_pool_release(None, None, 1, ctypes.byref(own)) == kv.KVARN_E_INVALID_ARG
    assert kv.PagePool(0).num_free == 0


def test_pages_only_for_full_tiles_and_ascending_ids():
    pool = kv.PagePool(16)
    pt = np.full((4, 5), -1, np.int32)
    own = np.zeros(4, np.int32)
    pool.reserve(np.array([0, 127, 128, 3 * 128 + 5], np.int32), pt, own)
    assert own.tolist() == [0, 0, 1, 3]
    assert pt[2, 0] == 0 and pt[3, :3].tolist() == [1, 2, 3]
    assert (pt[:2] == -1).all() and (pt[2, 1:] == -1).all() and (pt[3, 3:] == -1).all()
    assert pool.num_free == 12
    # a shorter length keeps the pages; the same length takes none
    pool.reserve(np.array([0, 0, 0, 3 * 128], np.int32), pt, own)
    assert own.tolist() == [0, 0, 1, 3] and pool.num_free == 12


def test_reserve_before_the_append_that_fills_a_tile():
    """kvarn_append_token at length L quantises tile L/128 into page_table[L/128] when (L+1) % 128 == 0:
    reserving for L + 1 gives that entry a page exactly then."""
    pool = kv.PagePool(8)
    pt = np.full((1, 4), -1, np.int32)
    own = np.zeros(1, np.int32)
    for L in range(0, 3 * 128):
        pool.reserve(np.array([L + 1], np.int32), pt, own)
        fills = (L + 1) % 128 == 0
        assert own[0] == (L + 1) // 128
        if fills:
            assert pt[0, L // 128] >= 0
        assert (pt[0, own[0]:] == -1).all()


def test_out_of_pages_changes_nothing():
    pool = kv.PagePool(5)
    pt = np.full((3, 4), -1, np.int32)
    own = np.zeros(3, np.int32)
    pool.reserve(np.array([256, 0, 0], np.int32), pt, own)
    before = _state(pool, pt, own)
    with pytest.raises(kv.KvarnError) as e:
        pool.reserve(np.array([256, 256, 256], np.int32), pt, own)  # needs 0 + 2 + 2 > 3 free
    assert e.value.status == kv.KVARN_E_OUT_OF_PAGES
    after = _state(pool, pt, own)
    assert before[0] == after[0] and (before[1] == after[1]).all() and (before[2] == after[2]).all()
    pool.reserve(np.array([256, 256, 0], np.int32), pt, own)  # 2 of the 3 free pages
    assert pool.num_free == 1


@pytest.mark.parametrize("new_lens,owned", [
    ([5 * 128], [0]),        # needs 5 entries, the row holds 4
    ([-1], [0]),             # negative length
    ([0], [5]),              # more owned than the row holds
    ([0], [-1]),             # negative count
])
def test_invalid_reservations_change_nothing(new_lens, owned):
    pool = kv.PagePool(16)
    pt = np.full((1, 4), -1, np.int32)
    own = np.asarray(owned, np.int32)
    before = _state(pool, pt, own)
    with pytest.raises(kv.KvarnError) as e:
        pool.reserve(np.asarray(new_lens, np.int32), pt, own)
    assert e.value.status == kv.KVARN_E_INVALID_ARG
    after = _state(pool, pt, own)
    assert before[0] == after[0] and (before[1] == after[1]).all() and (before[2] == after[2]).all()


def test_release_returns_pages_and_rejects_foreign_or_repeated_ids():
    pool = kv.PagePool(6)
    pt = np.full((2, 3), -1, np.int32)
    own = np.zeros(2, np.int32)
    pool.reserve(np.array([3 * 128, 2 * 128], np.int32), pt, own)
    assert pool.num_free == 1
    row1 = pt[1].copy()
    pool.release(pt, own, 1)
    assert own.tolist() == [3, 0] and (pt[1] == -1).all() and pool.num_free == 3
    # releasing the same ids again (a stale copy of the row) is rejected
    stale = row1.copy()
    cnt = np.array([2], np.int32)
    with pytest.raises(kv.KvarnError):
        pool.release(stale, cnt, 0)
    assert cnt[0] == 2 and (stale == row1).all() and pool.num_free == 3
    # an id repeated within one row, and an id outside the pool, are rejected
    dup = np.array([pt[0, 0], pt[0, 0], -1], np.int32)
    with pytest.raises(kv.KvarnError):
        pool.release(dup, np.array([2], np.int32), 0)
    with pytest.raises(kv.KvarnError):
        pool.release(np.array([6, -1, -1], np.int32), np.array([1], np.int32), 0)
    assert pool.num_free == 3
    # freed pages are handed out again, most recently freed first
    pool.reserve(np.array([3 * 128, 128], np.int32), pt, own)
    assert pt[1, 0] == row1[0]


def _check_invariants(pool, pt, own, num_pages):
    ids = np.concatenate([pt[s, :own[s]] for s in range(pt.shape[0])])
    assert len(np.unique(ids)) == len(ids), "a page owned twice"
    assert ((ids >= 0) & (ids < num_pages)).all()
    assert pool.num_free == num_pages - len(ids)


def test_randomised_against_a_plain_model():
    rng = np.random.default_rng(5)
    num_pages, B, maxp = 40, 6, 9
    pool = kv.PagePool(num_pages)
    pt = np.full((B, maxp), -1, np.int32)
    own = np.zeros(B, np.int32)
    lens = np.zeros(B, np.int64)
    for _ in range(600):
        if rng.random() < 0.15:
            s = int(rng.integers(B))
            pool.release(pt, own, s)
            lens[s] = 0
        else:
            grow = rng.integers(0, 200, B) * (rng.random(B) < 0.5)
            new = np.minimum(lens + grow, maxp * 128 + 127).astype(np.int32)
            want = np.maximum(new // 128, own)
            need = int((want - own).sum())
            free = pool.num_free
            if need > free:
                with pytest.raises(kv.KvarnError) as e:
                    pool.reserve(new, pt, own)
                assert e.value.status == kv.KVARN_E_OUT_OF_PAGES
            else:
                pool.reserve(new, pt, own)
                assert (own == want).all()
                lens = np.maximum(lens, new)
        _check_invariants(pool, pt, own, num_pages)


def test_threads_share_one_pool():
    num_pages, T, maxp = 64, 4, 8
    pool = kv.PagePool(num_pages)
    errors = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        pt = np.full((1, maxp), -1, np.int32)
        own = np.zeros(1, np.int32)
        held = []
        try:
            for _ in range(300):
                try:
                    pool.reserve(np.array([int(rng.integers(0, maxp * 128))], np.int32), pt, own)
                except kv.KvarnError as e:
                    assert e.status == kv.KVARN_E_OUT_OF_PAGES
                held.append(pt[0, :own[0]].copy())
                if rng.random() < 0.3:
                    pool.release(pt, own, 0)
            pool.release(pt, own, 0)
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(T)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors
    assert pool.num_free == num_pages
