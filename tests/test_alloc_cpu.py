"""The library's block allocator and append-slot mapping (host only): the
free-and-reuse pool of the nanoserve "Day 17" page ("What I added today",
"Post angle"), checked against plain Python bookkeeping."""
import numpy as np
import pytest

import paged_kv_cache_13_amd as pkv


def test_seed_zero_hands_blocks_out_in_order_and_a_seed_shuffles():
    a = pkv.BlockAllocator(12, seed=0)
    assert list(a.allocate(5)) == [0, 1, 2, 3, 4]
    b = pkv.BlockAllocator(12, seed=99)
    got = b.allocate(12)
    assert sorted(got) == list(range(12)) and list(got) != list(range(12))
    c = pkv.BlockAllocator(12, seed=99)
    assert list(c.allocate(12)) == list(got)  # seeded: reproducible


def test_exhaustion_takes_nothing_and_frees_are_reused():
    a = pkv.BlockAllocator(6, seed=3)
    x = a.allocate(4)
    with pytest.raises(pkv.KVCacheExhausted):
        a.allocate(3)
    assert a.num_free == 2
    a.free(x[:2])
    assert a.num_free == 4
    y = a.allocate(2)
    assert set(y) == set(x[:2])  # the freed blocks come straight back


@pytest.mark.parametrize("bad", [[-1], [6], [0, 0]])
def test_bad_frees_are_refused_whole(bad):
    a = pkv.BlockAllocator(6, seed=0)
    a.allocate(3)  # blocks 0, 1, 2 in use
    with pytest.raises(pkv.PkvError):
        a.free(bad + [1])
    assert a.num_free == 3
    a.free([1])
    with pytest.raises(pkv.PkvError):  # a double free
        a.free([1])
    assert a.num_free == 4


def test_append_slots_cross_block_boundaries():
    a = pkv.BlockAllocator(20, seed=5)
    bs = 4
    row = np.full(6, -1, dtype=np.int32)
    s1 = a.append_slots(row, bs, 0, 6)         # two blocks
    s2 = a.append_slots(row, bs, 6, 1)         # still in the second block
    s3 = a.append_slots(row, bs, 7, 2)         # takes a third
    assert a.num_free == 17
    slots = np.concatenate([s1, s2, s3])
    want = [int(row[p // bs]) * bs + p % bs for p in range(9)]
    assert list(slots) == want
    assert len(set(row[:3])) == 3 and (row[3:] == -1).all()
    with pytest.raises(pkv.PkvError):          # beyond the row's 6 blocks
        a.append_slots(row, bs, 9, 16)
    small = pkv.BlockAllocator(2, seed=0)
    r2 = np.full(4, -1, dtype=np.int32)
    small.append_slots(r2, bs, 0, 8)
    with pytest.raises(pkv.KVCacheExhausted):
        small.append_slots(r2, bs, 8, 1)
    assert (r2[2:] == -1).all() and small.num_free == 0


def test_churn_keeps_the_books():
    # sequences start, grow and finish at random; no block is ever held by two
    # live sequences, and every block is free or held by exactly one
    rng = np.random.default_rng(0)
    nb, bs, width, slots_n = 64, 8, 16, 10
    a = pkv.BlockAllocator(nb, seed=11)
    tables = np.full((slots_n, width), -1, dtype=np.int32)
    lens = np.zeros(slots_n, dtype=np.int64)
    exhausted = 0
    for step in range(2000):
        r = int(rng.integers(slots_n))
        if lens[r] and rng.random() < 0.15:  # finish: give the blocks back
            held = -(-int(lens[r]) // bs)
            a.free(tables[r, :held])
            tables[r] = -1
            lens[r] = 0
            continue
        k = int(rng.integers(1, 12))
        if lens[r] + k > width * bs:
            continue
        try:
            a.append_slots(tables[r], bs, int(lens[r]), k)
            lens[r] += k
        except pkv.KVCacheExhausted:
            exhausted += 1
        held = [tables[i, :-(-int(lens[i]) // bs)] for i in range(slots_n)]
        flat = np.concatenate(held)
        assert len(flat) == len(set(flat.tolist()))
        assert a.num_free + len(flat) == nb
    assert exhausted > 0  # the pool did run out, and recovered
