"""The KV block manager (dec_pool_*), host only: the pool rules of "Candle model runner" section
2.2 (references, prefix index, LRU cache of released full blocks) as its tests name them:
capacity is all-or-nothing, references balance, full blocks register, release caches, lookup
reacquires, the oldest cached block is evicted first, a pool without blocks is refused."""

import pytest

from decoder_forward_pass_amd import binding as B

FREE, USED, CACHED = B.DEC_BLOCK_FREE, B.DEC_BLOCK_USED, B.DEC_BLOCK_CACHED


def pool(n=4, bt=16, cache=True):
    return B.BlockPool(n, bt, cache)


def test_rejects_zero_capacity():
    with pytest.raises(B.DecError) as e:
        B.BlockPool(0, 16)
    assert e.value.code == B.DEC_E_ARG


def test_capacity_is_all_or_nothing():
    p = pool(4)
    a = p.alloc(3)
    assert a == [0, 1, 2] and p.counts() == (1, 3, 0)
    with pytest.raises(B.DecError) as e:
        p.alloc(2)
    assert e.value.code == B.DEC_E_CAPACITY
    assert p.counts() == (1, 3, 0)  # the failed call took nothing
    assert p.alloc(1) == [3]


def test_references_balance():
    p = pool(2)
    (i,) = p.alloc(1)
    p.retain(i)
    assert p.info(i)[:2] == (USED, 2)
    p.release(i)
    assert p.info(i)[:2] == (USED, 1)
    p.release(i)
    assert p.info(i)[0] == FREE and p.counts() == (2, 0, 0)
    for bad in (p.release, p.retain):
        with pytest.raises(B.DecError) as e:
            bad(i)  # not allocated
        assert e.value.code == B.DEC_E_BLOCK
    with pytest.raises(B.DecError):
        p.retain(7)  # outside the pool


def test_only_full_blocks_register_and_release_caches_them():
    p = pool(3, bt=4)
    i, j = p.alloc(2)
    p.set_fill(i, 3)
    with pytest.raises(B.DecError) as e:
        p.register(i, 11)
    assert e.value.code == B.DEC_E_ARG
    p.set_fill(i, 4)
    assert p.register(i, 11) == i
    with pytest.raises(B.DecError):
        p.set_fill(i, 2)  # a registered block stays full
    with pytest.raises(B.DecError):
        p.set_fill(j, 5)  # beyond block_tokens
    p.release(i)
    assert p.info(i)[0] == CACHED and p.counts() == (1, 1, 1)
    # lookup reacquires the cached block with one reference
    assert p.lookup(11) == i
    assert p.info(i)[:2] == (USED, 1) and p.counts() == (1, 2, 0)
    # a second lookup of a used block adds a reference
    assert p.lookup(11) == i and p.info(i)[1] == 2
    assert p.lookup(12) == -1


def test_a_key_keeps_its_first_block():
    p = pool(3, bt=2)
    i, j = p.alloc(2)
    for b in (i, j):
        p.set_fill(b, 2)
    assert p.register(i, 5) == i
    assert p.register(j, 5) == i  # already indexed to i
    p.release(j)
    assert p.info(j)[0] == FREE  # j was never registered: freed, not cached


def test_exhausted_allocation_evicts_the_oldest_cached_block():
    p = pool(3, bt=1)
    ids = p.alloc(3)
    for n, b in enumerate(ids):
        p.set_fill(b, 1)
        p.register(b, 100 + n)
    for b in ids:  # released oldest first: 0, 1, 2
        p.release(b)
    assert p.counts() == (0, 0, 3)
    (x,) = p.alloc(1)
    assert x == ids[0]  # the oldest cached block
    assert p.lookup(100) == -1  # its key left the index
    assert p.lookup(101) == ids[1] and p.lookup(102) == ids[2]  # the newer ones stay
    # reacquired blocks leave the LRU: a further allocation has no room
    with pytest.raises(B.DecError) as e:
        p.alloc(1)
    assert e.value.code == B.DEC_E_CAPACITY


def test_without_prefix_caching_released_blocks_are_freed():
    p = pool(2, bt=1, cache=False)
    (i,) = p.alloc(1)
    p.set_fill(i, 1)
    p.register(i, 9)
    p.release(i)
    assert p.info(i)[0] == FREE and p.lookup(9) == -1


def test_prefix_key_names_the_whole_prefix():
    k1 = B.dec_prefix_key(0, [1, 2, 3, 4])
    assert k1 == B.dec_prefix_key(0, [1, 2, 3, 4])
    assert k1 != B.dec_prefix_key(0, [1, 2, 4, 3])  # order matters
    assert B.dec_prefix_key(k1, [5, 6]) != B.dec_prefix_key(B.dec_prefix_key(0, [9, 9, 9, 9]), [5, 6])
    assert B.dec_prefix_key(0, []) != B.dec_prefix_key(1, [])


def test_a_registered_block_keeps_its_one_key():
    # a second key for a block would leave the first key's entry naming the block after it is
    # freed and handed to another sequence, whose K/V a later lookup would then share
    for cache in (True, False):
        p = pool(2, bt=4, cache=cache)
        (i,) = p.alloc(1)
        p.set_fill(i, 4)
        assert p.register(i, 101) == i
        assert p.register(i, 101) == i  # the same key again is fine
        with pytest.raises(B.DecError) as e:
            p.register(i, 202)
        assert e.value.code == B.DEC_E_ARG
        assert p.lookup(202) == -1
        p.release(i)


def test_lookup_never_returns_a_free_block():
    # without prefix caching a released registered block is freed and its key dropped: a
    # lookup misses, and the block goes to a new owner without the old key naming it
    p = pool(2, bt=4, cache=False)
    (i,) = p.alloc(1)
    p.set_fill(i, 4)
    p.register(i, 7)
    p.release(i)
    assert p.info(i)[0] == FREE
    assert p.lookup(7) == -1
    a = p.alloc(2)
    assert i in a
    assert p.lookup(7) == -1
    assert p.info(i)[:2] == (USED, 1)
