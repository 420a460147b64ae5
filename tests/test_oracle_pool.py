"""Pin of the slot-pool simulator against a trace worked out by hand from the
policy (lowest free slot first; victim = min (count, last_use, expert id)
among unpinned slots; counts halved once per aging period)."""
import pytest

from oracle.pool_sim import PoolBusy, PoolFull, PoolSim


def test_hand_trace_three_slots():
    p = PoolSim(n_layers=1, n_experts=6, slots=3, aging_period=4, blob_bytes=100)
    # step 0: two misses fill slots 0 and 1
    assert p.acquire(0, [0, 1], 0) == [(0, False, 0, -1), (1, False, 1, -1)]
    p.release(0)
    # step 1: expert 1 hits (count 2); expert 2 takes free slot 2
    assert p.acquire(0, [1, 2], 1) == [(1, True, 1, -1), (2, False, 2, -1)]
    p.release(0)
    # step 2: expert 1 hits first (pinned, count 3); expert 3 evicts the
    # unpinned minimum: e0 (count 1, last 0) < e2 (count 1, last 1)
    assert p.acquire(0, [3, 1], 2) == [(3, False, 0, 0), (1, True, 1, -1)]
    p.release(0)
    # step 3: e2 (1, 1) < e3 (1, 2) < e1 (3, 2) -> e2 leaves slot 2
    assert p.acquire(0, [0], 3) == [(0, False, 2, 2)]
    p.release(0)
    # step 4 opens epoch 1: counts e3 1->0, e1 3->1, e0 1->0.  e0 hits (count 1);
    # the miss evicts min over unpinned {e3 (0, 2), e1 (1, 2)} = e3.
    assert p.acquire(0, [2, 0], 4) == [(2, False, 0, 3), (0, True, 2, -1)]
    p.release(0)
    # explicit eviction of an unpinned expert frees its slot
    p.evict(0, 1)
    # step 5: e4 takes the free slot 1; e5 ties e2 and e0 at (1, 4): lower id e0 goes
    assert p.acquire(0, [4, 5], 5) == [(4, False, 1, -1), (5, False, 2, 0)]
    with pytest.raises(PoolBusy):
        p.evict(0, 4)
    # two misses but no free or evictable slot (e2 is requested, e4/e5 pinned)
    with pytest.raises(PoolFull):
        p.acquire(0, [0, 1, 2], 6)
    p.release(0)
    assert p.stats() == dict(hits=3, misses=8, evictions=5, bytes_h2d=800, prefetches=0)
    assert p.expert_in[0] == [2, 4, 5]
    assert p.count[0] == [1, 1, 1]          # the failed call changed nothing


def test_aging_skips_several_epochs():
    p = PoolSim(1, 4, 2, aging_period=2)
    p.acquire(0, [0], 0)
    p.release(0)
    for s in (0, 0, 0):
        p.acquire(0, [0], s)
        p.release(0)
    assert p.count[0][0] == 4
    p.acquire(0, [1], 7)            # epoch 3: shift by 3 -> 4 >> 3 = 0
    assert p.count[0][0] == 0
    p2 = PoolSim(1, 4, 2, aging_period=0)
    p2.acquire(0, [0], 0)
    p2.release(0)
    p2.acquire(0, [0], 1000)
    assert p2.count[0][0] == 2      # no aging


def test_input_errors():
    p = PoolSim(2, 4, 2, 4)
    with pytest.raises(ValueError):
        p.acquire(0, [1, 1], 0)
    with pytest.raises(ValueError):
        p.acquire(0, [4], 0)
    with pytest.raises(PoolFull):
        p.acquire(1, [0, 1, 2], 0)
    p.evict(1, 3)                    # not resident: no-op
    assert p.stats()["evictions"] == 0


def test_hand_trace_prefetch():
    p = PoolSim(n_layers=1, n_experts=8, slots=3, aging_period=0, blob_bytes=10)
    assert p.acquire(0, [0, 1], 0) == [(0, False, 0, -1), (1, False, 1, -1)]
    p.release(0)
    # step 1: e1 is resident (left alone); e2 takes free slot 2; e3 evicts the
    # only candidate not requested here, e0 (count 1, last 0); both enter with
    # count 0, last_use 1, unpinned
    assert p.prefetch(0, [1, 2, 3], 1) == [(2, 2, -1), (3, 0, 0)]
    assert (p.count[0], p.last_use[0], p.pinned[0]) == ([0, 1, 0], [1, 0, 1], [False, False, False])
    # the acquire of the same step hits e1 and e3 (e3: count 0 -> 1, as a miss
    # would have left it); the miss e4 evicts the mispredicted e2 (count 0)
    assert p.acquire(0, [1, 3, 4], 1) == [(1, True, 1, -1), (3, True, 0, -1), (4, False, 2, 2)]
    assert p.count[0] == [1, 2, 1]
    p.release(0)
    # step 2: nothing requested is resident.  e5 evicts min of (1,1,e3) (2,1,e1)
    # (1,1,e4) = e3; e6 then e4 (e5 is now protected); e7 then e1; e0 finds no
    # candidate (every slot holds a requested expert) and is skipped
    assert p.prefetch(0, [5, 6, 7, 0], 2) == [(5, 0, 3), (6, 2, 4), (7, 1, 1)]
    # step 3: e5 hits and is pinned; a prefetch of e0 may not take its slot:
    # candidates e7 (0, 2) and e6 (0, 2) tie on (count, last_use), lower id e6 goes
    assert p.acquire(0, [5], 3) == [(5, True, 0, -1)]
    assert p.prefetch(0, [0], 3) == [(0, 2, 6)]
    assert p.stats() == dict(hits=3, misses=3, evictions=6, bytes_h2d=90, prefetches=6)
    assert p.expert_in[0] == [5, 7, 0]


def test_prefetch_ages_and_validates():
    p = PoolSim(1, 4, 2, aging_period=2)
    p.acquire(0, [0], 0)
    p.release(0)
    p.acquire(0, [0], 1)
    p.release(0)
    assert p.count[0][0] == 2
    assert p.prefetch(0, [1], 4) == [(1, 1, -1)]   # epoch 2: 2 >> 2 = 0
    assert p.count[0] == [0, 0]
    with pytest.raises(ValueError):
        p.prefetch(0, [2, 2], 5)
    with pytest.raises(ValueError):
        p.prefetch(0, [4], 5)
