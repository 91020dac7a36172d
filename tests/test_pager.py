"""Slot bookkeeping of the bank pager (CPU only): loads into free slots first, hits
refresh a user's age, the least recently used user not in the request gives up its
slot, a request never evicts one of its own users, and a request larger than the pool
is refused."""
import pytest

from tenant_serving_amd.pager import SlotLRU


def test_fill_then_evict_least_recently_used():
    lru = SlotLRU(3)
    loads, ev = lru.ensure([4, 1, 4, 7, -1])
    assert loads == [(4, 0), (1, 1), (7, 2)] and ev == []
    assert lru.ensure([1, 7]) == ([], [])          # hits only; 4 is now the oldest
    loads, ev = lru.ensure([9])
    assert ev == [4] and loads == [(9, 0)]          # 9 takes 4's slot
    loads, ev = lru.ensure([4, 9])                  # 1 is oldest now, 9 is requested
    assert ev == [1] and loads == [(4, 1)]
    assert {u: k for u, k in lru.slot.items()} == {7: 2, 9: 0, 4: 1}


def test_request_never_evicts_its_own_users():
    lru = SlotLRU(2)
    lru.ensure([0, 1])
    loads, ev = lru.ensure([1, 2])                  # 0 goes, not 1
    assert ev == [0] and loads == [(2, 0)]
    loads, ev = lru.ensure([2, 0])                  # 1 goes
    assert ev == [1] and loads == [(0, 1)]


def test_oversized_request_and_drop():
    lru = SlotLRU(2)
    with pytest.raises(ValueError):
        lru.ensure([0, 1, 2])
    with pytest.raises(ValueError):
        SlotLRU(0)
    lru.ensure([5, 6])
    lru.drop(5)
    assert not lru.resident(5) and lru.free == [0]
    assert lru.ensure([8]) == ([(8, 0)], [])
