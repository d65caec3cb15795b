"""Host-side expert slot planner (CPU only), through the C ABI.

Policy (Mference system design, "Load and ownership"): a fixed number of slots per layer,
least-frequently-used eviction with recency as the tie-breaker, a hit reuses its slot and a
miss takes an evictable slot. Pinned by hand-worked cases and by random request sequences
against a separately written Python model of the same policy, plus invariants after every
request (every requested expert resident, slots hold distinct experts, the table agrees).
"""
import numpy as np
import pytest

from quantized_moe_bit_amd import binding as B


class ModelLFU:
    """Plain reference: per slot (expert, uses since fill, last request); free slots first."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.expert = [None] * S
        self.uses = [0] * S
        self.last = [-1] * S
        self.req = 0

    def where(self, e):
        return self.expert.index(e) if e in self.expert else -1

    def plan(self, experts, protect=()):
        want = sorted(set(int(e) for e in experts))
        kept = {self.where(int(e)) for e in protect if int(e) not in want and self.where(int(e)) >= 0}
        if len(want) + len(kept) > self.S:
            return None
        r = self.req
        self.req += 1
        used_now = set(kept)   # protected residents are not evictable by this request
        misses = []
        for e in want:
            s = self.where(e)
            if s >= 0:
                self.uses[s] += 1
                self.last[s] = r
                used_now.add(s)
            else:
                misses.append(e)
        fills = []
        for e in misses:
            free = [s for s in range(self.S) if self.expert[s] is None]
            if free:
                s = free[0]
            else:
                s = min((s for s in range(self.S) if s not in used_now),
                        key=lambda s: (self.uses[s], self.last[s], s))
            self.expert[s], self.uses[s], self.last[s] = e, 1, r
            used_now.add(s)
            fills.append((e, s))
        return [self.where(int(e)) for e in experts], fills

    def table(self):
        t = np.full(self.E, -1, np.int32)
        for s, e in enumerate(self.expert):
            if e is not None:
                t[e] = s
        return t


def test_hand_worked_lfu_and_recency():
    c = B.SlotCache(8, 2)
    assert c.plan([0]) == ([0], [(0, 0)])
    assert c.plan([1]) == ([1], [(1, 1)])
    # expert 0 used again: slot 0 has 2 uses, slot 1 one use
    assert c.plan([0]) == ([0], [])
    # a miss evicts the least-used resident (expert 1 in slot 1)
    assert c.plan([2]) == ([1], [(2, 1)])
    assert list(c.table()[:4]) == [0, -1, 1, -1]
    c.close()
    # equal use counts: the oldest last use goes first
    c = B.SlotCache(8, 2)
    c.plan([5])
    c.plan([6])
    assert c.plan([7]) == ([0], [(7, 0)])
    c.close()


def test_request_protects_its_own_experts_and_dedups():
    c = B.SlotCache(8, 2)
    c.plan([0])
    c.plan([1])
    c.plan([1])   # expert 1: two uses; expert 0: one use, older
    # expert 0 is listed with a miss: the miss may not evict it, so expert 1 (more uses) goes
    assert c.plan([0, 3]) == ([0, 1], [(3, 1)])
    # duplicates count once and map to one slot
    slot_of, fills = c.plan([3, 3, 3])
    assert list(slot_of) == [1, 1, 1] and fills == []
    c.close()


def test_capacity_refused_without_change():
    c = B.SlotCache(8, 2)
    c.plan([4])
    before = c.table().copy()
    with pytest.raises(B.MoeError) as ei:
        c.plan([0, 1, 2])
    assert ei.value.status == B.MOE_E_CAPACITY
    np.testing.assert_array_equal(c.table(), before)
    with pytest.raises(B.MoeError):
        c.plan([8])   # expert out of range
    c.close()
    with pytest.raises(B.MoeError):
        B.SlotCache(8, 9)   # more slots than experts


def test_protected_experts_keep_their_slots():
    """Planning the next tile while the current one is queued: the current tile's experts are
    protected (not evicted, no use counted), so the next tile's misses take other slots."""
    c = B.SlotCache(16, 4)
    assert c.plan([0, 1]) == ([0, 1], [(0, 0), (1, 1)])
    assert c.plan([2, 3], protect=[0, 1]) == ([2, 3], [(2, 2), (3, 3)])
    # tile {4, 5} while {2, 3} is queued: 0 and 1 (one use each) are evicted, 2 and 3 kept
    assert c.plan([4, 5], protect=[2, 3]) == ([0, 1], [(4, 0), (5, 1)])
    # protection counts no use: 2 and 3 still have one use each, like 4 and 5; the oldest go
    assert c.plan([6, 7], protect=[4, 5]) == ([2, 3], [(6, 2), (7, 3)])
    # a protected expert that the request itself lists is an ordinary hit
    assert c.plan([6, 8], protect=[6, 7]) == ([2, 0], [(8, 0)])
    # the request plus the kept protected experts must fit
    before = c.table().copy()
    with pytest.raises(B.MoeError) as ei:
        c.plan([9, 10, 11], protect=[6, 8])
    assert ei.value.status == B.MOE_E_CAPACITY
    np.testing.assert_array_equal(c.table(), before)
    c.close()


@pytest.mark.parametrize("E,S,k,seed", [(32, 8, 4, 3), (128, 16, 8, 4)])
def test_random_tiles_with_protection_match_model(E, S, k, seed):
    """Tiles of at most half the slots, each planned while the previous tile is protected."""
    rng = np.random.default_rng(seed)
    c = B.SlotCache(E, S)
    m = ModelLFU(E, S)
    prev = []
    for _ in range(300):
        tile = rng.choice(E, size=int(rng.integers(1, S // 2 + 1)), replace=False).astype(np.int32)
        got = c.plan(tile, protect=prev)
        want = m.plan(tile, protect=prev)
        assert list(got[0]) == want[0] and got[1] == want[1]
        t = c.table()
        np.testing.assert_array_equal(t, m.table())
        assert np.all(t[tile] >= 0) and np.all(t[np.array(prev, np.int32)] >= 0) if len(prev) else True
        prev = tile.tolist()
    c.close()


@pytest.mark.parametrize("E,S,k,seed", [(32, 8, 4, 0), (128, 16, 8, 1), (64, 64, 8, 2)])
def test_random_requests_match_model(E, S, k, seed):
    rng = np.random.default_rng(seed)
    # skewed expert popularity, so hits, misses and evictions all occur
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p = rng.permutation(p / p.sum())
    c = B.SlotCache(E, S)
    m = ModelLFU(E, S)
    fills_total = 0
    for _ in range(400):
        n = int(rng.integers(1, k + 1))
        req = rng.choice(E, size=n, replace=True, p=p).astype(np.int32)
        got = c.plan(req)
        want = m.plan(req)
        assert list(got[0]) == want[0] and got[1] == want[1]
        t = c.table()
        np.testing.assert_array_equal(t, m.table())
        assert np.all(t[req] >= 0)                                 # every requested expert resident
        res = t[t >= 0]
        assert len(set(res.tolist())) == len(res) and res.max(initial=-1) < S   # distinct slots
        fills_total += len(got[1])
    assert 0 < fills_total < 400 * k
