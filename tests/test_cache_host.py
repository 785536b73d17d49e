"""CPU tests of the slot-pool cache's host LRU through the C ABI.

The cache runs on a caller-supplied synchronous backend (moe_cache_create_ex)
whose pools are numpy buffers and whose copies are memmove, so the whole host
side of the cache -- lookup of raw ids, LRU decisions, slot tables, uploads,
statistics, groups below the budget floor and the rollback of a failed
upload -- runs here without a GPU.  Decisions are compared with the oracle's
LRU simulation (T4 MoE-cache report, "What the MoE cache caches": one LRU
pool per (type, shape) group, keys (layer, expert)); the bytes that land in
the slots are compared with the host experts they were copied from.
"""
import ctypes

import numpy as np
import pytest

import oracle
import quantized_expert_ffn_router_amd as moe
from quantized_expert_ffn_router_amd import _lib

Q8_0, Q4_K = 1, 2


class HostPools:
    """Numpy-backed pools; copy() can be made to fail on chosen calls."""

    def __init__(self):
        self.bufs = {}
        self.copies = 0
        self.fail = None  # fail(n_expert_copy, nbytes) -> bool, for expert-sized copies only
        self.expert_copies = 0
        self.expert_sizes = set()

    def alloc(self, n):
        b = np.zeros(n + 256, np.uint8)
        addr = (b.ctypes.data + 255) & ~255
        self.bufs[addr] = b
        return addr

    def release(self, p):
        self.bufs.pop(p, None)

    def copy(self, dst, src, n):
        self.copies += 1
        if n in self.expert_sizes:
            self.expert_copies += 1
            if self.fail is not None and self.fail(self.expert_copies, n):
                return 1
        ctypes.memmove(dst, src, n)
        return 0


class Setup:
    """A small cached stack: `layers` layers over groups of (qtype, H, I)."""

    def __init__(self, group_descs, layer_group, E, slots, seed=0):
        self.descs = [moe.ExpertDesc.of((q, q, q), H, I) for q, H, I in group_descs]
        self.eb = [moe.moe_expert_bytes(d) for d in self.descs]
        self.layer_group = list(layer_group)
        self.L = len(layer_group)
        self.E = E
        rng = np.random.default_rng(seed)
        self.host = [rng.integers(0, 256, self.eb[g], dtype=np.uint8) for g in layer_group for _ in range(E)]
        self.pools = HostPools()
        self.pools.expert_sizes = set(self.eb)
        self.backend = _lib.CacheBackend.of(self.pools.alloc, self.pools.release, self.pools.copy)
        self.slots = list(slots)
        self.cache = _lib.Cache(self.descs, self.slots, self.layer_group, E,
                                [h.ctypes.data for h in self.host], backend=self.backend)

    def expert_bytes(self, l, e):
        return self.host[l * self.E + e]

    def table(self, l):
        p = self.cache.expert_ptrs(l)
        return [v or 0 for v in (ctypes.c_void_p * self.E).from_address(p)]

    def read(self, addr, n):
        return np.frombuffer((ctypes.c_uint8 * n).from_address(addr), np.uint8)

    def check_tables(self, resident):
        """Every table entry is NULL unless its expert is resident, and then
        the slot it names holds exactly that expert's bytes."""
        for l in range(self.L):
            for e, a in enumerate(self.table(l)):
                if (l, e) in resident:
                    assert a != 0, (l, e)
                    assert np.array_equal(self.read(a, self.eb[self.layer_group[l]]), self.expert_bytes(l, e)), (l, e)
                else:
                    assert a == 0, (l, e)


def _oracle_state(slots, layer_group, LL, EE):
    """Keys resident after the oracle LRU runs over (LL, EE)."""
    ref = oracle.lru(slots, layer_group, LL, EE)
    res = set()
    for l, e, v_l, v_e in zip(LL, EE, ref.victim_layer, ref.victim_expert):
        if v_l >= 0:
            res.discard((int(v_l), int(v_e)))
        res.add((int(l), int(e)))
    return ref, res


def _random_steps(rng, n_steps, L, E, T, k, skew=1.5):
    p = np.arange(1, E + 1, dtype=np.float64) ** -skew
    p /= p.sum()
    steps = []
    for _ in range(n_steps):
        for l in range(L):
            ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
            steps.append((l, ids))
    return steps


def test_lookup_dedups_raw_ids_ascending():
    s = Setup([(Q8_0, 256, 64)], [0, 0], 8, [6])
    ex, slot, hit, vl, ve = s.cache.lookup(1, 3, 2, np.array([5, 2, 2, 7, 5, 0], np.int32))
    assert ex.tolist() == [0, 2, 5, 7]
    assert hit.tolist() == [0, 0, 0, 0] and slot.tolist() == [0, 1, 2, 3]
    s.cache.upload(1, None)
    ex, slot, hit, vl, ve = s.cache.lookup(1, 1, 2, np.array([7, 3], np.int32))
    assert ex.tolist() == [3, 7] and hit.tolist() == [0, 1] and slot.tolist() == [4, 3]
    with pytest.raises(moe.MoeError) as ei:
        s.cache.lookup(0, 1, 2, np.array([1, 2], np.int32))  # layer 1's misses not uploaded yet
    assert ei.value.name == "MOE_ERR_STATE"
    s.cache.upload(1, None)
    with pytest.raises(moe.MoeError) as ei:
        s.cache.lookup(0, 1, 2, np.array([1, 8], np.int32))
    assert ei.value.name == "MOE_ERR_ARG"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_host_lru_trace_tables_and_bytes_match_oracle(seed):
    """Two groups (Q8_0 and Q4_K experts), pools small enough to thrash:
    hit/miss/victim trace, statistics, slot tables (evicted entries NULL) and
    the bytes in every slot against the oracle LRU and the host experts."""
    rng = np.random.default_rng(seed)
    lg = [0, 1, 0, 1, 1]
    E, T, k = 12, 2, 2
    s = Setup([(Q8_0, 256, 64), (Q4_K, 256, 64)], lg, E, [7, 9], seed=seed)
    LL, EE, hits, vls, ves = [], [], [], [], []
    for l, ids in _random_steps(rng, 12, len(lg), E, T, k):
        ex, slot, hit, vl, ve = s.cache.lookup(l, T, k, ids.ravel())
        assert ex.tolist() == sorted(set(ids.ravel().tolist()))
        s.cache.upload(l, None)
        LL += [l] * len(ex)
        EE += ex.tolist()
        hits.append(hit)
        vls.append(vl)
        ves.append(ve)
    ref, resident = _oracle_state(s.slots, lg, np.array(LL, np.int32), np.array(EE, np.int32))
    assert np.array_equal(np.concatenate(hits), ref.hit)
    assert np.array_equal(np.concatenate(vls), ref.victim_layer)
    assert np.array_equal(np.concatenate(ves), ref.victim_expert)
    st = s.cache.stats()
    assert st["lookups"] == len(LL) and st["hits"] == int(ref.hit.sum())
    assert st["evictions"] == int((ref.victim_layer >= 0).sum())
    assert st["upload_bytes"] == sum(s.eb[lg[l]] for l, h in zip(LL, ref.hit) if not h)
    assert st["lookups_le8"] == len(LL) and st["lookups_9_32"] == 0
    s.check_tables(resident)


def test_group_below_floor_stays_resident():
    """A plan with one group at 0 slots: its layers' experts are uploaded once
    and stay resident, their lookups are all hits in slot -1 and count in no
    statistic; the other group caches as usual.  All groups at 0: refused."""
    lg = [0, 1, 1, 0]
    E = 6
    s = Setup([(Q8_0, 256, 64), (Q4_K, 256, 64)], lg, E, [0, 5])
    assert "resident" in _lib.lib().moe_last_error().decode()
    for l in (0, 3):
        ex, slot, hit, vl, ve = s.cache.lookup(l, 2, 2, np.array([4, 1, 1, 5], np.int32))
        assert ex.tolist() == [1, 4, 5] and hit.all() and (slot == -1).all() and (vl == -1).all()
        s.cache.upload(l, None)
    for l, ids in ((1, [0, 2]), (2, [2, 3]), (1, [4, 5]), (2, [0, 1])):
        s.cache.lookup(l, 1, 2, np.array(ids, np.int32))
        s.cache.upload(l, None)
    st = s.cache.stats()
    assert st["lookups"] == 8 and st["hits"] == 0
    LL = np.array([1, 1, 2, 2, 1, 1, 2, 2], np.int32)
    EE = np.array([0, 2, 2, 3, 4, 5, 0, 1], np.int32)
    _, resident = _oracle_state(s.slots, lg, LL, EE)
    resident |= {(l, e) for l in (0, 3) for e in range(E)}
    s.check_tables(resident)
    with pytest.raises(moe.MoeError) as ei:
        Setup([(Q8_0, 256, 64), (Q4_K, 256, 64)], lg, E, [0, 0])
    assert ei.value.name == "MOE_ERR_BUDGET"


@pytest.mark.parametrize("fail_at", [1, 2, 3])
def test_failed_upload_rolls_back_from_the_failing_miss(fail_at):
    """A copy failure at the fail_at-th miss of a thrashing layer-step: the
    misses before it stay, every later decision of the lookup is undone
    (keys, recency, free slots, evicted keys, tables, statistics).  A retry
    of the same step and the steps after it then follow the oracle LRU over
    the sequence whose failed lookup stops before that miss."""
    rng = np.random.default_rng(7)
    lg = [0, 0, 0]
    E, T, k = 10, 2, 2
    s = Setup([(Q4_K, 256, 64)], lg, E, [6], seed=3)
    steps = _random_steps(rng, 10, len(lg), E, T, k)
    LL, EE, got = [], [], []
    fail_step = 13
    for i, (l, ids) in enumerate(steps):
        ex, slot, hit, vl, ve = s.cache.lookup(l, T, k, ids.ravel())
        if i == fail_step:
            misses = np.flatnonzero(hit == 0)
            assert len(misses) >= fail_at, "the step must have enough misses"
            cut = int(misses[fail_at - 1])  # decisions before the failing miss survive
            before = s.pools.expert_copies
            s.pools.fail = lambda n, nb: n == before + fail_at
            with pytest.raises(moe.MoeError) as ei:
                s.cache.upload(l, None)
            assert ei.value.name == "MOE_ERR_HIP"
            s.pools.fail = None
            LL += [l] * cut
            EE += ex[:cut].tolist()
            got.append(hit[:cut])
            ref, resident = _oracle_state(s.slots, lg, np.array(LL, np.int32), np.array(EE, np.int32))
            st = s.cache.stats()
            assert st["lookups"] == len(LL) and st["hits"] == int(ref.hit.sum())
            assert st["evictions"] == int((ref.victim_layer >= 0).sum())
            # the keys the undone decisions had evicted are back in their
            # slots: looked up one by one, each must hit (the oracle agrees)
            back = [(int(a), int(b)) for a, b in zip(vl[cut:], ve[cut:]) if a >= 0]
            assert back, "the failed step must have undone an eviction"
            for vl_, ve_ in back:
                ex1, _, hit1, _, _ = s.cache.lookup(vl_, 1, 1, np.array([ve_], np.int32))
                s.cache.upload(vl_, None)
                assert hit1.tolist() == [1]
                LL.append(vl_)
                EE.append(ve_)
                got.append(hit1)
            # then the failed step again
            ex, slot, hit, vl, ve = s.cache.lookup(l, T, k, ids.ravel())
        s.cache.upload(l, None)
        LL += [l] * len(ex)
        EE += ex.tolist()
        got.append(hit)
    ref, resident = _oracle_state(s.slots, lg, np.array(LL, np.int32), np.array(EE, np.int32))
    assert np.array_equal(np.concatenate(got), ref.hit)
    s.check_tables(resident)


def test_placement_plan_fit_and_all_cached():
    """The placement planner (T4 MoE-cache report, "Two ways to run"): FIT
    reserves the cache budget, makes whole layers resident in layer order
    while they fit (first fit), and plans the slots over the layers left;
    ALL_CACHED gives every layer to the cache, as moe_cache_plan does."""
    descs = [moe.ExpertDesc.of((Q8_0,) * 3, 256, 64), moe.ExpertDesc.of((Q4_K,) * 3, 256, 64)]
    eb = [moe.moe_expert_bytes(d) for d in descs]
    assert eb == [104448, 55296]
    lg = [0, 1, 0, 1, 1]
    E, k = 8, 2
    layer = [E * eb[g] for g in lg]  # 835,584 / 442,368 bytes per layer
    # FIT: 2,000,000 bytes of VRAM, 400,000 for the cache: 1,600,000 left for layers.
    # layer 0 (835,584) fits -> 764,416 left; layer 1 (442,368) fits -> 322,048;
    # layer 2 (835,584) no; layer 3 (442,368) no; layer 4 no.
    # cached: group 0 one layer, group 1 two layers; denominator 104,448 + 2 * 55,296 = 215,040
    # group 0: floor(400,000 * 1 / 215,040) - 1 = 0 -> below k=2: refused (outputs still filled);
    # group 1: floor(400,000 * 2 / 215,040) - 1 = 3 - 1 = 2
    st, state, slots = moe.moe_placement_plan(descs, lg, E, 2_000_000, 400_000, k, moe.MOE_PLACE_FIT)
    assert st == -4 and state.tolist() == [-1, -2, 0, 1, 1] and slots.tolist() == [0, 2]
    st, state, slots = moe.moe_placement_plan(descs, lg, E, 3_000_000, 1_500_000, k, moe.MOE_PLACE_FIT)
    # 1,500,000 for layers: layer 0 fits (664,416 left), layer 1 fits (222,048), the rest no
    assert st == 0 and state.tolist() == [-1, -2, 0, 1, 1]
    # group 0: floor(1,500,000 / 215,040) - 1 = 6 - 1 = 5; group 1: floor(3,000,000 / 215,040) - 1 = 13 - 1 = 12
    assert slots.tolist() == [5, 12]
    # every layer fits: all resident, no slots
    st, state, slots = moe.moe_placement_plan(descs, lg, E, 10_000_000, 100, k, moe.MOE_PLACE_FIT)
    assert st == 0 and (state < 0).all() and slots.tolist() == [0, 0]
    # ALL_CACHED: the plain planner over all layers
    st, state, slots = moe.moe_placement_plan(descs, lg, E, 3_000_000, 0, k, moe.MOE_PLACE_ALL_CACHED)
    st_p, slots_p = moe.moe_cache_plan(descs, [2, 3], 3_000_000, k)
    assert st == 0 and state.tolist() == lg and slots.tolist() == slots_p.tolist()
    with pytest.raises(moe.MoeError):
        moe.moe_placement_plan(descs, lg, E, 100, 200, k, moe.MOE_PLACE_FIT)  # cache above the budget


def test_resident_layers_beside_cached_layers():
    """Layers placed resident (group entry -(g+1)) keep all their experts and
    make no lookups; the cached layers of the same group follow the oracle
    LRU over their own lookups."""
    rng = np.random.default_rng(3)
    lg = [0, 0, 0, 0]
    E, T, k = 10, 2, 2
    s = Setup([(Q4_K, 256, 64)], [-1, 0, -1, 0], E, [5], seed=5)
    LL, EE, got = [], [], []
    for l, ids in _random_steps(rng, 8, 4, E, T, k):
        ex, slot, hit, vl, ve = s.cache.lookup(l, T, k, ids.ravel())
        s.cache.upload(l, None)
        if l in (0, 2):
            assert hit.all() and (slot == -1).all()
            continue
        LL += [l] * len(ex)
        EE += ex.tolist()
        got.append(hit)
    ref, resident = _oracle_state([5], lg, np.array(LL, np.int32), np.array(EE, np.int32))
    assert np.array_equal(np.concatenate(got), ref.hit)
    st = s.cache.stats()
    assert st["lookups"] == len(LL) and st["hits"] == int(ref.hit.sum())
    resident |= {(l, e) for l in (0, 2) for e in range(E)}
    s.check_tables(resident)


def test_large_batch_staging_copies_cached_experts_and_leaves_the_lru():
    """Batches above 32 tokens bypass the slots (T4 MoE-cache report, "What
    the MoE cache caches"): the layer's distinct experts are staged in a
    caller area, copied from their slots when cached (large_copies) or from
    host memory (large_uploads).  The staged bytes are the experts' bytes,
    the table names them, the counts follow the oracle LRU's resident set at
    that point, and the LRU afterwards still follows the oracle over the
    small-batch lookups alone."""
    rng = np.random.default_rng(9)
    lg = [0, 0, 0]
    E, T, k = 12, 2, 2
    s = Setup([(Q4_K, 256, 64)], lg, E, [6], seed=2)
    eb = s.eb[0]
    staging = s.pools.alloc(E * eb)
    table = s.pools.alloc(8 * E)
    LL, EE, got = [], [], []
    copies = uploads = 0
    for i, (l, ids) in enumerate(_random_steps(rng, 10, 3, E, T, k)):
        ex, slot, hit, vl, ve = s.cache.lookup(l, T, k, ids.ravel())
        s.cache.upload(l, None)
        LL += [l] * len(ex)
        EE += ex.tolist()
        got.append(hit)
        if i % 7 == 6:
            big = rng.integers(0, E, 40 * 3).astype(np.int32)  # a 40-token batch, top-3
            m = l  # the layer just looked up: some of its experts are in slots
            _, resident = _oracle_state([6], lg, np.array(LL, np.int32), np.array(EE, np.int32))
            s.cache.stage_large(m, 40, 3, big, staging, E * eb, table)
            want = sorted(set(big.tolist()))
            tab = [v or 0 for v in (ctypes.c_void_p * E).from_address(table)]
            for u, e in enumerate(want):
                assert tab[e] == staging + u * eb
                assert np.array_equal(s.read(tab[e], eb), s.expert_bytes(m, e))
            assert all(tab[e] == 0 for e in range(E) if e not in want)
            c = sum((m, e) in resident for e in want)
            copies += c
            uploads += len(want) - c
            st = s.cache.stats()
            assert st["large_copies"] == copies and st["large_uploads"] == uploads
    ref, resident = _oracle_state([6], lg, np.array(LL, np.int32), np.array(EE, np.int32))
    assert np.array_equal(np.concatenate(got), ref.hit)
    assert copies > 0 and uploads > 0
    st = s.cache.stats()
    assert st["lookups"] == len(LL)
    with pytest.raises(moe.MoeError) as ei:
        s.cache.stage_large(0, 32, 2, np.zeros(64, np.int32), staging, E * eb, table)
    assert ei.value.name == "MOE_ERR_BATCH"
    with pytest.raises(moe.MoeError) as ei:
        s.cache.stage_large(0, 40, 3, np.arange(120, dtype=np.int32) % E, staging, eb, table)
    assert ei.value.name == "MOE_ERR_ARG"
    s.check_tables(resident)
