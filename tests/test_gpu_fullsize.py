"""Parity at full size, in the launch configurations bench.py times.

Stacks are built the way bench.py builds them (experts repacked into pinned
host buffers, then uploaded or kept behind the slot pool), one decode step
is captured as a HIP graph and replayed on tie-free tokens, and every
token's final state is compared with the oracle's chain through all layers
and each layer's routing with the oracle's (exact sets):

- the Qwen3-30B-A3B-shaped Q4_K stack (48 layers, H=2048, 128 experts,
  top-8, I=768, about 16 GB of experts resident) at T=1 and T=8;
- the same shape with a Zipf(1.1) router bias at T=32 (the MFMA path);
- the mixed Q4_K/Q6_K stack (24 layers, 64 routed top-2 + 2 shared experts,
  I=1408) at T=1 and T=4;
- the slot-pool cache's whole decode trace (512 single-token steps through
  48 layers, pools of 10 % and 60 % of the routed expert bytes, host and
  device LRU): its lookups must be the distinct experts of the oracle's
  routing of the trace (stored by tests/golden/make_cache_trace.py), its
  hit/miss/victim trace the oracle LRU's over them, bit for bit, and sampled
  steps' states the oracle chain's.

The oracle only evaluates the selected experts, and its chains run in a
thread pool (its C code releases the interpreter lock).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import quantized_expert_ffn_router_amd as moe
from helpers import REL_L2_BAR, TIE_GAP, ExpertCache, centered_rel_l2, layer_specs, oracle_layers, sets_equal
from quantized_expert_ffn_router_amd.stack import CachedStack, ResidentStack, pack_layer

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cache_trace_qwen3_zipf.npz")


def _say(*a):
    print("[fullsize]", *a, flush=True)


def _pack(cfg, pool):
    specs = layer_specs(cfg)
    packed = []
    for l in range(cfg.n_layers):
        exs = list(pool.map(lambda e: W.expert(cfg, l, e), range(cfg.E + cfg.n_shared)))
        packed.append(pack_layer(specs[l], l, lambda _l, e: exs[e]))
    return specs, packed


def _resident(cfg, T_max):
    _say("building", cfg.name)
    with ThreadPoolExecutor(THREADS) as pool:
        specs, packed = _pack(cfg, pool)
    st = ResidentStack(specs, None, T_max=T_max, packed=packed)
    del packed
    _say("built")
    return cfg, st


@pytest.fixture(scope="module")
def qwen3():
    return _resident(W.qwen3_30b_a3b_q4k(T=8), 8)


@pytest.fixture(scope="module")
def qwen3_zipf():
    return _resident(W.qwen3_30b_a3b_q4k_zipf(T=32), 32)


@pytest.fixture(scope="module")
def mixed():
    return _resident(W.mixed_shared_q4k_q6k(T=4), 4)


def _tie_free_chains(cfg, olayers, step, T):
    """T tokens of a step, each the first attempt whose oracle chain has all
    layers' k-th/(k+1)-th gaps >= TIE_GAP, with those chains."""
    def one(t):
        for a in range(64):
            x = W.token(cfg, step, t, a)
            outs = oracle.stack_token(olayers, x)
            if min(float(o.route.gap[0]) for o in outs) >= TIE_GAP:
                return x, outs
        raise RuntimeError(f"no tie-free draw for token {t}")
    with ThreadPoolExecutor(THREADS) as pool:
        res = list(pool.map(one, range(T)))
    return np.stack([r[0] for r in res]), [r[1] for r in res]


def _graph_step_parity(cfg, st, T, step, chain=False):
    """chain: the layers through moe_layer_forward_chain (no routing outputs:
    the final states against the oracle chains)."""
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts)
    x, ref = _tie_free_chains(cfg, olayers, step, T)
    _say(cfg.name, "T", T, "chain" if chain else "", "oracle chains done")
    h = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.n_layers, T, cfg.k), dtype=torch.int32, device="cuda")
    if chain:
        assert st.chainable(T)
        idx.fill_(-1)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        h.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            if chain:
                st.step(h, chain=True)
            else:
                st.step(h, idx)
    torch.cuda.synchronize()
    worst = 0.0
    for rep in range(2):  # replays with eager work between them
        h.copy_(torch.from_numpy(x))
        graph.replay()
        torch.cuda.synchronize()
        hg, ig = h.cpu().numpy(), idx.cpu().numpy()
        st.step(torch.zeros_like(h))
        torch.cuda.synchronize()
        for t in range(T):
            for l, o in enumerate(ref[t]):
                if not chain:
                    assert sets_equal(ig[l, t][None], o.route.idx), f"replay {rep} layer {l} token {t}"
            href = ref[t][-1].h_next
            e1 = oracle.rel_l2(hg[t], href)
            e2 = centered_rel_l2(hg[t] - x[t], href - x[t])
            worst = max(worst, e1, e2)
            assert e1 <= REL_L2_BAR and e2 <= REL_L2_BAR, (rep, t, e1, e2)
        _say("replay", rep, "ok, worst rel-L2 %.3g" % worst)


@pytest.mark.parametrize("T", [1, 8])
def test_fullsize_graph_step(qwen3, T):
    cfg, st = qwen3
    _graph_step_parity(cfg, st, T, 1000 + T)


def test_fullsize_chain_graph_step(qwen3):
    """48 chained single-token layers (one route launch, then each layer's
    FFN kernels start the next layer's router dots) in a graph."""
    cfg, st = qwen3
    _graph_step_parity(cfg, st, 1, 1500, chain=True)


def test_fullsize_zipf_t32_graph_step(qwen3_zipf):
    """48 layers at 32 tokens: every layer on the MFMA path."""
    cfg, st = qwen3_zipf
    _graph_step_parity(cfg, st, 32, 2000)


@pytest.mark.parametrize("T", [1, 4])
def test_fullsize_mixed_shared_graph_step(mixed, T):
    """24 layers, Q4_K then Q6_K, two shared experts."""
    cfg, st = mixed
    _graph_step_parity(cfg, st, T, 3000 + T)


def test_fullsize_mixed_shared_chain_graph_step(mixed):
    """The 24 mixed layers chained at one token (Q4_K then Q6_K kernels, two
    shared experts' contributions to the next routers, down rows padded)."""
    cfg, st = mixed
    _graph_step_parity(cfg, st, 1, 3500, chain=True)


# ---------------------------------------------------------------- the cache's whole trace

@pytest.fixture(scope="module")
def cache_trace():
    g = np.load(GOLDEN, allow_pickle=False)
    cfg = W.qwen3_cache_trace()
    assert str(g["config"]) == cfg.name
    _say("packing", cfg.name, "in pinned host memory")
    with ThreadPoolExecutor(THREADS) as pool:
        specs, packed = _pack(cfg, pool)
    _say("packed")
    yield cfg, specs, packed, g["attempts"].astype(np.int64), g["ids"].astype(np.int32)
    del packed


@pytest.mark.parametrize("device_lookup", [False, True], ids=["host_lru", "device_lru_graph"])
@pytest.mark.parametrize("fraction", [0.1, 0.6])
def test_cache_full_trace_against_oracle_lru(cache_trace, fraction, device_lookup):
    cfg, specs, packed, att, ids = cache_trace
    steps = ids.shape[0]
    desc = moe.ExpertDesc.of(cfg.qtypes(0), cfg.H, cfg.I)
    eb = moe.moe_expert_bytes(desc)
    budget = int(fraction * cfg.n_layers * cfg.E * eb)
    st, slots = moe.moe_cache_plan([desc], [cfg.n_layers], budget, cfg.k)
    rc, oslots = oracle.cache_plan([eb], [cfg.n_layers], budget, cfg.k)
    assert st == 0 and rc == 0 and np.array_equal(slots, oslots)
    _say("trace", dict(steps=steps, fraction=fraction, slots=int(slots[0]), device=device_lookup))
    xs = np.stack([W.token(cfg, s, 0, int(att[s])) for s in range(steps)])[:, None, :]
    sample = (0, steps // 2, steps - 1)
    cs = CachedStack(specs, packed, slots, T_max=1, device_lookup=device_lookup,
                     trace_capacity=steps * cfg.n_layers * cfg.k if device_lookup else 0)
    got = {}
    try:
        hb = torch.from_numpy(xs[0]).to("cuda")
        if device_lookup:
            # the bench's configuration: one captured step, replayed per token
            # (the capture itself runs no lookup)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                cs.step(hb)
            torch.cuda.synchronize()
        else:
            cs.trace = []
        xs_dev = torch.from_numpy(xs).to("cuda")
        for s in range(steps):
            hb.copy_(xs_dev[s])
            if device_lookup:
                graph.replay()
            else:
                cs.step(hb)
            if s in sample:
                got[s] = hb.cpu().numpy()[0]
        torch.cuda.synchronize()
        LL, EE = oracle.lookup_sequence(ids)
        if device_lookup:
            gl, ge, hit, vl, ve = cs.device_trace()
            del graph
        else:
            gl = np.concatenate([np.full(len(e), l, np.int32) for l, e, *_ in cs.trace])
            ge = np.concatenate([e for _, e, *_ in cs.trace]).astype(np.int32)
            hit = np.concatenate([t[2] for t in cs.trace])
            vl = np.concatenate([t[3] for t in cs.trace])
            ve = np.concatenate([t[4] for t in cs.trace])
        # the GPU routed every step as the oracle did ...
        assert len(gl) == len(LL)
        bad = np.nonzero((gl != LL) | (ge != EE))[0]
        assert bad.size == 0, f"first differing lookup {bad[:1]} of {len(LL)}"
        # ... and its cache made the oracle LRU's decisions
        ref = oracle.lru(slots, [0] * cfg.n_layers, LL, EE)
        assert np.array_equal(hit, ref.hit)
        assert np.array_equal(vl, ref.victim_layer)
        assert np.array_equal(ve, ref.victim_expert)
        s_ = cs.cache.stats()
        n_hit = int(ref.hit.sum())
        assert s_["lookups"] == len(LL) and s_["hits"] == n_hit
        assert s_["evictions"] == int((ref.victim_layer >= 0).sum())
        assert s_["upload_bytes"] == (len(LL) - n_hit) * eb
        _say("hit rate %.4f over %d lookups, %d evictions" % (n_hit / len(LL), len(LL), s_["evictions"]))
    finally:
        cs.close()
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts)
    with ThreadPoolExecutor(THREADS) as pool:
        refs = list(pool.map(lambda s: oracle.stack_token(olayers, xs[s, 0])[-1].h_next, sample))
    for s, href in zip(sample, refs):
        e1 = oracle.rel_l2(got[s], href)
        assert e1 <= REL_L2_BAR, (s, e1)
