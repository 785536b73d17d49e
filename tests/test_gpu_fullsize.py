"""Parity at full size, in the launch configuration bench.py times.

The Qwen3-30B-A3B-shaped Q4_K stack (48 layers, H=2048, 128 experts, top-8,
I=768, about 16 GB of experts resident) is built the way bench.py builds it
(experts repacked into pinned host buffers, then uploaded), one decode step
is captured as a HIP graph, and graph replays run tie-free tokens at T=1 and
T=8.  Every token's final state is compared with the oracle's 48-layer
chain, and each layer's routing with the oracle's (exact sets).  The oracle
only evaluates the selected experts, so it finishes in seconds.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
from helpers import REL_L2_BAR, ExpertCache, centered_rel_l2, chain_min_gap, oracle_layers, sets_equal
from quantized_expert_ffn_router_amd.stack import LayerSpec, ResidentStack, pack_layer

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[fullsize]", *a, flush=True)


@pytest.fixture(scope="module")
def stack():
    cfg = W.qwen3_30b_a3b_q4k(T=8)
    _say("building", cfg.name)
    specs = [LayerSpec(cfg.qtypes(l), cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_shared, W.router(cfg, l),
                       W.zipf_bias(cfg, l)) for l in range(cfg.n_layers)]
    packed = []
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
        for l in range(cfg.n_layers):
            exs = list(pool.map(lambda e: W.expert(cfg, l, e), range(cfg.E)))
            packed.append(pack_layer(specs[l], l, lambda _l, e: exs[e]))
    st = ResidentStack(specs, None, T_max=8, packed=packed)
    del packed
    _say("built")
    return cfg, st


@pytest.mark.parametrize("T", [1, 8])
def test_fullsize_graph_step(stack, T):
    cfg, st = stack
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts)
    x, att = W.tie_free_tokens(cfg, 1000 + T, T, chain_min_gap(olayers))
    _say("T", T, "attempts", att)
    h = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.n_layers, T, cfg.k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        h.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            st.step(h, idx)
    torch.cuda.synchronize()
    ref = [oracle.stack_token(olayers, x[t]) for t in range(T)]
    for rep in range(2):  # replays with eager work between them
        h.copy_(torch.from_numpy(x))
        graph.replay()
        torch.cuda.synchronize()
        hg, ig = h.cpu().numpy(), idx.cpu().numpy()
        st.step(torch.zeros_like(h))
        torch.cuda.synchronize()
        for t in range(T):
            for l, o in enumerate(ref[t]):
                assert sets_equal(ig[l, t][None], o.route.idx), f"replay {rep} layer {l} token {t}"
            href = ref[t][-1].h_next
            e1 = oracle.rel_l2(hg[t], href)
            e2 = centered_rel_l2(hg[t] - x[t], href - x[t])
            assert e1 <= REL_L2_BAR and e2 <= REL_L2_BAR, (rep, t, e1, e2)
        _say("replay", rep, "max rel-L2 over tokens ok")
