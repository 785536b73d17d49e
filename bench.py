#!/usr/bin/env python3
"""Decode throughput of the Qwen3-30B-A3B-shaped Q4_K MoE layer stack on one MI355X.

Workload: 48 MoE layers, hidden 2048, 128 experts per layer, top-8,
expert intermediate 768, experts in Q4_K super-blocks (all ~16 GB resident in
HBM), fp32 router and activations, synthetic seeded data.  A step is one
decode step of the whole stack for a batch of T tokens (default T=1; the
same line also reports T=8): per layer RMSNorm, router GEMV, softmax top-k,
grouping, gate/up matvecs with SiLU(gate)*up, down matvec, weighted combine
and the residual add.  Every step reads a fresh input state, so the experts
selected differ from step to step.

Timed region: K replays of a HIP graph of one step (each preceded by a
device copy of that step's input into the graph's state buffer), bracketed
by synchronisation; value = T*K / elapsed.

A single token's step chains its layers (moe_layer_forward_chain): one
route launch, then per layer a gate/up and a down launch, which also start
the next layer's router dot products.

Roofline: the expert FFN (the gate/up and down kernels of moe_layer_ffn,
which read the selected experts' bytes) timed with HIP events on the launch
stream, layer by layer, in steps launched behind a delay kernel so that they
run back to back.  achieved = sum over layer-steps of U * expert_bytes /
sum of FFN durations, U = distinct experts of the layer-step.  For the
chained single-token step the FFN is a chained layer's two launches (layers
after the first), and their bytes also count the next router's E*H*4.
traffic =
HBM bytes per FFN launch measured with the FETCH_SIZE and WRITE_SIZE
counters (scaled by a copy kernel of known size), read from the committed
counter summary under profiles/ and reported only while the kernel sources
hash to the values recorded there.

cache: the same stack with its routed experts in pinned host memory behind
an HBM slot pool of 10 % and of 60 % of the routed expert bytes (LRU, misses
uploaded on a side stream), Zipf(1.1)-biased routing, 512 single-token
steps from a cold pool: tokens/s, hit rates, misses per token and the
upload rate over PCIe (upload bytes / summed copy intervals).

cpu_baseline: the fp64 oracle on the host, on a bounded sample (a few tokens
through a few layers), scaled to tokens/s of the whole stack.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode tokens/s (layer stack) + achieved HBM GB/s on expert bytes read"
HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
MFMA_I8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix peak

# the FFN kernels each batch size runs on (the library's choice for all-Q4_K
# experts: dot products at T=1, integer MFMA at T=2..8, fp16 MFMA above)
FFN_KERNELS = {
    "dot": "expert FFN (k_gate_up + k_down of moe_layer_ffn)",
    "chain": "expert FFN of a chained single-token layer (k_gate_up + k_down of moe_layer_forward_chain, "
             "with the next layer's router dots)",
    "i8": "expert FFN (k_gate_up_i8 + k_down_i8: integer MFMA)",
    "f16": "expert FFN (k_gate_up_mfma + k_down_mfma: fp16 MFMA)",
}


def ffn_path(T: int) -> str:
    return "dot" if T == 1 else "i8" if T <= 8 else "f16"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "expert_ffn_qwen3_30b_q4k_hbm_traffic.md")
KERNEL_SOURCES = ("moe_kernels.hip", "moe_internal.h")


def measured_traffic(T: int):
    """HBM bytes per FFN launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, calibrated on a copy kernel), or None when that summary has no
    figure for T or was taken on kernel sources other than the current ones."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"kernel_sources_sha256:(.*)", text)
    if not m:
        return None
    recorded = dict(zip(m.group(1).split()[0::2], m.group(1).split()[1::2]))
    csrc = os.path.join(ROOT, "quantized_expert_ffn_router_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != recorded.get(name):
                return None
    m = re.search(rf"traffic_bytes_per_launch T={T}: (\d+)", text)
    return int(m.group(1)) if m else None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def build_stack(cfg, threads: int, keep_layers: int = 0, T_max: int = 8):
    """Generate and repack every expert into pinned per-layer host buffers,
    upload them as a resident stack, and keep the canonical bytes of the
    first `keep_layers` layers for the CPU baseline."""
    import workloads as W
    from quantized_expert_ffn_router_amd.stack import LayerSpec, ResidentStack, pack_layer

    specs = [LayerSpec(cfg.qtypes(l), cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_shared, W.router(cfg, l),
                       W.zipf_bias(cfg, l)) for l in range(cfg.n_layers)]
    pool = ThreadPoolExecutor(threads)
    kept = {}
    packed = []
    n = cfg.E + cfg.n_shared
    for l in range(cfg.n_layers):
        exs = list(pool.map(lambda e: W.expert(cfg, l, e), range(n)))
        if l < keep_layers:
            kept.update({(l, e): exs[e] for e in range(n)})
        packed.append(pack_layer(specs[l], l, lambda _l, e: exs[e]))
        if l % 8 == 0:
            log(f"generated layer {l}/{cfg.n_layers}")
    pool.shutdown()
    st = ResidentStack(specs, None, T_max=T_max, packed=packed)
    return st, kept, specs, packed


def throughput(st, T: int, K: int, Wm: int, H: int, seed: int):
    import torch
    dev = st.device
    g = torch.Generator(device="cpu").manual_seed(seed)
    xs = torch.randn((Wm + K, T, H), generator=g, dtype=torch.float32).to(dev)
    h = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    # eager reference of one step, then capture
    h.copy_(xs[0])
    st.step(h)
    ref = h.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        h.copy_(xs[0])
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            st.step(h)
    torch.cuda.synchronize()
    for rep in range(3):  # graph replays must match the eager step
        h.copy_(xs[0])
        graph.replay()
        torch.cuda.synchronize()
        # the experts' outputs are summed with float atomics: equal up to rounding order,
        # which compounds over the layers (about 1e-5 after 48); a routing difference
        # would move the state by 1e-2 or more
        err = (torch.linalg.vector_norm(h - ref) / torch.linalg.vector_norm(ref)).item()
        if not err <= 1e-4:
            raise RuntimeError(f"graph replay differs from the eager step (rel-L2 {err:.3g})")
        st.step(h)  # eager work between replays
        torch.cuda.synchronize()
    for s in range(Wm):
        h.copy_(xs[s])
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    for s in range(K):
        evs[s].record()
        h.copy_(xs[Wm + s])
        graph.replay()
    evs[K].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    per = np.array([evs[s].elapsed_time(evs[s + 1]) for s in range(K)])
    pct = {f"p{q}": round(float(np.percentile(per, q)), 4) for q in (10, 50, 90)}
    return T * K / el, el / K * 1e3, pct


U_LOG = {}  # batch size -> distinct experts (with shared) of each timed layer-step, in launch order


def chain_timing(st, steps: int, H: int, seed: int):
    """A single token's chained step (as ResidentStack.step runs it), HIP
    events around each layer's moe_layer_forward_chain, launched behind a
    delay.  Layers after the first are their two FFN kernels only (the gate/up
    launch also takes the next router's dots with the input state, the down
    launch those of the experts' contributions), so their algorithmic bytes
    are the k experts' bytes plus the next router's; the first layer's call
    also holds the step's one route launch, whose time beyond an FFN launch
    is spread over the layers as route_us."""
    import torch
    import quantized_expert_ffn_router_amd as moe
    dev = st.device
    nl = len(st.layers)
    g = torch.Generator(device="cpu").manual_seed(seed + 7)
    xs = torch.randn((steps, 1, H), generator=g, dtype=torch.float32).to(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nl)]
    tot_bytes = tot_ffn_ms = tot_first_ms = tot_flop = 0.0
    n_ffn = 0
    for s in range(steps):
        h = xs[s].clone()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)  # keep the GPU busy while the step is enqueued
        for l in range(nl):
            sp = st.layers[l]
            nxt = st.layers[l + 1] if l + 1 < nl else None
            ev[l][0].record()
            moe.moe_layer_forward_chain(st.descs[l], h, 1, st.routers[l], st.biases[l], sp.E, sp.k,
                                        st.expert_ptrs(l), st.shared_ptrs(l), sp.n_shared, st.eps, l > 0,
                                        None if nxt is None else st.routers[l + 1], 0 if nxt is None else nxt.E,
                                        l & 1, st.ws, st.ws_bytes)
            ev[l][1].record()
        torch.cuda.synchronize()
        for l in range(nl):
            ms = ev[l][0].elapsed_time(ev[l][1])
            if l == 0:
                tot_first_ms += ms
                continue
            sp = st.layers[l]
            U = sp.k + sp.n_shared  # a single token's experts are distinct
            U_LOG.setdefault(1, []).append(int(U))
            nxt_bytes = st.layers[l + 1].E * sp.H * 4 if l + 1 < nl else 0
            tot_bytes += U * st.expert_bytes[l] + nxt_bytes
            tot_flop += 2.0 * U * 3 * sp.H * sp.I
            tot_ffn_ms += ms
            n_ffn += 1
    ffn_ms = tot_ffn_ms / n_ffn
    route_ms = max(0.0, tot_first_ms / steps - ffn_ms) / nl
    return dict(ffn_us=ffn_ms * 1e3, route_us=route_ms * 1e3, bytes_per_launch=tot_bytes / n_ffn,
                gbps=tot_bytes / (tot_ffn_ms * 1e-3) / 1e9, launches=n_ffn,
                tflops=tot_flop / (tot_ffn_ms * 1e-3) / 1e12, flop_per_launch=tot_flop / n_ffn)


def ffn_timing(st, T: int, steps: int, H: int, seed: int):
    """HIP events around each layer's moe_layer_ffn, launched behind a delay."""
    import torch
    import quantized_expert_ffn_router_amd as moe
    dev = st.device
    nl = len(st.layers)
    k = st.layers[0].k
    g = torch.Generator(device="cpu").manual_seed(seed + 7)
    xs = torch.randn((steps, T, H), generator=g, dtype=torch.float32).to(dev)
    idx = torch.empty((nl, T, k), dtype=torch.int32, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nl)]
    tot_bytes = 0.0
    tot_ffn_ms = 0.0
    tot_route_ms = 0.0
    tot_pairs = 0
    tot_flop = 0.0
    n_ffn = 0
    for s in range(steps):
        h = xs[s]
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)  # keep the GPU busy while the step is enqueued
        for l in range(nl):
            sp = st.layers[l]
            ev[l][0].record()
            # a single token's ids are distinct, so U = k; not asking for them
            # lets the route launch leave the routing to the FFN's workgroups,
            # as moe_layer_forward does in the timed graph
            moe.moe_layer_route(st.descs[l], h, T, st.routers[l], st.biases[l], sp.E, sp.k, st.expert_ptrs(l),
                                st.shared_ptrs(l), sp.n_shared, st.eps, idx[l] if T > 1 else None, None, st.ws,
                                st.ws_bytes)
            ev[l][1].record()
            moe.moe_layer_ffn(st.descs[l], h, T, sp.E, sp.k, st.expert_ptrs(l), st.shared_ptrs(l), sp.n_shared,
                              st.ws, st.ws_bytes)
            ev[l][2].record()
        torch.cuda.synchronize()
        ids = idx.cpu().numpy()
        for l in range(nl):
            # distinct routed experts plus the always-read shared experts
            U = (len(np.unique(ids[l])) if T > 1 else k) + st.layers[l].n_shared
            U_LOG.setdefault(T, []).append(int(U))
            tot_bytes += U * st.expert_bytes[l]
            tot_pairs += T * (st.layers[l].k + st.layers[l].n_shared)
            tot_flop += 2.0 * T * (st.layers[l].k + st.layers[l].n_shared) * 3 * st.layers[l].H * st.layers[l].I
            tot_ffn_ms += ev[l][1].elapsed_time(ev[l][2])
            tot_route_ms += ev[l][0].elapsed_time(ev[l][1])
            n_ffn += 1
    return dict(ffn_us=tot_ffn_ms / n_ffn * 1e3, route_us=tot_route_ms / n_ffn * 1e3,
                bytes_per_launch=tot_bytes / n_ffn, gbps=tot_bytes / (tot_ffn_ms * 1e-3) / 1e9, launches=n_ffn,
                tflops=tot_flop / (tot_ffn_ms * 1e-3) / 1e12, flop_per_launch=tot_flop / n_ffn)


def cache_leg(cfg, specs, packed, fractions, steps: int, seed: int, n_req: int = 4):
    """The same stack with its routed experts in pinned host memory behind an
    HBM slot pool of `fraction` of the routed expert bytes, Zipf(1.1)-biased
    routing, `steps` single-token decode steps from a cold pool.  Then n_req
    concurrent requests sharing the pool, decoded as one n_req-token batch
    per step (the device LRU as a HIP graph)."""
    import torch
    import workloads as W
    import quantized_expert_ffn_router_amd as moe
    from quantized_expert_ffn_router_amd.stack import CachedStack, LayerSpec

    zcfg = W.qwen3_cache_trace(cfg.n_layers)  # the same experts and routers, Zipf(1.1) bias
    zspecs = [LayerSpec(s.qtypes, s.H, s.I, s.E, s.k, s.n_shared, s.router, W.zipf_bias(zcfg, l))
              for l, s in enumerate(specs)]
    desc = moe.ExpertDesc.of(cfg.qtypes(0), cfg.H, cfg.I)
    eb = moe.moe_expert_bytes(desc)
    total = cfg.n_layers * cfg.E * eb
    g = torch.Generator(device="cpu").manual_seed(seed)
    # the decode trace: token s of the trace's seeded stream at step s (the
    # parity test replays the same stream, redrawing the few near-tie tokens)
    xs = torch.from_numpy(np.stack([W.token(zcfg, s_, 0) for s_ in range(steps + 2)])[:, None, :]).to("cuda")
    legs = []
    for f in fractions:
        st, slots = moe.moe_cache_plan([desc], [cfg.n_layers], int(f * total), cfg.k)
        if st != 0:
            legs.append({"pool_fraction": f, "error": "budget below the floor"})
            continue
        # warm the kernels on a pool that is then discarded, so the timed trace starts cold
        cs = CachedStack(zspecs, packed, slots, T_max=1)
        for s_ in range(2):
            cs.step(xs[steps + s_].clone())
        cs.close()
        del cs
        cs = CachedStack(zspecs, packed, slots, T_max=1)
        cs.time_copies = True
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(steps):
            cs.step(xs[s_].clone())
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        stats = cs.cache.stats()
        copy_s = cs.copy_ms() * 1e-3
        cs.close()
        leg = {
            "pool_fraction": f, "slots": int(slots[0]), "tokens_per_s": round(steps / el, 2),
            "hit_rate": round(stats["hits"] / stats["lookups"], 4),
            "hit_rate_le8": round(stats["hits_le8"] / max(1, stats["lookups_le8"]), 4),
            "misses_per_token": round(stats["misses"] / steps, 2),
            "upload_bytes": int(stats["upload_bytes"]),
            "upload_GBps": round(stats["upload_bytes"] / copy_s / 1e9, 2) if copy_s > 0 else None,
        }
        # the same trace with the LRU on the device: eager steps, then replays
        # of one captured step (input copied in before each replay); each run
        # starts from a cold pool and must reproduce the host run's counts
        # ("ffn_copies_graph": the misses copied inside the FFN launch, moe_cache_ffn_device)
        for mode in ("eager", "graph", "ffn_copies_graph"):
            cs = CachedStack(zspecs, packed, slots, T_max=1, device_lookup=True,
                             ffn_copies=mode == "ffn_copies_graph")
            hb = xs[0].clone()
            if mode != "eager":
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    cs.step(hb)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s_ in range(steps):
                hb.copy_(xs[s_])
                if mode != "eager":
                    graph.replay()
                else:
                    cs.step(hb)
            torch.cuda.synchronize()
            el_d = time.perf_counter() - t0
            ds = cs.cache.stats()
            if mode != "eager":
                del graph
            cs.close()
            same = all(ds[k_] == stats[k_] for k_ in ("lookups", "hits", "misses", "evictions", "upload_bytes"))
            if not same:
                raise RuntimeError(f"device LRU counts {ds} differ from the host LRU's {stats}")
            leg[f"device_lru_{mode}_tokens_per_s"] = round(steps / el_d, 2)
        # cross-layer prefetch (device LRU, graph): at each layer the next
        # layers' routers on its input state predict their experts, whose
        # copies run on a side stream during the current layer
        for depth, mode in ((2, "eager"), (2, "graph")):
            cs = CachedStack(zspecs, packed, slots, T_max=1, device_lookup=True, prefetch_depth=depth)
            hb = xs[0].clone()
            torch.cuda.synchronize()
            if mode == "graph":
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    cs.step(hb)
                torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s_ in range(steps):
                hb.copy_(xs[s_])
                if mode == "graph":
                    graph.replay()
                else:
                    cs.step(hb)
            torch.cuda.synchronize()
            el_p = time.perf_counter() - t0
            ps = cs.cache.stats()
            if mode == "graph":
                del graph
            cs.close()
            leg[f"prefetch_{depth}_{mode}"] = {
                "tokens_per_s": round(steps / el_p, 2),
                "lookups": ps["lookups"], "misses": ps["misses"],
                "misses_per_token": round(ps["misses"] / steps, 2),
                "upload_GB": round(ps["upload_bytes"] / 1e9, 3),
            }
        # a prompt-sized batch through the cache: 64 single-token steps fill
        # the pool, then 128-token batches stage their experts (copied from
        # the slots that hold them, else read from host memory), LRU untouched
        cs = CachedStack(zspecs, packed, slots, T_max=1, device_lookup=True)
        for s_ in range(64):
            cs.step(xs[s_].clone())
        xp = torch.randn((4, 128, cfg.H), generator=g, dtype=torch.float32).to("cuda")
        cs.prompt_step(xp[0].clone())
        torch.cuda.synchronize()
        cs.cache.reset_stats()
        t0 = time.perf_counter()
        for s_ in range(1, 4):
            cs.prompt_step(xp[s_].clone())
        torch.cuda.synchronize()
        el_p = time.perf_counter() - t0
        ps = cs.cache.stats()
        cs.close()
        leg["prompt_128"] = {"tokens_per_s": round(3 * 128 / el_p, 1),
                             "experts_copied_from_slots_per_step": round(ps["large_copies"] / 3, 1),
                             "experts_uploaded_per_step": round(ps["large_uploads"] / 3, 1)}
        # n_req concurrent requests: one n_req-token batch per step, fresh
        # tokens each step, from a cold pool
        if n_req > 1:
            xr = torch.randn((steps, n_req, cfg.H), generator=g, dtype=torch.float32).to("cuda")
            cs = CachedStack(zspecs, packed, slots, T_max=n_req, device_lookup=True)
            hb = xr[0].clone()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                cs.step(hb)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s_ in range(steps):
                hb.copy_(xr[s_])
                graph.replay()
            torch.cuda.synchronize()
            el_r = time.perf_counter() - t0
            rs = cs.cache.stats()
            del graph
            cs.close()
            leg[f"requests_{n_req}"] = {
                "tokens_per_s": round(n_req * steps / el_r, 2),
                "hit_rate": round(rs["hits"] / rs["lookups"], 4),
                "misses_per_step": round(rs["misses"] / steps, 2),
            }
        # hit rate and throughput against concurrency (T4 report, "When the
        # cache hurts": N requests decode as one N-token batch, or a
        # speculative verification of N-1 drafts): device LRU as a graph,
        # cold pool, max(16, 256/N) steps of N fresh tokens
        curve = {}
        for nq in (1, 2, 4, 8, 16, 32):
            nsteps = max(16, 256 // nq)
            xq = torch.randn((nsteps, nq, cfg.H), generator=g, dtype=torch.float32).to("cuda")
            cs = CachedStack(zspecs, packed, slots, T_max=nq, device_lookup=True)
            hb = xq[0].clone()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                cs.step(hb)
            torch.cuda.synchronize()
            cs.cache.reset_stats()
            t0 = time.perf_counter()
            for s_ in range(nsteps):
                hb.copy_(xq[s_])
                graph.replay()
            torch.cuda.synchronize()
            el_q = time.perf_counter() - t0
            qs = cs.cache.stats()
            del graph
            cs.close()
            curve[str(nq)] = {"tokens_per_s": round(nq * nsteps / el_q, 1),
                              "hit_rate": round(qs["hits"] / max(1, qs["lookups"]), 4),
                              "misses_per_step": round(qs["misses"] / nsteps, 1), "steps": nsteps}
        leg["concurrency_curve"] = curve
        legs.append(leg)
        log(f"cache {f:.0%}: {legs[-1]}")
    # placement (T4 report, "Two ways to run"): the 60 % budget spent FIT-style,
    # whole layers resident and a pool of 10 % of the expert bytes for the
    # rest, against the 60 % pool above (every layer cached)
    fit = None
    st_, state, slots = moe.moe_placement_plan([desc], [0] * cfg.n_layers, cfg.E, int(0.6 * total), int(0.1 * total),
                                               cfg.k, moe.MOE_PLACE_FIT)
    if st_ == 0:
        cs = CachedStack(zspecs, packed, slots, T_max=1, device_lookup=True, resident=[x < 0 for x in state])
        hb = xs[0].clone()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs.step(hb)
        torch.cuda.synchronize()
        cs.cache.reset_stats()
        t0 = time.perf_counter()
        for s_ in range(steps):
            hb.copy_(xs[s_])
            graph.replay()
        torch.cuda.synchronize()
        el_f = time.perf_counter() - t0
        fs = cs.cache.stats()
        del graph
        cs.close()
        fit = {"vram_fraction": 0.6, "cache_fraction": 0.1, "resident_layers": int((state < 0).sum()),
               "slots": int(slots[0]), "tokens_per_s": round(steps / el_f, 2),
               "hit_rate_cached_layers": round(fs["hits"] / max(1, fs["lookups"]), 4),
               "misses_per_token": round(fs["misses"] / steps, 2)}
        log(f"placement FIT: {fit}")
    return {"placement_fit": fit,
            "workload": f"same {cfg.n_layers}-layer stack, routed experts in pinned host memory, Zipf(1.1) router "
                        f"bias, {steps} single-token steps from a cold pool, one pool (all layers Q4_K); tokens_per_s: "
                        f"LRU on the host (per-layer id copy and synchronization); device_lru_*: LRU and miss "
                        f"copies on the device, eager and as a captured HIP graph (ffn_copies_graph: the misses copied by the FFN's gate/up launch, moe_cache_ffn_device); prompt_128: 128-token batches after 64 steps, "
                        f"staged beside the slots (device LRU, eager); concurrency_curve: N fresh tokens per step (N requests, or "
                        f"a speculative verification of N-1 drafts), device LRU graph, cold pool; prefetch_D_eager / prefetch_D_graph: the device LRU, eager and as a graph, with cross-layer prefetch of depth D (lookups include the prefetches); requests_N: N concurrent requests "
                        f"sharing the pool, one N-token batch per step (device LRU, graph; hit rate over the "
                        f"step's distinct experts per layer)",
            "legs": legs}


def prompt_leg(st, cfg, T: int, steps: int, seed: int):
    """A prompt-sized batch of T tokens through the resident stack
    (ResidentStack.prompt_step: moe_rmsnorm, moe_route_topk, moe_expert_ffn
    per layer, eager launches), fresh N(0,1) states each step; the distinct
    experts per layer-step are counted from the routing of one step."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    xs = torch.randn((steps + 2, T, cfg.H), generator=g, dtype=torch.float32).to("cuda")
    idx = torch.empty((cfg.n_layers, T, cfg.k), dtype=torch.int32, device="cuda")
    for s_ in range(2):
        h = xs[steps + s_].clone()
        st.prompt_step(h, idx if s_ == 1 else None)
    torch.cuda.synchronize()
    uniq = float(np.mean([len(np.unique(idx[l].cpu().numpy())) for l in range(cfg.n_layers)]))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    hs = [xs[s_].clone() for s_ in range(steps)]
    torch.cuda.synchronize()
    e0.record()
    for s_ in range(steps):
        st.prompt_step(hs[s_])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    eb = cfg.expert_bytes(0)
    return {"batch": T, "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "distinct_experts_per_layer": round(uniq, 1),
            "expert_GBps": round(uniq * eb * cfg.n_layers / (ms * 1e-3) / 1e9, 1),
            "workload": f"{T} fresh tokens per step through the {cfg.n_layers}-layer stack (moe_rmsnorm, "
                        f"moe_route_topk, moe_expert_ffn per layer; MFMA FFN in work entries of at most "
                        f"32 pairs); expert_GBps = distinct experts x expert bytes x layers / step time"}


def cache_leg_groups(cfg, specs, packed, fractions, steps: int, T: int, seed: int):
    """A stack of several (type, shape) groups (the mixed Q4_K / Q6_K stack)
    with its routed experts in pinned host memory behind one slot pool per
    group (the planner splits the budget), shared experts resident, `steps`
    decode steps of T fresh tokens from a cold pool, the device LRU replayed
    as a HIP graph: tokens/s, hit rate, misses per step."""
    import torch
    import quantized_expert_ffn_router_amd as moe
    from quantized_expert_ffn_router_amd.stack import CachedStack

    keys, lg = [], []
    for l in range(cfg.n_layers):
        if cfg.qtypes(l) not in keys:
            keys.append(cfg.qtypes(l))
        lg.append(keys.index(cfg.qtypes(l)))
    descs = [moe.ExpertDesc.of(q, cfg.H, cfg.I) for q in keys]
    eb = [moe.moe_expert_bytes(d) for d in descs]
    per_group = [lg.count(g) for g in range(len(keys))]
    total = sum(cfg.E * eb[g] for g in lg)
    g = torch.Generator(device="cpu").manual_seed(seed)
    xs = torch.randn((steps, T, cfg.H), generator=g, dtype=torch.float32).to("cuda")
    legs = []
    for f in fractions:
        st_, slots = moe.moe_cache_plan(descs, per_group, int(f * total), cfg.k)
        cs = CachedStack(specs, packed, slots, T_max=T, device_lookup=True)
        hb = xs[0].clone()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs.step(hb)
        torch.cuda.synchronize()
        cs.cache.reset_stats()
        t0 = time.perf_counter()
        for s_ in range(steps):
            hb.copy_(xs[s_])
            graph.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        rs = cs.cache.stats()
        del graph
        cs.close()
        legs.append({"pool_fraction": f, "slots": [int(x) for x in slots], "tokens_per_s": round(T * steps / el, 2),
                     "hit_rate": round(rs["hits"] / max(1, rs["lookups"]), 4),
                     "misses_per_step": round(rs["misses"] / steps, 2)})
        log(f"cache (groups) {f:.0%}: {legs[-1]}")
    return {"workload": f"{cfg.n_layers}-layer mixed Q4_K/Q6_K stack, two slot pools (one per type), shared experts "
                        f"resident, {steps} steps of {T} fresh tokens, device LRU as a HIP graph; the pools start "
                        f"with the capture step's experts", "legs": legs}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_CPU_SNIPPET = r"""
import sys, time, json
sys.path.insert(0, {root!r})
import oracle, workloads as W
import numpy as np
def layers(cfg, n):
    ex = {{}}
    def fn(l):
        def g(e):
            if (l, e) not in ex:
                ex[(l, e)] = W.expert(cfg, l, e)
            return ex[(l, e)]
        return g
    return [oracle.LayerWeights(cfg.qtypes(l), cfg.H, cfg.I, cfg.down_k(l), cfg.E, cfg.k, W.router(cfg, l),
                                W.zipf_bias(cfg, l), fn(l), cfg.n_shared) for l in range(n)], ex
out = {{}}
# C1: the tiny single Q8_0 layer, per token
c1 = W.tiny_q8_0(seed=1)
lw, _ = layers(c1, 1)
xs = [W.token(c1, 99, t) for t in range(64)]
oracle.stack_token(lw, xs[0])
t0 = time.perf_counter()
for x in xs:
    oracle.stack_token(lw, x)
out["c1_tokens_per_s"] = len(xs) / (time.perf_counter() - t0)
# the 48-layer Qwen3-30B-A3B-shaped stack: {n_tok} tokens through {n_lay} layers (experts generated outside the timing)
c2 = W.qwen3_30b_a3b_q4k(T=1)
lw, ex = layers(c2, {n_lay})
xs = [W.token(c2, 99, t) for t in range({n_tok})]
for x in xs:
    oracle.stack_token(lw, x)  # generates the routed experts (untimed)
t0 = time.perf_counter()
for x in xs:
    oracle.stack_token(lw, x)
el = time.perf_counter() - t0
out["c2_s_per_token_layer"] = el / (len(xs) * {n_lay})
print(json.dumps(out))
"""


def cpu_baseline(n_tokens: int, n_layers: int, threads: int):
    """The oracle as it stands, timed on the host on bounded samples, in child
    processes with OMP_NUM_THREADS = 1 and = all cores: C1 (one layer) per
    token, and the 48-layer stack per token from n_tokens tokens through
    n_layers layers (scaled to 48; the oracle handles each token on its own,
    so a batch of 8 costs 8 tokens); and the exact LRU simulation of a
    512-step x 48-layer lookup trace (Zipf-skewed ids drawn on the host) at
    the 10 % and 60 % pools."""
    import subprocess
    import oracle
    res = {}
    for nth in (1, threads):
        env = dict(os.environ, OMP_NUM_THREADS=str(nth))
        code = _CPU_SNIPPET.format(root=ROOT, n_tok=n_tokens if nth > 1 else max(2, n_tokens // 16),
                                   n_lay=n_layers)
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=900)
        if r.returncode != 0:
            raise RuntimeError(f"oracle timing failed: {r.stderr[-2000:]}")
        res[nth] = json.loads(r.stdout.strip().splitlines()[-1])
    # LRU simulation over a trace of the C4 size
    rng = np.random.default_rng(4)
    p = np.arange(1, 129, dtype=np.float64) ** -1.1
    p /= p.sum()
    perms = [rng.permutation(128) for _ in range(48)]
    LL, EE = [], []
    for s_ in range(512):
        for l in range(48):
            e = np.unique(perms[l][rng.choice(128, 8, replace=False, p=p)])
            LL.append(np.full(len(e), l, np.int32))
            EE.append(e.astype(np.int32))
    LL, EE = np.concatenate(LL), np.concatenate(EE)
    lru_s = {}
    for name, slots in (("pool_10pct_613_slots", 613), ("pool_60pct_3685_slots", 3685)):
        t0 = time.perf_counter()
        oracle.lru([slots], [0] * 48, LL, EE)
        lru_s[name] = round(time.perf_counter() - t0, 3)
    all_c = res[threads]
    tps = 1.0 / (all_c["c2_s_per_token_layer"] * 48)
    return dict(value=round(tps, 4), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{n_tokens} single-token decodes through {n_layers} of the 48 layers of the Qwen3-30B-A3B-"
                       f"shaped Q4_K stack (fp64 oracle, {threads} threads), scaled to 48 layers; the oracle "
                       f"handles each token on its own, so T=8 costs 8 tokens",
                cpu_model=_cpu_model(), nproc=os.cpu_count(),
                single_thread_tokens_per_s=round(1.0 / (res[1]["c2_s_per_token_layer"] * 48), 4),
                batch8_tokens_per_s=round(tps, 4),
                c1_tokens_per_s={"all_cores": round(all_c["c1_tokens_per_s"], 1),
                                 "single_thread": round(res[1]["c1_tokens_per_s"], 1)},
                lru_simulation_s={"lookups": int(len(LL)), **lru_s})


def roof_hbm(tm, traffic=None, kernel="expert FFN (k_gate_up + k_down of moe_layer_ffn)"):
    return {"bound": "hbm", "achieved": round(tm["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(tm["gbps"] / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
            "bytes_per_launch": round(tm["bytes_per_launch"]), "us_per_launch": round(tm["ffn_us"], 3),
            "launches": tm["launches"]}


def resident_leg(st, T: int, args, seed: int, traffic=None, kernel=None):
    """Throughput (graph replays) and the per-layer FFN roofline of one stack at batch T."""
    tps, ms, pct = throughput(st, T, args.steps, args.warmup, st.layers[0].H, seed=seed)
    chained = T == 1 and st.chainable(1)  # what st.step ran in the timed graph
    if chained:
        tm = chain_timing(st, args.timing_steps, st.layers[0].H, seed=seed)
    else:
        tm = ffn_timing(st, T, args.timing_steps, st.layers[0].H, seed=seed)
    path = "chain" if chained else ffn_path(T)
    leg = {"value": round(tps, 2), "unit": "tokens/s", "ms_per_step": round(ms, 4), "step_ms_percentiles": pct,
           "roofline": roof_hbm(tm, traffic, kernel or FFN_KERNELS[path]),
           "route_us_per_layer": round(tm["route_us"], 3)}
    if path not in ("dot", "chain") and kernel is None:
        # the matrix cores: the pairs' algorithmic operations (2 per multiply-add of gate, up
        # and down) per FFN launch, against the dense peak of the type the kernels issue on
        peak = MFMA_I8_PEAK_TOPS if path == "i8" else MFMA_FP16_PEAK_TFLOPS
        leg["mfma"] = {"bound": "mfma", "achieved": round(tm["tflops"], 2), "peak": peak,
                       "unit": "TOP/s (int8)" if path == "i8" else "TFLOP/s",
                       "frac": round(tm["tflops"] / peak, 4), "flop_per_launch": round(tm["flop_per_launch"])}
    log(f"T={T}: {tps:.1f} tok/s, {ms:.3f} ms/step {pct}; FFN {tm['ffn_us']:.2f} us/launch "
        f"{tm['gbps']:.0f} GB/s ({tm['bytes_per_launch'] / 1e6:.2f} MB), route {tm['route_us']:.2f} us")
    return leg, tm


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1, help="tokens per decode step of the headline value")
    ap.add_argument("--also-batch", type=int, default=8, help="second batch size reported in the same line (0: none)")
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--timing-steps", type=int, default=10)
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the oracle timing")
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--cpu-layers", type=int, default=8)
    ap.add_argument("--cache-steps", type=int, default=512, help="decode steps of each slot-pool leg (0: none)")
    ap.add_argument("--prompt-batch", type=int, default=128, help="tokens of the prompt-sized batch leg (0: none)")
    ap.add_argument("--prompt-steps", type=int, default=10)
    ap.add_argument("--zipf-t32", type=int, default=1, help="the Zipf-biased T=32 leg (MFMA path); 0: none")
    ap.add_argument("--zero-mean", type=int, default=1, help="the zero-mean-field stack at T=8; 0: none")
    ap.add_argument("--mixed", type=int, default=1, help="the mixed Q4_K/Q6_K shared-expert stack legs; 0: none")
    ap.add_argument("--zipf", action="store_true", help="Zipf(1.1) router bias on the headline stack")
    ap.add_argument("--u-log", default="", metavar="PATH",
                    help="write the distinct experts of every timed FFN launch (by batch size, in launch order) "
                         "as JSON, to match per-dispatch counters against the algorithmic bytes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB three times (reads and writes MIB MiB "
                         "each), the reference dispatch for scaling HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the decode path runs on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}); an expert-parallel layout over "
              f"several GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 18  # fp32 elements in MIB MiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read": n * 4, "bytes_written": n * 4,
                          "dispatches": 3}), flush=True)
        return
    import workloads as W
    import quantized_expert_ffn_router_amd as moe
    moe.lib()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    cfg = W.qwen3_30b_a3b_q4k(T=args.batch, n_layers=args.layers)
    if args.zipf:
        cfg = cfg.with_(zipf_s=1.1)
    log(f"building {cfg.name}: {cfg.n_layers} layers x {cfg.E} experts x {cfg.expert_bytes(0)} B")
    t0 = time.time()
    Tmax = max(8, args.batch, args.also_batch, 32 if args.zipf_t32 else 0)
    st, kept, specs, packed = build_stack(cfg, args.threads, 0, T_max=Tmax)
    log(f"stack resident in {time.time() - t0:.1f} s")

    res = {}
    for T in [args.batch] + ([args.also_batch] if args.also_batch and args.also_batch != args.batch else []):
        res[T] = resident_leg(st, T, args, seed=T, traffic=measured_traffic(T))

    zipf32 = None
    if args.zipf_t32:
        # the same stack at T=32 with the Zipf(1.1) router bias (skewed expert loads, MFMA path)
        zc = cfg.with_(zipf_s=1.1, T=32)
        saved = st.biases
        st.biases = [torch.from_numpy(W.zipf_bias(zc, l)).to(st.device) for l in range(cfg.n_layers)]
        zipf32, _ = resident_leg(st, 32, args, seed=32, traffic=measured_traffic(32))
        zipf32["config"] = {"workload": f"the same {cfg.n_layers}-layer Q4_K stack at T=32, Zipf(1.1) router bias "
                                        f"(per-layer permutation), fresh N(0,1) states every step"}
        st.biases = saved

    prompt = None
    if args.prompt_batch:
        prompt = prompt_leg(st, cfg, args.prompt_batch, args.prompt_steps, seed=7)
        log(f"prompt: {prompt}")

    cache = None
    if args.cache_steps:
        cache = cache_leg(cfg, specs, packed, (0.1, 0.6), args.cache_steps, seed=4)
    del st, packed, specs
    torch.cuda.empty_cache()

    zero_mean = None
    if args.zero_mean:
        zcfg = W.qwen3_30b_a3b_q4k(T=8, n_layers=args.layers).with_(zero_mean=True)
        log(f"building {zcfg.name} (zero-mean fields)")
        zst, _, _, zpacked = build_stack(zcfg, args.threads, 0, T_max=8)
        del zpacked
        zero_mean, _ = resident_leg(zst, 8, args, seed=88)
        zero_mean["config"] = {"workload": f"{zcfg.n_layers}-layer Qwen3-30B-A3B-shaped Q4_K stack with zero-mean "
                                           f"weights (dmin = 7.5 d), T=8: states keep no common offset, so the "
                                           f"8 tokens route apart"}
        del zst
        torch.cuda.empty_cache()

    mixed = None
    if args.mixed:
        mcfg = W.mixed_shared_q4k_q6k(T=1)
        log(f"building {mcfg.name}")
        mst, _, mspecs, mpacked = build_stack(mcfg, args.threads, 0, T_max=8)
        mixed = {}
        for T in (1, 4):
            mixed[f"t{T}"], _ = resident_leg(
                mst, T, args, seed=100 + T,
                kernel=None if T == 1 else "expert FFN (k_gate_up_i8 + k_down_i8 on the Q4_K layers, "
                                           "k_gate_up + k_down on the Q6_K layers)")
        mixed["config"] = {"workload": f"{mcfg.n_layers} layers, H=2048, 64 routed (top-2) + 2 shared experts, "
                                       f"I=1408 (down rows padded to 1536), layers 0-11 Q4_K, 12-23 Q6_K, all "
                                       f"resident; FFN bytes per launch include the two shared experts"}
        del mst
        torch.cuda.empty_cache()
        if args.cache_steps:
            mixed["cache"] = cache_leg_groups(mcfg, mspecs, mpacked, (0.1, 0.6), min(args.cache_steps, 256), 4,
                                              seed=9)
        del mpacked

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(args.cpu_tokens, args.cpu_layers, args.threads)
        log(f"cpu baseline {cpu['value']:.4f} tok/s ({cpu['sample']})")

    T = args.batch
    head, tm = res[T]
    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "step_ms_percentiles": head["step_ms_percentiles"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "q4_k weights x int8-piece activations, fp32 scales/accumulate",
        "data": "synthetic (seeded Q4_K fields, N(0,1) states, N(0,0.02^2) router)",
        "config": {"workload": f"qwen3-30b-a3b-shaped Q4_K MoE stack: {cfg.n_layers} layers, H=2048, E=128, "
                               f"top-8, I=768, T={T}, all experts resident",
                   "layers": cfg.n_layers, "batch": T, "expert_bytes": cfg.expert_bytes(0)},
        "roofline": head["roofline"],
        "route_us_per_layer": head["route_us_per_layer"],
        "cpu_baseline": cpu,
    }
    if args.also_batch and args.also_batch in res and args.also_batch != T:
        out[f"batch{args.also_batch}"] = res[args.also_batch][0]
    out["zero_mean_batch8"] = zero_mean
    out["zipf_batch32"] = zipf32
    out["mixed_shared"] = mixed
    out["prompt"] = prompt
    out["cache"] = cache
    if args.u_log:
        with open(args.u_log, "w") as f:
            json.dump({str(k): v for k, v in U_LOG.items()}, f)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
