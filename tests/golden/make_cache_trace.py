"""Writes cache_trace_qwen3_zipf.npz: the oracle's routing of the slot-pool
cache's full decode trace (512 single-token steps through the 48-layer
Qwen3-30B-A3B-shaped Q4_K stack with a Zipf(1.1) router bias; workloads'
qwen3_cache_trace), for the GPU test that replays the trace through the
cache and compares its hit/miss/victim trace with the oracle LRU.

Step s runs token workloads.token(cfg, s, 0, a) for the smallest attempt a
whose chain has every layer's k-th/(k+1)-th logit gap >= 1e-4, so that the
GPU's routing of the same token must equal the oracle's exactly.  Stored:
attempts uint8 [steps], ids uint8 [steps, layers, k] (each layer's experts in
ascending id), gap float32 [steps] (the chain's smallest gap).

Only the oracle and the seeded input generators are used.  Run from the
repository root:  python tests/golden/make_cache_trace.py  (several minutes
on 8 cores; about 10 GB of memory for the generated experts).
"""
import functools
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

STEPS = 512
GAP = 1e-4
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cache_trace_qwen3_zipf.npz")


def main():
    cfg = W.qwen3_cache_trace()
    cache = {}

    def expert(layer, e):
        key = (layer, e)
        if key not in cache:
            cache[key] = W.expert(cfg, layer, e)
        return cache[key]

    layers = [oracle.LayerWeights(cfg.qtypes(l), cfg.H, cfg.I, cfg.down_k(l), cfg.E, cfg.k, W.router(cfg, l),
                                  W.zipf_bias(cfg, l), functools.partial(expert, l), cfg.n_shared)
              for l in range(cfg.n_layers)]

    def one(step):
        for a in range(64):
            outs = oracle.stack_token(layers, W.token(cfg, step, 0, a))
            gap = min(float(o.route.gap[0]) for o in outs)
            if gap >= GAP:
                ids = np.stack([np.sort(o.route.idx.ravel()) for o in outs]).astype(np.uint8)
                return a, ids, gap
        raise RuntimeError(f"no tie-free draw at step {step}")

    with ThreadPoolExecutor(os.cpu_count() or 1) as pool:
        res = list(pool.map(one, range(STEPS)))
    att = np.array([r[0] for r in res], np.uint8)
    ids = np.stack([r[1] for r in res])
    gap = np.array([r[2] for r in res], np.float32)
    np.savez_compressed(OUT, attempts=att, ids=ids, gap=gap,
                        config=np.array(cfg.name), steps=np.int32(STEPS), min_gap=np.float64(GAP))
    print(f"{OUT}: {STEPS} steps, {int((att > 0).sum())} redrawn, smallest gap {gap.min():.3g}, "
          f"{len(cache)} distinct experts")


if __name__ == "__main__":
    main()
