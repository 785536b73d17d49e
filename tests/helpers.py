"""Shared helpers of the GPU parity tests: oracle layers, tie-free inputs,
and comparison metrics.  Only tests import this module."""
from __future__ import annotations

import functools
from typing import Dict, List, Sequence

import numpy as np

import oracle
import workloads as W

REL_L2_BAR = 1e-3     # tolerance on fp32 FFN outputs
W_REL_BAR = 1e-5      # renormalised routing weights
TIE_GAP = 1e-4        # minimum k-th / (k+1)-th logit gap of generated inputs


class ExpertCache:
    """Memoises generated experts of one config (generation dominates small tests)."""

    def __init__(self, cfg: W.MoEConfig):
        self.cfg = cfg
        self._d: Dict = {}

    def __call__(self, layer: int, e: int):
        key = (layer, e)
        if key not in self._d:
            self._d[key] = W.expert(self.cfg, layer, e)
        return self._d[key]


def oracle_layers(cfg: W.MoEConfig, experts: ExpertCache, n_layers: int = None) -> List[oracle.LayerWeights]:
    n = cfg.n_layers if n_layers is None else n_layers
    return [oracle.LayerWeights(cfg.qtypes(l), cfg.H, cfg.I, cfg.down_k(l), cfg.E, cfg.k,
                                W.router(cfg, l), W.zipf_bias(cfg, l),
                                functools.partial(experts, l), cfg.n_shared) for l in range(n)]


def layer_specs(cfg: W.MoEConfig, n_layers: int = None):
    from quantized_expert_ffn_router_amd.stack import LayerSpec
    n = cfg.n_layers if n_layers is None else n_layers
    return [LayerSpec(cfg.qtypes(l), cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_shared, W.router(cfg, l),
                      W.zipf_bias(cfg, l)) for l in range(n)]


def chain_min_gap(layers: Sequence[oracle.LayerWeights]):
    """min over layers of the oracle's k-th/(k+1)-th logit gap for one token."""
    def f(x):
        outs = oracle.stack_token(layers, x)
        return min(float(o.route.gap[0]) for o in outs)
    return f


def centered_rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return oracle.rel_l2(a - a.mean(axis=-1, keepdims=True), b - b.mean(axis=-1, keepdims=True))


def sets_equal(gpu_idx: np.ndarray, ref_idx: np.ndarray) -> bool:
    return np.array_equal(np.sort(gpu_idx, axis=-1), np.sort(ref_idx, axis=-1))


def weights_by_expert(idx: np.ndarray, w: np.ndarray):
    return [dict(zip(map(int, i), map(float, ww))) for i, ww in zip(idx, w)]


def weights_close(gi, gw, ri, rw, rel=W_REL_BAR) -> bool:
    a = weights_by_expert(gi, gw)
    b = weights_by_expert(ri, rw)
    for da, db in zip(a, b):
        if set(da) != set(db):
            return False
        for e in da:
            if abs(da[e] - db[e]) > rel * abs(db[e]):
                return False
    return True


def dev_read(addr: int, nbytes: int) -> np.ndarray:
    """Copy nbytes of device memory at a raw address to the host (hipMemcpy
    of the HIP runtime that torch and libmoe share)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    out = np.empty(nbytes, np.uint8)
    rc = hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(addr), ctypes.c_size_t(nbytes),
                       ctypes.c_int(2))  # hipMemcpyDeviceToHost
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
    return out


def resident_keys(slots, layer_group, LL, EE):
    """(layer, expert) keys in the pools after the oracle LRU runs over (LL, EE)."""
    ref = oracle.lru(slots, layer_group, LL, EE)
    res = set()
    for l, e, v_l, v_e in zip(LL, EE, ref.victim_layer, ref.victim_expert):
        if v_l >= 0:
            res.discard((int(v_l), int(v_e)))
        res.add((int(l), int(e)))
    return ref, res
