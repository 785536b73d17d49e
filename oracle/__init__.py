"""Plain fp64 CPU oracle for the decode-time MoE expert FFN.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only callers.  It shares no code with the GPU
library (quantized_expert_ffn_router_amd); neither imports the other.

The arithmetic lives in moe_oracle.c (fp64 dequantization by the closed
forms, fp64 matvecs, router/top-k, grouping, slot planner, exact LRU).  This
module builds that file with gcc, binds it with ctypes, and composes the
per-token MoE layer and the layer stack from it:

    xhat   = RMSNorm(h)                          (weightless, eps 1e-6)
    idx, w = top-k of router logits, softmax renormalised over the k
    y      = sum_j w_j * FFN_{idx_j}(xhat) + sum_s FFN_shared_s(xhat)
    h'     = h + y

Sources: routing and the softmax top-k follow the MoE offload blog
(mhpn.cn, section 3.1); gate/up/down expert tensors and the cache's scope
(router and shared experts never cached) follow the T4 MoE-cache report
(kongchang.com, section "What the MoE cache caches"); shared always-active
experts follow the laptop 16B MoE post (lpnh.cn, section 2.1).  The SiLU
gating, the renormalisation and the residual pre-norm stack are readings of
points the pages leave open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

RMS_EPS = 1e-6


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (-O2, OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, f64, u64 = ctypes.c_int, ctypes.c_double, ctypes.c_uint64
        L.orc_half.restype = f64
        L.orc_half.argtypes = [ctypes.c_uint16]
        L.orc_dequant_row.argtypes = [i32, P, i32, P]
        L.orc_qmatvec.argtypes = [i32, P, i32, i32, P, P]
        L.orc_rmsnorm.argtypes = [P, i32, f64, P]
        L.orc_route.argtypes = [P, P, P, i32, i32, i32, P, P, P, P]
        L.orc_silu.restype = f64
        L.orc_silu.argtypes = [f64]
        L.orc_expert_ffn.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.orc_group.argtypes = [P, i32, i32, i32, P, P, P]
        L.orc_cache_plan.argtypes = [i32, P, P, u64, i32, P]
        L.orc_lru.argtypes = [i32, P, P, i32, i32, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------------------
# primitives

BLOCK_WEIGHTS = {1: 32, 2: 256, 3: 256}
BLOCK_BYTES = {1: 34, 2: 144, 3: 210}


def half(bits: int) -> float:
    return lib().orc_half(bits)


def dequant_row(qtype: int, row: np.ndarray, k: int) -> np.ndarray:
    out = np.empty(k, np.float64)
    row = _c(row, np.uint8)
    if lib().orc_dequant_row(qtype, _p(row), k, _p(out)) != 0:
        raise ValueError("bad qtype or row length")
    return out


def dequant_matrix(qtype: int, w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8).reshape(n, -1)
    return np.stack([dequant_row(qtype, w[r], k) for r in range(n)])


def qmatvec(qtype: int, w: np.ndarray, n: int, k: int, x: np.ndarray) -> np.ndarray:
    w = _c(w, np.uint8)
    x = _c(x, np.float64)
    y = np.empty(n, np.float64)
    if lib().orc_qmatvec(qtype, _p(w), n, k, _p(x), _p(y)) != 0:
        raise ValueError("bad qtype or shape")
    return y


def rmsnorm(h: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Weightless RMSNorm of the state as given (fp64; an fp32 state is
    passed exactly)."""
    h = _c(h, np.float64)
    out = np.empty(h.shape, np.float64)
    for t in range(h.shape[0]) if h.ndim == 2 else [None]:
        src = h[t] if t is not None else h
        dst = np.empty(src.shape[0], np.float64)
        lib().orc_rmsnorm(_p(np.ascontiguousarray(src)), src.shape[0], eps, _p(dst))
        if t is None:
            out = dst
        else:
            out[t] = dst
    return out


@dataclass
class Route:
    idx: np.ndarray      # int32 [T, k], ordered by (logit desc, id asc)
    w: np.ndarray        # fp64 [T, k], renormalised softmax over the k winners
    logits: np.ndarray   # fp64 [T, E]
    gap: np.ndarray      # fp64 [T], k-th minus (k+1)-th logit


def route(x: np.ndarray, wr: np.ndarray, bias: Optional[np.ndarray], k: int) -> Route:
    """x: fp64 [T, H] (already normalised), wr: fp32 [E, H], bias: fp32 [E] or None."""
    x = np.atleast_2d(_c(x, np.float64))
    wr = _c(wr, np.float32)
    E, H = wr.shape
    b = None if bias is None else _c(bias, np.float32)
    T = x.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lg = np.empty((T, E), np.float64)
    gap = np.empty(T, np.float64)
    for t in range(T):
        xi = np.ascontiguousarray(x[t])
        ii = np.empty(k, np.int32)
        ww = np.empty(k, np.float64)
        ll = np.empty(E, np.float64)
        g = np.empty(1, np.float64)
        if lib().orc_route(_p(xi), _p(wr), _p(b), E, H, k, _p(ii), _p(ww), _p(ll), _p(g)) != 0:
            raise ValueError("bad k")
        idx[t], w[t], lg[t], gap[t] = ii, ww, ll, g[0]
    return Route(idx, w, lg, gap)


def silu(g: float) -> float:
    return lib().orc_silu(g)


@dataclass
class FFNOut:
    g: np.ndarray
    u: np.ndarray
    a: np.ndarray   # SiLU(g)*u, zero-padded to the down row length
    o: np.ndarray


def expert_ffn(qtypes: Tuple[int, int, int], H: int, I: int, kd: int,
               gate: np.ndarray, up: np.ndarray, down: np.ndarray, x: np.ndarray) -> FFNOut:
    qg, qu, qd = qtypes
    gate, up, down = (_c(m, np.uint8) for m in (gate, up, down))
    x = _c(x, np.float64)
    g = np.empty(I, np.float64)
    u = np.empty(I, np.float64)
    a = np.empty(kd, np.float64)
    o = np.empty(H, np.float64)
    rc = lib().orc_expert_ffn(qg, qu, qd, H, I, kd, _p(gate), _p(up), _p(down), _p(x),
                              _p(g), _p(u), _p(a), _p(o))
    if rc != 0:
        raise ValueError(f"orc_expert_ffn failed ({rc})")
    return FFNOut(g, u, a, o)


@dataclass
class Grouping:
    count: np.ndarray    # int32 [E]
    offset: np.ndarray   # int32 [E+1]
    pairs: np.ndarray    # int32 [T*k], entries t*k+j ordered by (expert, token, slot)


def group(idx: np.ndarray, E: int) -> Grouping:
    idx = _c(idx, np.int32)
    T, k = idx.shape
    count = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    pairs = np.empty(T * k, np.int32)
    if lib().orc_group(_p(idx), T, k, E, _p(count), _p(off), _p(pairs)) != 0:
        raise ValueError("expert id out of range")
    return Grouping(count, off, pairs)


def cache_plan(expert_bytes: Sequence[int], layers: Sequence[int], budget: int, top_k: int
               ) -> Tuple[int, np.ndarray]:
    eb = np.asarray(expert_bytes, np.int64)
    ly = np.asarray(layers, np.int32)
    slots = np.empty(len(eb), np.int32)
    rc = lib().orc_cache_plan(len(eb), _p(eb), _p(ly), int(budget), top_k, _p(slots))
    return rc, slots


@dataclass
class LRUTrace:
    hit: np.ndarray            # uint8 [n]
    victim_layer: np.ndarray   # int32 [n], -1 = none
    victim_expert: np.ndarray  # int32 [n]
    slot: np.ndarray           # int32 [n]


def lru(slots: Sequence[int], layer_group: Sequence[int], lookups_layer: np.ndarray,
        lookups_expert: np.ndarray) -> LRUTrace:
    sl = np.asarray(slots, np.int32)
    lg = np.asarray(layer_group, np.int32)
    ll = _c(lookups_layer, np.int32)
    le = _c(lookups_expert, np.int32)
    n = ll.shape[0]
    hit = np.empty(n, np.uint8)
    vl = np.empty(n, np.int32)
    ve = np.empty(n, np.int32)
    so = np.empty(n, np.int32)
    rc = lib().orc_lru(len(sl), _p(sl), _p(lg), len(lg), n, _p(ll), _p(le), _p(hit), _p(vl), _p(ve), _p(so))
    if rc != 0:
        raise ValueError(f"orc_lru failed ({rc})")
    return LRUTrace(hit, vl, ve, so)


def lookup_sequence(ids: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """ids: int [steps, layers, T*k] routed expert ids.  Returns the (layer,
    expert) lookup order: step by step, layer by layer, and within each
    layer-step the distinct experts once each in ascending id."""
    L_, E_ = [], []
    steps, layers = ids.shape[:2]
    for s in range(steps):
        for l in range(layers):
            for e in np.unique(ids[s, l]):
                L_.append(l)
                E_.append(int(e))
    return np.asarray(L_, np.int32), np.asarray(E_, np.int32)


def prefetch_lookup_sequence(ids: np.ndarray, pred: np.ndarray, targets: Sequence[Sequence[int]]
                             ) -> Tuple[np.ndarray, np.ndarray]:
    """Lookup order of a stack that prefetches the experts of later layers
    while the current one computes (Laptop post, section 2.3).  ids, pred:
    int [steps, layers, T*k], the routed ids and the ids predicted for each
    layer; targets[l]: the layers whose predicted experts are looked up at
    layer l, after layer l's own lookup.  Within each lookup the distinct
    ids come once each in ascending order, as in lookup_sequence."""
    L_, E_ = [], []
    steps, layers = ids.shape[:2]
    for s in range(steps):
        for l in range(layers):
            for m, row in [(l, ids[s, l])] + [(m, pred[s, m]) for m in targets[l]]:
                for e in np.unique(row):
                    L_.append(m)
                    E_.append(int(e))
    return np.asarray(L_, np.int32), np.asarray(E_, np.int32)


# ---------------------------------------------------------------------------
# layer and stack composition (per token; tokens are independent)

@dataclass
class LayerWeights:
    qtypes: Tuple[int, int, int]
    H: int
    I: int
    kd: int
    E: int
    k: int
    router: np.ndarray                 # fp32 [E, H]
    bias: Optional[np.ndarray]         # fp32 [E] or None
    expert: Callable[[int], object]    # e -> object with .gate .up .down canonical bytes
    n_shared: int = 0                  # shared experts are expert(E + s)


@dataclass
class LayerOut:
    xhat: np.ndarray   # fp64 [H]
    route: Route
    y: np.ndarray      # fp64 [H]
    h_next: np.ndarray  # fp64 [H]
    per_expert: Dict[int, FFNOut]


def moe_layer_token(lw: LayerWeights, h: np.ndarray, keep: bool = False) -> LayerOut:
    """One pre-norm residual MoE layer on one token.  h is the residual
    state, normalised and added to exactly as given (stack_token rounds it
    to fp32 between layers, the state's storage type)."""
    xhat = rmsnorm(np.asarray(h, np.float64))
    r = route(xhat[None, :], lw.router, lw.bias, lw.k)
    y = np.zeros(lw.H, np.float64)
    per = {}
    for j in range(lw.k):
        e = int(r.idx[0, j])
        ex = lw.expert(e)
        f = expert_ffn(lw.qtypes, lw.H, lw.I, lw.kd, ex.gate, ex.up, ex.down, xhat)
        y += r.w[0, j] * f.o
        if keep:
            per[e] = f
    for s in range(lw.n_shared):
        ex = lw.expert(lw.E + s)
        f = expert_ffn(lw.qtypes, lw.H, lw.I, lw.kd, ex.gate, ex.up, ex.down, xhat)
        y += f.o
        if keep:
            per[lw.E + s] = f
    return LayerOut(xhat, r, y, np.asarray(h, np.float64) + y, per)


def stack_token(layers: Sequence[LayerWeights], h0: np.ndarray, keep: bool = False,
                round_state_to_fp32: bool = True) -> List[LayerOut]:
    """Run one token through the layer stack.  The residual state is rounded
    to fp32 between layers (the state's storage type); everything inside a
    layer is fp64."""
    outs = []
    h = np.asarray(h0, np.float64)
    for lw in layers:
        o = moe_layer_token(lw, h, keep)
        outs.append(o)
        h = o.h_next.astype(np.float32).astype(np.float64) if round_state_to_fp32 else o.h_next
    return outs


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))
