"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_Q8_0, MOE_Q4_K, MOE_Q6_K = 1, 2, 3

EXPORTED = [
    "moe_last_error", "moe_expert_bytes", "moe_down_k", "moe_repack_expert",
    "moe_rmsnorm", "moe_route_topk", "moe_group_tokens", "moe_workspace_bytes",
    "moe_workspace_init", "moe_workspace_status", "moe_set_spin_limit", "moe_expert_ffn", "moe_layer_route", "moe_layer_ffn", "moe_layer_forward",
    "moe_layer_forward_noalloc", "moe_layer_forward_chain", "moe_layer_chain_supported",
    "moe_cache_plan", "moe_placement_plan", "moe_cache_create", "moe_cache_create_ex", "moe_cache_lookup", "moe_cache_upload",
    "moe_cache_expert_ptrs", "moe_cache_stats", "moe_cache_reset_stats", "moe_cache_destroy",
    "moe_cache_device_enable", "moe_cache_lookup_device", "moe_cache_lookup_device_route", "moe_cache_ffn_device",
    "moe_cache_prefetch_device",
    "moe_cache_trace_read",
    "moe_cache_stage_large", "moe_cache_stage_large_device",
]

_STATUS = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_QTYPE",
           -4: "MOE_ERR_BUDGET", -5: "MOE_ERR_CAPACITY", -6: "MOE_ERR_HIP", -7: "MOE_ERR_BATCH",
           -8: "MOE_ERR_STATE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


class ExpertDesc(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_int32), ("up", ctypes.c_int32), ("down", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32)]

    @classmethod
    def of(cls, qtypes, H: int, I: int) -> "ExpertDesc":
        return cls(int(qtypes[0]), int(qtypes[1]), int(qtypes[2]), int(H), int(I))


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "lookups", "hits", "misses", "evictions", "upload_bytes",
        "lookups_le8", "hits_le8", "lookups_9_32", "hits_9_32", "large_copies", "large_uploads")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


BackendAlloc = ctypes.CFUNCTYPE(ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p))
BackendRelease = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)
BackendCopy = ctypes.CFUNCTYPE(ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t)


class CacheBackend(ctypes.Structure):
    """moe_cache_backend: a synchronous pool allocator and copier (see moe.h)."""
    _fields_ = [("user", ctypes.c_void_p), ("alloc", BackendAlloc), ("release", BackendRelease),
                ("copy", BackendCopy)]

    @classmethod
    def of(cls, alloc, release, copy) -> "CacheBackend":
        """Python callables alloc(nbytes) -> address (0 on failure), release(address),
        copy(dst, src, nbytes) -> 0 on success.  The returned structure keeps the
        ctypes thunks alive; keep it alive as long as the cache."""
        def _alloc(_u, n, out):
            a = int(alloc(int(n)) or 0)
            out[0] = a
            return 0 if a else 1

        def _release(_u, p):
            release(int(p or 0))

        def _copy(_u, dst, src, n):
            return int(copy(int(dst or 0), int(src or 0), int(n)))

        b = cls(None, BackendAlloc(_alloc), BackendRelease(_release), BackendCopy(_copy))
        b._keep = (_alloc, _release, _copy)
        return b


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with quantized_expert_ffn_router_amd/build.py")
    L = ctypes.CDLL(_LIB_PATH)
    P, i32, u64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(ExpertDesc)
    sig = {
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_expert_bytes": (ctypes.c_int64, [D]),
        "moe_down_k": (i32, [D]),
        "moe_repack_expert": (i32, [D, P, P, P, P, sz]),
        "moe_rmsnorm": (i32, [P, i32, i32, f32, P, P]),
        "moe_route_topk": (i32, [P, i32, i32, P, P, i32, i32, P, P, P, P]),
        "moe_group_tokens": (i32, [P, i32, i32, i32, P, P, P, P]),
        "moe_workspace_bytes": (sz, [D, i32, i32, i32, i32]),
        "moe_workspace_init": (i32, [P, sz, P]),
        "moe_workspace_status": (i32, [P, sz, P, P]),
        "moe_set_spin_limit": (None, [ctypes.c_uint32, i32]),
        "moe_expert_ffn": (i32, [D, P, i32, i32, i32, P, P, P, P, i32, P, i32, P, P, sz, P]),
        "moe_layer_route": (i32, [D, P, i32, P, P, i32, i32, P, P, i32, f32, P, P, P, sz, P]),
        "moe_layer_ffn": (i32, [D, P, i32, i32, i32, P, P, i32, P, sz, P]),
        "moe_layer_forward": (i32, [D, P, i32, P, P, i32, i32, P, P, i32, f32, P, P, P, sz, P]),
        "moe_layer_forward_noalloc": (i32, [D, P, i32, P, P, i32, i32, P, P, i32, f32, P, P, P]),
        "moe_layer_forward_chain": (i32, [D, P, i32, P, P, i32, i32, P, P, i32, f32, i32, P, i32, i32, P, sz, P]),
        "moe_layer_chain_supported": (i32, [D, i32, i32]),
        "moe_cache_plan": (i32, [D, P, i32, u64, i32, P]),
        "moe_placement_plan": (i32, [D, i32, P, i32, i32, u64, u64, i32, i32, P, P]),
        "moe_cache_create": (i32, [D, i32, P, P, i32, i32, P, ctypes.POINTER(P)]),
        "moe_cache_create_ex": (i32, [D, i32, P, P, i32, i32, P, ctypes.POINTER(CacheBackend), ctypes.POINTER(P)]),
        "moe_cache_lookup": (i32, [P, i32, i32, i32, P, P, P, P, P, P, P]),
        "moe_cache_upload": (i32, [P, i32, P, P]),
        "moe_cache_expert_ptrs": (P, [P, i32]),
        "moe_cache_stats": (i32, [P, ctypes.POINTER(CacheStats)]),
        "moe_cache_reset_stats": (i32, [P]),
        "moe_cache_device_enable": (i32, [P, i32]),
        "moe_cache_lookup_device": (i32, [P, i32, P, i32, i32, P]),
        "moe_cache_lookup_device_route": (i32, [P, i32, P, sz, i32, P]),
        "moe_cache_ffn_device": (i32, [P, i32, D, P, i32, P, i32, P, f32, i32, P, i32, i32, P, sz, P]),
        "moe_cache_prefetch_device": (i32, [P, i32, P, i32, i32, P, P]),
        "moe_cache_trace_read": (i32, [P, P, i32, P]),
        "moe_cache_stage_large": (i32, [P, i32, i32, i32, P, P, sz, P, P]),
        "moe_cache_stage_large_device": (i32, [P, i32, i32, i32, P, P, sz, P, P]),
        "moe_cache_destroy": (None, [P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(st: int):
    if st != 0:
        raise MoeError(st, lib().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device/host address of a torch tensor or numpy array (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _desc(d) -> ExpertDesc:
    return d if isinstance(d, ExpertDesc) else ExpertDesc.of(*d)


# ---------------------------------------------------------------- layout

def moe_expert_bytes(desc) -> int:
    n = lib().moe_expert_bytes(ctypes.byref(_desc(desc)))
    if n < 0:
        raise MoeError(-2, "bad expert desc")
    return n


def moe_down_k(desc) -> int:
    n = lib().moe_down_k(ctypes.byref(_desc(desc)))
    if n < 0:
        raise MoeError(-2, "bad expert desc")
    return n


def moe_repack_expert(desc, gate: np.ndarray, up: np.ndarray, down: np.ndarray, out: Optional[np.ndarray] = None
                      ) -> np.ndarray:
    """Host repack of one expert (canonical blocks -> slot layout)."""
    d = _desc(desc)
    n = moe_expert_bytes(d)
    if out is None:
        out = np.empty(n, np.uint8)
    g, u, dn = (np.ascontiguousarray(a, np.uint8) for a in (gate, up, down))
    _check(lib().moe_repack_expert(ctypes.byref(d), g.ctypes.data, u.ctypes.data, dn.ctypes.data,
                                   out.ctypes.data, out.nbytes))
    return out


# ---------------------------------------------------------------- steps

def moe_rmsnorm(h, T: int, H: int, eps: float, xhat, stream=None):
    _check(lib().moe_rmsnorm(_ptr(h), T, H, eps, _ptr(xhat), _stream(stream)))


def moe_route_topk(x, T: int, H: int, w_router, bias, E: int, k: int, idx, w, logits=None, stream=None):
    _check(lib().moe_route_topk(_ptr(x), T, H, _ptr(w_router), _ptr(bias), E, k, _ptr(idx), _ptr(w),
                                _ptr(logits), _stream(stream)))


def moe_group_tokens(idx, T: int, k: int, E: int, count, offset, pairs, stream=None):
    _check(lib().moe_group_tokens(_ptr(idx), T, k, E, _ptr(count), _ptr(offset), _ptr(pairs), _stream(stream)))


def moe_workspace_bytes(desc, T: int, k: int, E: int, n_shared: int = 0) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(_desc(desc)), T, k, E, n_shared)
    if n == 0:
        raise MoeError(-1, "bad workspace arguments")
    return n


def moe_workspace_init(ws, nbytes: int, stream=None):
    """ws None: the static scratch of moe_layer_forward_noalloc on the current device."""
    _check(lib().moe_workspace_init(_ptr(ws), nbytes, _stream(stream)))


MOE_WS_KEYS_TIMEOUT, MOE_WS_TOPK_TIMEOUT = 1, 2
MOE_WS_STATUS_OFFSET = 147456  # byte offset of the status word in every workspace


def moe_workspace_status(ws, nbytes: int, stream=None) -> int:
    """The workspace's status word (MOE_WS_* bits; 0 = no wait gave up).
    Stream-synchronous.  ws None: the static scratch of the current device."""
    out = ctypes.c_uint32(0)
    _check(lib().moe_workspace_status(_ptr(ws), nbytes, ctypes.byref(out), _stream(stream)))
    return int(out.value)


def moe_set_spin_limit(rounds: int, withhold_keys: bool = False):
    """Test hook: polling rounds before the route launch's waits give up
    (0: default); withhold_keys makes every wait for the keys give up."""
    lib().moe_set_spin_limit(int(rounds), 1 if withhold_keys else 0)


def moe_expert_ffn(desc, x, T: int, k: int, E: int, idx, w, expert_ptrs, shared_ptrs, n_shared: int, y,
                   accumulate: int, act_out, ws, ws_bytes: int, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(_desc(desc)), _ptr(x), T, k, E, _ptr(idx), _ptr(w), _ptr(expert_ptrs),
                                _ptr(shared_ptrs), n_shared, _ptr(y), accumulate, _ptr(act_out), _ptr(ws),
                                ws_bytes, _stream(stream)))


def moe_layer_forward(desc, h, T: int, w_router, bias, E: int, k: int, expert_ptrs, shared_ptrs, n_shared: int,
                      eps: float, idx_out, w_out, ws, ws_bytes: int, stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(_desc(desc)), _ptr(h), T, _ptr(w_router), _ptr(bias), E, k,
                                   _ptr(expert_ptrs), _ptr(shared_ptrs), n_shared, eps, _ptr(idx_out),
                                   _ptr(w_out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward_noalloc(desc, h, T: int, w_router, bias, E: int, k: int, expert_ptrs, shared_ptrs,
                              n_shared: int, eps: float, idx_out, w_out, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(_desc(desc)), _ptr(h), T, _ptr(w_router), _ptr(bias), E, k,
                                           _ptr(expert_ptrs), _ptr(shared_ptrs), n_shared, eps, _ptr(idx_out),
                                           _ptr(w_out), _stream(stream)))


def moe_layer_forward_chain(desc, h, T: int, w_router, bias, E: int, k: int, expert_ptrs, shared_ptrs,
                            n_shared: int, eps: float, chain_in: bool, next_router, next_E: int, parity: int,
                            ws, ws_bytes: int, stream=None):
    _check(lib().moe_layer_forward_chain(ctypes.byref(_desc(desc)), _ptr(h), T, _ptr(w_router), _ptr(bias), E, k,
                                         _ptr(expert_ptrs), _ptr(shared_ptrs), n_shared, eps, int(bool(chain_in)),
                                         _ptr(next_router), next_E, parity, _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_chain_supported(desc, T: int, E: int) -> bool:
    return bool(lib().moe_layer_chain_supported(ctypes.byref(_desc(desc)), T, E))


def moe_layer_route(desc, h, T: int, w_router, bias, E: int, k: int, expert_ptrs, shared_ptrs, n_shared: int,
                    eps: float, idx_out, w_out, ws, ws_bytes: int, stream=None):
    _check(lib().moe_layer_route(ctypes.byref(_desc(desc)), _ptr(h), T, _ptr(w_router), _ptr(bias), E, k,
                                 _ptr(expert_ptrs), _ptr(shared_ptrs), n_shared, eps, _ptr(idx_out), _ptr(w_out),
                                 _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_ffn(desc, h, T: int, E: int, k: int, expert_ptrs, shared_ptrs, n_shared: int, ws, ws_bytes: int,
                  stream=None):
    _check(lib().moe_layer_ffn(ctypes.byref(_desc(desc)), _ptr(h), T, E, k, _ptr(expert_ptrs), _ptr(shared_ptrs),
                               n_shared, _ptr(ws), ws_bytes, _stream(stream)))


# ---------------------------------------------------------------- cache

def moe_cache_plan(descs: Sequence, layers_per_group: Sequence[int], budget_bytes: int, top_k: int):
    """Returns (status, slots).  status is 0 or the MOE_ERR_BUDGET code."""
    n = len(descs)
    arr = (ExpertDesc * n)(*[_desc(d) for d in descs])
    lay = np.asarray(layers_per_group, np.int32)
    slots = np.zeros(n, np.int32)
    st = lib().moe_cache_plan(arr, lay.ctypes.data, n, int(budget_bytes), top_k, slots.ctypes.data)
    if st not in (0, -4):
        _check(st)
    return st, slots


MOE_PLACE_FIT, MOE_PLACE_ALL_CACHED = 1, 2


def moe_placement_plan(descs: Sequence, layer_group: Sequence[int], E: int, vram_bytes: int, cache_bytes: int,
                       top_k: int, mode: int):
    """Returns (status, layer_state, slots); status is 0 or the MOE_ERR_BUDGET
    code.  layer_state[l] = g (cached) or -(g+1) (resident)."""
    n = len(descs)
    arr = (ExpertDesc * n)(*[_desc(d) for d in descs])
    lg = np.ascontiguousarray(layer_group, np.int32)
    state = np.zeros(lg.shape[0], np.int32)
    slots = np.zeros(n, np.int32)
    st = lib().moe_placement_plan(arr, n, lg.ctypes.data, lg.shape[0], E, int(vram_bytes), int(cache_bytes), top_k,
                                  mode, state.ctypes.data, slots.ctypes.data)
    if st not in (0, -4):
        _check(st)
    return st, state, slots


class Cache:
    """Owner of a moe_cache* (moe_cache_create / moe_cache_create_ex / moe_cache_destroy)."""

    def __init__(self, descs: Sequence, slots: Sequence[int], layer_group: Sequence[int], E: int,
                 host_expert_ptrs: Sequence[int], backend: Optional[CacheBackend] = None):
        n = len(descs)
        self._descs = (ExpertDesc * n)(*[_desc(d) for d in descs])
        self._slots = np.asarray(slots, np.int32)
        self._lg = np.asarray(layer_group, np.int32)
        self._hp = np.asarray(host_expert_ptrs, np.uint64)
        self._backend = backend
        self.n_layers = len(self._lg)
        self.E = E
        h = ctypes.c_void_p()
        self.h = None
        if backend is None:
            st = lib().moe_cache_create(self._descs, n, self._slots.ctypes.data, self._lg.ctypes.data,
                                        self.n_layers, E, self._hp.ctypes.data, ctypes.byref(h))
        else:
            st = lib().moe_cache_create_ex(self._descs, n, self._slots.ctypes.data, self._lg.ctypes.data,
                                           self.n_layers, E, self._hp.ctypes.data, ctypes.byref(backend),
                                           ctypes.byref(h))
        _check(st)
        self.h = h

    def lookup(self, layer: int, T: int, k: int, idx: np.ndarray):
        """Host LRU lookup of one layer-step from its raw selected ids (host
        int32 [T*k]).  Returns (experts, slot, hit, victim_layer,
        victim_expert) over the step's distinct experts, ascending."""
        ids = np.ascontiguousarray(np.asarray(idx).reshape(-1)[:T * k], np.int32)
        if ids.shape[0] != T * k:
            raise ValueError("idx must hold T*k ids")
        ex = np.empty(T * k, np.int32)
        n = ctypes.c_int32()
        slot = np.empty(T * k, np.int32)
        hit = np.empty(T * k, np.uint8)
        vl = np.empty(T * k, np.int32)
        ve = np.empty(T * k, np.int32)
        _check(lib().moe_cache_lookup(self.h, layer, T, k, ids.ctypes.data, ex.ctypes.data, ctypes.byref(n),
                                      slot.ctypes.data, hit.ctypes.data, vl.ctypes.data, ve.ctypes.data))
        m = n.value
        return ex[:m], slot[:m], hit[:m], vl[:m], ve[:m]

    def upload(self, layer: int, copy_stream, done_event=None):
        ev = None if done_event is None else done_event.cuda_event if hasattr(done_event, "cuda_event") else done_event
        cs = None if (copy_stream is None and self._backend is not None) else _stream(copy_stream)
        _check(lib().moe_cache_upload(self.h, layer, cs, ev))

    def enable_device(self, trace_capacity: int = 0):
        """Move the LRU state to the device (moe_cache_device_enable)."""
        _check(lib().moe_cache_device_enable(self.h, int(trace_capacity)))

    def lookup_device(self, layer: int, idx, T: int, k: int, stream=None):
        """Device lookup + miss uploads of one layer-step (moe_cache_lookup_device);
        idx: int32 [T, k] contiguous, on the device."""
        import torch
        if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous() or idx.numel() < T * k:
            raise ValueError("idx must be a contiguous int32 device tensor of T*k ids")
        _check(lib().moe_cache_lookup_device(self.h, layer, idx.data_ptr(), T, k, _stream(stream)))

    def lookup_device_route(self, layer: int, ws, ws_bytes: int, k: int, stream=None):
        """Device lookup of a single token from the logit keys the preceding
        moe_layer_route (without idx_out) left in ws (moe_cache_lookup_device_route)."""
        _check(lib().moe_cache_lookup_device_route(self.h, layer, _ptr(ws), ws_bytes, k, _stream(stream)))

    def ffn_device(self, layer: int, desc, h, k: int, shared_ptrs, n_shared: int, ws, ws_bytes: int,
                   bias=None, eps: float = 0.0, chain_in: bool = False, next_router=None, next_E: int = 0,
                   parity: int = 0, stream=None):
        """A single token's device lookup and the layer's FFN, the misses copied
        inside the FFN launch; chained layers as in moe_layer_forward_chain
        (moe_cache_ffn_device)."""
        _check(lib().moe_cache_ffn_device(self.h, layer, ctypes.byref(_desc(desc)), _ptr(h), k, _ptr(shared_ptrs),
                                          n_shared, _ptr(bias), eps, int(bool(chain_in)), _ptr(next_router), next_E,
                                          parity, _ptr(ws), ws_bytes, _stream(stream)))

    def prefetch_device(self, layer: int, idx, T: int, k: int, copy_stream, stream=None):
        """Prefetch of predicted ids for `layer` (moe_cache_prefetch_device):
        the lookup on `stream`, the miss copies on `copy_stream`."""
        import torch
        if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous() or idx.numel() < T * k:
            raise ValueError("idx must be a contiguous int32 device tensor of T*k ids")
        _check(lib().moe_cache_prefetch_device(self.h, layer, idx.data_ptr(), T, k, _stream(stream),
                                               _stream(copy_stream)))

    def stage_large(self, layer: int, T: int, k: int, idx, staging, staging_bytes: int, table_out, stream=None):
        """Stage a large batch's experts (moe_cache_stage_large): idx host
        int32 [T*k] (numpy), staging / table_out device addresses or tensors."""
        ids = np.ascontiguousarray(np.asarray(idx).reshape(-1)[:T * k], np.int32)
        cs = None if (stream is None and self._backend is not None) else _stream(stream)
        _check(lib().moe_cache_stage_large(self.h, layer, T, k, ids.ctypes.data, _ptr(staging), int(staging_bytes),
                                           _ptr(table_out), cs))

    def stage_large_device(self, layer: int, T: int, k: int, idx, staging, staging_bytes: int, table_out, stream=None):
        """moe_cache_stage_large_device: idx a device int32 tensor of T*k ids."""
        _check(lib().moe_cache_stage_large_device(self.h, layer, T, k, _ptr(idx), _ptr(staging), int(staging_bytes),
                                                  _ptr(table_out), _stream(stream)))

    def trace_read(self, capacity: int) -> np.ndarray:
        """The device trace: int32 [n, 4] (layer, expert, hit, evicted key or -1)."""
        out = np.empty((max(capacity, 0), 4), np.int32)
        n = ctypes.c_int32()
        _check(lib().moe_cache_trace_read(self.h, out.ctypes.data, out.shape[0], ctypes.byref(n)))
        return out[:min(n.value, out.shape[0])]

    def expert_ptrs(self, layer: int) -> int:
        p = lib().moe_cache_expert_ptrs(self.h, layer)
        if not p:
            _check(-1)
        return p

    def stats(self) -> dict:
        s = CacheStats()
        _check(lib().moe_cache_stats(self.h, ctypes.byref(s)))
        return s.as_dict()

    def reset_stats(self):
        _check(lib().moe_cache_reset_stats(self.h))

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
