"""A decode-time MoE layer stack whose experts are resident in HBM.

Each layer's experts are repacked (moe_repack_expert) into the slot layout
and stored back to back in one device buffer per layer; a device table of
their addresses (routed experts, then shared ones) is what moe_layer_forward
reads.  A decode step runs the layers in order on one stream, each layer a
pre-norm residual block h += MoE(RMSNorm(h)).

The expert bytes come from a caller-supplied function returning canonical
GGUF blocks (gate [I,H], up [I,H], down [H,Ipad]); nothing here draws data.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib as L


@dataclass
class LayerSpec:
    qtypes: Tuple[int, int, int]
    H: int
    I: int
    E: int
    k: int
    n_shared: int
    router: np.ndarray            # fp32 [E, H]
    bias: Optional[np.ndarray]    # fp32 [E] or None


def pack_layer(spec: LayerSpec, layer: int, expert_fn: Callable[[int, int], object]) -> torch.Tensor:
    """Pinned host buffer of one layer's experts (routed, then shared) in the
    slot layout, back to back."""
    desc = L.ExpertDesc.of(spec.qtypes, spec.H, spec.I)
    eb = L.moe_expert_bytes(desc)
    n = spec.E + spec.n_shared
    host = torch.empty(n * eb, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()
    for e in range(n):
        ex = expert_fn(layer, e)
        L.moe_repack_expert(desc, ex.gate, ex.up, ex.down, hv[e * eb:(e + 1) * eb])
    return host


class ResidentStack:
    def __init__(self, layers: Sequence[LayerSpec], expert_fn: Optional[Callable[[int, int], object]],
                 T_max: int = 8, device: str = "cuda", eps: float = 1e-6, threads: int = 8,
                 packed: Optional[Sequence[torch.Tensor]] = None):
        """Experts come from expert_fn(layer, e) (canonical blocks) or, when
        `packed` is given, from pinned per-layer buffers made by pack_layer."""
        self.layers = list(layers)
        self.device = torch.device(device)
        self.eps = eps
        self.T_max = T_max
        self.descs = [L.ExpertDesc.of(s.qtypes, s.H, s.I) for s in self.layers]
        self.expert_bytes = [L.moe_expert_bytes(d) for d in self.descs]
        self.bufs: List[torch.Tensor] = []
        self.tables: List[torch.Tensor] = []
        self.routers: List[torch.Tensor] = []
        self.biases: List[Optional[torch.Tensor]] = []
        for li, spec in enumerate(self.layers):
            n = spec.E + spec.n_shared
            eb = self.expert_bytes[li]
            host = packed[li] if packed is not None else pack_layer(spec, li, expert_fn)
            dev = torch.empty(n * eb, dtype=torch.uint8, device=self.device)
            dev.copy_(host, non_blocking=False)
            base = dev.data_ptr()
            tab = torch.tensor([base + e * eb for e in range(n)], dtype=torch.int64).to(self.device)
            self.bufs.append(dev)
            self.tables.append(tab)
            self.routers.append(torch.from_numpy(np.ascontiguousarray(spec.router, np.float32)).to(self.device))
            self.biases.append(None if spec.bias is None else
                               torch.from_numpy(np.ascontiguousarray(spec.bias, np.float32)).to(self.device))
        self.ws_bytes = max(L.moe_workspace_bytes(d, T_max, s.k, s.E, s.n_shared)
                            for d, s in zip(self.descs, self.layers))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        L.moe_workspace_init(self.ws, self.ws_bytes)

    def expert_ptrs(self, layer: int) -> int:
        return self.tables[layer].data_ptr()

    def shared_ptrs(self, layer: int) -> Optional[int]:
        s = self.layers[layer]
        return self.tables[layer].data_ptr() + 8 * s.E if s.n_shared else None

    def layer_forward(self, layer: int, h: torch.Tensor, idx_out=None, w_out=None, stream=None, split=False):
        """One layer through moe_layer_forward or, with split=True, through its
        two halves moe_layer_route and moe_layer_ffn."""
        s = self.layers[layer]
        T = h.shape[0]
        if split:
            L.moe_layer_route(self.descs[layer], h, T, self.routers[layer], self.biases[layer], s.E, s.k,
                              self.expert_ptrs(layer), self.shared_ptrs(layer), s.n_shared, self.eps,
                              idx_out, w_out, self.ws, self.ws_bytes, stream)
            L.moe_layer_ffn(self.descs[layer], h, T, s.E, s.k, self.expert_ptrs(layer), self.shared_ptrs(layer),
                            s.n_shared, self.ws, self.ws_bytes, stream)
            return
        L.moe_layer_forward(self.descs[layer], h, T, self.routers[layer], self.biases[layer], s.E, s.k,
                            self.expert_ptrs(layer), self.shared_ptrs(layer), s.n_shared, self.eps,
                            idx_out, w_out, self.ws, self.ws_bytes, stream)

    def chainable(self, T: int) -> bool:
        """Whether a step of T tokens can chain its layers (moe_layer_forward_chain)."""
        return all(L.moe_layer_chain_supported(d, T, s.E) for d, s in zip(self.descs, self.layers))

    def step(self, h: torch.Tensor, idx_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None,
             stream=None, split=False, chain: Optional[bool] = None):
        """One decode step through every layer; h [T, H] fp32 is updated in place.
        idx_out / w_out, if given, are [L, T, k] and receive each layer's routing.
        chain: layers through moe_layer_forward_chain (each layer's FFN starts
        the next layer's router dots; no route launch after the first layer);
        None chains whenever the step allows it (no routing outputs, no split)."""
        T = h.shape[0]
        if chain is None:
            chain = idx_out is None and w_out is None and not split and self.chainable(T)
        if chain:
            n = len(self.layers)
            for li, s in enumerate(self.layers):
                nxt = self.layers[li + 1] if li + 1 < n else None
                L.moe_layer_forward_chain(self.descs[li], h, T, self.routers[li], self.biases[li], s.E, s.k,
                                          self.expert_ptrs(li), self.shared_ptrs(li), s.n_shared, self.eps,
                                          li > 0, None if nxt is None else self.routers[li + 1],
                                          0 if nxt is None else nxt.E, li & 1, self.ws, self.ws_bytes, stream)
            return
        for li in range(len(self.layers)):
            self.layer_forward(li, h, None if idx_out is None else idx_out[li],
                               None if w_out is None else w_out[li], stream, split)

    def prompt_step(self, h: torch.Tensor, idx_out: Optional[torch.Tensor] = None,
                    w_out: Optional[torch.Tensor] = None, stream=None):
        """The same layer stack for a prompt-sized batch (up to 256 tokens, past
        the layer calls' 32): per layer moe_rmsnorm, moe_route_topk and
        moe_expert_ffn adding into h.  idx_out / w_out, if given, are [L, T, k]."""
        T, H = h.shape
        key = (T, H)
        if getattr(self, "_prompt_key", None) != key:
            kmax = max(s.k for s in self.layers)
            self._pxhat = torch.empty((T, H), dtype=torch.float32, device=self.device)
            self._pidx = torch.empty(T * kmax, dtype=torch.int32, device=self.device)
            self._pw = torch.empty(T * kmax, dtype=torch.float32, device=self.device)
            self._pws_bytes = max(L.moe_workspace_bytes(d, T, s.k, s.E, s.n_shared)
                                  for d, s in zip(self.descs, self.layers))
            self._pws = torch.empty(self._pws_bytes, dtype=torch.uint8, device=self.device)
            L.moe_workspace_init(self._pws, self._pws_bytes)
            self._prompt_key = key
        for li, s in enumerate(self.layers):
            idx = self._pidx[:T * s.k].view(T, s.k) if idx_out is None else idx_out[li]
            w = self._pw[:T * s.k].view(T, s.k) if w_out is None else w_out[li]
            L.moe_rmsnorm(h, T, H, self.eps, self._pxhat, stream)
            L.moe_route_topk(self._pxhat, T, H, self.routers[li], self.biases[li], s.E, s.k, idx, w, None, stream)
            L.moe_expert_ffn(self.descs[li], self._pxhat, T, s.k, s.E, idx, w, self.expert_ptrs(li),
                             self.shared_ptrs(li), s.n_shared, h, 1, None, self._pws, self._pws_bytes, stream)


class CachedStack:
    """A decode-time MoE stack whose routed experts live in pinned host memory
    behind an HBM slot-pool cache (moe_cache_*); shared experts and routers
    stay resident.  Layers are grouped by expert shape and type, one slot
    pool per group.  Per layer of a step: moe_layer_route; the ids are copied
    to the host; the step's distinct experts are looked up in ascending id
    (hits refresh their recency, misses take a free or the least recently
    used slot); the misses are uploaded on a side stream, which the compute
    stream then waits for; moe_layer_ffn reads the experts through the
    cache's slot table of the layer.  Layers of a group that the plan left
    with 0 slots (below the budget floor) keep their experts resident.

    device_lookup=True keeps the LRU state on the device instead
    (moe_cache_device_enable): each layer is then moe_layer_route,
    moe_cache_lookup_device (lookup and miss copies) and moe_layer_ffn on the
    current stream, with no host synchronization, so a whole step can be
    captured in a HIP graph.  trace_capacity > 0 keeps the device's lookup
    trace (device_trace).  ffn_copies (the default; device lookup without
    prefetch) copies a single token's misses inside the FFN's gate/up launch
    (moe_cache_ffn_device), so that the hit experts' work overlaps the
    copies and no copy launch runs; False keeps the copy launch.  chain=True
    (with ffn_copies) chains single-token steps as ResidentStack.step does:
    one route launch per step, each layer's FFN launches leaving the next
    layer's router dots, from which the next lookup forms its keys (measured
    no faster than the route launch it saves, so not the default).

    prefetch_depth=d > 0 (device_lookup only) adds cross-layer prefetch: at
    layer l, after its lookup, the layers up to l+d not prefetched yet in
    this step (1..d at layer 0, then l+d) have their experts predicted by
    applying their routers to layer l's input state (moe_layer_route on a
    workspace of their own) and looked up with moe_cache_prefetch_device, whose
    miss copies run on copy_stream beside the rest of the step.
    """

    def __init__(self, layers: Sequence[LayerSpec], packed: Sequence[torch.Tensor], slots: Sequence[int],
                 T_max: int = 8, device: str = "cuda", eps: float = 1e-6, device_lookup: bool = False,
                 trace_capacity: int = 0, prefetch_depth: int = 0, resident: Optional[Sequence[bool]] = None,
                 ffn_copies: bool = True, chain: bool = False):
        """resident[l] (e.g. from moe_placement_plan) keeps layer l's experts
        resident in HBM, outside the cache."""
        if prefetch_depth and not device_lookup:
            raise ValueError("prefetch_depth needs device_lookup")
        self.prefetch_depth = int(prefetch_depth)
        self.layers = list(layers)
        self.device = torch.device(device)
        self.eps = eps
        self.T_max = T_max
        self.packed = list(packed)
        self.descs = [L.ExpertDesc.of(s.qtypes, s.H, s.I) for s in self.layers]
        self.expert_bytes = [L.moe_expert_bytes(d) for d in self.descs]
        keys = []
        self.layer_group = []
        for s in self.layers:
            key = (tuple(s.qtypes), s.H, s.I)
            if key not in keys:
                keys.append(key)
            self.layer_group.append(keys.index(key))
        self.group_descs = [L.ExpertDesc.of(q, H, I) for q, H, I in keys]
        Es = {s.E for s in self.layers}
        if len(Es) != 1:
            raise ValueError("all layers of a cached stack need the same expert count")
        self.E = Es.pop()
        host_ptrs = []
        for li, s in enumerate(self.layers):
            base = self.packed[li].data_ptr()
            host_ptrs += [base + e * self.expert_bytes[li] for e in range(s.E)]
        self.slots = list(slots)
        self.resident = [bool(r) for r in resident] if resident is not None else [False] * len(self.layers)
        state = [-(g + 1) if r else g for g, r in zip(self.layer_group, self.resident)]
        self.cache = L.Cache(self.group_descs, self.slots, state, self.E, host_ptrs)
        # shared experts, routers and biases resident
        self.shared: List[Optional[torch.Tensor]] = []
        self.shared_tabs: List[Optional[torch.Tensor]] = []
        self.routers: List[torch.Tensor] = []
        self.biases: List[Optional[torch.Tensor]] = []
        for li, s in enumerate(self.layers):
            eb = self.expert_bytes[li]
            if s.n_shared:
                dev = self.packed[li][s.E * eb:(s.E + s.n_shared) * eb].to(self.device)
                self.shared.append(dev)
                self.shared_tabs.append(torch.tensor([dev.data_ptr() + j * eb for j in range(s.n_shared)],
                                                     dtype=torch.int64).to(self.device))
            else:
                self.shared.append(None)
                self.shared_tabs.append(None)
            self.routers.append(torch.from_numpy(np.ascontiguousarray(s.router, np.float32)).to(self.device))
            self.biases.append(None if s.bias is None else
                               torch.from_numpy(np.ascontiguousarray(s.bias, np.float32)).to(self.device))
        self.ws_bytes = max(L.moe_workspace_bytes(d, T_max, s.k, s.E, s.n_shared)
                            for d, s in zip(self.descs, self.layers))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        L.moe_workspace_init(self.ws, self.ws_bytes)
        kmax = max(s.k for s in self.layers)
        # ids of a layer-step: the first T*k entries, contiguous [T, k]
        self.idx_dev = torch.empty(T_max * kmax, dtype=torch.int32, device=self.device)
        self.idx_host = torch.empty(T_max * kmax, dtype=torch.int32, pin_memory=True)
        if self.prefetch_depth:
            H = self.layers[0].H
            self._fidx = torch.empty(T_max * kmax, dtype=torch.int32, device=self.device)
            self._fw = torch.empty(T_max * kmax, dtype=torch.float32, device=self.device)
            # the predictions' own workspace: the layer route kernel (router rows
            # spread over many workgroups) computes them, and its grouping and
            # records must not overwrite the current layer's
            self._fws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
            L.moe_workspace_init(self._fws, self.ws_bytes)
        self.device_lookup = device_lookup
        # a single token's misses copied inside the FFN launch (moe_cache_ffn_device;
        # device lookup without prefetch)
        self.ffn_copies = bool(ffn_copies) and device_lookup and not self.prefetch_depth
        # single-token steps chained as ResidentStack.step chains them (one route
        # launch per step; moe_cache_ffn_device with the hand-off of router dots)
        self.chain = bool(chain) and self.ffn_copies and all(
            L.moe_layer_chain_supported(dd, 1, s.E) for dd, s in zip(self.descs, self.layers))
        self.trace_capacity = trace_capacity
        if device_lookup:
            self.cache.enable_device(trace_capacity)
        # layers whose single-token route launch leaves the logit keys (E <= 128,
        # the dot-product path): their device lookup selects from the keys
        self._keys_lookup = [s.E <= 128 and s.H <= 4096 and not self.resident[li] for li, s in enumerate(self.layers)]
        self.copy_stream = torch.cuda.Stream(device=self.device)
        self.trace: Optional[list] = None
        self.time_copies = False       # record events around each layer's uploads
        self.copy_events: list = []

    def shared_ptrs(self, layer: int) -> Optional[int]:
        t = self.shared_tabs[layer]
        return None if t is None else t.data_ptr()

    def layer_forward(self, layer: int, h: torch.Tensor):
        s = self.layers[layer]
        T = h.shape[0]
        d = self.descs[layer]
        idx = self.idx_dev[:T * s.k].view(T, s.k)
        if self.chain and T == 1:
            nxt = self.layers[layer + 1] if layer + 1 < len(self.layers) else None
            if layer == 0:  # the step's one route launch
                L.moe_layer_route(d, h, T, self.routers[0], self.biases[0], s.E, s.k, None, self.shared_ptrs(0),
                                  s.n_shared, self.eps, None, None, self.ws, self.ws_bytes)
            self.cache.ffn_device(layer, d, h, s.k, self.shared_ptrs(layer), s.n_shared, self.ws, self.ws_bytes,
                                  bias=self.biases[layer], eps=self.eps, chain_in=layer > 0,
                                  next_router=None if nxt is None else self.routers[layer + 1],
                                  next_E=0 if nxt is None else nxt.E, parity=layer & 1)
            return
        if self.device_lookup and T == 1 and self._keys_lookup[layer]:
            # a single token: the route launch only writes the logit keys, and
            # the lookup kernel picks the top-k from them (no routing tail)
            L.moe_layer_route(d, h, T, self.routers[layer], self.biases[layer], s.E, s.k, None,
                              self.shared_ptrs(layer), s.n_shared, self.eps, None, None, self.ws, self.ws_bytes)
            if self.ffn_copies:
                self.cache.ffn_device(layer, d, h, s.k, self.shared_ptrs(layer), s.n_shared, self.ws, self.ws_bytes)
                return
            self.cache.lookup_device_route(layer, self.ws, self.ws_bytes, s.k)
            if self.prefetch_depth:
                self._prefetch(layer, h)
            L.moe_layer_ffn(d, h, T, s.E, s.k, self.cache.expert_ptrs(layer), self.shared_ptrs(layer), s.n_shared,
                            self.ws, self.ws_bytes)
            return
        L.moe_layer_route(d, h, T, self.routers[layer], self.biases[layer], s.E, s.k, None, self.shared_ptrs(layer),
                          s.n_shared, self.eps, idx, None, self.ws, self.ws_bytes)
        if self.device_lookup:
            self.cache.lookup_device(layer, idx, T, s.k)
            if self.prefetch_depth:
                self._prefetch(layer, h)
            L.moe_layer_ffn(d, h, T, s.E, s.k, self.cache.expert_ptrs(layer), self.shared_ptrs(layer), s.n_shared,
                            self.ws, self.ws_bytes)
            return
        ih = self.idx_host[:T * s.k].view(T, s.k)
        ih.copy_(idx, non_blocking=True)
        torch.cuda.current_stream(self.device).synchronize()
        experts, slot, hit, vl, ve = self.cache.lookup(layer, T, s.k, ih.numpy())
        if self.trace is not None:
            self.trace.append((layer, experts.copy(), hit.copy(), vl.copy(), ve.copy()))
        timed = self.time_copies and not hit.all()
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.copy_stream)
        self.cache.upload(layer, self.copy_stream)
        if timed:
            e1.record(self.copy_stream)
            self.copy_events.append((e0, e1))
        torch.cuda.current_stream(self.device).wait_stream(self.copy_stream)
        L.moe_layer_ffn(d, h, T, s.E, s.k, self.cache.expert_ptrs(layer), self.shared_ptrs(layer), s.n_shared,
                        self.ws, self.ws_bytes)

    def prompt_step(self, h: torch.Tensor, idx_out: Optional[torch.Tensor] = None):
        """A prompt-sized batch (33..256 tokens) through the cached stack: such
        batches leave the slots alone (T4 MoE-cache report, "What the MoE cache
        caches"); per layer moe_rmsnorm, moe_route_topk, the staging of the
        selected experts (copied from their slots when cached, else read from
        host memory; moe_cache_stage_large or _device) and moe_expert_ffn over
        the staged table, adding into h.  idx_out, if given, is [L, T, k]."""
        T, H = h.shape
        key = (T, H)
        if getattr(self, "_prompt_key", None) != key:
            kmax = max(s.k for s in self.layers)
            self._pxhat = torch.empty((T, H), dtype=torch.float32, device=self.device)
            self._pidx = torch.empty(T * kmax, dtype=torch.int32, device=self.device)
            self._pw = torch.empty(T * kmax, dtype=torch.float32, device=self.device)
            self._pws_bytes = max(L.moe_workspace_bytes(d, T, s.k, s.E, s.n_shared)
                                  for d, s in zip(self.descs, self.layers))
            self._pws = torch.empty(self._pws_bytes, dtype=torch.uint8, device=self.device)
            L.moe_workspace_init(self._pws, self._pws_bytes)
            self._stage_bytes = max(min(s.E, T * s.k) * eb for s, eb in zip(self.layers, self.expert_bytes))
            self._staging = torch.empty(self._stage_bytes, dtype=torch.uint8, device=self.device)
            self._stab = torch.zeros(self.E, dtype=torch.int64, device=self.device)
            self._pidx_host = torch.empty(T * kmax, dtype=torch.int32, pin_memory=True)
            self._prompt_key = key
        for li, s in enumerate(self.layers):
            idx = self._pidx[:T * s.k].view(T, s.k) if idx_out is None else idx_out[li]
            w = self._pw[:T * s.k].view(T, s.k)
            L.moe_rmsnorm(h, T, H, self.eps, self._pxhat)
            L.moe_route_topk(self._pxhat, T, H, self.routers[li], self.biases[li], s.E, s.k, idx, w, None)
            if self.device_lookup:
                self.cache.stage_large_device(li, T, s.k, idx, self._staging, self._stage_bytes, self._stab)
            else:
                ih = self._pidx_host[:T * s.k]
                ih.copy_(idx.reshape(-1), non_blocking=True)
                torch.cuda.current_stream(self.device).synchronize()
                self.cache.stage_large(li, T, s.k, ih.numpy(), self._staging, self._stage_bytes, self._stab)
            L.moe_expert_ffn(self.descs[li], self._pxhat, T, s.k, s.E, idx, w, self._stab, self.shared_ptrs(li),
                             s.n_shared, h, 1, None, self._pws, self._pws_bytes)

    def prefetch_targets(self, layer: int) -> List[int]:
        """Layers whose experts are prefetched at `layer` (before its FFN)."""
        d, n = self.prefetch_depth, len(self.layers)
        first = 1 if layer == 0 else layer + d
        return [m for m in range(first, min(layer + d, n - 1) + 1)] if d else []

    def _prefetch(self, layer: int, h: torch.Tensor):
        T = h.shape[0]
        for m in self.prefetch_targets(layer):
            s = self.layers[m]
            idx = self._fidx[:T * s.k].view(T, s.k)
            L.moe_layer_route(self.descs[m], h, T, self.routers[m], self.biases[m], s.E, s.k, None,
                              self.shared_ptrs(m), s.n_shared, self.eps, idx, self._fw[:T * s.k].view(T, s.k),
                              self._fws, self.ws_bytes)
            self.cache.prefetch_device(m, idx, T, s.k, self.copy_stream)

    def step(self, h: torch.Tensor):
        """One decode step through every layer; h [T, H] fp32 is updated in place."""
        for li in range(len(self.layers)):
            self.layer_forward(li, h)

    def device_trace(self):
        """The device lookups so far as (layer, expert, hit, victim_layer,
        victim_expert) int32 arrays (device_lookup with a trace_capacity)."""
        t = self.cache.trace_read(self.trace_capacity)
        vk = t[:, 3]
        vl = np.where(vk >= 0, vk // self.E, -1).astype(np.int32)
        ve = np.where(vk >= 0, vk % self.E, -1).astype(np.int32)
        return t[:, 0].copy(), t[:, 1].copy(), t[:, 2].astype(np.uint8), vl, ve

    def copy_ms(self) -> float:
        """Sum of the timed upload intervals (after a synchronisation)."""
        return sum(a.elapsed_time(b) for a, b in self.copy_events)

    def close(self):
        torch.cuda.synchronize(self.device)
        self.cache.close()
