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


class ResidentStack:
    def __init__(self, layers: Sequence[LayerSpec], expert_fn: Callable[[int, int], object],
                 T_max: int = 8, device: str = "cuda", eps: float = 1e-6, threads: int = 8):
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
            host = torch.empty(n * eb, dtype=torch.uint8, pin_memory=True)
            hv = host.numpy()
            for e in range(n):
                ex = expert_fn(li, e)
                L.moe_repack_expert(self.descs[li], ex.gate, ex.up, ex.down, hv[e * eb:(e + 1) * eb])
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

    def step(self, h: torch.Tensor, idx_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None,
             stream=None, split=False):
        """One decode step through every layer; h [T, H] fp32 is updated in place.
        idx_out / w_out, if given, are [L, T, k] and receive each layer's routing."""
        for li in range(len(self.layers)):
            self.layer_forward(li, h, None if idx_out is None else idx_out[li],
                               None if w_out is None else w_out[li], stream, split)
