"""GPU test of moe_layer_forward_noalloc, the allocation-free variant of
moe_layer_forward for callers that cannot allocate: it must give the same
routing and, to the parity bar, the same updated state as moe_layer_forward
with a workspace, on two calls in a row (the second with a smaller batch, so
that the shared static scratch keeps the first call's contents), and refuse
a layer whose scratch need exceeds the static array before enqueuing
anything."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W
import quantized_expert_ffn_router_amd as moe
from helpers import REL_L2_BAR, ExpertCache, layer_specs
from quantized_expert_ffn_router_amd.stack import ResidentStack

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[noalloc]", *a, flush=True)


def _pair(st, layer, x):
    """One layer on x through moe_layer_forward (workspace) and through
    moe_layer_forward_noalloc; returns both states and routings."""
    s = st.layers[layer]
    T = x.shape[0]
    outs = []
    for noalloc in (False, True):
        h = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        idx = torch.full((T, s.k), -1, dtype=torch.int32, device=DEV)
        w = torch.zeros((T, s.k), dtype=torch.float32, device=DEV)
        if noalloc:
            moe.moe_layer_forward_noalloc(st.descs[layer], h, T, st.routers[layer], st.biases[layer], s.E, s.k,
                                          st.expert_ptrs(layer), st.shared_ptrs(layer), s.n_shared, st.eps, idx, w)
        else:
            st.layer_forward(layer, h, idx, w)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    return outs


@pytest.mark.parametrize("cfg", [W.qwen3_30b_a3b_q4k(T=8, n_layers=2).with_(E=32),
                                 W.mixed_shared_q4k_q6k(T=4, n_layers=2)], ids=["q4k_e32_k8", "mixed_shared"])
def test_noalloc_matches_workspace_entry_point(cfg):
    experts = ExpertCache(cfg)
    st = ResidentStack(layer_specs(cfg), experts, T_max=8, device=DEV)
    for call, (layer, T) in enumerate([(0, 8), (1, 1)]):  # the second call: a smaller batch
        x = W.tokens(cfg, 500 + call, T)
        (ha, ia, wa), (hb, ib, wb) = _pair(st, layer, x)
        assert np.array_equal(np.sort(ia, axis=1), np.sort(ib, axis=1)), (call, ia, ib)
        assert np.allclose(wa, wb, rtol=1e-6, atol=0), call
        err = float(np.linalg.norm(hb - ha) / np.linalg.norm(ha))
        _say(cfg.name, f"call {call} T={T} layer {layer}: rel-L2 {err:.3g}")
        assert err <= REL_L2_BAR


def test_noalloc_refuses_oversized_layer():
    """H = 8192, I = 6144 at 32 tokens with 8 shared experts needs about 26 MiB
    of scratch, more than the 8 MiB array: refused on the host, nothing run."""
    d = moe.ExpertDesc.of((W.Q6_K,) * 3, 8192, 6144)
    need = moe.moe_workspace_bytes(d, 32, 8, 1024, 8)
    assert need > (8 << 20)
    h = torch.zeros((32, 8192), dtype=torch.float32, device=DEV)
    wr = torch.zeros((1024, 8192), dtype=torch.float32, device=DEV)
    tab = torch.zeros(1024, dtype=torch.int64, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(d, h, 32, wr, None, 1024, 8, tab, tab, 8, 1e-6, None, None)
    assert ei.value.name == "MOE_ERR_CAPACITY"
    torch.cuda.synchronize()
