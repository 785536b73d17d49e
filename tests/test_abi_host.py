"""Host-side checks of the C ABI (no GPU calls): the library loads, exports
every function include/moe.h declares, validates arguments before touching
the GPU, plans cache slots as the T4 MoE-cache report prints, and repacks
experts by pure byte permutation into the documented tile layout."""
import json
import os
import re

import numpy as np
import pytest

import workloads as W
import quantized_expert_ffn_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = moe.lib()
    decl = _declared()
    assert len(decl) >= 19
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(moe.EXPORTED) == decl


def test_argument_errors_are_host_side():
    L = moe.lib()
    d = moe.ExpertDesc.of((W.Q4_K,) * 3, 2048, 768)
    fake = 0x1000
    ws_need = moe.moe_workspace_bytes(d, 8, 8, 128, 0)

    def st(**kw):
        a = dict(desc=d, h=fake, T=8, wr=fake, bias=None, E=128, k=8, ep=fake, sp=None, ns=0, ws=fake, wsb=ws_need)
        a.update(kw)
        import ctypes
        return L.moe_layer_forward(ctypes.byref(a["desc"]), a["h"], a["T"], a["wr"], a["bias"], a["E"], a["k"],
                                   a["ep"], a["sp"], a["ns"], 1e-6, None, None, a["ws"], a["wsb"], 0)

    assert st(T=33) == -7 and st(T=0) == -7
    assert st(k=129) == -1 and st(k=0) == -1 and st(E=2000) == -1
    assert st(desc=moe.ExpertDesc.of((7, 2, 2), 2048, 768)) == -3
    assert st(desc=moe.ExpertDesc.of((W.Q4_K,) * 3, 2000, 768)) == -2
    assert st(desc=moe.ExpertDesc.of((W.Q4_K,) * 3, 2048, 700)) == -2
    assert st(h=None) == -1 and st(ns=1) == -1
    assert st(wsb=ws_need - 1) == -1
    assert b"workspace too small" in L.moe_last_error()
    with pytest.raises(moe.MoeError) as ei:  # the stand-alone router takes up to 256 tokens
        moe.moe_route_topk(fake, 257, 2048, fake, None, 128, 8, fake, fake, None, stream=0)
    assert ei.value.name == "MOE_ERR_BATCH"
    # moe_expert_ffn takes up to 256 tokens, the layer calls up to 32
    assert moe.moe_workspace_bytes(d, 256, 8, 128, 0) > moe.moe_workspace_bytes(d, 32, 8, 128, 0) > 0
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_bytes(d, 257, 8, 128, 0)
    with pytest.raises(moe.MoeError):
        moe.moe_group_tokens(fake, 4, 9, 8, fake, fake, fake, stream=0)


def test_layer_chain_support_and_argument_checks():
    """moe_layer_chain_supported is a host rule (one token on the single-token
    kernels, E <= 128, H <= 4096); moe_layer_forward_chain refuses what the
    rule refuses, and bad next_E / parity, before anything is enqueued."""
    import ctypes
    L = moe.lib()
    q4 = moe.ExpertDesc.of((W.Q4_K,) * 3, 2048, 768)
    assert moe.moe_layer_chain_supported(q4, 1, 128)
    assert not moe.moe_layer_chain_supported(q4, 2, 128)
    assert not moe.moe_layer_chain_supported(q4, 1, 129)
    assert moe.moe_layer_chain_supported(moe.ExpertDesc.of((W.Q8_0,) * 3, 4096, 512), 1, 48)
    assert not moe.moe_layer_chain_supported(moe.ExpertDesc.of((W.Q4_K,) * 3, 8192, 512), 1, 64)
    assert not moe.moe_layer_chain_supported(moe.ExpertDesc.of((7, 2, 2), 2048, 768), 1, 64)
    fake = 0x1000
    wsb = moe.moe_workspace_bytes(q4, 1, 8, 128, 0)

    def st(T=1, E=128, chain_in=1, nxt=fake, nE=128, parity=0):
        return L.moe_layer_forward_chain(ctypes.byref(q4), fake, T, fake, None, E, 8, fake, None, 0, 1e-6,
                                         chain_in, nxt, nE, parity, fake, wsb, 0)

    assert st(T=2) == -1 and b"chaining takes one token" in L.moe_last_error()
    assert st(E=200) == -1
    assert st(nE=129) == -1 and st(nE=0) == -1
    assert st(parity=2) == -1 and b"parity" in L.moe_last_error()
    assert st(T=40) == -7  # the layer calls' own batch limit comes first


def test_cache_plan_through_abi_reproduces_page_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "t4_cache_plan_example.json")))
    pr = g["printed"]
    descs = [moe.ExpertDesc.of((W.Q4_K,) * 3, g["H"], g["I"]),
             moe.ExpertDesc.of((W.Q4_K, W.Q4_K, W.Q6_K), g["H"], g["I"])]
    assert moe.moe_expert_bytes(descs[0]) == 2_654_208
    assert moe.moe_expert_bytes(descs[1]) == 3_059_712
    st, slots = moe.moe_cache_plan(descs, [24, 24], pr["budget_mib"] << 20, g["top_k"])
    assert st == 0 and list(slots) == [pr["slots_per_group"]] * 2
    st, slots = moe.moe_cache_plan(descs, [24, 24], pr["floor_ok_mib"] << 20, g["top_k"])
    assert st == 0 and min(slots) >= g["top_k"]
    st, slots = moe.moe_cache_plan(descs, [24, 24], pr["floor_fail_mib"] << 20, g["top_k"])
    assert st == -4 and max(slots) == 0


@pytest.mark.parametrize("qt", [W.Q8_0, W.Q4_K, W.Q6_K])
def test_repack_is_a_byte_permutation_with_documented_tiles(qt):
    cfg = W.MoEConfig("repack", 1, 512, 2, 1, 128, ((qt,) * 3,), seed=9)
    ex = W.expert(cfg, 0, 1)
    d = moe.ExpertDesc.of(cfg.qtypes(0), cfg.H, cfg.I)
    out = moe.moe_repack_expert(d, ex.gate, ex.up, ex.down)
    assert out.nbytes == cfg.expert_bytes(0) == moe.moe_expert_bytes(d)
    assert np.array_equal(np.sort(out), np.sort(ex.concat()))
    # row 5, K-group 1 of the gate matrix: its first 16 canonical bytes sit at
    # tile (0, 1), lane 5 of the first 16-byte plane
    S = cfg.H // 256
    tb = {W.Q8_0: 17408, W.Q4_K: 9216, W.Q6_K: 13440}[qt]
    row = ex.gate[5]
    if qt == W.Q4_K:
        first16 = row[144:160]
        at = 1 * tb + 5 * 16
    elif qt == W.Q6_K:
        first16 = row[210:226]
        at = 1 * tb + 5 * 16
    else:
        first16 = row[8 * 34 + 2:8 * 34 + 18]   # block 8 (K-group 1) quant bytes 0-15
        at = 1 * tb + 5 * 16
    assert np.array_equal(out[at:at + 16], first16)
    assert S == 2


def test_prefetch_schedule():
    """Cross-layer prefetch schedule (host logic): at layer 0 the next d
    layers, then l+d, never past the last layer; every layer after the
    first is prefetched exactly once per step, before its own lookup."""
    from types import SimpleNamespace
    from quantized_expert_ffn_router_amd.stack import CachedStack
    for n, d in [(4, 1), (4, 2), (48, 2), (3, 5), (1, 2)]:
        obj = SimpleNamespace(prefetch_depth=d, layers=[None] * n)
        sched = [CachedStack.prefetch_targets(obj, l) for l in range(n)]
        flat = [m for t in sched for m in t]
        assert sorted(flat) == list(range(1, n)) and len(flat) == len(set(flat))
        assert all(l < m <= l + d for l, t in enumerate(sched) for m in t)
    assert [CachedStack.prefetch_targets(SimpleNamespace(prefetch_depth=2, layers=[None] * 5), l)
            for l in range(5)] == [[1, 2], [3], [4], [], []]
    assert CachedStack.prefetch_targets(SimpleNamespace(prefetch_depth=0, layers=[None] * 5), 0) == []


def test_workspace_status_argument_checks_without_gpu():
    """moe_workspace_status rejects a null status or a workspace too small to
    hold the word on the host, before any HIP call."""
    import ctypes
    L = moe.lib()
    out = ctypes.c_uint32(7)
    assert L.moe_workspace_status(ctypes.c_void_p(4096), 1 << 20, None, None) == -1
    assert L.moe_workspace_status(ctypes.c_void_p(4096), moe.MOE_WS_STATUS_OFFSET, ctypes.byref(out), None) == -1
    assert b"status word" in L.moe_last_error()


def test_cache_lookup_device_route_argument_checks_without_gpu():
    """moe_cache_lookup_device_route refuses a null cache or workspace on the
    host, before any HIP call."""
    import ctypes
    L = moe.lib()
    assert L.moe_cache_lookup_device_route(None, 0, ctypes.c_void_p(4096), 1 << 20, 8, None) == -1
    assert L.moe_cache_lookup_device_route(ctypes.c_void_p(8), 0, None, 1 << 20, 8, None) == -1
