"""GPU parity of every step of the decode path against the CPU oracle.

Each test prints the case it runs (shape, seed, entry point) before any GPU
work, so a failing run names its case.  Inputs are seeded; routing inputs
are redrawn until the oracle's k-th/(k+1)-th logit gap is at least 1e-4.
Bars: exact for ids, counts, offsets and grouped order; rel 1e-5 on the
renormalised weights; rel-L2 <= 1e-3 on fp32 outputs (also after removing
each vector's mean, and on zero-mean weight variants, so that the common
offset of Q4_K weights cannot hide an error).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import quantized_expert_ffn_router_amd as moe
from quantized_expert_ffn_router_amd.stack import ResidentStack

from helpers import (REL_L2_BAR, TIE_GAP, ExpertCache, centered_rel_l2, chain_min_gap, layer_specs,
                     oracle_layers, sets_equal, weights_close)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


# ---------------------------------------------------------------- rmsnorm
@pytest.mark.parametrize("T,H", [(1, 256), (7, 2048), (32, 4096)])
def test_rmsnorm(T, H):
    _say("moe_rmsnorm", T, H)
    h = np.random.default_rng(T).standard_normal((T, H)).astype(np.float32) * 3
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    moe.moe_rmsnorm(_dev(h), T, H, 1e-6, out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(h)
    assert oracle.rel_l2(out.cpu().numpy(), ref) < 1e-6


# ---------------------------------------------------------------- router / top-k
ROUTE_CASES = [
    # (T, H, E, k, zipf, seed)
    (1, 256, 8, 2, False, 1),
    (8, 2048, 128, 8, False, 2),
    (32, 2048, 128, 8, True, 3),
    (5, 512, 5, 5, False, 4),        # k == E, E not a multiple of 4
    (3, 768, 61, 7, False, 5),
    (2, 1024, 1000, 16, False, 6),
    # prompt-sized batches (moe_route_topk takes up to 256 tokens)
    (64, 512, 64, 6, False, 7),
    (256, 256, 16, 4, True, 8),
    # limits: E = 1024 experts, k = 64
    (3, 512, 1024, 64, False, 9),
]


def _tie_free_route_inputs(T, H, E, k, zipf, seed):
    rng = np.random.default_rng(seed)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = None
    if zipf:
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        bias = np.log(p / p.sum())[rng.permutation(E)].astype(np.float32)
    xs = []
    while len(xs) < T:
        x = oracle.rmsnorm(rng.standard_normal(H).astype(np.float32)).astype(np.float32)
        r = oracle.route(x[None].astype(np.float64), wr, bias, k)
        if r.gap[0] >= TIE_GAP:
            xs.append(x)
    return np.stack(xs), wr, bias


@pytest.mark.parametrize("T,H,E,k,zipf,seed", ROUTE_CASES)
def test_route_topk(T, H, E, k, zipf, seed):
    _say("moe_route_topk", dict(T=T, H=H, E=E, k=k, zipf=zipf, seed=seed))
    x, wr, bias = _tie_free_route_inputs(T, H, E, k, zipf, seed)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    moe.moe_route_topk(_dev(x), T, H, _dev(wr), None if bias is None else _dev(bias), E, k, idx, w, lg)
    torch.cuda.synchronize()
    ref = oracle.route(x.astype(np.float64), wr, bias, k)
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    assert sets_equal(gi, ref.idx)
    assert weights_close(gi, gw, ref.idx, ref.w)
    assert np.max(np.abs(lg.cpu().numpy() - ref.logits)) < 2e-5
    # ids come out by descending logit
    glg = lg.cpu().numpy()
    for t in range(T):
        vals = glg[t, gi[t]]
        assert np.all(vals[:-1] >= vals[1:])


# ---------------------------------------------------------------- grouping
@pytest.mark.parametrize("T,k,E,seed", [(1, 2, 8, 0), (5, 3, 7, 1), (8, 8, 128, 2), (32, 8, 128, 3),
                                        (32, 1, 1000, 4), (17, 64, 64, 5)])
def test_group_tokens(T, k, E, seed):
    _say("moe_group_tokens", T, k, E, seed)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    count = torch.empty(E, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pairs = torch.empty(T * k, dtype=torch.int32, device=DEV)
    moe.moe_group_tokens(_dev(idx), T, k, E, count, off, pairs)
    torch.cuda.synchronize()
    ref = oracle.group(idx, E)
    assert np.array_equal(count.cpu().numpy(), ref.count)
    assert np.array_equal(off.cpu().numpy(), ref.offset)
    assert np.array_equal(pairs.cpu().numpy(), ref.pairs)


# ---------------------------------------------------------------- expert FFN
def _upload_experts(cfg, layer, experts: ExpertCache, n):
    d = moe.ExpertDesc.of(cfg.qtypes(layer), cfg.H, cfg.I)
    eb = moe.moe_expert_bytes(d)
    host = np.empty(n * eb, np.uint8)
    for e in range(n):
        ex = experts(layer, e)
        moe.moe_repack_expert(d, ex.gate, ex.up, ex.down, host[e * eb:(e + 1) * eb])
    buf = _dev(host)
    tab = torch.tensor([buf.data_ptr() + e * eb for e in range(n)], dtype=torch.int64, device=DEV)
    return d, buf, tab


FFN_CASES = [
    # (qtypes, H, I, E, k, ns, T, zero_mean)
    ((W.Q8_0,) * 3, 256, 512, 8, 2, 0, 1, False),
    ((W.Q4_K,) * 3, 512, 192, 6, 2, 0, 3, False),
    ((W.Q4_K,) * 3, 512, 192, 6, 2, 0, 3, True),
    ((W.Q6_K,) * 3, 512, 320, 5, 3, 1, 8, False),     # I=320: down rows padded to 512
    ((W.Q4_K, W.Q4_K, W.Q6_K), 768, 256, 9, 4, 2, 11, False),
    ((W.Q8_0, W.Q8_0, W.Q4_K), 1024, 128, 4, 4, 0, 32, False),
    ((W.Q4_K,) * 3, 2048, 768, 16, 8, 0, 8, True),
    # all-Q4_K experts with 2..8 tokens take the integer-MFMA path
    ((W.Q4_K,) * 3, 1024, 320, 8, 4, 2, 5, False),      # shared experts, ragged I (down rows padded to 512)
    ((W.Q4_K,) * 3, 8192, 256, 8, 2, 0, 8, False),      # H = 8192: 32 super-blocks per gate/up row
    ((W.Q4_K,) * 3, 2048, 1408, 64, 2, 2, 4, True),     # the mixed stack's Q4_K shape: I = 1408, 1536 down columns
    # all-Q4_K experts with more than 8 tokens take the MFMA path
    ((W.Q4_K,) * 3, 512, 192, 6, 2, 0, 9, False),       # just above the threshold; down rows padded
    ((W.Q4_K,) * 3, 1024, 320, 8, 8, 0, 32, False),     # every token on every expert: 32 columns; ragged I
    ((W.Q4_K,) * 3, 2048, 768, 128, 8, 2, 16, True),    # shared experts, zero-mean weights
    ((W.Q4_K,) * 3, 2048, 768, 16, 8, 0, 32, False),    # the Qwen3-30B-A3B shape at T=32
    # prompt-sized batches (T > 32): entries of at most 32 pairs per expert on the
    # MFMA path (every expert here has more), of at most 4 on the dot-product path
    ((W.Q4_K,) * 3, 512, 192, 8, 8, 0, 64, False),      # 64 pairs per expert: two entries each
    ((W.Q4_K,) * 3, 1024, 320, 16, 4, 1, 256, True),    # 256 tokens, a shared expert of 8 entries
    ((W.Q6_K, W.Q6_K, W.Q8_0), 512, 128, 6, 2, 1, 48, False),
    # limits and degenerate cases: H = 8192 (the largest), k = 64 (the largest),
    # a single expert (E = k = 1: weight one)
    ((W.Q8_0,) * 3, 8192, 64, 4, 2, 0, 2, False),
    ((W.Q4_K,) * 3, 256, 64, 64, 64, 0, 2, False),
    ((W.Q4_K,) * 3, 512, 128, 1, 1, 0, 3, False),
]


@pytest.mark.parametrize("qt,H,I,E,k,ns,T,zm", FFN_CASES)
@pytest.mark.parametrize("accumulate", [0, 1])
def test_expert_ffn(qt, H, I, E, k, ns, T, zm, accumulate):
    _say("moe_expert_ffn", dict(qt=qt, H=H, I=I, E=E, k=k, ns=ns, T=T, zero_mean=zm, acc=accumulate))
    cfg = W.MoEConfig("ffn-case", 1, H, E, k, I, (qt,), n_shared=ns, zero_mean=zm, seed=100 + T)
    experts = ExpertCache(cfg)
    d, buf, tab = _upload_experts(cfg, 0, experts, E + ns)
    rng = np.random.default_rng(T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    wts /= wts.sum(axis=1, keepdims=True)
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    kd = moe.moe_down_k(d)
    P = T * (k + ns)
    ws_bytes = moe.moe_workspace_bytes(d, T, k, E, ns)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    moe.moe_workspace_init(ws, ws_bytes)
    y = _dev(y0)
    act = torch.full((P, kd), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_expert_ffn(d, _dev(x), T, k, E, _dev(idx), _dev(wts), tab, tab[E:] if ns else None, ns, y, accumulate,
                       act, ws, ws_bytes)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    ag = act.cpu().numpy()
    # oracle
    grp = oracle.group(idx, E)
    yref = y0.astype(np.float64) * accumulate
    per = {}
    for t in range(T):
        for e in list(idx[t]) + [E + s for s in range(ns)]:
            ex = experts(0, int(e))
            per[(t, int(e))] = oracle.expert_ffn(qt, H, I, kd, ex.gate, ex.up, ex.down, x[t].astype(np.float64))
        yref[t] += sum(float(wts[t, j]) * per[(t, int(idx[t, j]))].o for j in range(k))
        yref[t] += sum(per[(t, E + s)].o for s in range(ns))
    # activations in grouped order: routed pairs by (expert, token), then shared experts by token
    order = [divmod(int(p), k) for p in grp.pairs]
    aref = [per[(t, int(idx[t, j]))].a for t, j in order]
    aref += [per[(t, E + s)].a for s in range(ns) for t in range(T)]
    aref = np.stack(aref)
    ag = ag[:, :I]
    aref = aref[:, :I]
    assert np.all(np.isfinite(ag))
    assert oracle.rel_l2(ag, aref) <= REL_L2_BAR
    assert centered_rel_l2(ag, aref) <= REL_L2_BAR
    assert oracle.rel_l2(yg, yref) <= REL_L2_BAR
    assert centered_rel_l2(yg - y0 * accumulate, yref - y0 * accumulate) <= REL_L2_BAR
    print("rel-L2 act %.3g y %.3g" % (oracle.rel_l2(ag, aref), oracle.rel_l2(yg, yref)))


# ---------------------------------------------------------------- fused layer and stack
def _run_stack_and_compare(cfg, n_layers, T, step=0, T_max=None, split=False, prompt=False, routing=True):
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts, n_layers)
    x, att = W.tie_free_tokens(cfg, step, T, chain_min_gap(olayers))
    _say("stack", cfg.name, dict(layers=n_layers, T=T, step=step, attempts=att))
    st = ResidentStack(layer_specs(cfg, n_layers), experts, T_max=T_max or T)
    h = _dev(x)
    idx = torch.empty((n_layers, T, cfg.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((n_layers, T, cfg.k), dtype=torch.float32, device=DEV)
    if prompt:
        st.prompt_step(h, idx, wts)
    elif routing:
        st.step(h, idx, wts, split=split)
    else:  # no routing outputs: no route tail where the FFN ranks the keys
        st.step(h, None, None, split=split)
    torch.cuda.synchronize()
    hg, ig, wg = h.cpu().numpy(), idx.cpu().numpy(), wts.cpu().numpy()
    href = []
    for t in range(T):
        outs = oracle.stack_token(olayers, x[t])
        for l, o in enumerate(outs):
            if not routing:
                continue
            assert sets_equal(ig[l, t][None], o.route.idx), f"layer {l} token {t}"
            assert weights_close(ig[l, t][None], wg[l, t][None], o.route.idx, o.route.w), f"layer {l} token {t}"
        href.append(outs[-1].h_next)
    href = np.stack(href)
    e1 = oracle.rel_l2(hg, href)
    e2 = centered_rel_l2(hg - x, href - x)
    print("rel-L2 h %.3g, centered update %.3g" % (e1, e2))
    assert e1 <= REL_L2_BAR and e2 <= REL_L2_BAR
    return st


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_layer_tiny_q8_0(seed):
    _run_stack_and_compare(W.tiny_q8_0(seed=seed), 1, 1)


@pytest.mark.parametrize("T", [1, 2])
def test_layer_wide_router(T):
    """E=200 experts: T=1 ranks the 200 keys (ids above 128 read from the
    expert table in the grouping), T=2 takes the per-wave radix select."""
    _run_stack_and_compare(W.tiny_q8_0(seed=6).with_(E=200, k=6), 1, T)


@pytest.mark.parametrize("T,E,k", [(17, 200, 6), (24, 64, 1), (32, 128, 8)])
def test_layer_per_token_topk(T, E, k):
    """Batches above 16 tokens rank each token's router keys in a workgroup
    of its own (4, 1 and 2 keys per lane for E=200, 64 and 128)."""
    _run_stack_and_compare(W.tiny_q8_0(seed=8).with_(E=E, k=k), 1, T)


@pytest.mark.parametrize("T", [1, 8])
def test_layer_qwen3_shape_q4k(T):
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=T), 1, T)


@pytest.mark.parametrize("T,E,k,routing", [(5, 200, 6, True), (3, 200, 10, False), (8, 128, 8, False), (2, 64, 4, False)])
def test_layer_q4k_batch_ranked_in_ffn(T, E, k, routing):
    """2..8 tokens on the integer-MFMA path: every gate/up workgroup ranks
    each token's logit keys (the lane-group bound for k <= 8, the bitonic one
    above; 4 keys per lane for E=200); without routing outputs the route
    launch has no tail at all."""
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=T).with_(E=E, k=k, seed=9), 1, T, routing=routing)


def test_layer_qwen3_shape_q4k_zero_mean():
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=4).with_(zero_mean=True, seed=7), 1, 4)


def test_layer_qwen3_shape_zipf_t32():
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k_zipf(T=32), 1, 32)


@pytest.mark.parametrize("T,first", [(1, 0), (4, 12)])
def test_layer_mixed_shared_q6k(T, first):
    cfg = W.mixed_shared_q4k_q6k(T=T)
    # layer `first` of the mixed stack (0: Q4_K group, 12: Q6_K group)
    sub = cfg.with_(n_layers=1, layer_qtypes=(cfg.qtypes(first),), seed=cfg.seed + first)
    _run_stack_and_compare(sub, 1, T)


# single tokens on Q4_K experts of several shapes (the route launch hands the
# logit keys to k_gate_up, whose workgroups rank them; k_down follows)
T1_SHAPES = [
    # H, I, E, k, n_shared, seed
    (1024, 512, 64, 4, 0, 31),    # four gate/up K-groups, down rows of 2
    (512, 320, 37, 3, 1, 32),     # odd E (a one-row router workgroup), I padded 320 -> 512, a shared expert
    (2048, 768, 128, 1, 0, 33),   # top-1 of 128
    (256, 2048, 16, 12, 2, 34),   # one gate/up K-group, down rows of 8 K-groups, 14 work items
]


@pytest.mark.parametrize("H,I,E,k,ns,seed", T1_SHAPES)
def test_layer_single_token_shapes(H, I, E, k, ns, seed):
    """Two layers back to back (the second route launch finds the keys that
    the first layer's kernels left)."""
    cfg = W.qwen3_30b_a3b_q4k(T=1, n_layers=2).with_(H=H, I=I, E=E, k=k, n_shared=ns, seed=seed)
    _run_stack_and_compare(cfg, 2, 1)


def _run_chain_and_compare(cfg, n_layers, step=0):
    """Chained single-token layers (moe_layer_forward_chain: one route launch,
    then each layer's FFN kernels start the next layer's router dots): the
    final state against the oracle chain, and against the same stack run
    unchained (the same sums in another order)."""
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts, n_layers)
    x, att = W.tie_free_tokens(cfg, step, 1, chain_min_gap(olayers))
    _say("chain", cfg.name, dict(layers=n_layers, step=step, attempts=att))
    st = ResidentStack(layer_specs(cfg, n_layers), experts, T_max=1)
    assert st.chainable(1)
    h = _dev(x)
    st.step(h, chain=True)
    hu = _dev(x)
    st.step(hu, chain=False)
    torch.cuda.synchronize()
    hg, hun = h.cpu().numpy(), hu.cpu().numpy()
    href = oracle.stack_token(olayers, x[0])[-1].h_next[None]
    e1 = oracle.rel_l2(hg, href)
    e2 = centered_rel_l2(hg - x, href - x)
    e3 = centered_rel_l2(hg - x, hun - x)
    print("rel-L2 h %.3g, centered update %.3g, against unchained %.3g" % (e1, e2, e3))
    assert np.all(np.isfinite(hg))
    assert e1 <= REL_L2_BAR and e2 <= REL_L2_BAR
    # the same experts and fp32 sums in another order: far tighter than the
    # oracle bar (a routing difference would move the update by >1e-2)
    assert e3 <= 1e-4


@pytest.mark.parametrize("H,I,E,k,ns,seed", T1_SHAPES)
def test_chain_single_token_shapes(H, I, E, k, ns, seed):
    """Three chained layers per shape: ragged I (down rows padded, cleared by
    the gate/up launch when no route launch runs), odd E (partial 16-lane
    groups of router rows never straddle), shared experts adding to the next
    router's dots, H from 256 to 2048."""
    cfg = W.qwen3_30b_a3b_q4k(T=1, n_layers=3).with_(H=H, I=I, E=E, k=k, n_shared=ns, seed=seed + 100)
    _run_chain_and_compare(cfg, 3)


def test_chain_q8_0_and_wide_h():
    """Q8_0 experts (their own gate/up and down instantiations) at H=4096, the
    largest chained state (two state words per gate/up thread)."""
    cfg = W.tiny_q8_0(seed=41).with_(H=4096, I=512, E=48, k=4, n_layers=3, layer_qtypes=((W.Q8_0,) * 3,) * 3)
    _run_chain_and_compare(cfg, 3)


def test_chain_biased_router():
    """A router bias (Zipf(1.1) over the experts): the keys need 1/RMS before
    the rank (without a bias the raw dot sums are ranked)."""
    _run_chain_and_compare(W.qwen3_30b_a3b_q4k_zipf(T=1, n_layers=4).with_(seed=17), 4)


def test_chain_qwen3_shape_6_layers():
    _run_chain_and_compare(W.qwen3_30b_a3b_q4k(T=1, n_layers=6).with_(seed=13), 6)


def test_chain_mixed_shared_q6k():
    """Q4_K layers then Q6_K layers chained (the chain crosses the type
    change), two shared experts, I=1408."""
    cfg = W.mixed_shared_q4k_q6k(T=1)
    Q4, Q6 = W.Q4_K, W.Q6_K
    sub = cfg.with_(n_layers=4, layer_qtypes=((Q4,) * 3,) * 2 + ((Q6,) * 3,) * 2, seed=cfg.seed + 41)
    _run_chain_and_compare(sub, 4)


def test_chain_unsupported_is_refused():
    """Two tokens, or E above 128, cannot chain: MOE_ERR_ARG, nothing run."""
    cfg = W.qwen3_30b_a3b_q4k(T=2, n_layers=2).with_(seed=9)
    experts = ExpertCache(cfg)
    st = ResidentStack(layer_specs(cfg, 2), experts, T_max=2)
    assert not st.chainable(2) and st.chainable(1)
    h = _dev(W.tokens(cfg, 0, 2))
    with pytest.raises(moe.MoeError, match="MOE_ERR_ARG"):
        st.step(h, chain=True)


def test_stack_qwen3_shape_6_layers_t1():
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=1, n_layers=6).with_(seed=12), 6, 1)


def test_stack_qwen3_shape_4_layers_t8():
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=8, n_layers=4), 4, 8)


def test_stack_mixed_shared_6_layers_t4():
    """Three Q4_K layers then three Q6_K layers, 64 routed (top-2) + 2 shared
    experts, I=1408 (down rows padded to 1536), T=4, through the whole stack."""
    cfg = W.mixed_shared_q4k_q6k(T=4)
    Q4, Q6 = W.Q4_K, W.Q6_K
    sub = cfg.with_(n_layers=6, layer_qtypes=((Q4,) * 3,) * 3 + ((Q6,) * 3,) * 3, seed=cfg.seed + 21)
    _run_stack_and_compare(sub, 6, 4)


@pytest.mark.parametrize("T", [1, 8, 24])
def test_stack_split_route_then_ffn(T):
    """moe_layer_route followed by moe_layer_ffn, the two halves of a layer."""
    _run_stack_and_compare(W.qwen3_30b_a3b_q4k(T=T, n_layers=2).with_(seed=5), 2, T, split=True)


def test_stack_prompt_batch_t96():
    """A prompt-sized batch (96 tokens, past the layer calls' 32) through two
    all-Q4_K layers by moe_rmsnorm + moe_route_topk + moe_expert_ffn: 8
    experts at top-4, so each expert takes about 48 tokens, two MFMA work
    entries of at most 32."""
    cfg = W.qwen3_30b_a3b_q4k(T=96, n_layers=2).with_(H=512, I=192, E=8, k=4, seed=11)
    _run_stack_and_compare(cfg, 2, 96, T_max=8, prompt=True)


def test_mixed_shared_split():
    cfg = W.mixed_shared_q4k_q6k(T=4)
    sub = cfg.with_(n_layers=1, layer_qtypes=(cfg.qtypes(12),), seed=cfg.seed + 3)
    _run_stack_and_compare(sub, 1, 4, split=True)


def test_zero_state_stays_zero():
    cfg = W.tiny_q8_0(seed=3)
    experts = ExpertCache(cfg)
    _say("zero state", cfg.name)
    st = ResidentStack(layer_specs(cfg), experts, T_max=2)
    h = torch.zeros((2, cfg.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((1, 2, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((1, 2, cfg.k), dtype=torch.float32, device=DEV)
    st.step(h, idx, w)
    torch.cuda.synchronize()
    assert torch.all(h == 0).item()
    # all logits equal: the lowest ids win, weights uniform
    assert np.array_equal(idx.cpu().numpy()[0], np.tile(np.arange(cfg.k, dtype=np.int32), (2, 1)))
    assert np.allclose(w.cpu().numpy(), 1.0 / cfg.k)


def test_workspace_reuse_across_sizes():
    """Counters are left at zero: one workspace serves calls of different T."""
    cfg = W.qwen3_30b_a3b_q4k(T=8, n_layers=1).with_(seed=11)
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts, 1)
    _say("workspace reuse", cfg.name)
    st = ResidentStack(layer_specs(cfg, 1), experts, T_max=8)
    for T in (8, 1, 5, 8):
        x, _ = W.tie_free_tokens(cfg, T, T, chain_min_gap(olayers))
        h = _dev(x)
        st.step(h)
        torch.cuda.synchronize()
        href = np.stack([oracle.stack_token(olayers, x[t])[-1].h_next for t in range(T)])
        assert oracle.rel_l2(h.cpu().numpy(), href) <= REL_L2_BAR
