"""Failure visibility of the route launch's bounded waits (GPU).

The route launch hands logit keys (and, above 16 tokens, each token's top-k)
between its workgroups through the workspace, behind bounded polls.  These
tests check that the workspace's status word reads 0 after normal calls;
that a set word makes later routed calls on the workspace give NaN weights
and NaN outputs (sticky) until moe_workspace_init; that withheld keys (a
hand-off that never comes) make every wait give up and set its bit; that a single token,
whose expert FFN ranks the router's logits itself without any hand-off,
still gets the exact state update; and, with the polling bound cut to one
round from the host, that every call is either exact against the oracle
with the word clear or NaN with a bit set.  No wait is
unbounded and every index stays in range on the give-up path, so nothing
here can hang or fault a kernel.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import quantized_expert_ffn_router_amd as moe
from quantized_expert_ffn_router_amd.stack import ResidentStack

from helpers import REL_L2_BAR, ExpertCache, chain_min_gap, layer_specs, oracle_layers, sets_equal, weights_close

pytestmark = pytest.mark.gpu
DEV = "cuda"

# T=1 with the routing requested (the single-token tail), T=8 (the tail
# ranks every token), T=24 (a top-k workgroup per token)
CASES = [(1, 64, 4), (8, 64, 4), (24, 64, 4)]


def _say(*a):
    print("[case]", *a, flush=True)


def _setup(T, E, k, seed=9):
    cfg = W.tiny_q8_0(seed=seed).with_(E=E, k=k)
    experts = ExpertCache(cfg)
    olayers = oracle_layers(cfg, experts, 1)
    x, _ = W.tie_free_tokens(cfg, 0, T, chain_min_gap(olayers))
    st = ResidentStack(layer_specs(cfg, 1), experts, T_max=T)
    return cfg, olayers, x, st


def _step(st, x, cfg, want_routing=True):
    T = x.shape[0]
    h = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    idx = torch.empty((1, T, cfg.k), dtype=torch.int32, device=DEV) if want_routing else None
    w = torch.empty((1, T, cfg.k), dtype=torch.float32, device=DEV) if want_routing else None
    st.step(h, idx, w)
    torch.cuda.synchronize()
    return (h.cpu().numpy(), None if idx is None else idx.cpu().numpy()[0],
            None if w is None else w.cpu().numpy()[0])


def _status(st):
    return moe.moe_workspace_status(st.ws, st.ws_bytes)


def _exact(olayers, x, hg, ig, wg):
    href = []
    for t in range(x.shape[0]):
        o = oracle.stack_token(olayers, x[t])[0]
        if ig is not None:
            assert sets_equal(ig[t][None], o.route.idx), f"token {t}"
            assert weights_close(ig[t][None], wg[t][None], o.route.idx, o.route.w), f"token {t}"
        href.append(o.h_next)
    e = oracle.rel_l2(hg, np.stack(href))
    assert e <= REL_L2_BAR, e


def _refused(olayers, x, hg, ig, wg, E):
    """A refused or given-up route: NaN weights, ids in range; the state is
    NaN, except for a single token (its FFN routes from the logits)."""
    assert np.isnan(wg).all()
    assert ((ig >= 0) & (ig < E)).all()
    if x.shape[0] == 1:
        _exact(olayers, x, hg, None, None)
    else:
        assert np.isnan(hg).all()


def _plant(st, bit):
    off = moe.MOE_WS_STATUS_OFFSET
    st.ws[off:off + 4].view(torch.int32)[0] = bit
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,E,k", CASES)
def test_status_word_sticky_until_init(T, E, k):
    cfg, olayers, x, st = _setup(T, E, k)
    _say("status sticky", dict(T=T, E=E, k=k))
    hg, ig, wg = _step(st, x, cfg)
    assert _status(st) == 0
    _exact(olayers, x, hg, ig, wg)
    # a wait of an earlier call gave up: every routed call refuses
    _plant(st, moe.MOE_WS_KEYS_TIMEOUT)
    for _ in range(2):
        hg, ig, wg = _step(st, x, cfg)
        _refused(olayers, x, hg, ig, wg, E)
        assert _status(st) == moe.MOE_WS_KEYS_TIMEOUT
    if T == 1:
        # without routing outputs the single token's route launch has no
        # tail at all: nothing reads a hand-off array
        hg, _, _ = _step(st, x, cfg, want_routing=False)
        _exact(olayers, x, hg, None, None)
        assert _status(st) == moe.MOE_WS_KEYS_TIMEOUT
    moe.moe_workspace_init(st.ws, st.ws_bytes)
    assert _status(st) == 0
    hg, ig, wg = _step(st, x, cfg)
    _exact(olayers, x, hg, ig, wg)
    assert _status(st) == 0


@pytest.mark.parametrize("T,E,k", CASES)
def test_give_up_path_forced_by_tiny_spin_limit(T, E, k):
    """Polls cut to one round: the waits give up whenever the senders are
    late.  Each call is exact with a clear word, or NaN with a bit set (then
    the workspace is cleared for the next call)."""
    cfg, olayers, x, st = _setup(T, E, k, seed=10)
    _say("give-up forced", dict(T=T, E=E, k=k))
    n_gave_up = 0
    moe.moe_set_spin_limit(1)
    try:
        for _ in range(12):
            hg, ig, wg = _step(st, x, cfg)
            s = _status(st)
            assert s & ~(moe.MOE_WS_KEYS_TIMEOUT | moe.MOE_WS_TOPK_TIMEOUT) == 0
            if s:
                n_gave_up += 1
                _refused(olayers, x, hg, ig, wg, E)
                moe.moe_workspace_init(st.ws, st.ws_bytes)
            else:
                _exact(olayers, x, hg, ig, wg)
    finally:
        moe.moe_set_spin_limit(0)
        torch.cuda.synchronize()
    print("gave up in %d of 12 calls" % n_gave_up)
    # back at the default bound, on the cleared workspace
    moe.moe_workspace_init(st.ws, st.ws_bytes)
    hg, ig, wg = _step(st, x, cfg)
    assert _status(st) == 0
    _exact(olayers, x, hg, ig, wg)


@pytest.mark.parametrize("T,E,k,bit", [(1, 64, 4, 1), (8, 64, 4, 1), (24, 64, 4, 2)])
def test_give_up_path_forced_by_withheld_keys(T, E, k, bit):
    """The router workgroups store no keys (a hand-off that never comes) and
    the polls are cut to four rounds: every wait gives up, deterministically.
    T=24 fails in the per-token top-k workgroups, whose give-up the tail
    then meets (MOE_WS_TOPK_TIMEOUT); the others in the tail itself."""
    cfg, olayers, x, st = _setup(T, E, k, seed=11)
    _say("give-up by withheld keys", dict(T=T, E=E, k=k))
    moe.moe_set_spin_limit(4, True)
    try:
        hg, ig, wg = _step(st, x, cfg)
        s = _status(st)
    finally:
        moe.moe_set_spin_limit(0)
        torch.cuda.synchronize()
    assert s == bit, s
    _refused(olayers, x, hg, ig, wg, E)
    # sticky: keys flow again, but the word still refuses
    hg, ig, wg = _step(st, x, cfg)
    _refused(olayers, x, hg, ig, wg, E)
    assert _status(st) == bit
    moe.moe_workspace_init(st.ws, st.ws_bytes)
    hg, ig, wg = _step(st, x, cfg)
    assert _status(st) == 0
    _exact(olayers, x, hg, ig, wg)


def test_static_scratch_status_and_clear():
    """ws NULL addresses the no-allocation entry point's static scratch."""
    cfg, olayers, x, st = _setup(4, 64, 4, seed=12)
    _say("static scratch status")
    moe.moe_workspace_init(None, 0)
    h = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    moe.moe_layer_forward_noalloc(st.descs[0], h, 4, st.routers[0], st.biases[0], cfg.E, cfg.k, st.expert_ptrs(0),
                                  st.shared_ptrs(0), cfg.n_shared, st.eps, None, None)
    torch.cuda.synchronize()
    assert moe.moe_workspace_status(None, 0) == 0
    _exact(olayers, x, h.cpu().numpy(), None, None)
