"""Pins of the CPU oracle to facts other than itself.

Each test ties one oracle function to something independent of its own
code: hand-packed blocks whose fields are stated semantically, the numbers
the T4 MoE-cache report prints, IEEE half values, closed forms, library
routines (numpy matmul / softmax / sort) on the same inputs, and brute force
on tiny inputs.  Each is chosen so that a plausible mistake in the oracle
(a dropped term, a wrong sign, a wrong bit or byte index, a transposed
operand, an off-by-one in the planner) fails at least one of them.
"""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _hex(s):
    return bytes.fromhex(s.replace(" ", ""))


# ---------------------------------------------------------------- fp16
@pytest.mark.parametrize("bits,val", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x3800, 0.5), (0x7BFF, 65504.0),
    (0x0400, 2.0 ** -14), (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24),
    (0x3555, 0.333251953125), (0x8000, -0.0), (0x0000, 0.0),
])
def test_half_textbook_values(bits, val):
    assert oracle.half(bits) == val


def test_half_matches_numpy_everywhere():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got[~np.isnan(ref)]), np.isinf(ref[~np.isnan(ref)]))


# ---------------------------------------------------------------- block formats
def test_block_sizes_reproduce_page_expert_total():
    """Q4_K = 144 B and Q6_K = 210 B per 256 weights reproduce the printed
    16.35 GiB of experts for Qwen3-30B-A3B Q4_K_M (T4 MoE-cache report)."""
    g = _gold("t4_cache_plan_example.json")
    H, I, E = g["H"], g["I"], g["E"]
    q4 = W.matrix_bytes(W.Q4_K, I, H)
    assert q4 == 884_736
    e_a = 3 * q4
    e_b = 2 * q4 + W.matrix_bytes(W.Q6_K, H, I)
    total = 24 * E * (e_a + e_b)
    assert round(total / 2 ** 30, 2) == g["printed"]["expert_total_gib"]
    assert W.QBYTES[W.Q8_0] == 34  # GPU-offload research notes, section 1.2


def test_q8_0_hand_block():
    g = _gold("hand_blocks.json")["q8_0"]
    blk = _hex(g["d_bits"])[::-1] + bytes((q & 0xFF) for q in g["q"])
    assert len(blk) == 34
    got = oracle.dequant_row(W.Q8_0, np.frombuffer(blk, np.uint8), 32)
    assert np.array_equal(got, g["d"] * np.array(g["q"], np.float64))


def _q4k_expected(g):
    q = []
    chunk = _hex(g["qs_hex_chunk"])
    assert len(chunk) == 32
    v = np.empty(256)
    for c in range(4):
        for i in range(32):
            qlo = i % 16
            qhi = 15 - (i % 16)
            v[64 * c + i] = g["d"] * g["sc"][2 * c] * qlo - g["dmin"] * g["m"][2 * c]
            v[64 * c + 32 + i] = g["d"] * g["sc"][2 * c + 1] * qhi - g["dmin"] * g["m"][2 * c + 1]
    return v


@pytest.mark.parametrize("name", ["q4_k_small_scales", "q4_k_high_bits"])
def test_q4_k_hand_block(name):
    g = _gold("hand_blocks.json")[name]
    blk = (_hex(g["d_bits"])[::-1] + _hex(g["dmin_bits"])[::-1] + _hex(g["scales_hex"])
           + _hex(g["qs_hex_chunk"]) * 4)
    assert len(blk) == 144
    got = oracle.dequant_row(W.Q4_K, np.frombuffer(blk, np.uint8), 256)
    assert np.array_equal(got, _q4k_expected(g))


def test_q6_k_hand_block():
    g = _gold("hand_blocks.json")["q6_k_ramp"]
    ql = bytes(((l % 16) * 0x11) for _ in range(2) for l in range(64))
    qh = bytes((0x88 if l < 16 else 0xDD) for _ in range(2) for l in range(32))
    sc = bytes((s & 0xFF) for s in g["sc"])
    blk = ql + qh + sc + _hex(g["d_bits"])[::-1]
    assert len(blk) == 210
    got = oracle.dequant_row(W.Q6_K, np.frombuffer(blk, np.uint8), 256)
    exp = np.array([g["d"] * g["sc"][p // 16] * ((p % 64) - 32) for p in range(256)], np.float64)
    assert np.array_equal(got, exp)


def _pack_q6_k(q, sc, d_bits):
    """Independent packer written from the format description (inverse of the unpack)."""
    ql = bytearray(128)
    qh = bytearray(64)
    for n in range(2):
        for l in range(32):
            a, b, c, e = q[128 * n + l], q[128 * n + 32 + l], q[128 * n + 64 + l], q[128 * n + 96 + l]
            ql[64 * n + l] = (a & 15) | ((c & 15) << 4)
            ql[64 * n + 32 + l] = (b & 15) | ((e & 15) << 4)
            qh[32 * n + l] = (a >> 4) | ((b >> 4) << 2) | ((c >> 4) << 4) | ((e >> 4) << 6)
    return bytes(ql) + bytes(qh) + bytes(s & 0xFF for s in sc) + d_bits.to_bytes(2, "little")


def test_q6_k_roundtrip_asymmetric():
    rng = random.Random(7)
    for trial in range(20):
        q = [rng.randrange(64) for _ in range(256)]
        sc = [rng.randrange(-128, 128) for _ in range(16)]
        blk = _pack_q6_k(q, sc, 0x3C00)
        got = oracle.dequant_row(W.Q6_K, np.frombuffer(blk, np.uint8), 256)
        exp = np.array([sc[p // 16] * (q[p] - 32) for p in range(256)], np.float64)
        assert np.array_equal(got, exp)


def _pack_q4_k(q, sc, m, d_bits, dmin_bits):
    """Independent packer for Q4_K (inverse of the unpack), from the format description."""
    s = bytearray(12)
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    qs = bytearray(128)
    for c in range(4):
        for i in range(32):
            qs[32 * c + i] = q[64 * c + i] | (q[64 * c + 32 + i] << 4)
    return d_bits.to_bytes(2, "little") + dmin_bits.to_bytes(2, "little") + bytes(s) + bytes(qs)


def test_q4_k_roundtrip_random_fields():
    rng = random.Random(11)
    for trial in range(20):
        q = [rng.randrange(16) for _ in range(256)]
        sc = [rng.randrange(64) for _ in range(8)]
        m = [rng.randrange(64) for _ in range(8)]
        blk = _pack_q4_k(q, sc, m, 0x3C00, 0x3800)
        got = oracle.dequant_row(W.Q4_K, np.frombuffer(blk, np.uint8), 256)
        exp = np.array([sc[p // 32] * q[p] - 0.5 * m[p // 32] for p in range(256)], np.float64)
        assert np.array_equal(got, exp)


def test_q4_k_min_term_isolated_and_signed():
    """q = 0 everywhere leaves exactly -dmin*m of each sub-block."""
    m = [0, 1, 2, 3, 60, 61, 62, 63]
    blk = _pack_q4_k([0] * 256, [63] * 8, m, 0x3C00, 0x4000)  # d=1, dmin=2
    got = oracle.dequant_row(W.Q4_K, np.frombuffer(blk, np.uint8), 256)
    assert np.array_equal(got, np.repeat(-2.0 * np.array(m, np.float64), 32))


def test_q6_k_offset_32_is_zero():
    blk = _pack_q6_k([32] * 256, [127] * 16, 0x5BFF)
    got = oracle.dequant_row(W.Q6_K, np.frombuffer(blk, np.uint8), 256)
    assert np.all(got == 0.0)


def test_dequant_rejects_partial_blocks():
    with pytest.raises(ValueError):
        oracle.dequant_row(W.Q4_K, np.zeros(144, np.uint8), 128)


# ---------------------------------------------------------------- matvec orientation
@pytest.mark.parametrize("qt", [W.Q8_0, W.Q4_K, W.Q6_K])
def test_qmatvec_matches_numpy_on_dequantized(qt):
    rng = np.random.default_rng(3)
    n, k = 64, 512
    w = W.quant_matrix(qt, rng, n, k)
    dense = oracle.dequant_matrix(qt, w, n, k)
    x = rng.standard_normal(k)
    y = oracle.qmatvec(qt, w, n, k, x)
    assert np.allclose(y, dense @ x, rtol=1e-12, atol=1e-12)
    # one-hot input returns a column: catches a transposed operand
    for col in (0, 37, k - 1):
        e = np.zeros(k)
        e[col] = 1.0
        assert np.array_equal(oracle.qmatvec(qt, w, n, k, e), dense[:, col])


# ---------------------------------------------------------------- SiLU and RMSNorm
def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for x in (0.1, 1.0, 3.7, 12.5):
        assert math.isclose(oracle.silu(x) - oracle.silu(-x), x, rel_tol=1e-14)
        assert math.isclose(oracle.silu(x), x / (1 + math.exp(-x)), rel_tol=1e-15)
    assert math.isclose(oracle.silu(40.0), 40.0, rel_tol=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_rmsnorm_closed_forms():
    c = np.full(64, 3.0, np.float32)
    got = oracle.rmsnorm(c)
    assert np.allclose(got, 3.0 / math.sqrt(9.0 + oracle.RMS_EPS), rtol=1e-15)
    x = np.random.default_rng(0).standard_normal(2048).astype(np.float32) * 50
    xh = oracle.rmsnorm(x)
    assert math.isclose(float(np.sqrt(np.mean(xh ** 2))), 1.0, rel_tol=1e-9)
    assert np.allclose(xh, x / np.sqrt(np.mean(x.astype(np.float64) ** 2) + 1e-6), rtol=1e-13)


# ---------------------------------------------------------------- router
def test_route_brute_force_and_softmax():
    rng = np.random.default_rng(5)
    for trial in range(30):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        H = 16
        x = rng.standard_normal((3, H))
        wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
        b = (rng.standard_normal(E)).astype(np.float32)
        r = oracle.route(x, wr, b, k)
        for t in range(3):
            lg = x[t] @ wr.astype(np.float64).T + b.astype(np.float64)
            assert np.allclose(r.logits[t], lg, rtol=1e-13, atol=1e-13)
            order = sorted(range(E), key=lambda e: (-r.logits[t][e], e))
            assert list(r.idx[t]) == order[:k]
            sel = lg[order[:k]]
            p = np.exp(lg - lg.max())
            p /= p.sum()
            ren = p[order[:k]] / p[order[:k]].sum()
            assert np.allclose(r.w[t], ren, rtol=1e-12)
            assert math.isclose(r.w[t].sum(), 1.0, rel_tol=1e-14)
            if k < E:
                assert math.isclose(r.gap[t], r.logits[t][order[k - 1]] - r.logits[t][order[k]], rel_tol=0, abs_tol=1e-15)
            else:
                assert math.isinf(r.gap[t])


def test_route_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(9)
    E, H = 6, 8
    x = rng.standard_normal((1, H))
    wr = rng.standard_normal((E, H)).astype(np.float32)
    r = oracle.route(x, wr, None, E)
    lg = r.logits[0]
    p = np.exp(lg - lg.max())
    p /= p.sum()
    assert np.allclose(r.w[0], p[r.idx[0]], rtol=1e-13)


def test_route_two_experts_closed_form_and_ties():
    x = np.ones((1, 4))
    wr = np.zeros((5, 4), np.float32)
    b = np.array([0.0, 1.5, -2.0, 1.5, 0.25], np.float32)
    r = oracle.route(x, wr, b, 2)
    assert list(r.idx[0]) == [1, 3]          # equal logits: lower id first
    assert np.allclose(r.w[0], [0.5, 0.5])
    b2 = np.array([0.0, 2.0, -1.0, 0.5, 0.1], np.float32)
    r2 = oracle.route(x, wr, b2, 2)
    assert list(r2.idx[0]) == [1, 3]
    assert math.isclose(r2.w[0][0], 1.0 / (1.0 + math.exp(0.5 - 2.0)), rel_tol=1e-14)
    rz = oracle.route(x, wr, None, 3)
    assert list(rz.idx[0]) == [0, 1, 2] and np.allclose(rz.w[0], 1 / 3)


# ---------------------------------------------------------------- expert FFN and layer
def _tiny_cfg():
    return W.MoEConfig("pin", 1, 256, 4, 2, 64, ((W.Q4_K, W.Q4_K, W.Q8_0),), seed=21)


def test_expert_ffn_composition_matches_dense_numpy():
    cfg = _tiny_cfg()
    ex = W.expert(cfg, 0, 1)
    x = np.random.default_rng(1).standard_normal(cfg.H)
    qg, qu, qd = cfg.qtypes(0)
    f = oracle.expert_ffn(cfg.qtypes(0), cfg.H, cfg.I, cfg.down_k(0), ex.gate, ex.up, ex.down, x)
    Wg = oracle.dequant_matrix(qg, ex.gate, cfg.I, cfg.H)
    Wu = oracle.dequant_matrix(qu, ex.up, cfg.I, cfg.H)
    Wd = oracle.dequant_matrix(qd, ex.down, cfg.H, cfg.down_k(0))
    g = Wg @ x
    u = Wu @ x
    a = np.zeros(cfg.down_k(0))
    a[:cfg.I] = g / (1 + np.exp(-g)) * u
    assert np.allclose(f.g, g, rtol=1e-12) and np.allclose(f.u, u, rtol=1e-12)
    assert np.array_equal(f.a, a) or np.allclose(f.a, a, rtol=1e-14)
    assert np.allclose(f.o, Wd @ a, rtol=1e-11)
    z = oracle.expert_ffn(cfg.qtypes(0), cfg.H, cfg.I, cfg.down_k(0), ex.gate, ex.up, ex.down, np.zeros(cfg.H))
    assert np.all(z.o == 0.0)


def _layer(cfg, layer, override=None):
    return oracle.LayerWeights(cfg.qtypes(layer), cfg.H, cfg.I, cfg.down_k(layer), cfg.E, cfg.k,
                               W.router(cfg, layer), W.zipf_bias(cfg, layer),
                               override or (lambda e: W.expert(cfg, layer, e)), cfg.n_shared)


def test_layer_identical_experts_give_that_expert():
    """All experts equal: sum of renormalised weights is one, so y = o."""
    cfg = _tiny_cfg()
    same = W.expert(cfg, 0, 0)
    lw = _layer(cfg, 0, lambda e: same)
    h = W.token(cfg, 0, 0)
    out = oracle.moe_layer_token(lw, h)
    f = oracle.expert_ffn(cfg.qtypes(0), cfg.H, cfg.I, cfg.down_k(0), same.gate, same.up, same.down, out.xhat)
    assert np.allclose(out.y, f.o, rtol=1e-13)
    assert np.allclose(out.h_next, h.astype(np.float64) + f.o, rtol=1e-13)


def test_shared_experts_are_added_with_weight_one():
    cfg = _tiny_cfg().with_(n_shared=2)
    lw = _layer(cfg, 0)
    h = W.token(cfg, 0, 1)
    out = oracle.moe_layer_token(lw, h, keep=True)
    y = sum(out.route.w[0, j] * out.per_expert[int(out.route.idx[0, j])].o for j in range(cfg.k))
    y = y + out.per_expert[cfg.E].o + out.per_expert[cfg.E + 1].o
    assert np.allclose(out.y, y, rtol=1e-13)


# ---------------------------------------------------------------- layer stack
def _dense_layer(cfg, layer, h):
    """One pre-norm residual MoE layer written out densely in numpy from the
    dequantized matrices (dequant_matrix is pinned above by hand-packed
    blocks): RMSNorm, logits, top-k by a stable argsort, softmax over the
    winners, SiLU(gate)*up, down, weighted sum, residual add."""
    h = np.asarray(h, np.float64)
    x = h / np.sqrt(np.mean(h * h) + oracle.RMS_EPS)
    wr = W.router(cfg, layer).astype(np.float64)
    b = W.zipf_bias(cfg, layer)
    lg = wr @ x + (0.0 if b is None else b.astype(np.float64))
    order = np.argsort(-lg, kind="stable")[:cfg.k]
    p = np.exp(lg[order] - lg[order].max())
    p /= p.sum()
    qg, qu, qd = cfg.qtypes(layer)
    y = np.zeros(cfg.H)
    for wj, e in zip(p, order):
        ex = W.expert(cfg, layer, int(e))
        g = oracle.dequant_matrix(qg, ex.gate, cfg.I, cfg.H) @ x
        u = oracle.dequant_matrix(qu, ex.up, cfg.I, cfg.H) @ x
        a = np.zeros(cfg.down_k(layer))
        a[:cfg.I] = g / (1 + np.exp(-g)) * u
        y += wj * (oracle.dequant_matrix(qd, ex.down, cfg.H, cfg.down_k(layer)) @ a)
    return sorted(int(e) for e in order), h + y


def test_stack_token_chains_h_next_with_fp32_rounding():
    """Two layers composed by hand from the dense definition: layer 1 must
    see layer 0's h_next (state plus MoE output, not the MoE output alone),
    rounded to fp32 between the layers; with the rounding switched off the
    chain must follow the unrounded state instead, and the two differ."""
    cfg = W.MoEConfig("pin2", 2, 256, 6, 2, 64, ((W.Q4_K, W.Q4_K, W.Q4_K), (W.Q6_K, W.Q6_K, W.Q8_0)),
                      zipf_s=1.1, seed=33)
    lw = [_layer(cfg, l) for l in range(2)]
    h0 = W.token(cfg, 0, 0)
    ids0, h1 = _dense_layer(cfg, 0, h0)
    h1r = h1.astype(np.float32).astype(np.float64)
    assert not np.array_equal(h1r, h1)  # the rounding is visible at this state
    ids1r, h2r = _dense_layer(cfg, 1, h1r)
    ids1u, h2u = _dense_layer(cfg, 1, h1)
    outs = oracle.stack_token(lw, h0)
    assert sorted(outs[0].route.idx[0].tolist()) == ids0
    assert np.allclose(outs[0].h_next, h1, rtol=1e-12, atol=0)
    assert sorted(outs[1].route.idx[0].tolist()) == ids1r
    assert np.allclose(outs[1].xhat, h1r / np.sqrt(np.mean(h1r * h1r) + oracle.RMS_EPS), rtol=1e-13, atol=0)
    assert np.allclose(outs[1].h_next, h2r, rtol=1e-12, atol=0)
    outs_u = oracle.stack_token(lw, h0, round_state_to_fp32=False)
    assert sorted(outs_u[1].route.idx[0].tolist()) == ids1u
    assert np.allclose(outs_u[1].h_next, h2u, rtol=1e-12, atol=0)
    # the rounded and unrounded chains part by far more than the 1e-12 bars above
    assert np.max(np.abs(outs_u[1].xhat - outs[1].xhat)) > 1e-9 * np.max(np.abs(outs[1].xhat))


@pytest.mark.parametrize("a,b,want", [
    ([1.0, 0.0], [2.0, 0.0], 0.5),                      # the reference's norm is the denominator
    ([2.0, 0.0], [1.0, 0.0], 1.0),
    ([0.0, 5.0], [3.0, 4.0], math.sqrt(10.0) / 5.0),    # ||(-3, 1)|| / 5
    ([[1.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 2.0]], math.sqrt(5.0) / 2.0),  # whole array, not per row
    ([3.0, 4.0], [0.0, 0.0], 5.0),                      # zero reference: the absolute norm
    ([1.0, -2.0, 2.0], [1.0, -2.0, 2.0], 0.0),
])
def test_rel_l2_closed_forms(a, b, want):
    assert math.isclose(oracle.rel_l2(np.array(a), np.array(b)), want, rel_tol=1e-15, abs_tol=0.0)


def test_rel_l2_scale_invariant_and_relative():
    b = np.random.default_rng(5).standard_normal(1000)
    assert math.isclose(oracle.rel_l2(b * (1 + 1e-3), b), 1e-3, rel_tol=1e-9)
    assert math.isclose(oracle.rel_l2(1e6 * b * (1 - 2e-4), 1e6 * b), 2e-4, rel_tol=1e-9)


# ---------------------------------------------------------------- grouping
def test_group_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(50):
        E = int(rng.integers(1, 20))
        T = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        g = oracle.group(idx, E)
        brute = []
        for e in range(E):
            assert g.count[e] == int((idx == e).sum())
            for t in range(T):
                for j in range(k):
                    if idx[t, j] == e:
                        brute.append(t * k + j)
        assert list(g.pairs) == brute
        assert g.offset[0] == 0 and g.offset[-1] == T * k
        for e in range(E):
            seg = g.pairs[g.offset[e]:g.offset[e + 1]]
            assert all(idx.ravel()[p] == e for p in seg)


# ---------------------------------------------------------------- slot planner
def test_cache_plan_reproduces_page_example():
    g = _gold("t4_cache_plan_example.json")
    H, I, E, k = g["H"], g["I"], g["E"], g["top_k"]
    q4 = W.matrix_bytes(W.Q4_K, I, H)
    e_bytes = [3 * q4, 2 * q4 + W.matrix_bytes(W.Q6_K, H, I)]
    layers = [24, 24]
    pr = g["printed"]
    rc, slots = oracle.cache_plan(e_bytes, layers, pr["budget_mib"] * 2 ** 20, k)
    assert rc == 0 and list(slots) == [pr["slots_per_group"]] * 2
    assert round(100 * slots[0] / (24 * E), 1) == pr["share_of_experts_pct"]
    rc, slots = oracle.cache_plan(e_bytes, layers, pr["floor_ok_mib"] * 2 ** 20, k)
    assert rc == 0 and all(s >= k for s in slots)
    rc, slots = oracle.cache_plan(e_bytes, layers, pr["floor_fail_mib"] * 2 ** 20, k)
    assert rc == -1 and all(s == 0 for s in slots)


def test_cache_plan_single_group_fraction():
    # one group, budget covering exactly 10 experts of 4 layers -> floor(10) - 1
    rc, s = oracle.cache_plan([1000], [4], 10_000, 2)
    assert rc == 0 and list(s) == [9]
    rc, s = oracle.cache_plan([1000], [4], 2_999, 2)
    assert rc == -1 and list(s) == [0]


# ---------------------------------------------------------------- LRU
def test_lru_hand_worked_sequence():
    seq = [1, 2, 3, 1, 4, 2, 5, 1, 3, 4]
    tr = oracle.lru([3], [0], np.zeros(len(seq), np.int32), np.array(seq, np.int32))
    assert list(tr.hit) == [0, 0, 0, 1, 0, 0, 0, 0, 0, 0]
    assert list(tr.victim_expert) == [-1, -1, -1, -1, 2, 3, 1, 4, 2, 5]
    assert list(tr.slot) == [0, 1, 2, 0, 1, 2, 0, 1, 2, 0]


def _mattson_hits(keys, cap):
    """Stack-distance brute force: a reference hits iff fewer than `cap`
    distinct keys were referenced since its previous reference."""
    out = []
    for i, k in enumerate(keys):
        prev = None
        for j in range(i - 1, -1, -1):
            if keys[j] == k:
                prev = j
                break
        if prev is None:
            out.append(0)
        else:
            out.append(1 if len(set(keys[prev + 1:i])) < cap else 0)
    return out


def _brute_victims(keys, cap):
    """Victim = resident key whose last use is oldest (scan of the history)."""
    resident = []
    vic = []
    for i, k in enumerate(keys):
        if k in resident:
            vic.append(None)
            continue
        if len(resident) < cap:
            resident.append(k)
            vic.append(None)
            continue
        last = {r: max(j for j in range(i) if keys[j] == r) for r in resident}
        v = min(resident, key=lambda r: last[r])
        resident.remove(v)
        resident.append(k)
        vic.append(v)
    return vic


def test_lru_matches_stack_distance_and_victim_scan():
    rng = random.Random(3)
    for trial in range(25):
        n_layers = rng.randrange(1, 4)
        n_exp = rng.randrange(2, 10)
        cap = rng.randrange(1, 8)
        keys = [(rng.randrange(n_layers), rng.randrange(n_exp)) for _ in range(120)]
        tr = oracle.lru([cap], [0] * n_layers, np.array([k[0] for k in keys], np.int32),
                        np.array([k[1] for k in keys], np.int32))
        assert list(tr.hit) == _mattson_hits(keys, cap)
        vic = _brute_victims(keys, cap)
        for i, v in enumerate(vic):
            if v is None:
                assert tr.victim_layer[i] == -1 and tr.victim_expert[i] == -1
            else:
                assert (tr.victim_layer[i], tr.victim_expert[i]) == v


def test_lru_groups_are_independent_pools():
    keys = [(0, 1), (1, 1), (0, 2), (1, 2), (0, 1), (1, 1)]
    tr = oracle.lru([2, 1], [0, 1], np.array([k[0] for k in keys], np.int32),
                    np.array([k[1] for k in keys], np.int32))
    # group 0 (layer 0, 2 slots) keeps experts 1 and 2; group 1 (layer 1, 1 slot) thrashes
    assert list(tr.hit) == [0, 0, 0, 0, 1, 0]
    assert list(tr.victim_layer) == [-1, -1, -1, 1, -1, 1]
    assert list(tr.victim_expert) == [-1, -1, -1, 1, -1, 2]


def test_lru_large_capacity_gives_compulsory_misses_only():
    rng = random.Random(5)
    keys = [(rng.randrange(3), rng.randrange(6)) for _ in range(200)]
    tr = oracle.lru([18], [0, 0, 0], np.array([k[0] for k in keys], np.int32),
                    np.array([k[1] for k in keys], np.int32))
    first = []
    seen = set()
    for k in keys:
        first.append(0 if k not in seen else 1)
        seen.add(k)
    assert list(tr.hit) == first


def test_prefetch_lookup_sequence_order():
    """Worked by hand: at layer 0 the predicted experts of layers 1 and 2 are
    looked up right after layer 0's own; an empty schedule is the plain
    order; a perfect prediction on a pool that holds everything turns every
    later lookup of the prefetched layers into hits."""
    ids = np.array([[[3, 1], [2, 2], [0, 4]]], np.int32)
    pred = np.array([[[9, 9], [5, 2], [4, 4]]], np.int32)
    L, E = oracle.prefetch_lookup_sequence(ids, pred, [[1, 2], [], []])
    assert list(L) == [0, 0, 1, 1, 2, 1, 2, 2] and list(E) == [1, 3, 2, 5, 4, 2, 0, 4]
    L0, E0 = oracle.prefetch_lookup_sequence(ids, pred, [[], [], []])
    L1, E1 = oracle.lookup_sequence(ids)
    assert np.array_equal(L0, L1) and np.array_equal(E0, E1)
    tr = oracle.lru([16], [0, 0, 0], *oracle.prefetch_lookup_sequence(ids, ids, [[1, 2], [], []]))
    assert list(tr.hit) == [0, 0, 0, 0, 0, 1, 1, 1]


def test_lookup_sequence_order():
    ids = np.array([[[3, 1, 3, 0], [2, 2, 2, 2]]], np.int32)
    L, E = oracle.lookup_sequence(ids)
    assert list(L) == [0, 0, 0, 1] and list(E) == [0, 1, 3, 2]
