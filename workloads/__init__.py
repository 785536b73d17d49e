"""Seeded synthetic inputs for the decode-time MoE expert FFN.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no arithmetic of the method itself: it only draws
random fields and lays the quantized-block bytes out in the public GGUF
block format (Q8_0, Q4_K, Q6_K), so that both sides read identical bytes.

Every array is a pure function of (config seed, layer, expert, matrix) or
(config seed, step, token, attempt), drawn through numpy's PCG64 from a
SeedSequence built on that tuple.  Any single expert can therefore be
regenerated on its own, which lets the oracle check sampled tokens of a
16 GB layer stack without materialising the whole stack.

Workload shapes follow the configurations the method is measured on:
a tiny single Q8_0 layer, a Qwen3-30B-A3B-shaped 48-layer Q4_K stack
(the model measured in the T4 MoE-cache report, kongchang.com, section
"T4 results"), the same stack with Zipf-skewed routing, the slot-pool cache
trace, and a mixed Q4_K/Q6_K stack with two always-active shared experts
(the 64 routed + 2 shared layout of the laptop 16B MoE post, lpnh.cn, §1.1).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

# qtype codes (same numbering as the C ABI)
Q8_0 = 1
Q4_K = 2
Q6_K = 3

QNAME = {Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K"}

# weights per block and bytes per block of each format
QK = {Q8_0: 32, Q4_K: 256, Q6_K: 256}
QBYTES = {Q8_0: 34, Q4_K: 144, Q6_K: 210}

# salts that keep the different random streams of one config apart
_SALT_ROUTER = 1_000_001
_SALT_BIAS = 1_000_002
_SALT_X = 2_000_000


def padded_k(qtype: int, k: int) -> int:
    """Row length after padding up to a whole number of blocks."""
    b = QK[qtype]
    return (k + b - 1) // b * b


def matrix_bytes(qtype: int, n: int, k: int) -> int:
    """Bytes of an [n, k] matrix in `qtype` blocks (rows padded to whole blocks)."""
    return n * (padded_k(qtype, k) // QK[qtype]) * QBYTES[qtype]


@dataclass(frozen=True)
class MoEConfig:
    name: str
    n_layers: int
    H: int
    E: int
    k: int
    I: int
    # per-layer (gate, up, down) qtypes
    layer_qtypes: Tuple[Tuple[int, int, int], ...]
    n_shared: int = 0
    zipf_s: Optional[float] = None
    zero_mean: bool = False
    seed: int = 1
    T: int = 1

    def qtypes(self, layer: int) -> Tuple[int, int, int]:
        return self.layer_qtypes[layer]

    def down_k(self, layer: int) -> int:
        """Row length of the down matrix: I padded to whole 256-weight groups
        (the padded columns multiply a zero tail of the activation)."""
        return (self.I + 255) // 256 * 256

    def expert_bytes(self, layer: int) -> int:
        qg, qu, qd = self.qtypes(layer)
        return (matrix_bytes(qg, self.I, self.H) + matrix_bytes(qu, self.I, self.H)
                + matrix_bytes(qd, self.H, self.down_k(layer)))

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


def _uniform_layers(n: int, q: int) -> Tuple[Tuple[int, int, int], ...]:
    return tuple((q, q, q) for _ in range(n))


def tiny_q8_0(seed: int = 1) -> MoEConfig:
    """Single MoE layer: T=1, H=256, E=8, top-2, I=512, Q8_0 experts."""
    return MoEConfig("tiny-q8_0-H256-E8-k2-I512", 1, 256, 8, 2, 512,
                     _uniform_layers(1, Q8_0), seed=seed, T=1)


def qwen3_30b_a3b_q4k(T: int = 1, seed: int = 2, n_layers: int = 48) -> MoEConfig:
    """Qwen3-30B-A3B-shaped stack: 48 layers, H=2048, E=128, top-8, I=768, Q4_K."""
    return MoEConfig(f"qwen3-30b-a3b-shaped-q4k-L{n_layers}-T{T}", n_layers, 2048, 128, 8, 768,
                     _uniform_layers(n_layers, Q4_K), seed=seed, T=T)


def qwen3_30b_a3b_q4k_zipf(T: int = 32, seed: int = 3, n_layers: int = 48) -> MoEConfig:
    """Same stack with a Zipf(s=1.1) per-expert router bias (skewed expert loads)."""
    return MoEConfig(f"qwen3-30b-a3b-shaped-q4k-zipf-L{n_layers}-T{T}", n_layers, 2048, 128, 8, 768,
                     _uniform_layers(n_layers, Q4_K), zipf_s=1.1, seed=seed, T=T)


def qwen3_cache_trace(n_layers: int = 48) -> MoEConfig:
    """The slot-pool cache's decode trace stack: the Qwen3-30B-A3B-shaped
    Q4_K stack (same experts and routers, seed 2) with a Zipf(s=1.1) router
    bias; each decode step is one fresh N(0, 1) token."""
    return qwen3_30b_a3b_q4k(T=1, n_layers=n_layers).with_(
        zipf_s=1.1, name=f"qwen3-30b-a3b-shaped-q4k-zipf-cache-trace-L{n_layers}")


def mixed_shared_q4k_q6k(T: int = 1, seed: int = 5, n_layers: int = 24) -> MoEConfig:
    """24 layers, H=2048, 64 routed (top-2) + 2 shared experts, I=1408;
    layers 0-11 Q4_K, 12-23 Q6_K (down rows padded to 1536)."""
    half = n_layers // 2
    lq = tuple([(Q4_K,) * 3] * half + [(Q6_K,) * 3] * (n_layers - half))
    return MoEConfig(f"mixed-shared-q4k-q6k-L{n_layers}-T{T}", n_layers, 2048, 64, 2, 1408, lq,
                     n_shared=2, seed=seed, T=T)


# ---------------------------------------------------------------------------
# random streams


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def _fp16_bits(vals: np.ndarray) -> np.ndarray:
    """Round fp64 draws to IEEE half (numpy's round-to-nearest-even) and return the bits."""
    return vals.astype(np.float16).view(np.uint16)


def q8_0_matrix(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """[n, k/32*34] uint8: per block fp16 d ~ U[0.001, 0.01], then 32 int8 q ~ U{-127..127}."""
    nb = n * (k // 32)
    blk = np.empty((nb, 34), np.uint8)
    blk[:, 0:2] = _fp16_bits(rng.uniform(0.001, 0.01, nb)).view(np.uint8).reshape(nb, 2)
    blk[:, 2:34] = rng.integers(-127, 128, (nb, 32), dtype=np.int8).view(np.uint8)
    return blk.reshape(n, -1)


def q4_k_matrix(rng: np.random.Generator, n: int, k: int, zero_mean: bool = False) -> np.ndarray:
    """[n, k/256*144] uint8.  Block = fp16 d, fp16 dmin, 12 scale bytes, 128 quant bytes.

    Scale and quant bytes are uniform random bytes, so every 6-bit scale/min
    and every 4-bit quant is uniform on its range.  d ~ U[0.001, 0.01].
    dmin ~ U[0.001, 0.01]; with zero_mean it is 7.5*d instead, which centres
    the weight distribution (E[q] = 7.5 and E[sc] = E[m]).
    """
    nb = n * (k // 256)
    blk = np.frombuffer(rng.bytes(nb * 144), np.uint8).reshape(nb, 144).copy()
    d = rng.uniform(0.001, 0.01, nb)
    dmin = 7.5 * d if zero_mean else rng.uniform(0.001, 0.01, nb)
    blk[:, 0:2] = _fp16_bits(d).view(np.uint8).reshape(nb, 2)
    blk[:, 2:4] = _fp16_bits(dmin).view(np.uint8).reshape(nb, 2)
    return blk.reshape(n, -1)


def q6_k_matrix(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """[n, k/256*210] uint8.  Block = 128 low-nibble bytes, 64 high-bit bytes,
    16 int8 sub-scales (uniform random bytes), then fp16 d ~ U[0.001, 0.01]."""
    nb = n * (k // 256)
    blk = np.frombuffer(rng.bytes(nb * 210), np.uint8).reshape(nb, 210).copy()
    blk[:, 208:210] = _fp16_bits(rng.uniform(0.001, 0.01, nb)).view(np.uint8).reshape(nb, 2)
    return blk.reshape(n, -1)


def quant_matrix(qtype: int, rng: np.random.Generator, n: int, k: int, zero_mean: bool = False) -> np.ndarray:
    kp = padded_k(qtype, k)
    if qtype == Q8_0:
        return q8_0_matrix(rng, n, kp)
    if qtype == Q4_K:
        return q4_k_matrix(rng, n, kp, zero_mean)
    if qtype == Q6_K:
        return q6_k_matrix(rng, n, kp)
    raise ValueError(f"unknown qtype {qtype}")


@dataclass
class ExpertBytes:
    """One expert's three matrices in canonical block bytes (row-major, blocks along k)."""
    gate: np.ndarray   # [I, H/bs*bb]
    up: np.ndarray     # [I, H/bs*bb]
    down: np.ndarray   # [H, Ipad/bs*bb]

    def concat(self) -> np.ndarray:
        return np.concatenate([self.gate.ravel(), self.up.ravel(), self.down.ravel()])


def expert(cfg: MoEConfig, layer: int, e: int) -> ExpertBytes:
    """Expert e of a layer; e in [E, E+n_shared) are the shared experts."""
    qg, qu, qd = cfg.qtypes(layer)
    mats = []
    for m, (q, n, kk) in enumerate(((qg, cfg.I, cfg.H), (qu, cfg.I, cfg.H), (qd, cfg.H, cfg.down_k(layer)))):
        mats.append(quant_matrix(q, _rng(cfg.seed, layer, e, m), n, kk, cfg.zero_mean))
    return ExpertBytes(*mats)


def router(cfg: MoEConfig, layer: int) -> np.ndarray:
    """fp32 router weights [E, H] ~ N(0, 0.02^2)."""
    return (_rng(cfg.seed, layer, _SALT_ROUTER).standard_normal((cfg.E, cfg.H)) * 0.02).astype(np.float32)


def zipf_bias(cfg: MoEConfig, layer: int) -> Optional[np.ndarray]:
    """fp32 [E] logit bias ln p_{pi(e)}, p_r proportional to r^-s over ranks 1..E,
    pi a seeded per-layer permutation of the experts.  None when unbiased."""
    if cfg.zipf_s is None:
        return None
    ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = ranks ** (-cfg.zipf_s)
    p /= p.sum()
    perm = _rng(cfg.seed, layer, _SALT_BIAS).permutation(cfg.E)
    return np.log(p[perm]).astype(np.float32)


def token(cfg: MoEConfig, step: int, t: int, attempt: int = 0) -> np.ndarray:
    """fp32 [H] input state of token t at decode step `step` ~ N(0, 1)."""
    return _rng(cfg.seed, _SALT_X, step, t, attempt).standard_normal(cfg.H).astype(np.float32)


def tokens(cfg: MoEConfig, step: int, T: int, attempts: Optional[Sequence[int]] = None) -> np.ndarray:
    att = attempts if attempts is not None else [0] * T
    return np.stack([token(cfg, step, t, att[t]) for t in range(T)])


def tie_free_tokens(cfg: MoEConfig, step: int, T: int, min_gap_of, gap: float = 1e-4,
                    max_attempts: int = 64) -> Tuple[np.ndarray, list]:
    """Draw T tokens, redrawing any token whose routing has a near-tie.

    `min_gap_of(x)` is supplied by the caller (the oracle in tests) and returns
    the smallest gap, over all layers, between the k-th and (k+1)-th router
    logit of the token's chain.  A token is redrawn from the next attempt
    sub-seed until the gap is at least `gap`.  Returns (x [T,H], attempts).
    """
    xs, atts = [], []
    for t in range(T):
        for a in range(max_attempts):
            x = token(cfg, step, t, a)
            if min_gap_of(x) >= gap:
                xs.append(x)
                atts.append(a)
                break
        else:
            raise RuntimeError(f"no tie-free draw for token {t} in {max_attempts} attempts")
    return np.stack(xs), atts
