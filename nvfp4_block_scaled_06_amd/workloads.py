"""Seeded synthetic router workloads (inputs only; none of the method's arithmetic).

Shared by the tests, the benchmark and the oracle's CPU-baseline timing, so
that both sides of every parity check see the same bytes. Every tensor comes
from ``numpy.random.default_rng([0, cfg, tensor_id + 100 * layer])`` and bf16
values are fp32 samples rounded to nearest-even bf16.

Tensor ids: x = 0, gate weights = 1, bias = 2, outlier channel set = 3,
per-token magnitudes = 4.

The five router shapes (D = hidden size, E = routed experts, k = experts
per token, r = routed scale):

====  ==============  =====  ====  ===  ==  ===  ====================================
cfg   name            T      D     E    k   r    structure
====  ==============  =====  ====  ===  ==  ===  ====================================
1     tiny            4      256   16   2   1.0  x ~ N(0,1); bias ~ U(-0.01, 0.01)
2     decode          1      7168  256  8   2.5  61 layer sets (x token, W, bias each)
3     batched_decode  64     7168  256  8   2.5  61 layer sets; 72 of 7168 channels x50
4     prefill         8192   7168  256  8   2.5  x[t] = m_t * N(0,1), m_t ~ LogNormal(0,0.5)
5     large_prefill   32768  7168  384  8   2.5  x ~ Student-t(4); bias ~ U(-0.05, 0.05)
====  ==============  =====  ====  ===  ==  ===  ====================================

Gate weights are bf16 N(0, 0.02^2) in every config. Grouped-layer shapes
(configs 11..13) are listed in GROUPED_CONFIGS.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class RouterConfig:
    cfg: int
    name: str
    T: int
    D: int
    E: int
    k: int
    routed_scale: float
    layers: int
    bias_half_width: float


CONFIGS = {
    1: RouterConfig(1, "tiny", 4, 256, 16, 2, 1.0, 1, 0.01),
    2: RouterConfig(2, "decode", 1, 7168, 256, 8, 2.5, 61, 0.01),
    3: RouterConfig(3, "batched_decode", 64, 7168, 256, 8, 2.5, 61, 0.01),
    4: RouterConfig(4, "prefill", 8192, 7168, 256, 8, 2.5, 1, 0.01),
    5: RouterConfig(5, "large_prefill", 32768, 7168, 384, 8, 2.5, 1, 0.05),
}

OUTLIER_CHANNELS = 72  # 1 % of 7168
OUTLIER_FACTOR = 50.0
W_STD = 0.02


def rng(cfg, tensor_id, layer=0):
    return np.random.default_rng([0, int(cfg), int(tensor_id) + 100 * int(layer)])


def bf16_bits(a):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_x(cfg, layer=0):
    """Activations [T, D] as bf16 bit patterns."""
    c = CONFIGS[cfg]
    if cfg in (1, 2):
        a = rng(cfg, 0, layer).standard_normal((c.T, c.D), dtype=np.float32)
    elif cfg == 3:
        a = rng(cfg, 0, layer).standard_normal((c.T, c.D), dtype=np.float32)
        ch = rng(cfg, 3).choice(c.D, OUTLIER_CHANNELS, replace=False)
        a[:, ch] *= np.float32(OUTLIER_FACTOR)
    elif cfg == 4:
        a = rng(cfg, 0, layer).standard_normal((c.T, c.D), dtype=np.float32)
        m = rng(cfg, 4, layer).lognormal(0.0, 0.5, size=c.T).astype(np.float32)
        a *= m[:, None]
    elif cfg == 5:
        a = rng(cfg, 0, layer).standard_t(4.0, size=(c.T, c.D)).astype(np.float32)
    else:
        raise ValueError(cfg)
    return bf16_bits(a)


def make_w(cfg, layer=0):
    """Gate weights [E, D] as bf16 bit patterns (quantized later by each side)."""
    c = CONFIGS[cfg]
    a = rng(cfg, 1, layer).standard_normal((c.E, c.D), dtype=np.float32) * np.float32(W_STD)
    return bf16_bits(a)


def make_bias(cfg, layer=0):
    """Selection bias [E] fp32."""
    c = CONFIGS[cfg]
    h = c.bias_half_width
    return rng(cfg, 2, layer).uniform(-h, h, size=c.E).astype(np.float32)


@dataclass(frozen=True)
class GroupedConfig:
    """A grouped linear layer: G groups of padded_rows rows each (flattened to [G * P, D]) and G weights
    [N, D], one per group."""
    cfg: int
    name: str
    G: int
    P: int
    D: int
    N: int


# Grouped layers (the step after the router: the routed experts' projections). No sizes are given for them, so
# these take a DeepSeek-V3-shaped expert: D = 7168 in, N = 4096 out (the gate and up projections of a
# 2048-wide expert side by side), G = 8 groups (the k = 8 experts a token is routed to). Decode: one row per
# group; prefill: 1024 rows per group (8192 routed rows).
GROUPED_CONFIGS = {
    11: GroupedConfig(11, "grouped_tiny", 3, 5, 256, 48),
    12: GroupedConfig(12, "grouped_decode", 8, 1, 7168, 4096),
    13: GroupedConfig(13, "grouped_prefill", 8, 1024, 7168, 4096),
}


def make_grouped_x(gcfg):
    """Flattened activations [G * P, D] bf16: N(0,1) rows times a LogNormal(0, 0.5) magnitude per row."""
    c = GROUPED_CONFIGS[gcfg]
    a = rng(gcfg, 0).standard_normal((c.G * c.P, c.D), dtype=np.float32)
    a *= rng(gcfg, 4).lognormal(0.0, 0.5, size=c.G * c.P).astype(np.float32)[:, None]
    return bf16_bits(a)


def make_grouped_w(gcfg, g):
    """Group g's weight [N, D] bf16 ~ N(0, 0.02^2)."""
    c = GROUPED_CONFIGS[gcfg]
    return bf16_bits(rng(gcfg, 1, g).standard_normal((c.N, c.D), dtype=np.float32) * np.float32(W_STD))


def sample_rows(T, n, seed=0):
    """Sorted distinct row indices for checks at full size (first and last row included)."""
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng([1, int(seed), int(T)]).choice(T, n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], r]))
