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

Gate weights are bf16 N(0, 0.02^2) in every config.
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


def sample_rows(T, n, seed=0):
    """Sorted distinct row indices for checks at full size (first and last row included)."""
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng([1, int(seed), int(T)]).choice(T, n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], r]))
