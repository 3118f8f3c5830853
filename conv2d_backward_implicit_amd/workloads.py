"""Seeded synthetic workloads: shapes and input generators only.

This module holds no convolution arithmetic.  It is the one piece shared by
the tests, the benchmark and the smoke check: it names the problem shapes and
draws the seeded grad_out / weight arrays that both the HIP path and the CPU
oracle consume.

Shapes are the ResNet/ImageNet-style layer shapes the method is exercised on;
every extent, including the output extent, is written out literally.
Inputs are drawn with numpy's PCG64 generator (``default_rng(seed)``) in
float64, grad_out first and weight second, then cast to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import numpy as np


@dataclass(frozen=True)
class ConvShape:
    name: str
    batch: int
    in_channels: int
    in_h: int
    in_w: int
    out_channels: int
    kernel_h: int
    kernel_w: int
    stride: int
    padding_h: int
    padding_w: int
    out_h: int
    out_w: int
    f16_staged: bool = False
    # distribution of grad_out / weight: "uniform" -> U[-1, 1] for both;
    # "normal" -> grad_out ~ N(0, 1), weight ~ N(0, 2 / weight_fan_in)
    dist: str = "normal"
    weight_fan_in: int = 1

    def as_dict(self):
        return asdict(self)

    @property
    def go_shape(self):
        return (self.batch, self.out_channels, self.out_h, self.out_w)

    @property
    def w_shape(self):
        return (self.out_channels, self.in_channels, self.kernel_h, self.kernel_w)

    @property
    def gi_shape(self):
        return (self.batch, self.in_channels, self.in_h, self.in_w)

    @property
    def useful_flops(self) -> int:
        """2 * N * Co * OH * OW * Ci * KH * KW (every output-pixel x tap pair)."""
        return (2 * self.batch * self.out_channels * self.out_h * self.out_w
                * self.in_channels * self.kernel_h * self.kernel_w)

    @property
    def compulsory_bytes(self) -> int:
        """fp32 grad_out + weight read once, fp32 grad_input written once."""
        n = (self.batch * self.out_channels * self.out_h * self.out_w
             + self.out_channels * self.in_channels * self.kernel_h * self.kernel_w
             + self.batch * self.in_channels * self.in_h * self.in_w)
        return 4 * n


# The five workloads; the index is also the seed of its inputs.
CONFIGS = [
    ConvShape("tiny_n1_c8_k16_8x8_3x3_s1", 1, 8, 8, 8, 16, 3, 3, 1, 1, 1, 8, 8,
              dist="uniform"),
    ConvShape("resnet_stage1_n32_c64_k64_56x56_3x3_s1", 32, 64, 56, 56, 64, 3, 3,
              1, 1, 1, 56, 56, weight_fan_in=64 * 9),
    ConvShape("strided_down_n32_c128_k256_56x56_3x3_s2", 32, 128, 56, 56, 256, 3,
              3, 2, 1, 1, 28, 28, weight_fan_in=128 * 9),
    ConvShape("pointwise_n64_c256_k1024_14x14_1x1_f16", 64, 256, 14, 14, 1024, 1,
              1, 1, 0, 0, 14, 14, f16_staged=True, weight_fan_in=256),
    ConvShape("stem_n16_c3_k64_224x224_7x7_s2", 16, 3, 224, 224, 64, 7, 7, 2, 3,
              3, 112, 112, weight_fan_in=3 * 49),
]

# The workload the headline throughput is quoted on: the largest one, and
# the one that runs the stride-residue path (3x3, stride 2, 128 -> 256
# channels at 56x56).
HEADLINE = 2


def by_name(name: str) -> ConvShape:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def draw(shape: ConvShape, seed: int):
    """(grad_out, weight) as float32 arrays, drawn from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    if shape.dist == "uniform":
        go = rng.uniform(-1.0, 1.0, size=shape.go_shape)
        w = rng.uniform(-1.0, 1.0, size=shape.w_shape)
    elif shape.dist == "normal":
        go = rng.standard_normal(size=shape.go_shape)
        w = rng.standard_normal(size=shape.w_shape) * np.sqrt(2.0 / shape.weight_fan_in)
    else:
        raise ValueError(shape.dist)
    return go.astype(np.float32), w.astype(np.float32)


def draw_forward(shape: ConvShape, seed: int):
    """(x, weight) for the forward convolution of ``shape``: x [N, Ci, H, W]
    with grad_out's distribution and weight as in ``draw`` (float32)."""
    rng = np.random.default_rng(seed)
    if shape.dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape.gi_shape)
        w = rng.uniform(-1.0, 1.0, size=shape.w_shape)
    elif shape.dist == "normal":
        x = rng.standard_normal(size=shape.gi_shape)
        w = rng.standard_normal(size=shape.w_shape) * np.sqrt(2.0 / shape.weight_fan_in)
    else:
        raise ValueError(shape.dist)
    return x.astype(np.float32), w.astype(np.float32)


def draw_integers(shape: ConvShape, seed: int, lo: int = -4, hi: int = 4):
    """(grad_out, weight) with integer values in [lo, hi], stored as float32.

    Such values are exact in float16 and float32, so any summation order of
    products stays exact while partial sums stay below 2**24.
    """
    rng = np.random.default_rng(seed)
    go = rng.integers(lo, hi + 1, size=shape.go_shape)
    w = rng.integers(lo, hi + 1, size=shape.w_shape)
    return go.astype(np.float32), w.astype(np.float32)


def random_shape(rng: np.random.Generator, max_n=2, max_c=5, max_hw=9, max_k=5,
                 max_s=3, name="random") -> ConvShape:
    """A small random problem: any stride, asymmetric padding up to k.

    Output extents follow the forward-convolution size rule
    floor((in + 2p - k) / s) + 1 and the draw is repeated until both are >= 1.
    """
    while True:
        n = int(rng.integers(1, max_n + 1))
        ci = int(rng.integers(1, max_c + 1))
        co = int(rng.integers(1, max_c + 1))
        kh = int(rng.integers(1, max_k + 1))
        kw = int(rng.integers(1, max_k + 1))
        s = int(rng.integers(1, max_s + 1))
        ph = int(rng.integers(0, kh + 1))
        pw = int(rng.integers(0, kw + 1))
        h = int(rng.integers(1, max_hw + 1))
        w = int(rng.integers(1, max_hw + 1))
        oh = (h + 2 * ph - kh) // s + 1 if h + 2 * ph >= kh else 0
        ow = (w + 2 * pw - kw) // s + 1 if w + 2 * pw >= kw else 0
        if oh >= 1 and ow >= 1:
            return ConvShape(name, n, ci, h, w, co, kh, kw, s, ph, pw, oh, ow,
                             dist="uniform")


# ---- RMSNorm-fused matrix product (C = RmsNorm(X, g) x W) ---------------------

@dataclass(frozen=True)
class RmsShape:
    """X [m, k] tokens x hidden, g [k] norm scale, W [k, n] projection."""
    name: str
    m: int
    k: int
    n: int
    eps: float = 1e-6

    @property
    def useful_flops(self) -> int:
        return 2 * self.m * self.k * self.n

    @property
    def compulsory_bytes(self) -> int:
        return 4 * (self.m * self.k + self.k + self.k * self.n + self.m * self.n)


# The source page gives no sizes; these stand in: a ragged case the oracle
# finishes at once, and LLM-style projections (tokens x hidden -> out).
RMS_CONFIGS = [
    RmsShape("rms_tiny_m7_k45_n19", 7, 45, 19),
    RmsShape("rms_proj_m8192_k4096_n4096", 8192, 4096, 4096),
    RmsShape("rms_mlp_up_m4096_k4096_n11008", 4096, 4096, 11008),
    RmsShape("rms_ragged_m3000_k1000_n1500", 3000, 1000, 1500),
]

RMS_HEADLINE = 1


def rms_by_name(name: str) -> RmsShape:
    for c in RMS_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def draw_rms(shape: RmsShape, seed: int):
    """(x, g, w) as float32: x ~ N(0, 1), g ~ 1 + 0.1 N(0, 1), w ~ N(0, 1/k),
    drawn in that order from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((shape.m, shape.k))
    g = 1.0 + 0.1 * rng.standard_normal(shape.k)
    w = rng.standard_normal((shape.k, shape.n)) / np.sqrt(shape.k)
    return x.astype(np.float32), g.astype(np.float32), w.astype(np.float32)


# ---- attention dV (dV of softmax(QK^T / sqrt(D)) V, grouped kv heads) ---------

@dataclass(frozen=True)
class MhaShape:
    """q, dO [q_seq, heads, D]; k, dV [kv_seq, kv_heads, D]; lse [q_seq, heads, 2].
    Query pos sees key t when t <= pos (causal) and pos < t + window (window
    > 0)."""
    name: str
    q_seq: int
    kv_seq: int
    heads: int
    kv_heads: int
    head_dim: int = 64
    window: int = 0
    causal: bool = True

    def pairs(self) -> int:
        """(query, key) pairs the mask lets through, per head."""
        n = 0
        for t in range(self.kv_seq):
            start = t if self.causal else 0
            end = min(self.q_seq, t + self.window) if self.window > 0 else self.q_seq
            n += max(0, end - start)
        return n

    @property
    def useful_flops(self) -> int:
        # per visible (query, head, key): the score (2 D) and its dV term (2 D)
        return 4 * self.head_dim * self.heads * self.pairs()

    @property
    def compulsory_bytes(self) -> int:
        return 4 * (2 * self.q_seq * self.heads * self.head_dim + self.q_seq * self.heads * 2
                    + 2 * self.kv_seq * self.kv_heads * self.head_dim)


# The source page gives no sizes; these stand in: a ragged case the oracle
# finishes at once, and LLM-style single sequences (32 query heads sharing 8
# kv heads, head dimension 64).
MHA_CONFIGS = [
    MhaShape("mha_tiny_s37_h4_kv2_causal", 37, 37, 4, 2),
    MhaShape("mha_s4096_h32_kv8_causal", 4096, 4096, 32, 8),
    MhaShape("mha_s4096_h32_kv8_causal_window512", 4096, 4096, 32, 8, window=512),
    MhaShape("mha_s2048_h16_kv16_full", 2048, 2048, 16, 16, causal=False),
]

MHA_HEADLINE = 1


def mha_by_name(name: str) -> MhaShape:
    for c in MHA_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def draw_mha(shape: MhaShape, seed: int):
    """(q, k, dout) as float32 N(0, 1), drawn in that order from
    ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((shape.q_seq, shape.heads, shape.head_dim))
    k = rng.standard_normal((shape.kv_seq, shape.kv_heads, shape.head_dim))
    g = rng.standard_normal((shape.q_seq, shape.heads, shape.head_dim))
    return q.astype(np.float32), k.astype(np.float32), g.astype(np.float32)
