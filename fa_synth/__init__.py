"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no attention arithmetic.  It only draws i.i.d. normal
values and rounds them to bfloat16 (or IEEE half) bit patterns, so that the
GPU path and the CPU oracle see exactly the same input bits.

Recipe (the same for every workload): numpy ``Generator(PCG64(seed))``
standard normals drawn in float32, multiplied by ``sigma``, rounded to
bfloat16 with round-to-nearest-even on the bit pattern (or to binary16 by
numpy's round-to-nearest-even cast).  Tensors are contiguous
``[B, H, L, D]`` with D innermost; a workload's ``layout`` only says how the
GPU side places them.

Block masks (inputs of the block-sparse calls) are uint8
``[ceil(Lq/64), ceil(Lk/64)]`` arrays, 1 = the 64 x 64 block is kept:
``random_block_mask`` draws each entry Bernoulli(density) from its own
seeded generator; ``window_block_mask`` keeps, for every query block, the
key blocks that overlap a band of ``window`` keys ending at the block's last
query row (bottom-right aligned, as the causal diagonal), plus the first
``sink_blocks`` key blocks.

``ramp_bits`` builds inputs whose scores rise steadily along the keys
(a shared direction u in Q and K, K's component along it growing with the
key index), so that a row's running maximum keeps growing from key block to
key block.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "normal_bf16_bits",
    "normal_f16_bits",
    "f16_bits_from_f32",
    "normal_bits",
    "AttnShape",
    "WORKLOADS",
    "make_inputs",
    "MASK_BLOCK",
    "random_block_mask",
    "window_block_mask",
    "block_mask_of",
    "ramp_bits",
]

MASK_BLOCK = 64


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite (normal draws), so no NaN special case is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast: round to nearest
    even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_f16_bits(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """The draws of normal_bf16_bits rounded to binary16 instead."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f16_bits_from_f32(x)


def normal_bits(shape, seed: int, sigma: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """normal_bf16_bits or normal_f16_bits by element type name."""
    if dtype == "bf16":
        return normal_bf16_bits(shape, seed, sigma)
    if dtype == "f16":
        return normal_f16_bits(shape, seed, sigma)
    raise ValueError(f"unknown element type {dtype}")


def normal_bf16_bits(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return bf16_bits_from_f32(x)


def ramp_bits(B: int, Hq: int, Hkv: int, Lq: int, Lk: int, D: int, seed: int, rise: float,
              scale: float, dtype: str = "bf16") -> dict:
    """Q, K, V, dO bits whose scores q_i . k_j * scale are about rise * j / Lk
    plus noise of standard deviation about 0.25.

    u is the unit vector (1, ..., 1) / sqrt(D).  q_i = 4 u + 0.5 n with n a
    normal draw made orthogonal to u; k_j = b_j u + 0.5 n' likewise, with
    b_j = rise * (j / Lk) / (4 * scale).  V and dO are plain normal draws.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    u = np.full(D, 1.0 / math.sqrt(D), dtype=np.float64)

    def noise(shape):
        n = rng.standard_normal(size=shape)
        return n - (n @ u)[..., None] * u

    q = 4.0 * u + 0.5 * noise((B, Hq, Lq, D))
    b = rise * (np.arange(Lk) / Lk) / (4.0 * scale)
    k = b[None, None, :, None] * u + 0.5 * noise((B, Hkv, Lk, D))
    v = rng.standard_normal(size=(B, Hkv, Lk, D))
    do = rng.standard_normal(size=(B, Hq, Lq, D))
    conv = bf16_bits_from_f32 if dtype == "bf16" else f16_bits_from_f32
    return {n: conv(x.astype(np.float32)) for n, x in (("q", q), ("k", k), ("v", v), ("do", do))}


@dataclass(frozen=True)
class AttnShape:
    """One attention problem: sizes, softmax scale, masking and input recipe."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    causal: bool
    sigma: float = 1.0
    seed: int = 0
    scale: float | None = None  # None -> float32(1/sqrt(D))
    backward: bool = True
    q_sigma_mult: float = 1.0  # extra factor on Q only (peaked-softmax variant)
    # block mask recipe: None (dense), ("window", keys, sink_blocks) or
    # ("random", density, seed)
    mask: tuple | None = None
    dtype: str = "bf16"    # element type of q, k, v, dO and the outputs: "bf16" or "f16"
    layout: str = "bhld"   # "bhld" (contiguous [B, H, L, D]) or "bshd" ([B, L, H, D] buffers)

    @property
    def softmax_scale(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)
        return float(np.float32(s))

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


# The workloads the library is measured and checked on.  Seeds follow
# seed = 1000*workload + 100*sub-run; tensor t in (q, k, v, dO) adds t.
WORKLOADS = {
    "tiny": AttnShape("tiny", 1, 2, 1, 128, 128, 64, True, seed=1000),
    "train8k": AttnShape("train8k", 1, 32, 8, 8192, 8192, 128, True, seed=2000),
    "dense4k_d64": AttnShape("dense4k_d64", 2, 16, 16, 4096, 4096, 64, False, sigma=0.5, seed=3000),
    "dense4k_d96": AttnShape("dense4k_d96", 2, 16, 16, 4096, 4096, 96, False, sigma=0.5, seed=3100),
    "d256_8192": AttnShape("d256_8192", 1, 16, 2, 8192, 8192, 256, True, seed=4000, scale=1.0 / 16, backward=False),
    "d256_4064x4096": AttnShape("d256_4064x4096", 1, 16, 2, 4064, 4096, 256, True, seed=4100, scale=1.0 / 16, backward=False),
    "d256_8200": AttnShape("d256_8200", 1, 16, 2, 8200, 8200, 256, True, seed=4200, scale=1.0 / 16, backward=False),
    "long23k": AttnShape("long23k", 1, 32, 8, 23040, 23040, 128, True, seed=5000),
    "d256_train8k": AttnShape("d256_train8k", 1, 16, 2, 8192, 8192, 256, True, seed=6000, scale=1.0 / 16),
    # the 8192-token training shape under a sliding-window block mask: each
    # query block keeps the key blocks that meet the 1024 keys before its
    # last row
    # the 8192-token training shape in IEEE half, and in bf16 with every
    # tensor a [B, L, H, D] buffer (sequence-major) passed as a strided view
    "train8k_f16": AttnShape("train8k_f16", 1, 32, 8, 8192, 8192, 128, True, seed=2200, dtype="f16"),
    "train8k_bshd": AttnShape("train8k_bshd", 1, 32, 8, 8192, 8192, 128, True, seed=2300, layout="bshd"),
    # decode-style: one query row per head against 32768 keys (the head-dim
    # 256 page measures decode at L = 1, S = 32768, 32/8 heads)
    "decode32k_d256": AttnShape("decode32k_d256", 1, 32, 8, 1, 32768, 256, True, seed=7100, scale=1.0 / 16),
    "decode32k_d128": AttnShape("decode32k_d128", 1, 32, 8, 1, 32768, 128, True, seed=7200),
    "train8k_window": AttnShape("train8k_window", 1, 32, 8, 8192, 8192, 128, True, seed=2100,
                                mask=("window", 1024, 0)),
    # the same window plus the first key block kept for every query block (a
    # "sink" column: one key tile seen by every query tile)
    "train8k_sink": AttnShape("train8k_sink", 1, 32, 8, 8192, 8192, 128, True, seed=2100,
                              mask=("window", 1024, 1)),
}


def make_inputs(shape: AttnShape, with_grad: bool | None = None) -> dict:
    """Return uint16 bf16 bit arrays q, k, v (and dO when a backward is wanted)."""
    if with_grad is None:
        with_grad = shape.backward
    s, dt = shape.seed, shape.dtype
    out = {
        "q": normal_bits((shape.B, shape.Hq, shape.Lq, shape.D), s + 0, shape.sigma * shape.q_sigma_mult, dt),
        "k": normal_bits((shape.B, shape.Hkv, shape.Lk, shape.D), s + 1, shape.sigma, dt),
        "v": normal_bits((shape.B, shape.Hkv, shape.Lk, shape.D), s + 2, shape.sigma, dt),
    }
    if with_grad:
        out["do"] = normal_bits((shape.B, shape.Hq, shape.Lq, shape.D), s + 3, shape.sigma, dt)
    return out


def random_block_mask(Lq: int, Lk: int, density: float, seed: int) -> np.ndarray:
    """uint8 [ceil(Lq/64), ceil(Lk/64)], each entry 1 with probability `density`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (-(-Lq // MASK_BLOCK), -(-Lk // MASK_BLOCK))
    return (rng.random(shape) < density).astype(np.uint8)


def window_block_mask(Lq: int, Lk: int, window: int, sink_blocks: int = 0) -> np.ndarray:
    """Local-attention band: query block i keeps key block j when keys
    [64j, 64j+63] meet [last - window + 1, last], last = 64i + 63 + (Lk - Lq)
    (the last key its last row may see under the bottom-right diagonal);
    the first `sink_blocks` key blocks are always kept."""
    nqb, nkb = -(-Lq // MASK_BLOCK), -(-Lk // MASK_BLOCK)
    i = np.arange(nqb)[:, None]
    j = np.arange(nkb)[None, :]
    last = np.minimum(i * MASK_BLOCK + MASK_BLOCK - 1, Lq - 1) + (Lk - Lq)
    lo = last - window + 1
    keep = (j * MASK_BLOCK + MASK_BLOCK - 1 >= lo) & (j * MASK_BLOCK <= last)
    keep |= j < sink_blocks
    return keep.astype(np.uint8)


def block_mask_of(shape: AttnShape):
    """The workload's block mask (uint8 [ceil(Lq/64), ceil(Lk/64)]) or None."""
    if shape.mask is None:
        return None
    kind = shape.mask[0]
    if kind == "window":
        return window_block_mask(shape.Lq, shape.Lk, shape.mask[1], shape.mask[2])
    if kind == "random":
        return random_block_mask(shape.Lq, shape.Lk, shape.mask[1], shape.mask[2])
    raise ValueError(f"unknown mask recipe {shape.mask}")
