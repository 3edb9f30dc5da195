"""Seeded synthetic inputs for the Nystrom self-attention forward.

This module holds random-number draws and storage-format conversion only (bf16
round-to-nearest-even of the drawn values); it holds none of the attention
arithmetic. Both the fp64 oracle (in tests and the CPU baseline) and the HIP path
receive exactly the arrays produced here: the bf16 configurations hand the same bits
to the GPU (as raw uint16) and, upcast exactly, to the oracle.

The workloads stand in for the GLUE/IMDB/LRA runs that the Nystromformer page reports
(abstract; main findings), which need datasets and trained weights that are not
available: Q, K, V are iid Gaussian per head, the depthwise-convolution weights are a
seeded uniform draw rescaled per head. Shapes are the five workload configurations
below.

Draw order for one input set: Q, then K, then V (fp32 standard normal, scaled), then
the conv weights; generator ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    n: int
    d: int
    m: int
    conv_width: int = 33
    pinv_iters: int = 6
    dtype: str = BF16
    qk_std: float = 1.0
    v_std: float = 1.0
    seed: int = 0

    @property
    def seg_len(self) -> int:
        return self.n // self.m

    @property
    def bh(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        return self.B * self.n

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workload shapes. "N(0,2)" for the very-long case is read as variance 2.
CONFIGS = {
    "tiny": Config("tiny", 1, 1, 64, 32, 8, dtype=F32, seed=1001),
    "bert": Config("bert", 32, 12, 512, 64, 64, seed=1002),
    "long": Config("long", 16, 8, 4096, 64, 64, seed=1003),
    "large_m": Config("large_m", 4, 8, 16384, 64, 256, seed=1004),
    "very_long": Config("very_long", 2, 16, 65536, 128, 128, qk_std=float(np.sqrt(2.0)),
                        seed=1005),
}
CONFIG_ORDER = ["tiny", "bert", "long", "large_m", "very_long"]
METRIC_CONFIG = "long"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs cannot overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """One seeded input set.

    ``q, k, v``: float64 copies of the exact values the device sees, [B, H, n, d].
    ``q_dev, k_dev, v_dev``: the device payload (uint16 bf16 bits, or float32).
    ``w``: float32 conv weights [H, W] (the same values for device and oracle).
    """
    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray
    q_dev: np.ndarray
    k_dev: np.ndarray
    v_dev: np.ndarray


def _quantize(x: np.ndarray, dtype: str):
    x = x.astype(np.float32)
    if dtype == BF16:
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == F32:
        return x, x.astype(np.float64)
    raise ValueError(dtype)


def conv_weights(rng: np.random.Generator, H: int, W: int) -> np.ndarray:
    """U(-1/sqrt(W), +1/sqrt(W)) per tap, each head rescaled to L2 norm 0.5."""
    w = rng.uniform(-1.0 / np.sqrt(W), 1.0 / np.sqrt(W), size=(H, W))
    w = 0.5 * w / np.linalg.norm(w, axis=1, keepdims=True)
    return w.astype(np.float32)


def _assemble(cfg: Config, q, k, v, w) -> Inputs:
    qd, q64 = _quantize(q, cfg.dtype)
    kd, k64 = _quantize(k, cfg.dtype)
    vd, v64 = _quantize(v, cfg.dtype)
    return Inputs(cfg, q64, k64, v64, np.ascontiguousarray(w, dtype=np.float32), qd, kd, vd)


def make_inputs(cfg: Config, seed: int | None = None, family: str = "iid") -> Inputs:
    """Draw one input set. ``family`` selects a structure:

    * ``iid``: Q, K ~ N(0, qk_std^2), V ~ N(0, v_std^2).
    * ``clustered``: each segment's tokens share a centre c ~ N(0, 2^2) per segment
      plus N(0, 1) noise, for Q and for K; V iid. The landmark part of the output
      then dominates the mean-of-V part.
    * ``block_sep``: Q = K, every token of segment j equals c_j = r * e_j with
      r = sqrt(30 sqrt(d)), so the landmark logits are 30 on the diagonal and 0 off
      it (needs m <= d). V iid.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, H, n, d, m = cfg.B, cfg.H, cfg.n, cfg.d, cfg.m
    shape = (B, H, n, d)
    if family == "iid":
        q = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg.qk_std)
        k = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg.qk_std)
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg.v_std)
    elif family == "clustered":
        l = n // m
        cq = rng.standard_normal((B, H, m, d), dtype=np.float32) * np.float32(2.0)
        ck = rng.standard_normal((B, H, m, d), dtype=np.float32) * np.float32(2.0)
        q = np.repeat(cq, l, axis=2) + rng.standard_normal(shape, dtype=np.float32)
        k = np.repeat(ck, l, axis=2) + rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
    elif family == "block_sep":
        if m > d:
            raise ValueError("block_sep needs m <= d")
        l = n // m
        r = np.float32(np.sqrt(30.0 * np.sqrt(d)))
        c = np.zeros((m, d), dtype=np.float32)
        c[np.arange(m), np.arange(m)] = r
        q = np.broadcast_to(np.repeat(c, l, axis=0), shape).copy()
        k = q.copy()
        v = rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError(family)
    w = conv_weights(rng, H, cfg.conv_width)
    return _assemble(cfg, q, k, v, w)


def make_well_conditioned_square(n: int, d: int, seed: int, scale: float = 0.5,
                                 dtype: str = F32, B: int = 1, H: int = 1,
                                 conv_width: int = 33, tied: bool = False) -> Inputs:
    """Inputs for the m = n case (one token per segment). With ``tied`` K = Q, so the
    logits are largest on the diagonal and the n x n softmax kernel stays close to a
    scaled identity (small condition number)."""
    cfg = Config(f"square_n{n}", B, H, n, d, n, conv_width=conv_width, dtype=dtype,
                 seed=seed)
    rng = np.random.default_rng(seed)
    shape = (B, H, n, d)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if tied:
        k = q.copy()
    v = rng.standard_normal(shape, dtype=np.float32)
    w = conv_weights(rng, H, conv_width)
    return _assemble(cfg, q, k, v, w)


def ragged_lengths(cfg: Config, seed: int) -> list:
    """Valid lengths of a padded batch: one seeded uniform draw per batch element in
    [max(m, n // 2), n] (a length mix like a bucketed batch of real sequences), with
    the first element at full length."""
    rng = np.random.default_rng(seed + 7919)
    lo = max(cfg.m, cfg.n // 2)
    lens = [int(x) for x in rng.integers(lo, cfg.n + 1, size=cfg.B)]
    lens[0] = cfg.n
    return lens


@dataclass
class LayerInputs:
    """Seeded inputs of the projected layer: x [B, n, D], w_qkv [3 H d, D], w_o [D, H d]
    as bf16 bit patterns (``*_dev``) and their exact float64 values, plus conv weights
    [H, W] fp32."""
    cfg: Config
    D: int
    x: np.ndarray
    w_qkv: np.ndarray
    w_o: np.ndarray
    w: np.ndarray
    x_dev: np.ndarray
    w_qkv_dev: np.ndarray
    w_o_dev: np.ndarray


def make_layer_inputs(cfg: Config, D: int | None = None, seed: int | None = None) -> LayerInputs:
    """x ~ N(0, 1); weights ~ N(0, 1/fan_in) (Q, K, V and the output then have unit
    variance per feature, like the core's own iid inputs); conv weights as
    ``conv_weights``. D defaults to H d. Draw order: x, w_qkv, w_o, conv weights;
    generator ``numpy.random.default_rng(seed + 104729)``."""
    D = cfg.H * cfg.d if D is None else D
    HD = cfg.H * cfg.d
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 104729)
    x = rng.standard_normal((cfg.B, cfg.n, D), dtype=np.float32)
    wq = rng.standard_normal((3 * HD, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    wo = rng.standard_normal((D, HD), dtype=np.float32) * np.float32(1.0 / np.sqrt(HD))
    w = conv_weights(rng, cfg.H, cfg.conv_width)
    (xd, x64), (wqd, wq64), (wod, wo64) = (_quantize(a, BF16) for a in (x, wq, wo))
    return LayerInputs(cfg, D, x64, wq64, wo64, w, xd, wqd, wod)
