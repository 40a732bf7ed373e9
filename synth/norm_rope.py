"""Seeded inputs for the per-head Q/K RMSNorm + rotary step.

Only builds inputs: bf16 q/k tensors, float32 norm weights and the float32
per-token ``[cos | sin]`` table (standard rotary frequencies base^(-2i/r) at
integer positions).  Holds none of the normalisation or rotation arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .workloads import _normal_bf16


@dataclass(frozen=True)
class NormRopeWorkload:
    wid: int
    name: str
    tokens: int
    hq: int
    hkv: int
    d: int
    rotary_dim: int
    interleaved: bool
    eps: float = 1e-6


# Shapes of the attention workloads' q and k (the step runs right before
# attention); the pairing/geometry follows the two contracts the pages name:
# half-split with rotary_dim 96 of head_dim 128, and interleaved pairs.
NORM_ROPE_WORKLOADS = {
    1: NormRopeWorkload(1, "tiny_partial", 37, 4, 2, 64, 48, True),
    2: NormRopeWorkload(2, "qwen_image_joint", 4608, 24, 24, 128, 128, True),
    3: NormRopeWorkload(3, "tiny_halfsplit", 29, 3, 3, 128, 96, False),
    4: NormRopeWorkload(4, "cosmos_video", 32768, 32, 32, 128, 96, False),
    5: NormRopeWorkload(5, "long_video_gqa", 75776, 40, 8, 128, 96, False),
}


def rope_table(positions: np.ndarray, rotary_dim: int, base: float = 10000.0,
               dtype=np.float32) -> np.ndarray:
    """[T, rotary_dim] = [cos(pos * f_i) | sin(pos * f_i)], f_i = base^(-2i/rotary_dim)
    (float32 for the kernel; float64 for checks that need cos^2 + sin^2 = 1)."""
    half = rotary_dim // 2
    f = base ** (-2.0 * np.arange(half, dtype=np.float64) / max(rotary_dim, 1))
    ang = np.asarray(positions, dtype=np.float64)[:, None] * f[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(dtype)


def make_norm_rope_inputs(w: NormRopeWorkload, seed_base: int | None = None) -> dict:
    """q [T, Hq, D], k [T, Hkv, D] (uint16 bf16 bits), q_weight/k_weight [D] and
    table [T, rotary_dim] (float32), plus rotary_dim, interleaved, eps."""
    base = 7000 + 100 * w.wid if seed_base is None else seed_base
    rng = np.random.default_rng(base + 2)
    return {
        "q": _normal_bf16(base, (w.tokens, w.hq, w.d)),
        "k": _normal_bf16(base + 1, (w.tokens, w.hkv, w.d)),
        "q_weight": (1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32),
        "k_weight": (1.0 + 0.1 * rng.standard_normal(w.d)).astype(np.float32),
        "table": rope_table(np.arange(w.tokens), w.rotary_dim),
        "rotary_dim": w.rotary_dim,
        "interleaved": w.interleaved,
        "eps": w.eps,
    }
