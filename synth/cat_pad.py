"""Seeded inputs for the fused cat + pad of causal Conv3D caches.

The pages measure the op on the eight activation shapes of Cosmos3's VAE
decode without listing them; these synthetic shapes stand in for them: a
causal video decoder (kernel 3 in time and space, so spatial pads of 1 and a
time-left pad of 2 that the cached frames fill) from a 88x160 latent to
704x1280 frames, bf16.  Only builds inputs; holds none of the op.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .workloads import _normal_bf16


@dataclass(frozen=True)
class CatPadCase:
    name: str
    b: int
    c: int
    t: int
    h: int
    w: int
    cache_frames: int
    padding: tuple          # (w_left, w_right, h_left, h_right, t_left, t_right)


CAT_PAD_CASES = [
    CatPadCase("latent_in", 1, 16, 2, 88, 160, 2, (1, 1, 1, 1, 0, 0)),
    CatPadCase("mid_512", 1, 512, 2, 88, 160, 2, (1, 1, 1, 1, 0, 0)),
    CatPadCase("mid_512_first", 1, 512, 2, 88, 160, 0, (1, 1, 1, 1, 2, 0)),
    CatPadCase("up1_512", 1, 512, 4, 176, 320, 2, (1, 1, 1, 1, 0, 0)),
    CatPadCase("up2_256", 1, 256, 8, 352, 640, 2, (1, 1, 1, 1, 0, 0)),
    CatPadCase("up2_256_partial", 1, 256, 8, 352, 640, 1, (1, 1, 1, 1, 1, 0)),
    CatPadCase("up3_128", 1, 128, 8, 704, 1280, 2, (1, 1, 1, 1, 0, 0)),
    CatPadCase("up3_128_first", 1, 128, 8, 704, 1280, 0, (1, 1, 1, 1, 2, 0)),
]


def make_cat_pad_inputs(case: CatPadCase, seed: int = 900) -> dict:
    """x [B, C, T, H, W] and cache [B, C, Tc, H, W] as uint16 bf16 bit arrays."""
    x = _normal_bf16(seed, (case.b, case.c, case.t, case.h, case.w))
    cache = _normal_bf16(seed + 1, (case.b, case.c, case.cache_frames, case.h, case.w))
    return {"x": x, "cache": cache, "padding": case.padding}
