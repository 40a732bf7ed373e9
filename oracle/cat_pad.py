"""Plain CPU oracle for the fused cat + pad + zero-fill of causal Conv3D
feature caches.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the library.

Written from sglang PR #29281's review (Cosmos3 VAE decode): the op takes the
current activations x, the cached frames of the previous chunk cache_x and a
padding list, and does in one pass what was a concatenation of the cache and
x along time followed by a padding with zeros
(``fused_causal_conv3d_cat_pad(x, cache_x, padding)``; the kernel performs
cat + pad + zero-fill at once; the padding list follows the usual order of a
5-D pad, last dimension first, and the page notes the time-right pad is 0 in
the supported pattern).

    out = zero_pad(concat([cache_x, x], axis=time), padding)
    padding = (w_left, w_right, h_left, h_right, t_left, t_right)

Readings (also listed in the design notes):
* tensors are [B, C, T, H, W], contiguous; cache_x may have zero frames;
* ``padding`` applies to the concatenation (a caller that pads for a causal
  kernel has already taken the cached frames off the time-left pad);
* pads are non-negative (no cropping); the op is pure data movement, so the
  result is bit-exact, zeros included (+0.0).

Pinned by ``tests/test_oracle_cat_pad.py``.
"""
from __future__ import annotations

import numpy as np


def out_shape(x_shape, cache_frames: int, padding) -> tuple:
    b, c, t, h, w = x_shape
    wl, wr, hl, hr, tl, tr = padding
    return (b, c, cache_frames + t + tl + tr, h + hl + hr, w + wl + wr)


def cat_pad(x: np.ndarray, cache_x, padding) -> np.ndarray:
    """Concatenate cache_x and x along time, then zero-pad (same dtype)."""
    if any(p < 0 for p in padding) or len(padding) != 6:
        raise ValueError("padding is six non-negative pads")
    wl, wr, hl, hr, tl, tr = padding
    cat = x if cache_x is None or cache_x.shape[2] == 0 else np.concatenate([cache_x, x], axis=2)
    return np.pad(cat, ((0, 0), (0, 0), (tl, tr), (hl, hr), (wl, wr)), mode="constant", constant_values=0)
