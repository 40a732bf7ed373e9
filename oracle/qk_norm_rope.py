"""Plain float64 CPU oracle for the per-head Q/K RMSNorm + rotary embedding
that produces the attention inputs.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the HIP path.

What it computes, per token t and head h of q ([T, Hq, D]) and of k
([T, Hkv, D]), written from the vLLM-Omni diffusion performance-patterns
guide, section "Q/K RMSNorm + RoPE", and the Cosmos3 attention snippet of
sglang PR #26973's review (norm of q and k over head_dim, then rotary, then
attention):

    y   = x / sqrt(mean_d(x_d^2) + eps) * w            (RMSNorm over head_dim,
                                                          weight w per channel)
    out = rotate(y) on the first rotary_dim channels; channels at or past
          rotary_dim pass through ("partial rotary": rotated prefix, pass-through
          suffix)

The rotation takes pair i (0 <= i < rotary_dim / 2) of channels (a, b) and
angle tables cos_i = table[t, i], sin_i = table[t, rotary_dim/2 + i] (the
guide's non-interleaved ``[cos | sin]`` table, one row per token):

    out_a = y_a cos_i - y_b sin_i
    out_b = y_b cos_i + y_a sin_i

with the pairing given by the layout flag of the guide's rotary embedding:
interleaved (GPT-J style, is_neox_style=False): (a, b) = (2i, 2i+1);
half-split (NeoX style, is_neox_style=True):    (a, b) = (i, i + rotary_dim/2).

Readings where the pages are silent (also listed in the design notes):
* the rotation direction is the usual one, (y_a + j y_b) * exp(j angle);
* weights and the table are float32 inputs; q and k are bf16 and the result is
  rounded to bf16 once, at the end (this oracle returns it unrounded);
* the table row of a token is its row in the packed tensor (q and k share it).

Every function below is pinned by ``tests/test_oracle_norm_rope.py``.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (float64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_pairs(rotary_dim: int, interleaved: bool) -> list[tuple[int, int, int]]:
    """(pair index i, channel a, channel b) for every rotated pair."""
    if rotary_dim % 2:
        raise ValueError("rotary_dim must be even")
    half = rotary_dim // 2
    if interleaved:
        return [(i, 2 * i, 2 * i + 1) for i in range(half)]
    return [(i, i, i + half) for i in range(half)]


def apply_rope(y: np.ndarray, table: np.ndarray, rotary_dim: int, interleaved: bool) -> np.ndarray:
    """Rotate y [T, H, D] by the per-token [cos | sin] table [T, rotary_dim]."""
    y = np.asarray(y, dtype=np.float64)
    table = np.asarray(table, dtype=np.float64)
    half = rotary_dim // 2
    out = y.copy()
    for i, a, b in rope_pairs(rotary_dim, interleaved):
        c = table[:, i][:, None]          # [T, 1], shared by every head of the token
        s = table[:, half + i][:, None]
        out[:, :, a] = y[:, :, a] * c - y[:, :, b] * s
        out[:, :, b] = y[:, :, b] * c + y[:, :, a] * s
    return out


def qk_norm_rope(q, k, q_weight, k_weight, table, rotary_dim: int, interleaved: bool, eps: float):
    """(q_out, k_out) in float64: RMSNorm per head, then the rotary embedding."""
    qo = apply_rope(rms_norm(q, q_weight, eps), table, rotary_dim, interleaved)
    ko = apply_rope(rms_norm(k, k_weight, eps), table, rotary_dim, interleaved)
    return qo, ko
