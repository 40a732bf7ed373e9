"""Synthetic, seeded workloads with the shapes of the pages' DiT attention calls.

Every tensor is packed token-major ``[tokens, heads, head_dim]`` in bf16 (kept
here as the raw 16-bit patterns in ``numpy.uint16`` so that the CPU oracle and
the GPU path see exactly the same bits).

Segment metadata (all int32, host side):

* ``cu_q``            B+1 offsets of each batch row's query slots (pad slots included)
* ``cu_prefix``       B+1 offsets into ``k_prefix`` / ``v_prefix``
* ``cu_suffix_real``  2B+1 alternating boundaries ``[s_0, s_0+R_0, s_1, s_1+R_1, ..., end]``:
                      segment 2b is row b's real suffix, segment 2b+1 its tail pad.

Query slots of a row end with that row's suffix slots, so its last ``pad_b``
query slots are pad rows.

Values: q, k_prefix, v_prefix, k_suffix, v_suffix are drawn i.i.d. N(0, 1) in
float32 from ``numpy.random.default_rng(1000 * workload_id + tensor_index)`` in
that order (tensor_index 0..4), then rounded to bf16 with round-to-nearest-even.
Pad slots (of q, k_suffix, v_suffix) are zero-filled by default, following the
zero-pad convention of the unified SP shard helper (sglang PR #30107 review,
key source snippet of ``sp_shard_utils.shard_like``). ``pad_fill="garbage"``
fills them with N(0, 100) draws and ``pad_fill="nan"`` with quiet NaNs, to show
that the pad is never read.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

TENSOR_NAMES = ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")
SUBSET_SEED = 777_000
_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape description of one attention call (no tensors)."""

    wid: int
    name: str
    hq: int
    hkv: int
    d: int
    prefix: Sequence[int]        # P_b per batch row
    suffix_real: Sequence[int]   # R_b per batch row
    suffix_pad: Sequence[int]    # pad_b per batch row
    queries: str                 # "suffix" or "prefix+suffix"

    @property
    def batch(self) -> int:
        return len(self.prefix)

    @property
    def scale(self) -> float:
        return float(self.d) ** -0.5

    def q_slots(self) -> List[int]:
        out = []
        for p, r, pad in zip(self.prefix, self.suffix_real, self.suffix_pad):
            out.append(r + pad + (p if self.queries == "prefix+suffix" else 0))
        return out

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_slots())]).astype(np.int32)

    def cu_prefix(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.prefix)]).astype(np.int32)

    def cu_suffix_real(self) -> np.ndarray:
        bounds = [0]
        for r, pad in zip(self.suffix_real, self.suffix_pad):
            start = bounds[-1]
            bounds.append(start + r)
            bounds.append(start + r + pad)
        return np.asarray(bounds, dtype=np.int32)

    def tokens(self):
        """(query slots, prefix tokens, suffix slots) totals."""
        return (int(self.cu_q()[-1]), int(self.cu_prefix()[-1]),
                int(self.cu_suffix_real()[-1]))

    def pad_query_mask(self) -> np.ndarray:
        """Boolean over query slots: True where the slot is a tail-pad row."""
        cu = self.cu_q()
        mask = np.zeros(int(cu[-1]), dtype=bool)
        for b, pad in enumerate(self.suffix_pad):
            if pad:
                mask[cu[b + 1] - pad:cu[b + 1]] = True
        return mask

    def pad_suffix_mask(self) -> np.ndarray:
        cs = self.cu_suffix_real()
        mask = np.zeros(int(cs[-1]), dtype=bool)
        for b in range(self.batch):
            mask[cs[2 * b + 1]:cs[2 * b + 2]] = True
        return mask


WORKLOADS = {
    1: Workload(1, "tiny", 2, 2, 64, [8], [21], [3], "suffix"),
    2: Workload(2, "qwen_image_joint", 24, 24, 128, [512], [4096], [0], "prefix+suffix"),
    3: Workload(3, "cfg_pair_varlen", 24, 24, 128, [77, 512], [8190, 8190], [2, 2],
                "prefix+suffix"),
    4: Workload(4, "cosmos_video", 32, 32, 128, [1024], [32760], [8], "suffix"),
    5: Workload(5, "long_video_gqa", 40, 8, 128, [256], [75600], [176], "suffix"),
}


def custom_workload(hq, hkv, d, prefix, suffix_real, suffix_pad, queries="suffix",
                    wid=100, name="custom") -> Workload:
    return Workload(wid, name, hq, hkv, d, list(prefix), list(suffix_real),
                    list(suffix_pad), queries)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (NaN -> quiet NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    for s in range(0, xf.size, _CHUNK):
        u = xf[s:s + _CHUNK].view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(xf[s:s + _CHUNK])
        if nan.any():
            r[nan] = 0x7FC0
        of[s:s + _CHUNK] = r
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = rng.standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[s:s + m] = round_to_bf16_bits(x)
    return out.reshape(shape)


def make_inputs(w: Workload, pad_fill: str = "zero", seed_base: Optional[int] = None):
    """Build the five bf16 tensors (as uint16 bit arrays) plus metadata.

    Returns a dict with keys q, k_prefix, v_prefix, k_suffix, v_suffix (uint16
    arrays shaped [T, H, D]), cu_q, cu_prefix, cu_suffix_real (int32), scale.
    """
    base = 1000 * w.wid if seed_base is None else seed_base
    tq, tp, ts = w.tokens()
    shapes = {
        "q": (tq, w.hq, w.d),
        "k_prefix": (tp, w.hkv, w.d),
        "v_prefix": (tp, w.hkv, w.d),
        "k_suffix": (ts, w.hkv, w.d),
        "v_suffix": (ts, w.hkv, w.d),
    }
    out = {}
    for idx, name in enumerate(TENSOR_NAMES):
        out[name] = _normal_bf16(base + idx, shapes[name])
    qpad = w.pad_query_mask()
    spad = w.pad_suffix_mask()
    fills = (("q", qpad), ("k_suffix", spad), ("v_suffix", spad))
    for j, (name, mask) in enumerate(fills):
        n = int(mask.sum())
        if n == 0:
            continue
        if pad_fill == "zero":
            out[name][mask] = 0
        elif pad_fill == "garbage":
            out[name][mask] = _normal_bf16(base + 50 + j, (n,) + shapes[name][1:], sigma=10.0)
        elif pad_fill == "nan":
            out[name][mask] = 0x7FC0
        else:
            raise ValueError(f"unknown pad_fill {pad_fill!r}")
    out["cu_q"] = w.cu_q()
    out["cu_prefix"] = w.cu_prefix()
    out["cu_suffix_real"] = w.cu_suffix_real()
    out["scale"] = w.scale
    return out


def real_query_tokens(w: Workload) -> np.ndarray:
    """Global indices of the real (non-pad) query slots, in order."""
    return np.nonzero(~w.pad_query_mask())[0]


def sample_query_rows(w: Workload, per_head: int, seed: int = SUBSET_SEED) -> np.ndarray:
    """Seeded subset of real query slots per query head: int64 array [Hq, n].

    Head h draws ``per_head`` distinct real rows with
    ``default_rng(seed + h).choice(..., replace=False)`` and sorts them.  If a
    head has fewer real rows than requested, all of them are returned.
    """
    real = real_query_tokens(w)
    n = min(per_head, real.size)
    rows = np.empty((w.hq, n), dtype=np.int64)
    for h in range(w.hq):
        pick = np.random.default_rng(seed + h).choice(real.size, n, replace=False)
        rows[h] = np.sort(real[pick])
    return rows
