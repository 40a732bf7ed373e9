"""Plain float64 CPU oracle for split prefix/suffix, tail-pad-skipping,
non-causal (bidirectional) attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the HIP path.

What it computes (the plain definition, not the tiled algorithm):

For batch row b, query head h and every real query slot i of that row,

    K_b = concat(k_prefix[row b's prefix], k_suffix[row b's real suffix])   (pad keys dropped)
    V_b = concat(v_prefix[...],            v_suffix[...])
    s_ij = scale * <q_i, k_j>
    out_i = sum_j exp(s_ij - LSE_i) v_j,   LSE_i = ln sum_j exp(s_ij)

and pad query slots get ``out = 0`` and ``LSE = -inf``.

Passages followed:
* K/V arrive as a prefix and a suffix; without sequence parallelism the layer
  concatenates them on the sequence axis (prefix first) and runs plain
  attention (sglang PR #26973 review, core-logic snippet of
  ``forward_with_replicated_kv_prefix`` in the attention layer).
* The tail pad of each row is its own varlen segment that attention skips: it
  never enters the softmax and needs no mask or repacking (sglang PR #30107
  review, implementation breakdown item 4 and the layout-invariant docstring of
  ``sp_shard_utils``).
* Letting zero pad K/V into the softmax biases every real token (same page,
  motivation section): ``keep_pad=True`` reproduces that bug as a negative
  control.
* Attention is non-causal with softmax scale head_dim**-0.5 in BSND layout
  (vLLM-Omni performance-patterns guide, shared attention wiring section); the
  scale is taken as an argument.
* Grouped-query attention: query head h reads kv head h // (Hq / Hkv); Hq must
  be a multiple of Hkv (same guide, USP section on GQA; the per-rank contiguous
  head slices in sglang PR #26973's split path imply this block grouping).

Readings where the pages are silent (also listed in the design notes):
* ``cu_suffix_real`` holds 2B+1 alternating boundaries: segment 2b is row b's
  real suffix, segment 2b+1 its tail pad.
* The last pad_b query slots of row b are its pad rows.
* LSE is the natural log over the scaled scores, stored [Hq, Tq].

Inputs may be float arrays of any precision or bf16 bit patterns held in
``numpy.uint16``; both are widened exactly to float64 before any arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np

QUERY_CHUNK = 512


@dataclasses.dataclass(frozen=True)
class RowSegments:
    """Integer bookkeeping of one batch row (all counts are token counts)."""

    q_start: int      # first query slot of the row
    q_slots: int      # Lq_b: query slots, pad included
    q_real: int       # Nq_b = Lq_b - pad_b
    p_start: int      # first prefix token of the row
    p_len: int        # P_b
    s_start: int      # first suffix slot of the row
    s_real: int       # R_b
    s_pad: int        # pad_b
    keys: int         # Nk_b = P_b + R_b


def widen(x) -> np.ndarray:
    """Exact widening to float64.  uint16 input is read as bf16 bit patterns."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _check_offsets(name: str, cu: np.ndarray) -> None:
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError(f"{name}: needs at least one offset")
    if cu[0] != 0:
        raise ValueError(f"{name}[0] must be 0")
    if np.any(np.diff(cu) < 0):
        raise ValueError(f"{name} must be non-decreasing")


def decode_segments(cu_q, cu_prefix, cu_suffix_real) -> List[RowSegments]:
    """Per-row bookkeeping from the three offset arrays.

    Row b owns query slots cu_q[b]:cu_q[b+1], prefix tokens
    cu_prefix[b]:cu_prefix[b+1], real suffix slots
    cu_suffix_real[2b]:cu_suffix_real[2b+1] and tail-pad slots
    cu_suffix_real[2b+1]:cu_suffix_real[2b+2] -- the pad is a segment of its
    own (sglang PR #30107 review, implementation breakdown item 4).
    """
    cq = np.asarray(cu_q, dtype=np.int64)
    cp = np.asarray(cu_prefix, dtype=np.int64)
    cs = np.asarray(cu_suffix_real, dtype=np.int64)
    for name, cu in (("cu_q", cq), ("cu_prefix", cp), ("cu_suffix_real", cs)):
        _check_offsets(name, cu)
    batch = cq.size - 1
    if cp.size != batch + 1 or cs.size != 2 * batch + 1:
        raise ValueError("offset arrays must have B+1, B+1 and 2B+1 entries")
    rows = []
    for b in range(batch):
        q_slots = int(cq[b + 1] - cq[b])
        s_real = int(cs[2 * b + 1] - cs[2 * b])
        s_pad = int(cs[2 * b + 2] - cs[2 * b + 1])
        p_len = int(cp[b + 1] - cp[b])
        if s_pad > q_slots:
            raise ValueError(f"row {b}: more pad slots than query slots")
        q_real = q_slots - s_pad
        keys = p_len + s_real
        if q_real > 0 and keys == 0:
            raise ValueError(f"row {b}: real queries but no keys")
        rows.append(RowSegments(int(cq[b]), q_slots, q_real, int(cp[b]), p_len,
                                int(cs[2 * b]), s_real, s_pad, keys))
    return rows


def valid_flops(rows: Sequence[RowSegments], hq: int, d: int) -> int:
    """Multiply-add work over valid tokens: sum_b Hq * 4 * D * Nq_b * Nk_b
    (2*D for QK^T and 2*D for PV per query/key pair)."""
    return sum(hq * 4 * d * r.q_real * r.keys for r in rows)


def kv_head(h: int, hq: int, hkv: int) -> int:
    """Block grouping of query heads onto kv heads."""
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def row_kv(k_prefix, v_prefix, k_suffix, v_suffix, seg: RowSegments, hk: int,
           keep_pad: bool = False):
    """Explicitly concatenated K_b, V_b (float64, [Nk, D]) for one row and kv head.

    Prefix rows come first, then the real suffix rows; the tail pad is dropped
    unless ``keep_pad`` (the unmasked-pad bug used as a negative control)."""
    s_end = seg.s_start + seg.s_real + (seg.s_pad if keep_pad else 0)
    k = np.concatenate([widen(k_prefix[seg.p_start:seg.p_start + seg.p_len, hk]),
                        widen(k_suffix[seg.s_start:s_end, hk])], axis=0)
    v = np.concatenate([widen(v_prefix[seg.p_start:seg.p_start + seg.p_len, hk]),
                        widen(v_suffix[seg.s_start:s_end, hk])], axis=0)
    return k, v


def softmax_attention(qr: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Dense softmax(scale * q k^T) v with its natural-log LSE, float64.

    The row max is subtracted before exp; this leaves the result unchanged in
    exact arithmetic and only avoids overflow."""
    s = (qr @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1)
    out = (e @ v) / z[:, None]
    lse = m[:, 0] + np.log(z)
    return out, lse


def attention(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
              cu_suffix_real, scale: float, keep_pad: bool = False):
    """Full oracle: out [Tq, Hq, D] float64 and lse [Hq, Tq] float64.

    ``q`` is [Tq, Hq, D]; the four K/V tensors are [T, Hkv, D].  Pad query rows
    get out = 0 and lse = -inf."""
    tq, hq, d = q.shape
    hkv = k_prefix.shape[1]
    rows = decode_segments(cu_q, cu_prefix, cu_suffix_real)
    out = np.zeros((tq, hq, d), dtype=np.float64)
    lse = np.full((hq, tq), -np.inf, dtype=np.float64)
    for seg in rows:
        if seg.q_real == 0:
            continue
        for h in range(hq):
            k, v = row_kv(k_prefix, v_prefix, k_suffix, v_suffix, seg,
                          kv_head(h, hq, hkv), keep_pad)
            for c0 in range(0, seg.q_real, QUERY_CHUNK):
                c1 = min(seg.q_real, c0 + QUERY_CHUNK)
                t0, t1 = seg.q_start + c0, seg.q_start + c1
                o, l = softmax_attention(widen(q[t0:t1, h]), k, v, scale)
                out[t0:t1, h] = o
                lse[h, t0:t1] = l
    return out, lse


def attention_rows(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                   cu_suffix_real, scale: float, rows_per_head, keep_pad: bool = False,
                   heads=None):
    """Oracle on a chosen set of query slots per head.

    ``rows_per_head`` is an int array [Hq, n] of global query-slot indices.
    Returns out [len(heads), n, D] and lse [len(heads), n] (float64); a pad
    slot yields zeros and -inf like in :func:`attention`."""
    tq, hq, d = q.shape
    hkv = k_prefix.shape[1]
    segs = decode_segments(cu_q, cu_prefix, cu_suffix_real)
    starts = np.asarray([s.q_start for s in segs], dtype=np.int64)
    heads = list(range(hq)) if heads is None else list(heads)
    rows_per_head = np.asarray(rows_per_head, dtype=np.int64)
    n = rows_per_head.shape[1]
    out = np.zeros((len(heads), n, d), dtype=np.float64)
    lse = np.full((len(heads), n), -np.inf, dtype=np.float64)
    for hi, h in enumerate(heads):
        toks = rows_per_head[h]
        owner = np.searchsorted(starts, toks, side="right") - 1
        for b, seg in enumerate(segs):
            sel = np.nonzero((owner == b) & (toks < seg.q_start + seg.q_real))[0]
            if sel.size == 0:
                continue
            k, v = row_kv(k_prefix, v_prefix, k_suffix, v_suffix, seg,
                          kv_head(h, hq, hkv), keep_pad)
            for c0 in range(0, sel.size, QUERY_CHUNK):
                part = sel[c0:c0 + QUERY_CHUNK]
                o, l = softmax_attention(widen(q[toks[part], h]), k, v, scale)
                out[hi, part] = o
                lse[hi, part] = l
    return out, lse


def compare(gpu_out, gpu_lse, ref_out, ref_lse):
    """Error summary in float32 over the given (real) rows: max-abs and
    mean-abs of out, max-abs of lse."""
    go = np.asarray(gpu_out, dtype=np.float32)
    ro = np.asarray(ref_out, dtype=np.float64).astype(np.float32)
    diff = np.abs(go - ro)
    gl = np.asarray(gpu_lse, dtype=np.float32)
    rl = np.asarray(ref_lse, dtype=np.float64).astype(np.float32)
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "mean_abs": float(diff.mean()) if diff.size else 0.0,
        "lse_max_abs": float(np.abs(gl - rl).max()) if gl.size else 0.0,
    }


def lse_merge(parts_out, parts_lse):
    """Combine partial attentions over disjoint key sets by their LSE:
    out = sum_k exp(lse_k - lse) out_k with lse = ln sum_k exp(lse_k)."""
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in parts_lse])
    top = lses.max(axis=0)
    empty = top == -np.inf                 # no keys in any part: out 0, lse -inf
    top = np.where(empty, 0.0, top)
    w = np.exp(lses - top)
    z = w.sum(axis=0)
    zs = np.where(empty, 1.0, z)
    lse = np.where(empty, -np.inf, top + np.log(zs))
    out = sum(wk[..., None] * np.asarray(ok, dtype=np.float64)
              for wk, ok in zip(w, parts_out)) / zs[..., None]
    return out, lse

