"""Pins for the fp64 oracle: checks against things the pages and the
mathematics fix, none of which re-runs the oracle's own formula.

* brute force with Python loops (math.fsum / math.exp, no max shift) on tiny
  inputs, with K/V gathered from the workload's per-row lengths rather than
  from the offset arrays;
* torch's float64 scaled_dot_product_attention on explicitly concatenated K/V;
* split == concat, pad-content invariance, GQA == repeated K/V, key-order
  invariance (non-causal), row sums, closed forms, the LSE merge identity;
* the unmasked-pad bug visibly differs (sglang PR #30107 review, motivation);
* hand-derived integer bookkeeping of the five workloads;
* planted mistakes in the oracle are caught by at least one pin.
"""

import importlib
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

fp64 = importlib.import_module("oracle.fp64")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY_CASES = [
    # (hq, hkv, d, prefix, suffix_real, suffix_pad, queries)
    (2, 2, 64, [8], [21], [3], "suffix"),                        # workload 1
    (4, 2, 8, [3, 0, 5], [7, 4, 0], [2, 1, 3], "prefix+suffix"),
    (3, 1, 4, [2, 6], [9, 1], [0, 4], "suffix"),
    (2, 1, 8, [0, 2, 4], [5, 0, 3], [1, 3, 0], "suffix"),          # an all-pad row
]


def _args(x):
    return [x[k] for k in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix",
                           "cu_q", "cu_prefix", "cu_suffix_real")]


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _case(i, pad_fill="garbage", seed=None):
    hq, hkv, d, p, r, pad, qm = TINY_CASES[i]
    w = synth.custom_workload(hq, hkv, d, p, r, pad, qm, wid=300 + i)
    return w, synth.make_inputs(w, pad_fill=pad_fill, seed_base=seed)


def brute_force(w, x, scale=None, keep_pad=False):
    """Definition written out with Python loops over the workload's own row
    lengths.  Returns {(token, head): (out list, lse)} for real query slots."""
    scale = w.scale if scale is None else scale
    q, kp, vp, ks, vs = (_f64(x[n]) for n in synth.TENSOR_NAMES)
    res = {}
    q_off = p_off = s_off = 0
    for b in range(w.batch):
        P, R, pad = w.prefix[b], w.suffix_real[b], w.suffix_pad[b]
        lq = R + pad + (P if w.queries == "prefix+suffix" else 0)
        nq = lq - pad
        nsuf = R + (pad if keep_pad else 0)
        for h in range(w.hq):
            hk = (h * w.hkv) // w.hq
            keys = [kp[p_off + j, hk] for j in range(P)] + [ks[s_off + j, hk] for j in range(nsuf)]
            vals = [vp[p_off + j, hk] for j in range(P)] + [vs[s_off + j, hk] for j in range(nsuf)]
            for i in range(nq):
                t = q_off + i
                s = [scale * math.fsum(float(q[t, h, e]) * float(kk[e]) for e in range(w.d))
                     for kk in keys]
                ex = [math.exp(v) for v in s]
                z = math.fsum(ex)
                o = [math.fsum(ex[j] * float(vals[j][e]) for j in range(len(keys))) / z
                     for e in range(w.d)]
                res[(t, h)] = (o, math.log(z))
        q_off += lq
        p_off += P
        s_off += R + pad
    return res


def _check_against_brute(w, x, out, lse, keep_pad=False, tol=1e-12):
    ref = brute_force(w, x, keep_pad=keep_pad)
    pad = w.pad_query_mask()
    for (t, h), (o, l) in ref.items():
        o = np.asarray(o)
        if not np.all(np.abs(out[t, h] - o) <= tol * np.maximum(1.0, np.abs(o))):
            return False
        if abs(lse[h, t] - l) > tol * max(1.0, abs(l)):
            return False
    for t in np.nonzero(pad)[0]:
        if np.any(out[t] != 0.0) or np.any(lse[:, t] != -np.inf):
            return False
    return len(ref) == int((~pad).sum()) * w.hq


@pytest.mark.parametrize("i", range(len(TINY_CASES)))
def test_brute_force_tiny(i):
    w, x = _case(i)
    out, lse = oracle.attention(*_args(x), x["scale"])
    assert _check_against_brute(w, x, out, lse)


def test_brute_force_keep_pad_variant():
    w, x = _case(0, pad_fill="zero")
    out, lse = oracle.attention(*_args(x), x["scale"], keep_pad=True)
    assert _check_against_brute(w, x, out, lse, keep_pad=True)


@pytest.mark.parametrize("i", range(len(TINY_CASES)))
def test_sdpa_float64(i):
    """Dense SDPA (torch, CPU, float64) on K/V concatenated with torch.cat."""
    w, x = _case(i)
    out, _ = oracle.attention(*_args(x), x["scale"])
    q, kp, vp, ks, vs = (torch.from_numpy(_f64(x[n])) for n in synth.TENSOR_NAMES)
    q_off = p_off = s_off = 0
    for b in range(w.batch):
        P, R, pad = w.prefix[b], w.suffix_real[b], w.suffix_pad[b]
        lq = R + pad + (P if w.queries == "prefix+suffix" else 0)
        nq = lq - pad
        g = w.hq // w.hkv
        if nq:
            k = torch.cat([kp[p_off:p_off + P], ks[s_off:s_off + R]], dim=0)
            v = torch.cat([vp[p_off:p_off + P], vs[s_off:s_off + R]], dim=0)
            k = k.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
            v = v.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
            qq = q[q_off:q_off + nq].permute(1, 0, 2).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq[None], k[None], v[None], scale=w.scale)[0].permute(1, 0, 2).numpy()
            np.testing.assert_allclose(out[q_off:q_off + nq], ref, rtol=1e-12, atol=1e-13)
        q_off += lq
        p_off += P
        s_off += R + pad


def test_split_equals_concat():
    """Prefix+suffix given separately == the same keys given as one suffix
    (sglang PR #26973 review: the non-SP branches concatenate then attend)."""
    w, x = _case(1)
    out, lse = oracle.attention(*_args(x), x["scale"])
    # Rebuild every row with an empty prefix and suffix = [prefix | real | pad].
    q_off, p_off, s_off = 0, 0, 0
    new_ks, new_vs, cu_s = [], [], [0]
    for b in range(w.batch):
        P, R, pad = w.prefix[b], w.suffix_real[b], w.suffix_pad[b]
        for src_p, src_s, dst in ((x["k_prefix"], x["k_suffix"], new_ks),
                                  (x["v_prefix"], x["v_suffix"], new_vs)):
            dst.append(np.concatenate([src_p[p_off:p_off + P], src_s[s_off:s_off + R + pad]]))
        cu_s += [cu_s[-1] + P + R, cu_s[-1] + P + R + pad]
        p_off += P
        s_off += R + pad
    kp0 = x["k_prefix"][:0]
    out2, lse2 = oracle.attention(x["q"], kp0, kp0, np.concatenate(new_ks), np.concatenate(new_vs),
                                  x["cu_q"], np.zeros(w.batch + 1, np.int32),
                                  np.asarray(cu_s, np.int32), x["scale"])
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("fill", ["garbage", "nan"])
def test_pad_content_invariance(fill):
    w, xz = _case(1, pad_fill="zero")
    _, xg = _case(1, pad_fill=fill)
    a, la = oracle.attention(*_args(xz), xz["scale"])
    b, lb = oracle.attention(*_args(xg), xg["scale"])
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    pad = w.pad_query_mask()
    assert np.all(a[pad] == 0.0) and np.all(la[:, pad] == -np.inf)


def test_row_sums_and_constant_values():
    w, x = _case(1)
    out, lse = oracle.attention(*_args(x), x["scale"])
    q, kp, _, ks, _ = (_f64(x[n]) for n in synth.TENSOR_NAMES)
    # sum_j exp(s_ij - LSE_i) == 1, scores re-derived with fsum loops
    t, h = 2, 3                       # row 0, real query 2, head 3 -> kv head 1
    keys = [kp[j, 1] for j in range(3)] + [ks[j, 1] for j in range(7)]
    s = [w.scale * math.fsum(float(a) * float(c) for a, c in zip(q[t, h], k)) for k in keys]
    assert abs(math.fsum(math.exp(v - lse[h, t]) for v in s) - 1.0) < 1e-14
    # V == c everywhere -> out == c
    c = 0.8125
    for name in ("v_prefix", "v_suffix"):
        x[name] = np.full_like(x[name], synth.round_to_bf16_bits(np.float32([c]))[0])
    out_c, _ = oracle.attention(*_args(x), x["scale"])
    real = ~w.pad_query_mask()
    assert np.max(np.abs(out_c[real] - c)) < 1e-14


def test_closed_forms():
    w, x = _case(1)
    vp, vs = _f64(x["v_prefix"]), _f64(x["v_suffix"])
    # scale = 0: uniform weights -> mean of the row's real V rows, LSE = ln Nk
    out, lse = oracle.attention(*_args(x), 0.0)
    row0 = np.concatenate([vp[0:3, 0], vs[0:7, 0]])          # row 0, kv head 0
    np.testing.assert_allclose(out[0, 0], row0.mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - math.log(10)) < 1e-14
    # constant K: same uniform weights
    x2 = dict(x)
    for name in ("k_prefix", "k_suffix"):
        x2[name] = np.full_like(x[name], synth.round_to_bf16_bits(np.float32([0.5]))[0])
    out2, _ = oracle.attention(*_args(x2), x["scale"])
    np.testing.assert_allclose(out2[0, 0], row0.mean(axis=0), rtol=0, atol=1e-14)
    # a single key: out = v_0, LSE = s_00
    w1 = synth.custom_workload(2, 1, 8, [0], [1], [2], "suffix", wid=350)
    x1 = synth.make_inputs(w1, pad_fill="garbage")
    o1, l1 = oracle.attention(*_args(x1), w1.scale)
    q1, k1, v1 = _f64(x1["q"]), _f64(x1["k_suffix"]), _f64(x1["v_suffix"])
    assert np.array_equal(o1[0, 1], v1[0, 0])
    s00 = w1.scale * math.fsum(float(a) * float(b) for a, b in zip(q1[0, 1], k1[0, 0]))
    assert abs(l1[1, 0] - s00) < 1e-15


def test_gqa_equals_repeated_kv():
    w, x = _case(1)       # Hq=4, Hkv=2
    out, lse = oracle.attention(*_args(x), x["scale"])
    g = w.hq // w.hkv
    x2 = dict(x)
    for name in ("k_prefix", "v_prefix", "k_suffix", "v_suffix"):
        x2[name] = np.repeat(x[name], g, axis=1)              # head order 0,0,1,1
    out2, lse2 = oracle.attention(*_args(x2), x["scale"])
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_key_order_invariance():
    """Non-causal: putting the suffix keys before the prefix keys changes
    nothing but rounding."""
    w = synth.custom_workload(3, 3, 16, [6], [11], [2], "suffix", wid=360)
    x = synth.make_inputs(w, pad_fill="garbage")
    out, lse = oracle.attention(*_args(x), w.scale)
    # swapped roles: prefix <- real suffix, suffix <- prefix (+ same pad block)
    new_kp, new_vp = x["k_suffix"][:11], x["v_suffix"][:11]
    new_ks = np.concatenate([x["k_prefix"], x["k_suffix"][11:]])
    new_vs = np.concatenate([x["v_prefix"], x["v_suffix"][11:]])
    out2, lse2 = oracle.attention(x["q"], new_kp, new_vp, new_ks, new_vs, x["cu_q"],
                                  np.asarray([0, 11], np.int32), np.asarray([0, 6, 8], np.int32),
                                  w.scale)
    real = ~w.pad_query_mask()
    assert np.max(np.abs(out - out2)) < 1e-13
    assert np.max(np.abs(lse[:, real] - lse2[:, real])) < 1e-13
    assert np.array_equal(lse[:, ~real], lse2[:, ~real])


def test_lse_merge_of_prefix_and_suffix_parts():
    """Attention over the prefix keys alone and over the suffix keys alone,
    merged through their LSE, equals attention over both key sets (the merge
    a ring/split-K schedule would apply to the LSE output)."""
    w, x = _case(2)                         # every row has P > 0 and R > 0
    out, lse = oracle.attention(*_args(x), x["scale"])
    # prefix only: the suffix keeps each row's pad slots but no real keys
    cs_pad = [0]
    for pad in w.suffix_pad:
        cs_pad += [cs_pad[-1], cs_pad[-1] + pad]
    zpad = np.zeros((cs_pad[-1],) + x["k_suffix"].shape[1:], np.uint16)
    o_p, l_p = oracle.attention(x["q"], x["k_prefix"], x["v_prefix"], zpad, zpad, x["cu_q"],
                                x["cu_prefix"], np.asarray(cs_pad, np.int32), x["scale"])
    # suffix only: empty prefix
    o_s, l_s = oracle.attention(x["q"], x["k_prefix"][:0], x["v_prefix"][:0], x["k_suffix"],
                                x["v_suffix"], x["cu_q"], np.zeros(w.batch + 1, np.int32),
                                x["cu_suffix_real"], x["scale"])
    real = ~w.pad_query_mask()
    m_out, m_lse = oracle.lse_merge([o_p, o_s], [l_p.T, l_s.T])
    np.testing.assert_allclose(m_out[real], out[real], rtol=0, atol=1e-13)
    np.testing.assert_allclose(m_lse[real], lse.T[real], rtol=0, atol=1e-13)


def test_unmasked_pad_visibly_differs():
    meta = json.load(open(os.path.join(GOLDEN, "unmasked_pad_mae.json")))
    w = synth.WORKLOADS[1]
    x = synth.make_inputs(w)
    a, _ = oracle.attention(*_args(x), x["scale"])
    b, _ = oracle.attention(*_args(x), x["scale"], keep_pad=True)
    real = ~w.pad_query_mask()
    assert np.abs(a[real] - b[real]).mean() > 5e-3      # >= 5x the mean-abs tolerance
    lo, hi = meta["check_band"]
    maes = []
    for s in range(8):
        w2 = synth.custom_workload(2, 2, 64, [0], [15], [1], "suffix", wid=400 + s)
        x2 = synth.make_inputs(w2)
        a2, _ = oracle.attention(*_args(x2), w2.scale)
        b2, _ = oracle.attention(*_args(x2), w2.scale, keep_pad=True)
        r2 = ~w2.pad_query_mask()
        maes.append(np.abs(a2[r2] - b2[r2]).mean())
    assert lo < float(np.mean(maes)) < hi


def test_integer_bookkeeping_golden():
    gold = json.load(open(os.path.join(GOLDEN, "segments.json")))["workloads"]
    for wid, g in gold.items():
        w = synth.WORKLOADS[int(wid)]
        assert list(w.cu_q()) == g["cu_q"]
        assert list(w.cu_prefix()) == g["cu_prefix"]
        assert list(w.cu_suffix_real()) == g["cu_suffix_real"]
        rows = oracle.decode_segments(g["cu_q"], g["cu_prefix"], g["cu_suffix_real"])
        assert [[r.q_start, r.q_slots, r.q_real, r.p_start, r.p_len, r.s_start, r.s_real,
                 r.s_pad, r.keys] for r in rows] == g["rows"]
        assert oracle.valid_flops(rows, g["hq"], g["d"]) == g["valid_flops"]


@pytest.mark.parametrize("cu", [
    ([1, 4], [0, 2], [0, 1, 3]),            # cu_q[0] != 0
    ([0, 4], [0, 2], [0, 3, 1]),            # non-monotone
    ([0, 4], [0, 2], [0, 1]),               # wrong count
    ([0, 2], [0, 2], [0, 1, 4]),            # pad 3 > 2 query slots
    ([0, 3], [0, 0], [0, 0, 1]),            # real queries, no keys
])
def test_decode_rejects_bad_segments(cu):
    with pytest.raises(ValueError):
        oracle.decode_segments(*cu)


def test_subset_rows_match_full():
    w, x = _case(1)
    out, lse = oracle.attention(*_args(x), x["scale"])
    rows = synth.sample_query_rows(w, 5)
    o2, l2 = oracle.attention_rows(*_args(x), x["scale"], rows)
    for h in range(w.hq):
        assert np.array_equal(o2[h], out[rows[h], h]) and np.array_equal(l2[h], lse[h, rows[h]])


# ---------------------------------------------------------------- planted mistakes

def _pins_hold():
    """A quick run of the pins above; False as soon as one fails."""
    try:
        for i in range(len(TINY_CASES)):
            w, x = _case(i)
            out, lse = oracle.attention(*_args(x), x["scale"])
            if not _check_against_brute(w, x, out, lse):
                return False
        test_pad_content_invariance("garbage")
        test_row_sums_and_constant_values()
        test_gqa_equals_repeated_kv()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def _mut_no_scale(qr, k, v, scale):
    return _orig_softmax(qr, k, v, 1.0)


def _mut_v_is_k(qr, k, v, scale):
    return _orig_softmax(qr, k, k, scale)


def _mut_no_norm(qr, k, v, scale):
    o, l = _orig_softmax(qr, k, v, scale)
    return o * np.exp(l)[:, None], l


def _mut_lse_log2(qr, k, v, scale):
    o, l = _orig_softmax(qr, k, v, scale)
    return o, l / math.log(2.0)


def _mut_gqa_modulo(h, hq, hkv):
    return h % hkv


def _mut_keep_pad(k_prefix, v_prefix, k_suffix, v_suffix, seg, hk, keep_pad=False):
    return _orig_row_kv(k_prefix, v_prefix, k_suffix, v_suffix, seg, hk, True)


def _mut_suffix_off_by_one(k_prefix, v_prefix, k_suffix, v_suffix, seg, hk, keep_pad=False):
    seg2 = fp64.RowSegments(seg.q_start, seg.q_slots, seg.q_real, seg.p_start, seg.p_len,
                            seg.s_start + 1, seg.s_real, seg.s_pad, seg.keys)
    return _orig_row_kv(k_prefix, v_prefix, k_suffix, v_suffix, seg2, hk, keep_pad)


def _mut_pad_rows_first(cu_q, cu_prefix, cu_suffix_real):
    rows = _orig_decode(cu_q, cu_prefix, cu_suffix_real)
    return [fp64.RowSegments(r.q_start + r.s_pad, r.q_slots, r.q_real, r.p_start, r.p_len,
                             r.s_start, r.s_real, r.s_pad, r.keys) for r in rows]


_orig_softmax = fp64.softmax_attention
_orig_row_kv = fp64.row_kv
_orig_decode = fp64.decode_segments

MUTANTS = [
    ("softmax_attention", _mut_no_scale),
    ("softmax_attention", _mut_v_is_k),
    ("softmax_attention", _mut_no_norm),
    ("softmax_attention", _mut_lse_log2),
    ("kv_head", _mut_gqa_modulo),
    ("row_kv", _mut_keep_pad),
    ("row_kv", _mut_suffix_off_by_one),
    ("decode_segments", _mut_pad_rows_first),
]


def test_pins_hold_on_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(fp64, name, mutant)
    assert not _pins_hold()
