"""Pins for the fp64 RMSNorm + rotary oracle (oracle/qk_norm_rope.py): checks
against what the pages and the mathematics fix, none of which re-runs the
oracle's own array formula.

* brute force with Python scalars: math.fsum for the mean square and a complex
  multiply (y_a + j y_b) * (cos + j sin) for each rotated pair, with the
  pairing written from the guide's description of the two layouts;
* the mean square of a unit-weight, eps = 0 result is exactly 1 (rotations
  preserve it): a sum-for-mean slip breaks it;
* zero angle is the identity, a quarter turn maps (a, b) -> (-b, a);
* rotary relative-position property on a standard frequency table;
* half-split equals interleaved after the channel permutation that maps pair
  (i, i + r/2) to (2i, 2i + 1);
* partial rotary leaves channels at or past rotary_dim as the plain RMSNorm;
* scale invariance of the normalisation and linearity in the weight;
* planted mistakes in the oracle are caught by at least one pin.
(vLLM-Omni diffusion performance-patterns guide, section "Q/K RMSNorm + RoPE".)
"""

import importlib
import math

import numpy as np
import pytest

import oracle
import synth

nr = importlib.import_module("oracle.qk_norm_rope")


def _inputs(t, hq, hkv, d, rot, interleaved, eps, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d)) * 3.0
    wq = 1.0 + 0.3 * rng.standard_normal(d)
    wk = 1.0 + 0.3 * rng.standard_normal(d)
    table = synth.rope_table(np.arange(t) * 7 + 3, rot, dtype=np.float64)
    return q, k, wq, wk, table, rot, interleaved, eps


def _brute_row(x, w, cs, rot, interleaved, eps):
    """One head row: RMSNorm with math.fsum, then complex rotation per pair."""
    d = len(x)
    ms = math.fsum(float(v) * float(v) for v in x) / d
    inv = 1.0 / math.sqrt(ms + eps)
    y = [float(x[i]) * inv * float(w[i]) for i in range(d)]
    out = list(y)
    half = rot // 2
    for i in range(half):
        if interleaved:
            a, b = 2 * i, 2 * i + 1          # GPT-J style: even/odd neighbours
        else:
            a, b = i, half + i               # NeoX style: first half with second half
        z = complex(y[a], y[b]) * complex(float(cs[i]), float(cs[half + i]))
        out[a], out[b] = z.real, z.imag
    return out


def _brute(q, wq, table, rot, interleaved, eps):
    t, h, d = q.shape
    out = np.empty((t, h, d))
    for ti in range(t):
        for hi in range(h):
            out[ti, hi] = _brute_row(q[ti, hi], wq, table[ti], rot, interleaved, eps)
    return out


BRUTE_CASES = [
    (5, 3, 1, 16, 16, True, 1e-6),
    (4, 2, 2, 16, 16, False, 1e-6),
    (3, 2, 1, 32, 12, True, 0.25),
    (3, 1, 1, 32, 20, False, 0.25),
    (2, 2, 2, 64, 48, False, 1e-5),
    (2, 1, 1, 8, 0, True, 0.5),
]


def _check_brute(case, seed=11):
    q, k, wq, wk, table, rot, il, eps = _inputs(*case, seed=seed)
    qo, ko = oracle.qk_norm_rope(q, k, wq, wk, table, rot, il, eps)
    ok = np.allclose(qo, _brute(q, wq, table, rot, il, eps), rtol=1e-12, atol=1e-12)
    ok &= np.allclose(ko, _brute(k, wk, table, rot, il, eps), rtol=1e-12, atol=1e-12)
    return bool(ok)


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force(case):
    assert _check_brute(case)


def test_unit_mean_square():
    rng = np.random.default_rng(5)
    for il in (True, False):
        x = rng.standard_normal((6, 3, 32)) * 5.0
        table = synth.rope_table(np.arange(6), 24, dtype=np.float64)
        out, _ = oracle.qk_norm_rope(x, x[:, :1], np.ones(32), np.ones(32), table, 24, il, 0.0)
        ms = (out * out).mean(axis=-1)
        assert np.allclose(ms, 1.0, rtol=0, atol=1e-13)


def test_zero_angle_is_identity_and_quarter_turn():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 2, 16))
    w = 1.0 + rng.random(16)
    plain = np.empty_like(x)
    for ti in range(2):
        for hi in range(2):
            plain[ti, hi] = _brute_row(x[ti, hi], w, np.zeros(0), 0, True, 1e-6)
    ident = np.concatenate([np.ones((2, 8)), np.zeros((2, 8))], axis=1)     # cos 1, sin 0
    quarter = np.concatenate([np.zeros((2, 8)), np.ones((2, 8))], axis=1)   # cos 0, sin 1
    for il in (True, False):
        out, _ = oracle.qk_norm_rope(x, x, w, w, ident, 16, il, 1e-6)
        assert np.allclose(out, plain, rtol=0, atol=1e-14)
        out, _ = oracle.qk_norm_rope(x, x, w, w, quarter, 16, il, 1e-6)
        a = np.arange(0, 16, 2) if il else np.arange(8)
        b = a + 1 if il else a + 8
        assert np.allclose(out[..., a], -plain[..., b], atol=1e-14)
        assert np.allclose(out[..., b], plain[..., a], atol=1e-14)


def test_relative_position():
    """<rope(q, m), rope(k, n)> depends on m - n only (unit weights, standard table)."""
    rng = np.random.default_rng(8)
    qv = rng.standard_normal(32)
    kv = rng.standard_normal(32)
    for il in (True, False):
        def dot(m, n):
            table = synth.rope_table(np.array([m, n]), 32, dtype=np.float64)
            x = np.stack([qv, kv])[:, None, :]
            out, _ = oracle.qk_norm_rope(x, x, np.ones(32), np.ones(32), table, 32, il, 0.0)
            return float(out[0, 0] @ out[1, 0])
        assert abs(dot(5, 2) - dot(105, 102)) < 1e-9
        assert abs(dot(5, 2) - dot(2, 5)) > 1e-6          # but it is not symmetric in general


def test_halfsplit_is_permuted_interleaved():
    rng = np.random.default_rng(9)
    d, rot = 32, 20
    x = rng.standard_normal((3, 2, d))
    w = 1.0 + 0.2 * rng.standard_normal(d)
    table = synth.rope_table(np.arange(3) + 1, rot, dtype=np.float64)
    perm = np.arange(d)                                    # interleaved channel -> half-split channel
    perm[0:rot:2] = np.arange(rot // 2)
    perm[1:rot:2] = np.arange(rot // 2) + rot // 2
    hs, _ = oracle.qk_norm_rope(x, x, w, w, table, rot, False, 1e-6)
    il, _ = oracle.qk_norm_rope(x[..., perm], x[..., perm], w[perm], w[perm], table, rot, True, 1e-6)
    assert np.allclose(il, hs[..., perm], rtol=0, atol=1e-14)


def test_partial_rotary_passthrough():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((4, 3, 64))
    w = 1.0 + 0.2 * rng.standard_normal(64)
    table = synth.rope_table(np.arange(4) + 9, 48, dtype=np.float64)
    for il in (True, False):
        out, _ = oracle.qk_norm_rope(x, x, w, w, table, 48, il, 1e-6)
        for ti in range(4):
            for hi in range(3):
                ref = _brute_row(x[ti, hi], w, np.zeros(0), 0, True, 1e-6)
                assert np.allclose(out[ti, hi, 48:], ref[48:], rtol=0, atol=1e-14)


def test_scale_invariance_and_weight_linearity():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 2, 16))
    w = 1.0 + 0.2 * rng.standard_normal(16)
    table = synth.rope_table(np.arange(3), 16, dtype=np.float64)
    base, _ = oracle.qk_norm_rope(x, x, w, w, table, 16, False, 0.0)
    scaled, _ = oracle.qk_norm_rope(x * 37.0, x, w, w, table, 16, False, 0.0)
    assert np.allclose(scaled, base, rtol=1e-13, atol=1e-13)
    wider, _ = oracle.qk_norm_rope(x, x, 2.5 * w, w, table, 16, False, 0.0)
    assert np.allclose(wider, 2.5 * base, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- planted mistakes

def _pins_hold():
    try:
        for case in BRUTE_CASES:
            if not _check_brute(case):
                return False
        test_unit_mean_square()
        test_zero_angle_is_identity_and_quarter_turn()
        test_partial_rotary_passthrough()
        test_halfsplit_is_permuted_interleaved()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


_orig_rms = nr.rms_norm
_orig_pairs = nr.rope_pairs
_orig_rope = nr.apply_rope


def _mut_sin_sign(y, table, rot, il):
    t = np.array(table, dtype=np.float64)
    t[:, rot // 2:] *= -1.0
    return _orig_rope(y, t, rot, il)


def _mut_cos_sin_swapped(y, table, rot, il):
    t = np.array(table, dtype=np.float64)
    t = np.concatenate([t[:, rot // 2:], t[:, :rot // 2]], axis=1)
    return _orig_rope(y, t, rot, il)


def _mut_pairing_swapped(rot, il):
    return _orig_pairs(rot, not il)


def _mut_sum_not_mean(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * w


def _mut_eps_outside(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * w


def _mut_weight_first(x, w, eps):
    return _orig_rms(np.asarray(x, dtype=np.float64) * w, np.ones_like(w), eps)


def _mut_drop_passthrough(y, table, rot, il):
    out = _orig_rope(y, table, rot, il)
    out[..., rot:] = 0.0
    return out


def _mut_table_by_head(y, table, rot, il):
    t = np.asarray(table)[::-1]                      # rows of the wrong tokens
    return _orig_rope(y, t, rot, il)


MUTANTS = [
    ("apply_rope", _mut_sin_sign),
    ("apply_rope", _mut_cos_sin_swapped),
    ("rope_pairs", _mut_pairing_swapped),
    ("rms_norm", _mut_sum_not_mean),
    ("rms_norm", _mut_eps_outside),
    ("rms_norm", _mut_weight_first),
    ("apply_rope", _mut_drop_passthrough),
    ("apply_rope", _mut_table_by_head),
]


def test_pins_hold_on_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(nr, name, mutant)
    assert not _pins_hold()
