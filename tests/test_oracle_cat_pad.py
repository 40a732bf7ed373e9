"""Pins for the cat + pad oracle (oracle/cat_pad.py), none re-running its
numpy calls:

* brute force: every output element from explicit index arithmetic (Python
  loops) on small shapes, bit for bit (uint16 payloads, so any bit pattern);
* special cases: no cache is a plain pad, no padding is a plain
  concatenation, and the interior slice is exactly [cache ; x];
* the padded border is all zeros and the element sum is preserved;
* planted mistakes are caught.
(sglang PR #29281 review: cat + pad + zero-fill of causal Conv3D caches.)
"""

import importlib

import numpy as np
import pytest

import oracle

cp = importlib.import_module("oracle.cat_pad")


def _rand(shape, seed):
    return np.random.default_rng(seed).integers(1, 65535, size=shape, dtype=np.uint16)


def _brute(x, cache, padding):
    wl, wr, hl, hr, tl, tr = padding
    b, c, t, h, w = x.shape
    tc = 0 if cache is None else cache.shape[2]
    shp = (b, c, tc + t + tl + tr, h + hl + hr, w + wl + wr)
    out = np.empty(shp, dtype=x.dtype)
    for i0 in range(shp[0]):
        for i1 in range(shp[1]):
            for it in range(shp[2]):
                for ih in range(shp[3]):
                    for iw in range(shp[4]):
                        tt, hh, ww = it - tl, ih - hl, iw - wl
                        if 0 <= tt < tc + t and 0 <= hh < h and 0 <= ww < w:
                            src = cache if tt < tc else x
                            out[i0, i1, it, ih, iw] = src[i0, i1, tt if tt < tc else tt - tc, hh, ww]
                        else:
                            out[i0, i1, it, ih, iw] = 0
    return out


CASES = [
    ((1, 2, 3, 4, 5), 2, (1, 1, 1, 1, 0, 0)),
    ((2, 1, 2, 3, 9), 0, (1, 1, 1, 1, 2, 0)),
    ((1, 3, 1, 2, 2), 1, (0, 3, 2, 0, 1, 1)),
    ((1, 1, 2, 1, 1), 3, (0, 0, 0, 0, 0, 0)),
    ((1, 2, 0, 2, 3), 2, (2, 1, 0, 1, 0, 0)),
]


def _check(case, seed=3):
    shape, tc, pad = case
    x = _rand(shape, seed)
    cache = _rand(shape[:2] + (tc,) + shape[3:], seed + 1) if tc else None
    got = cp.cat_pad(x, cache, pad)
    ok = got.shape == cp.out_shape(shape, tc, pad) and got.dtype == x.dtype
    return bool(ok and np.array_equal(got, _brute(x, cache, pad)))


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    assert _check(case)


def test_special_cases():
    x = _rand((1, 2, 3, 4, 6), 7)
    cache = _rand((1, 2, 2, 4, 6), 8)
    # no cache: the pad alone
    out = cp.cat_pad(x, None, (1, 2, 0, 1, 2, 0))
    assert out.shape == (1, 2, 5, 5, 9)
    assert np.array_equal(out[:, :, 2:, 0:4, 1:7], x)
    # no padding: the concatenation alone, cache frames first
    out = cp.cat_pad(x, cache, (0,) * 6)
    assert np.array_equal(out[:, :, :2], cache) and np.array_equal(out[:, :, 2:], x)
    # interior of a padded result
    out = cp.cat_pad(x, cache, (1, 1, 1, 1, 1, 0))
    assert np.array_equal(out[:, :, 1:3, 1:5, 1:7], cache)
    assert np.array_equal(out[:, :, 3:6, 1:5, 1:7], x)


def test_border_zero_and_sum():
    x = np.random.default_rng(9).standard_normal((2, 3, 2, 5, 7))
    cache = np.random.default_rng(10).standard_normal((2, 3, 1, 5, 7))
    out = cp.cat_pad(x, cache, (2, 1, 1, 3, 1, 0))
    mask = np.ones(out.shape, dtype=bool)
    mask[:, :, 1:4, 1:6, 2:9] = False
    assert np.all(out[mask] == 0.0)
    assert np.isclose(out.sum(), x.sum() + cache.sum(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

_orig = cp.cat_pad


def _mut_cache_after(x, cache, padding):
    return _orig(cache if cache is not None and cache.shape[2] else x,
                 x if cache is not None and cache.shape[2] else None, padding)


def _mut_pad_order(x, cache, padding):
    wl, wr, hl, hr, tl, tr = padding
    return _orig(x, cache, (wr, wl, hr, hl, tl, tr))


def _mut_drop_cache(x, cache, padding):
    return _orig(x, None, padding)


def _mut_h_w_swapped(x, cache, padding):
    wl, wr, hl, hr, tl, tr = padding
    return _orig(x, cache, (hl, hr, wl, wr, tl, tr))


MUTANTS = [_mut_cache_after, _mut_pad_order, _mut_drop_cache, _mut_h_w_swapped]


def _pins_hold():
    try:
        return all(_check(c) for c in CASES)
    except (ValueError, IndexError, TypeError):
        return False


def test_pins_hold_on_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(cp, "cat_pad", mutant)
    assert not _pins_hold()
