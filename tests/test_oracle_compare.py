"""Pins of ``oracle.compare``, the error summary every attention parity verdict
is taken from (the GPU output against the oracle, compared in float32 over
real query rows: max-abs and mean-abs of out, max-abs of the LSE).

The expected values are fixed by hand-built arrays whose entries and errors
are exact binary fractions, so each expectation is an exact number:

* known max-abs, mean-abs and LSE max-abs, with errors of both signs;
* the comparison is taken in float32: an fp64 reference that rounds to the
  GPU's value in float32 compares as equal;
* a NaN anywhere in the GPU output or LSE makes the summary fail the bar;
* empty inputs summarise to zeros;
* the summary is over every element of any shape (rows x heads x features).

Planted mistakes in ``compare`` (mean for max, one slice only, no float32
cast, NaN swallowed, signed differences) must each make a pin fail.
"""

import numpy as np
import pytest

import oracle
from oracle import fp64

MAX_ABS, MEAN_ABS, LSE_ABS = 1e-2, 1e-3, 1e-3


def _meets_bar(err):
    return err["max_abs"] <= MAX_ABS and err["mean_abs"] <= MEAN_ABS and err["lse_max_abs"] <= LSE_ABS


def _case():
    """ref out [3, 4, 8] and lse [3, 4]; the GPU copy differs by +0.5 at one
    element, -0.25 at another, and by -0.125 in one LSE entry."""
    rng = np.random.default_rng(11)
    ref_o = np.round(rng.standard_normal((3, 4, 8)) * 64) / 64          # multiples of 2^-6
    ref_l = np.round(rng.standard_normal((3, 4)) * 64) / 64
    go = ref_o.astype(np.float32).copy()
    go[1, 2, 5] += 0.5
    go[2, 0, 0] -= 0.25
    gl = ref_l.astype(np.float32).copy()
    gl[0, 3] -= 0.125
    return go, gl, ref_o, ref_l


def _pins_hold(compare) -> bool:
    try:
        go, gl, ro, rl = _case()
        e = compare(go, gl, ro, rl)
        assert e["max_abs"] == 0.5
        assert e["mean_abs"] == pytest.approx(0.75 / 96, rel=1e-6)
        assert e["lse_max_abs"] == 0.125
        assert not _meets_bar(e)

        # identical values: zero everywhere, the bar is met
        e = compare(ro.astype(np.float32), rl.astype(np.float32), ro, rl)
        assert e == {"max_abs": 0.0, "mean_abs": 0.0, "lse_max_abs": 0.0}
        assert _meets_bar(e)

        # errors just inside the bar pass it
        go2 = ro.astype(np.float32).copy()
        go2[0, 0, 0] += np.float32(2.0 ** -7)                # 7.8e-3 < 1e-2, mean 8.1e-5
        gl2 = rl.astype(np.float32).copy()
        gl2[2, 1] += np.float32(2.0 ** -10)                  # 9.8e-4 < 1e-3
        e = compare(go2, gl2, ro, rl)
        assert e["max_abs"] == 2.0 ** -7 and e["lse_max_abs"] == 2.0 ** -10
        assert _meets_bar(e)

        # float32 comparison: 1 + 2^-30 rounds to 1.0f, so it equals a GPU 1.0
        e = compare(np.ones((2, 2), np.float32), np.full(2, -3.0, np.float32),
                    np.full((2, 2), 1.0 + 2.0 ** -30), np.full(2, -3.0 - 2.0 ** -28))
        assert e["max_abs"] == 0.0 and e["mean_abs"] == 0.0 and e["lse_max_abs"] == 0.0

        # a NaN in the output or in the LSE fails the bar
        go3 = ro.astype(np.float32).copy()
        go3[2, 3, 7] = np.nan
        assert not _meets_bar(compare(go3, rl.astype(np.float32), ro, rl))
        gl3 = rl.astype(np.float32).copy()
        gl3[1, 1] = np.nan
        assert not _meets_bar(compare(ro.astype(np.float32), gl3, ro, rl))

        # an inf where the reference is finite fails it too
        gl4 = rl.astype(np.float32).copy()
        gl4[0, 0] = -np.inf
        assert not _meets_bar(compare(ro.astype(np.float32), gl4, ro, rl))

        # empty inputs summarise to zeros
        e = compare(np.zeros((0, 4, 8), np.float32), np.zeros((0, 4), np.float32),
                    np.zeros((0, 4, 8)), np.zeros((0, 4)))
        assert e == {"max_abs": 0.0, "mean_abs": 0.0, "lse_max_abs": 0.0}

        # every element counts, wherever it sits
        for idx in [(0, 0, 0), (2, 3, 7), (1, 0, 4)]:
            g = ro.astype(np.float32).copy()
            g[idx] += 1.0
            e = compare(g, rl.astype(np.float32), ro, rl)
            assert e["max_abs"] == 1.0 and e["mean_abs"] == pytest.approx(1.0 / 96, rel=1e-6)
    except AssertionError:
        return False
    return True


def test_compare_pins_hold():
    assert _pins_hold(oracle.compare)


# ---------------------------------------------------------------- planted mistakes

def _summary(go, gl, ro, rl, reduce_max, reduce_mean, cast=np.float32, absolute=True):
    go = np.asarray(go, dtype=cast)
    ro = np.asarray(ro, dtype=np.float64).astype(cast)
    d = go - ro
    d = np.abs(d) if absolute else d
    gl = np.asarray(gl, dtype=cast)
    rl = np.asarray(rl, dtype=np.float64).astype(cast)
    dl = np.abs(gl - rl) if absolute else gl - rl
    return {"max_abs": float(reduce_max(d)) if d.size else 0.0,
            "mean_abs": float(reduce_mean(d)) if d.size else 0.0,
            "lse_max_abs": float(reduce_max(dl)) if dl.size else 0.0}


def _mut_mean_for_max(go, gl, ro, rl):
    return _summary(go, gl, ro, rl, np.mean, np.mean)


def _mut_first_slice_only(go, gl, ro, rl):
    return _summary(go, gl, ro, rl, lambda d: d[0].max(), lambda d: d[0].mean())


def _mut_no_fp32_cast(go, gl, ro, rl):
    return _summary(go, gl, ro, rl, np.max, np.mean, cast=np.float64)


def _mut_nan_swallowed(go, gl, ro, rl):
    return _summary(go, gl, ro, rl, np.nanmax, np.nanmean)


def _mut_signed(go, gl, ro, rl):
    return _summary(go, gl, ro, rl, np.max, np.mean, absolute=False)


MUTANTS = [_mut_mean_for_max, _mut_first_slice_only, _mut_no_fp32_cast, _mut_nan_swallowed,
           _mut_signed]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_planted_compare_mistake_is_caught(mutant):
    assert not _pins_hold(mutant)


def test_oracle_package_exports_the_pinned_compare():
    assert oracle.compare is fp64.compare
