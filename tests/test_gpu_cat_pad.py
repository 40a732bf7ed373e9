"""GPU parity of jpa_causal_cat_pad (the HIP kernel through the C ABI) with the
cat + pad oracle: bit for bit, on shapes chosen to exercise every path (16-
byte aligned rows, rows shifted by odd and even left pads, chunks crossing
rows, rows narrower than a chunk, a ragged final chunk, no cache, no frames,
no padding), on seeded random small shapes, and on the eight synthetic
decoder shapes at full size with the oracle on two channels (channels are
independent)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_transformer_joint_non_amd import jpa

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rand(shape, seed):
    return np.random.default_rng(seed).integers(1, 65535, size=shape, dtype=np.uint16)


CASES = [
    # (b, c, t, h, w, cache_frames, padding)
    (1, 3, 2, 5, 16, 2, (1, 1, 1, 1, 0, 0)),
    (1, 2, 2, 4, 16, 2, (0, 0, 1, 1, 0, 0)),        # aligned rows, no column shift
    (2, 3, 3, 5, 13, 1, (2, 3, 1, 0, 1, 0)),        # even left pad, ragged rows
    (1, 4, 1, 7, 21, 0, (5, 2, 2, 2, 2, 0)),        # odd left pad > 1, no cache
    (1, 2, 2, 3, 5, 2, (1, 1, 1, 1, 0, 0)),         # rows narrower than a chunk
    (1, 1, 1, 1, 1, 1, (0, 0, 0, 0, 0, 1)),         # 2 output elements: a ragged final chunk
    (1, 2, 0, 4, 24, 3, (1, 0, 0, 1, 0, 0)),        # cache only
    (1, 2, 3, 4, 24, 0, (0, 0, 0, 0, 0, 0)),        # a copy
    (1, 2, 2, 6, 40, 2, (9, 7, 0, 0, 0, 2)),        # wide pads, time-right pad
    (3, 5, 2, 9, 31, 2, (1, 1, 1, 1, 0, 0)),
]


@pytest.mark.parametrize("case", CASES)
def test_bit_exact_small(case):
    b, c, t, h, w, tc, pad = case
    x = _rand((b, c, t, h, w), 1)
    cache = _rand((b, c, tc, h, w), 2) if tc else None
    out = jpa.jpa_causal_cat_pad(_dev(x), None if cache is None else _dev(cache), pad)
    torch.cuda.synchronize()
    ref = oracle.cat_pad(x, cache, pad)
    assert tuple(out.shape) == ref.shape
    assert np.array_equal(_host_bits(out), ref)


def _random_case(seed):
    r = np.random.default_rng(1000 + seed)
    b, c, t, h = (int(v) for v in (r.integers(1, 3), r.integers(1, 6), r.integers(0, 4), r.integers(1, 12)))
    w, tc = int(r.integers(1, 70)), int(r.integers(0, 3))
    pad = tuple(int(v) for v in r.integers(0, 4, 6))
    if t + tc == 0:
        t = 1
    return b, c, t, h, w, tc, pad


@pytest.mark.parametrize("seed", range(24))
def test_bit_exact_random(seed):
    """Seeded random shapes and pads: rows of every width against the chunk
    size, so that waves mix in-row chunks, row edges and multi-row chunks."""
    b, c, t, h, w, tc, pad = _random_case(seed)
    x = _rand((b, c, t, h, w), 10 + seed)
    cache = _rand((b, c, tc, h, w), 50 + seed) if tc else None
    out = jpa.jpa_causal_cat_pad(_dev(x), None if cache is None else _dev(cache), pad)
    torch.cuda.synchronize()
    assert np.array_equal(_host_bits(out), oracle.cat_pad(x, cache, pad))


@pytest.mark.parametrize("case", synth.CAT_PAD_CASES, ids=[c.name for c in synth.CAT_PAD_CASES])
def test_decoder_shapes(case):
    inp = synth.make_cat_pad_inputs(case)
    x, cache = _dev(inp["x"]), _dev(inp["cache"]) if case.cache_frames else None
    out = jpa.jpa_causal_cat_pad(x, cache, case.padding)
    torch.cuda.synchronize()
    # every channel, bit for bit, in blocks of 32 channels to bound host memory
    for c0 in range(0, case.c, 32):
        c1 = min(case.c, c0 + 32)
        ref = oracle.cat_pad(inp["x"][:, c0:c1], inp["cache"][:, c0:c1] if case.cache_frames else None,
                             case.padding)
        got = _host_bits(out[:, c0:c1].contiguous())
        assert got.shape == ref.shape and np.array_equal(got, ref), (case.name, c0)
        del ref, got


def test_output_fully_written():
    """Every output element is written (pads as +0.0), whatever was there."""
    x = _rand((1, 2, 2, 5, 11), 3)
    cache = _rand((1, 2, 1, 5, 11), 4)
    pad = (1, 2, 1, 1, 1, 0)
    shape = oracle.out_shape(x.shape, 1, pad)
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    jpa.jpa_causal_cat_pad(_dev(x), _dev(cache), pad, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(_host_bits(out), oracle.cat_pad(x, cache, pad))
