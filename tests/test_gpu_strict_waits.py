"""Race check of the attention kernel's copy pipeline.

libjpa_strict_waits.so is built from the same sources with JPA_STRICT_WAITS:
at every per-tile barrier the kernel waits for all of its tile copies,
including the newest prefetch that the release build leaves in flight.  The
arithmetic and its order are the same, so both builds must give identical
bits; a tile read from LDS before its copy landed would show up as a
difference here (and, with NaN in the pad slots, as NaN)."""

import sys

import numpy as np
import pytest
import torch

import synth
from diffusion_transformer_joint_non_amd import jpa

import gpu_harness as gh

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return jpa.load_library(), jpa.load_strict_waits_library()


def _both(libs, call):
    """call() under the release build, then under the check build."""
    res = []
    saved = jpa._lib
    try:
        for lib in libs:
            jpa._lib = lib
            o, l = call()
            torch.cuda.synchronize()
            res.append((o.view(torch.int16).clone(), l.view(torch.int32).clone()))
            del o, l
    finally:
        jpa._lib = saved
    return res


CASES = [
    ("workload 1", lambda: synth.WORKLOADS[1]),
    ("workload 2", lambda: synth.WORKLOADS[2]),
    ("workload 3", lambda: synth.WORKLOADS[3]),
    ("GQA 8/2 D=64, ragged", lambda: synth.custom_workload(8, 2, 64, [77, 0, 300], [1000, 513, 5],
                                                          [37, 0, 200], "prefix+suffix", wid=810)),
    ("D=128, short rows", lambda: synth.custom_workload(4, 4, 128, [3, 64, 1], [0, 65, 130],
                                                       [9, 0, 1], "suffix", wid=811)),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
@pytest.mark.parametrize("path", ["forward", "forward_ws"])
def test_strict_waits_build_is_bit_identical(libs, ci, path):
    name, make = CASES[ci]
    w = make()
    x = synth.make_inputs(w, pad_fill="nan")
    dev = gh.device_inputs(x)
    args = (dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"], dev["v_suffix"],
            x["cu_q"], x["cu_prefix"], x["cu_suffix_real"], x["scale"])
    if path == "forward":
        call = lambda: jpa.jpa_forward(*args)
    else:
        # a forced split puts piece boundaries in every item of the last round
        ws = torch.empty(jpa.jpa_workspace_bytes(w.d, 37), dtype=torch.uint8, device="cuda")
        call = lambda: jpa.jpa_forward_ws(*args, workspace=ws, split_wgs=37)
    _say(f"{name}, {path}: release then strict-waits build")
    (o0, l0), (o1, l1) = _both(libs, call)
    assert torch.equal(o0, o1), f"{int((o0 != o1).sum())} output elements differ"
    assert torch.equal(l0, l1), f"{int((l0 != l1).sum())} lse entries differ"
    real = torch.from_numpy(~w.pad_query_mask()).cuda()
    assert not torch.isnan(o0.view(torch.bfloat16)[real].float()).any()
