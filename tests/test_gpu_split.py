"""GPU parity of jpa_forward_ws: the last round of work items cut into balanced
key ranges (pieces) whose partial results a second kernel merges.

The split changes only the order of the sums, so outputs must meet the same
oracle bar as jpa_forward; forced splits (split_wgs > 0) exercise items cut
into many pieces, pieces starting in the mixed first tiles, all-pad items and
several rows per launch."""

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


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    jpa.load_library()


def _run_ws(x, split_wgs, dev=None, ws=None):
    dev = dev or gh.device_inputs(x)
    d = dev["q"].shape[2]
    if ws is None:
        ws = torch.zeros(jpa.jpa_workspace_bytes(d, split_wgs), dtype=torch.uint8, device="cuda")
    o, l = jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                              dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                              x["scale"], workspace=ws, split_wgs=split_wgs)
    torch.cuda.synchronize()
    return o, l


SPLIT_CASES = [
    ((4, 2, 128, [77], [300], [37], "prefix+suffix"), (3, 8, 13, 64)),
    ((6, 3, 128, [0, 130], [513, 64], [0, 200], "suffix"), (5, 16, 200)),
    ((3, 3, 64, [64, 1, 5], [64, 0, 1000], [64, 2, 0], "prefix+suffix"), (7, 40)),
    ((2, 1, 128, [3, 0, 2], [0, 40, 0], [9, 0, 300], "suffix"), (3, 8)),
    ((8, 8, 128, [511], [257], [255], "suffix"), (9, 100)),
]


@pytest.mark.parametrize("ci", range(len(SPLIT_CASES)))
def test_forced_split_matches_oracle(ci):
    shape, splits = SPLIT_CASES[ci]
    w = synth.custom_workload(*shape, wid=700 + ci)
    x = synth.make_inputs(w, pad_fill="garbage")
    dev = gh.device_inputs(x)
    for sw in splits:
        _say(f"split case {ci} {shape} split_wgs={sw}")
        o, l = _run_ws(x, sw, dev)
        oh, lh = gh.host(o, l)
        gh.assert_parity_full(w, x, oh, lh)


def test_auto_split_cfg_pair_matches_unsplit():
    """CFG pair: 1608 items on 256 units leave a last round 28 % full, so the
    automatic split engages; it must agree with the unsplit call to rounding
    and be deterministic."""
    w = synth.WORKLOADS[3]
    x = synth.make_inputs(w)
    dev = gh.device_inputs(x)
    o0, l0 = gh.run(x, dev)
    o1, l1 = _run_ws(x, 0, dev)
    o2, l2 = _run_ws(x, 0, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    real = torch.from_numpy(~w.pad_query_mask())
    a, b = o0.float().cpu(), o1.float().cpu()
    d = (a[real] - b[real]).abs()
    assert float(d.max()) <= 4e-3 and float(d.mean()) <= 5e-5, (float(d.max()), float(d.mean()))
    assert torch.equal(a[~real], b[~real])
    la, lb = l0.cpu(), l1.cpu()
    assert float((la[:, real] - lb[:, real]).abs().max()) <= 1e-5
    assert torch.equal(la[:, ~real], lb[:, ~real])


def test_workspace_reuse_and_smaller_calls():
    """One workspace serves consecutive calls of different shapes (no state
    is kept in it between calls)."""
    ws = torch.zeros(jpa.jpa_workspace_bytes(128, 16), dtype=torch.uint8, device="cuda")
    for shape in [(4, 2, 128, [77], [300], [37], "prefix+suffix"),
                  (2, 2, 128, [5], [70], [1], "suffix"),
                  (4, 2, 128, [77], [300], [37], "prefix+suffix")]:
        w = synth.custom_workload(*shape, wid=750)
        x = synth.make_inputs(w)
        o, l = _run_ws(x, 16, ws=ws)
        oh, lh = gh.host(o, l)
        gh.assert_parity_full(w, x, oh, lh)


def test_split_without_lse():
    w = synth.custom_workload(4, 2, 128, [77], [300], [37], "prefix+suffix", wid=760)
    x = synth.make_inputs(w)
    dev = gh.device_inputs(x)
    ws = torch.zeros(jpa.jpa_workspace_bytes(128, 8), dtype=torch.uint8, device="cuda")
    o, l = jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                              dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                              x["scale"], with_lse=False, workspace=ws, split_wgs=8)
    torch.cuda.synchronize()
    assert l is None
    o_ref, _ = _run_ws(x, 8, dev)
    assert torch.equal(o, o_ref)
