"""jpa_forward_scratch, the allocation-free variant of jpa_forward_ws (its
cut items' partial results in the library's static device scratch instead of
a caller workspace), called through the C ABI: its output equals
jpa_forward_ws's with the same split, bit for bit, on two calls in a row (the
second with a smaller input, so stale scratch contents from the first call
would show), and meets the oracle bar."""

import ctypes
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


def _c_call(lib, dev, x, out, lse, split_wgs):
    """jpa_forward_scratch straight through ctypes on torch's current stream."""
    d = [jpa.descriptor(dev[n]) for n in gh.NAMES]
    od = jpa.descriptor(out)
    cq, cp, cs = (np.ascontiguousarray(x[n], dtype=np.int32) for n in ("cu_q", "cu_prefix", "cu_suffix_real"))
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return lib.jpa_forward_scratch(*[ctypes.byref(t) for t in d], cq.size - 1, P(cq), P(cp), P(cs),
                                   float(x["scale"]), ctypes.byref(od), ctypes.c_void_p(lse.data_ptr()),
                                   int(split_wgs), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (workload, split_wgs): the CFG-pair workload with the library's own choice
# (its last round is cut over the compute units), then a smaller ragged GQA
# call forced over 37 ranges
CALLS = [
    (synth.WORKLOADS[3], 0),
    (synth.custom_workload(6, 2, 128, [77, 128], [1000, 300], [13, 40], "prefix+suffix", wid=720), 37),
]


def test_scratch_entry_matches_workspace_entry_twice():
    lib = jpa.load_library()
    for i, (w, split) in enumerate(CALLS):
        _say(f"call {i}: {w.name} split_wgs={split}")
        x = synth.make_inputs(w, pad_fill="garbage")
        dev = gh.device_inputs(x)
        tq = dev["q"].shape[0]
        out_s = torch.full_like(dev["q"], float("nan"))
        lse_s = torch.full((w.hq, tq), float("nan"), dtype=torch.float32, device="cuda")
        st = _c_call(lib, dev, x, out_s, lse_s, split)
        assert st == jpa.JPA_OK, jpa.jpa_status_str(st)
        o_w, l_w = jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                                      dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                                      x["scale"], split_wgs=split)
        torch.cuda.synchronize()
        assert np.array_equal(gh.bits(out_s), gh.bits(o_w)), f"call {i}: out differs"
        assert np.array_equal(lse_s.cpu().numpy().view(np.int32), l_w.cpu().numpy().view(np.int32)), \
            f"call {i}: lse differs"
        err = gh.assert_parity_full(w, x, *gh.host(out_s, lse_s))
        _say(f"call {i}: bit-identical to jpa_forward_ws; oracle {err}")
        del dev, out_s, lse_s, o_w, l_w


def test_scratch_entry_rejects_more_ranges_than_it_holds():
    w = CALLS[1][0]
    x = synth.make_inputs(w)
    dev = gh.device_inputs(x)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((w.hq, dev["q"].shape[0]), dtype=torch.float32, device="cuda")
    lib = jpa.load_library()
    assert _c_call(lib, dev, x, out, lse, jpa.SCRATCH_MAX_WGS + 1) == jpa.JPA_ERR_SCRATCH
    assert _c_call(lib, dev, x, out, lse, -1) == jpa.JPA_ERR_VALUE
    assert _c_call(lib, dev, x, out, lse, jpa.SCRATCH_MAX_WGS) == jpa.JPA_OK
    torch.cuda.synchronize()
