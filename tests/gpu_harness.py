"""Shared helpers of the GPU tests: move seeded inputs to the device, call the
HIP library through the C ABI binding, compare with the oracle."""

import numpy as np
import torch

import oracle
from diffusion_transformer_joint_non_amd import jpa

# Parity bar, compared in float32 over real query rows.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3

NAMES = ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")


def to_device(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda", non_blocking=False)


def device_inputs(x):
    return {n: to_device(x[n]) for n in NAMES}


def run(x, dev=None, scale=None, with_lse=True, out=None, lse=None, **override):
    dev = dev or device_inputs(x)
    args = dict(dev)
    args.update(override)
    o, l = jpa.jpa_forward(args["q"], args["k_prefix"], args["v_prefix"], args["k_suffix"],
                           args["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                           x["scale"] if scale is None else scale, out=out, lse=lse,
                           with_lse=with_lse)
    torch.cuda.synchronize()
    return o, l


def run_ws(x, dev=None):
    """The call bench.py times: jpa_forward_ws with its cached workspace, the
    library deciding whether to balance the last round of work items."""
    dev = dev or device_inputs(x)
    o, l = jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                              dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                              x["scale"], workspace="auto")
    torch.cuda.synchronize()
    return o, l


def host(o, l):
    """bf16 out -> float32 numpy, lse -> float32 numpy."""
    return o.float().cpu().numpy(), (None if l is None else l.cpu().numpy())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy()


def assert_pad_rows(w, out, lse):
    pad = w.pad_query_mask()
    assert np.all(out[pad] == 0.0), "pad query rows must be written as zeros"
    assert np.all(np.signbit(out[pad]) == False)  # noqa: E712  (+0.0, not -0.0)
    if lse is not None:
        assert np.all(lse[:, pad] == -np.inf), "pad query rows must get LSE = -inf"


def oracle_full(x, scale=None):
    return oracle.attention(*[x[n] for n in NAMES], x["cu_q"], x["cu_prefix"],
                            x["cu_suffix_real"], x["scale"] if scale is None else scale)


def assert_parity_full(w, x, out, lse, scale=None, ref=None):
    ref_o, ref_l = oracle_full(x, scale) if ref is None else ref
    real = ~w.pad_query_mask()
    err = oracle.compare(out[real], lse[:, real].T if lse is not None else np.zeros(0),
                         ref_o[real], ref_l[:, real].T if lse is not None else np.zeros(0))
    assert err["max_abs"] <= MAX_ABS, err
    assert err["mean_abs"] <= MEAN_ABS, err
    assert err["lse_max_abs"] <= LSE_ABS, err
    assert_pad_rows(w, out, lse)
    return err


def assert_parity_rows(out, lse, rows, ref_o, ref_l):
    """out [Tq, Hq, D], lse [Hq, Tq]; rows [Hq, n]; ref [Hq, n, D] / [Hq, n]."""
    hq = rows.shape[0]
    go = np.stack([out[rows[h], h] for h in range(hq)])
    gl = np.stack([lse[h, rows[h]] for h in range(hq)])
    err = oracle.compare(go, gl, ref_o, ref_l)
    assert err["max_abs"] <= MAX_ABS, err
    assert err["mean_abs"] <= MEAN_ABS, err
    assert err["lse_max_abs"] <= LSE_ABS, err
    return err
