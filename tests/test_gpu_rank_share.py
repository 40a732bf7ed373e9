"""GPU checks of the sequence-parallel pieces around the kernel:

* rank-share mode: one rank's heads of a head-parallel (Ulysses) split, with
  the replicated prefix passed as a head-sliced view (pointer offset and the
  full token stride; no copy, sglang PR #26973 review, split path), equals
  the same heads of the unsplit call bit for bit, and the oracle;
* the host shard planner's offsets drive the kernel: a tail-padded suffix
  (sglang PR #30107 review, layout invariant) gathered as [real | pad] and a
  rank's local [valid | pad] chunk, pad slots filled with garbage, match the
  oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_transformer_joint_non_amd import jpa
from gpu_harness import MAX_ABS, MEAN_ABS, LSE_ABS, to_device

pytestmark = pytest.mark.gpu


def _oracle_check(x, o, l, w):
    ref_o, ref_l = oracle.attention(*[x[n] for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix",
                                                     "cu_q", "cu_prefix", "cu_suffix_real")], x["scale"])
    real = ~w.pad_query_mask()
    go, gl = o.float().cpu().numpy(), l.cpu().numpy()
    err = oracle.compare(go[real], gl[:, real].T, ref_o[real], ref_l[:, real].T)
    assert err["max_abs"] <= MAX_ABS and err["mean_abs"] <= MEAN_ABS and err["lse_max_abs"] <= LSE_ABS, err
    assert np.all(go[~real] == 0.0)


@pytest.mark.parametrize("hq,hkv,sp", [(8, 8, 4), (8, 2, 2), (10, 2, 2)])
def test_rank_share_equals_slice_of_full_call(hq, hkv, sp):
    w = synth.custom_workload(hq, hkv, 128, [300], [1200], [13], "suffix", wid=61)
    x = synth.make_inputs(w)
    dev = {n: to_device(x[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")}
    o_full, l_full = jpa.jpa_forward(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"], dev["v_suffix"],
                                     x["cu_q"], x["cu_prefix"], x["cu_suffix_real"], x["scale"])
    torch.cuda.synchronize()
    hq_r, hkv_r = hq // sp, hkv // sp
    for r in range(sp):
        qs = slice(r * hq_r, (r + 1) * hq_r)
        ks = slice(r * hkv_r, (r + 1) * hkv_r)
        # per-rank q/k/v after the exchange are contiguous; the prefix is a view
        q = dev["q"][:, qs].contiguous()
        k_suf = dev["k_suffix"][:, ks].contiguous()
        v_suf = dev["v_suffix"][:, ks].contiguous()
        kp_view, vp_view = dev["k_prefix"][:, ks], dev["v_prefix"][:, ks]
        assert kp_view.stride(0) == hkv * 128 and not kp_view.is_contiguous() or hkv_r == hkv
        o, l = jpa.jpa_forward(q, kp_view, vp_view, k_suf, v_suf, x["cu_q"], x["cu_prefix"],
                               x["cu_suffix_real"], x["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_full[:, qs].contiguous().view(torch.int16)), r
        assert torch.equal(l, l_full[qs]), r
    _oracle_check(x, o_full, l_full, w)


def _planned_case(seq_len, sp, rank, gathered, prefixes, qp, mult=1):
    """Inputs laid out by the shard planner's offsets, pad slots garbage."""
    sh = jpa.jpa_shard_plan(seq_len, sp, rank)
    if gathered:
        # after a head-parallel exchange every rank holds the whole padded sequence
        g = jpa.JpaShard(sh.orig_len, sh.local_len * sp, sh.num_pad, 1, 0, sh.num_pad, sh.orig_len)
        sh = g
    cu_q, cu_p, cu_s = jpa.jpa_tail_segments(sh, mult, prefixes, qp)
    real = sh.local_real_len * mult
    pad = sh.local_pad * mult
    w = synth.custom_workload(4, 2, 128, prefixes, [real] * len(prefixes), [pad] * len(prefixes),
                              "prefix+suffix" if qp else "suffix", wid=62)
    assert list(w.cu_q()) == list(cu_q) and list(w.cu_suffix_real()) == list(cu_s)
    x = synth.make_inputs(w, pad_fill="garbage")
    return w, x, (cu_q, cu_p, cu_s)


@pytest.mark.parametrize("seq_len,sp,rank,gathered,prefixes,qp", [
    (1001, 4, 0, True, [96], True),        # gathered [1001 real | 3 pad]
    (1001, 4, 3, False, [96], False),      # last rank's local chunk [248 | 3]
    (5, 4, 2, False, [40, 7], True),       # a chunk with pad that is not the last
    (4096, 8, 7, False, [512], True),      # no pad
])
def test_planner_offsets_drive_the_kernel(seq_len, sp, rank, gathered, prefixes, qp):
    w, x, (cu_q, cu_p, cu_s) = _planned_case(seq_len, sp, rank, gathered, prefixes, qp)
    dev = {n: to_device(x[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")}
    o, l = jpa.jpa_forward(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"], dev["v_suffix"],
                           cu_q, cu_p, cu_s, x["scale"])
    torch.cuda.synchronize()
    _oracle_check(x, o, l, w)
