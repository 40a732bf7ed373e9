"""The library's calls can be captured in a HIP graph (torch.cuda.CUDAGraph):
they allocate nothing, never synchronise and record no memset.  Each graph is
replayed several times with eager work and synchronisations in between, and
every replay must equal the eager result bit for bit."""

import numpy as np
import pytest
import torch

import synth
from diffusion_transformer_joint_non_amd import jpa
from gpu_harness import to_device

pytestmark = pytest.mark.gpu


def _replay_and_check(capture, eager_outs, outs):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            capture()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        for o in outs:
            o.view(torch.int16).fill_(-1)                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager_outs):
            assert torch.equal(o.view(torch.int16) if o.dtype != torch.float32 else o,
                               e.view(torch.int16) if e.dtype != torch.float32 else e), f"replay {i}"


@pytest.mark.parametrize("split", [0, 64])
def test_attention_graph_replays(split):
    w = synth.WORKLOADS[3] if split else synth.WORKLOADS[2]
    x = synth.make_inputs(w)
    dev = {n: to_device(x[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")}
    out = torch.empty_like(dev["q"])
    lse = torch.empty((w.hq, dev["q"].shape[0]), dtype=torch.float32, device="cuda")
    ws = jpa.workspace_for(out.device, 0, w.d, split) if split else None

    def call(stream=None):
        jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"], dev["v_suffix"],
                           x["cu_q"], x["cu_prefix"], x["cu_suffix_real"], x["scale"], out=out, lse=lse,
                           workspace=ws, split_wgs=split, stream=stream)
    call()
    torch.cuda.synchronize()
    eager_o, eager_l = out.clone(), lse.clone()
    _replay_and_check(lambda: call(torch.cuda.current_stream()), [eager_o, eager_l], [out, lse])


def test_norm_rope_and_cat_pad_graph_replays():
    nw = synth.NORM_ROPE_WORKLOADS[2]
    nx = synth.make_norm_rope_inputs(nw)
    q, k = to_device(nx["q"]), to_device(nx["k"])
    wq, wk = torch.from_numpy(nx["q_weight"]).cuda(), torch.from_numpy(nx["k_weight"]).cuda()
    tab = torch.from_numpy(nx["table"]).cuda()
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    case = synth.CAT_PAD_CASES[1]
    inp = synth.make_cat_pad_inputs(case)
    cx = torch.from_numpy(np.ascontiguousarray(inp["x"]).view(np.int16)).view(torch.bfloat16).cuda()
    cc = torch.from_numpy(np.ascontiguousarray(inp["cache"]).view(np.int16)).view(torch.bfloat16).cuda()
    co = jpa.jpa_causal_cat_pad(cx, cc, case.padding)

    def call(stream=None):
        jpa.jpa_qk_norm_rope(q, k, wq, wk, tab, nw.rotary_dim, nw.interleaved, nw.eps, q_out=qo, k_out=ko,
                             stream=stream)
        jpa.jpa_causal_cat_pad(cx, cc, case.padding, out=co, stream=stream)
    call()
    torch.cuda.synchronize()
    eager = [qo.clone(), ko.clone(), co.clone()]
    _replay_and_check(lambda: call(torch.cuda.current_stream()), eager, [qo, ko, co])
