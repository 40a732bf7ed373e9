"""Host-side checks of the C ABI (no GPU needed; no kernel is run).

* the in-tree libjpa.so loads and exports every function include/*.h declares,
  and so does its strict-waits check build;
* jpa_plan's integers equal the hand-derived workload bookkeeping and the
  oracle's decoding, bit for bit;
* every validation error of jpa_validate is reachable from the host;
* on a machine without a GPU, jpa_forward reports JPA_ERR_HIP instead of crashing;
* every argument check of jpa_qk_norm_rope is reachable from the host, and a
  call that passes them reaches the launch (JPA_ERR_HIP without a GPU).
"""

import ctypes
import glob
import json
import os
import re

import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_transformer_joint_non_amd import jpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jpa.h")


def _declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        names += re.findall(r"JPA_API\s+[\w\s\*]+?\b(jpa_\w+)\s*\(", open(h).read())
    return names


def test_library_exports_every_declared_symbol():
    lib = jpa.load_library()
    names = _declared_functions()
    assert set(names) == set(jpa.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_strict_waits_build_exports_the_same_symbols():
    """The check build (attention kernel waiting for every tile copy at each
    barrier) is a drop-in twin of libjpa.so."""
    lib = jpa.load_strict_waits_library()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    assert lib.jpa_abi_version() == jpa.load_library().jpa_abi_version()


def test_abi_version_and_status_strings():
    m = re.search(r"#define JPA_ABI_VERSION (\d+)", open(HEADER).read())
    assert jpa.jpa_abi_version() == int(m.group(1))
    for code in range(9):
        s = jpa.jpa_status_str(code)
        assert s.startswith("JPA_")
    assert jpa.jpa_status_str(99) == "JPA_ERR_UNKNOWN"


def test_plan_matches_golden_workloads():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "segments.json")))["workloads"]
    for wid, g in gold.items():
        rows, flops = jpa.jpa_plan(g["cu_q"], g["cu_prefix"], g["cu_suffix_real"], g["hq"], g["d"])
        assert [list(r) for r in rows] == g["rows"]
        assert flops == g["valid_flops"]


def _random_segments(rng, batch):
    prefix = rng.integers(0, 300, batch)
    real = rng.integers(0, 5000, batch)
    pad = rng.integers(0, 200, batch)
    both = rng.random(batch) < 0.5
    prefix = np.where((real == 0) & (prefix == 0), 1, prefix)
    lq = real + pad + np.where(both, prefix, 0)
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_p = np.concatenate([[0], np.cumsum(prefix)])
    cs = [0]
    for r, pd in zip(real, pad):
        cs += [cs[-1] + r, cs[-1] + r + pd]
    return cu_q, cu_p, np.asarray(cs)


def test_plan_matches_oracle_decoding_random():
    rng = np.random.default_rng(5)
    for trial in range(200):
        batch = int(rng.integers(0, 70))
        cq, cp, cs = _random_segments(rng, batch)
        hq, d = int(rng.choice([1, 8, 40])), int(rng.choice([64, 128]))
        rows, flops = jpa.jpa_plan(cq, cp, cs, hq, d)
        ref = oracle.decode_segments(cq, cp, cs)
        assert [tuple(r) for r in rows] == [
            (s.q_start, s.q_slots, s.q_real, s.p_start, s.p_len, s.s_start, s.s_real, s.s_pad, s.keys)
            for s in ref]
        assert flops == oracle.valid_flops(ref, hq, d)


# ------------------------------------------------------------ validation paths

def _valid_call(d=64, hq=4, hkv=2):
    w = synth.custom_workload(hq, hkv, d, [3, 5], [7, 4], [2, 1], "prefix+suffix")
    tq, tp, ts = w.tokens()
    bf = torch.bfloat16
    return dict(
        q=torch.zeros(tq, hq, d, dtype=bf), k_prefix=torch.zeros(tp, hkv, d, dtype=bf),
        v_prefix=torch.zeros(tp, hkv, d, dtype=bf), k_suffix=torch.zeros(ts, hkv, d, dtype=bf),
        v_suffix=torch.zeros(ts, hkv, d, dtype=bf), cu_q=list(w.cu_q()),
        cu_prefix=list(w.cu_prefix()), cu_suffix_real=list(w.cu_suffix_real()),
        scale=d ** -0.5, out=torch.zeros(tq, hq, d, dtype=bf))


def _validate(**kw):
    return jpa.jpa_validate(**kw)


def test_validate_accepts_valid_call():
    assert _validate(**_valid_call()) == jpa.JPA_OK
    assert _validate(**_valid_call(d=128, hq=6, hkv=6)) == jpa.JPA_OK
    kw = _valid_call()
    kw["lse"] = torch.zeros(4, kw["q"].shape[0])
    assert _validate(**kw) == jpa.JPA_OK


def test_validate_accepts_strided_views():
    kw = _valid_call(d=128, hq=4, hkv=2)
    fused = torch.zeros(kw["k_suffix"].shape[0], 4 + 2 * 2, 128, dtype=torch.bfloat16)
    kw["k_suffix"] = fused[:, 4:6]
    kw["v_suffix"] = fused[:, 6:8]           # token-strided slice of a fused QKV
    assert _validate(**kw) == jpa.JPA_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda kw: kw.update(q=kw["q"].half()), jpa.JPA_ERR_DTYPE),
    (lambda kw: kw.update(k_suffix=kw["k_suffix"].float()), jpa.JPA_ERR_DTYPE),
    (lambda kw: kw.update(q=torch.zeros(kw["q"].shape[0], 4, 96, dtype=torch.bfloat16)), jpa.JPA_ERR_SHAPE),
    (lambda kw: kw.update(q=torch.zeros(kw["q"].shape[0], 3, 64, dtype=torch.bfloat16),
                          out=torch.zeros(kw["q"].shape[0], 3, 64, dtype=torch.bfloat16)),
     jpa.JPA_ERR_SHAPE),                                             # Hq % Hkv != 0
    (lambda kw: kw.update(out=torch.zeros(kw["q"].shape[0], 2, 64, dtype=torch.bfloat16)),
     jpa.JPA_ERR_SHAPE),                                             # out heads
    (lambda kw: kw.update(v_prefix=kw["v_prefix"][:-1]), jpa.JPA_ERR_SHAPE),   # tokens vs cu
    (lambda kw: kw.update(q=kw["q"][:-1], out=kw["out"][:-1]), jpa.JPA_ERR_SHAPE),
    (lambda kw: kw.update(k_suffix=kw["k_suffix"][:, :1]), jpa.JPA_ERR_SHAPE),  # kv heads
    (lambda kw: kw.update(out=torch.zeros(kw["q"].shape[0] * 4 * 64 + 4, dtype=torch.bfloat16)[4:]
                          .view(kw["q"].shape[0], 4, 64)), jpa.JPA_ERR_LAYOUT),  # misaligned
    (lambda kw: kw.update(k_prefix=torch.zeros(kw["k_prefix"].shape[0], 2, 68, dtype=torch.bfloat16)
                          [:, :, :64].as_strided(kw["k_prefix"].shape, (132, 66, 1))),
     jpa.JPA_ERR_LAYOUT),                                            # strides not multiples of 8
    (lambda kw: kw.update(out=torch.zeros(kw["q"].shape[0] + 8, 64, dtype=torch.bfloat16)
                          .as_strided(kw["q"].shape, (64, 8, 1))), jpa.JPA_ERR_LAYOUT),  # overlap
    (lambda kw: kw.update(cu_q=[1] + kw["cu_q"][1:]), jpa.JPA_ERR_SEGMENTS),
    (lambda kw: kw.update(cu_prefix=[0, 6, 5]), jpa.JPA_ERR_SEGMENTS),
    (lambda kw: kw.update(cu_suffix_real=[0, 7, 6, 10, 12]), jpa.JPA_ERR_SEGMENTS),
    (lambda kw: kw.update(scale=float("nan")), jpa.JPA_ERR_VALUE),
    (lambda kw: kw.update(scale=-0.5), jpa.JPA_ERR_VALUE),
    (lambda kw: kw.update(scale=float("inf")), jpa.JPA_ERR_VALUE),
])
def test_validate_rejects(mutate, code):
    kw = _valid_call()
    mutate(kw)
    assert _validate(**kw) == code


def test_validate_output_overlap():
    """out shares no element with K/V (other workgroups keep reading them);
    it is q itself or disjoint from q; lse shares no byte with any tensor."""
    bf = torch.bfloat16
    kw = _valid_call()
    tq, ts = kw["q"].shape[0], kw["k_suffix"].shape[0]
    # out aliasing a K/V input
    for name in ("k_prefix", "v_prefix", "k_suffix", "v_suffix"):
        k2 = dict(kw)
        src = k2[name]
        big = torch.zeros(max(tq, src.shape[0]), 4, 64, dtype=bf)
        k2[name] = big[:src.shape[0], :src.shape[1]]
        k2["out"] = big[:tq]
        assert _validate(**k2) == jpa.JPA_ERR_LAYOUT, name
    # in place: out is q, the same view
    k2 = dict(kw)
    k2["out"] = k2["q"]
    assert _validate(**k2) == jpa.JPA_OK
    # out shifted one token against q in one buffer
    buf = torch.zeros(tq + 1, 4, 64, dtype=bf)
    k2 = dict(kw)
    k2["q"], k2["out"] = buf[:-1], buf[1:]
    assert _validate(**k2) == jpa.JPA_ERR_LAYOUT
    # q, k, v and out as disjoint column windows of one fused buffer are fine,
    # and the same windows overlapping by one head are not
    fused = torch.zeros(tq, 4 + 2 + 2 + 4, 64, dtype=bf)
    k2 = dict(kw)
    k2["cu_suffix_real"] = [0, tq - 3, tq - 3, tq, tq]   # a layout whose suffix has tq slots
    k2["cu_prefix"] = [0, 0, 0]
    k2["cu_q"] = [0, tq - 3, tq]
    k2["k_prefix"] = k2["v_prefix"] = torch.zeros(0, 2, 64, dtype=bf)
    k2["q"], k2["k_suffix"], k2["v_suffix"], k2["out"] = (fused[:, 0:4], fused[:, 4:6],
                                                          fused[:, 6:8], fused[:, 8:12])
    assert _validate(**k2) == jpa.JPA_OK
    k2["out"] = fused[:, 7:11]
    assert _validate(**k2) == jpa.JPA_ERR_LAYOUT
    # lse inside out, inside q, inside a K/V tensor
    for name in ("out", "q", "k_suffix"):
        k2 = dict(kw)
        host = torch.zeros(k2[name].numel() * 2 + 64 + 16 * tq, dtype=torch.uint8)
        t = host[:k2[name].numel() * 2].view(bf).view(k2[name].shape)
        k2[name] = t
        k2["lse"] = host[64:64 + 16 * tq].view(torch.float32).view(4, tq)
        assert _validate(**k2) == jpa.JPA_ERR_LAYOUT, name
    # a separate lse is fine
    k2 = dict(kw)
    k2["lse"] = torch.zeros(4, tq)
    assert _validate(**k2) == jpa.JPA_OK


def test_validate_rejects_pad_longer_than_row_and_keyless_rows():
    # pad 3 > 2 query slots
    bf = torch.bfloat16
    z = lambda n, h=2: torch.zeros(n, h, 64, dtype=bf)
    assert jpa.jpa_validate(z(2), z(1), z(1), z(4), z(4), [0, 2], [0, 1], [0, 1, 4], 0.1, z(2)) \
        == jpa.JPA_ERR_SEGMENTS
    # real queries but no keys
    assert jpa.jpa_validate(z(3), z(0), z(0), z(1), z(1), [0, 3], [0, 0], [0, 0, 1], 0.1, z(3)) \
        == jpa.JPA_ERR_SEGMENTS
    # an all-pad row with no keys is fine
    assert jpa.jpa_validate(z(3), z(0), z(0), z(3), z(3), [0, 3], [0, 0], [0, 0, 3], 0.1, z(3)) \
        == jpa.JPA_OK
    # empty batch is fine
    assert jpa.jpa_validate(z(0), z(0), z(0), z(0), z(0), [0], [0], [0], 0.1, z(0)) == jpa.JPA_OK


def test_null_pointers_and_bad_counts_from_c():
    lib = jpa.load_library()
    kw = _valid_call()
    d = [jpa.descriptor(kw[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")]
    od = jpa.descriptor(kw["out"])
    cq = np.asarray(kw["cu_q"], np.int32)
    cp = np.asarray(kw["cu_prefix"], np.int32)
    cs = np.asarray(kw["cu_suffix_real"], np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    args = [ctypes.byref(x) for x in d]
    assert lib.jpa_validate(*args, 2, P(cq), P(cp), P(cs), 0.1, ctypes.byref(od), None) == 0
    assert lib.jpa_validate(None, *args[1:], 2, P(cq), P(cp), P(cs), 0.1, ctypes.byref(od), None) \
        == jpa.JPA_ERR_NULL
    assert lib.jpa_validate(*args, 2, None, P(cp), P(cs), 0.1, ctypes.byref(od), None) \
        == jpa.JPA_ERR_NULL
    assert lib.jpa_validate(*args, 2, P(cq), P(cp), P(cs), 0.1, None, None) == jpa.JPA_ERR_NULL
    assert lib.jpa_validate(*args, -1, P(cq), P(cp), P(cs), 0.1, ctypes.byref(od), None) \
        == jpa.JPA_ERR_VALUE
    d0 = jpa.descriptor(kw["q"])
    d0.data = None
    assert lib.jpa_validate(ctypes.byref(d0), *args[1:], 2, P(cq), P(cp), P(cs), 0.1,
                            ctypes.byref(od), None) == jpa.JPA_ERR_NULL
    lse_bad = ctypes.c_void_p(np.zeros(200, np.float32).ctypes.data + 2)
    assert lib.jpa_validate(*args, 2, P(cq), P(cp), P(cs), 0.1, ctypes.byref(od), lse_bad) \
        == jpa.JPA_ERR_LAYOUT
    # jpa_plan rejects what validation rejects and tolerates NULL outputs
    assert lib.jpa_plan(2, P(cq), P(cp), P(cs), 4, 64, None, None) == 0
    bad = np.asarray([0, 7, 6, 10, 12], np.int32)
    assert lib.jpa_plan(2, P(cq), P(cp), P(bad), 4, 64, None, None) == jpa.JPA_ERR_SEGMENTS


def test_scratch_entry_checks_before_the_device():
    """jpa_forward_scratch validates like jpa_forward and rejects a split
    over more key ranges than its static scratch holds, on the host, before
    any device query (so these statuses come back on a machine without a
    GPU as well)."""
    lib = jpa.load_library()
    kw = _valid_call()
    d = [jpa.descriptor(kw[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")]
    od = jpa.descriptor(kw["out"])
    cq, cp, cs = (np.asarray(kw[n], np.int32) for n in ("cu_q", "cu_prefix", "cu_suffix_real"))
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def call(wgs, scale=0.1, lse=None):
        return lib.jpa_forward_scratch(*[ctypes.byref(x) for x in d], 2, P(cq), P(cp), P(cs), scale,
                                       ctypes.byref(od), lse, wgs, None)

    assert call(jpa.SCRATCH_MAX_WGS + 1) == jpa.JPA_ERR_SCRATCH
    assert call(1 << 30) == jpa.JPA_ERR_SCRATCH
    assert call(-1) == jpa.JPA_ERR_VALUE
    assert call(8, scale=float("nan")) == jpa.JPA_ERR_VALUE          # argument errors first
    assert call(jpa.SCRATCH_MAX_WGS + 1, scale=-1.0) == jpa.JPA_ERR_VALUE
    assert "JPA_SCRATCH_MAX_WGS" in jpa.jpa_status_str(jpa.JPA_ERR_SCRATCH)
    m = re.search(r"#define JPA_SCRATCH_MAX_WGS (\d+)", open(HEADER).read())
    assert int(m.group(1)) == jpa.SCRATCH_MAX_WGS
    if not torch.cuda.is_available():
        assert call(8) == jpa.JPA_ERR_HIP


def test_prepared_forward_validates_once_and_reaches_the_launch():
    """PreparedForward marshals the arguments once; a bad call is rejected at
    construction, a good one reaches the launch (JPA_ERR_HIP without a GPU)."""
    kw = _valid_call()
    args = [kw[n] for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix", "cu_q", "cu_prefix",
                            "cu_suffix_real", "scale")]
    lse = torch.zeros(4, kw["q"].shape[0])
    call = jpa.prepare_forward(*args, out=kw["out"], lse=lse, workspace=None, stream=0)
    assert call.out is kw["out"] and call.lse is lse
    if not torch.cuda.is_available():
        with pytest.raises(jpa.JpaError) as e:
            call()
        assert e.value.status == jpa.JPA_ERR_HIP
    bad = list(args)
    bad[8] = float("nan")
    with pytest.raises(jpa.JpaArgumentError):
        jpa.prepare_forward(*bad, out=kw["out"], lse=lse, workspace=None, stream=0)
    with pytest.raises(jpa.JpaArgumentError):
        jpa.prepare_forward(*args, out=kw["q"][:, :2],
                            workspace=None, stream=0, with_lse=False)


def test_kv_token_stride_limit():
    # K/V rows are addressed with a 24-bit multiply of the byte stride: token
    # strides of 2^23 elements or more are rejected (only for K/V tensors).
    lib = jpa.load_library()
    kw = _valid_call()
    d = [jpa.descriptor(kw[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")]
    od = jpa.descriptor(kw["out"])
    cq, cp, cs = (np.asarray(kw[n], np.int32) for n in ("cu_q", "cu_prefix", "cu_suffix_real"))
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def check(which, stride):
        # jpa_validate never dereferences tensor data: each view gets its own
        # 1 TiB-spaced address range, so a huge stride overlaps nothing
        dd = [jpa.descriptor(kw[n], data_ptr=(i + 1) << 40)
              for i, n in enumerate(("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix"))]
        dd[which].token_stride = stride
        o = jpa.descriptor(kw["out"], data_ptr=6 << 40)
        return lib.jpa_validate(*[ctypes.byref(x) for x in dd], 2, P(cq), P(cp), P(cs), 0.1,
                                ctypes.byref(o), None)

    for which in (1, 2, 3, 4):
        assert check(which, (1 << 23) - 8) == jpa.JPA_OK
        assert check(which, 1 << 23) == jpa.JPA_ERR_LAYOUT
    assert check(0, 1 << 23) == jpa.JPA_OK       # queries are not limited


def test_workspace_size_and_errors():
    lib = jpa.load_library()
    # partial outputs [2*wgs][256][D] fp32 + partial LSE [2*wgs][256] fp32
    for d in (64, 128):
        for wgs in (1, 8, 256):
            assert jpa.jpa_workspace_bytes(d, wgs) == 2 * wgs * 256 * d * 4 + 2 * wgs * 256 * 4
    assert jpa.jpa_workspace_bytes(96, 8) == 0
    kw = _valid_call()
    d = [jpa.descriptor(kw[n]) for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")]
    od = jpa.descriptor(kw["out"])
    cq, cp, cs = (np.asarray(kw[n], np.int32) for n in ("cu_q", "cu_prefix", "cu_suffix_real"))
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    need = jpa.jpa_workspace_bytes(64, 8)
    buf = np.zeros(need + 512, np.uint8)
    base = buf.ctypes.data
    aligned = (base + 255) // 256 * 256

    def call(ptr, nbytes, wgs):
        return lib.jpa_forward_ws(*[ctypes.byref(x) for x in d], 2, P(cq), P(cp), P(cs), 0.1,
                                  ctypes.byref(od), None, ctypes.c_void_p(ptr), nbytes, wgs, None)

    assert call(aligned + 16, need, 8) == jpa.JPA_ERR_LAYOUT        # not 256-byte aligned
    assert call(aligned, need - 1, 8) == jpa.JPA_ERR_VALUE          # too small
    assert call(aligned, need, -1) == jpa.JPA_ERR_VALUE             # negative split
    # argument errors come first, before any workspace or device question
    bad = np.asarray([1, 5, 9], np.int32)
    assert lib.jpa_forward_ws(*[ctypes.byref(x) for x in d], 2, P(bad), P(cp), P(cs), 0.1,
                              ctypes.byref(od), None, ctypes.c_void_p(aligned + 16), need, 8,
                              None) == jpa.JPA_ERR_SEGMENTS


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
def test_forward_without_gpu_reports_hip_error():
    kw = _valid_call()
    kw["out"] = torch.zeros_like(kw["q"])
    with pytest.raises(jpa.JpaError) as e:
        jpa.jpa_forward(**kw, lse=torch.zeros(4, kw["q"].shape[0]), stream=0)
    assert e.value.status == jpa.JPA_ERR_HIP


def test_forward_rejects_before_any_launch():
    kw = _valid_call()
    kw["scale"] = -1.0
    with pytest.raises(jpa.JpaArgumentError) as e:
        jpa.jpa_forward(**kw, lse=torch.zeros(4, kw["q"].shape[0]), stream=0)
    assert e.value.status == jpa.JPA_ERR_VALUE


# ---------------------------------------------------------------- jpa_qk_norm_rope

_FAKE = 1 << 20            # 16-byte aligned host-side stand-in; never dereferenced


def _nr_tensor(tokens, heads, d, base=_FAKE, ts=None, hs=None, dtype=jpa.JPA_DTYPE_BF16):
    hs = d if hs is None else hs
    ts = heads * hs if ts is None else ts
    return jpa.JpaTensor(base, tokens, ts, heads, hs, d, dtype)


def _nr_call(q, k, qo, ko, rot=96, il=0, eps=1e-6, wq=_FAKE, wk=_FAKE, table=_FAKE, tstride=96):
    lib = jpa.load_library()
    return lib.jpa_qk_norm_rope(ctypes.byref(q) if q else None, ctypes.byref(k) if k else None,
                                ctypes.c_void_p(wq) if wq else None, ctypes.c_void_p(wk) if wk else None,
                                ctypes.c_void_p(table) if table else None, tstride, rot, il, eps,
                                ctypes.byref(qo) if qo else None, ctypes.byref(ko) if ko else None, None)


def _nr_valid():
    T, hq, hkv, d = 40, 4, 2, 128
    q = _nr_tensor(T, hq, d, base=_FAKE)
    k = _nr_tensor(T, hkv, d, base=_FAKE * 2)
    qo = _nr_tensor(T, hq, d, base=_FAKE * 3)
    ko = _nr_tensor(T, hkv, d, base=_FAKE * 4)
    return q, k, qo, ko


@pytest.mark.parametrize("case,code", [
    ("null_q", jpa.JPA_ERR_NULL), ("null_kout", jpa.JPA_ERR_NULL), ("null_weight", jpa.JPA_ERR_NULL),
    ("null_table", jpa.JPA_ERR_NULL), ("dtype", jpa.JPA_ERR_DTYPE), ("head_dim_96", jpa.JPA_ERR_SHAPE),
    ("tokens_differ", jpa.JPA_ERR_SHAPE), ("out_heads", jpa.JPA_ERR_SHAPE), ("rot_odd", jpa.JPA_ERR_SHAPE),
    ("rot_too_big", jpa.JPA_ERR_SHAPE), ("eps_negative", jpa.JPA_ERR_VALUE), ("eps_nan", jpa.JPA_ERR_VALUE),
    ("interleaved_2", jpa.JPA_ERR_VALUE), ("weight_misaligned", jpa.JPA_ERR_LAYOUT),
    ("table_stride", jpa.JPA_ERR_LAYOUT), ("data_misaligned", jpa.JPA_ERR_LAYOUT),
    ("head_stride_small", jpa.JPA_ERR_LAYOUT), ("out_overlaps_in", jpa.JPA_ERR_LAYOUT),
    ("qout_overlaps_k", jpa.JPA_ERR_LAYOUT), ("outs_overlap", jpa.JPA_ERR_LAYOUT),
    ("fused_views_overlap", jpa.JPA_ERR_LAYOUT),
])
def test_norm_rope_rejects(case, code):
    q, k, qo, ko = _nr_valid()
    kw = {}
    if case == "null_q": q = None
    elif case == "null_kout": ko = None
    elif case == "null_weight": kw["wk"] = 0
    elif case == "null_table": kw["table"] = 0
    elif case == "dtype": k.dtype = 0
    elif case == "head_dim_96":
        q, k, qo, ko = (_nr_tensor(40, h, 96, base=b) for h, b in ((4, _FAKE), (2, 2 * _FAKE), (4, 3 * _FAKE), (2, 4 * _FAKE)))
    elif case == "tokens_differ": k.tokens = 39
    elif case == "out_heads": qo.heads = 3
    elif case == "rot_odd": kw["rot"] = 95
    elif case == "rot_too_big": kw.update(rot=130, tstride=130)
    elif case == "eps_negative": kw["eps"] = -1e-6
    elif case == "eps_nan": kw["eps"] = float("nan")
    elif case == "interleaved_2": kw["il"] = 2
    elif case == "weight_misaligned": kw["wq"] = _FAKE + 4
    elif case == "table_stride": kw["tstride"] = 80
    elif case == "data_misaligned": q.data = _FAKE + 8
    elif case == "head_stride_small": k.head_stride = 120
    elif case == "out_overlaps_in": qo.data = _FAKE + 2 * 128
    elif case == "qout_overlaps_k": qo.data = 2 * _FAKE
    elif case == "outs_overlap": ko.data = 3 * _FAKE + 16
    elif case == "fused_views_overlap":
        # q and k slices of one fused buffer whose column windows meet
        ts = (4 + 2 + 2) * 128
        q = _nr_tensor(40, 4, 128, base=_FAKE, ts=ts)
        k = _nr_tensor(40, 2, 128, base=_FAKE + 2 * 3 * 128, ts=ts)
        qo, ko = q, k
    assert _nr_call(q, k, qo, ko, **kw) == code


def test_norm_rope_empty_is_a_no_op():
    q, k, qo, ko = (_nr_tensor(0, h, 128, base=0) for h in (4, 2, 4, 2))
    assert _nr_call(q, k, qo, ko, table=0) == jpa.JPA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
@pytest.mark.parametrize("case", ["separate", "in_place", "fused_in_place", "no_rotary", "d64_interleaved"])
def test_norm_rope_valid_calls_reach_the_launch(case):
    q, k, qo, ko = _nr_valid()
    kw = {}
    if case == "in_place":
        qo, ko = q, k
    elif case == "fused_in_place":
        ts = (4 + 2 + 2) * 128                 # [T, Hq + 2 Hkv, D] fused QKV, v untouched
        q = _nr_tensor(40, 4, 128, base=_FAKE, ts=ts)
        k = _nr_tensor(40, 2, 128, base=_FAKE + 2 * 4 * 128, ts=ts)
        qo, ko = q, k
    elif case == "no_rotary":
        kw.update(rot=0, table=0, tstride=0)
    elif case == "d64_interleaved":
        q, k, qo, ko = (_nr_tensor(40, h, 64, base=b) for h, b in ((4, _FAKE), (2, 2 * _FAKE), (4, 3 * _FAKE), (2, 4 * _FAKE)))
        kw.update(rot=48, il=1, tstride=48)
    assert _nr_call(q, k, qo, ko, **kw) == jpa.JPA_ERR_HIP


# ---------------------------------------------------------------- jpa_causal_cat_pad

def _cp_call(x=_FAKE, cache=2 * _FAKE, dims=(1, 4, 2, 8, 16), tc=2, pad=(1, 1, 1, 1, 0, 0), out=4 * _FAKE):
    lib = jpa.load_library()
    b, c, t, h, w = dims
    p = (ctypes.c_int32 * 6)(*pad)
    return lib.jpa_causal_cat_pad(ctypes.c_void_p(x) if x else None, ctypes.c_void_p(cache) if cache else None,
                                  b, c, t, tc, h, w, p, ctypes.c_void_p(out) if out else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=0), jpa.JPA_ERR_NULL), (dict(x=0), jpa.JPA_ERR_NULL), (dict(cache=0), jpa.JPA_ERR_NULL),
    (dict(pad=(1, -1, 1, 1, 0, 0)), jpa.JPA_ERR_VALUE), (dict(dims=(1, 4, -2, 8, 16)), jpa.JPA_ERR_SHAPE),
    (dict(dims=(1, 4, 2, 8, 70000)), jpa.JPA_ERR_SHAPE), (dict(dims=(64, 1024, 64, 256, 256)), jpa.JPA_ERR_SHAPE),
    (dict(x=_FAKE + 8), jpa.JPA_ERR_LAYOUT), (dict(out=_FAKE + 64), jpa.JPA_ERR_LAYOUT),
    (dict(out=2 * _FAKE + 32), jpa.JPA_ERR_LAYOUT),
])
def test_cat_pad_rejects(kw, code):
    assert _cp_call(**kw) == code


def test_cat_pad_empty_and_uncached():
    assert _cp_call(dims=(0, 4, 2, 8, 16), x=0, cache=0, out=0) == jpa.JPA_OK
    if not torch.cuda.is_available():
        assert _cp_call(cache=0, tc=0) == jpa.JPA_ERR_HIP       # valid call reaches the launch
