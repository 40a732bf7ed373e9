"""The C shard planner (include/jpa_shard.h) against the shard-plan oracle,
bit for bit, over a faked world of ranks (every rank of every world size is
planned in one process, like the page's _fake_sp tests); its error paths; and
that the offsets it emits pass jpa_forward's own validation.
(sglang PR #30107 review: build_shard_plan, SpShard, tail_attn_meta.)"""

import numpy as np
import pytest

import oracle
from diffusion_transformer_joint_non_amd import jpa

LENS = [0, 1, 2, 3, 5, 7, 15, 16, 17, 77, 511, 512, 4095, 4096, 8190, 32760, 75600, 1_000_003]
WORLDS = [1, 2, 3, 4, 5, 7, 8, 16]


@pytest.mark.parametrize("sp_size", WORLDS)
def test_plan_matches_oracle_for_every_rank(sp_size):
    for n in LENS:
        for r in range(sp_size):
            c = jpa.jpa_shard_plan(n, sp_size, r)
            o = oracle.build_shard_plan(n, sp_size, r)
            got = (c.orig_len, c.local_len, c.num_pad, c.sp_size, c.sp_rank, c.local_pad, c.local_real_len)
            want = (o.orig_len, o.local_len, o.num_pad, o.sp_size, o.sp_rank, o.local_pad, o.local_real_len)
            assert got == want, (n, sp_size, r)
            for m in (1, 2, 16):
                assert jpa.jpa_tail_attn_meta(c, m) == oracle.tail_attn_meta(o, m)


@pytest.mark.parametrize("n,sp_size,m,prefixes,qp", [
    (4096, 8, 1, [512], True), (4095, 8, 1, [512], True), (8190, 4, 1, [77, 512], True),
    (32760, 8, 1, [1024], False), (75600, 8, 1, [256], False), (5, 4, 3, [8, 0, 3], False),
    (1, 4, 16, [4, 4], True), (0, 2, 1, [3], True), (100, 3, 2, [], False),
])
def test_segments_match_oracle(n, sp_size, m, prefixes, qp):
    for r in range(sp_size):
        c = jpa.jpa_tail_segments(jpa.jpa_shard_plan(n, sp_size, r), m, prefixes, qp)
        o = oracle.tail_segments(oracle.build_shard_plan(n, sp_size, r), m, prefixes, qp)
        for a, b in zip(c, o):
            assert list(a) == list(b)


def test_segments_pass_forward_validation():
    """Offsets of every rank of a 4-way split of the Cosmos-like suffix form a
    valid jpa_forward call (host check only; no device touched)."""
    import torch
    for r in range(4):
        sh = jpa.jpa_shard_plan(32760, 4, r)
        cu_q, cu_p, cu_s = jpa.jpa_tail_segments(sh, 1, [1024], False)
        tq, tp, ts = int(cu_q[-1]), int(cu_p[-1]), int(cu_s[-1])
        mk = lambda t, h: torch.empty((t, h, 128), dtype=torch.bfloat16)
        q, kp, ks = mk(tq, 8), mk(tp, 8), mk(ts, 8)
        assert jpa.jpa_validate(q, kp, kp, ks, ks, cu_q, cu_p, cu_s, 128 ** -0.5, torch.empty_like(q)) == jpa.JPA_OK
        rows, _ = jpa.jpa_plan(cu_q, cu_p, cu_s, 8, 128)
        assert rows[0][6] == sh.local_real_len and rows[0][7] == sh.local_pad


def test_errors():
    import ctypes
    lib = jpa.load_library()
    out = jpa.JpaShard()
    assert lib.jpa_shard_plan(10, 4, 4, ctypes.byref(out)) == jpa.JPA_ERR_VALUE
    assert lib.jpa_shard_plan(10, 0, 0, ctypes.byref(out)) == jpa.JPA_ERR_VALUE
    assert lib.jpa_shard_plan(-1, 2, 0, ctypes.byref(out)) == jpa.JPA_ERR_VALUE
    assert lib.jpa_shard_plan(10, 2, 0, None) == jpa.JPA_ERR_NULL
    sh = jpa.jpa_shard_plan(100, 4, 1)
    with pytest.raises(jpa.JpaArgumentError):
        jpa.jpa_tail_attn_meta(sh, 0)
    with pytest.raises(jpa.JpaArgumentError):
        jpa.jpa_tail_segments(sh, 1, [-1], True)
    with pytest.raises(jpa.JpaArgumentError) as e:
        jpa.jpa_tail_segments(jpa.jpa_shard_plan(2**31, 1, 0), 1, [0], True)
    assert e.value.status == jpa.JPA_ERR_SEGMENTS
