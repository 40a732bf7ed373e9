"""Pins for the shard-plan oracle (oracle/shard_plan.py), none of which re-runs
its own formulas:

* brute force: the padded global sequence materialised as a list (real
  tokens, then the pad block) and cut into sp_size equal chunks;
* the page's SpShard property (all pad on the last rank) wherever it holds,
  num_pad <= local_len, and the review's degenerate case seq_len = 1,
  sp_size = 4;
* sums over a faked world of ranks (like the page's _fake_sp tests);
* the segment offsets decode, through the attention oracle's own decoder and
  the seeded workload builder, to the rows they describe;
* planted mistakes are caught.
(sglang PR #30107 review: sp_shard_utils, build_shard_plan, tail_attn_meta.)
"""

import importlib

import numpy as np
import pytest

import oracle
import synth

sp = importlib.import_module("oracle.shard_plan")
PAD = -1

SWEEP = [(n, s) for n in (0, 1, 2, 3, 5, 7, 16, 31, 77, 512, 4095, 4096, 32760) for s in (1, 2, 3, 4, 8)]


def _brute(seq_len, sp_size):
    local = -(-seq_len // sp_size) if sp_size > 1 else seq_len
    glob = list(range(seq_len)) + [PAD] * (local * sp_size - seq_len)
    return [glob[r * local:(r + 1) * local] for r in range(sp_size)]


def _check_brute(seq_len, sp_size):
    chunks = _brute(seq_len, sp_size)
    for r, chunk in enumerate(chunks):
        s = sp.build_shard_plan(seq_len, sp_size, r)
        if s.local_len != len(chunk) or s.local_pad != chunk.count(PAD):
            return False
        if s.local_real_len != len(chunk) - chunk.count(PAD):
            return False
        if PAD in chunk and chunk.index(PAD) != s.local_real_len:      # [valid | pad] per rank
            return False
        if s.num_pad != sum(c.count(PAD) for c in chunks):
            return False
    return True


@pytest.mark.parametrize("seq_len,sp_size", SWEEP)
def test_brute_force(seq_len, sp_size):
    assert _check_brute(seq_len, sp_size)


def test_page_formula_where_it_holds():
    for n, s in SWEEP:
        for r in range(s):
            sh = sp.build_shard_plan(n, s, r)
            if sh.num_pad <= sh.local_len:
                assert sh.local_pad == (sh.num_pad if r == s - 1 else 0)


def test_degenerate_case():
    plans = [sp.build_shard_plan(1, 4, r) for r in range(4)]
    assert [p.local_len for p in plans] == [1, 1, 1, 1]
    assert [p.num_pad for p in plans] == [3, 3, 3, 3]
    assert [p.local_real_len for p in plans] == [1, 0, 0, 0]
    assert [p.local_pad for p in plans] == [0, 1, 1, 1]
    for p in plans:
        meta = sp.tail_attn_meta(p, 1)
        assert meta["max_seqlen_tail"] >= p.num_pad and meta["valid_len"] == p.local_real_len


def test_world_sums():
    for n, s in SWEEP:
        plans = [sp.build_shard_plan(n, s, r) for r in range(s)]
        assert sum(p.local_real_len for p in plans) == n
        assert sum(p.local_pad for p in plans) == plans[0].num_pad
        assert all(p.local_real_len >= 0 and p.local_pad >= 0 for p in plans)
        assert plans[0].num_pad < max(s, 1)


def test_no_pad_means_no_meta():
    assert sp.tail_attn_meta(sp.build_shard_plan(4096, 1, 0), 1) is None
    assert sp.tail_attn_meta(sp.build_shard_plan(4096, 8, 3), 2) is None
    m = sp.tail_attn_meta(sp.build_shard_plan(4095, 8, 7), 2)
    assert m == {"tail": True, "valid_len": 2 * 511, "max_seqlen_tail": 2 * 511}


def _check_segments(seq_len, sp_size, rank, mult, prefixes, qp):
    s = sp.build_shard_plan(seq_len, sp_size, rank)
    cu_q, cu_p, cu_s = sp.tail_segments(s, mult, prefixes, qp)
    rows = oracle.decode_segments(np.asarray(cu_q), np.asarray(cu_p), np.asarray(cu_s))
    w = synth.custom_workload(1, 1, 64, prefixes, [s.local_real_len * mult] * len(prefixes),
                              [s.local_pad * mult] * len(prefixes),
                              "prefix+suffix" if qp else "suffix")
    same = (list(w.cu_q()) == list(cu_q) and list(w.cu_prefix()) == list(cu_p)
            and list(w.cu_suffix_real()) == list(cu_s))
    ok = all(r.p_len == p and r.s_real == s.local_real_len * mult and r.s_pad == s.local_pad * mult
             for r, p in zip(rows, prefixes))
    return same and ok


@pytest.mark.parametrize("seq_len,sp_size,rank,mult,prefixes,qp", [
    (4096, 8, 7, 1, [512], True), (4095, 8, 7, 1, [512], True), (4095, 8, 0, 1, [77, 512], True),
    (32760, 4, 3, 1, [1024], False), (5, 4, 2, 3, [8, 0, 3], False), (1, 4, 3, 16, [4], True),
])
def test_segments_decode_to_the_rows(seq_len, sp_size, rank, mult, prefixes, qp):
    assert _check_segments(seq_len, sp_size, rank, mult, prefixes, qp)


# ---------------------------------------------------------------- planted mistakes

def _pins_hold():
    try:
        for n, s in SWEEP:
            if not _check_brute(n, s):
                return False
        test_degenerate_case()
        test_world_sums()
        test_no_pad_means_no_meta()
        if not _check_segments(4095, 8, 7, 1, [512], True) or not _check_segments(5, 4, 2, 3, [8, 0, 3], False):
            return False
    except (AssertionError, ValueError, IndexError, TypeError):
        return False
    return True


_orig_plan = sp.build_shard_plan
_orig_meta = sp.tail_attn_meta
_orig_segs = sp.tail_segments


def _mut_floor(seq_len, sp_size, sp_rank):
    s = _orig_plan(seq_len, sp_size, sp_rank)
    local = seq_len // sp_size if sp_size > 1 else seq_len
    return sp.Shard(seq_len, local, 0, sp_size, sp_rank, 0, local)


def _mut_all_pad_last(seq_len, sp_size, sp_rank):
    s = _orig_plan(seq_len, sp_size, sp_rank)
    pad = s.num_pad if sp_rank == sp_size - 1 else 0
    return sp.Shard(s.orig_len, s.local_len, s.num_pad, sp_size, sp_rank, pad, s.local_len - pad)


def _mut_pad_first_rank(seq_len, sp_size, sp_rank):
    s = _orig_plan(seq_len, sp_size, sp_rank)
    pad = s.num_pad if sp_rank == 0 and sp_size > 1 else 0
    return sp.Shard(s.orig_len, s.local_len, s.num_pad, sp_size, sp_rank, pad, s.local_len - pad)


def _mut_meta_no_max(shard, m):
    r = _orig_meta(shard, m)
    if r is not None:
        r["max_seqlen_tail"] = r["valid_len"]
    return r


def _mut_segments_pad_as_real(shard, m, prefixes, qp):
    cu_q, cu_p, cu_s = _orig_segs(shard, m, prefixes, qp)
    cu_s = [cu_s[0]] + [cu_s[2 * i + 2] for i in range(len(prefixes)) for _ in (0, 1)]
    return cu_q, cu_p, cu_s


def _mut_segments_no_prefix_queries(shard, m, prefixes, qp):
    return _orig_segs(shard, m, prefixes, False)


MUTANTS = [
    ("build_shard_plan", _mut_floor),
    ("build_shard_plan", _mut_all_pad_last),
    ("build_shard_plan", _mut_pad_first_rank),
    ("tail_attn_meta", _mut_meta_no_max),
    ("tail_segments", _mut_segments_pad_as_real),
    ("tail_segments", _mut_segments_no_prefix_queries),
]


def test_pins_hold_on_the_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(sp, name, mutant)
    assert not _pins_hold()
