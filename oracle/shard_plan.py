"""Plain Python oracle for the sequence-parallel tail-pad shard plan and the
attention segment offsets it implies.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the library.

Written from sglang PR #30107's review (the sp_shard_utils module: the
SpShard facts, build_shard_plan, tail_attn_meta, and the layout invariant in
its docstring):

* a sequence of seq_len real tokens is split evenly over sp_size ranks:
  local_len = ceil(seq_len / sp_size) per rank, num_pad = local_len * sp_size
  - seq_len pad tokens in total;
* layout invariant: the gathered sequence is the real tokens followed by one
  contiguous pad block at its global tail;
* per rank: local_pad pad rows, local_real_len = local_len - local_pad real
  rows; the attention of a rank sees each batch row as [valid | pad] with
  valid = local_real_len * seqlen_multiplier (tail_attn_meta), and the pad as
  its own segment (implementation item 4);
* tail_attn_meta's max_seqlen_tail is max(valid, num_pad) (the review's fix
  for the FlashAttention contract); no metadata when there is no pad.

Reading where the page is at odds with itself: the SpShard property puts all
num_pad pad rows on the last rank, which is what the invariant gives only
while num_pad <= local_len.  When num_pad > local_len (e.g. the review's
degenerate test case seq_len = 1, sp_size = 4, or seq_len = 5, sp_size = 4)
the tail block covers more than the last chunk; this oracle follows the
invariant: a rank's pad rows are its chunk's overlap with the global tail
block [seq_len, local_len * sp_size).  Both agree whenever num_pad <= local_len.

Every function below is pinned by ``tests/test_oracle_shard_plan.py``.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Shard:
    orig_len: int
    local_len: int
    num_pad: int
    sp_size: int
    sp_rank: int
    local_pad: int
    local_real_len: int


def build_shard_plan(seq_len: int, sp_size: int, sp_rank: int) -> Shard:
    """Even tail-padded shard of seq_len tokens for rank sp_rank of sp_size."""
    if seq_len < 0 or sp_size < 1 or not 0 <= sp_rank < sp_size:
        raise ValueError("bad shard arguments")
    if sp_size == 1:
        return Shard(seq_len, seq_len, 0, 1, 0, 0, seq_len)
    local_len = -(-seq_len // sp_size)
    num_pad = local_len * sp_size - seq_len
    start, end = sp_rank * local_len, (sp_rank + 1) * local_len
    local_pad = max(0, end - max(start, seq_len))          # overlap with [seq_len, local_len * sp_size)
    return Shard(seq_len, local_len, num_pad, sp_size, sp_rank, local_pad, local_len - local_pad)


def tail_attn_meta(shard: Shard, seqlen_multiplier: int):
    """None without pad, else the valid length and the safe max_seqlen of the tail."""
    if shard.num_pad == 0:
        return None
    valid = shard.local_real_len * seqlen_multiplier
    return {"tail": True, "valid_len": valid, "max_seqlen_tail": max(valid, shard.num_pad)}


def tail_segments(shard: Shard, seqlen_multiplier: int, prefix_lens, queries_include_prefix: bool):
    """Offsets of the attention call of one rank: every batch row b has a
    prefix of prefix_lens[b] tokens and a suffix of local_len * m slots whose
    last local_pad * m are pad.  Returns (cu_q, cu_prefix, cu_suffix_real)."""
    m = seqlen_multiplier
    slots = shard.local_len * m
    real = shard.local_real_len * m
    cu_q, cu_p, cu_s = [0], [0], [0]
    for p in prefix_lens:
        cu_q.append(cu_q[-1] + slots + (p if queries_include_prefix else 0))
        cu_p.append(cu_p[-1] + p)
        cu_s.append(cu_s[-1] + real)
        cu_s.append(cu_s[-2] + slots)
    return cu_q, cu_p, cu_s
