"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never uses it and
the two share no code.
"""

from .fp64 import (  # noqa: F401
    RowSegments,
    attention,
    attention_rows,
    compare,
    decode_segments,
    kv_head,
    lse_merge,
    row_kv,
    softmax_attention,
    valid_flops,
    widen,
)
from .qk_norm_rope import (  # noqa: F401
    apply_rope,
    qk_norm_rope,
    rms_norm,
    rope_pairs,
)
from .shard_plan import (  # noqa: F401
    Shard,
    build_shard_plan,
    tail_attn_meta,
    tail_segments,
)
from .cat_pad import cat_pad, out_shape  # noqa: F401
