"""Thin ctypes binding over libjpa's C ABI (include/jpa.h,
include/jpa_norm_rope.h, include/jpa_shard.h and include/jpa_cat_pad.h), same
names.

Argument marshalling only: every step of the attention runs in the HIP
library.  PyTorch supplies device memory and the current stream; nothing else
is used from it.  If the library is not built this module raises on load --
there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libjpa.so")
STRICT_LIB_PATH = os.path.join(os.path.dirname(_LIB_PATH), "libjpa_strict_waits.so")

JPA_OK = 0
JPA_ERR_NULL = 1
JPA_ERR_DTYPE = 2
JPA_ERR_SHAPE = 3
JPA_ERR_LAYOUT = 4
JPA_ERR_SEGMENTS = 5
JPA_ERR_VALUE = 6
JPA_ERR_HIP = 7
JPA_ERR_SCRATCH = 8
SCRATCH_MAX_WGS = 256  # JPA_SCRATCH_MAX_WGS
JPA_DTYPE_BF16 = 1
BLOCK_M = 256          # query rows per workgroup (for launch accounting only)

EXPORTED = ("jpa_forward", "jpa_forward_ws", "jpa_forward_scratch", "jpa_workspace_bytes", "jpa_validate", "jpa_plan",
            "jpa_status_str", "jpa_abi_version", "jpa_qk_norm_rope", "jpa_shard_plan",
            "jpa_tail_attn_meta", "jpa_tail_segments", "jpa_causal_cat_pad")


class JpaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("tokens", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("head_stride", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class JpaShard(ctypes.Structure):
    _fields_ = [("orig_len", ctypes.c_int64), ("local_len", ctypes.c_int64), ("num_pad", ctypes.c_int64),
                ("sp_size", ctypes.c_int32), ("sp_rank", ctypes.c_int32), ("local_pad", ctypes.c_int64),
                ("local_real_len", ctypes.c_int64)]


class JpaRowPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "q_start", "q_slots", "q_real", "prefix_start", "prefix_len",
        "suffix_start", "suffix_real", "suffix_pad", "keys")]

    def as_tuple(self):
        return tuple(getattr(self, n) for n, _ in self._fields_)


class JpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class JpaArgumentError(JpaError, ValueError):
    pass


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the in-tree libjpa.so (built by ``python -m
    diffusion_transformer_joint_non_amd.build``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(_LIB_PATH)
    return _lib


def load_strict_waits_library() -> ctypes.CDLL:
    """The check build of the same sources (JPA_STRICT_WAITS: the attention
    kernel waits for every tile copy at each barrier), for tests that compare
    it bit for bit with libjpa.so.  Nothing in this module calls it."""
    return _open(STRICT_LIB_PATH)


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{os.path.basename(path)} not found at {path}; build it with "
            "`python -m diffusion_transformer_joint_non_amd.build`")
    # Bind to the HIP runtime PyTorch uses: torch ships its own libamdhip64,
    # and the library's dependency on that soname resolves to whichever copy
    # is loaded first.  Loaded before torch, the library would bring in a
    # second runtime, and its calls would not see torch's device state.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    tp = ctypes.POINTER(JpaTensor)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.jpa_forward.restype = ctypes.c_int
    lib.jpa_forward.argtypes = [tp, tp, tp, tp, tp, ctypes.c_int32, i32p, i32p, i32p,
                                ctypes.c_float, tp, ctypes.c_void_p, ctypes.c_void_p]
    lib.jpa_forward_ws.restype = ctypes.c_int
    lib.jpa_forward_ws.argtypes = [tp, tp, tp, tp, tp, ctypes.c_int32, i32p, i32p, i32p,
                                   ctypes.c_float, tp, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    lib.jpa_forward_scratch.restype = ctypes.c_int
    lib.jpa_forward_scratch.argtypes = [tp, tp, tp, tp, tp, ctypes.c_int32, i32p, i32p, i32p,
                                        ctypes.c_float, tp, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p]
    lib.jpa_workspace_bytes.restype = ctypes.c_size_t
    lib.jpa_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.jpa_validate.restype = ctypes.c_int
    lib.jpa_validate.argtypes = [tp, tp, tp, tp, tp, ctypes.c_int32, i32p, i32p, i32p,
                                 ctypes.c_float, tp, ctypes.c_void_p]
    lib.jpa_plan.restype = ctypes.c_int
    lib.jpa_plan.argtypes = [ctypes.c_int32, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                             ctypes.POINTER(JpaRowPlan), ctypes.POINTER(ctypes.c_int64)]
    lib.jpa_status_str.restype = ctypes.c_char_p
    lib.jpa_status_str.argtypes = [ctypes.c_int]
    lib.jpa_abi_version.restype = ctypes.c_int32
    lib.jpa_abi_version.argtypes = []
    sp = ctypes.POINTER(JpaShard)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.jpa_shard_plan.restype = ctypes.c_int
    lib.jpa_shard_plan.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, sp]
    lib.jpa_tail_attn_meta.restype = ctypes.c_int
    lib.jpa_tail_attn_meta.argtypes = [sp, ctypes.c_int32, i32p, i64p, i64p]
    lib.jpa_tail_segments.restype = ctypes.c_int
    lib.jpa_tail_segments.argtypes = [sp, ctypes.c_int32, ctypes.c_int32, i32p, ctypes.c_int32, i32p, i32p, i32p]
    vp = ctypes.c_void_p
    lib.jpa_causal_cat_pad.restype = ctypes.c_int
    lib.jpa_causal_cat_pad.argtypes = [vp, vp] + [ctypes.c_int32] * 6 + [i32p, vp, vp]
    lib.jpa_qk_norm_rope.restype = ctypes.c_int
    lib.jpa_qk_norm_rope.argtypes = [tp, tp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, tp, tp, vp]
    return lib


def jpa_status_str(status: int) -> str:
    return load_library().jpa_status_str(int(status)).decode()


def jpa_abi_version() -> int:
    return int(load_library().jpa_abi_version())


def _raise_for(status: int):
    if status == JPA_OK:
        return
    msg = jpa_status_str(status)
    if status == JPA_ERR_HIP:
        raise JpaError(status, msg)
    raise JpaArgumentError(status, msg)


def _i32(arr) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int64))
    if a.size and (a.min() < -2**31 or a.max() >= 2**31):
        raise ValueError("offsets must fit in int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def descriptor(t, data_ptr: Optional[int] = None) -> JpaTensor:
    """jpa_tensor for a [tokens, heads, head_dim] bf16 torch tensor (or view)."""
    import torch
    if t.dim() != 3:
        raise ValueError("expected a [tokens, heads, head_dim] tensor")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError("head_dim must be contiguous")
    dtype = JPA_DTYPE_BF16 if t.dtype == torch.bfloat16 else 0
    return JpaTensor(t.data_ptr() if data_ptr is None else data_ptr, t.shape[0], t.stride(0),
                     t.shape[1], t.stride(1), t.shape[2], dtype)


def jpa_plan(cu_q: Sequence[int], cu_prefix: Sequence[int], cu_suffix_real: Sequence[int],
             heads_q: int, head_dim: int):
    """Per-row bookkeeping (list of 9-tuples, see jpa_row_plan) and the int64
    valid-token FLOP count, decoded by the C library on the host."""
    lib = load_library()
    cq, cp, cs = _i32(cu_q), _i32(cu_prefix), _i32(cu_suffix_real)
    batch = max(cq.size - 1, 0)
    if cp.size != batch + 1 or cs.size != 2 * batch + 1:
        raise JpaArgumentError(JPA_ERR_SEGMENTS, "offset arrays must have B+1, B+1, 2B+1 entries")
    rows = (JpaRowPlan * max(batch, 1))()
    flops = ctypes.c_int64(0)
    _raise_for(lib.jpa_plan(batch, _i32p(cq), _i32p(cp), _i32p(cs), int(heads_q), int(head_dim),
                            rows, ctypes.byref(flops)))
    return [rows[b].as_tuple() for b in range(batch)], int(flops.value)


def _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real):
    cq, cp, cs = _i32(cu_q), _i32(cu_prefix), _i32(cu_suffix_real)
    batch = max(cq.size - 1, 0)
    if cp.size != batch + 1 or cs.size != 2 * batch + 1:
        raise JpaArgumentError(JPA_ERR_SEGMENTS, "offset arrays must have B+1, B+1, 2B+1 entries")
    descs = [descriptor(t) for t in (q, k_prefix, v_prefix, k_suffix, v_suffix)]
    return cq, cp, cs, batch, descs


def jpa_validate(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real,
                 scale: float, out, lse=None) -> int:
    """Host-only check of a jpa_forward call; returns the jpa_status code."""
    lib = load_library()
    cq, cp, cs, batch, d = _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                                   cu_suffix_real)
    od = descriptor(out)
    return lib.jpa_validate(*[ctypes.byref(x) for x in d], batch, _i32p(cq), _i32p(cp), _i32p(cs),
                            float(scale), ctypes.byref(od),
                            None if lse is None else ctypes.c_void_p(lse.data_ptr()))


def jpa_workspace_bytes(head_dim: int, split_wgs: int = 0) -> int:
    """Workspace bytes jpa_forward_ws needs (split_wgs 0: the current device's
    compute units); 0 if head_dim is unsupported or the device unknown."""
    return int(load_library().jpa_workspace_bytes(int(head_dim), int(split_wgs)))


_workspaces = {}


def workspace_for(device, stream_handle: int, head_dim: int = 128, split_wgs: int = 0):
    """A workspace for jpa_forward_ws, cached per (device, stream, split_wgs,
    head_dim): calls on one stream are ordered, so they may share it (its
    contents do not matter between calls)."""
    import torch
    dev = torch.device(device)
    key = (dev.index, int(stream_handle), int(split_wgs), int(head_dim))
    ws = _workspaces.get(key)
    if ws is None:
        n = jpa_workspace_bytes(head_dim, split_wgs)
        if n == 0:
            raise JpaError(JPA_ERR_HIP, "cannot size the workspace for this device")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _prepare(q, out, lse, with_lse, stream):
    import torch
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and with_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[1], q.shape[0])):
        raise JpaArgumentError(JPA_ERR_SHAPE, "lse must be contiguous fp32 [Hq, Tq]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return out, lse, handle


def jpa_forward_ws(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real,
                   scale: float, out=None, lse=None, stream=None, with_lse: bool = True,
                   workspace="auto", split_wgs: int = 0):
    """jpa_forward with a workspace that balances the last round of work over
    every compute unit.  ``workspace``: "auto" (a cached buffer
    per device and stream), a uint8 CUDA tensor of at least
    jpa_workspace_bytes() bytes (contents do not matter), or None (then the
    call is jpa_forward's).  Returns (out, lse)."""
    lib = load_library()
    cq, cp, cs, batch, d = _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                                   cu_suffix_real)
    out, lse, handle = _prepare(q, out, lse, with_lse, stream)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", a tensor or None')
        workspace = workspace_for(q.device, handle, q.shape[2], split_wgs)
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    od = descriptor(out)
    st = lib.jpa_forward_ws(*[ctypes.byref(x) for x in d], batch, _i32p(cq), _i32p(cp), _i32p(cs),
                            float(scale), ctypes.byref(od),
                            None if lse is None else ctypes.c_void_p(lse.data_ptr()),
                            ws_ptr, ws_bytes, int(split_wgs), ctypes.c_void_p(handle))
    _raise_for(st)
    return out, lse


def jpa_forward_scratch(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real,
                        scale: float, out, lse=None, stream=None, split_wgs: int = 0):
    """jpa_forward_ws with the library's static device scratch in place of a
    workspace: the C call allocates nothing (for callers that cannot).  out
    (and lse, if wanted) must be given.  Calls that may overlap on one device
    race on the shared scratch.  Returns (out, lse)."""
    lib = load_library()
    if out is None:
        raise ValueError("jpa_forward_scratch writes into a given out (it allocates nothing)")
    cq, cp, cs, batch, d = _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                                   cu_suffix_real)
    out, lse, handle = _prepare(q, out, lse, False, stream)
    od = descriptor(out)
    st = lib.jpa_forward_scratch(*[ctypes.byref(x) for x in d], batch, _i32p(cq), _i32p(cp), _i32p(cs),
                                 float(scale), ctypes.byref(od),
                                 None if lse is None else ctypes.c_void_p(lse.data_ptr()),
                                 int(split_wgs), ctypes.c_void_p(handle))
    _raise_for(st)
    return out, lse


def jpa_forward(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real,
                scale: float, out=None, lse=None, stream=None, with_lse: bool = True):
    """Enqueue the attention on ``stream`` (default: torch's current stream).

    q [Tq, Hq, D], k/v prefix [Tp, Hkv, D], k/v suffix [Ts, Hkv, D]: bf16 CUDA
    (HIP) tensors or views with contiguous head_dim.  cu_* are host offsets
    (lists, numpy arrays or CPU tensors).  Returns (out, lse); out/lse are
    allocated here only when not given."""
    lib = load_library()
    cq, cp, cs, batch, d = _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                                   cu_suffix_real)
    out, lse, handle = _prepare(q, out, lse, with_lse, stream)
    od = descriptor(out)
    st = lib.jpa_forward(*[ctypes.byref(x) for x in d], batch, _i32p(cq), _i32p(cp), _i32p(cs),
                         float(scale), ctypes.byref(od),
                         None if lse is None else ctypes.c_void_p(lse.data_ptr()),
                         ctypes.c_void_p(handle))
    _raise_for(st)
    return out, lse


class PreparedForward:
    """One attention call with every argument marshalled once: descriptors,
    int32 offsets and the output buffers are built at construction, so each
    call only enqueues (jpa_forward_ws through ctypes with the prebuilt
    argument tuple).  For repeated calls on the same tensors, e.g. one DiT
    layer over denoising steps (vLLM-Omni performance-patterns guide: hoist
    request invariants out of the per-step path).  The tensors must stay
    alive and keep their shapes and storage; their contents may change
    between calls.  Validation runs once here, and again in the library on
    every call (host only)."""

    def __init__(self, q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix, cu_suffix_real,
                 scale: float, out=None, lse=None, with_lse: bool = True, workspace="auto",
                 split_wgs: int = 0, stream=None):
        import torch
        lib = load_library()
        cq, cp, cs, batch, d = _common(q, k_prefix, v_prefix, k_suffix, v_suffix, cu_q, cu_prefix,
                                       cu_suffix_real)
        out, lse, handle = _prepare(q, out, lse, with_lse, stream)
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", a tensor or None')
            workspace = workspace_for(q.device, handle, q.shape[2], split_wgs)
        self.out, self.lse = out, lse
        self._keep = (q, k_prefix, v_prefix, k_suffix, v_suffix, cq, cp, cs, workspace)
        self._descs = d + [descriptor(out)]
        self._fn = lib.jpa_forward_ws
        ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._head = (*[ctypes.byref(x) for x in d], batch, _i32p(cq), _i32p(cp), _i32p(cs),
                      ctypes.c_float(scale), ctypes.byref(self._descs[5]),
                      None if lse is None else ctypes.c_void_p(lse.data_ptr()),
                      ws_ptr, ctypes.c_size_t(ws_bytes), ctypes.c_int32(int(split_wgs)))
        self._stream = ctypes.c_void_p(handle)
        _raise_for(lib.jpa_validate(*self._head[:12]))

    def __call__(self, stream=None):
        """Enqueue the call on `stream` (default: the stream given at
        construction, else torch's current stream then).  Returns (out, lse)."""
        s = self._stream if stream is None else ctypes.c_void_p(
            stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
        st = self._fn(*self._head, s)
        if st:
            _raise_for(st)
        return self.out, self.lse


def prepare_forward(*args, **kwargs) -> PreparedForward:
    """PreparedForward(...): jpa_forward_ws's arguments marshalled once."""
    return PreparedForward(*args, **kwargs)


def jpa_qk_norm_rope(q, k, q_weight, k_weight, table, rotary_dim: int, interleaved: bool, eps: float,
                     q_out=None, k_out=None, stream=None):
    """Per-head RMSNorm of q [T, Hq, D] and k [T, Hkv, D] (bf16 CUDA tensors
    or views) with float32 weights [D], then the rotary embedding from the
    float32 table [T, >= rotary_dim] = [cos | sin] (interleaved or half-split
    pairs).  q_out/k_out: outputs (allocated when None; pass q/k for in
    place).  Returns (q_out, k_out)."""
    import torch
    lib = load_library()
    for name, w in (("q_weight", q_weight), ("k_weight", k_weight)):
        if w.dtype != torch.float32 or w.dim() != 1 or not w.is_contiguous():
            raise JpaArgumentError(JPA_ERR_SHAPE, f"{name} must be a contiguous float32 [head_dim]")
        if w.shape[0] != q.shape[2]:
            raise JpaArgumentError(JPA_ERR_SHAPE, f"{name} must have head_dim entries")
    table_ptr, table_stride = None, 0
    if table is not None and rotary_dim > 0:
        if table.dtype != torch.float32 or table.dim() != 2 or table.stride(1) != 1:
            raise JpaArgumentError(JPA_ERR_SHAPE, "table must be float32 [T, >= rotary_dim], rows contiguous")
        if table.shape[0] != q.shape[0] or table.shape[1] < rotary_dim:
            raise JpaArgumentError(JPA_ERR_SHAPE, "table must be [T, >= rotary_dim]")
        table_ptr, table_stride = ctypes.c_void_p(table.data_ptr()), table.stride(0)
    if q_out is None:
        q_out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if k_out is None:
        k_out = torch.empty_like(k, memory_format=torch.contiguous_format)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    d = [descriptor(x) for x in (q, k, q_out, k_out)]
    st = lib.jpa_qk_norm_rope(ctypes.byref(d[0]), ctypes.byref(d[1]), ctypes.c_void_p(q_weight.data_ptr()),
                              ctypes.c_void_p(k_weight.data_ptr()), table_ptr, int(table_stride),
                              int(rotary_dim), 1 if interleaved else 0, float(eps),
                              ctypes.byref(d[2]), ctypes.byref(d[3]), ctypes.c_void_p(handle))
    _raise_for(st)
    return q_out, k_out


def jpa_shard_plan(seq_len: int, sp_size: int, sp_rank: int) -> JpaShard:
    """Tail-padded even shard facts of rank sp_rank (host only)."""
    lib = load_library()
    out = JpaShard()
    _raise_for(lib.jpa_shard_plan(int(seq_len), int(sp_size), int(sp_rank), ctypes.byref(out)))
    return out


def jpa_tail_attn_meta(shard: JpaShard, seqlen_multiplier: int = 1):
    """None without pad, else {"tail", "valid_len", "max_seqlen_tail"}."""
    lib = load_library()
    has = ctypes.c_int32()
    valid = ctypes.c_int64()
    mx = ctypes.c_int64()
    _raise_for(lib.jpa_tail_attn_meta(ctypes.byref(shard), int(seqlen_multiplier), ctypes.byref(has),
                                      ctypes.byref(valid), ctypes.byref(mx)))
    if not has.value:
        return None
    return {"tail": True, "valid_len": valid.value, "max_seqlen_tail": mx.value}


def jpa_tail_segments(shard: JpaShard, seqlen_multiplier: int, prefix_lens, queries_include_prefix: bool):
    """(cu_q, cu_prefix, cu_suffix_real) int32 arrays of one rank's attention call."""
    lib = load_library()
    pl = _i32(prefix_lens)
    b = int(pl.size)
    cu_q = np.zeros(b + 1, dtype=np.int32)
    cu_p = np.zeros(b + 1, dtype=np.int32)
    cu_s = np.zeros(2 * b + 1, dtype=np.int32)
    _raise_for(lib.jpa_tail_segments(ctypes.byref(shard), int(seqlen_multiplier), b,
                                     _i32p(pl) if b else None, 1 if queries_include_prefix else 0,
                                     _i32p(cu_q), _i32p(cu_p), _i32p(cu_s)))
    return cu_q, cu_p, cu_s


def jpa_causal_cat_pad(x, cache, padding, out=None, stream=None):
    """[cache ; x] along time, zero-padded by padding = (w_left, w_right,
    h_left, h_right, t_left, t_right).  x [B, C, T, H, W] and cache
    [B, C, Tc, H, W] (or None): contiguous CUDA tensors with 2-byte elements.
    Returns out (allocated when None)."""
    import torch
    lib = load_library()
    if x.dim() != 5 or x.element_size() != 2 or not x.is_contiguous():
        raise JpaArgumentError(JPA_ERR_SHAPE, "x must be a contiguous 5-D tensor of 2-byte elements")
    b, c, t, h, w = x.shape
    tc = 0
    if cache is not None:
        if (cache.dim() != 5 or cache.dtype != x.dtype or not cache.is_contiguous()
                or tuple(cache.shape[:2]) != (b, c) or tuple(cache.shape[3:]) != (h, w)):
            raise JpaArgumentError(JPA_ERR_SHAPE, "cache must be a contiguous [B, C, Tc, H, W] like x")
        tc = cache.shape[2]
    pad = _i32(padding)
    if pad.size != 6:
        raise JpaArgumentError(JPA_ERR_SHAPE, "padding has six entries")
    shape = (b, c, tc + t + int(pad[4]) + int(pad[5]), h + int(pad[2]) + int(pad[3]), w + int(pad[0]) + int(pad[1]))
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape or out.dtype != x.dtype or not out.is_contiguous():
        raise JpaArgumentError(JPA_ERR_SHAPE, f"out must be a contiguous {shape} tensor like x")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    ptr = lambda v: ctypes.c_void_p(v.data_ptr()) if v is not None and v.numel() else None
    st = lib.jpa_causal_cat_pad(ptr(x), ptr(cache), b, c, t, tc, h, w, _i32p(pad), ptr(out), ctypes.c_void_p(handle))
    _raise_for(st)
    return out
