"""Python binding of libattn_jvp.so: fused teacher-forcing / block-causal
masked attention forward + JVP on MI355X (gfx950).

Argument marshalling only.  Every step of the operation runs in the HIP
library; PyTorch provides device memory and the stream.  The functions
mirror the C ABI of ``include/attn_jvp.h`` one to one:

    attn_jvp_create, attn_jvp_create_ex, attn_jvp_fwd, attn_jvp_bwd,
    attn_jvp_bwd_workspace_size, attn_jvp_destroy, attn_jvp_error_string,
    attn_jvp_last_error_detail, attn_jvp_plan_info, attn_jvp_plan_flops,
    attn_jvp_plan_bwd_flops, attn_jvp_plan_bwd_info, attn_jvp_launch_order,
    attn_jvp_bwd_launch_order, attn_jvp_row_ranges, attn_jvp_key_ranges,
    attn_jvp_tile_map, attn_jvp_create_ranges, attn_jvp_plan_table_size,
    attn_jvp_plan_table, attn_jvp_fwd_table, attn_jvp_fwd_primal

plus ``masked_attention_jvp(...)``, ``masked_attention_jvp_ranges(...)``,
``masked_attention_fwd(...)`` (no tangents) and ``masked_attention_bwd(...)``, which allocate the outputs (and the backward's
workspace, or a range-list plan's device table) and call ``attn_jvp_fwd`` /
``attn_jvp_fwd_table`` / ``attn_jvp_bwd`` on the current stream.  If the library is not built the
import of this module still works, but every call raises ``AttnJvpError``;
there is no fallback implementation.
"""
from __future__ import annotations

import collections
import ctypes
import os
import threading

import numpy as np

__all__ = [
    "ATTN_JVP_BF16", "ATTN_JVP_FP32", "ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO", "AttnJvpError", "Plan",
    "library_path", "attn_jvp_create", "attn_jvp_create_ex", "attn_jvp_fwd", "attn_jvp_destroy",
    "attn_jvp_error_string", "attn_jvp_last_error_detail", "attn_jvp_plan_info", "attn_jvp_plan_flops",
    "attn_jvp_launch_order", "attn_jvp_row_ranges", "attn_jvp_tile_map", "masked_attention_jvp",
    "attn_jvp_bwd", "attn_jvp_bwd_workspace_size", "attn_jvp_plan_bwd_flops", "attn_jvp_key_ranges",
    "attn_jvp_plan_bwd_info", "attn_jvp_bwd_launch_order", "attn_jvp_create_ranges", "attn_jvp_plan_table_size",
    "attn_jvp_plan_table", "attn_jvp_fwd_table", "masked_attention_jvp_ranges", "attn_jvp_fwd_primal",
    "attn_jvp_bwd_table", "masked_attention_bwd_ranges", "attn_jvp_fwd_primal_table", "masked_attention_fwd_ranges",
    "masked_attention_fwd",
    "masked_attention_bwd",
]

ATTN_JVP_BF16 = 0
ATTN_JVP_FP32 = 1
ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_JVP_LIBRARY selects another build of the same library (e.g. one made
# with different compile-time options); default: the in-tree build.
library_path = os.environ.get("ATTN_JVP_LIBRARY") or os.path.join(_HERE, "libattn_jvp.so")


class AttnJvpError(RuntimeError):
    def __init__(self, msg, code=None):
        super().__init__(msg)
        self.code = code


class _QueryGroup(ctypes.Structure):
    _fields_ = [("row_lo", ctypes.c_int32), ("row_hi", ctypes.c_int32),
                ("key_begin", ctypes.c_int32), ("key_end", ctypes.c_int32)]


class _MaskDesc(ctypes.Structure):
    _fields_ = [("tokens_per_frame", ctypes.c_int32), ("n_frames", ctypes.c_int32),
                ("frames_per_chunk", ctypes.c_int32), ("tf_layout", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(library_path):
            raise AttnJvpError(f"{library_path} is not built; run `python -m masked_attention_jvp_amd.build`")
        lib = ctypes.CDLL(library_path)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        P = ctypes.POINTER
        lib.attn_jvp_create.argtypes = [P(vp), P(_MaskDesc), i32, i32, i32, i32, f32]
        lib.attn_jvp_create_ex.argtypes = [P(vp), P(_MaskDesc), i32, i32, i32, i32, f32, ctypes.c_uint32]
        lib.attn_jvp_plan_flops.argtypes = [vp, P(i64)]
        lib.attn_jvp_fwd.argtypes = [vp] * 9 + [vp, vp]
        lib.attn_jvp_destroy.argtypes = [vp]
        lib.attn_jvp_error_string.argtypes = [ctypes.c_int]
        lib.attn_jvp_error_string.restype = ctypes.c_char_p
        lib.attn_jvp_last_error_detail.argtypes = []
        lib.attn_jvp_last_error_detail.restype = ctypes.c_char_p
        lib.attn_jvp_plan_info.argtypes = [vp, P(i64), P(i32), P(i32), P(i32), P(i32), P(i64), P(i64)]
        lib.attn_jvp_row_ranges.argtypes = [vp, P(i32), ctypes.c_size_t]
        lib.attn_jvp_launch_order.argtypes = [vp, P(i32), ctypes.c_size_t]
        lib.attn_jvp_tile_map.argtypes = [vp, P(ctypes.c_uint8), ctypes.c_size_t]
        lib.attn_jvp_bwd.argtypes = [vp] * 12
        lib.attn_jvp_bwd_workspace_size.argtypes = [vp, P(ctypes.c_size_t)]
        lib.attn_jvp_plan_bwd_flops.argtypes = [vp, P(i64)]
        lib.attn_jvp_key_ranges.argtypes = [vp, P(i32), ctypes.c_size_t]
        lib.attn_jvp_plan_bwd_info.argtypes = [vp, P(i32), P(i32), P(i32), P(i32)]
        lib.attn_jvp_bwd_launch_order.argtypes = [vp, P(i32), ctypes.c_size_t]
        lib.attn_jvp_create_ranges.argtypes = [P(vp), i32, i32, P(_QueryGroup), i32, P(i32), i32, i32, i32, i32, f32]
        lib.attn_jvp_plan_table_size.argtypes = [vp, P(ctypes.c_size_t)]
        lib.attn_jvp_plan_table.argtypes = [vp, vp, ctypes.c_size_t]
        lib.attn_jvp_fwd_table.argtypes = [vp] * 10 + [vp, vp]
        lib.attn_jvp_fwd_primal.argtypes = [vp] * 7
        lib.attn_jvp_bwd_table.argtypes = [vp] * 13
        lib.attn_jvp_fwd_primal_table.argtypes = [vp] * 8
        lib.attn_jvp_clock_sample.argtypes = [vp, vp]
        lib.attn_jvp_bwd_noalloc.argtypes = [vp] * 11
        for name in ("attn_jvp_create", "attn_jvp_create_ex", "attn_jvp_fwd", "attn_jvp_destroy",
                     "attn_jvp_plan_info", "attn_jvp_plan_flops", "attn_jvp_launch_order", "attn_jvp_row_ranges",
                     "attn_jvp_tile_map", "attn_jvp_bwd", "attn_jvp_bwd_workspace_size", "attn_jvp_plan_bwd_flops",
                     "attn_jvp_key_ranges", "attn_jvp_plan_bwd_info", "attn_jvp_bwd_launch_order",
                     "attn_jvp_create_ranges", "attn_jvp_plan_table_size", "attn_jvp_plan_table", "attn_jvp_fwd_table",
                     "attn_jvp_fwd_primal", "attn_jvp_bwd_table", "attn_jvp_fwd_primal_table",
                     "attn_jvp_clock_sample", "attn_jvp_bwd_noalloc"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def attn_jvp_error_string(code: int) -> str:
    return _load().attn_jvp_error_string(code).decode()


def attn_jvp_last_error_detail() -> str:
    return _load().attn_jvp_last_error_detail().decode()


def _check(code: int, what: str):
    if code != 0:
        raise AttnJvpError(f"{what}: {attn_jvp_error_string(code)}: {attn_jvp_last_error_detail()}", code)


class Plan:
    """Owns one attn_jvp_plan*; immutable after creation."""

    def __init__(self, handle, desc, batch, heads, head_dim, dtype, scale, flags=0):
        self._h = handle
        self.desc = tuple(desc)
        self.batch, self.heads, self.head_dim, self.dtype, self.scale = batch, heads, head_dim, dtype, scale
        self.flags = flags
        info = attn_jvp_plan_info(self)
        self.seq_len = info["seq_len"]
        self.info = info

    @property
    def handle(self):
        if self._h is None:
            raise AttnJvpError("plan already destroyed")
        return self._h

    @property
    def shape(self):
        return (self.batch, self.heads, self.seq_len, self.head_dim)

    def __del__(self):
        try:
            attn_jvp_destroy(self)
        except Exception:
            pass


def attn_jvp_create(desc, batch: int, heads: int, head_dim: int, dtype: int = ATTN_JVP_BF16,
                    softmax_scale: float = 0.0) -> Plan:
    """desc = (tokens_per_frame, n_frames, frames_per_chunk, tf_layout)."""
    lib = _load()
    h = ctypes.c_void_p()
    d = _MaskDesc(*[int(x) for x in desc])
    _check(lib.attn_jvp_create(ctypes.byref(h), ctypes.byref(d), int(batch), int(heads), int(head_dim),
                               int(dtype), float(softmax_scale or 0.0)), "attn_jvp_create")
    return Plan(h, desc, batch, heads, head_dim, dtype, softmax_scale)


def attn_jvp_create_ex(desc, batch: int, heads: int, head_dim: int, dtype: int = ATTN_JVP_BF16,
                       softmax_scale: float = 0.0, flags: int = 0) -> Plan:
    """attn_jvp_create with plan flags (ATTN_JVP_FLAG_*)."""
    lib = _load()
    h = ctypes.c_void_p()
    d = _MaskDesc(*[int(x) for x in desc])
    _check(lib.attn_jvp_create_ex(ctypes.byref(h), ctypes.byref(d), int(batch), int(heads), int(head_dim),
                                  int(dtype), float(softmax_scale or 0.0), int(flags)), "attn_jvp_create_ex")
    return Plan(h, desc, batch, heads, head_dim, dtype, softmax_scale, int(flags))


def attn_jvp_create_ranges(n_tokens: int, groups, batch: int, heads: int, head_dim: int,
                           dtype: int = ATTN_JVP_BF16, softmax_scale: float = 0.0) -> Plan:
    """Plan for a range-list mask: groups = [(row_lo, row_hi, [(key_lo, key_hi), ...]), ...]
    (half-open, sorted by row_lo, disjoint)."""
    lib = _load()
    groups = list(groups)
    qg = (_QueryGroup * max(1, len(groups)))()
    flat = []
    for i, (lo, hi, ivs) in enumerate(groups):
        b = len(flat) // 2
        for a, z in ivs:
            flat += [int(a), int(z)]
        qg[i] = _QueryGroup(int(lo), int(hi), b, len(flat) // 2)
    iv = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    h = ctypes.c_void_p()
    _check(lib.attn_jvp_create_ranges(ctypes.byref(h), int(n_tokens), len(groups), qg, len(flat) // 2, iv, int(batch),
                                      int(heads), int(head_dim), int(dtype), float(softmax_scale or 0.0)),
           "attn_jvp_create_ranges")
    plan = Plan(h, (int(n_tokens), len(groups)), batch, heads, head_dim, dtype, softmax_scale)
    plan.ranges = tuple((int(lo), int(hi), tuple((int(a), int(z)) for a, z in ivs)) for lo, hi, ivs in groups)
    return plan


def attn_jvp_plan_table_size(plan: Plan) -> int:
    v = ctypes.c_size_t()
    _check(_load().attn_jvp_plan_table_size(plan.handle, ctypes.byref(v)), "attn_jvp_plan_table_size")
    return v.value


def attn_jvp_plan_table(plan: Plan) -> np.ndarray:
    """A range-list plan's schedule table as int32 host words (to be copied to the device)."""
    n = attn_jvp_plan_table_size(plan)
    out = np.empty(n // 4, dtype=np.int32)
    _check(_load().attn_jvp_plan_table(plan.handle, out.ctypes.data_as(ctypes.c_void_p), n), "attn_jvp_plan_table")
    return out


def attn_jvp_plan_flops(plan: Plan) -> int:
    """Useful FLOPs of one attn_jvp_fwd call of the plan (all heads)."""
    v = ctypes.c_int64()
    _check(_load().attn_jvp_plan_flops(plan.handle, ctypes.byref(v)), "attn_jvp_plan_flops")
    return v.value


def attn_jvp_destroy(plan: Plan) -> None:
    if plan is not None and plan._h is not None:
        _check(_load().attn_jvp_destroy(plan._h), "attn_jvp_destroy")
        plan._h = None


def attn_jvp_plan_info(plan: Plan) -> dict:
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    vals = [i64(), i32(), i32(), i32(), i32(), i64(), i64()]
    _check(_load().attn_jvp_plan_info(plan.handle, *[ctypes.byref(v) for v in vals]), "attn_jvp_plan_info")
    keys = ["seq_len", "block_q", "block_k", "n_query_blocks", "n_key_tiles", "allowed_pairs_per_head",
            "visited_tiles_per_head"]
    return {k: v.value for k, v in zip(keys, vals)}


def attn_jvp_row_ranges(plan: Plan) -> np.ndarray:
    n = plan.seq_len
    out = np.empty((n, 4), dtype=np.int32)
    _check(_load().attn_jvp_row_ranges(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out.size),
           "attn_jvp_row_ranges")
    return out


def attn_jvp_key_ranges(plan: Plan) -> np.ndarray:
    """[N, 4] int32: per key j, the query rows [lo1, hi1) and [lo2, hi2) that attend to it."""
    n = plan.seq_len
    out = np.empty((n, 4), dtype=np.int32)
    _check(_load().attn_jvp_key_ranges(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out.size),
           "attn_jvp_key_ranges")
    return out


def attn_jvp_plan_bwd_info(plan: Plan) -> dict:
    """Backward geometry: dq block rows, dk/dv block keys, blocks per (b, h)."""
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(_load().attn_jvp_plan_bwd_info(plan.handle, *[ctypes.byref(v) for v in vals]), "attn_jvp_plan_bwd_info")
    return dict(zip(["block_q", "block_kv", "n_query_blocks", "n_key_blocks"], [v.value for v in vals]))


def attn_jvp_bwd_launch_order(plan: Plan) -> np.ndarray:
    """Task (b*H + h) * n_key_blocks + key block of each dk/dv workgroup."""
    n = plan.batch * plan.heads * attn_jvp_plan_bwd_info(plan)["n_key_blocks"]
    out = np.empty(n, dtype=np.int32)
    _check(_load().attn_jvp_bwd_launch_order(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n),
           "attn_jvp_bwd_launch_order")
    return out


def attn_jvp_bwd_workspace_size(plan: Plan) -> int:
    """Bytes of device workspace attn_jvp_bwd needs (8 B H N)."""
    v = ctypes.c_size_t()
    _check(_load().attn_jvp_bwd_workspace_size(plan.handle, ctypes.byref(v)), "attn_jvp_bwd_workspace_size")
    return v.value


def attn_jvp_plan_bwd_flops(plan: Plan) -> int:
    """Useful FLOPs of one attn_jvp_bwd call of the plan (all heads): 10 d per allowed pair."""
    v = ctypes.c_int64()
    _check(_load().attn_jvp_plan_bwd_flops(plan.handle, ctypes.byref(v)), "attn_jvp_plan_bwd_flops")
    return v.value


def attn_jvp_launch_order(plan: Plan) -> np.ndarray:
    """Query block handled by workgroup t of each (b, h)."""
    out = np.empty(plan.info["n_query_blocks"], dtype=np.int32)
    _check(_load().attn_jvp_launch_order(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out.size),
           "attn_jvp_launch_order")
    return out


def attn_jvp_tile_map(plan: Plan) -> np.ndarray:
    nq, nk = plan.info["n_query_blocks"], plan.info["n_key_tiles"]
    out = np.empty((nq, nk), dtype=np.uint8)
    _check(_load().attn_jvp_tile_map(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), out.size),
           "attn_jvp_tile_map")
    return out


def _torch_dtype(plan):
    import torch
    return torch.bfloat16 if plan.dtype == ATTN_JVP_BF16 else torch.float32


def _check_tensor(name, t, plan, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise AttnJvpError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise AttnJvpError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype != _torch_dtype(plan):
        raise AttnJvpError(f"{name} has dtype {t.dtype}, plan expects {_torch_dtype(plan)}")
    if tuple(t.shape) != tuple(shape):
        raise AttnJvpError(f"{name} has shape {tuple(t.shape)}, plan expects {tuple(shape)}")
    if not t.is_contiguous():
        raise AttnJvpError(f"{name} must be contiguous")


def attn_jvp_fwd(plan: Plan, q, k, v, tq, tk, tv, o, t_o, lse=None, stream=None) -> None:
    """Enqueue the operation on `stream` (default: torch's current stream)."""
    import torch
    ins = dict(q=q, k=k, v=v, tq=tq, tk=tk, tv=tv, o=o, t_o=t_o)
    for name, t in ins.items():
        _check_tensor(name, t, plan, plan.shape)
    dev = q.device
    for name, t in ins.items():
        if t.device != dev:
            raise AttnJvpError(f"{name} is on {t.device}, q is on {dev}")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != plan.shape[:3] or not lse.is_contiguous() \
                or lse.device != dev:
            raise AttnJvpError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        code = _load().attn_jvp_fwd(plan.handle, *[ctypes.c_void_p(t.data_ptr()) for t in ins.values()],
                                    ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                                    ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_fwd")


def attn_jvp_fwd_primal(plan: Plan, q, k, v, o, lse=None, stream=None) -> None:
    """o (and lse) of the plan's masked attention, without tangents."""
    import torch
    ins = dict(q=q, k=k, v=v, o=o)
    for name, t in ins.items():
        _check_tensor(name, t, plan, plan.shape)
    dev = q.device
    for name, t in ins.items():
        if t.device != dev:
            raise AttnJvpError(f"{name} is on {t.device}, q is on {dev}")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != plan.shape[:3] or not lse.is_contiguous() \
                or lse.device != dev:
            raise AttnJvpError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        code = _load().attn_jvp_fwd_primal(plan.handle, *[ctypes.c_void_p(t.data_ptr()) for t in ins.values()],
                                           ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                                           ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_fwd_primal")


def attn_jvp_clock_sample(out, stream=None) -> None:
    """Enqueue one clock sample (attn_jvp_clock_sample) into ``out``, a
    contiguous int64 device tensor of at least 32 elements: per XCD its
    number, its shader clock counter and the 100 MHz real-time counter."""
    import torch
    if out.dtype != torch.int64 or not out.is_contiguous() or out.numel() < 32 or out.device.type != "cuda":
        raise AttnJvpError("out must be a contiguous int64 CUDA tensor of at least 32 elements")
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    with torch.cuda.device(out.device):
        code = _load().attn_jvp_clock_sample(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_clock_sample")


def shader_clock_mhz(before, after) -> dict:
    """Average shader clock per XCD between two clock samples (host copies
    of the 32 int64 of attn_jvp_clock_sample): 100 MHz times the change of
    the XCD's shader counter over the change of the real-time counter."""
    b = np.asarray(before, dtype=np.int64).reshape(-1, 4)
    a = np.asarray(after, dtype=np.int64).reshape(-1, 4)
    start = {int(x): (int(t), int(rt)) for x, t, rt, _ in b}
    mhz = {}
    for x, t, rt, _ in a:
        x = int(x)
        if x in start and int(rt) > start[x][1]:
            mhz[x] = 100.0 * (int(t) - start[x][0]) / (int(rt) - start[x][1])
    return mhz


def attn_jvp_fwd_primal_table(plan: Plan, table, q, k, v, o, lse=None, stream=None) -> None:
    """attn_jvp_fwd_primal for a range-list plan, with its device table."""
    import torch
    ins = dict(q=q, k=k, v=v, o=o)
    for name, t in ins.items():
        _check_tensor(name, t, plan, plan.shape)
    dev = q.device
    _check_table(plan, table, dev)
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != plan.shape[:3] or not lse.is_contiguous() \
                or lse.device != dev:
            raise AttnJvpError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        code = _load().attn_jvp_fwd_primal_table(plan.handle, ctypes.c_void_p(table.data_ptr()),
                                                 *[ctypes.c_void_p(t.data_ptr()) for t in ins.values()],
                                                 ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                                                 ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_fwd_primal_table")


def _bwd_args(plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace):
    import torch
    ts = dict(q=q, k=k, v=v, o=o, d_o=d_o, dq=dq, dk=dk, dv=dv)
    for name, t in ts.items():
        _check_tensor(name, t, plan, plan.shape)
    dev = q.device
    extra = [("lse", lse)] + ([("workspace", workspace)] if workspace is not None else [])
    for name, t in list(ts.items()) + extra:
        if not isinstance(t, torch.Tensor) or t.device != dev:
            raise AttnJvpError(f"{name} must be a tensor on q's device ({dev})")
    if lse.dtype != torch.float32 or tuple(lse.shape) != plan.shape[:3] or not lse.is_contiguous():
        raise AttnJvpError("lse must be a contiguous float32 [B, H, N] tensor")
    if workspace is None:  # attn_jvp_bwd_noalloc: the library's own workspace
        return [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, d_o, dq, dk, dv)]
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() \
            or workspace.numel() * 4 < attn_jvp_bwd_workspace_size(plan):
        raise AttnJvpError(f"workspace must be a contiguous float32 tensor of at least "
                           f"{attn_jvp_bwd_workspace_size(plan)} bytes")
    return [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse, d_o, dq, dk, dv, workspace)]


def attn_jvp_bwd(plan: Plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace, stream=None) -> None:
    """Enqueue the backward (dq, dk, dv) on `stream` (default: torch's current
    stream).  `workspace` is a float32 CUDA tensor of at least
    attn_jvp_bwd_workspace_size(plan) bytes; on return it holds -delta and
    -lse log2(e) per row, [B, H, 2, N]."""
    import torch
    ptrs = _bwd_args(plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        code = _load().attn_jvp_bwd(plan.handle, *ptrs, ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_bwd")


def attn_jvp_bwd_noalloc(plan: Plan, q, k, v, o, lse, d_o, dq, dk, dv, stream=None) -> None:
    """attn_jvp_bwd with the library's fixed device workspace (allocates
    nothing; calls on one GPU must not overlap in time)."""
    import torch
    ptrs = _bwd_args(plan, q, k, v, o, lse, d_o, dq, dk, dv, None)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        code = _load().attn_jvp_bwd_noalloc(plan.handle, *ptrs, ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_bwd_noalloc")


def attn_jvp_bwd_table(plan: Plan, table, q, k, v, o, lse, d_o, dq, dk, dv, workspace, stream=None) -> None:
    """attn_jvp_bwd for a range-list plan; `table` is the plan's table as an
    int32 CUDA tensor (attn_jvp_plan_table copied to the device)."""
    import torch
    ptrs = _bwd_args(plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace)
    _check_table(plan, table, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        code = _load().attn_jvp_bwd_table(plan.handle, ctypes.c_void_p(table.data_ptr()), *ptrs,
                                          ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_bwd_table")


def _check_table(plan, table, dev):
    import torch
    if not isinstance(table, torch.Tensor) or table.device != dev or table.dtype != torch.int32 \
            or not table.is_contiguous() or table.numel() * 4 < attn_jvp_plan_table_size(plan):
        raise AttnJvpError("table must be the plan's int32 table as a contiguous tensor on q's device")


def attn_jvp_fwd_table(plan: Plan, table, q, k, v, tq, tk, tv, o, t_o, lse=None, stream=None) -> None:
    """attn_jvp_fwd for a range-list plan; `table` is the plan's table as an
    int32 CUDA tensor (attn_jvp_plan_table copied to the device)."""
    import torch
    ins = dict(q=q, k=k, v=v, tq=tq, tk=tk, tv=tv, o=o, t_o=t_o)
    for name, t in ins.items():
        _check_tensor(name, t, plan, plan.shape)
    dev = q.device
    _check_table(plan, table, dev)
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != plan.shape[:3] or not lse.is_contiguous() \
                or lse.device != dev:
            raise AttnJvpError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        code = _load().attn_jvp_fwd_table(plan.handle, ctypes.c_void_p(table.data_ptr()),
                                          *[ctypes.c_void_p(t.data_ptr()) for t in ins.values()],
                                          ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                                          ctypes.c_void_p(stream.cuda_stream))
    _check(code, "attn_jvp_fwd_table")


# Plans and range-list tables are cached per mask and shape for the
# convenience functions below, least recently used first out: a plan holds
# host memory only; a range-list entry also holds its device table, which
# each call marks as used on its stream, so that the allocator does not
# reuse the memory of an evicted table before that stream's work is done.
PLAN_CACHE_SIZE = 64
RANGE_CACHE_SIZE = 16
_plan_cache = collections.OrderedDict()
_plan_lock = threading.Lock()


def _cache_get(cache, key):
    hit = cache.get(key)
    if hit is not None:
        cache.move_to_end(key)
    return hit


def _cache_put(cache, key, value, size):
    cache[key] = value
    cache.move_to_end(key)
    while len(cache) > size:
        cache.popitem(last=False)


def _cached_plan(desc, shape, dtype, scale, flags=0):
    key = (tuple(int(x) for x in desc), tuple(shape), dtype, float(scale or 0.0), int(flags))
    with _plan_lock:
        p = _cache_get(_plan_cache, key)
        if p is None:
            b, h, _, d = shape
            p = attn_jvp_create_ex(desc, b, h, d, dtype, scale or 0.0, flags)
            if tuple(p.shape) != tuple(shape):
                raise AttnJvpError(f"mask {tuple(desc)} gives N={p.seq_len}, tensors have N={shape[2]}")
            _cache_put(_plan_cache, key, p, PLAN_CACHE_SIZE)
        return p


def masked_attention_jvp(q, k, v, tq, tk, tv, desc, scale=None, return_lse=False, clean_tangent_zero=False):
    """(o, t_o[, lse]) for [B, H, N, d] bf16 or fp32 CUDA tensors.  With
    clean_tangent_zero (teacher-forcing masks only) the clean halves of tq,
    tk, tv are taken as zero and never read."""
    import torch
    dtype = ATTN_JVP_BF16 if q.dtype == torch.bfloat16 else ATTN_JVP_FP32
    flags = ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO if clean_tangent_zero else 0
    plan = _cached_plan(desc, q.shape, dtype, scale, flags)
    o = torch.empty_like(q)
    t_o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_jvp_fwd(plan, q, k, v, tq, tk, tv, o, t_o, lse)
    return (o, t_o, lse) if return_lse else (o, t_o)


def masked_attention_fwd(q, k, v, desc, scale=None, return_lse=False):
    """(o[, lse]) of the masked attention alone (no tangents) for [B, H, N, d]
    bf16 or fp32 CUDA tensors: the forward that pairs with the backward."""
    import torch
    dtype = ATTN_JVP_BF16 if q.dtype == torch.bfloat16 else ATTN_JVP_FP32
    plan = _cached_plan(desc, q.shape, dtype, scale, 0)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_jvp_fwd_primal(plan, q, k, v, o, lse)
    return (o, lse) if return_lse else o


def masked_attention_bwd(q, k, v, o, lse, d_o, desc, scale=None, return_workspace=False):
    """(dq, dk, dv[, workspace]) of masked attention for [B, H, N, d] bf16 or
    fp32 CUDA tensors, from the forward's o and lse (masked_attention_jvp with
    return_lse=True) and the output gradient d_o."""
    import torch
    dtype = ATTN_JVP_BF16 if q.dtype == torch.bfloat16 else ATTN_JVP_FP32
    plan = _cached_plan(desc, q.shape, dtype, scale, 0)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device=q.device)
    attn_jvp_bwd(plan, q, k, v, o, lse, d_o, dq, dk, dv, ws)
    return (dq, dk, dv, ws) if return_workspace else (dq, dk, dv)


_range_cache = collections.OrderedDict()


def _cached_range_plan(q, groups, scale):
    """The plan of a range-list mask and its device table, cached per (mask,
    shape, dtype, scale, device)."""
    import torch
    dtype = ATTN_JVP_BF16 if q.dtype == torch.bfloat16 else ATTN_JVP_FP32
    b, h, n, d = q.shape
    key = (tuple((int(lo), int(hi), tuple((int(a), int(z)) for a, z in ivs)) for lo, hi, ivs in groups),
           tuple(q.shape), dtype, float(scale or 0.0), str(q.device))
    with _plan_lock:
        hit = _cache_get(_range_cache, key)
        if hit is None:
            plan = attn_jvp_create_ranges(n, groups, b, h, d, dtype, scale or 0.0)
            table = torch.from_numpy(attn_jvp_plan_table(plan)).to(q.device)
            hit = (plan, table)
            _cache_put(_range_cache, key, hit, RANGE_CACHE_SIZE)
    # the table is read by work enqueued on the current stream
    hit[1].record_stream(torch.cuda.current_stream(q.device))
    return hit


def masked_attention_jvp_ranges(q, k, v, tq, tk, tv, groups, scale=None, return_lse=False):
    """(o, t_o[, lse]) for a range-list mask: groups = [(row_lo, row_hi,
    [(key_lo, key_hi), ...]), ...]."""
    import torch
    plan, table = _cached_range_plan(q, groups, scale)
    o = torch.empty_like(q)
    t_o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_jvp_fwd_table(plan, table, q, k, v, tq, tk, tv, o, t_o, lse)
    return (o, t_o, lse) if return_lse else (o, t_o)


def masked_attention_bwd_ranges(q, k, v, o, lse, d_o, groups, scale=None, return_workspace=False):
    """(dq, dk, dv[, workspace]) for a range-list mask (groups as in
    masked_attention_jvp_ranges), from that forward's o and lse."""
    import torch
    plan, table = _cached_range_plan(q, groups, scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device=q.device)
    attn_jvp_bwd_table(plan, table, q, k, v, o, lse, d_o, dq, dk, dv, ws)
    return (dq, dk, dv, ws) if return_workspace else (dq, dk, dv)


def masked_attention_fwd_ranges(q, k, v, groups, scale=None, return_lse=False):
    """(o[, lse]) of a range-list mask without tangents (groups as in
    masked_attention_jvp_ranges): the forward that pairs with
    masked_attention_bwd_ranges."""
    import torch
    plan, table = _cached_range_plan(q, groups, scale)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_jvp_fwd_primal_table(plan, table, q, k, v, o, lse)
    return (o, lse) if return_lse else o
