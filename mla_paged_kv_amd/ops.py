"""Thin ctypes binding of libmla_paged_kv.so (declared in include/mla_paged_kv.h).

Argument marshalling only: the functions check tensor dtypes, shapes and
contiguity, pass raw device pointers and the current HIP stream, and raise
MLAError on a nonzero status.  Every step of the computation runs in the HIP
kernels; if the library is missing this module raises at import instead of
computing anything on the host.  torch supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MLA_PAGED_KV_LIB", os.path.join(_HERE, "libmla_paged_kv.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m mla_paged_kv_amd.build` "
        "(hipcc, gfx950). There is no host fallback."
    )

_lib = ctypes.CDLL(LIB_PATH)

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE_TOO_SMALL = -3
MLA_ERR_HIP = -4
KV_BF16_PAGED = 0
KV_FP8_PACKED = 1
KV_FP8_INDEXED = 2
KV_FP16_PAGED = 3
SCHED_AUTO, SCHED_GLOBAL, SCHED_REQUEST_LOCAL = 0, 1, 2
D_QK, D_V, PAGE, REC_BYTES = 576, 512, 64, 656
NOALLOC_SCRATCH_BYTES = 128 << 20  # MLA_NOALLOC_SCRATCH_BYTES
SCHED_META_INTS = 8

_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "mla_last_error_message": ([], ctypes.c_char_p),
    "mla_decode_num_parts": ([_i32, _i32, _i32, _i32, _i32, _P], _i32),
    "mla_plan_num_parts": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _P], _i32),
    "mla_decode_kernel_name": ([_i32, _i32, _i32, _i32], ctypes.c_char_p),
    "mla_decode_workspace_size": ([_i32, _i32, _i32, _i32], _sz),
    "mla_packed_kv_workspace_size": ([_i32, _i32, _i32], _sz),
    "mla_get_decode_metadata": ([_P, _i32, _i32, _i32, _i32, _i32, _P, _P, _P], _i32),
    "mla_decode_fwd": ([_P, _P, _i32, _i64, _P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _P, _P, _i32,
                        _P, _P, _P, _sz, _P], _i32),
    "mla_combine": ([_P, _P, _sz, _i32, _i32, _i32, _i32, _i32, _P, _P, _P], _i32),
    "mla_decode_fwd_noalloc": ([_P, _P, _i32, _i64, _P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _P, _P,
                                _i32, _P, _P, _P], _i32),
    "mla_pack_selected_kv": ([_P, _i64, _P, _P, _i32, _i32, _i32, _P, _sz, _P], _i32),
    "mla_patch_packed_kv": ([_P, _i64, _P, _P, _i32, _i32, _i32, _P, _i32, _P, _sz, _P], _i32),
    "mla_sparse_kv_format": ([_i32, _i32, _i32, _sz, _i32, _P], _i32),
    "mla_get_packed_decode_metadata": ([_P, _i32, _i32, _i32, _i32, _i32, _i32, _P, _P, _P], _i32),
    "mla_read_device_errors": ([_P, _P], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def mla_last_error_message() -> str:
    return (_lib.mla_last_error_message() or b"").decode()


def _check(status: int):
    if status != MLA_OK:
        raise MLAError(status, mla_last_error_message())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class BoundCall:
    """One entry point with its arguments checked and converted once.

    Calling it only crosses the C ABI: no tensor checks, no conversions.  For
    loops that issue the same launch many times (timed loops, a serving loop
    whose buffers stay put).  It keeps the tensors it points into alive; the
    stream is the one current when it was bound."""

    __slots__ = ("name", "_fn", "_args", "_keep")

    def __init__(self, name, args, keep):
        self.name = name
        self._fn = getattr(_lib, name)
        self._args = tuple(a if isinstance(a, t) or a is None else t(a) for a, t in zip(args, self._fn.argtypes))
        self._keep = tuple(keep)

    def __call__(self):
        status = self._fn(*self._args)
        if status != MLA_OK:
            raise MLAError(status, mla_last_error_message())


def _call(name, args, bind, keep=()):
    if bind:
        return BoundCall(name, args, keep)
    _check(getattr(_lib, name)(*args))
    return None


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------------------- raw entry points (same names)

def mla_decode_num_parts(batch, s_q, h_q, h_kv=1, kv_format=KV_BF16_PAGED) -> int:
    out = ctypes.c_int(0)
    _check(_lib.mla_decode_num_parts(batch, s_q, h_q, h_kv, kv_format, ctypes.byref(out)))
    return out.value


def mla_plan_num_parts(batch, s_q, h_q, kv_format, cus, wgs_per_cu, h_kv=1) -> int:
    out = ctypes.c_int(0)
    _check(_lib.mla_plan_num_parts(batch, s_q, h_q, h_kv, kv_format, cus, wgs_per_cu, ctypes.byref(out)))
    return out.value


def mla_decode_kernel_name(s_q, h_q, h_kv=1, kv_format=KV_BF16_PAGED) -> str:
    name = _lib.mla_decode_kernel_name(s_q, h_q, h_kv, kv_format)
    if name is None:
        raise MLAError(MLA_ERR_UNSUPPORTED, mla_last_error_message())
    return name.decode()


def mla_decode_workspace_size(batch, s_q, h_q, num_parts) -> int:
    return int(_lib.mla_decode_workspace_size(batch, s_q, h_q, num_parts))


def mla_packed_kv_workspace_size(batch, s_q, topk_capacity) -> int:
    return int(_lib.mla_packed_kv_workspace_size(batch, s_q, topk_capacity))


def mla_get_decode_metadata(seqlens, batch, s_q, h_q, h_kv, num_parts, sched_meta=None, num_splits=None,
                            stream=None, bind=False):
    """Scheduler metadata into (sched_meta, num_splits), allocated here if None.
    With bind=True the launch is not made: a BoundCall that makes it is returned."""
    _need(seqlens, "seqlens", torch.int32, (batch,))
    dev = seqlens.device
    if sched_meta is None:
        sched_meta = torch.empty((num_parts, SCHED_META_INTS), dtype=torch.int32, device=dev)
    if num_splits is None:
        num_splits = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _need(sched_meta, "sched_meta", torch.int32, (num_parts, SCHED_META_INTS))
    _need(num_splits, "num_splits", torch.int32, (batch + 1,))
    bound = _call("mla_get_decode_metadata", (_ptr(seqlens), batch, s_q, h_q, h_kv, num_parts, _ptr(sched_meta),
                                              _ptr(num_splits), _stream(stream)), bind,
                  (seqlens, sched_meta, num_splits))
    return bound if bind else (sched_meta, num_splits)


def _act_dtype(kv_format):
    return torch.float16 if kv_format == KV_FP16_PAGED else torch.bfloat16


def mla_get_packed_decode_metadata(topk_length, batch, s_q, h_q, topk_capacity, num_parts, policy=SCHED_AUTO,
                                   sched_meta=None, num_splits=None, stream=None, bind=False):
    _need(topk_length, "topk_length", torch.int32, (batch,))
    dev = topk_length.device
    if sched_meta is None:
        sched_meta = torch.empty((num_parts, SCHED_META_INTS), dtype=torch.int32, device=dev)
    if num_splits is None:
        num_splits = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _need(sched_meta, "sched_meta", torch.int32, (num_parts, SCHED_META_INTS))
    _need(num_splits, "num_splits", torch.int32, (batch + 1,))
    bound = _call("mla_get_packed_decode_metadata", (_ptr(topk_length), batch, s_q, h_q, topk_capacity, num_parts,
                                                     policy, _ptr(sched_meta), _ptr(num_splits), _stream(stream)),
                  bind, (topk_length, sched_meta, num_splits))
    return bound if bind else (sched_meta, num_splits)


def _decode_args(q, kv, kv_format, block_table, seqlens, sched_meta, num_splits, out, lse, topk_capacity):
    """Checks of the decode entry points' tensors; returns the sizes they pass."""
    _need(q, "q", _act_dtype(kv_format))
    b, s_q, h_q, d = q.shape
    if d != D_QK:
        raise ValueError(f"q last dim {d}, expected {D_QK}")
    h_kv = 1
    if kv_format in (KV_BF16_PAGED, KV_FP16_PAGED):
        _need(kv, "kcache", _act_dtype(kv_format))
        if kv.dim() != 4 or kv.shape[1] != PAGE or kv.shape[3] != D_QK:
            raise ValueError(f"kcache shape {tuple(kv.shape)}, expected [pages, 64, h_kv, 576]")
        h_kv = kv.shape[2]
        _need(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != b:
            raise ValueError("block_table must be [batch, max_pages]")
        num_pages, max_pages = kv.shape[0], block_table.shape[1]
    elif kv_format == KV_FP8_INDEXED:
        # the FP8 record pool itself; block_table carries the top-k token ids
        _need(kv, "kcache_fp8", torch.uint8)
        if tuple(kv.shape[1:]) != (PAGE, 1, REC_BYTES):
            raise ValueError(f"kcache_fp8 shape {tuple(kv.shape)}, expected [pages, 64, 1, 656]")
        _need(block_table, "indices", torch.int32)
        if block_table.dim() != 3 or block_table.shape[:2] != (b, s_q):
            raise ValueError("indices must be [batch, s_q, topk_capacity]")
        if topk_capacity == 0:
            topk_capacity = block_table.shape[2]
        if topk_capacity != block_table.shape[2]:
            raise ValueError(f"topk_capacity {topk_capacity} != indices.shape[2] {block_table.shape[2]}")
        num_pages, max_pages = kv.shape[0], 0
    else:
        _need(kv, "packed workspace", torch.uint8)
        num_pages, max_pages = 0, 0
    _need(seqlens, "seqlens", torch.int32, (b,))
    _need(sched_meta, "sched_meta", torch.int32)
    _need(num_splits, "num_splits", torch.int32, (b + 1,))
    _need(out, "out", _act_dtype(kv_format), (b, s_q, h_q, D_V))
    _need(lse, "lse", torch.float32, (b, s_q, h_q))
    return b, s_q, h_q, h_kv, num_pages, max_pages, topk_capacity


def mla_decode_fwd(q, kv, kv_format, block_table, seqlens, softmax_scale, causal, sched_meta, num_splits, out, lse,
                   workspace, topk_capacity=0, stream=None, bind=False):
    """Decode into out/lse (unsplit requests) and the workspace's partials.  With
    bind=True a BoundCall that makes the launch is returned instead."""
    args = _decode_args(q, kv, kv_format, block_table, seqlens, sched_meta, num_splits, out, lse, topk_capacity)
    b, s_q, h_q, h_kv, num_pages, max_pages, topk_capacity = args
    _need(workspace, "workspace", torch.uint8)
    return _call("mla_decode_fwd", (
        _ptr(q), _ptr(kv), kv_format, num_pages, _ptr(block_table) if kv_format != KV_FP8_PACKED else None,
        max_pages, _ptr(seqlens), topk_capacity, b, s_q, h_q, h_kv, float(softmax_scale), int(bool(causal)),
        _ptr(sched_meta), _ptr(num_splits), sched_meta.shape[0], _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)), bind, (q, kv, block_table, seqlens, sched_meta, num_splits, out, lse,
                                                     workspace))


def mla_decode_fwd_noalloc(q, kv, kv_format, block_table, seqlens, softmax_scale, causal, sched_meta, num_splits,
                           out, lse, topk_capacity=0, stream=None):
    """mla_decode_fwd + mla_combine with the split partials in the library's own
    device scratch (no workspace argument, nothing allocated by the call)."""
    args = _decode_args(q, kv, kv_format, block_table, seqlens, sched_meta, num_splits, out, lse, topk_capacity)
    b, s_q, h_q, h_kv, num_pages, max_pages, topk_capacity = args
    _check(_lib.mla_decode_fwd_noalloc(
        _ptr(q), _ptr(kv), kv_format, num_pages, _ptr(block_table) if kv_format != KV_FP8_PACKED else None,
        max_pages, _ptr(seqlens), topk_capacity, b, s_q, h_q, h_kv, float(softmax_scale), int(bool(causal)),
        _ptr(sched_meta), _ptr(num_splits), sched_meta.shape[0], _ptr(out), _ptr(lse), _stream(stream)))


def mla_combine(num_splits, workspace, batch, s_q, h_q, num_parts, out, lse, stream=None, kv_format=KV_BF16_PAGED,
                bind=False):
    """Merge the split partials into out/lse.  With bind=True a BoundCall that
    makes the launch is returned instead."""
    _need(num_splits, "num_splits", torch.int32, (batch + 1,))
    _need(workspace, "workspace", torch.uint8)
    _need(out, "out", _act_dtype(kv_format), (batch, s_q, h_q, D_V))
    _need(lse, "lse", torch.float32, (batch, s_q, h_q))
    return _call("mla_combine", (_ptr(num_splits), _ptr(workspace), workspace.numel(), batch, s_q, h_q, num_parts,
                                 kv_format, _ptr(out), _ptr(lse), _stream(stream)), bind,
                 (num_splits, workspace, out, lse))


def mla_pack_selected_kv(kcache_fp8, indices, topk_length, workspace=None, stream=None, bind=False):
    _need(kcache_fp8, "kcache_fp8", torch.uint8)
    if tuple(kcache_fp8.shape[1:]) != (PAGE, 1, REC_BYTES):
        raise ValueError(f"kcache_fp8 shape {tuple(kcache_fp8.shape)}, expected [pages, 64, 1, 656]")
    _need(indices, "indices", torch.int32)
    b, s_q, cap = indices.shape
    _need(topk_length, "topk_length", torch.int32, (b,))
    nbytes = mla_packed_kv_workspace_size(b, s_q, cap)
    if workspace is None:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=indices.device)
    _need(workspace, "workspace", torch.uint8)
    bound = _call("mla_pack_selected_kv", (_ptr(kcache_fp8), kcache_fp8.shape[0], _ptr(indices), _ptr(topk_length),
                                           b, s_q, cap, _ptr(workspace), workspace.numel(), _stream(stream)), bind,
                  (kcache_fp8, indices, topk_length, workspace))
    return bound if bind else workspace


def mla_patch_packed_kv(kcache_fp8, indices, topk_length, new_ids, workspace, stream=None):
    """Overwrite the packed slots that select one of `new_ids` (int32 [batch, n_new])
    with those records' current bytes."""
    _need(kcache_fp8, "kcache_fp8", torch.uint8)
    if tuple(kcache_fp8.shape[1:]) != (PAGE, 1, REC_BYTES):
        raise ValueError(f"kcache_fp8 shape {tuple(kcache_fp8.shape)}, expected [pages, 64, 1, 656]")
    _need(indices, "indices", torch.int32)
    b, s_q, cap = indices.shape
    _need(topk_length, "topk_length", torch.int32, (b,))
    _need(new_ids, "new_ids", torch.int32)
    if new_ids.dim() != 2 or new_ids.shape[0] != b:
        raise ValueError("new_ids must be [batch, n_new]")
    _need(workspace, "workspace", torch.uint8)
    _check(_lib.mla_patch_packed_kv(_ptr(kcache_fp8), kcache_fp8.shape[0], _ptr(indices), _ptr(topk_length), b, s_q,
                                    cap, _ptr(new_ids), new_ids.shape[1], _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return workspace


def mla_sparse_kv_format(batch, s_q, topk_capacity, workspace_budget_bytes, pack_hidden) -> int:
    out = ctypes.c_int(-1)
    _check(_lib.mla_sparse_kv_format(batch, s_q, topk_capacity, int(workspace_budget_bytes), int(bool(pack_hidden)),
                                     ctypes.byref(out)))
    return out.value


def mla_read_device_errors(stream=None) -> int:
    flags = ctypes.c_int(0)
    _check(_lib.mla_read_device_errors(ctypes.byref(flags), _stream(stream)))
    return flags.value


# ----------------------------------------------------------------------------- convenience: one decode step

class DecodePlan:
    """Split count, scheduler metadata and workspace for one decode step.

    Built once per step (the metadata depends only on the lengths) and reused by
    every layer of that step, as the scheduler metadata is meant to be."""

    def __init__(self, seqlens, s_q, h_q, kv_format=KV_BF16_PAGED, num_parts=None, stream=None, h_kv=1,
                 topk_capacity=None):
        b = seqlens.shape[0]
        self.batch, self.s_q, self.h_q, self.kv_format = b, s_q, h_q, kv_format
        self.num_parts = int(num_parts) if num_parts else mla_decode_num_parts(b, s_q, h_q, h_kv, kv_format)
        if kv_format in (KV_FP8_PACKED, KV_FP8_INDEXED):
            # the sparse paths' own scheduler call (seqlens = topk_length)
            if not topk_capacity:
                raise ValueError("DecodePlan: the FP8 formats need topk_capacity")
            self.sched_meta, self.num_splits = mla_get_packed_decode_metadata(
                seqlens, b, s_q, h_q, int(topk_capacity), self.num_parts, stream=stream)
        else:
            self.sched_meta, self.num_splits = mla_get_decode_metadata(seqlens, b, s_q, h_q, 1, self.num_parts,
                                                                       stream=stream)
        nbytes = mla_decode_workspace_size(b, s_q, h_q, self.num_parts)
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=seqlens.device)


def mla_decode(q, kv, block_table, seqlens, softmax_scale=None, causal=False, plan=None, kv_format=KV_BF16_PAGED,
               topk_capacity=0, out=None, lse=None, stream=None):
    """Metadata (unless a plan is given) -> decode -> combine.  Returns (out, lse)."""
    b, s_q, h_q, _ = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D_QK)
    if plan is None:
        h_kv = kv.shape[2] if kv_format in (KV_BF16_PAGED, KV_FP16_PAGED) else 1
        plan = DecodePlan(seqlens, s_q, h_q, kv_format, stream=stream, h_kv=h_kv, topk_capacity=topk_capacity)
    if out is None:
        out = torch.empty((b, s_q, h_q, D_V), dtype=_act_dtype(kv_format), device=q.device)
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=q.device)
    mla_decode_fwd(q, kv, kv_format, block_table, seqlens, softmax_scale, causal, plan.sched_meta, plan.num_splits,
                   out, lse, plan.workspace, topk_capacity=topk_capacity, stream=stream)
    mla_combine(plan.num_splits, plan.workspace, b, s_q, h_q, plan.num_parts, out, lse, stream=stream,
                kv_format=kv_format)
    return out, lse
