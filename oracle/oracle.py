"""CPU fp64 oracle for MLA decode over a paged KV cache (test infrastructure).

TEST INFRASTRUCTURE ONLY: the slow, plain reference that the GPU library is
checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library (``mla_paged_kv_amd``) and neither imports the other.

The arithmetic lives in ``mla_oracle.c`` (plain C, IEEE double, pthreads);
this module compiles it with gcc on first use and wraps it with ctypes.  The
scheduler partition (``sched_partition``) is integer bookkeeping and is written
here in plain Python, one block at a time.

Sources (page titles; the pages are the FlashMLA pull requests):
  * "Add SM80 (Ampere/A100) dense MLA decode kernel" -- Summary and Design:
    dense MLA decode, 576-dim latent K shared by all query heads, V = its first
    512 dims, 64-token pages, causal mask for multi-token queries, split-K
    partials merged by a combine kernel; Test plan: split-K via the combine.
  * "[SM90] Add packed selected-KV sparse decode" -- "SM90 packing kernel":
    656-byte record (512 B E4M3 NoPE, 16 B = 4 fp32 scales, 128 B = 64 bf16
    RoPE), byte-for-byte pack into 64-token tiles with a zero-filled invalid
    suffix; "Packed attention specialization": partial-tail masking.

Parity status: every function here is pinned by the tests in
``tests/test_oracle.py`` (brute force, closed forms, invariants, exhaustive
E4M3 table, byte counts the pages print).  None is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

D_QK = 576
D_V = 512
PAGE = 64
REC_BYTES = 656

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile mla_oracle.c into libmla_oracle.so next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3fn_to_f64.restype = f64
            lib.oracle_mla_decode.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, f64, i32, P, P, i32]
            lib.oracle_mla_decode.restype = i32
            lib.oracle_mla_decode_f16.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, f64, i32, P, P, i32]
            lib.oracle_mla_decode_f16.restype = i32
            lib.oracle_mla_decode_hkv.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, i32, i32, f64, i32, P, P, i32]
            lib.oracle_mla_decode_hkv.restype = i32
            lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_f64.restype = f64
            lib.oracle_mla_decode_partial.argtypes = [P, P, i64, P, i32, P, i32, i32, i32, f64, i32, P, P, P, P, i32]
            lib.oracle_mla_decode_partial.restype = i32
            lib.oracle_lse_combine.argtypes = [i32, P, P, P, P]
            lib.oracle_lse_combine.restype = i32
            lib.oracle_mla_sparse_decode.argtypes = [P, P, i64, P, P, i32, i32, i32, i32, f64, P, P, i32]
            lib.oracle_mla_sparse_decode.restype = i32
            lib.oracle_decode_record.argtypes = [P, i64, i64, P]
            lib.oracle_decode_record.restype = i32
            lib.oracle_pack_selected_kv.argtypes = [P, i64, P, P, i32, i32, i32, P]
            lib.oracle_pack_selected_kv.restype = i32
            _lib = lib
    return _lib


MAX_THREADS = 16  # the CPU share of one GPU on the machines this runs on


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check(st: int, what: str):
    if st != 0:
        names = {1: "bad argument", 2: "page id out of range", 3: "token index out of range", 4: "out of memory"}
        raise ValueError(f"oracle {what}: {names.get(st, st)}")


def e4m3fn_to_f64(code: int) -> float:
    """Decode one OCP E4M3FN byte (bias 7, subnormals, NaN = S.1111.111, no inf)."""
    return _load().oracle_e4m3fn_to_f64(int(code) & 0xFF)


def f16_to_f64(code: int) -> float:
    """IEEE binary16 bit pattern -> float (exact)."""
    return _load().oracle_f16_to_f64(int(code) & 0xFFFF)


def mla_decode(q_bits, kcache_bits, block_table, seqlens, scale, causal, nthreads=None, dtype="bf16"):
    """Dense decode.  q_bits uint16 [b, s_q, h_q, 576] (bf16 bit patterns, or
    IEEE binary16 ones with dtype="fp16"); kcache_bits uint16 [pages, 64, h_kv, 576]
    (same encoding; query head h reads KV head h // (h_q // h_kv)); block_table
    int32 [b, max_pages]; seqlens int32 [b].
    Returns (out fp64 [b, s_q, h_q, 512], lse fp64 [b, s_q, h_q])."""
    assert dtype in ("bf16", "fp16")
    h_kv = kcache_bits.shape[2]
    if h_kv != 1:
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kcache_bits = np.ascontiguousarray(kcache_bits, dtype=np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
        b, s_q, h_q, _ = q_bits.shape
        assert kcache_bits.shape[1] == PAGE and kcache_bits.shape[3] == D_QK and h_q % h_kv == 0
        out = np.zeros((b, s_q, h_q, D_V), np.float64)
        lse = np.zeros((b, s_q, h_q), np.float64)
        st = _load().oracle_mla_decode_hkv(
            _ptr(q_bits), _ptr(kcache_bits), kcache_bits.shape[0], _ptr(block_table), block_table.shape[1],
            _ptr(seqlens), b, s_q, h_q, h_kv, int(dtype == "fp16"), float(scale), int(bool(causal)), _ptr(out),
            _ptr(lse), nthreads or default_threads())
        _check(st, "mla_decode")
        return out, lse
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kcache_bits = np.ascontiguousarray(kcache_bits, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    b, s_q, h_q, d = q_bits.shape
    assert d == D_QK and kcache_bits.shape[1:] == (PAGE, 1, D_QK)
    assert block_table.shape[0] == b and seqlens.shape == (b,)
    out = np.zeros((b, s_q, h_q, D_V), np.float64)
    lse = np.zeros((b, s_q, h_q), np.float64)
    fn = _load().oracle_mla_decode if dtype == "bf16" else _load().oracle_mla_decode_f16
    st = fn(
        _ptr(q_bits), _ptr(kcache_bits), kcache_bits.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), b, s_q, h_q, float(scale), int(bool(causal)), _ptr(out), _ptr(lse),
        nthreads or default_threads())
    _check(st, "mla_decode")
    return out, lse


def mla_decode_partial(q_bits, kcache_bits, block_table, seqlens, scale, causal, split_lo, split_hi, nthreads=None):
    """Partial attention over keys j in [split_lo[r], split_hi[r]) of each request
    (intersected with the visible range).  Returns normalised (o, lse)."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kcache_bits = np.ascontiguousarray(kcache_bits, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    lo = np.ascontiguousarray(split_lo, dtype=np.int32)
    hi = np.ascontiguousarray(split_hi, dtype=np.int32)
    b, s_q, h_q, _ = q_bits.shape
    out = np.zeros((b, s_q, h_q, D_V), np.float64)
    lse = np.zeros((b, s_q, h_q), np.float64)
    st = _load().oracle_mla_decode_partial(
        _ptr(q_bits), _ptr(kcache_bits), kcache_bits.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), b, s_q, h_q, float(scale), int(bool(causal)), _ptr(lo), _ptr(hi), _ptr(out), _ptr(lse),
        nthreads or default_threads())
    _check(st, "mla_decode_partial")
    return out, lse


def lse_combine(o, lse):
    """Merge partials of one row: o [S, 512], lse [S] -> (out [512], lse)."""
    o = np.ascontiguousarray(o, dtype=np.float64).reshape(-1, D_V)
    lse = np.ascontiguousarray(lse, dtype=np.float64).reshape(-1)
    out = np.zeros(D_V, np.float64)
    lse_out = np.zeros(1, np.float64)
    _check(_load().oracle_lse_combine(lse.shape[0], _ptr(o), _ptr(lse), _ptr(out), _ptr(lse_out)), "lse_combine")
    return out, float(lse_out[0])


def mla_sparse_decode(q_bits, kcache_rec, indices, topk_length, scale, nthreads=None):
    """Sparse decode over top-k FP8 records.  kcache_rec uint8 [pages, 64, 1, 656];
    indices int32 [b, s_q, cap] (physical token ids); topk_length int32 [b]."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kcache_rec = np.ascontiguousarray(kcache_rec, dtype=np.uint8)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    topk_length = np.ascontiguousarray(topk_length, dtype=np.int32)
    b, s_q, h_q, _ = q_bits.shape
    cap = indices.shape[2]
    assert kcache_rec.shape[1:] == (PAGE, 1, REC_BYTES) and indices.shape[:2] == (b, s_q)
    out = np.zeros((b, s_q, h_q, D_V), np.float64)
    lse = np.zeros((b, s_q, h_q), np.float64)
    st = _load().oracle_mla_sparse_decode(
        _ptr(q_bits), _ptr(kcache_rec), kcache_rec.shape[0], _ptr(indices), _ptr(topk_length), b, s_q, h_q, cap,
        float(scale), _ptr(out), _ptr(lse), nthreads or default_threads())
    _check(st, "mla_sparse_decode")
    return out, lse


def decode_record(kcache_rec, phys):
    """Dequantised key (fp64 [576]) of the record at physical token id `phys`."""
    kcache_rec = np.ascontiguousarray(kcache_rec, dtype=np.uint8)
    k = np.zeros(D_QK, np.float64)
    _check(_load().oracle_decode_record(_ptr(kcache_rec), kcache_rec.shape[0], int(phys), _ptr(k)), "decode_record")
    return k


def pack_selected_kv(kcache_rec, indices, topk_length):
    """Byte-exact pack.  Returns uint8 [b * s_q, cap / 64, 64, 656]."""
    kcache_rec = np.ascontiguousarray(kcache_rec, dtype=np.uint8)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    topk_length = np.ascontiguousarray(topk_length, dtype=np.int32)
    b, s_q, cap = indices.shape
    ws = np.empty((b * s_q, cap // PAGE, PAGE, REC_BYTES), np.uint8)
    st = _load().oracle_pack_selected_kv(
        _ptr(kcache_rec), kcache_rec.shape[0], _ptr(indices), _ptr(topk_length), b, s_q, cap, _ptr(ws))
    _check(st, "pack_selected_kv")
    return ws


# --------------------------------------------------------------------------- scheduler
#
# The pages fix only that a request's KV range is split over several
# workgroups whose partial results a combine step merges, and that the number
# of partitions is a launch-time count (FlashMLA PR 183, "How the occupancy
# work went").  The partition rule itself is this library's reading, stated
# here as a definition:
#
#   blocks_r = ceil(max(len_r, 0) / 64), T = sum_r blocks_r, P' = min(P, T, L)
#   with L an optional split limit (the dense metadata call uses
#   dense_split_limit below; the packed call uses none, L = T).
#   Concatenate all requests' blocks in request order; part p < P' owns the
#   global blocks [floor(p*T/P'), floor((p+1)*T/P')) (at least one block each),
#   parts p >= P' own nothing.  A request's split count is the number of parts
#   that own at least one of its blocks; its splits take consecutive workspace
#   slots in part order, after the slots of all earlier requests.


def dense_split_limit(batch, total_blocks):
    """Split limit of the dense metadata call: at least 16 parts per request,
    more when the requests are long (one part per 4 blocks), at most 64 per
    request: max(16 b, min(ceil(T / 4), 64 b))."""
    b, T = int(batch), int(total_blocks)
    return max(16 * b, min(-(-T // 4), 64 * b))


def sched_partition(lengths, num_parts, split_limit=None):
    """Plain-Python scheduler oracle.

    Returns (meta int32 [P, 8], num_splits int32 [b + 1]) with, per part:
      meta[p] = [begin_req, begin_blk, end_req, end_blk_exclusive, begin_split, 0, 0, 0]
    and begin_req = -1 (all fields -1 except the zeros) for a part that owns no
    block.  num_splits is the exclusive prefix sum of per-request split counts.
    split_limit: "dense" for the dense metadata call's limit, None for none, or
    an int.
    """
    lengths = [max(int(x), 0) for x in lengths]
    P = int(num_parts)
    assert P >= 1
    blocks = [(n + PAGE - 1) // PAGE for n in lengths]
    T = sum(blocks)
    if split_limit == "dense":
        split_limit = dense_split_limit(len(lengths), T)
    Pe = min(P, T) if split_limit is None else min(P, T, int(split_limit))
    # owner of every global block, found by scanning the part boundaries
    bounds = [(p * T) // Pe for p in range(Pe + 1)] if Pe else [0]
    owner = []
    for g in range(T):
        p = 0
        while not (bounds[p] <= g < bounds[p + 1]):
            p += 1
        owner.append(p)
    # (request, block-in-request) of every global block
    where = []
    for r, nb in enumerate(blocks):
        for k in range(nb):
            where.append((r, k))
    # split counts: distinct owners of each request's blocks
    splits = []
    first_part = []
    g = 0
    for r, nb in enumerate(blocks):
        owners = sorted(set(owner[g:g + nb]))
        splits.append(len(owners))
        first_part.append(owners[0] if owners else -1)
        g += nb
    num_splits = np.zeros(len(lengths) + 1, np.int32)
    for r, s in enumerate(splits):
        num_splits[r + 1] = num_splits[r] + s
    meta = np.zeros((P, 8), np.int32)
    for p in range(P):
        mine = [i for i in range(T) if owner[i] == p]
        if not mine:
            meta[p, :5] = -1
            continue
        br, bk = where[mine[0]]
        er, ek = where[mine[-1]]
        meta[p, :5] = [br, bk, er, ek + 1, p - first_part[br]]
    return meta, num_splits


def sched_partition_request_local(lengths, num_parts):
    """Request-local partition (the "compact request-local scheduler" of "[SM90]
    Add packed selected-KV sparse decode", Scheduler policy; the page names it
    without defining it, so this is the reading: no part spans two requests).

    blocks_r = ceil(len_r / 64).  If more requests have a block than there are
    parts, returns None (the form needs one part per such request).  Otherwise
    B = the smallest piece size in blocks with sum_r ceil(blocks_r / B) <= P;
    request r gets n_r = ceil(blocks_r / B) pieces, piece i covering blocks
    [floor(i * b_r / n_r), floor((i + 1) * b_r / n_r)); parts are numbered in
    (request, piece) order and the parts after the last piece are empty.
    Same output format as sched_partition.
    """
    lengths = [max(int(x), 0) for x in lengths]
    P = int(num_parts)
    assert P >= 1
    blocks = [(n + PAGE - 1) // PAGE for n in lengths]
    T = sum(blocks)
    nonempty = sum(1 for x in blocks if x)
    if nonempty > P:
        return None
    meta = np.zeros((P, 8), np.int32)
    meta[:, :5] = -1
    num_splits = np.zeros(len(lengths) + 1, np.int32)
    if T == 0:
        return meta, num_splits
    B = (T + P - 1) // P
    while sum((x + B - 1) // B for x in blocks) > P:
        B += 1
    part = 0
    for r, nb in enumerate(blocks):
        n = (nb + B - 1) // B
        for i in range(n):
            meta[part, :5] = [r, (i * nb) // n, r, ((i + 1) * nb) // n, i]
            part += 1
        num_splits[r + 1] = num_splits[r] + n
    return meta, num_splits
