"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/mla_paged_kv.h declares, sizes workspaces by the documented
formulas, plans split counts, and rejects out-of-scope or malformed arguments
before anything is launched.

Pointer arguments here are dummies that the library never dereferences: every
call below fails validation first (it never reaches a HIP call), so the tests are
safe on a machine with or without a GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_paged_kv.h")

ops = pytest.importorskip("mla_paged_kv_amd.ops", reason="libmla_paged_kv.so not built")
lib = ops._lib
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: each call fails validation first
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(ops.EXPORTS)


def test_packed_workspace_size_matches_page_figure():
    # 2048 records x 656 B = 1,343,488 B per query row ("Runtime follow-up", FlashMLA PR 200)
    assert ops.mla_packed_kv_workspace_size(1, 1, 2048) == 1343488
    assert ops.mla_packed_kv_workspace_size(8, 1, 2048) == 8 * 1343488
    assert ops.mla_packed_kv_workspace_size(1, 1, 100) == 0   # not a multiple of 64
    assert ops.mla_packed_kv_workspace_size(0, 1, 64) == 0


def test_decode_workspace_size_formula():
    # (batch + num_parts) split slots x rows x (512 + 1) fp32
    assert ops.mla_decode_workspace_size(64, 1, 128, 256) == (64 + 256) * 128 * 513 * 4
    assert ops.mla_decode_workspace_size(1, 2, 16, 1) == 2 * 32 * 513 * 4
    assert ops.mla_decode_workspace_size(1, 1, 16, 0) == 0


@pytest.mark.parametrize("batch,s_q,h_q,cus,wgs,expect", [
    (64, 1, 128, 256, 1, 128),      # 64-row kernel: two row blocks per request -> 256 WG slots / 2
    (1, 1, 128, 256, 1, 64),        # capped at 64 pieces per request (the scheduler uses what the lengths need)
    (8, 1, 64, 256, 1, 256),        # 64-row kernel, one row block: all 256 WG slots (cap 8 x 64)
    (16, 2, 128, 256, 1, 64),       # 256 rows: four row blocks per request -> 256 / 4
    (4, 4, 128, 256, 1, 32),        # 512 rows: eight row blocks, 256 / 8
    (4, 1, 96, 256, 1, 128),        # 96 rows: two 64-row blocks (64-row kernel), 256 / 2
    (1, 1, 16, 256, 1, 64),
    (1000, 1, 128, 256, 1, 128),
])
def test_plan_num_parts(batch, s_q, h_q, cus, wgs, expect):
    assert ops.mla_plan_num_parts(batch, s_q, h_q, ops.KV_BF16_PAGED, cus, wgs) == expect


@pytest.mark.parametrize("fmt,batch,s_q,h_q,expect", [
    (ops.KV_FP8_PACKED, 8, 1, 64, 256),     # one row block per request; 32 pieces per request allowed
    (ops.KV_FP8_INDEXED, 2, 1, 128, 64),    # two row blocks: 128 slots, capped at 2 x 32
    (ops.KV_BF16_PAGED, 8, 1, 64, 256),     # the bf16 plan allows 64 per request
])
def test_plan_num_parts_fp8_cap(fmt, batch, s_q, h_q, expect):
    assert ops.mla_plan_num_parts(batch, s_q, h_q, fmt, 256, 1) == expect


@pytest.mark.parametrize("batch,s_q,h_q,h_kv", [(64, 1, 128, 2), (64, 1, 128, 4), (8, 2, 64, 4), (1, 1, 64, 4)])
def test_plan_num_parts_multi_kv_head(batch, s_q, h_q, h_kv):
    """Row blocks are counted per KV head: h_kv * ceil(s_q * h_q / h_kv / rows per workgroup)."""
    mkv = s_q * (h_q // h_kv)
    rb = 16 * (1 if mkv <= 16 else 2 if mkv <= 32 else 4)
    row_blocks = h_kv * ((mkv + rb - 1) // rb)
    want = min(max(256 // row_blocks, 1), batch * 64)
    assert ops.mla_plan_num_parts(batch, s_q, h_q, ops.KV_BF16_PAGED, 256, 1, h_kv=h_kv) == want


@pytest.mark.parametrize("s_q,h_q,h_kv,fmt,name", [
    (1, 128, 1, ops.KV_BF16_PAGED, "decode_ws_kernel<4, false, false>"),   # 128 rows: two 64-row workgroups
    (1, 16, 1, ops.KV_BF16_PAGED, "decode_ws_kernel<1, false, false>"),
    (1, 32, 1, ops.KV_FP16_PAGED, "decode_ws_kernel<2, true, false>"),
    (2, 128, 1, ops.KV_BF16_PAGED, "decode_ws_kernel<4, false, false>"),  # 256 rows: four 64-row workgroups
    (4, 128, 1, ops.KV_FP16_PAGED, "decode_ws_kernel<4, true, false>"),
    (2, 128, 2, ops.KV_BF16_PAGED, "decode_ws_kernel<4, false, true>"),    # several KV heads
    (1, 64, 1, ops.KV_FP8_PACKED, "decode_fp8ws_kernel<false>"),
    (16, 128, 1, ops.KV_FP8_INDEXED, "decode_fp8ws_kernel<true>"),
])
def test_decode_kernel_name(s_q, h_q, h_kv, fmt, name):
    assert ops.mla_decode_kernel_name(s_q, h_q, h_kv, fmt) == name


def test_decode_kernel_name_rejects_unsupported_shape():
    with pytest.raises(ops.MLAError):
        ops.mla_decode_kernel_name(1, 24, 1, ops.KV_BF16_PAGED)


def decode_call(**kw):
    args = dict(q=FAKE, kv=FAKE, fmt=ops.KV_BF16_PAGED, num_pages=16, bt=FAKE, max_pages=4, seqlens=FAKE, cap=0,
                batch=2, s_q=1, h_q=128, h_kv=1, scale=0.04, causal=0, meta=FAKE, ns=FAKE, parts=8, out=FAKE,
                lse=FAKE, ws=FAKE, ws_bytes=1 << 40, stream=NULL)
    args.update(kw)
    st = lib.mla_decode_fwd(args["q"], args["kv"], args["fmt"], args["num_pages"], args["bt"], args["max_pages"],
                            args["seqlens"], args["cap"], args["batch"], args["s_q"], args["h_q"], args["h_kv"],
                            args["scale"], args["causal"], args["meta"], args["ns"], args["parts"], args["out"],
                            args["lse"], args["ws"], args["ws_bytes"], args["stream"])
    return st, ops.mla_last_error_message()


@pytest.mark.parametrize("kw,status", [
    (dict(h_kv=3), ops.MLA_ERR_UNSUPPORTED),              # does not divide h_q = 128
    (dict(h_kv=0), ops.MLA_ERR_UNSUPPORTED),
    (dict(h_kv=32, h_q=128), ops.MLA_ERR_UNSUPPORTED),    # above 16
    (dict(fmt=ops.KV_FP8_PACKED, cap=2048, h_q=128, h_kv=2), ops.MLA_ERR_UNSUPPORTED),
    (dict(h_q=17), ops.MLA_ERR_UNSUPPORTED),
    (dict(h_q=144), ops.MLA_ERR_UNSUPPORTED),
    (dict(s_q=17, h_q=128), ops.MLA_ERR_UNSUPPORTED),     # 2176 rows > 2048
    (dict(fmt=7), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP16_PAGED, h_kv=5), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP16_PAGED, h_q=136), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP16_PAGED, bt=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(fmt=ops.KV_FP8_PACKED, cap=2048, h_q=96), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_PACKED, cap=2000, h_q=64), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_PACKED, cap=2048, h_q=128, s_q=17), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_PACKED, cap=2048, h_q=64, causal=1), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=96), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=100, h_q=64), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=64, s_q=33), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=128, causal=1), ops.MLA_ERR_UNSUPPORTED),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=128, bt=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=128, num_pages=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(fmt=ops.KV_FP8_INDEXED, cap=2048, h_q=128, num_pages=1 << 60), ops.MLA_ERR_UNSUPPORTED),
    (dict(batch=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(batch=9000), ops.MLA_ERR_UNSUPPORTED),
    (dict(s_q=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(q=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(out=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(bt=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(max_pages=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(parts=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(parts=100000), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.04), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=100), ops.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=NULL), ops.MLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_fails_closed(kw, status):
    st, msg = decode_call(**kw)
    assert st == status, msg
    assert msg


def test_metadata_and_combine_and_pack_fail_closed():
    assert lib.mla_get_decode_metadata(NULL, 2, 1, 128, 1, 8, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_get_decode_metadata(FAKE, 2, 1, 128, 1, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_get_decode_metadata(FAKE, 2, 1, 128, 3, 8, FAKE, FAKE, NULL) == ops.MLA_ERR_UNSUPPORTED
    assert lib.mla_combine(FAKE, FAKE, 10, 2, 1, 128, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_combine(NULL, FAKE, 1 << 40, 2, 1, 128, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_combine(FAKE, FAKE, 1 << 40, 2, 1, 128, 8, 9, FAKE, FAKE, NULL) == ops.MLA_ERR_UNSUPPORTED
    assert lib.mla_pack_selected_kv(FAKE, 16, FAKE, FAKE, 2, 1, 100, FAKE, 1 << 40, NULL) == ops.MLA_ERR_UNSUPPORTED
    assert lib.mla_pack_selected_kv(FAKE, 16, FAKE, FAKE, 2, 1, 128, FAKE, 10, NULL) == ops.MLA_ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_pack_selected_kv(FAKE, 0, FAKE, FAKE, 2, 1, 128, FAKE, 1 << 40, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert "multiple of 64" in ops.mla_last_error_message() or ops.mla_last_error_message()
    out = ctypes.c_int(0)
    assert lib.mla_plan_num_parts(1, 1, 128, 1, 0, 0, 1, ctypes.byref(out)) == ops.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_num_parts(1, 1, 128, 3, 0, ctypes.byref(out)) == ops.MLA_ERR_UNSUPPORTED


def test_sparse_kv_format_policy():
    need = ops.mla_packed_kv_workspace_size(8, 1, 2048)
    assert need == 8 * 2048 * 656
    assert ops.mla_sparse_kv_format(8, 1, 2048, need, True) == ops.KV_FP8_PACKED
    assert ops.mla_sparse_kv_format(8, 1, 2048, need - 1, True) == ops.KV_FP8_INDEXED  # over the budget
    assert ops.mla_sparse_kv_format(8, 1, 2048, 1 << 40, False) == ops.KV_FP8_INDEXED  # pack not hidden
    assert ops.mla_sparse_kv_format(2, 4, 128, 1 << 40, True) == ops.KV_FP8_PACKED
    out = ctypes.c_int(0)
    assert lib.mla_sparse_kv_format(8, 1, 100, 1 << 40, 1, ctypes.byref(out)) == ops.MLA_ERR_UNSUPPORTED
    assert lib.mla_sparse_kv_format(0, 1, 2048, 1 << 40, 1, ctypes.byref(out)) == ops.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_sparse_kv_format(8, 1, 2048, 1 << 40, 1, NULL) == ops.MLA_ERR_INVALID_ARGUMENT


def patch_call(**kw):
    args = dict(kv=FAKE, num_pages=16, idx=FAKE, tl=FAKE, batch=2, s_q=1, cap=128, ids=FAKE, n_new=1, ws=FAKE,
                ws_bytes=1 << 40, stream=NULL)
    args.update(kw)
    return lib.mla_patch_packed_kv(args["kv"], args["num_pages"], args["idx"], args["tl"], args["batch"], args["s_q"],
                                   args["cap"], args["ids"], args["n_new"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kv=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(ids=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(ws=NULL), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(n_new=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(n_new=65), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(batch=0), ops.MLA_ERR_INVALID_ARGUMENT),
    (dict(cap=100), ops.MLA_ERR_UNSUPPORTED),
    (dict(num_pages=1 << 40), ops.MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=2 * 128 * 656 - 1), ops.MLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_patch_fails_closed(kw, status):
    assert patch_call(**kw) == status
    assert ops.mla_last_error_message()


def test_packed_metadata_fails_closed():
    f = lib.mla_get_packed_decode_metadata
    assert f(NULL, 2, 1, 64, 2048, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 1, 64, 2048, 0, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 1, 64, 2048, 8, 3, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT   # unknown policy
    assert f(FAKE, 2, 1, 96, 2048, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_UNSUPPORTED        # h_q not 64/128
    assert f(FAKE, 2, 1, 64, 100, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_UNSUPPORTED         # capacity
    assert f(FAKE, 0, 1, 64, 2048, 8, 0, FAKE, FAKE, NULL) == ops.MLA_ERR_INVALID_ARGUMENT


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros((1, 1, 16, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops._need(q, "q", torch.bfloat16)
