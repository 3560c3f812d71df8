"""The decode entry point that allocates nothing (mla_decode_fwd_noalloc).

Its split partials live in the library's own device scratch instead of a caller
workspace.  Called through the C ABI, it must give bit for bit what
mla_decode_fwd + mla_combine give with a caller workspace (same kernels, same
partition), and match the oracle -- on two calls in a row, the second with a
smaller input, so that stale scratch contents from the first call cannot leak
into the second.
"""

import numpy as np
import pytest
import torch

from mla_paged_kv_amd import workloads as W
from oracle import oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

ops = pytest.importorskip("mla_paged_kv_amd.ops")


def _with_workspace(w, t, fmt, parts, kv, ix):
    b, s_q, h_q = w.batch, w.s_q, w.h_q
    meta, ns = ops.mla_get_decode_metadata(t["seqlens"], b, s_q, h_q, 1, parts)
    ws = torch.empty((ops.mla_decode_workspace_size(b, s_q, h_q, parts),), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device="cuda:0")
    ops.mla_decode_fwd(t["q"], kv, fmt, ix, t["seqlens"], w.scale, w.causal, meta, ns, out, lse, ws,
                       topk_capacity=w.topk_capacity)
    ops.mla_combine(ns, ws, b, s_q, h_q, parts, out, lse, kv_format=fmt)
    return meta, ns, out, lse


def _noalloc(w, t, fmt, meta, ns, kv, ix):
    b, s_q, h_q = w.batch, w.s_q, w.h_q
    out = torch.full((b, s_q, h_q, 512), 3.0, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((b, s_q, h_q), 3.0, dtype=torch.float32, device="cuda:0")
    ops.mla_decode_fwd_noalloc(t["q"], kv, fmt, ix, t["seqlens"], w.scale, w.causal, meta, ns, out, lse,
                               topk_capacity=w.topk_capacity)
    return out, lse


def test_noalloc_dense_two_calls_second_smaller():
    cases = [
        W.dense_workload("noalloc-1", 210, 4, 1, 128, [4096, 2049, 700, 1], pool_pages=120),
        W.dense_workload("noalloc-2", 211, 2, 2, 64, [300, 65], pool_pages=8, causal=True),
    ]
    for w in cases:
        G.say(f"no-alloc dense {w.name}: batch {w.batch}, s_q {w.s_q}, h_q {w.h_q}")
        t = G.dev_tensors(w)
        parts = ops.mla_decode_num_parts(w.batch, w.s_q, w.h_q, 1, ops.KV_BF16_PAGED)
        assert ops.mla_decode_workspace_size(w.batch, w.s_q, w.h_q, parts) <= ops.NOALLOC_SCRATCH_BYTES
        meta, ns, ref_o, ref_l = _with_workspace(w, t, ops.KV_BF16_PAGED, parts, t["kcache"], t["block_table"])
        out, lse = _noalloc(w, t, ops.KV_BF16_PAGED, meta, ns, t["kcache"], t["block_table"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        G.compare(w.name, out, lse, *O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale,
                                                    w.causal))


def test_noalloc_sparse_two_calls_second_smaller():
    cases = [
        W.sparse_workload("noalloc-fp8-1", 212, 4, 128, 512, [512, 300, 65, 512], context=4096),
        W.sparse_workload("noalloc-fp8-2", 213, 1, 64, 128, [100], context=1024),
    ]
    for w in cases:
        G.say(f"no-alloc fp8 by index {w.name}: batch {w.batch}, h_q {w.h_q}")
        t = G.dev_tensors(w)
        parts = ops.mla_decode_num_parts(w.batch, w.s_q, w.h_q, 1, ops.KV_FP8_INDEXED)
        meta, ns, ref_o, ref_l = _with_workspace(w, t, ops.KV_FP8_INDEXED, parts, t["kcache_rec"], t["indices"])
        out, lse = _noalloc(w, t, ops.KV_FP8_INDEXED, meta, ns, t["kcache_rec"], t["indices"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        G.compare(w.name, out, lse, *O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale))


def test_noalloc_rejects_partials_above_the_scratch():
    """A split count whose partials exceed the scratch is refused before any launch."""
    w = W.dense_workload("noalloc-big", 214, 2, 1, 128, [64, 64], pool_pages=2)
    t = G.dev_tensors(w)
    parts = 2100  # (2 + 2100) slots x 128 rows x 513 x 4 B > 128 MiB
    assert ops.mla_decode_workspace_size(2, 1, 128, parts) > ops.NOALLOC_SCRATCH_BYTES
    meta = torch.zeros((parts, 8), dtype=torch.int32, device="cuda:0")
    ns = torch.zeros((3,), dtype=torch.int32, device="cuda:0")
    out = torch.empty((2, 1, 128, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((2, 1, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ops.MLAError) as ei:
        ops.mla_decode_fwd_noalloc(t["q"], t["kcache"], ops.KV_BF16_PAGED, t["block_table"], t["seqlens"], w.scale,
                                   False, meta, ns, out, lse)
    assert ei.value.status == ops.MLA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in str(ei.value)
