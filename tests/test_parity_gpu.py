"""GPU parity: the HIP library (through its C ABI) against the CPU fp64 oracle.

Tolerances: out |gpu - ref| <= 1e-2 + 1e-2 |ref| element-wise (bf16 output),
lse |gpu - ref| <= 1e-3 (fp32), plus a relative-RMS alarm at 1e-2 because some
workloads' output RMS is below the absolute tolerance.  Integer and byte
results (scheduler records, packed workspace) must match exactly.
"""

import numpy as np
import pytest
import torch

from mla_paged_kv_amd import workloads as W
from oracle import oracle as O
from tests import gpu_helpers as G
from tests import rescale_rule as RR

pytestmark = pytest.mark.gpu

ops = pytest.importorskip("mla_paged_kv_amd.ops")


def oracle_dense(w):
    return O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, dtype=w.dtype)


def oracle_sparse(w):
    return O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)


# ----------------------------------------------------------------------------- scheduler

@pytest.mark.parametrize("lengths,P", [
    ([4096] * 64, 128), ([4096] * 3, 7), ([1, 64, 65, 0, 300], 4), ([0, 0], 3), ([10], 5),
    ([2048, 4096, 3000, 100], 9), ([64] * 5, 5), ([128, 64], 1), ([16384] * 16, 64),
    (list(np.random.default_rng(7).integers(0, 5000, size=300)), 200),
    ([1, 700, 2049], 64), ([300, 10, 0, 640], 50), ([4096], 256),
])
def test_sched_metadata_bit_exact(lengths, P):
    G.say(f"sched lengths[{len(lengths)}] P={P}")
    seq = torch.tensor(np.asarray(lengths, np.int32), device="cuda:0")
    meta, ns = ops.mla_get_decode_metadata(seq, len(lengths), 1, 128, 1, P)
    torch.cuda.synchronize()
    ref_meta, ref_ns = O.sched_partition(lengths, P, split_limit="dense")
    assert np.array_equal(meta.cpu().numpy(), ref_meta)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)


# ----------------------------------------------------------------------------- dense decode

DENSE_SMALL = [
    # name, seed, batch, s_q, h_q, seqlens, pool_pages, causal, num_parts
    ("one-page", 101, 1, 1, 16, [64], 2, False, 1),
    ("ragged-b3-h128", 102, 3, 1, 128, [1, 700, 2049], 60, False, None),
    ("ragged-b3-h128-p1", 102, 3, 1, 128, [1, 700, 2049], 60, False, 1),
    ("ragged-b3-h128-p5", 102, 3, 1, 128, [1, 700, 2049], 60, False, 5),
    ("ragged-b3-h128-p64", 102, 3, 1, 128, [1, 700, 2049], 60, False, 64),
    ("h16", 103, 2, 1, 16, [333, 64], 8, False, None),
    ("h32", 104, 2, 1, 32, [333, 65], 8, False, None),
    ("h48", 105, 2, 1, 48, [31, 500], 10, False, 3),
    ("h64", 106, 2, 1, 64, [129, 257], 10, False, None),
    ("h80", 107, 2, 1, 80, [1000, 7], 20, False, 4),
    ("h112", 108, 1, 1, 112, [777], 13, False, None),
    ("empty-request", 109, 3, 1, 64, [0, 50, 0], 2, False, None),
    ("causal-sq2-h128", 110, 3, 2, 128, [1, 100, 1000], 20, True, None),
    ("causal-sq2-h64-p1", 111, 2, 2, 64, [2, 95], 4, True, 1),
    ("causal-sq4-h64", 112, 2, 4, 64, [3, 300], 8, True, 6),
    ("noncausal-sq2-h128", 113, 2, 2, 128, [250, 64], 6, False, None),
    ("causal-sq4-h128", 114, 2, 4, 128, [4, 700], 12, True, None),        # 512 rows per request
    ("causal-sq16-h128-p3", 115, 1, 16, 128, [600], 10, True, 3),         # 2048 rows, the row cap
    ("causal-sq8-h48", 116, 2, 8, 48, [8, 200], 6, True, None),           # rows not a multiple of 64
]


@pytest.mark.parametrize("case", DENSE_SMALL, ids=[c[0] for c in DENSE_SMALL])
def test_dense_small(case):
    name, seed, b, s_q, h_q, seqlens, pool, causal, parts = case
    G.say(f"dense {name}")
    w = W.dense_workload(name, seed, b, s_q, h_q, seqlens, pool_pages=pool, causal=causal, num_parts=parts)
    out, lse, plan = G.run_dense(w)
    ref = oracle_dense(w)
    G.compare(name, out, lse, *ref)


DENSE_FP16 = [
    # name, seed, b, s_q, h_q, seqlens, pool pages, causal, forced parts, std
    ("fp16-ragged-h128", 120, 3, 1, 128, [1, 700, 2049], 60, False, None, 1.0),
    ("fp16-ragged-h128-p7", 121, 3, 1, 128, [64, 1000, 333], 40, False, 7, 1.0),
    ("fp16-h16", 122, 2, 1, 16, [333, 64], 8, False, None, 1.0),
    ("fp16-h48-p3", 123, 2, 1, 48, [31, 500], 10, False, 3, 1.0),
    ("fp16-causal-sq4-h64", 124, 2, 4, 64, [3, 300], 8, True, None, 1.0),
    ("fp16-large-values", 125, 2, 1, 128, [500, 129], 12, False, None, 8.0),  # scores far from 0, |x| up to ~40
]


@pytest.mark.parametrize("case", DENSE_FP16, ids=[c[0] for c in DENSE_FP16])
def test_dense_fp16(case):
    name, seed, b, s_q, h_q, seqlens, pool, causal, parts, std = case
    G.say(f"dense fp16 {name}")
    w = W.dense_workload(name, seed, b, s_q, h_q, seqlens, pool_pages=pool, causal=causal, num_parts=parts, std=std,
                         dtype="fp16")
    out, lse, plan = G.run_dense(w)
    assert out.dtype == torch.float16
    G.compare(name, out, lse, *oracle_dense(w))


DENSE_MULTI_KV = [
    # name, seed, b, s_q, h_q, h_kv, seqlens, pool pages, causal, forced parts, dtype
    ("hkv2-h128", 130, 3, 1, 128, 2, [1, 700, 2049], 60, False, None, "bf16"),
    ("hkv4-h128-p5", 131, 2, 1, 128, 4, [300, 1000], 24, False, 5, "bf16"),
    ("hkv4-h64-causal-sq3", 132, 2, 3, 64, 4, [5, 400], 10, True, None, "bf16"),
    ("hkv3-h48", 133, 2, 1, 48, 3, [129, 64], 6, False, None, "bf16"),
    ("hkv2-h128-fp16", 134, 2, 2, 128, 2, [64, 900], 20, True, 3, "fp16"),
]


@pytest.mark.parametrize("case", DENSE_MULTI_KV, ids=[c[0] for c in DENSE_MULTI_KV])
def test_dense_multi_kv_head(case):
    """Several KV heads against the oracle, and each query-head group bitwise
    equal to an h_kv = 1 decode of that group over its own KV head."""
    name, seed, b, s_q, h_q, h_kv, seqlens, pool, causal, parts, dtype = case
    G.say(f"dense multi-KV-head {name}")
    w = W.dense_workload(name, seed, b, s_q, h_q, seqlens, pool_pages=pool, causal=causal, num_parts=parts,
                         dtype=dtype, h_kv=h_kv)
    t = G.dev_tensors(w)
    fmt = ops.KV_FP16_PAGED if dtype == "fp16" else ops.KV_BF16_PAGED
    P = parts or ops.mla_decode_num_parts(b, s_q, h_q, h_kv, fmt)
    plan = ops.DecodePlan(t["seqlens"], s_q, h_q, fmt, num_parts=P, h_kv=h_kv)
    out, lse = ops.mla_decode(t["q"], t["kcache"], t["block_table"], t["seqlens"], w.scale, w.causal, plan=plan,
                              kv_format=fmt)
    torch.cuda.synchronize()
    G.compare(name, out, lse, *oracle_dense(w))
    g = h_q // h_kv
    for kk in range(h_kv):
        qg = t["q"][:, :, kk * g:(kk + 1) * g].contiguous()
        kg = t["kcache"][:, :, kk:kk + 1].contiguous()
        plan1 = ops.DecodePlan(t["seqlens"], s_q, g, fmt, num_parts=P)
        o1, l1 = ops.mla_decode(qg, kg, t["block_table"], t["seqlens"], w.scale, w.causal, plan=plan1, kv_format=fmt)
        torch.cuda.synchronize()
        og, lg = out[:, :, kk * g:(kk + 1) * g], lse[:, :, kk * g:(kk + 1) * g]
        assert torch.equal(o1, og) and torch.equal(l1, lg)


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_named_small_configs(cfg):
    G.say(f"config {cfg}")
    w = W.config(cfg)
    out, lse, plan = G.run_dense(w)
    G.say(f"  num_parts={plan.num_parts}")
    G.compare(cfg, out, lse, *oracle_dense(w))


def test_split_invariance_c2():
    G.say("split invariance c2")
    w = W.config("c2")
    ref = oracle_dense(w)
    t = G.dev_tensors(w)
    outs = []
    for parts in (1, 2, 7, 16, 64, 128):
        out, lse, _ = G.run_dense(w, t, num_parts=parts)
        G.compare(f"c2-parts{parts}", out, lse, *ref)
        outs.append(out.float().cpu().numpy())
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2e-2


def test_bitwise_determinism_and_page_permutation():
    G.say("determinism + page permutation")
    w = W.dense_workload("perm", 120, 2, 1, 128, [1500, 333], pool_pages=40, num_parts=6)
    a = G.run_dense(w)
    b = G.run_dense(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    perm = np.random.default_rng(1).permutation(40)
    inv = np.argsort(perm).astype(np.int32)
    w2 = G.sub_workload(w, [0, 1])
    w2.kcache_bits = np.ascontiguousarray(w.kcache_bits[perm])
    w2.block_table = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    c = G.run_dense(w2)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_nan_in_unreadable_slots_does_not_leak():
    G.say("NaN sentinel")
    w = W.dense_workload("nan", 121, 2, 1, 64, [70, 129], pool_pages=6)
    ref = oracle_dense(w)  # the oracle never reads those slots
    nan = np.uint16(0x7FC0)
    used = set()
    for r in range(2):
        n = int(w.seqlens[r])
        for k in range((n + 63) // 64):
            pg = w.block_table[r, k]
            used.add(int(pg))
            if k == (n - 1) // 64:
                w.kcache_bits[pg, n % 64 or 64:, 0, :] = nan
    for pg in range(6):
        if pg not in used:
            w.kcache_bits[pg] = nan
    out, lse, _ = G.run_dense(w)
    G.compare("nan-sentinel", out, lse, *ref)


# ----------------------------------------------------------------------------- full-size configurations (every row)

@pytest.mark.parametrize("cfg", ["c3", "h", "c4"])
def test_full_size_every_row(cfg):
    """The full configurations at the library's split count, every output row
    against the oracle."""
    G.say(f"full-size {cfg}")
    w = W.config(cfg)
    out, lse, plan = G.run_dense(w)
    G.say(f"  num_parts={plan.num_parts}")
    G.compare(f"{cfg}-full", out, lse, *oracle_dense(w))
    assert ops.mla_read_device_errors() == 0


# ----------------------------------------------------------------------------- long pieces, many splits

@pytest.mark.parametrize("parts", [1, None], ids=["one-piece", "library-parts"])
def test_long_context_sk65536(parts):
    """b=1, sk=65536 (1024 pages; the dense page's longest sweep point).  With one
    piece the request spans more pages than a workgroup caches, so the later page
    ids come from the direct lookup path."""
    G.say(f"sk=65536 parts={parts}")
    w = W.dense_workload("sk65536", 196, 1, 1, 128, [65536], pool_pages=1100, num_parts=parts)
    out, lse, plan = G.run_dense(w)
    G.say(f"  num_parts={plan.num_parts}")
    G.compare(f"sk65536-p{plan.num_parts}", out, lse, *oracle_dense(w))
    assert ops.mla_read_device_errors() == 0


def test_batch_128_ragged_every_row():
    """b=128 (the top of the dense page's test range) with ragged lengths from 1 to
    2048 tokens, at the library's split count, every row against the oracle."""
    G.say("b=128 ragged")
    rng = np.random.default_rng(197)
    seqlens = rng.integers(1, 2048, size=128, endpoint=True).astype(np.int32)
    pages = int(sum((int(n) + 63) // 64 for n in seqlens))
    w = W.dense_workload("b128", 197, 128, 1, 128, seqlens, pool_pages=pages + 16)
    out, lse, plan = G.run_dense(w)
    G.say(f"  num_parts={plan.num_parts}")
    G.compare("b128-ragged", out, lse, *oracle_dense(w))
    assert ops.mla_read_device_errors() == 0


@pytest.mark.parametrize("parts,least", [(128, 64), (200, 128)])
def test_combine_more_than_64_splits(parts, least):
    """One request cut into more than 64 splits (a 65536-token request next to
    three one-page ones, so that the split limit allows up to 64 parts per
    request on average): the combine's lse reductions run over several groups
    of 64."""
    lengths = [65536, 64, 64, 64]
    G.say(f"lengths {lengths} in {parts} parts")
    w = W.dense_workload("many-splits", 197, 4, 1, 128, lengths, pool_pages=1040, num_parts=parts)
    out, lse, plan = G.run_dense(w)
    ns = plan.num_splits.cpu().numpy()
    assert np.array_equal(ns, O.sched_partition(lengths, parts, split_limit="dense")[1])
    splits = int(ns[1])
    G.say(f"  request 0 in {splits} splits")
    assert splits > least
    G.compare(f"splits{parts}", out, lse, *oracle_dense(w))


# ----------------------------------------------------------------------------- online-softmax rescale branch
#
# With N(0, 1) inputs a row's score maximum never climbs 8 log2 units after a
# piece's first tile, so the rescale branch of the online softmax would never
# run.  These workloads plant high-scoring keys (tests/rescale_rule.py counts
# the resulting moves of the reference maximum with the kernels' own rule, and
# each test asserts there are some) in the middle of pieces, at the first key of
# a split, and in a partial last tile.

RESCALE_DENSE = [
    # name, seed, b, s_q, h_q, seqlens, pool pages, causal, forced parts, plants (request, key, beta), dtype, h_kv
    ("bf16-h128-p5", 190, 3, 1, 128, [1, 700, 2049], 60, False, 5,
     [(1, 150, 15.0), (1, 512, 30.0), (1, 699, 45.0), (2, 300, 12.0), (2, 960, 27.0), (2, 1100, 40.0),
      (2, 2048, 55.0)], "bf16", 1),
    ("bf16-h128-library", 191, 2, 1, 128, [4096, 1500], 100, False, None,
     [(0, 40, 12.0), (0, 1000, 26.0), (0, 2100, 40.0), (0, 4095, 55.0), (1, 700, 20.0), (1, 1499, 35.0)],
     "bf16", 1),
    ("bf16-h64-causal-sq2", 192, 2, 2, 64, [300, 1000], 30, True, 3,
     [(0, 100, 14.0), (0, 298, 30.0), (0, 299, 44.0), (1, 500, 13.0), (1, 998, 28.0), (1, 999, 43.0)], "bf16", 1),
    ("bf16-h16-p1", 193, 2, 1, 16, [333, 200], 10, False, 1,
     [(0, 70, 15.0), (0, 332, 30.0), (1, 130, 20.0), (1, 199, 36.0)], "bf16", 1),
    ("bf16-hkv2-h128", 194, 2, 1, 128, [900, 400], 24, False, 3,
     [(0, 300, 15.0), (0, 899, 32.0), (1, 399, 20.0)], "bf16", 2),
    ("fp16-h128-p4", 195, 2, 1, 128, [1000, 333], 24, False, 4,
     [(0, 200, 14.0), (0, 640, 28.0), (0, 999, 42.0), (1, 100, 15.0), (1, 332, 30.0)], "fp16", 1),
]


@pytest.mark.parametrize("case", RESCALE_DENSE, ids=[c[0] for c in RESCALE_DENSE])
def test_rescale_branch_dense(case):
    name, seed, b, s_q, h_q, seqlens, pool, causal, parts, plants, dtype, h_kv = case
    G.say(f"rescale dense {name}")
    w = W.dense_workload(name, seed, b, s_q, h_q, seqlens, pool_pages=pool, causal=causal, dtype=dtype, h_kv=h_kv)
    W.plant_dense(w, plants)
    fmt = ops.KV_FP16_PAGED if dtype == "fp16" else ops.KV_BF16_PAGED
    P = parts or ops.mla_decode_num_parts(b, s_q, h_q, h_kv, fmt)
    moves, ambiguous = RR.moves_for(w, P)
    G.say(f"  num_parts={P}: {moves} moves of the reference max after a piece's first tile "
          f"({ambiguous} comparisons within 0.5 of the threshold)")
    assert moves > 0
    t = G.dev_tensors(w)
    plan = ops.DecodePlan(t["seqlens"], s_q, h_q, fmt, num_parts=P, h_kv=h_kv)
    out, lse = ops.mla_decode(t["q"], t["kcache"], t["block_table"], t["seqlens"], w.scale, w.causal, plan=plan,
                              kv_format=fmt)
    torch.cuda.synchronize()
    G.compare(name, out, lse, *oracle_dense(w))


RESCALE_SPARSE = [
    # name, seed, b, h_q, cap, topk lengths, context, s_q, forced parts, plants (request, top-k position, beta)
    ("h64-tails", 200, 3, 64, 192, [192, 65, 100], 4096, 1, 4,
     [(0, 40, 14.0), (0, 64, 28.0), (0, 191, 42.0), (1, 64, 20.0), (2, 70, 15.0), (2, 99, 30.0)]),
    ("h128-topk2048", 201, 2, 128, 2048, [2048, 1800], 32768, 1, None,
     [(0, 100, 12.0), (0, 1024, 26.0), (0, 2047, 40.0), (1, 900, 15.0), (1, 1799, 30.0)]),
    ("h64-sq2", 202, 2, 64, 256, [256, 130], 2048, 2, 3,
     [(0, 10, 13.0), (0, 255, 30.0), (1, 129, 20.0)]),
]


@pytest.mark.parametrize("case", RESCALE_SPARSE, ids=[c[0] for c in RESCALE_SPARSE])
def test_rescale_branch_fp8(case):
    """The FP8 kernel's own online softmax (packed workspace and gathered by
    index) through the rescale branch, against the oracle and bitwise with each
    other."""
    name, seed, b, h, cap, topk, ctx, s_q, parts, plants = case
    G.say(f"rescale fp8 {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, s_q=s_q, num_parts=parts)
    W.plant_sparse(w, plants)
    P = parts or ops.mla_decode_num_parts(b, s_q, h, 1, ops.KV_FP8_PACKED)
    moves, ambiguous = RR.moves_for(w, P)
    G.say(f"  num_parts={P}: {moves} moves of the reference max after a piece's first tile "
          f"({ambiguous} comparisons within 0.5 of the threshold)")
    assert moves > 0
    t = G.dev_tensors(w)
    ref = oracle_sparse(w)
    out_p, lse_p, _, plan_p = G.run_sparse(w, t, num_parts=P)
    G.compare(name + "-packed", out_p, lse_p, *ref)
    out_i, lse_i, plan_i = G.run_sparse_indexed(w, t, num_parts=P)
    G.compare(name + "-indexed", out_i, lse_i, *ref)
    assert torch.equal(out_p, out_i) and torch.equal(lse_p, lse_i)


# ----------------------------------------------------------------------------- combine alone

def test_combine_kernel_against_oracle_partials():
    G.say("combine isolated")
    w = W.dense_workload("comb", 130, 3, 1, 32, [300, 0, 190], pool_pages=10, causal=False)
    # split points per request, as the scheduler would lay them out in slots
    cuts = {0: [0, 64, 128, 300], 2: [0, 100, 190]}
    P = 4
    ns = np.array([0, 3, 3, 5], np.int32)
    slots = w.batch + P
    M = w.s_q * w.h_q
    part_o = np.zeros((slots, M, 512), np.float32)
    part_l = np.full((slots, M), -np.inf, np.float32)
    for r, c in cuts.items():
        for i, (lo, hi) in enumerate(zip(c[:-1], c[1:])):
            lo_a = np.zeros(w.batch, np.int32)
            hi_a = np.zeros(w.batch, np.int32)
            lo_a[r], hi_a[r] = lo, hi
            po, pl = O.mla_decode_partial(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, False, lo_a,
                                          hi_a)
            part_o[ns[r] + i] = po[r].reshape(M, 512)
            part_l[ns[r] + i] = pl[r].reshape(M)
    ws = np.concatenate([part_o.reshape(-1), part_l.reshape(-1)]).view(np.uint8)
    ws_t = torch.from_numpy(ws.copy()).cuda()
    ns_t = torch.from_numpy(ns).cuda()
    out = torch.full((w.batch, 1, w.h_q, 512), 7.0, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((w.batch, 1, w.h_q), 7.0, dtype=torch.float32, device="cuda:0")
    ops.mla_combine(ns_t, ws_t, w.batch, 1, w.h_q, P, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_dense(w)
    # request 1 has no split: combine writes 0 / -inf
    G.compare("combine", out, lse, ref_o, ref_l)


# ----------------------------------------------------------------------------- scheduler for the sparse paths

SCHED_CASES = [
    ([2048] * 8, 256), ([1536, 2048, 1700, 1600], 64), ([1, 64, 65, 0, 300], 4), ([0, 0], 3), ([10], 5),
    ([2048, 4096, 3000, 100], 9), ([64] * 5, 5), ([128, 64], 2), ([4096], 256), ([700, 0, 2049], 7),
    (list(np.random.default_rng(5).integers(0, 3000, size=40)), 128),
    (list(np.random.default_rng(6).integers(0, 3000, size=3000)), 2048),
    ([64, 64, 64], 2),                                                  # more requests than parts: global
]


@pytest.mark.parametrize("lengths,P", SCHED_CASES)
def test_packed_metadata_bit_exact(lengths, P):
    b = len(lengths)
    tl = torch.tensor(np.asarray(lengths, np.int32), device="cuda:0")
    glob = O.sched_partition(lengths, P)
    loc = O.sched_partition_request_local(lengths, P) or glob
    for policy, ref in ((ops.SCHED_GLOBAL, glob), (ops.SCHED_REQUEST_LOCAL, loc)):
        meta, ns = ops.mla_get_packed_decode_metadata(tl, b, 1, 64, 64, P, policy=policy)
        torch.cuda.synchronize()
        assert np.array_equal(meta.cpu().numpy(), ref[0]), policy
        assert np.array_equal(ns.cpu().numpy(), ref[1]), policy


def test_packed_metadata_auto_policy():
    """AUTO is the global partition (measured faster on this GPU at every shape)."""
    lengths = [1536, 2048, 1700, 1600, 2048, 1800, 1900, 2000]
    P = 64
    loc = O.sched_partition_request_local(lengths, P)
    glob = O.sched_partition(lengths, P)
    assert not np.array_equal(loc[0], glob[0])
    tl = torch.tensor(np.asarray(lengths, np.int32), device="cuda:0")
    for s_q, h_q, ref in ((1, 64, glob), (2, 64, glob), (1, 128, glob), (4, 64, glob)):
        meta, ns = ops.mla_get_packed_decode_metadata(tl, 8, s_q, h_q, 2048, P)
        torch.cuda.synchronize()
        assert np.array_equal(meta.cpu().numpy(), ref[0]) and np.array_equal(ns.cpu().numpy(), ref[1]), (s_q, h_q)


@pytest.mark.parametrize("name,seed,b,h,cap,topk,ctx,s_q,parts", [
    ("rl-c5like", 180, 8, 64, 2048, [1536, 2048, 1700, 1600, 2048, 1800, 1900, 2000], 32768, 1, 64),
    ("rl-tails-sq2", 181, 3, 64, 192, [192, 65, 0], 4096, 2, 7),
])
def test_fp8_decode_with_request_local_metadata(name, seed, b, h, cap, topk, ctx, s_q, parts):
    G.say(f"fp8 request-local {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, s_q=s_q)
    t = G.dev_tensors(w)
    ref = oracle_sparse(w)
    meta, ns = ops.mla_get_packed_decode_metadata(t["seqlens"], b, s_q, h, cap, parts, policy=ops.SCHED_REQUEST_LOCAL)
    ws_d = torch.empty((ops.mla_decode_workspace_size(b, s_q, h, parts),), dtype=torch.uint8, device="cuda:0")
    packed = ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"])
    for fmt, kv, ix in ((ops.KV_FP8_PACKED, packed, None), (ops.KV_FP8_INDEXED, t["kcache_rec"], t["indices"])):
        out = torch.empty((b, s_q, h, 512), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.empty((b, s_q, h), dtype=torch.float32, device="cuda:0")
        ops.mla_decode_fwd(t["q"], kv, fmt, ix, t["seqlens"], w.scale, False, meta, ns, out, lse, ws_d,
                           topk_capacity=cap)
        ops.mla_combine(ns, ws_d, b, s_q, h, parts, out, lse)
        torch.cuda.synchronize()
        G.compare(f"{name}-{fmt}", out, lse, *ref)
    assert ops.mla_read_device_errors() == 0


# ----------------------------------------------------------------------------- FP8 pack + packed decode

@pytest.mark.parametrize("case", [
    ("full-tile-h64", 140, 1, 64, 64, [64], 512, 1),
    ("tails-h64", 141, 3, 64, 192, [192, 65, 1], 4096, 1),
    ("tails-h128", 142, 2, 128, 256, [100, 256], 2048, 1),
    ("pack-sq2", 143, 2, 64, 128, [128, 70], 1024, 2),
], ids=lambda c: c[0])
def test_pack_bytes_exact(case):
    name, seed, b, h, cap, topk, ctx, s_q = case
    G.say(f"pack {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, s_q=s_q)
    t = G.dev_tensors(w)
    ws = ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"])
    torch.cuda.synchronize()
    ref = O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens)
    assert np.array_equal(ws.cpu().numpy(), ref.reshape(-1))


SPARSE = [
    ("full-tile-h64", 150, 1, 64, 64, [64], 512, None),
    ("tails-h64", 151, 3, 64, 192, [192, 65, 1], 4096, None),
    ("tails-h64-p1", 151, 3, 64, 192, [192, 65, 1], 4096, 1),
    ("topk2048-h128", 152, 2, 128, 2048, [2048, 2048], 32768, None),
    ("tails-h128", 153, 3, 128, 512, [400, 17, 512], 8192, 7),
    ("empty-h64", 154, 2, 64, 128, [0, 77], 1024, None),
    # pieces longer than the 1024 top-k ids the by-index decode stages per piece: the
    # later tiles read their ids directly
    ("topk1500-h128-p1", 168, 1, 128, 2048, [1500], 8192, 1),
    ("topk3000-h64-p1", 155, 1, 64, 4096, [3000], 16384, 1),
    ("topk4096-h128-p3", 156, 2, 128, 4096, [4096, 2500], 32768, 3),
    # the tile pipeline's edges: pieces of 1..4 tiles (the first tile converted
    # before the loop, the rest one iteration ahead) ending at every kind of
    # tail, several requests per workgroup (LDS reused from one to the next)
    ("pipeline-edges-h64-p3", 169, 12, 64, 128, [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128], 4096, 3),
    ("pipeline-edges-h128", 170, 12, 128, 128, [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128], 4096, None),
]


# several query tokens per request, each with its own top-k list (workspace row r * s_q + s)
SPARSE_MULTI = [
    ("sq2-h128", 158, 2, 128, 256, [256, 100], 2048, 2, None),
    ("sq4-h64-tails", 159, 3, 64, 128, [128, 70, 1], 1024, 4, None),
    ("sq8-h64-p3", 160, 2, 64, 192, [150, 192], 4096, 8, 3),
    ("sq16-h128", 161, 2, 128, 128, [128, 90], 1024, 16, None),
    ("sq3-h64-tails", 162, 3, 64, 256, [256, 130, 3], 2048, 3, None),   # three tokens: the packed page's S_q = 3
    ("sq3-h128-p5", 163, 2, 128, 192, [192, 61], 2048, 3, 5),
]


@pytest.mark.parametrize("case", SPARSE_MULTI, ids=[c[0] for c in SPARSE_MULTI])
def test_fp8_multi_token(case):
    """Packed and by-index sparse decode with s_q > 1 against the oracle, and
    bitwise against each other."""
    name, seed, b, h, cap, topk, ctx, s_q, parts = case
    G.say(f"fp8 multi-token {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, s_q=s_q, num_parts=parts)
    t = G.dev_tensors(w)
    ref = oracle_sparse(w)
    out_p, lse_p, ws, _ = G.run_sparse(w, t)
    assert np.array_equal(ws.cpu().numpy(), O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens).reshape(-1))
    G.compare(name + "-packed", out_p, lse_p, *ref)
    out_i, lse_i, _ = G.run_sparse_indexed(w, t)
    G.compare(name + "-indexed", out_i, lse_i, *ref)
    assert torch.equal(out_p, out_i) and torch.equal(lse_p, lse_i)
    assert ops.mla_read_device_errors() == 0


@pytest.mark.parametrize("case", SPARSE, ids=[c[0] for c in SPARSE])
def test_fp8_packed_decode(case):
    name, seed, b, h, cap, topk, ctx, parts = case
    G.say(f"fp8 {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, num_parts=parts)
    out, lse, ws, plan = G.run_sparse(w)
    G.compare(name, out, lse, *oracle_sparse(w))


def test_config_c5():
    G.say("config c5")
    w = W.config("c5")
    out, lse, ws, plan = G.run_sparse(w)
    G.say(f"  num_parts={plan.num_parts}")
    ref_ws = O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens)
    assert np.array_equal(ws.cpu().numpy(), ref_ws.reshape(-1))
    G.compare("c5", out, lse, *oracle_sparse(w))


# ----------------------------------------------------------------------------- FP8 decode gathering by index

@pytest.mark.parametrize("case", SPARSE, ids=[c[0] for c in SPARSE])
def test_fp8_indexed_decode(case):
    """The decode that gathers the selected records itself matches the oracle and,
    bit for bit, the pack + packed decode (same arithmetic, same split)."""
    name, seed, b, h, cap, topk, ctx, parts = case
    G.say(f"fp8 indexed {name}")
    w = W.sparse_workload(name, seed, b, h, cap, topk, context=ctx, num_parts=parts)
    t = G.dev_tensors(w)
    out, lse, plan = G.run_sparse_indexed(w, t)
    G.compare(name, out, lse, *oracle_sparse(w))
    out_p, lse_p, _, plan_p = G.run_sparse(w, t)
    assert plan.num_parts == plan_p.num_parts
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)
    assert ops.mla_read_device_errors() == 0


def test_fp8_indexed_config_c5():
    G.say("config c5 indexed")
    w = W.config("c5")
    t = G.dev_tensors(w)
    out, lse, plan = G.run_sparse_indexed(w, t)
    G.say(f"  num_parts={plan.num_parts}")
    G.compare("c5-indexed", out, lse, *oracle_sparse(w))
    out_p, lse_p, _, _ = G.run_sparse(w, t)
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)


def test_fp8_nan_records_never_reach_the_output():
    """Records no row selects, including record 0 (which the by-index loader reads
    for keys past topk_length), hold E4M3 NaN bytes (0x7F / 0xFF): the by-index
    decode still matches the oracle and, bit for bit, the pack + packed decode."""
    G.say("fp8: NaN bytes in unselected records")
    w = W.sparse_workload("nan-pool", 157, 3, 64, 192, [150, 33, 192], context=2048)
    flat = w.kcache_rec.reshape(-1, 656)
    chosen = set()
    for r in range(w.batch):
        for i in range(w.s_q):
            chosen.update(int(x) for x in w.indices[r, i, :int(w.seqlens[r])])
    if 0 in chosen:  # keep record 0 unselected: swap its selection for a free id of the same page range
        free = next(x for x in range(1, 32 * 64) if x not in chosen)
        w.indices[w.indices == 0] = free
        chosen.discard(0)
        chosen.add(free)
    unselected = np.array(sorted(set(range(flat.shape[0])) - chosen))
    flat[unselected, :512] = np.where(np.arange(512) % 2 == 0, 0x7F, 0xFF).astype(np.uint8)
    assert 0 in set(unselected.tolist())
    ref = oracle_sparse(w)  # the oracle reads selected records only
    t = G.dev_tensors(w)
    out_i, lse_i, _ = G.run_sparse_indexed(w, t)
    G.compare("nan-pool-indexed", out_i, lse_i, *ref)
    out_p, lse_p, _, _ = G.run_sparse(w, t)
    G.compare("nan-pool-packed", out_p, lse_p, *ref)
    assert torch.equal(out_i, out_p) and torch.equal(lse_i, lse_p)
    assert ops.mla_read_device_errors() == 0


def test_fp8_indexed_ignores_ids_past_topk_length():
    """Ids at positions >= topk_length are never read: garbage there (even out of
    the pool) changes nothing and raises no flag."""
    G.say("fp8 indexed: garbage past topk_length")
    w = W.sparse_workload("tail-garbage", 155, 2, 128, 256, [130, 31], context=2048)
    t = G.dev_tensors(w)
    out, lse, _ = G.run_sparse_indexed(w, t)
    ops.mla_read_device_errors()
    for r, n in enumerate(w.seqlens):
        w.indices[r, :, n:] = -123456789
    t2 = dict(t, indices=torch.from_numpy(w.indices).to("cuda:0"))
    out2, lse2, _ = G.run_sparse_indexed(w, t2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert ops.mla_read_device_errors() == 0


# ----------------------------------------------------------------------------- early pack + current-token patch

def _current_token_case(seed):
    """A sparse workload, the ids of each request's "current" tokens (one
    selected, one not selected, and a -1 entry), and replacement records for them."""
    w = W.sparse_workload("patch", seed, 3, 64, 192, [192, 100, 0], context=2048, s_q=2)
    other = W.sparse_workload("patch-new", seed + 1000, 1, 64, 64, [64], context=4096)
    new_recs = other.kcache_rec.reshape(-1, 656)
    ids = np.full((w.batch, 3), -1, np.int32)
    sel_all = set(int(x) for x in w.indices.reshape(-1) if x >= 0)
    for r in range(w.batch):
        n = int(w.seqlens[r])
        if n > 0:
            ids[r, 0] = w.indices[r, 1, n // 2]              # selected by token 1 of the request
        pool_ids = np.arange(r * 32 * 64, (r + 1) * 32 * 64)  # this request's pages
        ids[r, 1] = int(next(i for i in pool_ids if int(i) not in sel_all))
    new_pool = w.kcache_rec.copy()
    flat = new_pool.reshape(-1, 656)
    for j, i in enumerate(x for x in ids.reshape(-1) if x >= 0):
        flat[i] = new_recs[j]
    return w, ids, new_pool


def _patched_run(w, ids, new_pool, side_stream):
    dev = torch.device("cuda:0")
    t = G.dev_tensors(w)
    kc = t["kcache_rec"]  # the pool as the early pack sees it
    ws = torch.empty((ops.mla_packed_kv_workspace_size(w.batch, w.s_q, w.topk_capacity),), dtype=torch.uint8,
                     device=dev)
    new_dev = torch.from_numpy(new_pool).to(dev)
    ids_dev = torch.from_numpy(ids).to(dev)
    torch.cuda.synchronize()
    if side_stream:
        # the pack runs on its own stream while the main stream writes the current
        # tokens' records into the pool (the pack may see old or new bytes for
        # them; the patch rewrites exactly those slots afterwards)
        side = torch.cuda.Stream()
        ev = torch.cuda.Event()
        with torch.cuda.stream(side):
            ops.mla_pack_selected_kv(kc, t["indices"], t["seqlens"], ws)
            ev.record(side)
        kc.copy_(new_dev)
        torch.cuda.current_stream().wait_event(ev)
    else:
        ops.mla_pack_selected_kv(kc, t["indices"], t["seqlens"], ws)
        kc.copy_(new_dev)  # the current step's records land in the pool
    ops.mla_patch_packed_kv(kc, t["indices"], t["seqlens"], ids_dev, ws)
    torch.cuda.synchronize()
    return t, ws


@pytest.mark.parametrize("side_stream", [False, True], ids=["same-stream", "side-stream"])
def test_patch_after_early_pack(side_stream):
    """Pack before the current tokens' records are written, write them, patch:
    the workspace equals a fresh pack of the new pool byte for byte, and the
    packed decode equals the by-index decode of the new pool bit for bit."""
    G.say(f"early pack + patch ({'side' if side_stream else 'same'} stream)")
    w, ids, new_pool = _current_token_case(170)
    ops.mla_read_device_errors()
    t, ws = _patched_run(w, ids, new_pool, side_stream)
    ref_ws = O.pack_selected_kv(new_pool, w.indices, w.seqlens)
    assert not np.array_equal(ref_ws, O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens))  # the patch matters
    assert np.array_equal(ws.cpu().numpy(), ref_ws.reshape(-1))
    plan = ops.DecodePlan(t["seqlens"], w.s_q, w.h_q, ops.KV_FP8_PACKED, topk_capacity=w.topk_capacity)
    out_p, lse_p = ops.mla_decode(t["q"], ws, None, t["seqlens"], w.scale, False, plan=plan,
                                  kv_format=ops.KV_FP8_PACKED, topk_capacity=w.topk_capacity)
    out_i, lse_i = ops.mla_decode(t["q"], t["kcache_rec"], t["indices"], t["seqlens"], w.scale, False, plan=plan,
                                  kv_format=ops.KV_FP8_INDEXED, topk_capacity=w.topk_capacity)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_i) and torch.equal(lse_p, lse_i)
    G.compare("patched", out_p, lse_p, *O.mla_sparse_decode(w.q_bits, new_pool, w.indices, w.seqlens, w.scale))
    assert ops.mla_read_device_errors() == 0


def test_patch_out_of_pool_id_sets_flag():
    G.say("device flag: patch id outside the pool")
    w = W.sparse_workload("patchbad", 171, 1, 64, 64, [10], context=512)
    limit = w.kcache_rec.shape[0] * 64
    w.indices[0, 0, 4] = limit + 3  # selected, outside the pool (the pack zero-fills and flags it)
    t = G.dev_tensors(w)
    ops.mla_read_device_errors()
    ws = ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"])
    ids = torch.tensor([[limit + 3]], dtype=torch.int32, device="cuda:0")
    ops.mla_patch_packed_kv(t["kcache_rec"], t["indices"], t["seqlens"], ids, ws)
    torch.cuda.synchronize()
    assert ops.mla_read_device_errors() & 2
    assert not ws.view(-1, 656)[4].any()  # the slot stays as the pack left it: zero


# ----------------------------------------------------------------------------- device-side contract checks

def test_out_of_range_page_sets_flag_without_fault():
    G.say("device flag: page out of range")
    ops.mla_read_device_errors()  # clear
    w = W.dense_workload("badpage", 160, 1, 1, 16, [100], pool_pages=2)
    w.block_table[0, 1] = 99  # the kernel must not read page 99; it clamps and flags
    G.run_dense(w)
    flags = ops.mla_read_device_errors()
    assert flags & 1
    assert ops.mla_read_device_errors() == 0


def test_out_of_range_topk_id_sets_flag_without_fault():
    G.say("device flag: top-k id out of range (indexed decode)")
    ops.mla_read_device_errors()  # clear
    w = W.sparse_workload("badid", 156, 1, 64, 64, [40], context=512)
    w.indices[0, 0, 3] = 64 * w.kcache_rec.shape[0] + 5  # one past-the-pool id in the valid prefix
    w.indices[0, 0, 7] = -2
    G.run_sparse_indexed(w)
    flags = ops.mla_read_device_errors()
    assert flags & 2
    assert ops.mla_read_device_errors() == 0


def test_topk_length_above_capacity_sets_flag_without_fault():
    G.say("device flag: topk_length above capacity (indexed decode)")
    ops.mla_read_device_errors()
    w = W.sparse_workload("longlen", 157, 2, 64, 64, [64, 10], context=512)
    t = G.dev_tensors(w)
    t["seqlens"] = torch.tensor([1000, 10], dtype=torch.int32, device="cuda:0")
    G.run_sparse_indexed(w, t)
    assert ops.mla_read_device_errors() & 4


def test_corrupt_metadata_sets_flag_without_fault():
    """A scheduler record that no scheduler produces (a negative block index) is
    refused by every decode kernel: it sets device flag bit 3 and skips the
    record, reading nothing through it."""
    G.say("device flag: corrupt scheduler records (dense, packed, by index)")
    ops.mla_read_device_errors()  # clear
    w = W.dense_workload("badmeta", 161, 2, 1, 128, [300, 200], pool_pages=12, num_parts=4)
    t = G.dev_tensors(w)
    plan = ops.DecodePlan(t["seqlens"], w.s_q, w.h_q, ops.KV_BF16_PAGED, num_parts=4)
    assert int(plan.sched_meta[0, 0]) == 0  # part 0 owns blocks (the record is live)
    plan.sched_meta[0, 1] = -3  # begin block
    ops.mla_decode(t["q"], t["kcache"], t["block_table"], t["seqlens"], w.scale, False, plan=plan)
    assert ops.mla_read_device_errors() & 8

    s = W.sparse_workload("badmeta8", 162, 2, 64, 128, [100, 70], context=512)
    ts = G.dev_tensors(s)
    ws = ops.mla_pack_selected_kv(ts["kcache_rec"], ts["indices"], ts["seqlens"])
    for fmt, kv, ix in ((ops.KV_FP8_PACKED, ws, None), (ops.KV_FP8_INDEXED, ts["kcache_rec"], ts["indices"])):
        plan = ops.DecodePlan(ts["seqlens"], s.s_q, s.h_q, fmt, num_parts=4, topk_capacity=s.topk_capacity)
        assert int(plan.sched_meta[1, 0]) >= 0
        plan.sched_meta[1, 3] = -1  # end block
        ops.mla_decode(ts["q"], kv, ix, ts["seqlens"], s.scale, False, plan=plan, kv_format=fmt,
                       topk_capacity=s.topk_capacity)
        assert ops.mla_read_device_errors() & 8, fmt
    assert ops.mla_read_device_errors() == 0


# ----------------------------------------------------------------------------- HIP graph capture

def test_hip_graph_replay_matches_eager():
    """The step (metadata, decode, combine) captured in a HIP graph: every replay
    equals the eager step bit for bit, with eager work (including on the
    workspace) between replays."""
    G.say("hip graph replay")
    w = W.dense_workload("graph", 130, 4, 1, 128, [700, 64, 2049, 1], pool_pages=60, num_parts=8)
    t = G.dev_tensors(w)
    b, s_q, h_q, parts = w.batch, w.s_q, w.h_q, 8
    dev = torch.device("cuda:0")
    meta = torch.empty((parts, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((b + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty((ops.mla_decode_workspace_size(b, s_q, h_q, parts),), dtype=torch.uint8, device=dev)
    out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)

    def step():
        ops.mla_get_decode_metadata(t["seqlens"], b, s_q, h_q, 1, parts, meta, ns)
        ops.mla_decode_fwd(t["q"], t["kcache"], ops.KV_BF16_PAGED, t["block_table"], t["seqlens"], w.scale,
                           w.causal, meta, ns, out, lse, ws)
        ops.mla_combine(ns, ws, b, s_q, h_q, parts, out, lse)

    step()
    torch.cuda.synchronize()
    G.compare("graph-eager", out, lse, *oracle_dense(w))
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        ws.fill_(0)
        meta.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs from the eager step"


# ----------------------------------------------------------------------------- launch log, canaries

def test_mla_log_prints_launch_lines():
    """MLA_LOG=1: one stderr line per launch, the decode's with its kernel, grid,
    split count, occupancy, LDS and VGPRs (checked in a child process, since the
    library reads the variable once)."""
    import os
    import subprocess
    import sys

    code = ("import numpy as np, torch\n"
            "from mla_paged_kv_amd import ops, workloads as W\n"
            "from tests import gpu_helpers as G\n"
            "w = W.dense_workload('log', 301, 2, 1, 128, [300, 70], pool_pages=8)\n"
            "G.run_dense(w)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MLA_LOG="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=120)
    G.say(r.stderr[-600:])
    assert r.returncode == 0
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[mla]")]
    dec = [ln for ln in lines if ln.startswith("[mla] decode")]
    assert len(dec) == 1 and "decode_ws_kernel<4, false, false>" in dec[0]
    for key in ("grid=", "num_parts=", "wgs_per_cu=", "lds=", "vgprs="):
        assert key in dec[0]
    assert any(ln.startswith("[mla] metadata") for ln in lines)
    assert any(ln.startswith("[mla] combine") for ln in lines)


def _padded(numel, dtype, canary):
    """A device buffer of `numel` elements with 4096 canary elements on each side;
    returns (whole buffer, the middle view)."""
    pad = 4096
    whole = torch.full((numel + 2 * pad,), canary, dtype=dtype, device="cuda")
    return whole, whole[pad:pad + numel]


def _canaries_intact(whole, canary):
    pad = 4096
    return bool(torch.all(whole[:pad] == canary)) and bool(torch.all(whole[-pad:] == canary))


@pytest.mark.parametrize("fmt", ["dense", "packed", "indexed"])
def test_no_writes_outside_the_buffers(fmt):
    """Canary-padded out, lse, workspace, metadata and packed workspace: no kernel
    writes outside the memory it was given."""
    G.say(f"canaries {fmt}")
    if fmt == "dense":
        w = W.dense_workload("canary", 302, 3, 2, 128, [1, 700, 129], pool_pages=20, causal=True, num_parts=5)
    else:
        w = W.sparse_workload("canary", 303, 3, 64, 256, [256, 70, 1], context=1024, s_q=2, num_parts=5)
    t = G.dev_tensors(w)
    b, s_q, h_q = w.batch, w.s_q, w.h_q
    P = w.num_parts
    ow, out_flat = _padded(b * s_q * h_q * 512, torch.int16, 0x7a5b)
    lw, lse_flat = _padded(b * s_q * h_q, torch.float32, -12345.5)
    mw, meta_flat = _padded(P * 8, torch.int32, 0x5a5a5a5a)
    nw, ns = _padded(b + 1, torch.int32, 0x5a5a5a5a)
    ww, ws = _padded(ops.mla_decode_workspace_size(b, s_q, h_q, P), torch.uint8, 0xA5)
    act = torch.bfloat16
    out = out_flat.view(act).view(b, s_q, h_q, 512)
    lse = lse_flat.view(b, s_q, h_q)
    meta = meta_flat.view(P, 8)
    if fmt == "dense":
        fmt_id, kv, ix = ops.KV_BF16_PAGED, t["kcache"], t["block_table"]
        ops.mla_get_decode_metadata(t["seqlens"], b, s_q, h_q, 1, P, meta, ns)
        cap = 0
    else:
        cap = w.topk_capacity
        ops.mla_get_packed_decode_metadata(t["seqlens"], b, s_q, h_q, cap, P, ops.SCHED_AUTO, meta, ns)
        if fmt == "packed":
            pw, pws = _padded(ops.mla_packed_kv_workspace_size(b, s_q, cap), torch.uint8, 0xA5)
            ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"], pws)
            torch.cuda.synchronize()
            assert _canaries_intact(pw, 0xA5)
            fmt_id, kv, ix = ops.KV_FP8_PACKED, pws, None
        else:
            fmt_id, kv, ix = ops.KV_FP8_INDEXED, t["kcache_rec"], t["indices"]
    ops.mla_decode_fwd(t["q"], kv, fmt_id, ix, t["seqlens"], w.scale, w.causal, meta, ns, out, lse, ws,
                       topk_capacity=cap)
    ops.mla_combine(ns, ws, b, s_q, h_q, P, out, lse)
    torch.cuda.synchronize()
    for whole, canary in ((ow, 0x7a5b), (lw, -12345.5), (mw, 0x5a5a5a5a), (nw, 0x5a5a5a5a), (ww, 0xA5)):
        assert _canaries_intact(whole, canary)
    ref = oracle_dense(w) if fmt == "dense" else oracle_sparse(w)
    G.compare(f"canary-{fmt}", out, lse, *ref)
    assert ops.mla_read_device_errors() == 0
