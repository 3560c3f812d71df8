"""Seeded random shapes against the oracle (GPU).

Each case draws its shape from a seeded generator: batch, query tokens, query
and KV heads, causal masking, element type, ragged and empty lengths and a
forced or library-chosen split count for the dense decode; heads, top-k
capacity, top-k lengths, query tokens and split count for the two sparse FP8
paths.  Every output row is compared with the oracle element by element (the
tolerances of tests/gpu_helpers.py), and the packed and by-index sparse
decodes must agree bit for bit.  The draws are printed before each case runs.
"""

import numpy as np
import pytest
import torch

from mla_paged_kv_amd import workloads as W
from oracle import oracle as O
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

ops = pytest.importorskip("mla_paged_kv_amd.ops")


def _dense_case(seed):
    rng = np.random.default_rng(9000 + seed)
    batch = int(rng.integers(1, 7))
    s_q = int(rng.choice([1, 1, 2, 3, 4]))
    h_kv = int(rng.choice([1, 1, 1, 2, 4]))
    # h_q: a multiple of 16 (of 16 h_kv with several KV heads) with s_q * h_q <= 512
    choices = [h for h in range(16, 129, 16) if h % h_kv == 0 and (h // h_kv) % 16 == 0 and s_q * h <= 512]
    h_q = int(rng.choice(choices))
    causal = bool(s_q > 1 and rng.random() < 0.6)
    dtype = "fp16" if rng.random() < 0.25 else "bf16"
    lens = rng.integers(0, 1600, size=batch)
    lens[rng.random(batch) < 0.15] = 0  # some empty requests
    if causal:
        lens = np.maximum(lens, rng.integers(0, s_q + 1, size=batch))
    parts = None if rng.random() < 0.4 else int(rng.integers(1, 40))
    return batch, s_q, h_q, h_kv, causal, dtype, [int(x) for x in lens], parts


@pytest.mark.parametrize("seed", range(12))
def test_random_dense_shapes(seed):
    batch, s_q, h_q, h_kv, causal, dtype, lens, parts = _dense_case(seed)
    G.say(f"random dense {seed}: b={batch} s_q={s_q} h_q={h_q} h_kv={h_kv} causal={causal} {dtype} "
          f"lens={lens} parts={parts}")
    pages = sum((n + 63) // 64 for n in lens)
    w = W.dense_workload(f"rand{seed}", 9100 + seed, batch, s_q, h_q, lens, pool_pages=pages + 4, causal=causal,
                         num_parts=parts, dtype=dtype, h_kv=h_kv)
    t = G.dev_tensors(w)
    fmt = ops.KV_FP16_PAGED if dtype == "fp16" else ops.KV_BF16_PAGED
    P = parts or ops.mla_decode_num_parts(batch, s_q, h_q, h_kv, fmt)
    plan = ops.DecodePlan(t["seqlens"], s_q, h_q, fmt, num_parts=P, h_kv=h_kv)
    out, lse = ops.mla_decode(t["q"], t["kcache"], t["block_table"], t["seqlens"], w.scale, w.causal, plan=plan,
                              kv_format=fmt)
    torch.cuda.synchronize()
    ref = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, dtype=w.dtype)
    G.compare(f"rand-dense-{seed}", out, lse, *ref)
    assert ops.mla_read_device_errors() == 0


def _sparse_case(seed):
    rng = np.random.default_rng(9500 + seed)
    batch = int(rng.integers(1, 6))
    h_q = int(rng.choice([64, 128]))
    s_q = int(rng.choice([1, 1, 2, 3]))
    cap = 64 * int(rng.integers(1, 17))
    topk = rng.integers(0, cap + 1, size=batch)
    topk[rng.random(batch) < 0.3] = cap  # full lists
    context = int(cap + 64 * rng.integers(0, 40))
    parts = None if rng.random() < 0.4 else int(rng.integers(1, 30))
    return batch, h_q, s_q, cap, [int(x) for x in topk], context, parts


@pytest.mark.parametrize("seed", range(8))
def test_random_sparse_shapes(seed):
    batch, h_q, s_q, cap, topk, context, parts = _sparse_case(seed)
    G.say(f"random sparse {seed}: b={batch} h_q={h_q} s_q={s_q} cap={cap} topk={topk} context={context} "
          f"parts={parts}")
    w = W.sparse_workload(f"rands{seed}", 9600 + seed, batch, h_q, cap, topk, context=context, s_q=s_q,
                          num_parts=parts)
    t = G.dev_tensors(w)
    ref = O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)
    out_p, lse_p, ws, _ = G.run_sparse(w, t)
    G.compare(f"rand-packed-{seed}", out_p, lse_p, *ref)
    out_i, lse_i, _ = G.run_sparse_indexed(w, t)
    G.compare(f"rand-indexed-{seed}", out_i, lse_i, *ref)
    assert torch.equal(out_p, out_i) and torch.equal(lse_p, lse_i)
    assert ops.mla_read_device_errors() == 0
