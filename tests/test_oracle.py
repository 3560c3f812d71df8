"""Pins for the CPU fp64 oracle (no GPU).

Each check ties the oracle to something other than itself: brute force on tiny
inputs (dense numpy formulation), closed forms (one key, equal scores, constant
V, zero and huge scale), invariants (split/merge, page permutation, causal
reductions), the exhaustive E4M3FN table from torch, hand-built FP8 records,
and byte counts the pages print (tests/golden/page_byte_facts.json).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from mla_paged_kv_amd import workloads as W
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_byte_facts.json")


def tiny_dense(seed, b, s_q, h, seqlens, pool, causal=False, scale=None, std=1.0):
    return W.dense_workload("tiny", seed, b, s_q, h, seqlens, pool_pages=pool, causal=causal, scale=scale, std=std)


def run_oracle(w, nthreads=4):
    return O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, nthreads=nthreads)


# ----------------------------------------------------------------------------- dense: brute force

@pytest.mark.parametrize("seed,b,s_q,h,seqlens,pool,causal", [
    (11, 2, 1, 4, [1, 130], 5, False),
    (12, 2, 3, 4, [65, 64], 4, True),
    (13, 1, 2, 3, [129], 4, True),
    (14, 3, 1, 2, [0, 7, 200], 8, False),
    (15, 2, 4, 2, [2, 70], 3, True),      # causal rows with no visible key (seqlen 2 < s_q)
])
def test_dense_matches_brute_force(seed, b, s_q, h, seqlens, pool, causal):
    w = tiny_dense(seed, b, s_q, h, seqlens, pool, causal=causal)
    out, lse = run_oracle(w)
    bo, bl = brute.dense(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, causal)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)
    assert np.all(lse[~fin] == -np.inf) and np.all(out[~fin] == 0)


@pytest.mark.parametrize("seed,b,s_q,h,seqlens,pool,causal", [
    (21, 2, 1, 4, [1, 130], 5, False),
    (22, 2, 3, 4, [65, 64], 4, True),
    (23, 3, 2, 2, [0, 7, 200], 8, True),
])
def test_dense_fp16_matches_brute_force(seed, b, s_q, h, seqlens, pool, causal):
    """The binary16 variant: same brute force with numpy's float16 decode."""
    w = W.dense_workload("tiny16", seed, b, s_q, h, seqlens, pool_pages=pool, causal=causal, dtype="fp16")
    out, lse = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, nthreads=3,
                            dtype="fp16")
    bo, bl = brute.dense(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, causal, dtype="fp16")
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)
    # decoding the same bits as bf16 gives a different result (the encoding is really used)
    ob, _ = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, nthreads=3)
    assert not np.allclose(ob, out)


@pytest.mark.parametrize("seed,b,s_q,h,h_kv,seqlens,pool,causal,dtype", [
    (31, 2, 1, 4, 2, [1, 130], 5, False, "bf16"),
    (32, 2, 2, 8, 4, [65, 90], 4, True, "bf16"),
    (33, 1, 3, 6, 3, [200], 4, True, "fp16"),
])
def test_dense_multi_kv_head_matches_brute_force(seed, b, s_q, h, h_kv, seqlens, pool, causal, dtype):
    w = W.dense_workload("tinyhk", seed, b, s_q, h, seqlens, pool_pages=pool, causal=causal, dtype=dtype, h_kv=h_kv)
    assert w.kcache_bits.shape[2] == h_kv
    out, lse = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, nthreads=3,
                            dtype=dtype)
    bo, bl = brute.dense(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, causal, dtype=dtype)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)


def test_multi_kv_head_groups_read_their_own_head():
    """Each group of h_q / h_kv query heads equals an h_kv = 1 decode over that KV head alone."""
    w = W.dense_workload("hkgroups", 34, 2, 2, 8, [70, 150], pool_pages=5, causal=True, h_kv=4)
    out, lse = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, w.causal, nthreads=3)
    for kk in range(4):
        o1, l1 = O.mla_decode(w.q_bits[:, :, 2 * kk:2 * kk + 2], w.kcache_bits[:, :, kk:kk + 1], w.block_table,
                              w.seqlens, w.scale, w.causal, nthreads=3)
        assert np.array_equal(o1, out[:, :, 2 * kk:2 * kk + 2]) and np.array_equal(l1, lse[:, :, 2 * kk:2 * kk + 2])


def test_f16_all_codes_match_numpy():
    """IEEE 754 binary16: every one of the 65536 codes against numpy's float16."""
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mine = np.array([O.f16_to_f64(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine)) and nan.sum() == 2 * 1023
    assert np.array_equal(mine[~nan], ref[~nan])
    assert O.f16_to_f64(0x3C00) == 1.0 and O.f16_to_f64(0x7BFF) == 65504.0 and O.f16_to_f64(0x0001) == 2.0 ** -24
    assert O.f16_to_f64(0x7C00) == math.inf and O.f16_to_f64(0xFC00) == -math.inf


def test_thread_count_does_not_change_result():
    w = tiny_dense(16, 2, 2, 4, [100, 190], 6, causal=True)
    a = run_oracle(w, nthreads=1)
    b = run_oracle(w, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- dense: closed forms

def test_one_key_gives_v_and_score():
    w = tiny_dense(21, 1, 1, 3, [1], 2)
    out, lse = run_oracle(w)
    k = brute.bf16(w.kcache_bits[w.block_table[0, 0], 0, 0])
    q = brute.bf16(w.q_bits[0, 0])
    for h in range(3):
        assert np.array_equal(out[0, 0, h], k[:512])  # p = 1 exactly
        exact = Fraction(w.scale) * sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(q[h], k))
        assert abs(lse[0, 0, h] - float(exact)) < 1e-12


def test_equal_scores_distinct_values_give_mean():
    # q NoPE part zero, every key shares the same RoPE part -> all scores equal,
    # so out = mean of V over keys and lse = s + ln n.
    w = tiny_dense(22, 1, 1, 2, [150], 4)
    q = W.bf16_bits_to_f32(w.q_bits).copy()
    q[..., :512] = 0
    w.q_bits = W.f32_to_bf16_bits(q)
    rope = w.kcache_bits[w.block_table[0, 0], 0, 0, 512:].copy()
    for j in range(150):
        w.kcache_bits[w.block_table[0, j // 64], j % 64, 0, 512:] = rope
    out, lse = run_oracle(w)
    n = 150
    keys = np.stack([brute.bf16(w.kcache_bits[w.block_table[0, j // 64], j % 64, 0]) for j in range(n)])
    qq = brute.bf16(w.q_bits[0, 0])
    for h in range(2):
        s = w.scale * float(np.dot(qq[h], keys[0]))
        np.testing.assert_allclose(out[0, 0, h], keys[:, :512].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[0, 0, h] - (s + math.log(n))) < 1e-12


def test_constant_v_rows_sum_to_one():
    # V = c for every key (RoPE dims random, q RoPE nonzero) -> out = c: the weights sum to 1.
    w = tiny_dense(23, 2, 2, 3, [90, 33], 4, causal=True)
    c = np.float32(0.8125)  # exact in bf16
    for r in range(2):
        for j in range(int(w.seqlens[r])):
            w.kcache_bits[w.block_table[r, j // 64], j % 64, 0, :512] = W.f32_to_bf16_bits(np.full(512, c))
    out, _ = run_oracle(w)
    np.testing.assert_allclose(out, np.full_like(out, float(c)), rtol=0, atol=1e-13)


def test_zero_scale_is_uniform_mean():
    w = tiny_dense(24, 1, 1, 2, [77], 3, scale=0.0)
    out, lse = run_oracle(w)
    keys = np.stack([brute.bf16(w.kcache_bits[w.block_table[0, j // 64], j % 64, 0]) for j in range(77)])
    np.testing.assert_allclose(out[0, 0, 0], keys[:, :512].mean(axis=0), rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - math.log(77)) < 1e-12


def test_huge_scale_selects_argmax_key():
    # Very peaked softmax: out = V of the highest-scoring key; a sign error would pick the lowest.
    w = tiny_dense(25, 1, 1, 4, [100], 2, scale=50.0)
    out, _ = run_oracle(w)
    keys = np.stack([brute.bf16(w.kcache_bits[w.block_table[0, j // 64], j % 64, 0]) for j in range(100)])
    q = brute.bf16(w.q_bits[0, 0])
    for h in range(4):
        s = keys @ q[h]
        top = np.argsort(s)[::-1]
        assert (s[top[0]] - s[top[1]]) * 50.0 > 40  # margin makes the one-hot exact to fp64
        np.testing.assert_allclose(out[0, 0, h], keys[top[0], :512], rtol=0, atol=1e-12)


def test_rope_dims_enter_the_score():
    # Flip only the RoPE part of one key: its score, and so the output, must change.
    w = tiny_dense(26, 1, 1, 1, [20], 1)
    a, la = run_oracle(w)
    w.kcache_bits[w.block_table[0, 0], 3, 0, 512:] ^= np.uint16(0x8000)
    b, lb = run_oracle(w)
    assert not np.allclose(a, b) and la[0, 0, 0] != lb[0, 0, 0]


def test_empty_request():
    w = tiny_dense(27, 2, 1, 2, [0, 10], 2)
    out, lse = run_oracle(w)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf) and np.all(np.isfinite(lse[1]))


# ----------------------------------------------------------------------------- dense: invariants

def test_causal_single_token_equals_noncausal():
    w = tiny_dense(31, 2, 1, 3, [70, 129], 5)
    a = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, False)
    b = O.mla_decode(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_row_equals_shorter_noncausal():
    # Row i of an s_q-token causal decode sees exactly seqlen - s_q + i + 1 keys (bottom-right alignment).
    w = tiny_dense(32, 1, 3, 2, [100], 2, causal=True)
    out, lse = run_oracle(w)
    for i in range(3):
        n = 100 - 3 + i + 1
        o2, l2 = O.mla_decode(w.q_bits[:, i:i + 1], w.kcache_bits, w.block_table, np.array([n], np.int32),
                              w.scale, False)
        assert np.array_equal(out[0, i], o2[0, 0]) and np.array_equal(lse[0, i], l2[0, 0])


@pytest.mark.parametrize("cuts", [[0, 64, 200], [0, 0, 1, 150, 200], [0, 199, 200, 200], [0, 37, 111, 200]])
def test_split_then_combine_equals_unsplit(cuts):
    w = tiny_dense(33, 1, 2, 3, [200], 4, causal=True)
    out, lse = run_oracle(w)
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        parts.append(O.mla_decode_partial(w.q_bits, w.kcache_bits, w.block_table, w.seqlens, w.scale, True,
                                          [lo], [hi]))
    for i in range(2):
        for h in range(3):
            o = np.stack([p[0][0, i, h] for p in parts])
            l = np.array([p[1][0, i, h] for p in parts])
            mo, ml = O.lse_combine(o, l)
            np.testing.assert_allclose(mo, out[0, i, h], rtol=0, atol=1e-12)
            assert abs(ml - lse[0, i, h]) < 1e-12


def test_combine_of_empty_parts():
    o, l = O.lse_combine(np.zeros((3, 512)), np.full(3, -np.inf))
    assert np.all(o == 0) and l == -np.inf


def test_page_permutation_invariance():
    w = tiny_dense(34, 2, 1, 2, [100, 160], 6)
    a = run_oracle(w)
    perm = np.random.default_rng(0).permutation(6)
    inv = np.argsort(perm)
    kc2 = w.kcache_bits[perm]                  # new page p holds old page perm[p]
    bt2 = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b = O.mla_decode(w.q_bits, kc2, bt2, w.seqlens, w.scale, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_out_of_range_page_is_an_error_not_a_read():
    w = tiny_dense(35, 1, 1, 1, [10], 1)
    w.block_table[0, 0] = 5
    with pytest.raises(ValueError):
        run_oracle(w)


# ----------------------------------------------------------------------------- FP8 E4M3FN

def test_e4m3fn_fixed_points():
    # OCP 8-bit floating point specification, E4M3: bias 7, max normal 448, min subnormal 2^-9, NaN S.1111.111
    assert O.e4m3fn_to_f64(0x00) == 0.0 and math.copysign(1, O.e4m3fn_to_f64(0x80)) < 0
    assert O.e4m3fn_to_f64(0x01) == 2.0 ** -9
    assert O.e4m3fn_to_f64(0x07) == 7 * 2.0 ** -9
    assert O.e4m3fn_to_f64(0x08) == 2.0 ** -6
    assert O.e4m3fn_to_f64(0x38) == 1.0
    assert O.e4m3fn_to_f64(0x7E) == 448.0 and O.e4m3fn_to_f64(0xFE) == -448.0
    assert math.isnan(O.e4m3fn_to_f64(0x7F)) and math.isnan(O.e4m3fn_to_f64(0xFF))
    assert O.e4m3fn_to_f64(0x77) == 240.0 and O.e4m3fn_to_f64(0x78) == 256.0


def test_e4m3fn_all_codes_match_torch():
    tab = brute.e4m3fn_table()
    mine = np.array([O.e4m3fn_to_f64(c) for c in range(256)])
    nan = np.isnan(tab)
    assert np.array_equal(nan, np.isnan(mine)) and nan.sum() == 2
    assert np.array_equal(mine[~nan], tab[~nan])


def test_record_decode_hand_built():
    rec = np.zeros((1, 64, 1, 656), np.uint8)
    r = rec[0, 5, 0]
    r[0] = 0x38            # 1.0   * scale0
    r[127] = 0xB8          # -1.0  * scale0
    r[128] = 0x40          # 2.0   * scale1
    r[511] = 0x01          # 2^-9  * scale3
    r[512:528] = np.array([0.5, 3.0, 1.0, 1024.0], "<f4").view(np.uint8)
    rope = np.zeros(64, np.float32)
    rope[0], rope[63] = 1.5, -0.25
    r[528:656] = W.f32_to_bf16_bits(rope).astype("<u2").view(np.uint8)
    k = O.decode_record(rec, 5)
    assert k[0] == 0.5 and k[127] == -0.5 and k[128] == 6.0 and k[511] == 1024.0 * 2.0 ** -9
    assert k[512] == 1.5 and k[575] == -0.25 and np.count_nonzero(k) == 6
    np.testing.assert_array_equal(k, brute.dequant_records(rec.reshape(-1, 656)[5:6])[0])


def small_sparse(seed, b, h, cap, topk, context, s_q=1):
    return W.sparse_workload("tiny-sparse", seed, b, h, cap, topk, context=context, s_q=s_q)


@pytest.mark.parametrize("seed,b,h,cap,topk,context,s_q", [
    (41, 2, 4, 128, [128, 70], 1024, 1),
    (42, 3, 2, 64, [1, 0, 64], 256, 2),
])
def test_sparse_matches_brute_force(seed, b, h, cap, topk, context, s_q):
    w = small_sparse(seed, b, h, cap, topk, context, s_q)
    out, lse = O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)
    bo, bl = brute.sparse(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)


def test_sparse_suffix_is_masked_not_zero_keys():
    w = small_sparse(43, 1, 2, 128, [70], 512)
    out, lse = O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)
    # Attending the 58 zero-filled suffix slots as keys would add 58 keys of score 0.
    with_zeros = np.log(np.exp(lse) + 58.0)
    assert np.all(np.abs(with_zeros - lse) > 1e-3)


def test_pack_matches_brute_force_bytes():
    w = small_sparse(44, 3, 1, 192, [192, 65, 0], 2048, s_q=2)
    ws = O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens)
    assert ws.shape == (6, 3, 64, 656)
    assert np.array_equal(ws, brute.pack(w.kcache_rec, w.indices, w.seqlens))
    assert np.all(ws[4:6] == 0)  # request 2 has topk_length 0: all zero


def test_sparse_equals_dense_over_packed_records():
    # Decoding from the pack (record k of a row at tile k//64, slot k%64) equals decoding by index.
    w = small_sparse(45, 2, 3, 128, [128, 90], 1024)
    ws = O.pack_selected_kv(w.kcache_rec, w.indices, w.seqlens)
    rows = ws.reshape(2, 128, 1, 656)  # one "page pool" of 2 rows x 2 tiles: tile-major = record-major
    ident = np.full((2, 1, 128), -1, np.int32)
    for r in range(2):
        ident[r, 0, :w.seqlens[r]] = r * 128 + np.arange(w.seqlens[r])
    pool = rows.reshape(4, 64, 1, 656)
    a = O.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale)
    b = O.mla_sparse_decode(w.q_bits, pool, ident, w.seqlens, w.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- scheduler partition

@pytest.mark.parametrize("limit", [None, "dense"])
@pytest.mark.parametrize("lengths,P", [
    ([4096] * 8, 32), ([4096] * 3, 7), ([1, 64, 65, 0, 300], 4), ([0, 0], 3), ([10], 5),
    ([2048, 4096, 3000, 100], 9), ([64] * 5, 5), ([128, 64], 1),
    ([1, 700, 2049], 64), ([300, 10, 0, 640], 50), ([4096], 256),   # more parts than blocks
    ([65536], 128), ([16384], 128), ([65536, 64, 64, 64], 200),     # cut by the dense split limit
])
def test_sched_partition_invariants(lengths, P, limit):
    meta, ns = O.sched_partition(lengths, P, split_limit=limit)
    blocks = [(max(n, 0) + 63) // 64 for n in lengths]
    T = sum(blocks)
    cum = np.concatenate([[0], np.cumsum(blocks)])
    P_all = P
    if limit == "dense":
        # the owner closed form below works with the number of parts in use
        P = min(P, max(16 * len(lengths), min(-(-T // 4), 64 * len(lengths))))
    owned = np.zeros(T, int)
    sizes = []
    assert meta.shape == (P_all, 8)
    assert np.all(meta[P:, :5] == -1) and np.all(meta[P:, 5:] == 0)
    for p in range(P):
        br, bk, er, ek, bs = meta[p, :5]
        assert np.all(meta[p, 5:] == 0)
        if br < 0:
            sizes.append(0)
            continue
        g0, g1 = cum[br] + bk, cum[er] + ek
        assert g1 > g0
        owned[g0:g1] += 1
        sizes.append(g1 - g0)
        # closed form of the owner part, independent of the scan
        assert brute.part_of(g0, T, P) == p and brute.part_of(g1 - 1, T, P) == p
        assert bs == p - brute.part_of(cum[br], T, P)
    assert np.all(owned == 1)
    if T:
        Pe = min(P, T)
        assert all(x > 0 for x in sizes[:Pe]) and all(x == 0 for x in sizes[Pe:])  # empty parts only trail
        assert max(sizes[:Pe]) - min(sizes[:Pe]) <= 1 and sum(sizes) == T
    for r, nb in enumerate(blocks):
        expect = 0 if nb == 0 else brute.part_of(cum[r] + nb - 1, T, P) - brute.part_of(cum[r], T, P) + 1
        assert ns[r + 1] - ns[r] == expect
    assert ns[-1] <= sum(1 for x in blocks if x) + P - 1


@pytest.mark.parametrize("b,T,want", [
    (1, 16, 16), (1, 64, 16), (1, 65, 17), (1, 256, 64), (1, 1024, 64), (2, 1024, 128), (4, 257, 65),
    (64, 4096, 1024), (16, 8192, 1024), (3, 45, 48), (1, 0, 16),
])
def test_dense_split_limit(b, T, want):
    """The dense metadata call's split limit: 16 parts per request, one per 4
    blocks beyond that, 64 per request at most (values worked by hand)."""
    assert O.dense_split_limit(b, T) == want


@pytest.mark.parametrize("lengths,P", [
    ([2048] * 8, 256), ([1536, 2048, 1700, 1600], 64), ([1, 64, 65, 0, 300], 4), ([0, 0], 3), ([10], 5),
    ([2048, 4096, 3000, 100], 9), ([64] * 5, 5), ([128, 64], 2), ([4096], 256), ([700, 0, 2049], 7),
    (list(np.random.default_rng(5).integers(0, 3000, size=40)), 128),
])
def test_request_local_partition_invariants(lengths, P):
    res = O.sched_partition_request_local(lengths, P)
    blocks = [(max(n, 0) + 63) // 64 for n in lengths]
    assert res is not None
    meta, ns = res
    T = sum(blocks)
    owned = [np.zeros(b, int) for b in blocks]
    pieces = {}
    used = 0
    for p in range(P):
        br, bk, er, ek, i = meta[p, :5]
        assert np.all(meta[p, 5:] == 0)
        if br < 0:
            assert np.all(meta[p, :5] == -1)
            assert all(meta[q, 0] < 0 for q in range(p, P))  # empty parts only trail
            break
        used += 1
        assert br == er and ek > bk  # never spans two requests
        owned[br][bk:ek] += 1
        pieces.setdefault(br, []).append((i, ek - bk, p))
    assert all(np.all(o == 1) for o in owned)  # every block exactly once
    assert used <= P and ns[-1] == used
    for r, nb in enumerate(blocks):
        got = sorted(pieces.get(r, []))
        assert ns[r + 1] - ns[r] == len(got)
        if nb:
            assert [g[0] for g in got] == list(range(len(got)))                    # split index in order
            assert [g[2] for g in got] == list(range(ns[r], ns[r] + len(got)))   # consecutive parts
            sizes = [g[1] for g in got]
            assert max(sizes) - min(sizes) <= 1                                    # balanced within the request
    # piece counts: ceil(b_r / B) for the smallest B (searched from 1 here) that fits in P parts
    if T:
        B = next(x for x in range(1, max(blocks) + 1) if sum((b + x - 1) // x for b in blocks) <= P)
        assert all(ns[r + 1] - ns[r] == (b + B - 1) // B for r, b in enumerate(blocks))


def test_request_local_partition_needs_a_part_per_request():
    assert O.sched_partition_request_local([64, 64, 64], 2) is None
    assert O.sched_partition_request_local([64, 0, 64], 2) is not None


# ----------------------------------------------------------------------------- numbers the pages print

def test_page_byte_facts():
    facts = {f["id"]: f["derived_bytes"] for f in json.load(open(GOLDEN))["facts"]}
    assert facts["q_tile_16_rows"] == 16 * W.D_QK * 2
    assert facts["kv_page_64_tokens"] == W.PAGE * W.D_QK * 2
    assert facts["kv_tile_16x3_stages"] == 16 * W.D_QK * 2 * 3
    assert facts["v_columns"] == W.D_V == O.D_V
    assert facts["fp8_record"] == W.REC_BYTES == O.REC_BYTES == 512 + 4 * 4 + 64 * 2
    assert facts["packed_workspace_per_row_topk2048"] == 2048 * O.REC_BYTES
    assert abs(facts["packed_workspace_per_row_topk2048"] / 2**20 - 1.281) < 5e-4
    w = W.dense_workload("kvbytes", 0, 2, 1, 1, [4096, 4096], pool_pages=128)
    assert w.kv_bytes() * 32 == facts["kv_cache_b64_sk4096"]
    assert abs(facts["kv_cache_b64_sk4096"] / 1e6 - 302) < 0.5
