"""Counts where the decode kernels' online softmax moves its reference maximum.

The kernels keep, per query row and per piece of the sequence, a reference
maximum m (log2 units, scale included).  After each 32-key tile they compare
the tile's maximum score x with m; if x > m + 8, m becomes x and everything
accumulated so far is rescaled by 2^(m_old - m_new).  The first tile of a piece
always sets m (from -inf); the tests care about the moves after it, which take
the rescale branch.

This module replays that rule in fp64 on the CPU (scores from the exact inputs),
so a test can assert that its workload really drives the kernels through the
branch before comparing their output with the oracle.  `margin` keeps only
moves that clear the threshold by that much, so fp32-versus-fp64 differences
in the scores cannot change the count.
"""

import math

import numpy as np

from mla_paged_kv_amd import workloads as W
from oracle import oracle as O

TILE = 32
THRESHOLD = 8.0
LOG2E = 1.0 / math.log(2.0)


def pieces(lengths, num_parts, split_limit=None):
    """(request, first key, end key) of every piece, from the scheduler partition
    (split_limit "dense" for the dense metadata call's partition)."""
    meta, _ = O.sched_partition(lengths, num_parts, split_limit=split_limit)
    out = []
    for br, bb, er, eb, _split in meta[:, :5]:
        if br < 0:
            continue
        for r in range(br, er + 1):
            n = int(lengths[r])
            nblk = (n + 63) // 64
            b0 = bb if r == br else 0
            b1 = eb if r == er else nblk
            lo, hi = 64 * int(b0), min(64 * int(b1), n)
            if hi > lo:
                out.append((r, lo, hi))
    return out


def count_moves(scores, lo, hi, threshold=THRESHOLD, margin=0.5):
    """scores: fp64 [rows, n] in log2 units (-inf where a key is not visible).
    Returns (robust moves after the first tile, ambiguous comparisons)."""
    m = np.full(scores.shape[0], -np.inf)
    moves = ambiguous = 0
    first = True
    for t0 in range(lo, hi, TILE):
        x = np.max(scores[:, t0:min(t0 + TILE, hi)], axis=1)
        d = x - (m + threshold)
        upd = d > 0
        if not first:
            moves += int(np.sum(d > margin))
            ambiguous += int(np.sum(np.isfinite(d) & (np.abs(d) <= margin)))
        m = np.where(upd, x, m)
        first = False
    return moves, ambiguous


def dense_scores(w, r):
    """Scores of request r, log2 units: [s_q * h_q, seqlen] (causal keys masked)."""
    n = int(w.seqlens[r])
    wide = (lambda b: b.view(np.float16).astype(np.float64)) if w.dtype == "fp16" else \
        (lambda b: W.bf16_bits_to_f32(b).astype(np.float64))
    j = np.arange(n)
    pages = w.block_table[r, j // 64]
    h_kv = w.kcache_bits.shape[2]
    keys = wide(w.kcache_bits[pages, j % 64])          # [n, h_kv, 576]
    q = wide(w.q_bits[r])                               # [s_q, h_q, 576]
    g = w.h_q // h_kv
    s = np.empty((w.s_q, w.h_q, n))
    for kvh in range(h_kv):
        s[:, kvh * g:(kvh + 1) * g] = q[:, kvh * g:(kvh + 1) * g] @ keys[:, kvh].T
    s *= w.scale * LOG2E
    if w.causal:
        for i in range(w.s_q):
            s[i, :, max(n - w.s_q + i + 1, 0):] = -np.inf
    return s.reshape(w.s_q * w.h_q, n)


def sparse_scores(w, r):
    """Scores of request r over its selected keys, log2 units: [s_q * h_q, topk_length]."""
    n = int(w.seqlens[r])
    q = W.bf16_bits_to_f32(w.q_bits[r]).astype(np.float64)  # [s_q, h_q, 576]
    s = np.empty((w.s_q, w.h_q, n))
    for i in range(w.s_q):
        keys = np.stack([O.decode_record(w.kcache_rec, int(w.indices[r, i, k])) for k in range(n)]) if n else \
            np.zeros((0, 576))
        s[i] = q[i] @ keys.T
    s *= w.scale * LOG2E
    return s.reshape(w.s_q * w.h_q, n)


def moves_for(w, num_parts, margin=0.5):
    """Total robust moves after the first tile over every piece of w, and the
    number of ambiguous comparisons."""
    scorer = sparse_scores if w.fp8 else dense_scores
    cache = {}
    total = amb = 0
    for r, lo, hi in pieces([int(x) for x in w.seqlens], num_parts, None if w.fp8 else "dense"):
        if r not in cache:
            cache[r] = scorer(w, r)
        mv, am = count_moves(cache[r], lo, hi, margin=margin)
        total += mv
        amb += am
    return total, amb
