"""Independent brute-force references used to pin the oracle (test helpers).

These are written as dense matrix computations in numpy (gather every visible
key into a matrix, one matmul for the scores, an explicit boolean mask, scipy's
logsumexp, one matmul for the output), which is a different formulation from
the oracle's per-row loops.  They exist only to check the oracle on tiny inputs.
"""

import numpy as np
from scipy.special import logsumexp

D_QK, D_V, PAGE, REC = 576, 512, 64, 656


def bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16(bits):
    """IEEE binary16 bit patterns -> float64 through numpy's float16."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def dense(q_bits, kcache_bits, block_table, seqlens, scale, causal, dtype="bf16"):
    dec = f16 if dtype == "fp16" else bf16
    q = dec(q_bits)                       # [b, s_q, h, 576]
    kc_all = dec(kcache_bits)             # [pages, 64, h_kv, 576]
    h_kv = kc_all.shape[2]
    b, s_q, h, _ = q.shape
    g = h // h_kv                         # query heads per KV head
    out = np.zeros((b, s_q, h, D_V))
    lse = np.full((b, s_q, h), -np.inf)
    for r in range(b):
        n = int(seqlens[r])
        if n == 0:
            continue
        j = np.arange(n)
        Kall = kc_all[block_table[r, j // PAGE], j % PAGE]   # [n, h_kv, 576]
        S = np.empty((s_q, h, n))
        for kk in range(h_kv):                                # heads of group kk use KV head kk
            Qg = q[r][:, kk * g:(kk + 1) * g].reshape(s_q * g, D_QK)
            S[:, kk * g:(kk + 1) * g] = scale * (Qg @ Kall[:, kk].T).reshape(s_q, g, n)
        mask = np.ones((s_q, n), bool)
        if causal:
            for i in range(s_q):
                mask[i] = j <= n - s_q + i
        S = np.where(mask[:, None, :], S, -np.inf)
        L = logsumexp(S, axis=2)                              # [s_q, h]
        ok = np.isfinite(L)
        P = np.where(ok[:, :, None], np.exp(S - np.where(ok, L, 0)[:, :, None]), 0.0)
        for kk in range(h_kv):
            out[r][:, kk * g:(kk + 1) * g] = P[:, kk * g:(kk + 1) * g] @ Kall[:, kk, :D_V]
        lse[r] = L
    return out, lse


def e4m3fn_table():
    """All 256 E4M3FN values from torch's own float8_e4m3fn type (library routine)."""
    import torch

    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def dequant_records(recs):
    """recs uint8 [n, 656] -> fp64 [n, 576] using the torch table + numpy views."""
    recs = np.ascontiguousarray(recs, np.uint8)
    tab = e4m3fn_table()
    nope = tab[recs[:, :512]]                                           # [n, 512]
    scales = recs[:, 512:528].copy().view("<f4").astype(np.float64)     # [n, 4]
    nope = nope * np.repeat(scales, 128, axis=1)
    rope = bf16(recs[:, 528:656].copy().view("<u2"))                    # [n, 64]
    return np.concatenate([nope, rope], axis=1)


def sparse(q_bits, kcache_rec, indices, topk_length, scale):
    q = bf16(q_bits)
    flat = kcache_rec.reshape(-1, REC)
    b, s_q, h, _ = q.shape
    out = np.zeros((b, s_q, h, D_V))
    lse = np.full((b, s_q, h), -np.inf)
    for r in range(b):
        n = int(topk_length[r])
        if n == 0:
            continue
        for i in range(s_q):
            K = dequant_records(flat[indices[r, i, :n]])
            S = scale * (q[r, i] @ K.T)
            L = logsumexp(S, axis=1)
            out[r, i] = np.exp(S - L[:, None]) @ K[:, :D_V]
            lse[r, i] = L
    return out, lse


def pack(kcache_rec, indices, topk_length):
    flat = kcache_rec.reshape(-1, REC)
    b, s_q, cap = indices.shape
    ws = np.zeros((b * s_q, cap, REC), np.uint8)
    for r in range(b):
        n = int(topk_length[r])
        for i in range(s_q):
            ws[r * s_q + i, :n] = flat[indices[r, i, :n]]
    return ws.reshape(b * s_q, cap // PAGE, PAGE, REC)


def part_of(g, T, P):
    """Closed form of the owner part of global block g under floor(p*T/P') boundaries, P' = min(P, T)."""
    Pe = min(P, T)
    return ((g + 1) * Pe - 1) // T
