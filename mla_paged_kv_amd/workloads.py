"""Seeded synthetic inputs for MLA decode over a paged KV cache.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no attention arithmetic: it only draws random numbers (numpy PCG64 in a
fixed order), rounds them to the input encodings (bf16 bit patterns, OCP E4M3
bytes via torch's float8_e4m3fn cast) and builds page tables.  It imports
neither the oracle nor the GPU binding.

Workload shapes follow the configurations the pages' problem statement uses
(FlashMLA PR 183 "Performance" table: b=64 sk=4096 and friends; FlashMLA PR 200
"L20X results": top-k 2048 selected records, H in {64, 128}).  Values are
N(0, 1) (times 0.5 where noted), the 64-token pages of a request are scattered
over a shuffled pool, cache slots that no request may read hold a large finite
sentinel (+-1e4) so that any leak shows up in the output, and unused
block-table entries are -1.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np

D_QK = 576
D_V = 512
PAGE = 64
REC_BYTES = 656
E4M3_MAX = 448.0
SENTINEL = 1.0e4


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs only (no overflow below 0xFFFF8000): add half an ulp, ties to even
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def abi_scale(scale=None) -> float:
    """The softmax scale as the C ABI receives it: a float (fp32) argument.  The
    workload stores that fp32 value, widened, so the oracle and the kernels see
    the same number (default 576^-0.5)."""
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    return float(np.float32(scale))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    s_q: int
    h_q: int
    scale: float
    causal: bool
    q_bits: np.ndarray                      # uint16 [b, s_q, h_q, 576]
    seqlens: np.ndarray                     # int32 [b] (sparse: topk_length)
    fp8: bool = False
    kcache_bits: Optional[np.ndarray] = None  # uint16 [pages, 64, h_kv, 576]
    block_table: Optional[np.ndarray] = None  # int32 [b, max_pages]
    kcache_rec: Optional[np.ndarray] = None   # uint8 [pages, 64, 1, 656]
    indices: Optional[np.ndarray] = None      # int32 [b, s_q, cap]
    topk_capacity: int = 0
    num_parts: Optional[int] = None           # forced split count (None = library's choice)
    dtype: str = "bf16"                       # encoding of q_bits / kcache_bits: "bf16" or "fp16" (IEEE binary16)

    @property
    def num_pages(self) -> int:
        return (self.kcache_rec if self.fp8 else self.kcache_bits).shape[0]

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: every visible key once (576 bf16, or one 656-B record)."""
        per = REC_BYTES if self.fp8 else D_QK * 2
        return int(np.sum(np.maximum(self.seqlens.astype(np.int64), 0))) * per

    def flops(self) -> int:
        """2 * (576 + 512) multiply-adds per (query row, visible key)."""
        total = 0
        for r in range(self.batch):
            n = int(self.seqlens[r])
            for i in range(self.s_q):
                vis = n
                if self.causal:
                    vis = min(max(n - self.s_q + i + 1, 0), n)
                total += vis * self.h_q
        return 2 * (D_QK + D_V) * total

    def digests(self) -> dict:
        out = {}
        for f in ("q_bits", "kcache_bits", "block_table", "seqlens", "kcache_rec", "indices"):
            a = getattr(self, f)
            if a is not None:
                out[f] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
        return out


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit patterns, round to nearest even (bf16, or IEEE binary16 via numpy)."""
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(x)


def _normal_bf16(rng: np.random.Generator, shape, std=1.0, dtype="bf16") -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _to_bits(x, dtype)


def _paged_pool(rng, num_pages, std, chunk=256, dtype="bf16", h_kv=1):
    """16-bit pool [pages, 64, h_kv, 576] of N(0, std^2) values, drawn page-chunk by page-chunk."""
    pool = np.empty((num_pages, PAGE, h_kv, D_QK), np.uint16)
    for p0 in range(0, num_pages, chunk):
        p1 = min(num_pages, p0 + chunk)
        pool[p0:p1] = _normal_bf16(rng, (p1 - p0, PAGE, h_kv, D_QK), std, dtype)
    return pool


def _seal_pool(pool, block_table, seqlens, dtype="bf16"):
    """Write the sentinel into every cache slot that no request may read."""
    used = np.zeros(pool.shape[0], bool)
    sent = _to_bits(np.array([SENTINEL, -SENTINEL], np.float32), dtype)
    pattern = np.resize(sent, D_QK)
    for r, n in enumerate(seqlens):
        n = int(n)
        npg = (n + PAGE - 1) // PAGE
        for k in range(npg):
            pg = block_table[r, k]
            used[pg] = True
            if k == npg - 1 and n % PAGE:
                pool[pg, n % PAGE:, :, :] = pattern
    pool[~used] = pattern


def dense_workload(name, seed, batch, s_q, h_q, seqlens, pool_pages, std=1.0, causal=False, scale=None,
                   max_pages=None, num_parts=None, block_table_mode="shuffled", dtype="bf16", h_kv=1) -> Workload:
    """Dense paged workload (bf16, or fp16 with dtype="fp16"; h_kv KV heads per
    token).  Draw order: q, pool, page permutation."""
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, np.int32)
    assert seqlens.shape == (batch,)
    pages_needed = [(int(n) + PAGE - 1) // PAGE for n in seqlens]
    if max_pages is None:
        max_pages = max(1, max(pages_needed) if pages_needed else 1)
    assert sum(pages_needed) <= pool_pages, "pool too small"
    q = _normal_bf16(rng, (batch, s_q, h_q, D_QK), std, dtype)
    pool = _paged_pool(rng, pool_pages, std, dtype=dtype, h_kv=h_kv)
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((batch, max_pages), -1, np.int32)
    pos = 0
    for r in range(batch):
        k = pages_needed[r]
        bt[r, :k] = perm[pos:pos + k]
        pos += k
    _seal_pool(pool, bt, seqlens, dtype)
    return Workload(name=name, seed=seed, batch=batch, s_q=s_q, h_q=h_q, scale=abi_scale(scale), causal=causal,
                    q_bits=q, seqlens=seqlens, kcache_bits=pool, block_table=bt, num_parts=num_parts, dtype=dtype)


def encode_records(x: np.ndarray) -> np.ndarray:
    """float32 [n, 576] -> n 656-byte records: per 128-dim NoPE block scale =
    amax/448 (fp32), code = E4M3 of x/scale; RoPE = bf16(x[512:576])."""
    import torch  # encoding only (float8_e4m3fn cast)

    n = x.shape[0]
    recs = np.empty((n, REC_BYTES), np.uint8)
    nope = x[:, :512].reshape(n, 4, 128)
    amax = np.max(np.abs(nope), axis=2).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(nope / scale[:, :, None], -E4M3_MAX, E4M3_MAX).reshape(n, 512)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    recs[:, :512] = codes
    recs[:, 512:528] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    recs[:, 528:656] = f32_to_bf16_bits(x[:, 512:]).astype("<u2").view(np.uint8).reshape(n, 128)
    return recs


def _records(rng, n_tokens, chunk=4096):
    """n_tokens records (encode_records) of x ~ N(0, 1)."""
    recs = np.empty((n_tokens, REC_BYTES), np.uint8)
    for t0 in range(0, n_tokens, chunk):
        t1 = min(n_tokens, t0 + chunk)
        recs[t0:t1] = encode_records(rng.standard_normal(size=(t1 - t0, D_QK), dtype=np.float32))
    return recs


def sparse_workload(name, seed, batch, h_q, cap, topk_lengths, context, s_q=1, scale=None,
                    num_parts=None) -> Workload:
    """Packed top-k FP8 workload.  Each request owns ceil(context/64) pages of the
    pool (request-disjoint), reached through its own shuffled page table; the
    top-k are `cap` logical positions drawn without replacement from
    [0, context) and translated to physical token ids; the invalid suffix is -1.
    Draw order: q, records, per-request page permutation, per-request positions."""
    rng = np.random.default_rng(seed)
    topk = np.asarray(topk_lengths, np.int32)
    assert topk.shape == (batch,) and cap % PAGE == 0
    ppr = (context + PAGE - 1) // PAGE
    pool_pages = batch * ppr
    q = _normal_bf16(rng, (batch, s_q, h_q, D_QK))
    recs = _records(rng, pool_pages * PAGE).reshape(pool_pages, PAGE, 1, REC_BYTES)
    indices = np.full((batch, s_q, cap), -1, np.int32)
    for r in range(batch):
        table = (r * ppr + rng.permutation(ppr)).astype(np.int64)
        for i in range(s_q):
            logical = rng.choice(context, size=cap, replace=False).astype(np.int64)
            phys = table[logical // PAGE] * PAGE + logical % PAGE
            n = int(topk[r])
            indices[r, i, :n] = phys[:n].astype(np.int32)
    return Workload(name=name, seed=seed, batch=batch, s_q=s_q, h_q=h_q, scale=abi_scale(scale), causal=False,
                    q_bits=q, seqlens=topk, fp8=True, kcache_rec=recs, indices=indices, topk_capacity=cap,
                    num_parts=num_parts)


# --------------------------------------------------------------------------- planted score jumps
#
# Inputs whose running score maximum jumps at chosen key positions, so that an
# online softmax has to move its reference maximum (and rescale what it has
# accumulated) in the middle of a piece, at a split boundary and in a partial
# last tile.  Every query row of request r gets a component u_r shared by all
# its heads and tokens (u_r ~ N(0, 1)^576); a planted key gets beta * u_r / 24
# added.  With the default scale 1/24 the planted key's score is then about
# beta + N(0, 2) for every head, against N(0, 2) for the other keys.


def _shared_directions(seed, batch):
    return np.random.default_rng(seed + 7919).standard_normal(size=(batch, D_QK), dtype=np.float32)


def plant_dense(w: Workload, plants) -> Workload:
    """Add the shared component to every query of w and beta * u_r / 24 to key j of
    request r for each (r, j, beta) in `plants` (positions below seqlen)."""
    u = _shared_directions(w.seed, w.batch)
    wide = (lambda b: b.view(np.float16).astype(np.float32)) if w.dtype == "fp16" else bf16_bits_to_f32
    q = wide(w.q_bits) + u[:, None, None, :]
    w.q_bits = _to_bits(q, w.dtype)
    for r, j, beta in plants:
        assert 0 <= j < int(w.seqlens[r])
        pg, sl = int(w.block_table[r, j // PAGE]), j % PAGE
        k = wide(w.kcache_bits[pg, sl]) + np.float32(beta / 24.0) * u[r][None, :]
        w.kcache_bits[pg, sl] = _to_bits(k, w.dtype)
    return w


def plant_sparse(w: Workload, plants) -> Workload:
    """The same for a top-k FP8 workload: (r, k, beta) boosts the record selected
    at top-k position k (k < topk_length[r]) of every query token of request r;
    the record is re-encoded from its decoded value plus the boost."""
    u = _shared_directions(w.seed, w.batch)
    q = bf16_bits_to_f32(w.q_bits) + u[:, None, None, :]
    w.q_bits = f32_to_bf16_bits(q)
    flat = w.kcache_rec.reshape(-1, REC_BYTES)
    import torch  # decoding the E4M3 bytes of the record being re-encoded

    for r, k, beta in plants:
        assert 0 <= k < int(w.seqlens[r])
        for i in range(w.s_q):
            idx = int(w.indices[r, i, k])
            rec = flat[idx]
            codes = torch.from_numpy(rec[:512].copy()).view(torch.float8_e4m3fn).float().numpy()
            sc = rec[512:528].view("<f4").astype(np.float32)
            x = np.empty(D_QK, np.float32)
            x[:512] = (codes.reshape(4, 128) * sc[:, None]).reshape(512)
            x[512:] = bf16_bits_to_f32(rec[528:656].view("<u2"))
            x += np.float32(beta / 24.0) * u[r]
            flat[idx] = encode_records(x[None, :])[0]
    return w


# --------------------------------------------------------------------------- named configurations

def config(name: str) -> Workload:
    """The named workloads.

    c1  b=1  s_q=1 h_q=16  sk=256 over a 4-page pool, N(0,1), no split
    c2  b=1  s_q=1 h_q=128 sk=4096 (64 pages) over a 256-page pool, N(0,1)*0.5, split-K + combine
    c3  b=64 s_q=1 h_q=128 sk ~ U{2048..4096}, pages scattered over the pool
    c4  b=16 s_q=2 causal h_q=128 sk=16384
    c5  b=8  s_q=1 h_q=64 top-k 2048 FP8 records from a 32768-token context, topk_length ~ U{1536..2048}
    h   b=64 s_q=1 h_q=128 sk=4096 (the headline bandwidth shape)
    """
    if name == "c1":
        return dense_workload("c1", 1, 1, 1, 16, [256], pool_pages=4, num_parts=1)
    if name == "c2":
        return dense_workload("c2", 2, 1, 1, 128, [4096], pool_pages=256, std=0.5)
    if name == "c3":
        rng = np.random.default_rng(3)
        seqlens = rng.integers(2048, 4096, size=64, endpoint=True).astype(np.int32)
        return dense_workload("c3", 3, 64, 1, 128, seqlens, pool_pages=4096, max_pages=64)
    if name == "c4":
        return dense_workload("c4", 4, 16, 2, 128, [16384] * 16, pool_pages=4096, causal=True)
    if name == "c5":
        rng = np.random.default_rng(5)
        topk = rng.integers(1536, 2048, size=8, endpoint=True).astype(np.int32)
        return sparse_workload("c5", 5, 8, 64, 2048, topk, context=32768)
    if name == "h":
        return dense_workload("h", 64, 64, 1, 128, [4096] * 64, pool_pages=4096)
    raise KeyError(name)


CONFIGS = ("c1", "c2", "c3", "c4", "c5", "h")
