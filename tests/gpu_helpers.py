"""Helpers for the GPU parity tests: move seeded workloads to the device, run the
library through its C ABI binding, and compare with the oracle."""

import sys

import numpy as np
import torch

from mla_paged_kv_amd import ops

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3
REL_RMS_ALARM = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensors(w, device="cuda:0"):
    t = {}
    act = torch.float16 if getattr(w, "dtype", "bf16") == "fp16" else torch.bfloat16
    t["q"] = torch.from_numpy(w.q_bits.view(np.int16)).to(device).view(act)
    t["seqlens"] = torch.from_numpy(w.seqlens).to(device)
    if w.fp8:
        t["kcache_rec"] = torch.from_numpy(w.kcache_rec).to(device)
        t["indices"] = torch.from_numpy(w.indices).to(device)
    else:
        t["kcache"] = torch.from_numpy(w.kcache_bits.view(np.int16)).to(device).view(act)
        t["block_table"] = torch.from_numpy(w.block_table).to(device)
    return t


def run_dense(w, t=None, num_parts=None):
    t = t or dev_tensors(w)
    parts = num_parts if num_parts is not None else w.num_parts
    fmt = ops.KV_FP16_PAGED if getattr(w, "dtype", "bf16") == "fp16" else ops.KV_BF16_PAGED
    plan = ops.DecodePlan(t["seqlens"], w.s_q, w.h_q, fmt, num_parts=parts)
    out, lse = ops.mla_decode(t["q"], t["kcache"], t["block_table"], t["seqlens"], w.scale, w.causal, plan=plan,
                              kv_format=fmt)
    torch.cuda.synchronize()
    return out, lse, plan


def run_sparse(w, t=None, num_parts=None):
    t = t or dev_tensors(w)
    ws = ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"])
    plan = ops.DecodePlan(t["seqlens"], w.s_q, w.h_q, ops.KV_FP8_PACKED, num_parts=num_parts or w.num_parts,
                          topk_capacity=w.topk_capacity)
    out, lse = ops.mla_decode(t["q"], ws, None, t["seqlens"], w.scale, False, plan=plan,
                              kv_format=ops.KV_FP8_PACKED, topk_capacity=w.topk_capacity)
    torch.cuda.synchronize()
    return out, lse, ws, plan


def run_sparse_indexed(w, t=None, num_parts=None):
    """Sparse FP8 decode straight from the record pool (records gathered by
    top-k id inside the decode, no pack)."""
    t = t or dev_tensors(w)
    plan = ops.DecodePlan(t["seqlens"], w.s_q, w.h_q, ops.KV_FP8_INDEXED, num_parts=num_parts or w.num_parts,
                          topk_capacity=w.topk_capacity)
    out, lse = ops.mla_decode(t["q"], t["kcache_rec"], t["indices"], t["seqlens"], w.scale, False, plan=plan,
                              kv_format=ops.KV_FP8_INDEXED, topk_capacity=w.topk_capacity)
    torch.cuda.synchronize()
    return out, lse, plan


def to_np(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(name, out, lse, ref_out, ref_lse):
    """Element-wise |gpu - ref| <= atol + rtol |ref| on out, |gpu - ref| <= 1e-3 on lse;
    rows the oracle calls empty (lse = -inf) must be exactly 0 / -inf.  Also
    reports max-abs, relative RMS and cosine and fails above 1e-2 relative RMS."""
    o, l = (out, lse) if isinstance(out, np.ndarray) else to_np(out, lse)
    assert o.shape == ref_out.shape and l.shape == ref_lse.shape
    empty = ~np.isfinite(ref_lse)
    assert np.all(np.isfinite(o)), f"{name}: non-finite output"
    assert np.all(o[empty] == 0) and np.all(l[empty] == -np.inf), f"{name}: empty rows not 0/-inf"
    err = np.abs(o - ref_out)
    bad = err > OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    lerr = np.abs(l[~empty] - ref_lse[~empty]) if (~empty).any() else np.zeros(1)
    num = np.linalg.norm(o - ref_out)
    den = np.linalg.norm(ref_out)
    rel_rms = num / den if den > 0 else num
    cos = float(np.sum(o * ref_out) / (np.linalg.norm(o) * den)) if den > 0 else 1.0
    say(f"  [{name}] out max_abs={err.max():.3e} rel_rms={rel_rms:.3e} cos={cos:.6f} "
        f"lse max_abs={lerr.max():.3e} bad={int(bad.sum())}/{bad.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} outputs outside atol/rtol 1e-2"
    assert lerr.max() <= LSE_ATOL, f"{name}: lse error {lerr.max()}"
    assert rel_rms <= REL_RMS_ALARM, f"{name}: relative RMS {rel_rms}"
    return rel_rms


def sub_workload(w, sel):
    """The same workload restricted to requests `sel` (rows are independent)."""
    import copy

    s = copy.copy(w)
    s.q_bits = np.ascontiguousarray(w.q_bits[sel])
    s.seqlens = np.ascontiguousarray(w.seqlens[sel])
    s.batch = len(sel)
    if w.fp8:
        s.indices = np.ascontiguousarray(w.indices[sel])
    else:
        s.block_table = np.ascontiguousarray(w.block_table[sel])
    return s
