"""Benchmark: achieved KV HBM bandwidth of MLA decode on one MI355X.

Default run (one JSON line on stdout): the headline workload -- b=64 requests,
s_q=1, h_q=128 query heads sharing one 576-dim latent KV head (V = its first
512 dims), 4096 cached tokens each, bf16, 64-token pages scattered over a
shuffled 4096-page pool (302 MB of KV).  One step is the whole hot path:
scheduler metadata + decode + combine.  Two copies of the pool alternate
between steps so that every step streams its KV from HBM (together more than
the 256 MB Infinity Cache).

  value            KV bytes per step / wall time per step, K steps launched back
                   to back on one stream through pre-bound C-ABI calls (no
                   per-call tensor checks), bracketed by device synchronisations.
  timed_region     the same region seen three ways: wall clock, a HIP-event span
                   on the stream, and the host's enqueue time per step (when the
                   enqueue time is below the event span, the host is not the
                   bound).
  decode_combine   the same loop without the metadata kernel (the metadata is
                   computed once per step and reused by every layer).
  kernels_ms       the decode alone launched K times back to back between two
                   HIP events (its mean duration), and per-kernel HIP-event
                   durations from a loop with an event between the kernels.
  graph_ms_per_step  the step replayed as a HIP graph (checked bitwise against
                   the eager step first).
  roofline         the decode kernel: algorithmic KV bytes per launch / its mean
                   duration back to back (HIP events), against 8 TB/s; `traffic` is the HBM bytes per
                   launch from the committed counter summary when it was taken on
                   the current kernel sources, else null.
  copy_bandwidth   a measured 1 GiB device-to-device copy (read + write bytes /
                   time), and value as a share of it.
  cpu_baseline     the fp64 oracle on the whole workload on the host cores, run
                   after the GPU measurements; the first step's output is checked
                   against it before anything is printed.
Before the W warmup steps, untimed steps run back to back for --warm-seconds so
that the GPU clock has ramped up when the measurements start.

Other modes (one JSON line per case):
  --configs   the five seeded test configurations and the headline shape, each
              timed cold (>= 512 MiB read between repetitions) as decode +
              combine over 5 alternating rounds (median and range of the round
              medians), metadata and pack reported separately, with the roofline
              of the binding unit; the oracle timed per configuration (median of
              3, plus 1-thread runs for the two single-request ones).
  --sweep     the dense page's twelve Performance configurations (same method,
              as a share of the measured copy bandwidth) and the packed page's
              B x S_q x H grid of top-k 2048 sparse decodes (packed with its pack,
              and by index), cold.
  --sparse    the sparse FP8 paths on two workloads as HIP graphs.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
FLUSH_BYTES = 512 << 20
ROUNDS = 5
PROFILE_PMC = os.path.join(ROOT, "profiles", "decode_kernel_h_profile.md")
KERNEL_SRCS = sorted(glob.glob(os.path.join(ROOT, "mla_paged_kv_amd", "csrc", "*.hip"))) + [
    os.path.join(ROOT, "mla_paged_kv_amd", "csrc", "mla_internal.h")]

# The dense page's Performance table ("Add SM80 (Ampere/A100) dense MLA decode
# kernel", Performance): batch, context length, query heads (128 unless noted).
DENSE_PAGE_CONFIGS = [(64, 4096, 128), (1, 4096, 64), (64, 1024, 128), (1, 16384, 128), (1, 256, 128),
                      (1, 1024, 128), (1, 4096, 128), (1, 65536, 128), (4, 1024, 128), (4, 4096, 128),
                      (16, 1024, 128), (16, 4096, 128)]
# The packed page's grid ("[SM90] Add packed selected-KV sparse decode", L20X
# results): top-k 2048, B x S_q x H.
PACKED_GRID_B = (1, 2, 4, 7, 8)
PACKED_GRID_SQ = (1, 2, 3, 4, 8, 16)
PACKED_GRID_H = (64, 128)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def emit(obj):
    print(json.dumps(obj), flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    if not os.path.exists(PROFILE_PMC):
        return None
    txt = open(PROFILE_PMC).read()
    m_src = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", txt)
    m_tot = re.search(r"hbm_bytes_per_decode_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_tot or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_tot.group(1))


def cpu_info() -> dict:
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def median_range(xs):
    import numpy as np

    xs = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(xs)), 5), "min": round(float(xs.min()), 5),
            "max": round(float(xs.max()), 5)}


# ----------------------------------------------------------------------------- timing

def timed_region(torch, stream, steps, issue):
    """Runs issue(i) for i < steps between two device synchronisations.  Returns
    wall ms/step, HIP-event span ms/step on `stream`, host enqueue us/step."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        issue(i)
    e1.record(stream)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return {"wall_ms_per_step": round((t1 - t0) * 1e3 / steps, 5),
            "event_span_ms_per_step": round(e0.elapsed_time(e1) / steps, 5),
            "host_enqueue_us_per_step": round((t_enq - t0) * 1e6 / steps, 2)}


def kernel_event_times(torch, stream, steps, calls_of_step):
    """Per-call HIP-event durations (ms): calls_of_step(i) -> list of zero-arg
    launches; an event is recorded before, between and after them."""
    import numpy as np

    n = len(calls_of_step(0))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        calls = calls_of_step(i)
        evs[i][0].record(stream)
        for k, c in enumerate(calls):
            c()
            evs[i][k + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([[e[k].elapsed_time(e[k + 1]) for k in range(n)] for e in evs])


def gpu_warm(torch, step, seconds):
    """Untimed back-to-back calls of step(i) for `seconds` (the clock ramps up)."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for i in range(10):
            step(n + i)
        n += 10
        torch.cuda.synchronize()
    return n


class Flusher:
    """Reads a buffer larger than the 256 MB Infinity Cache (and every L2), so
    that what follows reads its inputs from HBM.  A read, not a write: a
    written buffer would leave dirty lines whose write-back then competes with
    the measured kernel."""

    def __init__(self, torch, dev, nbytes=FLUSH_BYTES):
        self.buf = torch.ones((nbytes // 8,), dtype=torch.int64, device=dev)

    def __call__(self):
        self.buf.sum()


def cold_times(torch, stream, reps, calls, flush):
    """Each repetition: flush (untimed), then the calls between two events.
    Returns per-repetition ms for each call (array [reps, len(calls)])."""
    import numpy as np

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        flush()
        evs[i][0].record(stream)
        for k, c in enumerate(calls):
            c()
            evs[i][k + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([[e[k].elapsed_time(e[k + 1]) for k in range(len(calls))] for e in evs])


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """Measured device-to-device copy: (read + write bytes) / median time, GB/s."""
    import numpy as np

    src = torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)


# ----------------------------------------------------------------------------- workloads on the device

class DenseCase:
    """A dense workload on the device with its plan, buffers and pre-bound calls.
    `copies` pool copies (alternated between steps to keep the KV cold)."""

    def __init__(self, torch, ops, w, dev, copies=1, num_parts=None):
        import numpy as np

        self.w = w
        act = torch.float16 if getattr(w, "dtype", "bf16") == "fp16" else torch.bfloat16
        self.fmt = ops.KV_FP16_PAGED if act == torch.float16 else ops.KV_BF16_PAGED
        self.q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(act)
        pool = torch.from_numpy(w.kcache_bits.view(np.int16)).to(dev).view(act)
        self.pools = [pool] + [pool.clone() for _ in range(copies - 1)]
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.seqlens = torch.from_numpy(w.seqlens).to(dev)
        b, s_q, h_q = w.batch, w.s_q, w.h_q
        self.num_parts = num_parts or w.num_parts or ops.mla_decode_num_parts(b, s_q, h_q, 1, self.fmt)
        self.meta = torch.empty((self.num_parts, 8), dtype=torch.int32, device=dev)
        self.nsplit = torch.empty((b + 1,), dtype=torch.int32, device=dev)
        self.ws = torch.empty((ops.mla_decode_workspace_size(b, s_q, h_q, self.num_parts),), dtype=torch.uint8,
                              device=dev)
        self.out = torch.empty((b, s_q, h_q, 512), dtype=act, device=dev)
        self.lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
        self.kernel = ops.mla_decode_kernel_name(s_q, h_q, 1, self.fmt)
        self.ops = ops
        self.c_meta = ops.mla_get_decode_metadata(self.seqlens, b, s_q, h_q, 1, self.num_parts, self.meta,
                                                  self.nsplit, bind=True)
        self.c_dec = [ops.mla_decode_fwd(self.q, p, self.fmt, self.bt, self.seqlens, w.scale, w.causal, self.meta,
                                         self.nsplit, self.out, self.lse, self.ws, bind=True) for p in self.pools]
        self.c_comb = ops.mla_combine(self.nsplit, self.ws, b, s_q, h_q, self.num_parts, self.out, self.lse,
                                      kv_format=self.fmt, bind=True)

    def step_unbound(self, i):
        """The step through the checking entry points (reads the current stream
        at call time: usable under graph capture)."""
        o, w = self.ops, self.w
        o.mla_get_decode_metadata(self.seqlens, w.batch, w.s_q, w.h_q, 1, self.num_parts, self.meta, self.nsplit)
        o.mla_decode_fwd(self.q, self.pools[i % len(self.pools)], self.fmt, self.bt, self.seqlens, w.scale, w.causal,
                         self.meta, self.nsplit, self.out, self.lse, self.ws)
        o.mla_combine(self.nsplit, self.ws, w.batch, w.s_q, w.h_q, self.num_parts, self.out, self.lse,
                      kv_format=self.fmt)

    def step(self, i):
        self.c_meta()
        self.c_dec[i % len(self.c_dec)]()
        self.c_comb()

    def roof_us(self):
        """max(KV bytes / 8 TB/s, FLOP / 2.5 PFLOP/s) in us, and the binding unit."""
        t_hbm = self.w.kv_bytes() / (PEAK_HBM_GBS * 1e9) * 1e6
        t_mfma = self.w.flops() / (PEAK_BF16_TFLOPS * 1e12) * 1e6
        return (t_hbm, "hbm") if t_hbm >= t_mfma else (t_mfma, "mfma")


def cpu_leg_dense(w, out, lse, sel, threads, reps=1, gate=True):
    """The oracle on requests `sel` of w: checks the GPU output of those requests
    against it (raises on a mismatch), returns the median wall seconds of `reps`
    runs after one untimed run."""
    import numpy as np

    from oracle import oracle as orc
    from tests import gpu_helpers as G

    G.say = log
    sub = G.sub_workload(w, sel)
    dtype = getattr(w, "dtype", "bf16")
    args = (sub.q_bits, sub.kcache_bits, sub.block_table, sub.seqlens, w.scale, w.causal)
    ref = orc.mla_decode(*args, nthreads=threads, dtype=dtype)  # untimed: pages the pool in
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        orc.mla_decode(*args, nthreads=threads, dtype=dtype)
        ts.append(time.perf_counter() - t0)
    if gate:
        o_np = out.float().cpu().numpy().astype(np.float64)[sel]
        l_np = lse.cpu().numpy().astype(np.float64)[sel]
        G.compare(f"{w.name}-parity", o_np, l_np, ref[0], ref[1])
    return float(np.median(ts)), sub


# ----------------------------------------------------------------------------- headline

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-parts", type=int, default=0, help="force the split count (0 = library choice)")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed back-to-back steps before the warmup steps (the GPU clock ramps up)")
    ap.add_argument("--oracle-requests", type=int, default=64, help="requests in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph capture of the step (its bitwise check and its timing)")
    ap.add_argument("--profile-loop", action="store_true",
                    help="only warm up and run the step loop of --workload (for runs under a profiler)")
    ap.add_argument("--workload", default="h",
                    help="--profile-loop workload: h, c1..c5 or b64-h128-topk2048 (sparse: pack, packed decode "
                         "and by-index decode per step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="--profile-loop: end with one 1 GiB device-to-device copy (scales the HBM byte counters)")
    ap.add_argument("--configs", action="store_true", help="time the five test configurations and the headline")
    ap.add_argument("--sweep", action="store_true", help="the dense page's 12 configurations and the packed grid")
    ap.add_argument("--sweep-part", choices=("dense", "packed", "both"), default="both")
    ap.add_argument("--reps", type=int, default=100, help="cold repetitions per round (--configs, --sweep)")
    ap.add_argument("--sparse", action="store_true",
                    help="time the sparse FP8 paths instead (pack, patch, packed and by-index decode)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by request; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mla_paged_kv_amd import ops
    from mla_paged_kv_amd import workloads as W

    if args.profile_loop:
        return profile_loop(args)
    if args.sparse:
        return sparse_main(args)
    if args.configs:
        return configs_main(args)
    if args.sweep:
        return sweep_main(args)
    dev = torch.device("cuda:0")
    t0 = time.time()
    w = W.config("h")
    log(f"workload generated in {time.time() - t0:.1f}s")
    case = DenseCase(torch, ops, w, dev, copies=2, num_parts=args.num_parts or None)
    b, s_q, h_q = w.batch, w.s_q, w.h_q
    kv_bytes, flops = w.kv_bytes(), w.flops()
    stream = torch.cuda.current_stream()

    # ---- the first step's output is kept for the parity gate, which runs after
    # the GPU measurements (the oracle keeps the host busy for seconds, and an
    # idle GPU drops its clock)
    case.step(0)
    torch.cuda.synchronize()
    out0, lse0 = case.out.clone(), case.lse.clone()

    # ---- untimed: back-to-back steps for --warm-seconds (the clock ramps up),
    # then the W warmup steps, then per-kernel event times
    n_warm = gpu_warm(torch, case.step, args.warm_seconds)
    for i in range(args.warmup):
        case.step(i)
    kt = kernel_event_times(torch, stream, args.steps,
                            lambda i: [case.c_meta, case.c_dec[i % 2], case.c_comb])
    meta_ms, dec_ms, comb_ms = kt[:, 0], kt[:, 1], kt[:, 2]

    # ---- the timed region: whole steps, then decode + combine only
    reg = timed_region(torch, stream, args.steps, case.step)
    case.c_meta()
    reg_dc = timed_region(torch, stream, args.steps, lambda i: (case.c_dec[i % 2](), case.c_comb()))
    # the decode kernel alone: K launches back to back between two events (its
    # mean launch duration, without the gaps an event between kernels adds)
    reg_dec = timed_region(torch, stream, args.steps, lambda i: case.c_dec[i % 2]())
    ms_per_step = reg["wall_ms_per_step"]

    # ---- the step as a HIP graph (one per pool copy), checked bitwise against
    # the eager step over several replays with eager work in between, then timed
    graph_ms_per_step = None
    if not args.no_graph:
        graphs = []
        for i in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                case.step_unbound(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(2):
            case.step(i)
            torch.cuda.synchronize()
            ref_o, ref_l = case.out.clone(), case.lse.clone()
            for _ in range(3):
                case.out.fill_(0)
                case.lse.fill_(0)
                graphs[i].replay()
                torch.cuda.synchronize()
                if not (torch.equal(case.out, ref_o) and torch.equal(case.lse, ref_l)):
                    raise SystemExit(f"graph replay of pool {i} differs from the eager step")
                case.step(1 - i)  # eager work between replays
                torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % 2].replay()
        reg_g = timed_region(torch, stream, args.steps, lambda i: graphs[i % 2].replay())
        graph_ms_per_step = reg_g["wall_ms_per_step"]

    copy_gbs = copy_bandwidth(torch, dev)
    flags = ops.mla_read_device_errors()
    if flags:
        raise SystemExit(f"device error flags set: {flags}")

    # ---- parity gate + CPU baseline (the oracle on the same workload): raises
    # before anything is printed if the first step's output disagrees
    cpu_baseline = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc

        threads = orc.default_threads()
        sel = list(np.linspace(0, b - 1, args.oracle_requests).astype(int))
        dt, sub = cpu_leg_dense(w, out0, lse0, sel, threads)
        cpu_baseline = {
            "value": round(sub.kv_bytes() / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sel)} of {b} requests (all {h_q} heads, {int(w.seqlens[0])} keys each), fp64, "
                      f"{sub.flops() / dt / 1e9:.2f} GFLOP/s, {dt:.2f} s wall",
            **cpu_info(),
        }
        log(f"oracle: {dt:.2f}s on {threads} threads; parity ok")

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    dec_mean_s = reg_dec["event_span_ms_per_step"] * 1e-3
    achieved = kv_bytes / dec_mean_s / 1e9
    dc_ms = reg_dc["wall_ms_per_step"]
    emit({
        "metric": "achieved KV HBM GB/s (and % of peak) for MLA decode, b=64 h_q=128 sk=4096",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "MLA decode over a paged KV cache: b=64, s_q=1, h_q=128, h_kv=1, d_qk=576, d_v=512, "
                        "sk=4096, 64-token pages, bf16, N(0,1), seed 64",
            "batch": b, "s_q": s_q, "h_q": h_q, "seqlen": int(w.seqlens[0]), "page_tokens": 64,
            "num_parts": case.num_parts, "kv_bytes_per_step": kv_bytes, "flops_per_step": flops,
            "cold_kv": "two pool copies alternate per step",
            "launch": "pre-bound C-ABI calls on one stream (metadata, decode, combine)",
            "untimed_warm": f"{n_warm} steps over {args.warm_seconds} s, then the {args.warmup} warmup steps",
        },
        "timed_region": reg,
        "decode_combine": {**reg_dc, "GBps": round(kv_bytes / (dc_ms * 1e-3) / 1e9, 2),
                           "pct_of_peak_hbm": round(100.0 * kv_bytes / (dc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)},
        "graph_ms_per_step": graph_ms_per_step,
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "copy_bandwidth": {"measured_GBps": copy_gbs, "pct_of_measured_copy": round(100.0 * value / copy_gbs, 2),
                           "method": "1 GiB device-to-device copy, (read + write bytes) / median of 10"},
        "kernels_ms": {
            "decode_back_to_back": round(reg_dec["event_span_ms_per_step"], 5),
            "metadata": round(float(meta_ms.mean()), 5),
            "decode": round(float(dec_ms.mean()), 5),
            "decode_median": round(float(np.median(dec_ms)), 5),
            "decode_min": round(float(dec_ms.min()), 5),
            "combine": round(float(comb_ms.mean()), 5),
            "note": "decode_back_to_back: event span of K decode launches / K (roofline.achieved uses it); "
                    "the others: events between the kernels of each step",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": case.kernel,
            "algorithmic_bytes_per_launch": kv_bytes,
            "mfma_tflops": round(flops / dec_mean_s / 1e12, 2),
            "mfma_frac": round(flops / dec_mean_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_sources_sha256_16": kernel_source_hash(),
        },
        "cpu_baseline": cpu_baseline,
        "context": "FlashMLA SM80 kernel on A100: 632.9 GB/s at b=64 sk=4096 (its h_q is not stated; "
                   "36% of a measured 1747 GB/s copy) -- another machine and likely another head count",
    })


# ----------------------------------------------------------------------------- --profile-loop

def sparse_workload_named(W, name):
    if name == "c5":
        return W.config("c5")
    if name == "b64-h128-topk2048":
        return W.sparse_workload(name, 65, 64, 128, 2048, [2048] * 64, context=8192)
    raise SystemExit(f"unknown sparse workload {name}")


def profile_loop(args):
    """Warmup + K steps of one workload, nothing else on the device but an
    optional calibration copy: the run a profiler wraps."""
    import numpy as np
    import torch

    from mla_paged_kv_amd import ops
    from mla_paged_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.workload in ("h", "c1", "c2", "c3", "c4"):
        case = DenseCase(torch, ops, W.config(args.workload), dev, copies=2 if args.workload == "h" else 1,
                         num_parts=args.num_parts or None)
        step = case.step
        log(f"profile loop {args.workload}: {case.kernel}, {case.num_parts} parts")
    else:
        w = sparse_workload_named(W, args.workload)
        q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        rec = torch.from_numpy(w.kcache_rec).to(dev)
        idx = torch.from_numpy(w.indices).to(dev)
        tl = torch.from_numpy(w.seqlens).to(dev)
        b, s_q, h_q, cap = w.batch, w.s_q, w.h_q, w.topk_capacity
        ws = ops.mla_pack_selected_kv(rec, idx, tl)
        calls = [ops.mla_pack_selected_kv(rec, idx, tl, ws, bind=True)]
        for fmt in (ops.KV_FP8_PACKED, ops.KV_FP8_INDEXED):
            p = ops.DecodePlan(tl, s_q, h_q, fmt, topk_capacity=cap)
            out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
            kv, ix = (ws, None) if fmt == ops.KV_FP8_PACKED else (rec, idx)
            calls += [ops.mla_get_packed_decode_metadata(tl, b, s_q, h_q, cap, p.num_parts, ops.SCHED_AUTO,
                                                         p.sched_meta, p.num_splits, bind=True),
                      ops.mla_decode_fwd(q, kv, fmt, ix, tl, w.scale, False, p.sched_meta, p.num_splits, out, lse,
                                         p.workspace, topk_capacity=cap, bind=True),
                      ops.mla_combine(p.num_splits, p.workspace, b, s_q, h_q, p.num_parts, out, lse, bind=True)]
        step = lambda i: [c() for c in calls]  # noqa: E731
        log(f"profile loop {args.workload}: pack, packed and by-index decode")
    t_warm = time.perf_counter()
    n_warm = 0
    while time.perf_counter() - t_warm < args.warm_seconds:
        step(n_warm)
        n_warm += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    reg = timed_region(torch, stream, args.steps, step)
    log(f"profile loop: {reg}")
    if args.copy_calibration:
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    flags = ops.mla_read_device_errors()
    if flags:
        raise SystemExit(f"device error flags set: {flags}")


# ----------------------------------------------------------------------------- --configs

def _dense_cold_rounds(torch, cases, reps, flush, stream):
    """5 alternating rounds over the cases; per case and round the median of
    `reps` cold repetitions of [metadata, decode, combine].  Returns per case
    an array [rounds, 3] of medians (ms)."""
    import numpy as np

    res = {k: [] for k in cases}
    for rnd in range(ROUNDS):
        for k, c in cases.items():
            for i in range(3):
                c.step(i)
            t = cold_times(torch, stream, reps, [c.c_meta, c.c_dec[0], c.c_comb], flush)
            res[k].append(np.median(t, axis=0))
        log(f"round {rnd + 1}/{ROUNDS} done")
    return {k: np.array(v) for k, v in res.items()}


def _dense_line(name, c, rounds_ms, extra=None):
    w = c.w
    dc = rounds_ms[:, 1] + rounds_ms[:, 2]
    roof_us, bound = c.roof_us()
    dc_med = float(sorted(dc)[len(dc) // 2])
    dec_med = float(sorted(rounds_ms[:, 1])[len(dc) // 2])
    line = {
        "metric": "MLA decode + combine time, cold KV", "case": name, "unit": "us", "higher_is_better": False,
        "config": {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q,
                   "seqlen_total": int(w.seqlens.sum()), "causal": bool(w.causal), "num_parts": c.num_parts,
                   "kernel": c.kernel},
        "decode_combine_us": {k: round(v * 1e3, 2) for k, v in median_range(dc).items()},
        "decode_us": {k: round(v * 1e3, 2) for k, v in median_range(rounds_ms[:, 1]).items()},
        "combine_us": {k: round(v * 1e3, 2) for k, v in median_range(rounds_ms[:, 2]).items()},
        "metadata_us": {k: round(v * 1e3, 2) for k, v in median_range(rounds_ms[:, 0]).items()},
        "kv_bytes": w.kv_bytes(), "flops": w.flops(),
        "kv_GBps": round(w.kv_bytes() / (dc_med * 1e-3) / 1e9, 1),
        "tflops": round(w.flops() / (dc_med * 1e-3) / 1e12, 2),
        "roofline": {"bound": bound, "t_roof_us": round(roof_us, 3),
                     "frac_decode_combine": round(roof_us / (dc_med * 1e3), 4),
                     "frac_decode_kernel": round(roof_us / (dec_med * 1e3), 4)},
        "method": f"{ROUNDS} alternating rounds x median of cold repetitions ({FLUSH_BYTES >> 20} MiB read "
                  "before each); median and [min, max] of the round medians",
    }
    if extra:
        line.update(extra)
    return line


def configs_main(args):
    import numpy as np
    import torch

    from mla_paged_kv_amd import ops
    from mla_paged_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = Flusher(torch, dev)
    names = ("c1", "c2", "c3", "c4", "h")
    cases = {}
    for n in names:
        cases[n] = DenseCase(torch, ops, W.config(n), dev)
        log(f"{n}: {cases[n].kernel}, {cases[n].num_parts} parts")
    gpu_warm(torch, cases["h"].step, args.warm_seconds)
    copy_gbs = copy_bandwidth(torch, dev)
    rounds = _dense_cold_rounds(torch, cases, args.reps, flush, stream)
    # hot too: repetitions back to back, inputs left in the caches by the previous one
    hot = {n: kernel_event_times(torch, stream, args.reps, lambda i, c=c: [c.c_meta, c.c_dec[0], c.c_comb])
           for n, c in cases.items()}
    cpu = {}
    if not args.no_cpu_baseline:
        from oracle import oracle as orc

        threads = orc.default_threads()
        for n in names:
            w = cases[n].w
            sel = list(range(w.batch))
            dt, _ = cpu_leg_dense(w, cases[n].out, cases[n].lse, sel, threads, reps=3)
            cpu[n] = {"threads": threads, "median_s": round(dt, 4), "kv_GBps": round(w.kv_bytes() / dt / 1e9, 4),
                      "GFLOPs": round(w.flops() / dt / 1e9, 2)}
            if n in ("c1", "c2"):
                dt1, _ = cpu_leg_dense(w, cases[n].out, cases[n].lse, sel, 1, reps=3, gate=False)
                cpu[n]["one_thread"] = {"median_s": round(dt1, 4), "kv_GBps": round(w.kv_bytes() / dt1 / 1e9, 4),
                                        "GFLOPs": round(w.flops() / dt1 / 1e9, 2)}
            log(f"oracle {n}: {cpu[n]}")
    for n in names:
        c = cases[n]
        extra = {"pct_of_measured_copy": None, "measured_copy_GBps": copy_gbs}
        dc_med = float(np.median(rounds[n][:, 1] + rounds[n][:, 2]))
        extra["pct_of_measured_copy"] = round(100.0 * c.w.kv_bytes() / (dc_med * 1e-3) / 1e9 / copy_gbs, 2)
        h = hot[n][:, 1] + hot[n][:, 2]
        extra["hot_decode_combine_us"] = {k: round(v * 1e3, 2) for k, v in median_range(h).items()}
        extra["hot_decode_us"] = round(float(np.median(hot[n][:, 1])) * 1e3, 2)
        extra["hot_metadata_us"] = round(float(np.median(hot[n][:, 0])) * 1e3, 2)
        if n in cpu:
            extra["oracle"] = {**cpu[n], **cpu_info()}
        emit(_dense_line(n, c, rounds[n], extra))
    # C5: the sparse FP8 configuration (pack + packed decode, and by index)
    emit(_sparse_case_line(torch, ops, W.config("c5"), dev, stream, flush, args.reps, copy_gbs,
                           oracle=not args.no_cpu_baseline))
    flags = ops.mla_read_device_errors()
    if flags:
        raise SystemExit(f"device error flags set: {flags}")


# ----------------------------------------------------------------------------- --sweep

def _sparse_case_line(torch, ops, w, dev, stream, flush, reps, copy_gbs, oracle=True):
    """One sparse workload, cold: pack, packed decode + combine, by-index decode
    + combine (each with its metadata), checked first (by index bitwise equal to
    pack + packed; request 0 against the oracle)."""
    import numpy as np

    q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    rec = torch.from_numpy(w.kcache_rec).to(dev)
    idx = torch.from_numpy(w.indices).to(dev)
    tl = torch.from_numpy(w.seqlens).to(dev)
    b, s_q, h_q, cap = w.batch, w.s_q, w.h_q, w.topk_capacity
    ws = torch.empty((ops.mla_packed_kv_workspace_size(b, s_q, cap),), dtype=torch.uint8, device=dev)
    calls, outs = {}, {}
    for fmt, key in ((ops.KV_FP8_PACKED, "packed"), (ops.KV_FP8_INDEXED, "by_index")):
        parts = ops.mla_decode_num_parts(b, s_q, h_q, 1, fmt)
        meta = torch.empty((parts, 8), dtype=torch.int32, device=dev)
        ns = torch.empty((b + 1,), dtype=torch.int32, device=dev)
        pws = torch.empty((ops.mla_decode_workspace_size(b, s_q, h_q, parts),), dtype=torch.uint8, device=dev)
        out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
        kv, ix = (ws, None) if fmt == ops.KV_FP8_PACKED else (rec, idx)
        calls[key] = [ops.mla_get_packed_decode_metadata(tl, b, s_q, h_q, cap, parts, ops.SCHED_AUTO, meta, ns,
                                                         bind=True),
                      ops.mla_decode_fwd(q, kv, fmt, ix, tl, w.scale, False, meta, ns, out, lse, pws,
                                         topk_capacity=cap, bind=True),
                      ops.mla_combine(ns, pws, b, s_q, h_q, parts, out, lse, bind=True)]
        outs[key] = (out, lse, parts)
    pack = ops.mla_pack_selected_kv(rec, idx, tl, ws, bind=True)
    pack()
    for key in calls:
        for c in calls[key]:
            c()
    torch.cuda.synchronize()
    if not (torch.equal(outs["packed"][0], outs["by_index"][0]) and torch.equal(outs["packed"][1],
                                                                                    outs["by_index"][1])):
        raise SystemExit(f"{w.name}: by-index decode differs from pack + packed decode")
    line = {"metric": "sparse FP8 MLA decode time, cold", "case": w.name, "unit": "us", "higher_is_better": False,
            "config": {"workload": w.name, "batch": b, "s_q": s_q, "h_q": h_q, "topk_capacity": cap,
                       "topk_total": int(w.seqlens.sum()), "kernel_packed": ops.mla_decode_kernel_name(
                           s_q, h_q, 1, ops.KV_FP8_PACKED)}}
    if oracle:
        from oracle import oracle as orc
        from tests import gpu_helpers as G

        G.say = log
        sub = G.sub_workload(w, [0])
        t0 = time.perf_counter()
        ref = orc.mla_sparse_decode(sub.q_bits, w.kcache_rec, sub.indices, sub.seqlens, w.scale,
                                    nthreads=orc.default_threads())
        dt = time.perf_counter() - t0
        o, l = outs["packed"][0][:1], outs["packed"][1][:1]
        G.compare(f"{w.name}-request0", o, l, ref[0], ref[1])
        line["oracle_request0"] = {"s": round(dt, 4), "threads": orc.default_threads()}
    sel_bytes = int(w.seqlens.sum()) * s_q * ops.REC_BYTES
    flops = 2 * (576 + 512) * int(w.seqlens.sum()) * s_q * h_q
    t_pack = cold_times(torch, stream, reps, [pack], flush)[:, 0]
    res = {"pack_us": {k: round(v * 1e3, 2) for k, v in median_range(t_pack).items()},
           "pack_bytes_moved": 2 * sel_bytes}
    for key in calls:
        t = cold_times(torch, stream, reps, calls[key], flush)
        dc = t[:, 1] + t[:, 2]
        med = float(np.median(dc))
        t_roof = max(sel_bytes / (PEAK_HBM_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))
        th = kernel_event_times(torch, stream, reps, lambda i, cs=calls[key]: cs)
        res[key] = {"metadata_us": round(float(np.median(t[:, 0])) * 1e3, 2),
                    "hot_decode_combine_us": round(float(np.median(th[:, 1] + th[:, 2])) * 1e3, 2),
                    "decode_us": {k: round(v * 1e3, 2) for k, v in median_range(t[:, 1]).items()},
                    "decode_combine_us": {k: round(v * 1e3, 2) for k, v in median_range(dc).items()},
                    "num_parts": outs[key][2],
                    "selected_GBps": round(sel_bytes / (med * 1e-3) / 1e9, 1),
                    "tflops": round(flops / (med * 1e-3) / 1e12, 2),
                    "roofline": {"bound": "hbm" if sel_bytes / (PEAK_HBM_GBS * 1e9) >= flops / (
                        PEAK_BF16_TFLOPS * 1e12) else "mfma", "t_roof_us": round(t_roof * 1e6, 3),
                                 "frac_decode_combine": round(t_roof / (med * 1e-3), 4),
                                 "frac_decode_kernel": round(t_roof / (float(np.median(t[:, 1])) * 1e-3), 4)}}
    res["pack_then_packed_us"] = round(float(np.median(t_pack)) * 1e3 + res["packed"]["decode_combine_us"][
        "median"], 2)
    line.update(res)
    line["selected_bytes"] = sel_bytes
    line["flops"] = flops
    line["measured_copy_GBps"] = copy_gbs
    line["method"] = f"median and [min, max] of {reps} cold repetitions ({FLUSH_BYTES >> 20} MiB read before each)"
    return line


def sweep_main(args):
    import numpy as np
    import torch

    from mla_paged_kv_amd import ops
    from mla_paged_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = Flusher(torch, dev)
    gpu_warm(torch, lambda i: flush(), args.warm_seconds)
    copy_gbs = copy_bandwidth(torch, dev)
    log(f"measured copy bandwidth {copy_gbs} GB/s")
    if args.sweep_part in ("dense", "both"):
        cases = {}
        for (b, sk, h) in DENSE_PAGE_CONFIGS:
            name = f"b{b}-h{h}-sk{sk}"
            pool = max(b * sk // 64, 16)  # every page used once, shuffled; cold through the flush
            w = W.dense_workload(name, 1000 + len(cases), b, 1, h, [sk] * b, pool_pages=pool)
            cases[name] = DenseCase(torch, ops, w, dev)
            if not args.no_cpu_baseline:
                # request 0 against the oracle (the GPU tests cover the rest)
                cases[name].step(0)
                torch.cuda.synchronize()
                from oracle import oracle as orc

                cpu_leg_dense(w, cases[name].out, cases[name].lse, [0], orc.default_threads())
            log(f"{name}: {cases[name].kernel}, {cases[name].num_parts} parts")
        gpu_warm(torch, next(iter(cases.values())).step, args.warm_seconds)
        rounds = _dense_cold_rounds(torch, cases, args.reps, flush, stream)
        for name, c in cases.items():
            dc_med = float(np.median(rounds[name][:, 1] + rounds[name][:, 2]))
            emit(_dense_line(name, c, rounds[name], {
                "source": "dense page, Performance table", "measured_copy_GBps": copy_gbs,
                "pct_of_measured_copy": round(100.0 * c.w.kv_bytes() / (dc_med * 1e-3) / 1e9 / copy_gbs, 2)}))
        del cases
        torch.cuda.empty_cache()
    if args.sweep_part in ("packed", "both"):
        gpu_warm(torch, lambda i: flush(), args.warm_seconds)
        k = 0
        for h in PACKED_GRID_H:
            for b in PACKED_GRID_B:
                for s_q in PACKED_GRID_SQ:
                    w = W.sparse_workload(f"packed-B{b}-Sq{s_q}-H{h}", 2000 + k, b, h, 2048, [2048] * b,
                                          context=8192, s_q=s_q)
                    k += 1
                    line = _sparse_case_line(torch, ops, w, dev, stream, flush, args.reps, copy_gbs,
                                             oracle=not args.no_cpu_baseline and s_q * h <= 512)
                    line["source"] = "packed page, L20X grid"
                    emit(line)
                    torch.cuda.empty_cache()
    flags = ops.mla_read_device_errors()
    if flags:
        raise SystemExit(f"device error flags set: {flags}")


# ----------------------------------------------------------------------------- --sparse

def sparse_main(args):
    """Sparse FP8 decode step on two workloads, three ways, each captured as a HIP
    graph: the decode that gathers by id; pack + packed decode (pack not
    hidden); patch + packed decode (pack hidden in an earlier overlap window,
    only the current-token patch on the critical path).  Every path is checked
    against the oracle first.  Prints one JSON line."""
    import numpy as np
    import torch

    from mla_paged_kv_amd import ops
    from mla_paged_kv_amd import workloads as W
    from oracle import oracle as orc
    from tests import gpu_helpers as G

    G.say = log  # parity lines go to stderr: stdout carries the one JSON line
    dev = torch.device("cuda:0")
    cases = [("c5", W.config("c5")),
             ("b64-h128-topk2048", W.sparse_workload("b64-h128-topk2048", 65, 64, 128, 2048, [2048] * 64,
                                                     context=8192))]
    results = {}
    for name, w in cases:
        t = G.dev_tensors(w)
        b, s_q, h_q, cap = w.batch, w.s_q, w.h_q, w.topk_capacity
        sel_bytes = int(w.seqlens.sum()) * s_q * ops.REC_BYTES
        ws = torch.empty((ops.mla_packed_kv_workspace_size(b, s_q, cap),), dtype=torch.uint8, device=dev)
        ids = t["indices"][:, 0, :1].contiguous()  # one selected current token per request
        out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=dev)
        plans = {f: ops.DecodePlan(t["seqlens"], s_q, h_q, f, topk_capacity=cap)
                 for f in (ops.KV_FP8_INDEXED, ops.KV_FP8_PACKED)}

        def decode(fmt, policy=None):
            p = plans[fmt]
            ops.mla_get_packed_decode_metadata(t["seqlens"], b, s_q, h_q, cap, p.num_parts,
                                               ops.SCHED_AUTO if policy is None else policy, p.sched_meta,
                                               p.num_splits)
            kv, ix = (t["kcache_rec"], t["indices"]) if fmt == ops.KV_FP8_INDEXED else (ws, None)
            ops.mla_decode_fwd(t["q"], kv, fmt, ix, t["seqlens"], w.scale, False, p.sched_meta, p.num_splits, out,
                               lse, p.workspace, topk_capacity=cap)
            ops.mla_combine(p.num_splits, p.workspace, b, s_q, h_q, p.num_parts, out, lse)

        steps = {
            "by_index": lambda: decode(ops.KV_FP8_INDEXED),
            "pack_then_packed": lambda: (ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"], ws),
                                         decode(ops.KV_FP8_PACKED)),
            "patch_then_packed": lambda: (ops.mla_patch_packed_kv(t["kcache_rec"], t["indices"], t["seqlens"], ids,
                                                                  ws),
                                          decode(ops.KV_FP8_PACKED)),
            "by_index_request_local_sched": lambda: decode(ops.KV_FP8_INDEXED, ops.SCHED_REQUEST_LOCAL),
        }
        ref_o, ref_l = orc.mla_sparse_decode(w.q_bits, w.kcache_rec, w.indices, w.seqlens, w.scale,
                                             nthreads=orc.default_threads())
        ops.mla_pack_selected_kv(t["kcache_rec"], t["indices"], t["seqlens"], ws)
        row = {"batch": b, "h_q": h_q, "s_q": s_q, "topk_capacity": cap, "selected_bytes": sel_bytes}
        for key, fn in steps.items():
            fn()
            torch.cuda.synchronize()
            G.compare(f"{name}-{key}", out, lse, ref_o, ref_l)  # raises on a mismatch
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / args.steps
            G.compare(f"{name}-{key}-graph", out, lse, ref_o, ref_l)
            row[key + "_us"] = round(us, 2)
            row[key + "_selected_GBps"] = round(sel_bytes / (us * 1e-6) / 1e9, 1)
        results[name] = row
        log(f"{name}: {row}")
    flags = ops.mla_read_device_errors()
    if flags:
        raise SystemExit(f"device error flags set: {flags}")
    emit({
        "metric": "sparse FP8 MLA decode step time (metadata, [pack or patch], decode, combine)",
        "unit": "us", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "fp8 e4m3 records, bf16 MFMA", "data": "synthetic",
        "launch": "one HIP graph per path", "workloads": results,
    })


if __name__ == "__main__":
    main()
