"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-parity]

A step is one attn_fwd call over the whole workload (default: causal
grouped-query bf16, B=1 Hq=32 Hkv=8 S=8192 D=128) with the inputs already
resident in HBM.  K steps are timed with HIP events recorded on the stream the
kernel is launched on.  Prints one JSON line:

  value     effective TFLOP/s = unmasked FLOPs (4*D per visible (query, key)
            pair per query head) / time per step
  roofline  matrix-core bound (vector-ALU bound for fp32 workloads):
            achieved TFLOP/s of the attention kernel (its
            algorithmic FLOPs per launch / its average launch duration, which
            is the event-timed time per step: a step is exactly one launch of
            that kernel; the committed rocprofv3 kernel trace of the same
            command gives the same average) vs the MI355X dense bf16 peak;
            traffic = HBM bytes per launch from the committed rocprofv3 counter
            summary, or null when the kernel source changed since the counters
            were taken
  clock     the graphics clock sampled with amd-smi while the untimed steps
            run, and the same throughput as a percentage of CUs x 4096 FLOP
            x that clock (the dense peak at the clock the chip actually holds)
  inputs_sha256  SHA-256 of the bytes of q, k and v as uploaded
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload,
            timed on the host's cores (cores = the BLAS threads it ran on,
            host_cpu_count = os.cpu_count())

  parity    max abs error of the GPU output against the oracle's on that
            same sample (the oracle runs nowhere else in this script)

A decode workload (--workload decode_...) times one attn_decode call (its
split-merge kernel included) and reports achieved HBM bandwidth instead:
value = algorithmic bytes (the valid cache entries, q and o, each once) /
time per step, against the 8 TB/s HBM peak.

A workload with separate query and key lengths (--workload chunk_prefill_...
or cross_...) times one attn_fwd_ex call on its layout and reports effective
TFLOP/s as the default does.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP32_TFLOPS = 157.3   # vector fp32
PEAK_FP8_TFLOPS = 5033.2   # 256 CU x 2.4 GHz x 8192 dense FP8 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = ("kernel_bf16.hip", "gfx950_ops.h", "attn_kernels.h", "attn_sched.h")
DECODE_SOURCES = ("kernel_decode.hip", "gfx950_ops.h", "attn_decode.h", "attn_sched.h")
# committed HBM-traffic summaries per workload, with the sources their kernel is built from
TRAFFIC_SUMMARIES = {
    "causal_gqa_bf16_s8192": ("attn_fwd_bf16_causal_gqa_s8192_hbm_traffic.md", KERNEL_SOURCES),
    "local_global_bf16_s8192": ("attn_fwd_bf16_local_global_s8192.md", KERNEL_SOURCES),
    "causal_gqa_fp8_s8192": ("attn_fwd_fp8_causal_gqa_s8192.md",
                             ("kernel_fp8.hip", "gfx950_ops.h", "attn_kernels.h", "attn_sched.h")),
    "causal_mha_fp8_d64_s8192": ("attn_fwd_fp8_causal_mha_d64_s8192.md",
                                 ("kernel_fp8.hip", "gfx950_ops.h", "attn_kernels.h", "attn_sched.h")),
    "local_global_fp8_s8192": ("attn_fwd_fp8_local_global_s8192.md",
                               ("kernel_fp8.hip", "gfx950_ops.h", "attn_kernels.h", "attn_sched.h")),
    "decode_gqa_bf16_b16_l8192": ("attn_decode_bf16_gqa_b16_l8192.md", DECODE_SOURCES),
    "decode_gqa_bf16_b8_sq4_l16384": ("attn_decode_bf16_ragged_b8_sq4_l16384.md", DECODE_SOURCES),
    "decode_window_gqa_bf16_b16_w4096_l32768": ("attn_decode_bf16_window_b16_w4096_l32768.md",
                                                DECODE_SOURCES),
    "decode_mqa_bf16_b4_l65536": ("attn_decode_bf16_mqa_b4_l65536.md", DECODE_SOURCES),
}


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "transformer_attention_attn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary of this
    workload, if it was taken on the current kernel source."""
    if workload not in TRAFFIC_SUMMARIES:
        return None
    fname, sources = TRAFFIC_SUMMARIES[workload]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    txt = open(path, encoding="utf-8").read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    m_wl = re.search(r"workload:\s*(\S+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_hash and m_wl and m_b):
        return None
    if m_hash.group(1) != kernel_source_hash(sources) or m_wl.group(1) != workload:
        return None
    return float(m_b.group(1))


def host_threads() -> int:
    """Threads the host BLAS pool runs the oracle's NumPy products on."""
    try:
        from threadpoolctl import threadpool_info

        return int(max((x.get("num_threads", 1) for x in threadpool_info()), default=1))
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def max_abs_err(got, ref) -> float:
    import numpy as np

    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)))


def cpu_baseline(w, inputs, n_heads: int, seconds: float):
    """Time the oracle on batch 0 (all rows), one key/value head's query heads
    at a time, up to n_heads query heads or until `seconds` have passed.
    Returns (summary, oracle output [1, heads done, S, D])."""
    import numpy as np

    import oracle

    threads = host_threads()
    G = w.Hq // w.Hkv
    n_heads = min(n_heads, w.Hq)
    refs = []
    t0 = time.perf_counter()
    while sum(r.shape[1] for r in refs) < n_heads and time.perf_counter() - t0 < seconds:
        h = len(refs)  # key/value head; its query heads h*G .. h*G + G - 1 keep the head map
        refs.append(oracle.attention(inputs["q"][:1, h * G:(h + 1) * G], inputs["k"][:1, h:h + 1],
                                     inputs["v"][:1, h:h + 1], w.mask, w.window, w.global_idx,
                                     scale=w.scale))
    dt = time.perf_counter() - t0
    ref = np.concatenate(refs, axis=1)
    done = ref.shape[1]
    flops = oracle.effective_flops(1, done, w.S, w.D, w.mask, w.window, w.global_idx)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cpu_count": os.cpu_count(),
        "kind": "oracle",
        "sample": f"batch 0, query heads 0..{done - 1} of {w.Hq}, all {w.S} rows "
                  f"({flops:.3e} effective FLOPs in {dt:.2f} s, fp64 NumPy)",
        "seconds": dt,
    }, ref


def inputs_sha256(*tensors) -> dict:
    """SHA-256 of each tensor's bytes (q, k, v as uploaded)."""
    import torch

    out = {}
    for name, t in zip(("q", "k", "v"), tensors):
        b = t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()
        out[name] = hashlib.sha256(b).hexdigest()
    return out


class ClockSampler:
    """Samples the graphics clock with amd-smi in a background thread while
    the GPU is busy: up to `n` samples, each the mean over the XCDs of one
    amd-smi call; a sample with any XCD in deep sleep (a momentary gap
    between launches) is dropped.  result(): the median of the kept samples
    in MHz, or None where the tool or its output is unavailable."""

    def __init__(self, n: int = 6):
        import threading

        self.n = n
        self.mhz = []
        self.dropped = 0
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _gfx_clocks(node, found):
        if isinstance(node, dict):
            for key, val in node.items():
                if isinstance(key, str) and key.lower().startswith("gfx") and isinstance(val, dict):
                    clk = val.get("clk")
                    if isinstance(clk, dict) and isinstance(clk.get("value"), (int, float)):
                        found.append((float(clk["value"]), str(val.get("deep_sleep", "")).upper()))
                ClockSampler._gfx_clocks(val, found)
        elif isinstance(node, list):
            for x in node:
                ClockSampler._gfx_clocks(x, found)

    def _run(self):
        import subprocess

        for _ in range(self.n):
            if self._stop.is_set():
                break
            try:
                res = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"],
                                     capture_output=True, text=True, timeout=10)
                found = []
                self._gfx_clocks(json.loads(res.stdout), found)
            except Exception:  # noqa: BLE001 - the clock is an optional extra
                return
            if not found:
                return
            if any(ds == "ENABLED" for _, ds in found):
                self.dropped += 1
            else:
                self.mhz.append(sum(v for v, _ in found) / len(found))
            time.sleep(0.05)

    def start(self):
        self._thread.start()

    def alive(self):
        return self._thread.is_alive()

    def result(self):
        self._stop.set()
        self._thread.join(timeout=15)
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return v[len(v) // 2]


def calibration_copy(mib: int, dev):
    """One plain elementwise copy of `mib` MiB (fp32 in, fp32 out) whose HBM counters
    scale the attention kernels' (a fill kernel runs first to create the source)."""
    if mib <= 0:
        return
    import torch

    n = mib << 18  # fp32 elements
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)  # reads and writes exactly n * 4 bytes
    torch.cuda.synchronize()
    print(f"bench: calibration copy of {n * 4} bytes done", file=sys.stderr, flush=True)
    del src, dst


def decode_cpu_baseline(w, inputs, lens, n_seq: int = 1):
    """Time the decode oracle on the first n_seq sequences (all heads and rows).
    Returns (summary, oracle output [n_seq, Hq, Sq, D])."""
    import oracle

    threads = host_threads()
    n = min(n_seq, w.B)
    sub = [int(x) for x in lens[:n]]
    t0 = time.perf_counter()
    ref = oracle.decode_attention(inputs["q"][:n], inputs["k"][:n], inputs["v"][:n], w.mask,
                                  cache_len=sub, scale=w.scale, window=w.window)
    dt = time.perf_counter() - t0
    nbytes = decode_counts(w, sub)[0]
    return {
        "value": nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "host_cpu_count": os.cpu_count(),
        "kind": "oracle",
        "sample": f"sequences 0..{n - 1} of {w.B}, all {w.Hq} heads and {w.Sq} new positions "
                  f"({nbytes} cache bytes in {dt:.2f} s, fp64 NumPy)",
        "seconds": dt,
    }, ref


def decode_counts(w, lens):
    """(cache bytes read, effective FLOPs) of one decode call over the given
    sequence lengths: 2 * Hkv * D * 2 bytes per cached position some new query
    sees (under a window of w, the last min(L, w + Sq - 1) of a sequence); 4 * D
    FLOPs per visible (query row, position) pair and query head."""
    import numpy as np

    L = np.asarray([int(x) for x in lens], dtype=np.int64)
    read = np.minimum(L, w.window + w.Sq - 1) if w.mask == "causal_window" else L
    cache_bytes = int(2 * w.Hkv * w.D * 2 * read.sum())
    if w.mask == "full":
        pairs = int(w.Sq * L.sum())
    else:  # new position i of Sq sits at p = L - Sq + i and sees positions .. p
        i = np.arange(w.Sq, dtype=np.int64)
        p = L[:, None] - w.Sq + i[None, :]
        hi = np.clip(p + 1, 0, L[:, None])
        lo = np.clip(p - w.window + 1, 0, None) if w.mask == "causal_window" else 0
        pairs = int(np.maximum(hi - lo, 0).sum())
    return cache_bytes, 4 * w.D * pairs * w.Hq


def ex_visible_pairs(Sq, Skv, mask, window=0, global_idx=()) -> int:
    """Visible (query, key) pairs of one query head of one sequence of an
    attn_fwd_ex call: query i sits at key position p = i + Skv - Sq."""
    import numpy as np

    if mask == "full":
        return Sq * Skv
    p = np.arange(Sq, dtype=np.int64) + (Skv - Sq)
    if mask == "local_global":
        # the band |p - j| <= w, the global keys outside it, and every key for
        # a global query
        g = np.array(sorted({int(x) for x in global_idx if 0 <= int(x) < Skv}), dtype=np.int64)
        band = np.maximum(np.minimum(p + window, Skv - 1) - np.maximum(p - window, 0) + 1, 0)
        outside = (np.abs(p[:, None] - g[None, :]) > window).sum(axis=1) if g.size else 0
        n = band + outside
        if g.size:
            n = np.where(np.isin(p, g), Skv, n)
        return int(n.sum())
    hi = np.clip(p + 1, 0, Skv)
    lo = np.zeros_like(hi) if mask == "causal" else np.clip(p - window + 1, 0, Skv)
    return int(np.maximum(hi - lo, 0).sum())


def layout_pairs(words, S, causal, block=64) -> int:
    """Visible (query, key) pairs of one head under a block-sparse layout
    (uint32 bitmask rows over blocks of `block` positions)."""
    import numpy as np

    nb = -(-S // block)
    bits = np.unpackbits(np.ascontiguousarray(words, dtype="<u4").view(np.uint8),
                         bitorder="little").reshape(nb, -1)[:, :nb].astype(bool)
    start = np.arange(nb) * block
    width = np.minimum(start + block, S) - start       # keys of each block
    total = 0
    for I in range(nb):
        rows = np.arange(start[I], start[I] + width[I])
        J = np.nonzero(bits[I])[0]
        if causal:  # keys j <= i of each visible block, for every row i of block I
            total += int(np.clip(rows[:, None] - start[J][None, :] + 1, 0, width[J][None, :]).sum())
        else:
            total += int(width[J].sum()) * len(rows)
    return total


def ex_layout_words(w):
    """The workload's block-sparse layout from the library's builders, or None."""
    import transformer_attention_attn_amd as attn

    nb = w.n_blocks()
    if w.pattern == "strided":
        return attn.layout_strided(nb, *w.pattern_args)
    if w.pattern == "fixed":
        return attn.layout_fixed(nb, *w.pattern_args)
    if w.pattern == "bigbird":
        radius, g, _ = w.pattern_args
        return attn.layout_bigbird(nb, radius, g, w.rand_blocks())
    return None


def ex_effective_flops(w, batches=None) -> float:
    """4 * D FLOPs per visible pair and query head, summed over the sequences
    (each with its own valid lengths when the workload is padded)."""
    if w.pattern:
        nbat = w.B if batches is None else len(list(batches))
        return 4.0 * w.D * layout_pairs(ex_layout_words(w), w.Sq, w.mask == "causal") * w.Hq * nbat
    q_len, kv_len = w.lengths_qkv()
    total = 0
    for b in (range(w.B) if batches is None else batches):
        sq = w.Sq if q_len is None else int(q_len[b])
        skv = w.Skv if kv_len is None else int(kv_len[b])
        total += ex_visible_pairs(sq, skv, w.mask, w.window, w.global_idx)
    return 4.0 * w.D * total * w.Hq


def ex_cpu_baseline(w, inputs, seconds: float = 10.0):
    """Time the oracle head by head on batch 0 (all rows of each head) until
    `seconds` have passed.  Returns (summary, heads done, their oracle output)."""
    import numpy as np

    import oracle

    threads = host_threads()
    G = w.Hq // w.Hkv
    slopes = w.alibi_slopes()
    table = w.distance_bias()
    q_len, kv_len = w.lengths_qkv()
    lay = None
    if w.pattern:  # the oracle's own layout of the pattern
        nb = w.n_blocks()
        lay = (oracle.strided_layout(nb, *w.pattern_args) if w.pattern == "strided" else
               oracle.fixed_layout(nb, *w.pattern_args) if w.pattern == "fixed" else
               oracle.bigbird_layout(nb, w.pattern_args[0], w.pattern_args[1], w.rand_blocks()))
    refs = []
    t0 = time.perf_counter()
    while len(refs) < w.Hq and time.perf_counter() - t0 < seconds:
        a = len(refs)
        h = a // G
        if lay is not None:
            refs.append(oracle.block_sparse_attention(
                inputs["q"][:1, a:a + 1], inputs["k"][:1, h:h + 1], inputs["v"][:1, h:h + 1],
                lay, 64, w.mask == "causal", scale=w.scale))
            continue
        refs.append(oracle.cross_attention(
            inputs["q"][:1, a:a + 1], inputs["k"][:1, h:h + 1], inputs["v"][:1, h:h + 1],
            w.mask, w.window, scale=w.scale,
            alibi_slopes=None if slopes is None else slopes[a:a + 1].astype(np.float64),
            q_len=None if q_len is None else q_len[:1],
            kv_len=None if kv_len is None else kv_len[:1], global_idx=w.global_idx,
            dist_bias=None if table is None else table[a:a + 1]))
    dt = time.perf_counter() - t0
    n = len(refs)
    flops = ex_effective_flops(w, batches=[0]) / w.Hq * n
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cpu_count": os.cpu_count(),
        "kind": "oracle",
        "sample": f"batch 0, query heads 0..{n - 1} of {w.Hq} (as many as about {seconds:.0f} s "
                  f"allows), all {w.Sq} rows ({flops:.3e} effective FLOPs in {dt:.2f} s, "
                  f"fp64 NumPy)",
        "seconds": dt,
    }, n, np.concatenate(refs, axis=1)


def time_steps(step, stream, args):
    """Untimed warm-up (about `args.prewarm` seconds of steps, as the GPU clocks
    ramp up over the first ~100 ms of load, then `args.warmup` steps), then
    `args.steps` back-to-back steps with a HIP event recorded on the launch
    stream before each step and after the last.  Returns (mean ms per step over
    the whole timed region, prewarm steps, {"median_ms", "min_ms"} of the
    single steps)."""
    import torch

    t_warm = time.perf_counter()
    prewarm_steps = 0
    # the clock sample runs while the steps keep the GPU busy (the untimed
    # phase is extended until it has finished, by at most 15 s)
    sampler = ClockSampler() if getattr(args, "clock", False) else None
    started = False
    while True:
        el = time.perf_counter() - t_warm
        waiting = started and sampler.alive()
        if (el >= args.prewarm and not waiting) or el > args.prewarm + 15:
            break
        for _ in range(20):
            step()
        prewarm_steps += 20
        torch.cuda.synchronize()
        if sampler is not None and not started and el > 0.3:
            sampler.start()
            started = True
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    spread = {"median_ms": round(per[len(per) // 2], 6), "min_ms": round(per[0], 6)}
    if started:
        args.clock_mhz = sampler.result()
        args.clock_samples = {"kept": len(sampler.mhz), "dropped_deep_sleep": sampler.dropped}
    return ev[0].elapsed_time(ev[-1]) / args.steps, prewarm_steps, spread


def time_cold(step, stream, n: int, dev, mib: int = 512):
    """Cold-cache timing: before each of n steps, write a `mib` MiB scratch
    buffer on the same stream (evicting the caches), then time the step alone
    between two HIP events.  Returns {"median_ms", "min_ms", "steps", "flush_mib"}."""
    import torch

    scratch = torch.empty(mib << 18, dtype=torch.float32, device=dev)
    per = []
    for i in range(n):
        scratch.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b))
    del scratch
    per.sort()
    return {"median_ms": round(per[len(per) // 2], 6), "min_ms": round(per[0], 6), "steps": n,
            "flush_mib": mib}


def bench_decode(args, name):
    import numpy as np
    import torch

    import transformer_attention_attn_amd as attn
    import workloads

    w = workloads.DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"bench: decode workload {name} {w.describe()}", file=sys.stderr, flush=True)
    inputs = workloads.decode_workload_inputs(w)
    q, k, v = (torch.from_numpy(inputs[n + "_bits"].view(np.int16)).view(torch.bfloat16)
               .to(dev).contiguous() for n in ("q", "k", "v"))
    lens = w.cache_len()
    cl = torch.from_numpy(lens).to(dev)
    out = torch.empty_like(q)
    ws_n = attn.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Smax, w.D, w.mask, w.window)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    calibration_copy(args.calibrate_copy_mib, dev)

    def step():
        attn.decode(q, k, v, cache_len=cl, mask=w.mask, scale=w.scale, out=out, workspace=ws,
                    stream=stream, window=w.window)

    ms, prewarm_steps, spread = time_steps(step, stream, args)
    cache_bytes, flops = decode_counts(w, lens)
    qo_bytes = 2 * w.B * w.Hq * w.Sq * w.D * 2
    alg = cache_bytes + qo_bytes
    gbs = alg / (ms * 1e-3) / 1e9
    print(f"bench: {ms * 1e3:.1f} us/step, {gbs:.1f} GB/s algorithmic", file=sys.stderr,
          flush=True)
    result = {
        "metric": "decode attention achieved HBM GB/s (algorithmic bytes) + % of 8 TB/s, 1 GPU",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Smax": w.Smax, "D": w.D, "mask": w.mask, "lengths": w.lengths,
                   "algorithmic_bytes": alg, "effective_flops": flops,
                   "workspace_bytes": ws_n, "parallelism": "none"},
        "pct_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": committed_traffic(name),
        },
        "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "prewarm_steps": prewarm_steps,
        "step_spread": spread,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = decode_cpu_baseline(w, inputs, lens)
        if not args.no_parity:
            got = out[:ref.shape[0]].float().cpu().numpy()
            result["parity"] = {"sample": "the cpu_baseline sample",
                                "max_abs_err": max_abs_err(got, ref)}
    print(json.dumps(result), flush=True)
    return 0


def bench_ex(args, name):
    import numpy as np
    import torch

    import transformer_attention_attn_amd as attn
    import workloads

    w = workloads.EX_WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"bench: workload {name} {w.describe()}", file=sys.stderr, flush=True)
    inputs = workloads.ex_workload_inputs(w)

    def place(bits):
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        if w.layout == "bshd":  # [B][S][H][D] in memory, viewed as [B][H][S][D]
            return t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
        return t.to(dev).contiguous()

    q, k, v = (place(inputs[n + "_bits"]) for n in ("q", "k", "v"))
    slopes = w.alibi_slopes()
    q_len, kv_len = w.lengths_qkv()
    slopes_d, q_len_d, kv_len_d, bias_d = (None if x is None else torch.from_numpy(x).to(dev)
                                           for x in (slopes, q_len, kv_len, w.distance_bias()))
    words = ex_layout_words(w)
    layout_d = None if words is None else torch.from_numpy(words.view(np.int32)).to(dev)
    if w.layout == "bshd":
        out = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16,
                          device=dev).transpose(1, 2)
    else:
        out = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.bfloat16, device=dev)
    flops = ex_effective_flops(w)
    stream = torch.cuda.current_stream(dev)
    calibration_copy(args.calibrate_copy_mib, dev)

    def step():
        attn.fwd_ex(q, k, v, mask=w.mask, window=w.window, scale=w.scale, out=out,
                    stream=stream, alibi_slopes=slopes_d, q_len=q_len_d, kv_len=kv_len_d,
                    block_layout=layout_d, global_idx=list(w.global_idx) or None,
                    dist_bias=bias_d)

    ms, prewarm_steps, spread = time_steps(step, stream, args)
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"bench: {ms * 1e3:.1f} us/step, {tflops:.1f} effective TFLOP/s", file=sys.stderr,
          flush=True)
    peak = PEAK_BF16_TFLOPS
    result = {
        "metric": "effective attention TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, 1 GPU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Skv": w.Skv, "D": w.D, "mask": w.mask, "window": w.window,
                   "layout": w.layout, "alibi": w.alibi, "dist_bias": w.dist_bias,
                   "lengths": w.lengths,
                   "pattern": w.pattern, "pattern_args": list(w.pattern_args),
                   "effective_flops": flops, "parallelism": "none"},
        "pct_peak": round(100.0 * tflops / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": None,
        },
        "prewarm_steps": prewarm_steps,
        "step_spread": spread,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], n, ref = ex_cpu_baseline(w, inputs, args.cpu_seconds)
        if not args.no_parity:
            got = out[:1, :n].float().cpu().numpy()
            result["parity"] = {"sample": "the cpu_baseline sample",
                                "max_abs_err": max_abs_err(got, ref)}
    print(json.dumps(result), flush=True)
    return 0


def clock_line(tflops, dtype, cus, mhz, samples=None):
    """The sampled graphics clock (median of the busy samples, mean over the
    XCDs) and the throughput as a percentage of the dense matrix-core peak at
    that clock (CUs x FLOP/clk/CU x clock)."""
    per_clk = {"bf16": 4096, "fp8": 8192}.get(dtype)
    if mhz is None or per_clk is None:
        return {"sclk_mhz": mhz, "pct_of_peak_at_sclk": None, "samples": samples}
    peak = cus * per_clk * mhz * 1e6 / 1e12
    return {"sclk_mhz": round(mhz, 1), "peak_at_sclk_tflops": round(peak, 1),
            "pct_of_peak_at_sclk": round(100.0 * tflops / peak, 2), "samples": samples}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="oracle time budget of the cpu_baseline sample (whole key/value "
                         "groups of batch 0 until it is spent)")
    ap.add_argument("--no-clock", dest="clock", action="store_false",
                    help="do not sample the graphics clock with amd-smi")
    ap.add_argument("--prewarm", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache line (steps timed after a 512 MiB cache flush)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain elementwise copy of this many MiB (fp32 in, fp32 "
                         "out), whose HBM counters scale the attention kernel's")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "across GPUs the operation would shard by (batch, key/value head) with no "
              "communication, which is not built", file=sys.stderr)
        return 2

    import workloads

    name = args.workload or workloads.HEADLINE
    if name in workloads.DECODE_WORKLOADS:
        return bench_decode(args, name)
    if name in workloads.EX_WORKLOADS:
        return bench_ex(args, name)

    import torch

    import transformer_attention_attn_amd as attn

    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"bench: workload {name} {w.describe()}", file=sys.stderr, flush=True)
    inputs = workloads.workload_inputs(w)
    q, k, v = workloads.to_torch(inputs, w.dtype, dev)
    out = torch.empty(q.shape, dtype=torch.float32 if w.dtype == "fp32" else torch.bfloat16,
                      device=dev)
    g = list(w.global_idx) or None
    plan = attn.plan(w.B, w.Hq, w.Hkv, w.S, w.D, w.mask, w.window, g, w.dtype)
    flops = plan["effective_flops"]

    stream = torch.cuda.current_stream(dev)

    calibration_copy(args.calibrate_copy_mib, dev)

    def step():
        attn.fwd(q, k, v, mask=w.mask, window=w.window, global_idx=g, scale=w.scale, out=out,
                 stream=stream)

    ms, prewarm_steps, spread = time_steps(step, stream, args)
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"bench: {ms * 1e3:.1f} us/step, {tflops:.1f} effective TFLOP/s", file=sys.stderr,
          flush=True)

    peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(w.dtype, PEAK_FP32_TFLOPS)
    traffic = committed_traffic(name)
    # Q, K, V and O once each (K and V once per key/value head)
    esz = {"bf16": 2, "fp8": 1}.get(w.dtype, 4)
    osz = 4 if w.dtype == "fp32" else 2
    alg_bytes = (w.B * w.Hq * esz + 2 * w.B * w.Hkv * esz + w.B * w.Hq * osz) * w.S * w.D
    cold = None if args.no_cold else time_cold(step, stream, 20, dev)
    result = {
        "metric": "effective attention TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, 1 GPU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "mask": w.mask, "window": w.window, "global_idx": list(w.global_idx),
                   "effective_flops": flops, "parallelism": "none"},
        "pct_peak": round(100.0 * tflops / peak, 2),
        "roofline": {
            # the fp32 kernel runs on the vector ALUs (peak: the fp32 vector rate)
            "bound": "alu" if w.dtype == "fp32" else "mfma",
            "achieved": round(tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
        "prewarm_steps": prewarm_steps,
        "step_spread": spread,
        "algorithmic_bytes": alg_bytes,
        "algorithmic_gbs": round(alg_bytes / (ms * 1e-3) / 1e9, 2),
        "hbm_bytes_over_algorithmic": None if traffic is None else round(traffic / alg_bytes, 4),
        "cold_cache": cold,
        "gpu": torch.cuda.get_device_name(dev),
        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
        "clock": clock_line(tflops, w.dtype, torch.cuda.get_device_properties(dev)
                            .multi_processor_count, getattr(args, "clock_mhz", None),
                            getattr(args, "clock_samples", None)),
        "inputs_sha256": inputs_sha256(q, k, v),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(w, inputs, args.cpu_heads, args.cpu_seconds)
        if not args.no_parity:
            got = out[:1, :ref.shape[1]].float().cpu().numpy()
            result["parity"] = {"sample": "the cpu_baseline sample",
                                "max_abs_err": max_abs_err(got, ref)}

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
