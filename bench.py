"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-parity]

A step is one attn_fwd call over the whole workload (default: causal
grouped-query bf16, B=1 Hq=32 Hkv=8 S=8192 D=128) with the inputs already
resident in HBM.  K steps are timed with HIP events recorded on the stream the
kernel is launched on.  Prints one JSON line:

  value     effective TFLOP/s = unmasked FLOPs (4*D per visible (query, key)
            pair per query head) / time per step
  roofline  matrix-core bound: achieved TFLOP/s of the attention kernel (its
            algorithmic FLOPs per launch / its average launch duration) vs the
            MI355X dense bf16 peak; traffic = HBM bytes per launch from the
            committed rocprofv3 counter summary, or null when the kernel
            source changed since the counters were taken
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload,
            timed on the host's cores

A decode workload (--workload decode_...) times one attn_decode call (its
split-merge kernel included) and reports achieved HBM bandwidth instead:
value = algorithmic bytes (the valid cache entries, q and o, each once) /
time per step, against the 8 TB/s HBM peak.
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
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = ("kernel_bf16.hip", "gfx950_ops.h", "attn_kernels.h", "attn_sched.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_bf16_causal_gqa_s8192_hbm_traffic.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_attention_attn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source for this workload."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    txt = open(TRAFFIC_SUMMARY, encoding="utf-8").read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    m_wl = re.search(r"workload:\s*(\S+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_hash and m_wl and m_b):
        return None
    if m_hash.group(1) != kernel_source_hash() or m_wl.group(1) != workload:
        return None
    return float(m_b.group(1))


def cpu_baseline(w, inputs, n_heads: int):
    """Time the oracle on the first n_heads query heads of batch 0 (all rows)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((x.get("num_threads", 1) for x in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    G = w.Hq // w.Hkv
    n_heads = min(n_heads, w.Hq)
    n_kv = (n_heads + G - 1) // G
    q = inputs["q"][:1, :n_heads]
    k = inputs["k"][:1, :n_kv]
    v = inputs["v"][:1, :n_kv]
    # keep the head map: query head a of the sample still reads kv head a // G
    Hs = n_kv * G
    if Hs != n_heads:
        q = inputs["q"][:1, :Hs]
        n_heads = Hs
    t0 = time.perf_counter()
    oracle.attention(q, k, v, w.mask, w.window, w.global_idx, scale=w.scale)
    dt = time.perf_counter() - t0
    flops = oracle.effective_flops(1, n_heads, w.S, w.D, w.mask, w.window, w.global_idx)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"batch 0, query heads 0..{n_heads - 1} of {w.Hq}, all {w.S} rows "
                  f"({flops:.3e} effective FLOPs in {dt:.2f} s, fp64 NumPy)",
        "seconds": dt,
    }


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
    """Time the decode oracle on the first n_seq sequences (all heads and rows)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((x.get("num_threads", 1) for x in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    n = min(n_seq, w.B)
    sub = [int(x) for x in lens[:n]]
    t0 = time.perf_counter()
    oracle.decode_attention(inputs["q"][:n], inputs["k"][:n], inputs["v"][:n], w.mask,
                            cache_len=sub, scale=w.scale)
    dt = time.perf_counter() - t0
    nbytes = oracle.decode_cache_bytes(n, w.Hkv, w.D, sub, 2)
    return {
        "value": nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"sequences 0..{n - 1} of {w.B}, all {w.Hq} heads and {w.Sq} new positions "
                  f"({nbytes} cache bytes in {dt:.2f} s, fp64 NumPy)",
        "seconds": dt,
    }


def bench_decode(args, name):
    import numpy as np
    import torch

    import oracle
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
    ws_n = attn.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Smax, w.D, w.mask)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    calibration_copy(args.calibrate_copy_mib, dev)

    def step():
        attn.decode(q, k, v, cache_len=cl, mask=w.mask, scale=w.scale, out=out, workspace=ws,
                    stream=stream)

    t_warm = time.perf_counter()
    prewarm_steps = 0
    while time.perf_counter() - t_warm < args.prewarm:
        for _ in range(5):
            step()
        prewarm_steps += 5
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    cache_bytes = oracle.decode_cache_bytes(w.B, w.Hkv, w.D, lens, 2)
    qo_bytes = 2 * w.B * w.Hq * w.Sq * w.D * 2
    alg = cache_bytes + qo_bytes
    gbs = alg / (ms * 1e-3) / 1e9
    flops = oracle.decode_effective_flops(w.Hq, w.Sq, w.D, lens, w.mask)
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
            "traffic": None,
        },
        "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "prewarm_steps": prewarm_steps,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_parity:
        got = out.float().cpu().numpy()
        ref = oracle.decode_attention(inputs["q"][:1], inputs["k"][:1], inputs["v"][:1], w.mask,
                                      cache_len=[int(lens[0])], scale=w.scale)
        result["parity"] = {"batch": 0, "max_abs_err": float(np.max(np.abs(got[:1] - ref)))}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = decode_cpu_baseline(w, inputs, lens)
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--prewarm", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain elementwise copy of this many MiB (fp32 in, fp32 "
                         "out), whose HBM counters scale the attention kernel's")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the kernel shards by key/value head, see DESIGN.md", file=sys.stderr)
        return 2

    import workloads

    name = args.workload or workloads.HEADLINE
    if name in workloads.DECODE_WORKLOADS:
        return bench_decode(args, name)

    import numpy as np
    import torch

    import transformer_attention_attn_amd as attn

    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"bench: workload {name} {w.describe()}", file=sys.stderr, flush=True)
    inputs = workloads.workload_inputs(w)
    q, k, v = workloads.to_torch(inputs, w.dtype, dev)
    out = torch.empty_like(q)
    g = list(w.global_idx) or None
    plan = attn.plan(w.B, w.Hq, w.Hkv, w.S, w.D, w.mask, w.window, g, w.dtype)
    flops = plan["effective_flops"]

    stream = torch.cuda.current_stream(dev)

    calibration_copy(args.calibrate_copy_mib, dev)

    def step():
        attn.fwd(q, k, v, mask=w.mask, window=w.window, global_idx=g, scale=w.scale, out=out,
                 stream=stream)

    # Untimed warm-up: first about one second of steps (the GPU clocks ramp up
    # over the first ~100 ms of load), then the requested W warmup steps.
    t_warm = time.perf_counter()
    prewarm_steps = 0
    while time.perf_counter() - t_warm < args.prewarm:
        for _ in range(5):
            step()
        prewarm_steps += 5
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"bench: {ms * 1e3:.1f} us/step, {tflops:.1f} effective TFLOP/s", file=sys.stderr,
          flush=True)

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = committed_traffic(name)
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
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
        "prewarm_steps": prewarm_steps,
        "gpu": torch.cuda.get_device_name(dev),
        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
    }

    if not args.no_parity:
        import oracle

        rows = sorted({0, 1, 127, 128, w.S // 2, w.S - 1})
        ref = oracle.attention(inputs["q"][:1], inputs["k"][:1], inputs["v"][:1], w.mask,
                               w.window, w.global_idx, scale=w.scale, rows=rows)
        got = out[:1].float().cpu().numpy()[:, :, rows]
        result["parity"] = {"rows": rows, "batch": 0,
                            "max_abs_err": float(np.max(np.abs(got - ref)))}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_heads)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
