"""Benchmark of the MI355X W4A8 sparse-MoE decode path (one JSON line on stdout).

Workload timed for ``value``: the 42-layer MoE decode stack at 1 token (hidden 2560, 512 routed
experts, top-8 + 1 shared, SwiGLU width 768, MXFP4 experts, FP8 activations, unweighted RMSNorm on
each layer's input and a bf16 residual), ~67.6 GB of distinct expert weights resident in HBM, run
back to back through the C ABI (graph replays).  One step = one pass through all 42 layers.
``value`` is the algorithmic HBM bytes of a pass (router + the touched experts, counted from the
returned ids) divided by the pass time of K back-to-back steps.  Also reported:
  - the same stack at 4 tokens (disjoint top-8 sets, 33 experts per layer);
  - per-pass statistics (median, p10, p90, min) of both stacks, warm (back to back) and with the
    256 MB last-level cache flushed before every pass (a 1 GiB write outside the timed events);
  - kernel times of a layer launched kernel by kernel (events stamped by the launches themselves);
  - single layers at 1 and 4 tokens with the cache flushed between passes;
  - the roofline of the dominant 1-token kernel against 8 TB/s and against the practical read
    ceiling that a plain streaming-read probe reaches on the same box;
  - the FP8 LM head, the BF16 head it replaces, and the head's load-time quantisation;
  - the CPU oracle on a bounded sample of the same stack, on one thread and on every core;
  - the GPU, ROCm version and clocks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--graph-only]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode µs/token & achieved HBM GB/s (% of 8 TB/s), 1 and 4 tokens"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single", action="store_true", help="skip the single-layer measurements")
    ap.add_argument("--no-head", action="store_true", help="skip the FP8 LM-head measurement")
    ap.add_argument("--no-jit", action="store_true", help="skip the run-time compiled (hipRTC) kernels' measurement")
    ap.add_argument("--no-mfma", action="store_true", help="skip the matrix-core gate/up (MOE_F_MFMA) stack measurement")
    ap.add_argument("--graph-only", action="store_true",
                    help="time only graph replays of the stack (no direct-launch kernel timing, no single layers, "
                         "head or probe): the command to run under a kernel-trace profiler")
    ap.add_argument("--head-only", action="store_true",
                    help="time only the LM heads (and the copy probe with --copy-probe): the command to run under a "
                         "counter profiler for the head kernels")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (the reference kernel for HBM counters)")
    ap.add_argument("--summarize", metavar="DIR", nargs="+",
                    help="print a summary of the rocprofv3 CSV output in the DIRs (no GPU) and exit")
    ap.add_argument("--last", type=int, default=0,
                    help="with --summarize: also the mean duration of each kernel's last N dispatches")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.last)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_expert_gemv_amd as moe
    import synth

    if args.head_only:
        dev = torch.device("cuda:0")
        torch.cuda.init()
        stream = torch.cuda.current_stream()
        if args.copy_probe:
            copy_probe(torch, dev)
        print(json.dumps({"metric": "LM head", "lm_head": time_head(moe, dev, stream)}), flush=True)
        return

    man = json.load(open(os.path.join(ROOT, "tests", "golden", "manifest.json")))
    st = man["stack"]
    shape, L = synth.FLASH, st["layers"]
    dev = torch.device("cuda:0")
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    expert_bytes = shape.w13_bytes + shape.w13s_bytes + shape.w2_bytes + shape.w2s_bytes
    router_bytes = shape.num_experts * shape.hidden * 2

    def layer_tensors(seed, layer, attempt, bufs):
        r = synth.router(shape, seed, layer, attempt)
        bufs["router"].copy_(torch.from_numpy(r.view(np.int16)).view(torch.bfloat16))
        synth.fill_experts_device(bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"], shape, seed, layer,
                                  stream=stream.cuda_stream)

    n = shape.num_experts + shape.num_shared
    H, I = shape.hidden, shape.inter
    u8 = dict(dtype=torch.uint8, device=dev)
    bufs = {"router": torch.empty((shape.num_experts, H), dtype=torch.bfloat16, device=dev),
            "w13": torch.empty((n, 2 * I, H // 2), **u8), "w13_s": torch.empty((n, 2 * I, H // 32), **u8),
            "w2": torch.empty((n, H, I // 2), **u8), "w2_s": torch.empty((n, H, I // 32), **u8)}

    t0 = time.time()
    h = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, L, moe.F_RMSNORM_INPUT)
    for l in range(L):
        layer_tensors(st["seed"], l, st["router_attempts"][l], bufs)
        moe.moe_decode_set_layer(h, l, bufs["router"], bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"])
    torch.cuda.synchronize()
    info = moe.moe_decode_query(h)
    log(f"stack of {L} layers set in {time.time() - t0:.1f}s; variant {info['variant']}")

    x4_host = synth.tokens(H, st["seed"], 4, st["x_attempt"])
    x4 = torch.from_numpy(x4_host.view(np.int16)).to(dev).view(torch.bfloat16)
    x_out = torch.empty((4, H), dtype=torch.bfloat16, device=dev)

    def pass_bytes(T):
        ids = torch.empty((L, T, shape.top_k), dtype=torch.int32, device=dev)
        moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T], topk_ids=ids)
        torch.cuda.synchronize()
        idn = ids.cpu().numpy()
        distinct = [len(set(idn[l].reshape(-1).tolist())) for l in range(L)]
        return sum(router_bytes + (d + shape.num_shared) * expert_bytes for d in distinct), distinct

    def time_stack(T, steps, warmup):
        for _ in range(warmup):
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def pass_stats(T, passes, flush):
        """Each pass timed on its own (events around the pass only); with flush, a 1 GiB buffer is
        written before every pass, outside the events, to evict the last-level cache."""
        times = []
        for _ in range(passes):
            if flush is not None:
                flush.add_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
            e1.record(stream)
            times.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in times]) / L
        return {"us_per_layer_median": round(float(np.median(us)), 3), "p10": round(float(np.percentile(us, 10)), 3),
                "p90": round(float(np.percentile(us, 90)), 3), "min": round(float(us.min()), 3), "passes": passes}

    def kernel_times(T, runs):
        """Kernels launched one by one between kernel-stamped events: us per launch, per class."""
        moe.moe_decode_timing_enable(h, runs, 0)
        for _ in range(runs):
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
        t = moe.moe_decode_timing_read(h)
        moe.moe_decode_timing_enable(h, 0)
        return {c: t[c]["total_ms"] / t[c]["launches"] * 1e3 for c in moe.TIMING_CLASSES if t[c]["launches"]}

    def graph_breakdown(T, runs):
        """Graph-replayed passes whose kernels stamp the device wall clock per workgroup: per class the
        mean span (first workgroup's start to last workgroup's end) and the mean gap before it; spans
        and gaps of a layer add up to the layer's share of the pass."""
        moe.moe_decode_timing_enable(h, runs, 1)
        for _ in range(runs):
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
        t = moe.moe_decode_timing_read(h)
        moe.moe_decode_timing_enable(h, 0)
        out = {c: {"span_us": round(t[c]["total_ms"] / t[c]["launches"] * 1e3, 3),
                   "gap_before_us": round(t[c]["gap_ms"] / max(t[c]["gap_launches"], 1) * 1e3, 3)}
               for c in moe.TIMING_CLASSES if t[c]["launches"]}
        out["layer_us"] = round(sum(v["span_us"] + v["gap_before_us"] for v in out.values()), 3)
        return out

    if args.copy_probe:
        copy_probe(torch, dev)

    results = {}
    flush_buf = None if args.graph_only else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for T in (1, 4):
        nbytes, distinct = pass_bytes(T)
        ms = time_stack(T, args.steps, args.warmup)
        moe.moe_decode_check(h)  # no asynchronous device error
        gbs = nbytes / (ms * 1e-3) / 1e9
        results[T] = {"ms_per_pass": ms, "us_per_layer": ms * 1e3 / L, "tokens_per_s": T / (ms * 1e-3),
                      "bytes_per_pass": nbytes, "gb_s": gbs, "pct_of_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
                      "distinct_experts_per_layer": sorted(set(distinct))}
        log(f"stack T={T}: {ms * 1e3:.1f} us/pass, {ms * 1e3 / L:.2f} us/layer, {gbs:.0f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")
        if args.graph_only:
            continue
        npass = max(20, min(args.steps, 100))
        warm = pass_stats(T, npass, None)
        flushed = pass_stats(T, npass, flush_buf)
        kt = kernel_times(T, min(args.steps, 50))
        gb = graph_breakdown(T, min(args.steps, 20))
        results[T].update({"warm": warm, "flushed": flushed, "kernel_us_direct_launch": kt,
                           "kernel_sum_us_per_layer": round(sum(kt.values()), 3), "graph_replay_breakdown": gb})
        log(f"stack T={T}: per pass, warm {warm}; last-level cache flushed before each pass {flushed}; "
            f"kernels launched one by one (us) {kt}; graph replays, per-kernel span and gap before it (us) {gb}")
    if args.graph_only:
        r1 = results[1]
        print(json.dumps({"metric": METRIC, "value": round(r1["gb_s"], 1), "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r1["ms_per_pass"], 5),
                          "mode": "graph replays only", "stack_t4_ms_per_pass": round(results[4]["ms_per_pass"], 5)}),
              flush=True)
        moe.moe_decode_destroy(h)
        return
    del flush_buf
    # the same stack on kernels compiled at run time for this shape (hipRTC), against the
    # ahead-of-time build just timed
    jit = None
    if not args.no_jit:
        import tempfile
        moe.moe_decode_destroy(h)
        torch.cuda.synchronize()
        cache = tempfile.mkdtemp(prefix="moe_jit_cache_")  # an empty cache: the first create compiles
        os.environ["MOE_JIT_CACHE_DIR"] = cache
        t0 = time.time()
        h = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, L,
                                  moe.F_RMSNORM_INPUT | moe.F_JIT)
        create_s = time.time() - t0
        t0 = time.time()  # a second handle of the same shape loads the cached code object
        h2 = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, 1,
                                   moe.F_RMSNORM_INPUT | moe.F_JIT)
        cached_create_s = time.time() - t0
        cached = moe.moe_decode_query(h2)["jit_from_cache"]
        moe.moe_decode_destroy(h2)
        for l in range(L):
            layer_tensors(st["seed"], l, st["router_attempts"][l], bufs)
            moe.moe_decode_set_layer(h, l, bufs["router"], bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"])
        torch.cuda.synchronize()
        ji = moe.moe_decode_query(h)
        jit = {"variant": ji["variant"], "compile_ms": round(ji["jit_compile_ms"], 1),
               "from_cache": ji["jit_from_cache"], "create_s": round(create_s, 3),
               "second_create_from_cache": cached, "second_create_s": round(cached_create_s, 3)}
        for T in (1, 4):
            ms = time_stack(T, args.steps, args.warmup)
            jit[f"t{T}_us_per_layer"] = round(ms * 1e3 / L, 3)
            jit[f"t{T}_vs_ahead_of_time"] = round(results[T]["ms_per_pass"] / ms, 4)
        log(f"run-time compiled kernels: {jit}")
    # the same stack with the gate/up dot products on the matrix cores (MOE_F_MFMA, a per-handle choice)
    mfma = None
    if not args.no_mfma:
        moe.moe_decode_destroy(h)
        torch.cuda.synchronize()
        h = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, L,
                                  moe.F_RMSNORM_INPUT | moe.F_MFMA)
        for l in range(L):
            layer_tensors(st["seed"], l, st["router_attempts"][l], bufs)
            moe.moe_decode_set_layer(h, l, bufs["router"], bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"])
        torch.cuda.synchronize()
        mfma = {"variant": moe.moe_decode_query(h)["variant"]}
        for T in (1, 4):
            nbytes, _ = pass_bytes(T)
            ms = time_stack(T, args.steps, args.warmup)
            moe.moe_decode_check(h)
            mfma[f"t{T}_us_per_layer"] = round(ms * 1e3 / L, 3)
            mfma[f"t{T}_gb_s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            mfma[f"t{T}_vs_valu"] = round(results[T]["ms_per_pass"] / ms, 4)
        log(f"matrix-core gate/up stack: {mfma}")
    probe = hbm_probe(moe, torch, dev, stream)

    # single layers (1 and 4 tokens), last-level cache flushed between passes
    single = {}
    if not args.no_single:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        # layer_t4_overlap: a verify step whose 4 tokens share routed experts (correlated tokens,
        # rho 0.9); its bytes are counted from the distinct experts the run returns
        for name, key, T in (("layer_t1", "layer_t1", 1), ("layer_t4", "layer_t4", 4),
                             ("layer_t4_overlap", "layer_t4", 4)):
            m = man[key]
            h1 = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, 1)
            layer_tensors(m["seed"], 0, 0, bufs)
            moe.moe_decode_set_layer(h1, 0, bufs["router"], bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"])
            if name == "layer_t4_overlap":
                xh = synth.tokens_correlated(H, m["seed"], T, 0.9, 0)
            else:
                xh = synth.tokens(H, m["seed"], T, m["x_attempt"])
            xs = torch.from_numpy(xh.view(np.int16)).to(dev).view(torch.bfloat16)
            ids1 = torch.empty((1, T, shape.top_k), dtype=torch.int32, device=dev)
            moe.moe_decode_run(h1, xs, T, topk_ids=ids1)
            torch.cuda.synchronize()
            distinct = len(set(ids1.cpu().numpy().reshape(-1).tolist()))
            y = torch.empty((T, H), dtype=torch.float32, device=dev)
            times = []
            for i in range(args.warmup + args.steps):
                flush.add_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                moe.moe_decode_run(h1, xs, T, y=y)
                e1.record(stream)
                e1.synchronize()
                if i >= args.warmup:
                    times.append(e0.elapsed_time(e1) * 1e3)
            nbytes = router_bytes + (distinct + shape.num_shared) * expert_bytes
            med = float(np.median(times))
            single[name] = {"tokens": T, "distinct_routed_experts": distinct, "us_median": med,
                            "us_p10": float(np.percentile(times, 10)),
                            "us_p90": float(np.percentile(times, 90)), "bytes": nbytes,
                            "gb_s": nbytes / (med * 1e-6) / 1e9}
            log(f"single layer {name} ({distinct} routed experts, cache flushed): median {med:.1f} us, "
                f"{single[name]['gb_s']:.0f} GB/s")
            moe.moe_decode_destroy(h1)
        del flush

    # roofline of the dominant kernel of a 1-token layer (the one with the largest kernel time)
    kt1 = results[1]["kernel_us_direct_launch"]
    names = kernel_names(info["variant"], 1)
    kb = kernel_bytes(shape, 1, shape.top_k)
    per_kernel = {c: {"kernel": names[c], "bytes_per_launch": kb[c], "us_per_launch": round(kt1[c], 3),
                      "gb_s": round(kb[c] / (kt1[c] * 1e-6) / 1e9, 1)} for c in kt1}
    dom = max(kt1, key=lambda c: kt1[c])
    achieved = per_kernel[dom]["gb_s"]
    traffic = measured_traffic(names[dom])
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": names[dom],
                "bytes_per_launch": kb[dom], "us_per_launch": round(kt1[dom], 3), "all_kernels_t1": per_kernel,
                "practical_read_ceiling_gb_s": probe["best_gb_s"],
                "frac_of_practical_ceiling": round(achieved / probe["best_gb_s"], 4)}
    log(f"roofline: dominant {names[dom]} {kt1[dom]:.2f} us/launch, {achieved:.0f} GB/s; {per_kernel}")

    head = None if args.no_head else time_head(moe, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, st, x4_host[:1], expert_bytes, router_bytes)
    env = environment(torch)

    r1 = results[1]
    out = {"metric": METRIC, "value": round(r1["gb_s"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(r1["ms_per_pass"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "e2m1*e4m3->fp32", "data": "synthetic",
           "config": {"workload": "42-layer MoE decode stack, 1 token", "hidden": H, "experts": shape.num_experts,
                      "top_k": shape.top_k, "shared": shape.num_shared, "inter": I, "layers": L, "tokens": 1},
           "us_per_layer": round(r1["us_per_layer"], 3), "tokens_per_s": round(r1["tokens_per_s"], 1),
           "pct_of_hbm_peak": round(r1["pct_of_hbm_peak"], 2),
           "pct_of_practical_read_ceiling": round(100 * r1["gb_s"] / probe["best_gb_s"], 2),
           "stack_t1": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r1.items()},
           "stack_t4": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in results[4].items()},
           "single_layer": single, "lm_head": head, "hbm_read_probe": probe, "jit": jit, "mfma_gateup": mfma,
           "variant": info["variant"],
           "roofline": roofline, "cpu_baseline": cpu, "env": env}
    moe.moe_decode_destroy(h)
    print(json.dumps(out), flush=True)


COPY_PROBE_BYTES = 256 << 20
KERNEL_SOURCES = [os.path.join(ROOT, "mxfp4_expert_gemv_amd", "csrc", f)
                  for f in ("moe_kernels.hip", "moe_kernels_flash.hip", "moe_kernels.h", "moe_device.h", "moe_layout.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_stack_t1.md")


def copy_probe(torch, dev):
    """Four plain device-to-device copies of COPY_PROBE_BYTES: the reference dispatches that scale
    the HBM byte counters (each reads and writes COPY_PROBE_BYTES)."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log(f"copy probe: 4 copies of {COPY_PROBE_BYTES} bytes")


def source_digest():
    """Digest of the MoE kernels' device sources (the .hip file and the headers it compiles)."""
    import hashlib
    d = hashlib.sha256()
    for f in KERNEL_SOURCES:
        d.update(os.path.basename(f).encode() + b"\0" + open(f, "rb").read())
    return d.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when there is
    none or the kernel source has changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    block = text.split("```json")[1].split("```")[0] if "```json" in text else None
    if block is None:
        return None
    rec = json.loads(block)
    if rec.get("kernel_source_sha256_16") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


def ours(name):
    """A kernel of this library (not torch's or the runtime's, nor the input generator's)."""
    return any(k in name for k in ("moe::", "head::", "probe::"))


def summarize(dirs, last=0):
    """Markdown summary of rocprofv3 output in the given directories: the kernel statistics (--stats)
    of this library's kernels (with last: also the mean of each kernel's last `last` dispatches, from
    the kernel trace) and, when counter files are present, FETCH_SIZE / WRITE_SIZE per dispatch, each
    scaled by what the same counter reads for the 256 MiB copy probe (known to read and write 256 MiB),
    and the other counters per dispatch."""
    import csv
    import glob

    def rows(pattern):
        out = []
        for d in dirs:
            for f in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
                with open(f) as fh:
                    out += list(csv.DictReader(fh))
        return out

    stats = [r for r in rows("*kernel_stats.csv") if ours(r["Name"])]
    if stats:
        tail = {}
        if last:
            per = {}
            for r in rows("*kernel_trace.csv"):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            for n, v in per.items():
                v.sort()
                tail[n] = sum(d for _, d in v[-last:]) / len(v[-last:]) / 1e3
        print("| kernel | calls | average us | min us | max us | share % |" + (f" last {last}: average us |" if last else ""))
        print("|---|---:|---:|---:|---:|---:|" + ("---:|" if last else ""))
        for r in stats:
            t = f" {tail[r['Name']]:.2f} |" if last and r["Name"] in tail else (" |" if last else "")
            print(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |" + t)
    counters = rows("*counter_collection.csv")
    if counters:
        # the probe copies are the copy-kernel dispatches of the largest size; other copies (router
        # rows at set-up) are smaller and are left out
        probe = {}
        for r in counters:
            if "copyBuffer" in r["Kernel_Name"]:
                probe.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        scale = {}
        for c, vals in probe.items():
            big = [v for v in vals if v >= 0.5 * max(vals)]
            scale[c] = (COPY_PROBE_BYTES / 1024) / (sum(big) / len(big))
        acc = {}
        for r in counters:
            if "copyBuffer" in r["Kernel_Name"]:
                continue
            a = acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), [0.0, 0])
            a[0] += float(r["Counter_Value"])
            a[1] += 1
        kib = {k: v[0] / v[1] for k, v in acc.items()}
        sizes = {(n, c): v for (n, c), v in kib.items() if c in ("FETCH_SIZE", "WRITE_SIZE")}
        other = sorted({c for (_, c) in kib if c not in ("FETCH_SIZE", "WRITE_SIZE")})
        if other:  # one row per kernel, one column per counter (means per dispatch)
            print()
            print("| kernel | dispatches | " + " | ".join(other) + " |")
            print("|---|---:|" + "---:|" * len(other))
            for n in sorted({n for (n, c) in kib if c in other}):
                d = max(acc[(n, c)][1] for c in other if (n, c) in acc)
                print(f"| `{n}` | {d} | " + " | ".join(f"{kib[(n, c)]:.2f}" if (n, c) in kib else "" for c in other)
                      + " |")
        if not sizes:
            return
        print()
        print("| kernel | counter | mean per dispatch (KiB) | dispatches | scale (copy probe) | bytes per dispatch |")
        print("|---|---|---:|---:|---:|---:|")
        rec = {"kernel_source_sha256_16": source_digest(), "copy_probe_bytes": COPY_PROBE_BYTES, "scale": scale,
               "kernels": {}}
        for (n, c), v in sorted(sizes.items()):
            sc = scale.get(c)
            b = v * 1024 * sc if sc else None
            print(f"| `{n}` | {c} | {v:.2f} | {acc[(n, c)][1]} | {'' if sc is None else round(sc, 4)} | "
                  f"{'' if b is None else int(b)} |")
            if b is not None:
                k = rec["kernels"].setdefault(n, {"hbm_bytes_per_launch": 0})
                k[c] = int(b)
                k["hbm_bytes_per_launch"] += int(b)
        if rec["kernels"]:
            print()
            print("```json")
            print(json.dumps(rec, indent=1))
            print("```")


def kernel_bytes(shape, T, distinct):
    """Algorithmic HBM bytes of one launch of each kernel of a layer: the weights it must read once
    (router; gate/up and down halves of the touched experts) plus the activations it reads or writes
    in HBM; per-call scratch that stays in the L2 (logits, slot list, h) is not counted."""
    w13 = shape.w13_bytes + shape.w13s_bytes
    w2 = shape.w2_bytes + shape.w2s_bytes
    x = T * shape.hidden * 2
    return {"router": shape.num_experts * shape.hidden * 2 + x,
            "gateup": (distinct + shape.num_shared) * w13,
            "down": (distinct + shape.num_shared) * w2 + 2 * x}


def kernel_names(variant, T):
    """Full names of the kernels of a 1-2 token layer as the profiler lists them, from the library's
    variant string (gfx950-3k-gu<waves>x<blocks per lane>-dn<ksub>x<iters>-<launch>[-jit][-mfma][-flash]).
    "-flash": the ahead-of-time build with the layer shape folded in, in namespace moe::flash."""
    parts = variant.split("-")
    gu, dn = parts[2:4]
    bpl = int(gu[2:].split("x")[1])
    ksub, iters = (int(v) for v in dn[2:].split("x"))
    mf = "true" if "mfma" in parts[4:] else "false"
    ns = "moe::flash::" if "flash" in parts[4:] else "moe::"
    return {"router": f"void {ns}k1_router<{T}, {bpl}, {mf}, false>({ns}K1Args)",
            "gateup": f"void {ns}k2_gateup<{T}, {bpl}, {4 if T == 1 else 2}, {mf}, false>({ns}K2Args)",
            "down": f"void {ns}k3_down<{ksub}, {iters}, {T}, {T}, false>({ns}K3Args)"}


def _event_time_us(fn, stream, steps, warmup):
    """Mean µs per call of fn over `steps` back-to-back calls, event-timed on `stream`."""
    import torch

    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def time_head(moe, dev, stream, steps=50, warmup=5):
    """The FP8 LM head (vocab 157,184 x hidden 2,560, E4M3 rows with fp32 row scales, argmax only)
    at 1 and 4 tokens, back to back (its 403 MB exceed the 256 MB last-level cache).  Random codes
    (no NaN pattern) and scales: the timing does not depend on the values."""
    import torch

    V, H = 157184, 2560
    w = torch.randint(0, 0x7E, (V, H), dtype=torch.uint8, device=dev)
    w |= torch.randint(0, 2, (V, H), dtype=torch.uint8, device=dev) << 7
    scale = torch.full((V,), 1e-3, dtype=torch.float32, device=dev)
    hd = moe.fp8_head_create(w, scale)
    torch.cuda.synchronize()
    del w
    x = torch.randn((4, H), device=dev).to(torch.bfloat16)
    am = torch.empty((4,), dtype=torch.int32, device=dev)
    nbytes = V * H + V * 4
    out = {"vocab": V, "hidden": H, "bytes_per_call": nbytes}
    for T in (1, 4):
        us = _event_time_us(lambda: moe.fp8_head_run(hd, x[:T], am[:T]), stream, steps, warmup)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[f"t{T}"] = {"us": round(us, 2), "gb_s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        log(f"LM head T={T}: {us:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")
    # the head of a 4-token verify step: the same pass with the greedy acceptance of the 3 drafts
    # fused into its final reduction
    draft = torch.zeros((3,), dtype=torch.int32, device=dev)
    accept = torch.empty((1,), dtype=torch.int32, device=dev)
    us = _event_time_us(lambda: moe.fp8_head_verify(hd, x, draft, am, accept), stream, steps, warmup)
    gbs = nbytes / (us * 1e-6) / 1e9
    out["verify_t4"] = {"us": round(us, 2), "gb_s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                        "vs_plain_t4": round(us / out["t4"]["us"], 3)}
    log(f"LM head verify step T=4 (argmax + acceptance): {us:.1f} us, {us / out['t4']['us']:.3f}x the plain T=4 head")
    moe.fp8_head_destroy(hd)
    # the unquantised BF16 head it replaces (twice the bytes), for the comparison
    wb = (torch.randn((V, H), device=dev) * 0.02).to(torch.bfloat16)
    hb = moe.bf16_head_create(wb)
    torch.cuda.synchronize()
    del wb
    bbytes = V * H * 2
    for T in (1, 4):
        us = _event_time_us(lambda: moe.fp8_head_run(hb, x[:T], am[:T]), stream, steps, warmup)
        gbs = bbytes / (us * 1e-6) / 1e9
        out[f"bf16_t{T}"] = {"us": round(us, 2), "gb_s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                             "fp8_speedup": round(us / out[f"t{T}"]["us"], 3)}
        log(f"BF16 LM head T={T}: {us:.1f} us, {gbs:.0f} GB/s; FP8 head is {us / out[f't{T}']['us']:.2f}x faster")
    moe.fp8_head_destroy(hb)
    # the load-time quantisation of the head (fp32 rows in, E4M3 codes and row scales out)
    wf = torch.randn((V, H), device=dev) * 0.02
    codes = torch.empty((V, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((V,), dtype=torch.float32, device=dev)
    us = _event_time_us(lambda: moe.fp8_head_quantize(wf, codes, sc), stream, 10, 1)
    qbytes = V * H * 4 + V * H + V * 4
    out["quantize_fp32"] = {"us": round(us, 1), "bytes": qbytes, "gb_s": round(qbytes / (us * 1e-6) / 1e9, 1)}
    log(f"LM head quantisation (fp32 in): {us:.1f} us, {qbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    del wf, codes, sc
    return out


def hbm_probe(moe, torch, dev, stream, nbytes=4 << 30, reps=10):
    """Practical HBM read ceiling: the library's streaming-read probe (16-byte non-temporal loads, as
    the weight kernels use) over a 4 GiB buffer, far above the 256 MB last-level cache, at several
    grid sizes; the best is reported."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(65536, dtype=torch.int32, device=dev)
    by_grid = {}
    for grid in (1024, 2048, 4096, 8192, 16384):
        moe.moe_probe_stream_read(buf, out, grid)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            moe.moe_probe_stream_read(buf, out, grid)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        by_grid[grid] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del buf, out
    best = max(by_grid.values())
    log(f"streaming-read probe over {nbytes >> 20} MiB: GB/s by grid {by_grid}")
    return {"bytes": nbytes, "best_gb_s": best, "pct_of_8_tb_s": round(100 * best / HBM_PEAK_GBS, 2),
            "gb_s_by_grid": by_grid}


def environment(torch):
    """GPU, ROCm version and clocks of the box the numbers were taken on.  rocm-smi is sampled after
    the runs, with the GPU at rest, so its clock levels are the idle ones, not those of the timed
    kernels."""
    import subprocess
    env = {"gpu": torch.cuda.get_device_name(0),
           "compute_units": torch.cuda.get_device_properties(0).multi_processor_count}
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    for cmd in (["rocm-smi", "--showclocks"], ["rocm-smi", "--showpower"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            lines = [l.strip() for l in r.stdout.splitlines() if "GPU[" in l]
            env[" ".join(cmd[1:]) + " (GPU at rest)"] = lines[:12]
        except (OSError, subprocess.SubprocessError):
            env[" ".join(cmd[1:]) + " (GPU at rest)"] = None
    return env


def host_cpu():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(shape, st, x_host, expert_bytes, router_bytes, budget_s=10.0):
    """The oracle (C, fp64) run layer by layer along the same 1-token stack on the host cores until
    about budget_s of compute, once on one thread and once with its loops over independent rows
    split over every core available to the process; reported in GB/s of the same algorithmic
    bytes.  The main figure is the multi-threaded one."""
    import oracle

    hc = host_cpu()
    n = max(1, hc["affinity"])
    single = _oracle_leg(shape, st, x_host, expert_bytes, router_bytes, budget_s, 1)
    multi = _oracle_leg(shape, st, x_host, expert_bytes, router_bytes, budget_s, n)
    oracle.set_threads(1)
    return {"value": multi["gb_s"], "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"first {multi['layers']} layers of the 1-token 42-layer stack (compute only, weights "
                      f"pre-generated), oracle loops over independent rows on {n} threads",
            "us_per_layer": multi["us_per_layer"], "host": hc,
            "single_thread": {"value": single["gb_s"], "unit": "GB/s", "cores": 1, "layers": single["layers"],
                              "us_per_layer": single["us_per_layer"]}}


def _oracle_leg(shape, st, x_host, expert_bytes, router_bytes, budget_s, threads):
    import oracle
    import synth

    oracle.set_threads(threads)
    x = x_host.copy()
    spent, layers = 0.0, 0
    for l in range(st["layers"]):
        router = synth.router(shape, st["seed"], l, st["router_attempts"][l])
        t0 = time.perf_counter()
        xin = oracle.rmsnorm_bf16(x)
        ids = oracle.route(shape, router, xin)["ids"]
        spent += time.perf_counter() - t0
        experts = {e: synth.expert(shape, st["seed"], l, e) for e in list(ids[0]) + [shape.num_experts]}
        t0 = time.perf_counter()
        y, _ = oracle.moe_layer(shape, router, experts, xin, trace=False)
        x = oracle.residual_bf16(x, y)
        spent += time.perf_counter() - t0
        layers += 1
        if spent > budget_s:
            break
    per_layer = router_bytes + (shape.top_k + shape.num_shared) * expert_bytes
    gbs = layers * per_layer / spent / 1e9
    log(f"cpu oracle, {threads} thread(s): {layers} layers in {spent:.1f}s ({spent / layers * 1e3:.0f} ms/layer)")
    return {"gb_s": round(gbs, 4), "layers": layers, "us_per_layer": round(spent / layers * 1e6, 1)}


if __name__ == "__main__":
    main()
