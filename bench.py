"""Benchmark of the MI355X W4A8 sparse-MoE decode path (one JSON line on stdout).

Workload timed for ``value``: the 42-layer MoE decode stack at 1 token (hidden 2560, 512 routed
experts, top-8 + 1 shared, SwiGLU width 768, MXFP4 experts, FP8 activations, unweighted RMSNorm on
each layer's input and a bf16 residual), ~67.6 GB of distinct expert weights resident in HBM, run
back to back through the C ABI.  One step = one pass through all 42 layers.  ``value`` is the
algorithmic HBM bytes of a pass (router + the touched experts, counted from the returned ids)
divided by the pass time.  Also reported: the same stack at 4 tokens (disjoint top-8 sets, 33
experts per layer), single layers at 1 and 4 tokens with the 256 MB last-level cache flushed
between passes, the roofline of the dominant kernel (gate/up), and the CPU oracle timed on a
bounded sample of the same stack on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_expert_gemv_amd as moe
    import synth

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

    def kernel_times(T, runs):
        moe.moe_decode_timing_enable(h, runs)
        for _ in range(runs):
            moe.moe_decode_run(h, x4[:T], T, x_out=x_out[:T])
        t = moe.moe_decode_timing_read(h)
        moe.moe_decode_timing_enable(h, 0)
        return {c: t[c]["total_ms"] / max(t[c]["launches"], 1) * 1e3 for c in moe.TIMING_CLASSES}  # us/launch

    results = {}
    for T in (1, 4):
        nbytes, distinct = pass_bytes(T)
        ms = time_stack(T, args.steps, args.warmup)
        kt = kernel_times(T, min(args.steps, 50))
        gbs = nbytes / (ms * 1e-3) / 1e9
        results[T] = {"ms_per_pass": ms, "us_per_layer": ms * 1e3 / L, "tokens_per_s": T / (ms * 1e-3),
                      "bytes_per_pass": nbytes, "gb_s": gbs, "pct_of_hbm_peak": 100 * gbs / HBM_PEAK_GBS,
                      "distinct_experts_per_layer": sorted(set(distinct)), "kernel_us": kt}
        log(f"stack T={T}: {ms * 1e3:.1f} us/pass, {ms * 1e3 / L:.2f} us/layer, {gbs:.0f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s); per-kernel us {kt}")

    # single layers (1 and 4 tokens), last-level cache flushed between passes
    single = {}
    if not args.no_single:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for name, key, T in (("layer_t1", "layer_t1", 1), ("layer_t4", "layer_t4", 4)):
            m = man[key]
            h1 = moe.moe_decode_create(H, shape.num_experts, shape.top_k, shape.num_shared, I, 4, 1, 0)
            layer_tensors(m["seed"], 0, 0, bufs)
            moe.moe_decode_set_layer(h1, 0, bufs["router"], bufs["w13"], bufs["w13_s"], bufs["w2"], bufs["w2_s"])
            xs = torch.from_numpy(synth.tokens(H, m["seed"], T, m["x_attempt"]).view(np.int16)).to(dev)
            xs = xs.view(torch.bfloat16)
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
            distinct = len(set(sum(m["ids"], [])))
            nbytes = router_bytes + (distinct + shape.num_shared) * expert_bytes
            med = float(np.median(times))
            single[name] = {"tokens": T, "us_median": med, "us_p10": float(np.percentile(times, 10)),
                            "us_p90": float(np.percentile(times, 90)), "bytes": nbytes,
                            "gb_s": nbytes / (med * 1e-6) / 1e9}
            log(f"single layer T={T} (cache flushed): median {med:.1f} us, {single[name]['gb_s']:.0f} GB/s")
            moe.moe_decode_destroy(h1)
        del flush

    # roofline of the dominant kernel (gate/up: 61% of a 1-token layer's bytes)
    gu_bytes = (shape.top_k + shape.num_shared) * (shape.w13_bytes + shape.w13s_bytes)
    gu_us = results[1]["kernel_us"]["gateup"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "gateup_kernel<1>",
                "bytes_per_launch": gu_bytes, "us_per_launch": round(gu_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, st, x4_host[:1], expert_bytes, router_bytes)

    r1 = results[1]
    out = {"metric": METRIC, "value": round(r1["gb_s"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(r1["ms_per_pass"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "e2m1*e4m3->fp32", "data": "synthetic",
           "config": {"workload": "42-layer MoE decode stack, 1 token", "hidden": H, "experts": shape.num_experts,
                      "top_k": shape.top_k, "shared": shape.num_shared, "inter": I, "layers": L, "tokens": 1},
           "us_per_layer": round(r1["us_per_layer"], 3), "tokens_per_s": round(r1["tokens_per_s"], 1),
           "pct_of_hbm_peak": round(r1["pct_of_hbm_peak"], 2), "kernel_us_t1": r1["kernel_us"],
           "stack_t4": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in results[4].items()},
           "single_layer": single, "variant": info["variant"], "roofline": roofline, "cpu_baseline": cpu}
    moe.moe_decode_destroy(h)
    print(json.dumps(out), flush=True)


def cpu_baseline(shape, st, x_host, expert_bytes, router_bytes, budget_s=12.0):
    """The oracle (single-threaded C, fp64) run layer by layer along the same 1-token stack on the
    host cores until about budget_s of compute; reported in GB/s of the same algorithmic bytes."""
    import oracle
    import synth

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
    log(f"cpu oracle: {layers} layers in {spent:.1f}s ({spent / layers * 1e3:.0f} ms/layer)")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {layers} layers of the 1-token 42-layer stack (compute only, weights pre-generated)",
            "us_per_layer": round(spent / layers * 1e6, 1)}


if __name__ == "__main__":
    main()
