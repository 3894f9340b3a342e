"""Writes tests/golden/manifest.json: the seeded inputs of every workload, chosen with the oracle.

Calls only ``synth`` (input generator) and ``oracle`` (CPU reference).  For each workload it walks
the generator's ``attempt`` counter upward from 0 until the integer results are well posed:

  - routing: for every token, the first k+1 router logits in (value desc, index asc) order are
    separated by more than the sum of their fp32 summation-error bounds, so the ordered top-k
    ids cannot change under any fp32 accumulation order;
  - 4-token verify: in addition the four tokens' top-k sets are pairwise disjoint (32 distinct
    routed experts, "up to 32 experts" for a 4-position verify);
  - 42-layer stack: the router of each layer is re-drawn (its attempt counter) along the oracle's
    own trajectory until the 4-token conditions hold at that layer; the 1-token stack runs token 0;
  - LM head: for every token, top-1 and top-2 logits are separated by more than their bounds.

Run from the repository root:  python tests/golden/make_manifest.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "manifest.json")
LAYERS = 42


def margins_ok(ro, k):
    return all(oracle.topk_margin_ok(ro["logits"][t], ro["bounds"][t], k) for t in range(ro["ids"].shape[0]))


def disjoint(ids):
    flat = ids.reshape(-1)
    return len(set(flat.tolist())) == flat.size


def search_tokens(shape, seed, T, need_disjoint, router):
    for a in range(10000):
        x = synth.tokens(shape.hidden, seed, T, a)
        ro = oracle.route(shape, router, x)
        if margins_ok(ro, shape.top_k) and (not need_disjoint or disjoint(ro["ids"])):
            return a, ro
    raise RuntimeError("no attempt satisfied the margins")


def layer_entry(seed, a, ro):
    return {"seed": seed, "x_attempt": a, "ids": ro["ids"].tolist(),
            "min_gap_over_bound": float(min(_gap_ratio(ro, t) for t in range(ro["ids"].shape[0])))}


def _gap_ratio(ro, t):
    l, b = ro["logits"][t], ro["bounds"][t]
    k = ro["ids"].shape[1]
    order = np.lexsort((np.arange(l.size), -l))[: k + 1]
    return min((l[p] - l[q]) / (b[p] + b[q]) for p, q in zip(order[:-1], order[1:]))


def main():
    t0 = time.time()
    man = {"generator": "SplitMix64 counter generator (synth/synth_host.c)",
           "note": "attempt counters chosen by tests/golden/make_manifest.py with the oracle"}
    # tiny layer, 1 token (and a 4-token variant for parity of the multi-token path)
    router = synth.router(synth.TINY, 0)
    a, ro = search_tokens(synth.TINY, 0, 1, False, router)
    man["tiny"] = layer_entry(0, a, ro)
    a, ro = search_tokens(synth.TINY, 0, 4, False, router)
    man["tiny_t4"] = layer_entry(0, a, ro)
    # flash-shaped layer, 1 token
    router = synth.router(synth.FLASH, 1)
    a, ro = search_tokens(synth.FLASH, 1, 1, False, router)
    man["layer_t1"] = layer_entry(1, a, ro)
    # 4-token verify with disjoint routing
    router = synth.router(synth.FLASH, 2)
    a, ro = search_tokens(synth.FLASH, 2, 4, True, router)
    man["layer_t4"] = layer_entry(2, a, ro)
    print(f"single layers done ({time.time() - t0:.1f}s)", flush=True)

    # 42-layer stack along the oracle trajectory of 4 tokens
    shape = synth.FLASH
    seed = 3
    x = synth.tokens(shape.hidden, seed, 4, 0)
    stack = {"seed": seed, "layers": LAYERS, "x_attempt": 0, "router_attempts": [], "ids_t4": [],
             "distinct_t4": [], "min_gap_over_bound": []}
    for layer in range(LAYERS):
        xin = oracle.rmsnorm_bf16(x)
        for a in range(100000):
            router = synth.router(shape, seed, layer, a)
            ro = oracle.route(shape, router, xin)
            if margins_ok(ro, shape.top_k) and disjoint(ro["ids"]):
                break
        used = sorted(set(ro["ids"].reshape(-1).tolist())) + [shape.num_experts]
        experts = {e: synth.expert(shape, seed, layer, e) for e in used}
        y, _ = oracle.moe_layer(shape, router, experts, xin, trace=False)
        x = oracle.residual_bf16(x, y)
        stack["router_attempts"].append(a)
        stack["ids_t4"].append(ro["ids"].tolist())
        stack["distinct_t4"].append(len(used))
        stack["min_gap_over_bound"].append(float(min(_gap_ratio(ro, t) for t in range(4))))
        print(f"layer {layer}: router attempt {a}, rms(x) {np.sqrt(np.mean(oracle.bf16_decode(x).astype(np.float64) ** 2)):.1f}"
              f" ({time.time() - t0:.1f}s)", flush=True)
    stack["final_x_t4_bf16_sha"] = __import__("hashlib").sha256(x.tobytes()).hexdigest()
    man["stack"] = stack

    # FP8 LM head, 4 tokens; argmax margins
    V, H, hseed = synth.HEAD_VOCAB, 2560, 4
    Wq = np.empty((V, H), dtype=np.uint8)
    s = np.empty(V, dtype=np.float32)
    step = 16384
    for r0 in range(0, V, step):
        n = min(step, V - r0)
        Wq[r0:r0 + n], s[r0:r0 + n] = oracle.head_quantize(synth.head_weights(V, H, hseed, r0, n))
    print(f"head quantised ({time.time() - t0:.1f}s)", flush=True)
    for a in range(1000):
        xh = synth.tokens(H, hseed, 4, a)
        lg, bd, am = oracle.head_logits(Wq, s, xh)
        if all(oracle.argmax_margin_ok(lg[t], bd[t]) for t in range(4)):
            break
    man["head"] = {"seed": hseed, "vocab": V, "hidden": H, "x_attempt": a, "argmax": am.tolist(),
                   "top_logits": [float(lg[t, am[t]]) for t in range(4)]}
    print(f"head done ({time.time() - t0:.1f}s)", flush=True)
    with open(OUT, "w") as f:
        json.dump(man, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
