"""Pins for the oracle's MoE layer (CPU only).

The oracle walks the selected experts in rank order with fp64 loops.  These tests reach the same
quantities another way -- dense dequantised matrices for all experts, numpy matmuls, torch's
FP8 codec, a full stable sort, int64 exact block sums -- plus invariants whose value is fixed by
the mathematics (softmax sums to one, zero input gives zero output, power-of-two scaling is exact,
tokens are independent, expert labels do not matter).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def dense_mx(codes, scl, K):
    """Dense fp64 matrix of an MXFP4 tensor (codes [rows][K/2], scales [rows][K/32])."""
    lo = codes & 0xF
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], K)
    return E2M1[nib] * np.repeat(np.exp2(scl.astype(np.float64) - 127), 32, axis=1)


def torch_e4m3(v32):
    """(codes, decoded fp64) of an fp32 vector via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy(), t.to(torch.float64).numpy()


def brute_force_layer(shape, router, experts_all, x_bf16):
    """Dense reference of one layer for one token: every expert computed, routing as a mask."""
    H, I, E, k = shape.hidden, shape.inter, shape.num_experts, shape.top_k
    xf = oracle.bf16_decode(x_bf16).astype(np.float32)
    Wr = oracle.bf16_decode(router).astype(np.float64)
    logits = Wr @ xf.astype(np.float64)
    order = np.lexsort((np.arange(E), -logits))
    ids = order[:k]
    mask = np.zeros(E)
    z = np.exp(logits[ids] - logits[ids[0]])
    mask[ids] = z / z.sum()
    amax = np.float32(np.abs(xf).max())
    sx = amax / np.float32(448) if amax > 0 else np.float32(1)
    qx, xh = torch_e4m3(xf / sx)
    d_all = np.zeros((E + shape.num_shared, H))
    h_all = np.zeros((E + shape.num_shared, I), dtype=np.float32)
    for e in range(E + shape.num_shared):
        t = experts_all[e]
        W13 = dense_mx(t["w13"], t["w13_s"], H)
        gu = float(sx) * (W13 @ xh)
        g, u = gu[:I], gu[I:]
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        ah = np.float32(np.abs(h).max())
        sh = ah / np.float32(448) if ah > 0 else np.float32(1)
        _, hh = torch_e4m3(h / sh)
        d_all[e] = float(sh) * (dense_mx(t["w2"], t["w2_s"], I) @ hh)
        h_all[e] = h
    y = mask @ d_all[:E] + (d_all[E] if shape.num_shared else 0.0)
    return dict(logits=logits, ids=ids, w=mask[ids], sx=sx, qx=qx, d=d_all, h=h_all, y=y)


def tiny_case(shape=synth.TINY, seed=0, attempt=0, T=1):
    router = synth.router(shape, seed)
    x = synth.tokens(shape.hidden, seed, T, attempt)
    experts = {e: synth.expert(shape, seed, 0, e) for e in range(shape.num_experts + shape.num_shared)}
    return router, x, experts


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_layer_matches_dense_brute_force(seed):
    shape = synth.TINY
    router, x, experts = tiny_case(shape, seed)
    y, tr = oracle.moe_layer(shape, router, experts, x)
    ref = brute_force_layer(shape, router, experts, x[0])
    np.testing.assert_allclose(tr["logits"][0], ref["logits"], rtol=1e-13, atol=1e-13)
    assert list(tr["ids"][0]) == list(ref["ids"])
    np.testing.assert_allclose(tr["w"][0], ref["w"], rtol=1e-14)
    assert tr["sx"][0] == ref["sx"]
    assert (tr["qx"][0] == ref["qx"]).all()
    slots = list(tr["ids"][0]) + [shape.num_experts]
    for j, e in enumerate(slots):
        np.testing.assert_allclose(tr["h"][0, j], ref["h"][e], rtol=1e-6, atol=0)
        np.testing.assert_allclose(tr["d"][0, j], ref["d"][e], rtol=1e-12, atol=1e-9)
    err = np.abs(y[0] - ref["y"]).max() / np.abs(ref["y"]).max()
    assert err < 1e-7  # fp32 output rounding only


def test_block_sums_are_exact_int64():
    # Each term E2M1 * 2^(b-127) * E4M3 is (2*E2M1) * (E4M3 * 2^9) * 2^(b-121) * 2^-16 with the
    # first three factors integers; their int64 sum times 2^-16 is the exact dot product.
    shape = synth.FLASH
    seed = 1
    router = synth.router(shape, seed)
    x = synth.tokens(shape.hidden, seed, 1)
    ro = oracle.route(shape, router, x)
    e0 = int(ro["ids"][0][0])
    ex = {int(e): synth.expert(shape, seed, 0, int(e)) for e in list(ro["ids"][0]) + [shape.num_experts]}
    y, tr = oracle.moe_layer(shape, router, ex, x)
    c2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], dtype=np.int64)
    t = ex[e0]
    H, I = shape.hidden, shape.inter
    nib = np.stack([t["w13"] & 0xF, t["w13"] >> 4], axis=-1).reshape(2 * I, H)
    shift = np.repeat(t["w13_s"].astype(np.int64) - 121, 32, axis=1)
    assert shift.min() >= 0 and shift.max() <= 4
    _, xh = torch_e4m3(np.zeros(1, dtype=np.float32))  # warm torch
    xh = np.array([oracle.e4m3_decode(int(c)) for c in tr["qx"][0]])
    x9 = np.rint(xh * 512).astype(np.int64)
    assert (x9 == xh * 512).all()
    exact = (c2[nib] * x9[None, :] * (np.int64(1) << shift)).sum(axis=1)
    assert np.abs(exact).max() < 2 ** 52
    sx = float(tr["sx"][0])
    want = sx * (exact.astype(np.float64) * 2.0 ** -16)
    assert (tr["g"][0, 0] == want[:I]).all()
    assert (tr["u"][0, 0] == want[I:]).all()


def test_route_matches_stable_sort_and_fsum():
    shape = synth.FLASH
    for seed in range(3):
        router = synth.router(shape, seed)
        x = synth.tokens(shape.hidden, seed, 2)
        ro = oracle.route(shape, router, x)
        Wr = oracle.bf16_decode(router).astype(np.float64)
        for t in range(2):
            xf = oracle.bf16_decode(x[t]).astype(np.float64)
            for e in range(0, shape.num_experts, 37):
                p = Wr[e] * xf
                exact = math.fsum(p)
                assert abs(ro["logits"][t, e] - exact) <= 2560 * 2.0 ** -53 * np.abs(p).sum()
            l = ro["logits"][t]
            order = np.lexsort((np.arange(l.size), -l))
            assert list(ro["ids"][t]) == list(order[: shape.top_k])
            assert abs(ro["w"][t].sum() - 1.0) < 1e-15
            assert (np.diff(ro["w"][t]) <= 0).all()


def test_zero_input_gives_zero_output_and_lowest_ids():
    shape = synth.TINY
    router, _, experts = tiny_case(shape, 5)
    x = np.zeros((1, shape.hidden), dtype=np.uint16)
    y, tr = oracle.moe_layer(shape, router, experts, x)
    assert (y == 0).all()
    assert list(tr["ids"][0]) == list(range(shape.top_k))
    assert (tr["w"][0] == 1.0 / shape.top_k).all()
    assert tr["sx"][0] == 1.0 and (tr["sh"][0] == 1.0).all()


def test_single_expert_k1_no_shared_is_that_expert():
    shape = Shape(hidden=256, num_experts=16, top_k=1, num_shared=0, inter=64)
    router, x, experts = tiny_case(shape, 3)
    y, tr = oracle.moe_layer(shape, router, experts, x)
    assert tr["w"][0, 0] == 1.0
    assert (y[0] == tr["d"][0, 0].astype(np.float32)).all()
    ref = brute_force_layer(shape, router, experts, x[0])
    np.testing.assert_allclose(tr["d"][0, 0], ref["d"][tr["ids"][0, 0]], rtol=1e-12, atol=1e-9)


def test_down_scale_plus_one_doubles_that_expert_exactly():
    shape = synth.TINY
    router, x, experts = tiny_case(shape, 2)
    y0, tr0 = oracle.moe_layer(shape, router, experts, x)
    r = 1
    e = int(tr0["ids"][0, r])
    bumped = dict(experts)
    bumped[e] = dict(experts[e], w2_s=experts[e]["w2_s"] + 1)
    y1, tr1 = oracle.moe_layer(shape, router, bumped, x)
    assert (tr1["d"][0, r] == 2.0 * tr0["d"][0, r]).all()
    others = [j for j in range(shape.top_k + 1) if j != r]
    assert (tr1["d"][0, others] == tr0["d"][0, others]).all()
    delta = y1[0].astype(np.float64) - y0[0].astype(np.float64)
    np.testing.assert_allclose(delta, tr0["w"][0, r] * tr0["d"][0, r], rtol=1e-5,
                               atol=1e-6 * np.abs(y0).max())


def test_tokens_are_independent():
    shape = synth.TINY
    router, x, experts = tiny_case(shape, 4, T=4)
    y4, tr4 = oracle.moe_layer(shape, router, experts, x)
    for t in range(4):
        y1, tr1 = oracle.moe_layer(shape, router, experts, x[t:t + 1])
        assert (y1[0] == y4[t]).all()
        assert (tr1["ids"][0] == tr4["ids"][t]).all()


def test_expert_relabeling_leaves_output_unchanged():
    shape = synth.TINY
    router, x, experts = tiny_case(shape, 6)
    y0, tr0 = oracle.moe_layer(shape, router, experts, x)
    perm = np.random.default_rng(0).permutation(shape.num_experts)  # new label p holds old perm[p]
    router_p = router[perm]
    experts_p = {p: experts[int(perm[p])] for p in range(shape.num_experts)}
    experts_p[shape.num_experts] = experts[shape.num_experts]
    y1, tr1 = oracle.moe_layer(shape, router_p, experts_p, x)
    assert list(perm[tr1["ids"][0]]) == list(tr0["ids"][0])
    assert (y1 == y0).all()


def test_blas_gemv_special_case_for_one_expert():
    # Dequantised dense matrix times the decoded activation through numpy's matmul (BLAS).
    shape = synth.FLASH
    router = synth.router(shape, 1)
    x = synth.tokens(shape.hidden, 1, 1)
    ro = oracle.route(shape, router, x)
    ex = {int(e): synth.expert(shape, 1, 0, int(e)) for e in list(ro["ids"][0]) + [shape.num_experts]}
    y, tr = oracle.moe_layer(shape, router, ex, x)
    t = ex[shape.num_experts]
    hh = np.array([oracle.e4m3_decode(int(c)) for c in tr["qh"][0, -1]])
    d = float(tr["sh"][0, -1]) * (dense_mx(t["w2"], t["w2_s"], shape.inter) @ hh)
    np.testing.assert_allclose(tr["d"][0, -1], d, rtol=1e-13, atol=1e-10)
