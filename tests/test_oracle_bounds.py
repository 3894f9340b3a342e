"""Pins of the oracle's floating-point error bounds and of the margin rule built on them (CPU only).

The oracle reports, next to each fp64 router logit and LM-head logit, a bound on the error of ANY
fp32 evaluation of the same dot product: gamma_(H-1) * sum |p| with gamma_n = n u / (1 - n u),
u = 2^-24 (the classical bound for a sum of H terms rounded in any order), plus, for the FP8 head,
one more rounding of the final multiply by the row scale.  These bounds decide which seeds count as
well posed (the margin rule) and are the whole tolerance of the GPU logit comparisons, so they are
pinned from both sides here:

  sound  -- fp32 evaluations of the same products in several summation orders (natural, reversed,
            pairwise tree, random permutations, and the router kernel's order: per-lane sequential
            sums over interleaved 8-element units, then a 64-lane tree) all land within the bound;
  tight  -- on an adversarial input, whose every fp32 addition rounds the same way (a 1 followed by
            terms of half an ulp of 1, which round to even), the natural-order error reaches at
            least half the bound; a bound 16 times too loose fails this.

The margin helpers are pinned by hand cases: a gap exactly equal to the bound sum is not a
margin, and a failing pair at rank 3 of a top-8 is caught.
"""
import numpy as np
import pytest

import oracle
import synth

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


# ---- fp32 summation orders over the rows of a product matrix P [rows][n] (exact fp32 products) ---

def sum_natural(P):
    return np.add.accumulate(P.astype(np.float32), axis=1, dtype=np.float32)[:, -1]


def sum_reversed(P):
    return sum_natural(P[:, ::-1])


def sum_pairwise(P):
    P = P.astype(np.float32)
    n = 1 << int(np.ceil(np.log2(P.shape[1])))
    Q = np.zeros((P.shape[0], n), dtype=np.float32)
    Q[:, :P.shape[1]] = P
    while Q.shape[1] > 1:
        Q = (Q[:, 0::2] + Q[:, 1::2]).astype(np.float32)
    return Q[:, 0]


def sum_permuted(P, rng):
    return sum_natural(P[:, rng.permutation(P.shape[1])])


def sum_router_kernel_order(P):
    """Lane l of a 64-lane wave accumulates, in order, the 8-element units l, l + 64, l + 128, ...;
    the 64 lane partials are then summed by a pairwise tree over lane index."""
    rows, n = P.shape
    P = P.astype(np.float32).reshape(rows, n // 8, 8)
    lanes = np.zeros((rows, 64), dtype=np.float32)
    for u in range(n // 8):
        for e in range(8):
            lanes[:, u % 64] = (lanes[:, u % 64] + P[:, u, e]).astype(np.float32)
    return sum_pairwise(lanes)


def bf16_products(router, xf):
    """Exact fp32 products of bf16 router rows and a bf16 activation (8 + 8 significant bits)."""
    W = oracle.bf16_decode(router).astype(np.float32)
    return (W * xf[None, :]).astype(np.float32)


ORDERS = {"natural": sum_natural, "reversed": sum_reversed, "pairwise": sum_pairwise,
          "router_kernel": sum_router_kernel_order}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_router_bounds_hold_for_every_summation_order(seed):
    shape = synth.FLASH
    router = synth.router(shape, seed)[:96]
    x = synth.tokens(shape.hidden, seed, 1)
    small = synth.Shape(shape.hidden, 96, shape.top_k, 0, shape.inter)
    ro = oracle.route(small, router, x)
    P = bf16_products(router, oracle.bf16_decode(x[0]))
    # the products are exact, so their fp64 sum is the oracle's logit to within fp64 rounding
    assert np.abs(P.astype(np.float64).sum(axis=1) - ro["logits"][0]).max() <= 1e-12 * np.abs(P).sum(axis=1).max()
    rng = np.random.default_rng(seed)
    results = {name: f(P) for name, f in ORDERS.items()}
    for i in range(4):
        results[f"permutation{i}"] = sum_permuted(P, rng)
    for name, s in results.items():
        err = np.abs(s.astype(np.float64) - ro["logits"][0])
        assert (err <= ro["bounds"][0]).all(), name
    # the bound is gamma_(H-1) * sum |p|
    want = gamma(shape.hidden - 1) * np.abs(P.astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(ro["bounds"][0], want, rtol=1e-12)


def adversarial_router(H):
    """Row 0 of the router is 1 followed by 2^-12 everywhere, x is 1 followed by 2^-12: the products
    are 1 and H - 1 terms of 2^-24, half an ulp of 1, so every natural-order fp32 addition rounds
    back to 1 (ties to even) and the error is (H - 1) 2^-24."""
    one, small = 0x3F80, 0x3980  # bf16 bits of 1.0 and 2^-12
    router = np.full((8, H), small, dtype=np.uint16)
    router[:, 0] = one
    x = np.full((1, H), small, dtype=np.uint16)
    x[0, 0] = one
    return router, x


def test_router_bound_is_tight_on_an_adversarial_sum():
    H = 2560
    router, x = adversarial_router(H)
    ro = oracle.route(synth.Shape(H, 8, 2, 0, 64), router, x)
    s = sum_natural(bf16_products(router, oracle.bf16_decode(x[0])))
    assert s[0] == np.float32(1.0)
    err = abs(float(s[0]) - ro["logits"][0, 0])
    assert err == pytest.approx((H - 1) * U, rel=1e-12)
    assert err <= ro["bounds"][0, 0] <= 2 * err


def test_head_bounds_hold_for_every_summation_order():
    V, H = 64, 2560
    W = synth.head_weights(V, H, seed=5, rows=V)
    Wq, s = oracle.head_quantize(W)
    x = synth.tokens(H, 5, 2)
    lg, bd, _ = oracle.head_logits(Wq, s, x)
    table = oracle.e4m3_table()
    Wd = table[Wq].astype(np.float32)  # E4M3 values are exact in fp32
    rng = np.random.default_rng(5)
    for t in range(2):
        P = (Wd * oracle.bf16_decode(x[t])[None, :]).astype(np.float32)  # 4 x 8 significant bits: exact
        orders = {name: f(P) for name, f in ORDERS.items()}
        orders["permutation"] = sum_permuted(P, rng)
        for name, acc in orders.items():
            got = (acc * s).astype(np.float32).astype(np.float64)  # the final multiply by the row scale
            assert (np.abs(got - lg[t]) <= bd[t]).all(), (t, name)
        want = s.astype(np.float64) * gamma(H - 1) * np.abs(P.astype(np.float64)).sum(axis=1) + U * np.abs(lg[t])
        np.testing.assert_allclose(bd[t], want, rtol=1e-12)


def test_head_bound_is_tight_on_an_adversarial_sum():
    """Row 0: code 1.0 then the smallest subnormal 2^-9; x: 1.0 then 2^-15; scale 1.  Products are 1
    and 2^-24, so the natural-order fp32 sum stays 1 and its error reaches the bound."""
    H = 2560
    Wq = np.full((1, H), 0x01, dtype=np.uint8)
    Wq[0, 0] = 0x38
    x = np.full((1, H), 0x3800, dtype=np.uint16)  # bf16 2^-15
    x[0, 0] = 0x3F80
    lg, bd, _ = oracle.head_logits(Wq, np.ones(1, dtype=np.float32), x)
    P = (oracle.e4m3_table()[Wq].astype(np.float32) * oracle.bf16_decode(x[0])[None, :]).astype(np.float32)
    s = sum_natural(P)
    assert s[0] == np.float32(1.0)
    err = abs(float(s[0]) - lg[0, 0])
    assert err <= bd[0, 0] <= 2 * err


def test_bf16_head_bounds_hold_and_are_tight():
    V, H = 32, 1024
    Wb = synth.router(synth.Shape(H, V, 2, 0, 64), 3)
    x = synth.tokens(H, 3, 1)
    lg, bd, _ = oracle.head_logits_bf16(Wb, x)
    P = bf16_products(Wb, oracle.bf16_decode(x[0]))
    for name, f in ORDERS.items():
        assert (np.abs(f(P).astype(np.float64) - lg[0]) <= bd[0]).all(), name
    router, xa = adversarial_router(H)
    lg, bd, _ = oracle.head_logits_bf16(router, xa)
    err = abs(float(sum_natural(bf16_products(router, oracle.bf16_decode(xa[0])))[0]) - lg[0, 0])
    assert err <= bd[0, 0] <= 2 * err


# ---- margin helpers ----------------------------------------------------------------------------

def test_topk_margin_requires_a_strict_gap_above_the_bound_sum():
    k = 8
    logits = np.array([10.0 - i for i in range(12)])
    bounds = np.full(12, 0.25)
    assert oracle.topk_margin_ok(logits, bounds, k)
    # gap exactly equal to the sum of the two bounds: not a margin
    b = bounds.copy()
    b[3] = b[4] = 0.5
    assert not oracle.topk_margin_ok(logits, b, k)
    b[4] = 0.4999
    assert oracle.topk_margin_ok(logits, b, k)
    # a failing pair at rank 3 (between the 3rd and 4th selected logits)
    lg = logits.copy()
    lg[3] = lg[2] - 0.3
    assert not oracle.topk_margin_ok(lg, bounds, k)
    # the pair between rank k and k + 1 counts; pairs after it do not
    lg = logits.copy()
    lg[8] = lg[7] - 0.5
    assert not oracle.topk_margin_ok(lg, bounds, k)
    lg = logits.copy()
    lg[10] = lg[9] - 0.1
    assert oracle.topk_margin_ok(lg, bounds, k)


def test_topk_margin_orders_by_value_then_index():
    # shuffled positions: the helper must order by (value desc, index asc) before taking gaps
    rng = np.random.default_rng(0)
    base = np.array([10.0 - i for i in range(12)])
    perm = rng.permutation(12)
    assert oracle.topk_margin_ok(base[perm], np.full(12, 0.25), 8)
    tied = base[perm].copy()
    tied[perm.tolist().index(5)] = 10.0 - 4  # equal to rank 4: zero gap
    assert not oracle.topk_margin_ok(tied, np.full(12, 0.25), 8)


def test_argmax_margin_hand_cases():
    lg = np.array([1.0, 3.0, 2.0, 2.875])  # exact binary fractions: the gap is exactly 0.125
    assert not oracle.argmax_margin_ok(lg, np.full(4, 0.0625))  # gap == 0.0625 + 0.0625
    assert oracle.argmax_margin_ok(lg, np.full(4, 0.0624))
    assert oracle.argmax_margin_ok(np.array([5.0, 1.0]), np.zeros(2))
    assert not oracle.argmax_margin_ok(np.array([5.0, 5.0]), np.zeros(2))  # a tie is never a margin
