"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a temporary copy of ``oracle/moe_oracle.c`` (a dropped
term, a wrong sign, index, bias or block size, a transposed operand, the wrong tie rule), builds
it with gcc, and requires that at least one of the independent pin checks fails on it.  The
unmodified source must pass every check.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_layer import brute_force_layer, tiny_case

MUTANTS = {
    "nibble_order": ("(k & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 0xF)",
                     "(k & 1) ? (uint32_t)(byte & 0xF) : (uint32_t)(byte >> 4)"),
    "scale_block_64": ("(size_t)(K / 32) + (size_t)(k / 32)]]", "(size_t)(K / 32) + (size_t)(k / 64)]]"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e8m0_bias": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 128)"),
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_round_half_away": ("nearbyint(a / quantum)", "round(a / quantum)"),
    "bf16_truncate": ("v.u + 0x7FFFu + ((v.u >> 16) & 1u)", "v.u"),
    "topk_ties_high_index": ("if (best < 0 || logits[e] > logits[best]) best = e;",
                             "if (best < 0 || logits[e] >= logits[best]) best = e;"),
    "softmax_unnormalised": ("for (int r = 0; r < k; ++r) w[r] /= z;",
                             "for (int r = 0; r < k; ++r) w[r] /= (double)k;"),
    "act_scale_240": ("amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 240.0f : 1.0f"),
    "gate_up_swapped": ("ag += mx_elem(w13, w13s, H, i, c) * xh[c];\n                    au += mx_elem(w13, w13s, H, I + i, c) * xh[c];",
                        "ag += mx_elem(w13, w13s, H, I + i, c) * xh[c];\n                    au += mx_elem(w13, w13s, H, i, c) * xh[c];"),
    "silu_sign": ("G[i] / (1.0 + exp(-G[i]))", "G[i] / (1.0 + exp(G[i]))"),
    "down_unquantised_h": ("hh[i] = g_e4m3[qh[i]];", "hh[i] = (double)h[i] / sh;"),
    "down_k_reversed": ("mx_elem(w2, w2s, I, r, i)", "mx_elem(w2, w2s, I, r, I - 1 - i)"),
    "combine_unweighted": ("acc += w[j] * d[(size_t)j * H + r];", "acc += d[(size_t)j * H + r];"),
    "shared_dropped": ("if (S) acc += d[(size_t)k * H + r];", "(void)S;"),
    "rmsnorm_eps": ("sqrt(ss / (double)H + 1e-6)", "sqrt(ss / (double)H + 1e-2)"),
    "residual_sign": ("oracle_bf16_decode(x[i]) + y[i]", "oracle_bf16_decode(x[i]) - y[i]"),
    "head_scale_dropped": ("double lg = (double)scale[r] * acc;", "double lg = acc;"),
    "head_ties_high_index": ("if (lg > bestv) { bestv = lg; best = r; }", "if (lg >= bestv) { bestv = lg; best = r; }"),
    "router_bound_gamma_x16": ("if (bounds) bounds[e] = gamma * mag;", "if (bounds) bounds[e] = 16.0 * gamma * mag;"),
    "head_bound_gamma_x16": ("(double)scale[r] * gamma * mag + 0x1p-24 * fabs(lg);",
                             "(double)scale[r] * 16.0 * gamma * mag + 0x1p-24 * fabs(lg);"),
    "bf16_head_bound_gamma_x16": ("if (bounds) bounds[(size_t)t * V + r] = gamma * mag;",
                                  "if (bounds) bounds[(size_t)t * V + r] = 16.0 * gamma * mag;"),
    "router_bound_dropped": ("if (bounds) bounds[e] = gamma * mag;", "if (bounds) bounds[e] = 0.0;"),
}


def _checks():
    """Fast pin checks; returns the names of those that fail."""
    failed = []

    def run(name, fn):
        try:
            fn()
        except AssertionError:
            failed.append(name)

    def codecs():
        table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        assert [oracle.e2m1_decode(c) for c in range(8)] == table
        assert [oracle.e8m0_decode(b) for b in (121, 127)] == [2.0 ** -6, 1.0]
        ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        got = np.array([oracle.e4m3_decode(c) for c in range(256)])
        ok = ~np.isnan(ref)
        assert (got[ok] == ref[ok]).all()
        f = np.random.default_rng(0).uniform(-460, 460, 1 << 18).astype(np.float32)
        f = np.concatenate([f, (ref[1:0x7E] + ref[2:0x7F]).astype(np.float32) / 2])
        want = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (oracle.e4m3_encode(f) == want).all()
        g = np.random.default_rng(1).standard_normal(1 << 18).astype(np.float32)
        wb = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (oracle.bf16_encode(g) == wb).all()

    def layer():
        for seed in range(3):
            shape = synth.TINY
            router, x, experts = tiny_case(shape, seed)
            y, tr = oracle.moe_layer(shape, router, experts, x)
            ref = brute_force_layer(shape, router, experts, x[0])
            assert list(tr["ids"][0]) == list(ref["ids"])
            np.testing.assert_allclose(tr["w"][0], ref["w"], rtol=1e-12)
            assert np.abs(y[0] - ref["y"]).max() <= 1e-6 * np.abs(ref["y"]).max()

    def zero_input():
        shape = synth.TINY
        router, _, experts = tiny_case(shape, 5)
        y, tr = oracle.moe_layer(shape, router, experts, np.zeros((1, shape.hidden), dtype=np.uint16))
        assert (y == 0).all() and list(tr["ids"][0]) == list(range(shape.top_k))

    def stack():
        import torch.nn.functional as F
        x = synth.tokens(2560, 3, 2)
        ours = oracle.rmsnorm_bf16(x)
        ref = F.rms_norm(torch.from_numpy(oracle.bf16_decode(x).astype(np.float64)), (2560,), eps=1e-6)
        ref = ref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (ours == ref).mean() > 0.9999
        y = np.random.default_rng(2).standard_normal((2, 2560)).astype(np.float32) * 100
        r = (torch.from_numpy(oracle.bf16_decode(x)) + torch.from_numpy(y)).to(torch.bfloat16)
        assert (oracle.residual_bf16(x, y) == r.view(torch.int16).numpy().view(np.uint16)).all()

    def head():
        V, H = 400, 256
        W = synth.head_weights(V, H, seed=9, rows=V)
        x = synth.tokens(H, 9, 1)
        Wq, s = oracle.head_quantize(W)
        lg, _, am = oracle.head_logits(Wq, s, x)
        deq = torch.from_numpy(Wq).view(torch.float8_e4m3fn).double().numpy() * s.astype(np.float64)[:, None]
        np.testing.assert_allclose(lg[0], deq @ oracle.bf16_decode(x[0]).astype(np.float64), rtol=1e-12)
        W2 = W.copy()
        W2[V - 1] = W[int(am[0])]
        Wq2, s2 = oracle.head_quantize(W2)
        _, _, am2 = oracle.head_logits(Wq2, s2, x, want_logits=False, want_bounds=False)
        assert am2[0] == am[0]

    def bounds():
        import test_oracle_bounds as tb
        tb.test_router_bounds_hold_for_every_summation_order(0)
        tb.test_router_bound_is_tight_on_an_adversarial_sum()
        tb.test_head_bound_is_tight_on_an_adversarial_sum()
        tb.test_bf16_head_bounds_hold_and_are_tight()

    for name, fn in (("codecs", codecs), ("layer", layer), ("zero_input", zero_input), ("stack", stack),
                     ("head", head), ("bounds", bounds)):
        run(name, fn)
    return failed


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, c, "-o", path, "-lm"])


def test_unmodified_oracle_passes_every_check():
    assert _checks() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SRC).read()
    before, after = MUTANTS[name]
    assert src.count(before) == 1, name
    path = os.path.join(tmp_path, f"libmut_{name}.so")
    _build(src.replace(before, after), path)
    with oracle.using(path):
        failed = _checks()
    assert failed, f"mutant {name} passed every pin check"
