"""Pins for the oracle's FP8 LM head and the stack steps (CPU only)."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth


def test_head_quantize_matches_torch_cast():
    W = synth.head_weights(4096, 2560, seed=4, rows=512)
    Wq, s = oracle.head_quantize(W)
    amax = np.abs(W).max(axis=1).astype(np.float32)
    s_ref = amax / np.float32(448)
    assert (s == s_ref).all()
    q_ref = torch.from_numpy((W / s_ref[:, None]).astype(np.float32)).to(torch.float8_e4m3fn)
    assert (Wq == q_ref.view(torch.uint8).numpy()).all()
    # the row maximum maps to the largest code
    assert (np.abs(Wq.astype(np.int16) & 0x7F).max(axis=1) == 0x7E).all()


def test_head_zero_row_scale_is_one():
    W = np.zeros((3, 64), dtype=np.float32)
    W[1, 5] = -3.0
    Wq, s = oracle.head_quantize(W)
    assert s[0] == 1.0 and s[2] == 1.0 and (Wq[0] == 0).all()
    assert Wq[1, 5] == 0xFE


def _dequant(Wq, s):
    vals = torch.from_numpy(Wq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals * s.astype(np.float64)[:, None]


def test_head_logits_match_blas_and_argmax_brute_force():
    V, H = 3000, 2560
    W = synth.head_weights(V, H, seed=4, rows=V)
    Wq, s = oracle.head_quantize(W)
    x = synth.tokens(H, 4, 4)
    lg, bd, am = oracle.head_logits(Wq, s, x)
    xf = oracle.bf16_decode(x).astype(np.float64)
    dense = _dequant(Wq, np.ones(V, dtype=np.float32)) @ xf.T  # BLAS GEMV, unscaled
    ref = (dense * s.astype(np.float64)[:, None]).T
    np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-12)
    for t in range(4):
        m = lg[t].max()
        assert am[t] == np.flatnonzero(lg[t] == m)[0]
        assert (bd[t] > 0).all()


def test_head_duplicate_row_keeps_lowest_index():
    V, H = 500, 256
    W = synth.head_weights(V, H, seed=9, rows=V)
    x = synth.tokens(H, 9, 1)
    Wq, s = oracle.head_quantize(W)
    _, _, am = oracle.head_logits(Wq, s, x, want_logits=False, want_bounds=False)
    r = int(am[0])
    W2 = W.copy()
    W2[V - 1] = W[r]
    Wq2, s2 = oracle.head_quantize(W2)
    _, _, am2 = oracle.head_logits(Wq2, s2, x, want_logits=False, want_bounds=False)
    assert am2[0] == r
    # and the copy placed before the original wins
    W3 = W.copy()
    W3[0] = W[r]
    Wq3, s3 = oracle.head_quantize(W3)
    _, _, am3 = oracle.head_logits(Wq3, s3, x, want_logits=False, want_bounds=False)
    assert am3[0] == 0 or r == 0


def _bf16_bits(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_head_matches_blas_and_argmax_brute_force():
    V, H = 2000, 2560
    Wb = _bf16_bits(synth.head_weights(V, H, seed=6, rows=V))
    x = synth.tokens(H, 6, 3)
    lg, bd, am = oracle.head_logits_bf16(Wb, x)
    dense = oracle.bf16_decode(Wb).astype(np.float64) @ oracle.bf16_decode(x).astype(np.float64).T
    np.testing.assert_allclose(lg, dense.T, rtol=1e-12, atol=1e-12)
    for t in range(3):
        assert am[t] == np.flatnonzero(lg[t] == lg[t].max())[0]
        assert (bd[t] > 0).all()


def test_bf16_head_equals_fp8_head_on_power_of_two_scales():
    """Rows that are E4M3 values times a power of two are exact in bf16, and both heads then sum the
    same exact products: the BF16 oracle must return the FP8 oracle's logits bit for bit."""
    V, H = 700, 2560
    Wq, s = oracle.head_quantize(synth.head_weights(V, H, seed=8, rows=V))
    s2 = np.exp2(np.round(np.log2(s))).astype(np.float32)  # a power of two near each row scale
    vals = torch.from_numpy(Wq).view(torch.float8_e4m3fn).to(torch.float32).numpy() * s2[:, None]
    Wb = _bf16_bits(vals)
    assert ((Wb.astype(np.uint32) << 16).view(np.float32) == vals).all()  # exact in bf16
    x = synth.tokens(H, 8, 2)
    lg8, _, am8 = oracle.head_logits(Wq, s2, x)
    lgb, _, amb = oracle.head_logits_bf16(Wb, x)
    assert (lg8 == lgb).all() and (am8 == amb).all()


def test_fp8_head_halves_bf16_reads():
    V, H = synth.HEAD_VOCAB, 2560
    assert V * H == 402_391_040 and 2 * V * H == 804_782_080
    assert V * 4 == 628_736


def test_rmsnorm_matches_torch_rms_norm():
    x = synth.tokens(2560, 3, 4)
    ours = oracle.rmsnorm_bf16(x)
    xf = torch.from_numpy(oracle.bf16_decode(x).astype(np.float64))
    ref = F.rms_norm(xf, (2560,), eps=1e-6).to(torch.float32).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).mean() > 0.9999
    assert np.abs(oracle.bf16_decode(ours) - oracle.bf16_decode(ref)).max() <= 2.0 ** -7 * 4


def test_rmsnorm_constant_vector_closed_form():
    H = 256
    for c in (1.0, 2.0, -0.5, 1024.0):
        x = oracle.bf16_encode(np.full((1, H), c, dtype=np.float32))
        out = oracle.bf16_decode(oracle.rmsnorm_bf16(x))
        want = np.float32(c / np.sqrt(c * c + 1e-6))
        assert (out == oracle.bf16_decode(oracle.bf16_encode(np.array([want])))).all()


def test_rmsnorm_power_of_two_invariance():
    x = synth.tokens(2560, 11, 2)
    xf = oracle.bf16_decode(x)
    x4 = oracle.bf16_encode(xf * np.float32(4.0))  # exact: scaling bf16 by 4
    a, b = oracle.rmsnorm_bf16(x), oracle.rmsnorm_bf16(x4)
    # eps is negligible against mean(x^2) ~ 1, so both normalise to (nearly) the same vector
    assert (a == b).mean() > 0.999


def test_residual_matches_torch():
    x = synth.tokens(2560, 12, 2)
    y = (np.random.default_rng(1).standard_normal((2, 2560)) * 300).astype(np.float32)
    ours = oracle.residual_bf16(x, y)
    ref = (torch.from_numpy(oracle.bf16_decode(x)) + torch.from_numpy(y)).to(torch.bfloat16)
    assert (ours == ref.view(torch.int16).numpy().view(np.uint16)).all()


def test_mtp_accept_longest_matching_prefix():
    # 4 verify positions, 3 drafts: the drafts are accepted up to the first mismatch only
    assert oracle.mtp_accept([5, 7, 9, 11], [5, 7, 9]) == 3
    assert oracle.mtp_accept([5, 7, 9, 11], [6, 7, 9]) == 0
    assert oracle.mtp_accept([5, 7, 9, 11], [5, 8, 9]) == 1
    assert oracle.mtp_accept([5, 7, 9, 11], [5, 7, 10]) == 2
    assert oracle.mtp_accept([5, 7, 9, 11], [4, 7, 9]) == 0  # later matches do not count
    assert oracle.mtp_accept([3, 1], [3]) == 1 and oracle.mtp_accept([3, 1], [2]) == 0
    assert oracle.mtp_accept([3], []) == 0
