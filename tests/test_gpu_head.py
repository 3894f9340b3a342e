"""GPU parity of the FP8 LM head (C ABI) against the oracle: logits within the fp32 evaluation
bound the oracle reports, argmax exact (lowest index on ties)."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemv_amd as moe
import oracle
import synth
from gpu_cases import MANIFEST, dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quantised(V, H, seed):
    Wq = np.empty((V, H), dtype=np.uint8)
    s = np.empty(V, dtype=np.float32)
    step = 16384
    for r0 in range(0, V, step):
        n = min(step, V - r0)
        Wq[r0:r0 + n], s[r0:r0 + n] = oracle.head_quantize(synth.head_weights(V, H, seed, r0, n))
    return Wq, s


def _run(Wq, s, x, want_logits=True):
    w = torch.from_numpy(Wq).to(dev())
    sc = torch.from_numpy(s).to(dev())
    h = moe.fp8_head_create(w, sc)
    T = x.shape[0]
    am = torch.full((T,), -1, dtype=torch.int32, device=dev())
    lg = torch.empty((T, Wq.shape[0]), dtype=torch.float32, device=dev()) if want_logits else None
    moe.fp8_head_run(h, to_dev_u16(x), am, lg)
    torch.cuda.synchronize()
    moe.fp8_head_destroy(h)
    return am.cpu().numpy(), None if lg is None else lg.cpu().numpy()


@pytest.mark.parametrize("V,T,H", [(3000, 4, 2560), (64 * 7 + 5, 1, 2560), (1, 2, 2560), (700, 4, 256),
                                   (130, 3, 1024)])
def test_small_head_matches_oracle(V, T, H):
    Wq, s = _quantised(V, H, seed=13)
    x = synth.tokens(H, 13, T)
    lg_o, bd_o, am_o = oracle.head_logits(Wq, s, x)
    am, lg = _run(Wq, s, x)
    assert (np.abs(lg - lg_o) <= bd_o).all()
    for t in range(T):
        if V == 1 or oracle.argmax_margin_ok(lg_o[t], bd_o[t]):
            assert am[t] == am_o[t]


# 1,030 tiles of 64 rows, the last of 37: more tiles than the device's resident workgroups hold, so
# each workgroup walks several tiles (rounds), and the grid sized to those rounds leaves a few
# workgroups one tile fewer.
MULTI_V = 64 * 1029 + 37


@pytest.fixture(scope="module")
def multi_round_head():
    return _quantised(MULTI_V, 2560, seed=13)


def test_multi_round_ragged_head_matches_oracle(multi_round_head):
    """Every logit of a head whose tiles take several rounds, with a ragged last tile, within the
    oracle's fp32 evaluation bound; the argmax exact where it is well posed (1 and 4 tokens)."""
    Wq, s = multi_round_head
    for T in (1, 4):
        x = synth.tokens(2560, 13 + T, T)
        lg_o, bd_o, am_o = oracle.head_logits(Wq, s, x)
        am, lg = _run(Wq, s, x)
        bad = np.argwhere(np.abs(lg - lg_o) > bd_o)
        assert bad.size == 0, f"T={T}: {len(bad)} logits outside the bound, first (token, row) {bad[:3].tolist()}"
        for t in range(T):
            if oracle.argmax_margin_ok(lg_o[t], bd_o[t]):
                assert am[t] == am_o[t], f"T={T} token {t}: {am[t]} against {am_o[t]}"


def test_multi_round_duplicates_lowest_index_wins(multi_round_head):
    """Copies of the winning row spread over rounds and workgroups.  Copies at higher indices (later
    rounds, the ragged last tile) must lose to the original; copies then added at lower indices (the
    same workgroup's earlier rounds, the first tile) must win, the lowest index each time.  Equal rows
    give bit-equal logits (same products in the same order), so only the cross-tile and
    cross-workgroup reductions decide the index."""
    Wq0, s0 = multi_round_head
    x = synth.tokens(2560, 9, 1)
    lg_o, bd_o, am_o = oracle.head_logits(Wq0, s0, x)
    assert oracle.argmax_margin_ok(lg_o[0], bd_o[0]), "fixture: the winner must be well separated"
    r = int(am_o[0])
    tiles, tr = (MULTI_V + 63) // 64, r // 64
    stride = -(-tiles // 3)  # a workgroup's step between tiles when they take three rounds (512 resident)
    higher = sorted(i for i in {MULTI_V - 1, 64 * (tiles - 2) + 63, *(64 * t + 7 for t in (tr + stride, tr + 2 * stride)
                                                                        if t < tiles)} if i > r)
    lower = sorted((i for i in {*(64 * t + 5 for t in (tr - stride, tr - 2 * stride) if t >= 0), 3} if i < r),
                   reverse=True)
    assert len(higher) >= 2 and len(lower) >= 2, (r, higher, lower)
    Wq, s = Wq0.copy(), s0.copy()
    for i in higher:
        Wq[i], s[i] = Wq0[r], s0[r]
    am, _ = _run(Wq, s, x, want_logits=False)
    assert am[0] == r, f"copies at {higher} of row {r}: got {am[0]}"
    for i in lower:
        Wq[i], s[i] = Wq0[r], s0[r]
        am, _ = _run(Wq, s, x, want_logits=False)
        assert am[0] == i, f"copies of row {r} down to {i}: got {am[0]}"


def test_duplicate_rows_lowest_index_wins():
    V, H = 500, 2560
    Wq, s = _quantised(V, H, seed=9)
    x = synth.tokens(H, 9, 1)
    _, _, am_o = oracle.head_logits(Wq, s, x, want_logits=False, want_bounds=False)
    r = int(am_o[0])
    Wq[V - 1], s[V - 1] = Wq[r], s[r]
    Wq[r - 1 if r > 0 else 1], s[r - 1 if r > 0 else 1] = Wq[r], s[r]
    am, _ = _run(Wq, s, x, want_logits=False)
    assert am[0] == min(r - 1 if r > 0 else 1, r)


@pytest.mark.parametrize("T", [1, 4])
def test_full_head_argmax(T):
    m = MANIFEST["head"]
    V, H = m["vocab"], m["hidden"]
    Wq, s = _quantised(V, H, m["seed"])
    x = synth.tokens(H, m["seed"], 4, m["x_attempt"])[:T]
    am, lg = _run(Wq, s, x)
    assert am.tolist() == m["argmax"][:T]
    # sampled rows against the oracle's fp64 logits and fp32 bounds
    rows = np.unique(np.concatenate([np.arange(0, V, 997), np.array(m["argmax"][:T]), [V - 1]]))
    lg_o, bd_o, _ = oracle.head_logits(Wq[rows], s[rows], x)
    assert (np.abs(lg[:, rows] - lg_o) <= bd_o).all()


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _gpu_quantize(w: torch.Tensor):
    V, H = w.shape
    codes = torch.empty((V, H), dtype=torch.uint8, device=dev())
    scales = torch.empty((V,), dtype=torch.float32, device=dev())
    moe.fp8_head_quantize(w, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _crafted_rows(H):
    """Rows that exercise the rounding rules: an all-zero row (scale 1); a row whose maximum is 448
    (scale exactly 1) holding values halfway between E4M3 neighbours (ties go to the even code),
    subnormal-range values and their ties; a single nonzero element; a row of equal magnitudes."""
    rows = np.zeros((4, H), dtype=np.float32)
    ties = [448.0, 1.0625, 1.1875, -1.0625, -1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 2.0 ** -11,
            0.3, -0.3, 13.0, 17.0, 240.0, 432.0, 440.0]
    rows[1, :len(ties)] = ties
    rows[2, H // 3] = -0.037
    rows[3, :] = 0.5
    rows[3, 1::2] = -0.5
    return rows


@pytest.mark.parametrize("V,H", [(4099, 2560), (37, 256), (130, 1024)])
def test_quantize_rows_bit_exact_fp32_and_bf16(V, H):
    W = np.concatenate([_crafted_rows(H), synth.head_weights(V, H, 21)[: V - 4]])
    codes, scales = _gpu_quantize(torch.from_numpy(W).to(dev()))
    Wq_o, s_o = oracle.head_quantize(W)
    assert (scales.view(np.uint32) == s_o.view(np.uint32)).all()
    bad = np.argwhere(codes != Wq_o)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}"
    # the same rows in bf16: the device reads bf16, the oracle its exact fp32 value
    Wb = _bf16_bits(W)
    codes, scales = _gpu_quantize(torch.from_numpy(Wb.view(np.int16)).to(dev()).view(torch.bfloat16))
    Wq_o, s_o = oracle.head_quantize((Wb.astype(np.uint32) << 16).view(np.float32))
    assert (scales.view(np.uint32) == s_o.view(np.uint32)).all()
    assert (codes == Wq_o).all()


def test_full_head_quantised_on_device():
    """The full 157,184 x 2,560 head quantised on the device at load (fp32 in), bit-equal to the
    oracle's quantisation, then used by the FP8 head: the argmax is the oracle's."""
    m = MANIFEST["head"]
    V, H = m["vocab"], m["hidden"]
    codes = torch.empty((V, H), dtype=torch.uint8, device=dev())
    scales = torch.empty((V,), dtype=torch.float32, device=dev())
    step = 16384
    for r0 in range(0, V, step):
        n = min(step, V - r0)
        w = torch.from_numpy(synth.head_weights(V, H, m["seed"], r0, n)).to(dev())
        moe.fp8_head_quantize(w, codes[r0:r0 + n], scales[r0:r0 + n])
        torch.cuda.synchronize()
        del w
    Wq_o, s_o = _quantised(V, H, m["seed"])
    assert (scales.cpu().numpy().view(np.uint32) == s_o.view(np.uint32)).all()
    assert bool((codes == torch.from_numpy(Wq_o).to(dev())).all())
    h = moe.fp8_head_create(codes, scales)
    x = synth.tokens(H, m["seed"], 4, m["x_attempt"])
    am = torch.full((4,), -1, dtype=torch.int32, device=dev())
    moe.fp8_head_run(h, to_dev_u16(x), am)
    torch.cuda.synchronize()
    moe.fp8_head_destroy(h)
    assert am.cpu().numpy().tolist() == m["argmax"]


def _run_bf16(Wb, x):
    h = moe.bf16_head_create(torch.from_numpy(Wb.view(np.int16)).to(dev()).view(torch.bfloat16))
    T = x.shape[0]
    am = torch.full((T,), -1, dtype=torch.int32, device=dev())
    lg = torch.empty((T, Wb.shape[0]), dtype=torch.float32, device=dev())
    moe.fp8_head_run(h, to_dev_u16(x), am, lg)
    torch.cuda.synchronize()
    moe.fp8_head_destroy(h)
    return am.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("V,T,H", [(3000, 4, 2560), (64 * 5 + 3, 1, 2560), (200, 3, 512), (MULTI_V, 4, 2560)])
def test_bf16_head_matches_oracle(V, T, H):
    """The unquantised BF16 head (the comparison point of the FP8 head): logits within the fp32
    evaluation bound of the oracle's fp64 logits, argmax exact where it is well posed."""
    Wb = _bf16_bits(synth.head_weights(V, H, 17))
    x = synth.tokens(H, 17, T)
    lg_o, bd_o, am_o = oracle.head_logits_bf16(Wb, x)
    am, lg = _run_bf16(Wb, x)
    assert (np.abs(lg - lg_o) <= bd_o).all()
    for t in range(T):
        if oracle.argmax_margin_ok(lg_o[t], bd_o[t]):
            assert am[t] == am_o[t]


def test_full_bf16_head_argmax():
    m = MANIFEST["head"]
    V, H = m["vocab"], m["hidden"]
    Wb = np.concatenate([_bf16_bits(synth.head_weights(V, H, m["seed"], r0, min(16384, V - r0)))
                         for r0 in range(0, V, 16384)])
    x = synth.tokens(H, m["seed"], 4, m["x_attempt"])[:2]
    lg_o, bd_o, am_o = oracle.head_logits_bf16(Wb, x)
    am, lg = _run_bf16(Wb, x)
    for t in range(2):
        assert oracle.argmax_margin_ok(lg_o[t], bd_o[t])
        assert am[t] == am_o[t]
    rows = np.arange(0, V, 613)
    assert (np.abs(lg[:, rows] - lg_o[:, rows]) <= bd_o[:, rows]).all()


@pytest.mark.parametrize("T", [2, 3, 4])
def test_verify_accepts_longest_matching_prefix(T):
    """Greedy acceptance fused after the argmax: drafts built from the oracle's target tokens so that
    every accept count 0 .. T-1 occurs, plus a draft that matches only after a mismatch."""
    V, H = 3000, 2560
    Wq, s = _quantised(V, H, seed=13)
    x = synth.tokens(H, 13, T)
    lg_o, bd_o, am_o = oracle.head_logits(Wq, s, x)
    assert all(oracle.argmax_margin_ok(lg_o[t], bd_o[t]) for t in range(T))
    h = moe.fp8_head_create(torch.from_numpy(Wq).to(dev()), torch.from_numpy(s).to(dev()))
    xd = to_dev_u16(x)
    cases = []
    for n in range(T):  # the first n drafts match, draft n (if any) does not
        d = [int(am_o[i]) for i in range(T - 1)]
        if n < T - 1:
            d[n] = (d[n] + 1) % V
        cases.append(d)
    if T > 2:
        d = [int(am_o[i]) for i in range(T - 1)]
        d[0] = (d[0] + 7) % V
        cases.append(d)
    for d in cases:
        am = torch.full((T,), -1, dtype=torch.int32, device=dev())
        acc = torch.full((1,), -1, dtype=torch.int32, device=dev())
        moe.fp8_head_verify(h, xd, torch.tensor(d, dtype=torch.int32, device=dev()), am, acc)
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == am_o.tolist()
        assert int(acc.item()) == oracle.mtp_accept(am_o, d), (d, am_o.tolist())
    moe.fp8_head_destroy(h)


def _e4m3_boundaries():
    """For each positive E4M3 code c = 1 .. 126, the smallest positive fp32 bit pattern that the
    oracle encodes to c or above (bisection over bit patterns; the oracle's encoder is monotonic,
    which its exhaustive CPU pin establishes).  The oracle's code of any |v| <= 448 is then the number
    of boundaries at or below |v|'s bit pattern."""
    codes = np.arange(1, 127)
    lo = np.zeros(codes.size, dtype=np.int64)             # encodes below c
    hi = np.full(codes.size, 0x43E00000, dtype=np.int64)  # 448.0 encodes to 126 >= c
    while (hi - lo > 1).any():
        mid = (lo + hi) // 2
        enc = oracle.e4m3_encode(mid.astype(np.uint32).view(np.float32)).astype(np.int64)
        up = enc >= codes
        hi = np.where(up, mid, hi)
        lo = np.where(up, lo, mid)
    return hi


def test_device_e4m3_conversion_exhaustive_sweep():
    """Every fp32 bit pattern with |v| <= 448 (both signs), and NaNs, through the device's FP8
    conversion as the kernels use it (codes = RNE-satfinite(fl32(v / s)); each row holds 448, so its
    scale s is exactly 1 and fl32(v / s) = v), against the oracle's encoding.  Stops at the first
    mismatch.  Rows whose maximum exceeds 448 then check the saturation of quotients just above 448."""
    H = 2560
    bounds = torch.from_numpy(_e4m3_boundaries().astype(np.int32)).to(dev())
    top = 0x43E00000  # 448.0
    rows = 16384
    per = rows * (H - 1)
    codes = torch.empty((rows, H), dtype=torch.uint8, device=dev())
    scales = torch.empty((rows,), dtype=torch.float32, device=dev())
    checked = 0
    for sign in (0, 1):
        for p0 in range(0, top + 1, per):
            n = min(per, top + 1 - p0)
            nr = (n + H - 2) // (H - 1)
            bits = torch.arange(p0, p0 + nr * (H - 1), dtype=torch.int64, device=dev())
            bits = torch.clamp(bits, max=top).to(torch.int32)  # the tail of the last row repeats 448
            vals = torch.empty((nr, H), dtype=torch.int32, device=dev())
            vals[:, 0] = top
            vals[:, 1:] = bits.view(nr, H - 1)
            v = vals.view(torch.float32)
            if sign:
                v = -v
            moe.fp8_head_quantize(v, codes[:nr], scales[:nr])
            want = torch.searchsorted(bounds, bits, right=True, out_int32=True).to(torch.uint8) | (0x80 * sign)
            got = codes[:nr, 1:].reshape(-1)
            assert bool((scales[:nr] == 1.0).all()), "a row's scale is not exactly 1"
            bad = torch.nonzero(got != want)
            if bad.numel():
                i = int(bad[0])
                f = float(np.array([int(bits[i])], dtype=np.int32).view(np.float32)[0]) * (-1 if sign else 1)
                raise AssertionError(f"{bad.numel()} codes differ; first v = {f!r}: device {int(got[i]):#04x}, "
                                     f"oracle {int(want[i]):#04x}")
            checked += n
            del vals, v, bits, want
    assert checked == 2 * (top + 1)
    # NaNs (quiet, signalling, both signs) and quotients just above 448
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF812345, 0x7FFFFFFF], dtype=np.uint32)
    W = np.zeros((4, H), dtype=np.float32)
    W[0, 0] = 448.0
    W[0, 1:6] = nan_bits.view(np.float32)
    for r, amax in ((1, 448.01), (2, 455.0), (3, 464.0)):
        W[r, 0] = amax
        W[r, 1:64] = amax * (1 - np.arange(63, dtype=np.float32) * 2.0 ** -20)
        W[r, 64:128] = -W[r, 1:65]
    c, s = _gpu_quantize(torch.from_numpy(W).to(dev()))
    Wq_o, s_o = oracle.head_quantize(W)
    assert (s.view(np.uint32) == s_o.view(np.uint32)).all()
    assert (c == Wq_o).all(), np.argwhere(c != Wq_o)[:8]
