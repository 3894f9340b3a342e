"""Pins for the oracle's number-format codecs (CPU only).

Each codec is checked against something other than itself: the OCP MX value table, an
independent library conversion (torch's float8_e4m3fn and bfloat16 casts, both
round-to-nearest-even), and a brute-force nearest-of-256 search.  The encoders are swept over
every fp32 bit pattern.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle

CHUNK = 1 << 24


def _patterns(i):
    return np.arange(i * CHUNK, (i + 1) * CHUNK, dtype=np.uint64).astype(np.uint32).view(np.float32)


def test_e2m1_matches_ocp_value_table():
    # OCP Microscaling Formats v1.0, E2M1 element values for codes 0..7; codes 8..15 negate them.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for code in range(16):
        want = table[code & 7] * (-1.0 if code & 8 else 1.0)
        got = oracle.e2m1_decode(code)
        assert got == want and np.signbit(got) == bool(code & 8), code
    # The generator's "uniform over the 16 values": sixteen codes, fifteen distinct values (+-0).
    assert len({oracle.e2m1_decode(c) for c in range(16)}) == 15


def test_e8m0_scales():
    for b in range(255):
        assert oracle.e8m0_decode(b) == 2.0 ** (b - 127)
    assert np.isnan(oracle.e8m0_decode(255))
    assert [oracle.e8m0_decode(b) for b in range(121, 126)] == [2.0 ** e for e in range(-6, -1)]


def test_e4m3_decode_matches_torch_and_landmarks():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.signbit(got[0x80]) and got[0x80] == 0.0
    pos = got[:0x7F]
    assert (np.diff(pos) > 0).all()  # 127 strictly increasing non-negative finite values


def _check_e4m3_chunk(i):
    f = _patterns(i)
    ours = oracle.e4m3_encode(f)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(f)
    with np.errstate(invalid="ignore"):
        a = np.abs(f.astype(np.float64))
    inside = ~nan & (a <= 464.0)  # torch rounds to nearest even here; beyond it returns NaN
    bad = np.flatnonzero(inside & (ours != ref))
    sat = ~nan & (a > 464.0)
    want_sat = np.where(np.signbit(f), 0xFE, 0x7E).astype(np.uint8)
    bad_sat = np.flatnonzero(sat & (ours != want_sat))
    bad_nan = np.flatnonzero(nan & ((ours & 0x7F) != 0x7F))
    return len(bad) + len(bad_sat) + len(bad_nan), (f[bad[:3]], f[bad_sat[:3]], f[bad_nan[:3]])


def test_e4m3_encode_exhaustive_all_fp32_patterns():
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(_check_e4m3_chunk, range((1 << 32) // CHUNK)))
    nbad = sum(r[0] for r in res)
    assert nbad == 0, [r[1] for r in res if r[0]][:3]


def test_e4m3_encode_brute_force_nearest():
    # Independent of torch: nearest of the 127 non-negative finite E4M3 values by bisection,
    # ties to the code with even mantissa, |v| beyond 448 saturates.
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    rng = np.random.default_rng(7)
    mids = (vals[:-1] + vals[1:]) / 2
    probes = np.concatenate([
        mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64), vals,
        rng.uniform(0, 460, 200000), np.exp2(rng.uniform(-14, 9, 200000)),
    ]).astype(np.float32)
    probes = np.concatenate([probes, -probes])
    got = oracle.e4m3_encode(probes)
    a = np.abs(probes.astype(np.float64))
    hi = np.searchsorted(vals, a, side="left").clip(1, 126)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, hi)
    tie = dlo == dhi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= vals[126], 126, pick)
    pick = np.where(a <= vals[0], 0, pick)
    want = (pick | np.where(np.signbit(probes), 0x80, 0)).astype(np.uint8)
    assert (got == want).all(), probes[got != want][:5]


def _check_bf16_chunk(i):
    f = _patterns(i)
    ours = oracle.bf16_encode(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    bad = np.flatnonzero(~nan & (ours != ref))
    ours_f = (ours.astype(np.uint32) << 16).view(np.float32)
    bad_nan = np.flatnonzero(nan & ~np.isnan(ours_f))
    return len(bad) + len(bad_nan)


def test_bf16_encode_exhaustive_all_fp32_patterns():
    with ThreadPoolExecutor(8) as ex:
        nbad = sum(ex.map(_check_bf16_chunk, range((1 << 32) // CHUNK)))
    assert nbad == 0


@pytest.mark.parametrize("v,code", [(0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E), (1e30, 0x7E), (-np.inf, 0xFE),
                                    (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (1.0625, 0x38),
                                    (1.1875, 0x3A)])
def test_e4m3_encode_spot_values(v, code):
    # 2^-10 is halfway between 0 and 2^-9 (ties to even -> 0); 1.0625 is halfway between 1 and
    # 1.125 (-> 1.0, even mantissa); 1.1875 is halfway between 1.125 and 1.25 (-> 1.25).
    assert int(oracle.e4m3_encode(np.array([v], dtype=np.float32))[0]) == code
