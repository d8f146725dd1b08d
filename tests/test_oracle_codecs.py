"""Pins for the oracle's codecs against sources other than the oracle itself:
torch's / numpy's own dtype conversions (library routines), the published
code-point facts of the formats (tests/golden/format_facts.json) and brute force.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLDEN, "format_facts.json")) as f:
        return json.load(f)


# --------------------------------------------------------------- E4M3FN: every code
def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.dec_e4m3_n(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_published_facts():
    f = _facts()["e4m3fn"]
    for code, val in f["values"].items():
        assert O.dec_e4m3(int(code, 16)) == float(val), code
    assert max(O.dec_e4m3_n(np.arange(0x7F, dtype=np.uint8))) == f["max_finite"]


# ------------------------------------------------------- E2M1 / E8M0: every code
def test_e2m1_table():
    f = _facts()["e2m1"]
    mags = [float(v) for v in f["magnitudes"]]
    for c in range(16):
        v = O.dec_e2m1(c)
        assert abs(v) == mags[c & 7]
        assert bool(np.signbit(v)) == bool(c & 8)


def test_e2m1_matches_torch_fp4_unpack():
    # torch's float4_e2m1fn_x2 has no arithmetic; cross-check via the spec's
    # magnitude table and the sign bit only.
    f = _facts()["e2m1"]
    for c in range(16):
        expect = float(f["magnitudes"][c & 7]) * (-1.0 if c & 8 else 1.0)
        assert O.dec_e2m1(c) == expect


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    ours = np.array([O.dec_e8m0(c) for c in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


# ------------------------------------------------------------ bf16 / fp16: every code
def test_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.dec_bf16_n(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp16_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.dec_fp16_n(codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = O.round_bf16_n(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_bf16_single_rounding_from_double():
    # 1 + 2^-8 + 2^-30 is above the midpoint between 1 and 1 + 2^-7: a single
    # rounding gives 1 + 2^-7 (0x3F81).  Rounding through fp32 first would land
    # exactly on the midpoint and tie to 1.0 (0x3F80).
    assert O.round_bf16(1 + 2**-8 + 2**-30) == 0x3F81
    assert O.round_bf16(1 + 2**-8) == 0x3F80          # exact tie -> even
    assert O.round_bf16(1 + 3 * 2**-8) == 0x3F82      # exact tie -> even (up)
    assert O.round_bf16(-(1 + 2**-8 + 2**-30)) == 0xBF81
    assert O.round_bf16(3.5e38) == 0x7F80              # overflow -> inf
    assert O.round_bf16(2.0**-140) == 0x0000          # below half the least subnormal
    assert O.round_bf16(3 * 2.0**-134) == 0x0002      # subnormal tie 1.5 ulp -> even (2)


def test_round_bf16_identity_and_midpoints():
    # every finite bf16 value rounds to itself; every midpoint between two
    # consecutive positive finite codes rounds to the even one
    codes = np.arange(0, 0x7F80, dtype=np.uint16)
    vals = O.dec_bf16_n(codes)
    assert np.array_equal(O.round_bf16_n(vals), codes)
    mids = (vals[:-1] + vals[1:]) / 2.0     # exact in double
    got = O.round_bf16_n(mids)
    lo = codes[:-1]
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, expect)


# -------------------------------------------------------- E4M3 encoder: midpoints and sweeps
def _brute_e4m3(v):
    """Nearest finite E4M3FN value by exhaustive search over torch-decoded
    codes, ties to the code with even mantissa, then v's sign."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    a = np.abs(v.astype(np.float64))[:, None]
    d = np.abs(vals[None, :] - a)
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    return pick | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def test_e4m3_encoder_at_every_midpoint():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact
    pts = [vals, mids]
    up, dn = mids, mids
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up, dn]
    v = np.concatenate(pts)
    v = np.concatenate([v, -v])
    assert np.array_equal(O.enc_e4m3_n(v), _brute_e4m3(v))
    # below 464 torch's own RNE conversion agrees too
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.enc_e4m3_n(v), ref)


def test_e4m3_encoder_random_against_torch_and_brute_force():
    rng = np.random.default_rng(1)
    mag = np.exp2(rng.uniform(-14, np.log2(463.0), size=400_000)).astype(np.float32)
    v = mag * rng.choice([-1.0, 1.0], size=mag.size).astype(np.float32)
    ours = O.enc_e4m3_n(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(ours[:20_000], _brute_e4m3(v[:20_000]))


def test_e4m3_encoder_saturates_and_keeps_zero_sign():
    big = np.array([448.0, 464.0, 465.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert list(O.enc_e4m3_n(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    tiny = np.array([2.0**-11, -(2.0**-11), 0.0, -0.0, 2.0**-10 + 2.0**-20], np.float32)
    # 2^-11 is below half the smallest subnormal (2^-10): rounds to signed zero
    assert list(O.enc_e4m3_n(tiny)) == [0x00, 0x80, 0x00, 0x80, 0x01]
