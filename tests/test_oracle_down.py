"""Pins of the oracle's down GEMV on a given mid (orc_expert_down), which the
GPU parity tests apply to the device's own mid codes to judge the device's
down outputs: closed forms with block scales that a transposed or shifted
index would break, a single nonzero mid code, MXFP4 exponents at the ends of
the E8M0 range with -0 nibbles, an independent numpy pipeline built on torch's
decoders and a library matmul, and agreement with the whole-step oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.test_oracle_layer import _np_fp8, _np_mxfp4

F32 = np.float32


def test_fp8_all_one_codes_closed_form():
    """W codes all 1.0 (0x38) with a 2 x 3 grid of block scales S, mid codes
    all 1.0 with block scales t: y_h = 128 sum_b S[h/128, b] t[b]."""
    S = np.array([[1 / 8, 3 / 16, -1 / 4], [5 / 32, 1 / 64, 7 / 128]], F32)
    t = np.array([1 / 2, -3 / 4, 5 / 8], F32)
    codes = np.full((256, 384), 0x38, np.uint8)
    midq = np.full(384, 0x38, np.uint8)
    y, ya, yg = O.expert_down(O.FMT_FP8, codes, S, midq=midq, midqs=t)
    blk = 128 * (S.astype(float) @ t.astype(float))
    blk_abs = 128 * (np.abs(S.astype(float)) @ np.abs(t.astype(float)))
    assert np.array_equal(y, np.repeat(blk, 128))
    assert np.array_equal(ya, np.repeat(blk_abs, 128))
    # every term of a group of 8 is equal: the group maxima sum to y_abs / 8
    assert np.array_equal(yg, np.repeat(blk_abs, 128) / 8)
    # the transposed reading of the scale grid would give other values
    assert not np.allclose(blk, 128 * (S.astype(float)[:, ::-1] @ t.astype(float)))


def test_fp8_single_mid_code():
    """Only mid element k0 is nonzero (code 0xC4 = -3, block scale 1/4): y_h is
    W[h, k0] * S[h/128, k0/128] * -3/4 exactly, with W decoded by torch."""
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, (256, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x40  # no NaN codes
    S = (rng.random((2, 2)) + 0.5).astype(F32)
    for k0 in (0, 77, 128, 255):
        midq = np.zeros(256, np.uint8)
        midq[k0] = 0xC4
        midqs = np.array([0.25, 0.25], F32)
        y, ya, yg = O.expert_down(O.FMT_FP8, codes, S, midq=midq, midqs=midqs)
        w = torch.from_numpy(codes[:, k0].copy()).view(torch.float8_e4m3fn).double().numpy()
        expect = w * np.repeat(S[:, k0 // 128].astype(float), 128) * (-3.0 * 0.25)
        assert np.array_equal(y, expect)
        assert np.array_equal(ya, np.abs(expect))
        assert np.array_equal(yg, np.abs(expect))  # one nonzero term


def test_mxfp4_exponent_extremes_and_negative_zero():
    """MXFP4 rows whose E8M0 codes sit at 0, 1, 64, 127, 200 and 254, all
    nibbles 1.0 (0x2) except -0 nibbles (0x8) in every other group, mid given
    per 32-group as a small power of two: y_h = sum_g 2^(e-127) c_g n_g with
    n_g the group's count of 1.0 nibbles (exact in double)."""
    codes_e = [0, 1, 64, 127, 200, 254]
    H, I = len(codes_e) * 2, 128
    nib = np.full((H, I), 0x2, np.uint8)
    nib[:, 32:64:2] = 0x8          # group 1: half its elements are -0
    nib[:, 96:128] = 0x8           # group 3: all -0
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    e8 = np.zeros((H, I // 32), np.uint8)
    for i, c in enumerate(codes_e):
        e8[2 * i] = c
        e8[2 * i + 1] = [c, c, c, 254][: I // 32] if c != 254 else c
    cg = np.array([0.5, 2.0, -0.25, 8.0], F32)
    mid = np.repeat(cg, 32)
    y, ya, _ = O.expert_down(O.FMT_MXFP4, packed, e8, mid32=mid)
    count = np.array([32, 16, 32, 0], float)
    expect = np.array([sum(2.0 ** (int(e8[h, g]) - 127) * float(cg[g]) * count[g]
                           for g in range(4)) for h in range(H)])
    assert np.array_equal(y, expect)
    assert np.array_equal(ya, np.array([sum(2.0 ** (int(e8[h, g]) - 127) * abs(float(cg[g]))
                                            * count[g] for g in range(4)) for h in range(H)]))
    assert y[0] == 2.0 ** -127 * (0.5 * 32 + 2.0 * 16 - 0.25 * 32)


def test_against_independent_numpy_pipeline():
    rng = np.random.default_rng(22)
    # FP8: random finite codes, scales spanning 2^-30 .. 2^10
    codes = rng.integers(0, 256, (384, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    S = np.exp2(rng.integers(-30, 11, (3, 4))).astype(F32)
    midq = rng.integers(0, 256, 512).astype(np.uint8)
    midq[(midq & 0x7F) == 0x7F] = 0x11
    midqs = (rng.random(4) * 1e-3).astype(F32)
    y, ya, yg = O.expert_down(O.FMT_FP8, codes, S, midq=midq, midqs=midqs, nthreads=4)
    mhat = torch.from_numpy(midq).view(torch.float8_e4m3fn).double().numpy() * np.repeat(
        midqs.astype(float), 128)
    W = _np_fp8(codes, S)
    assert np.allclose(y, W @ mhat, rtol=0, atol=1e-13 * ya.max())
    assert np.allclose(ya, np.abs(W) @ np.abs(mhat), rtol=1e-13, atol=0)
    gm = np.abs(W * mhat[None, :]).reshape(W.shape[0], -1, 8).max(axis=2).sum(axis=1)
    assert np.allclose(yg, gm, rtol=1e-13, atol=0)
    assert (yg <= ya).all() and (8 * yg >= ya).all()
    # MXFP4: random nibbles (-0 included), E8M0 around 127, fp32 mid
    packed = rng.integers(0, 256, (256, 256)).astype(np.uint8)
    e8 = rng.integers(100, 150, (256, 16)).astype(np.uint8)
    mid = rng.standard_normal(512).astype(F32)
    y, ya, yg = O.expert_down(O.FMT_MXFP4, packed, e8, mid32=mid, nthreads=4)
    W = _np_mxfp4(packed, e8)
    assert np.allclose(y, W @ mid.astype(float), rtol=0, atol=1e-13 * ya.max())
    assert np.allclose(ya, np.abs(W) @ np.abs(mid.astype(float)), rtol=1e-13, atol=0)
    gm = np.abs(W * mid.astype(float)[None, :]).reshape(W.shape[0], -1, 8).max(axis=2).sum(axis=1)
    assert np.allclose(yg, gm, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fmt", [O.FMT_FP8, O.FMT_MXFP4])
def test_agrees_with_the_step_oracle(fmt):
    """On the step oracle's own mid codes (FP8) or mid (MXFP4) it reproduces
    the step's per-(row, pick) down outputs bit for bit (same sums, same order)."""
    import bit_moe_decode_amd.synth as S
    from tests.test_oracle_layer import _run_oracle
    layer = S.make_layer("tiny", routed_fmt=fmt, seed=1010)
    x = S.make_x(3, layer.hidden, seed=2010)
    _, d = _run_oracle(layer, x)
    for r in range(3):
        for j in range(8):
            e = int(d["ids"][r, j])
            m = [t.numpy() for t in layer.routed.expert(e)]
            if fmt == O.FMT_FP8:
                y, _, _ = O.expert_down(fmt, m[4], m[5], midq=d["midq"][r, j, :layer.inter],
                                        midqs=d["midqs"][r, j, :layer.inter // 128])
            else:
                y, _, _ = O.expert_down(fmt, m[4], m[5], mid32=d["mid"][r, j, :layer.inter])
                # the step keeps MXFP4 mid in double; the fp32 copy differs by its rounding
                yd = _np_mxfp4(m[4], m[5]) @ d["mid"][r, j, :layer.inter]
                assert np.allclose(y, yd, rtol=0, atol=1e-6 * np.abs(yd).max())
                continue
            assert np.array_equal(y, d["y"][r, j])


def test_rejects_missing_inputs():
    codes = np.zeros((128, 128), np.uint8)
    with pytest.raises(ValueError):
        O.expert_down(O.FMT_FP8, codes, np.ones((1, 1), F32))
    with pytest.raises(ValueError):
        O.expert_down(O.FMT_MXFP4, codes[:, :64], np.zeros((128, 4), np.uint8))


def test_q1_down_closed_form():
    """1-bit down: signs + except row block 1 (all -), group scale d[h/128][g],
    mid codes all 1.0 with block scales t: y_h = +-128 sum_g d[h/128][g] t[g]."""
    from tests.test_oracle_layer import _q1_const
    D = np.array([[1 / 16, 3 / 64], [5 / 32, 1 / 128]])
    t = np.array([0.5, -0.25], F32)
    blk = np.concatenate([_q1_const(128, 256, D[:1]), _q1_const(128, 256, D[1:], minus=True)])
    midq = np.full(256, 0x38, np.uint8)
    y, ya, yg = O.expert_down(O.FMT_Q1, blk, None, midq=midq, midqs=t)
    expect = np.concatenate([np.full(128, 128 * (D[0] @ t)), np.full(128, -128 * (D[1] @ t))])
    assert np.array_equal(y, expect)
    assert np.array_equal(ya, np.concatenate([np.full(128, 128 * (np.abs(D[0]) @ np.abs(t))),
                                              np.full(128, 128 * (np.abs(D[1]) @ np.abs(t)))]))
