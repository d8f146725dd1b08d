"""Pins of the oracle's dense FP8 GEMV (the tail's LM-head GEMV: E4M3 weights,
one fp32 scale per 128x128 block, bf16 input rows), independent of its own
code: a hand-worked single-weight case, the closed form for all-one codes with
varying block scales (block sums of x, computed here with numpy), and torch's
own float8_e4m3fn decoding of every finite code with a library matmul."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_single_weight_hand_worked():
    # W[3][5] = 2.0 (E4M3 0x40) in a block of scale 0.5; x[5] = 3.0: y[3] = 3.0, the rest 0
    codes = np.zeros((128, 128), np.uint8)
    codes[3, 5] = 0x40
    scales = np.full((1, 1), 0.5, np.float32)
    x = np.zeros((1, 128), np.float32)
    x[0, 5] = 3.0
    y16, y = O.gemv_fp8(codes, scales, _bf16_bits(x))
    want = np.zeros((1, 128))
    want[0, 3] = 3.0
    assert np.array_equal(y, want)
    assert y16[0, 3] == 0x4040 and int(np.count_nonzero(y16)) == 1  # bf16 3.0


def test_all_one_codes_closed_form():
    # codes 0x38 = 1.0 everywhere, scale 2^(nb - kb) per block:
    # y[r][n] = sum_kb 2^(n/128 - kb) * (sum of x[r] over block kb)
    n, k, rows = 256, 384, 3
    codes = np.full((n, k), 0x38, np.uint8)
    nb, kb = np.meshgrid(np.arange(n // 128), np.arange(k // 128), indexing="ij")
    scales = np.ldexp(1.0, nb - kb).astype(np.float32)
    rng = np.random.default_rng(7)
    xb = _bf16_bits(rng.standard_normal((rows, k)))
    xv = _bf16_vals(xb)
    bsum = xv.reshape(rows, k // 128, 128).sum(axis=2)                  # [rows, K/128]
    want = np.repeat(bsum @ scales.T.astype(np.float64), 128, axis=1)    # [rows, n]
    _, y = O.gemv_fp8(codes, scales, xb)
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rows", [1, 2, 8])
def test_against_torch_float8_decoding(rows):
    # every finite E4M3 code, decoded by torch's float8_e4m3fn, block scales
    # expanded with numpy, then one library matmul
    n, k = 256, 512
    rng = np.random.default_rng(11 + rows)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    codes = rng.choice(finite, size=(n, k))
    scales = (rng.random((n // 128, k // 128)) * 0.01 + 1e-4).astype(np.float32)
    xb = _bf16_bits(rng.standard_normal((rows, k)))
    w = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = w * np.kron(scales.astype(np.float64), np.ones((128, 128)))
    xv = _bf16_vals(xb)
    want = xv @ w.T
    _, y = O.gemv_fp8(codes, scales, xb, nthreads=4)
    bound = 1e-12 * (np.abs(xv) @ np.abs(w).T) + 1e-300
    assert (np.abs(y - want) <= bound).all()


def test_rows_are_independent():
    n, k = 128, 256
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    codes = rng.choice(finite, size=(n, k))
    scales = (rng.random((1, 2)) * 0.01 + 1e-3).astype(np.float32)
    xb = _bf16_bits(rng.standard_normal((4, k)))
    y16, y = O.gemv_fp8(codes, scales, xb)
    for r in range(4):
        y16r, yr = O.gemv_fp8(codes, scales, xb[r:r + 1])
        assert np.array_equal(y16r[0], y16[r]) and np.array_equal(yr[0], y[r])


def test_rejects_shapes_off_the_block_grid():
    # 100 rows is not a whole number of 128-row scale blocks
    with pytest.raises(ValueError):
        O.gemv_fp8(np.zeros((100, 128), np.uint8), np.zeros((0, 1), np.float32),
                   np.zeros((1, 128), np.uint16))
