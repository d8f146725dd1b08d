"""Pins of the oracle's dense bf16 GEMV (the tail's LM-head GEMV with the
weights kept in bf16, bf16 input rows), independent of its own code: a
hand-worked case, small integers whose products and sums are exact (so the
result is an exact integer matrix product, computed here in int64), torch's
own bfloat16 decoding with a library matmul in fp64, the bf16 rounding of the
stored output against torch's rounding, and row independence."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_hand_worked():
    # W = [[1, 2, 0.5], [-3, 0, 0.25]], x = [4, -1, 8]:
    # y0 = 4 - 2 + 4 = 6, y1 = -12 + 0 + 2 = -10
    w = _bf16_bits([[1.0, 2.0, 0.5], [-3.0, 0.0, 0.25]])
    x = _bf16_bits([[4.0, -1.0, 8.0]])
    y16, y = O.gemv_bf16(w, x)
    assert np.array_equal(y, [[6.0, -10.0]])
    assert y16[0, 0] == 0x40C0 and y16[0, 1] == 0xC120  # bf16 6.0 and -10.0


def test_small_integers_exact():
    # integers in [-8, 8] are exact in bf16, and every partial sum below 2^53
    # is exact in double: the oracle must equal the int64 matrix product
    n, k, rows = 200, 300, 5
    rng = np.random.default_rng(3)
    wi = rng.integers(-8, 9, size=(n, k))
    xi = rng.integers(-8, 9, size=(rows, k))
    _, y = O.gemv_bf16(_bf16_bits(wi), _bf16_bits(xi))
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))


@pytest.mark.parametrize("rows", [1, 2, 8])
def test_against_torch_bfloat16(rows):
    n, k = 192, 640
    rng = np.random.default_rng(17 + rows)
    wb = _bf16_bits(rng.standard_normal((n, k)) * 0.05)
    xb = _bf16_bits(rng.standard_normal((rows, k)))
    y16, y = O.gemv_bf16(wb, xb, nthreads=4)
    want = _bf16_vals(xb) @ _bf16_vals(wb).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
    # the stored output is y rounded once to bf16 (torch rounds fp32 -> bf16 to
    # nearest even; y is checked where its fp32 value is exact enough)
    ref16 = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (y16 == ref16).mean() > 0.999


def test_rows_independent():
    n, k = 64, 256
    rng = np.random.default_rng(5)
    wb = _bf16_bits(rng.standard_normal((n, k)))
    xb = _bf16_bits(rng.standard_normal((4, k)))
    _, y4 = O.gemv_bf16(wb, xb)
    for r in range(4):
        _, y1 = O.gemv_bf16(wb, xb[r:r + 1])
        assert np.array_equal(y1[0], y4[r])


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        O.gemv_bf16(np.zeros((4, 0), np.uint16), np.zeros((1, 0), np.uint16))
