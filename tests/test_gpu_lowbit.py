"""GPU parity of lowbit_gemv (1-bit group-128 dense decode GEMV) against the
fp64 oracle, through the C ABI.

Shapes: the dense 1-bit workload of the 1-Bit Turbo page (Q1_0_G128): a SwiGLU
MLP of hidden 2560 and intermediate 9728 (up and gate [9728, 2560], down
[2560, 9728]) and the LM head [151936, 2560], plus small and ragged shapes.
Weights: bits Bernoulli(0.5), group scales |N(0, 0.02)| in fp16; x ~ N(0, 1)
in bf16.

Bar: y is bf16 of an fp32 sum, so each output must lie within one bf16
rounding (2^-8 relative) plus the fp32 accumulation bound
(K + 8) * 2^-24 * sum|terms| of the fp64 value, and max |err| <= 2e-2 * max|ref|
over the vector.
"""
import numpy as np
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S
from oracle import oracle as O

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _say(*a):
    print(*a, flush=True)


def _abs_terms(blk, xf, n, k):
    """sum over the row's terms of |d_g * x_k| (fp64)."""
    d = blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8)
    dv = np.abs(d.view(np.float16).astype(np.float64))               # [n, G]
    xs = np.abs(xf.reshape(k // 128, 128)).sum(axis=1)                 # [G]
    return dv @ xs


def _check(n, k, seed, nthreads=16):
    _say(f"lowbit_gemv n={n} k={k} seed={seed}")
    blk = S.make_q1(n, k, seed=seed)
    x = S.make_x(1, k, seed=seed + 1)[0]
    xb = S.bf16_bits(x).numpy().view(np.uint16)
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    B.lowbit_gemv(blk.cuda(), x.cuda(), y, n, k)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    _, ref = O.lowbit_gemv_q1(blk.numpy(), xb, n, k, nthreads=nthreads)
    xf = x.float().numpy().astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + (k + 8) * U32 * _abs_terms(blk.numpy(), xf, n, k)
    err = np.abs(yg - ref)
    assert (err <= bound).all(), ("lowbit_gemv outside its rounding bound", n, k,
                                  int((err > bound).sum()), float((err / bound).max()))
    assert err.max() <= 2e-2 * np.abs(ref).max()
    return float(err.max() / np.abs(ref).max())


@pytest.mark.parametrize("n,k", [(1, 128), (5, 256), (3, 384), (1000, 1280), (257, 2560)])
def test_lowbit_small_and_ragged(n, k):
    _check(n, k, seed=n * 7 + k)


@pytest.mark.parametrize("n,k,name", [(9728, 2560, "up/gate"), (2560, 9728, "down"),
                                      (151936, 2560, "lm_head")])
def test_lowbit_turbo_shapes(n, k, name):
    rel = _check(n, k, seed=4242 + n % 1000)
    _say(f"  {name}: max err / max|ref| = {rel:.2e}")


def test_lowbit_max_k():
    _check(64, 16384, seed=99)


def test_lowbit_zero_rows_and_zero_n():
    k = 256
    blk = S.make_q1(4, k, seed=1).cuda()
    x = S.make_x(1, k, seed=2)[0].cuda()
    y = torch.full((4,), 7.0, dtype=torch.bfloat16, device="cuda")
    B.lowbit_gemv(blk, x, y, 4, k, rows=0)
    B.lowbit_gemv(blk, x, y, 0, k, rows=1)
    torch.cuda.synchronize()
    assert (y.float() == 7.0).all()
    assert B.lowbit_gemv_status(blk, x, y, 4, k, rows=9) == B.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("n,k", [(16384, 256), (16385, 768), (20000, 5632)])
def test_lowbit_table_form_edges(n, k):
    """The table form's edges: one chunk of K, a ragged last block of rows,
    and an odd number of chunks with 64-row blocks."""
    _check(n, k, seed=n + k)


def _check_rows(n, k, rows, seed, nthreads=16):
    """Several input rows at once (the MFMA form) against the oracle run on
    each row alone, with the single-row bound per output."""
    _say(f"lowbit_gemv n={n} k={k} rows={rows} seed={seed}")
    blk = S.make_q1(n, k, seed=seed)
    x = S.make_x(rows, k, seed=seed + 1)
    xb = S.bf16_bits(x).numpy().view(np.uint16)
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    B.lowbit_gemv(blk.cuda(), x.cuda(), y, n, k, rows=rows)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in range(rows):
        _, ref = O.lowbit_gemv_q1(blk.numpy(), xb[r], n, k, nthreads=nthreads)
        xf = x[r].float().numpy().astype(np.float64)
        bound = 2.0 ** -8 * np.abs(ref) + (k + 8) * U32 * _abs_terms(blk.numpy(), xf, n, k)
        err = np.abs(yg[r] - ref)
        assert (err <= bound).all(), ("row outside its rounding bound", r, n, k,
                                      int((err > bound).sum()), float((err / bound).max()))
        assert err.max() <= 2e-2 * np.abs(ref).max()
        worst = max(worst, float(err.max() / np.abs(ref).max()))
    return worst


@pytest.mark.parametrize("n,k,rows", [(5, 256, 2), (1000, 1280, 8), (9728, 2560, 4),
                                      (2560, 9728, 8), (64, 16384, 3), (151936, 2560, 8)])
def test_lowbit_several_rows(n, k, rows):
    """1-bit GEMV beyond batch 1: ragged rows and a ragged last 16-row slab,
    every K-part count, the MLP and LM-head shapes, K = 16384."""
    rel = _check_rows(n, k, rows, seed=n % 997 + k + rows)
    _say(f"  max err / max|ref| = {rel:.2e}")


def test_lowbit_several_rows_need_256_chunks():
    k = 384
    blk = S.make_q1(4, k, seed=1).cuda()
    x = S.make_x(2, k, seed=2).cuda()
    y = torch.empty(2, 4, dtype=torch.bfloat16, device="cuda")
    assert B.lowbit_gemv_status(blk, x, y, 4, k, rows=2) == B.MOE_ERR_UNSUPPORTED

