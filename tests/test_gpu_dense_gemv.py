"""GPU parity of lowbit_gemv's FP8 form (the tail's LM-head GEMV: E4M3
weights with one fp32 scale per 128x128 block, 1 to 8 bf16 input rows) and of
its bf16 form (the same GEMV with bf16 weights) against the fp64 oracle,
through the C ABI.

Shapes: small ones that take every K-part count (4, 2, 1) and ring depth
(4, 2, 1) of the kernel, and the LM head of 151,936 rows over the GLM hidden
size 6144 at 1 and 8 rows, checked on sampled 128-row blocks.  Weights: N(0,1)
quantised per 128x128 block (scale amax/448); x ~ N(0,1) in bf16.

bf16 form: weights N(0, 0.05^2) rounded to bf16, the same x; shapes that take
every K-part count (4, 2, 1) and ring depth (4, 2, 1) of its launcher, and the
same LM head at 1 and 8 rows.

Bar: each output within one bf16 rounding (2^-8 relative) plus the fp32
accumulation bound (K + 8) * 2^-24 * sum|terms| of the fp64 value, and
max |err| <= 2e-2 * max|ref| over the output.
"""
import numpy as np
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _weights(n, k, seed, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn(n, k, generator=g, device=device)
    codes, scales = S.encode_fp8_blocks(w)
    del w
    return codes.contiguous(), scales.contiguous()


def _check(codes, scales, x, y, blocks=None):
    """Compare y (GPU) with the oracle on the given 128-row blocks (all by default)."""
    n, k = codes.shape
    rows = x.shape[0]
    nb = n // 128
    blocks = list(range(nb)) if blocks is None else blocks
    idx = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    c = codes[torch.from_numpy(idx).to(codes.device)].cpu().numpy()
    s = scales[torch.tensor(blocks, device=scales.device)].cpu().numpy()
    xb = S.bf16_bits(x.cpu()).numpy().view(np.uint16)
    _, ref = O.gemv_fp8(c, s, xb, nthreads=16)
    yg = y.float().cpu().numpy().astype(np.float64)[:, idx]
    w = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64)
    w = w.abs() * torch.from_numpy(np.kron(s.astype(np.float64), np.ones((128, 128))))
    terms = (x.cpu().to(torch.float64).abs() @ w.T).numpy()
    bound = 2.0 ** -8 * np.abs(ref) + (k + 8) * 2.0 ** -24 * terms
    err = np.abs(yg - ref)
    assert (err <= bound).all(), ("outside the rounding bound", int((err > bound).sum()),
                                  float((err / np.maximum(bound, 1e-300)).max()))
    assert err.max() <= 2e-2 * np.abs(ref).max()
    return float(err.max() / np.abs(ref).max())


@pytest.mark.parametrize("n,k,rows", [(128, 128, 1), (256, 384, 3), (1024, 640, 8),
                                      (2048, 2048, 2), (384, 768, 5), (512, 1024, 4)])
def test_small_shapes(n, k, rows):
    _say(f"gemv_fp8 n={n} k={k} rows={rows}")
    codes, scales = _weights(n, k, seed=n + k + rows)
    x = S.make_x(rows, k, seed=rows + 17).cuda()
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    B.gemv_fp8(codes, scales, x, y, n, k, rows)
    torch.cuda.synchronize()
    _say("  rel", _check(codes, scales, x, y))


@pytest.mark.parametrize("rows", [1, 8])
def test_lm_head(rows):
    n, k = 151936, 6144
    _say(f"gemv_fp8 LM head [{n}, {k}] rows={rows}")
    codes, scales = _weights(n, k, seed=4200)
    x = S.make_x(rows, k, seed=4300 + rows).cuda()
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    B.gemv_fp8(codes, scales, x, y, n, k, rows)
    torch.cuda.synchronize()
    nb = n // 128
    blocks = sorted({0, 1, nb // 3, nb // 2, nb - 2, nb - 1})
    _say("  rel", _check(codes, scales, x, y, blocks))


def test_errors_and_no_ops():
    n, k = 256, 256
    codes, scales = _weights(n, k, seed=5)
    x = S.make_x(8, k, seed=6).cuda()
    y = torch.full((8, n), 3.0, dtype=torch.bfloat16, device="cuda")
    assert B.gemv_fp8_status(codes, scales, x, y, n, k, 0) == B.MOE_OK  # no-op
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    assert B.gemv_fp8_status(codes, scales, x, y, n, k, 9) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_fp8_status(codes, scales, x, y, 100, k, 1) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_fp8_status(codes, scales, x, y, n, 200, 1) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_fp8_status(codes, None, x, y, n, k, 1) == B.MOE_ERR_INVALID_ARG
    xm = torch.empty(8 * k + 4, dtype=torch.bfloat16, device="cuda")[4:].view(8, k)  # 8 bytes in
    assert B.gemv_fp8_status(codes, scales, xm, y, n, k, 1) == B.MOE_ERR_INVALID_ARG  # misaligned
    both = torch.empty(2 * k, dtype=torch.bfloat16, device="cuda")
    assert B.gemv_fp8_status(codes, scales, both[:k].view(1, k), both[64:64 + n].view(1, n),
                             n, k, 1) == B.MOE_ERR_INVALID_ARG  # x and y overlap


# ---- the bf16 form

def _bf16_weights(n, k, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(n, k, generator=g, device="cuda") * 0.05).to(torch.bfloat16)


def _check_bf16(w, x, y, blocks=None):
    """Compare y (GPU) with the oracle on the given 128-row blocks (all by default)."""
    n, k = w.shape
    nb = n // 128
    blocks = list(range(nb)) if blocks is None else blocks
    idx = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    wb = S.bf16_bits(w[torch.from_numpy(idx).to(w.device)].cpu()).numpy().view(np.uint16)
    xb = S.bf16_bits(x.cpu()).numpy().view(np.uint16)
    _, ref = O.gemv_bf16(wb, xb, nthreads=16)
    yg = y.float().cpu().numpy().astype(np.float64)[:, idx]
    terms = (x.cpu().to(torch.float64).abs() @ w[torch.from_numpy(idx).to(w.device)].cpu()
             .to(torch.float64).abs().T).numpy()
    bound = 2.0 ** -8 * np.abs(ref) + (k + 8) * 2.0 ** -24 * terms
    err = np.abs(yg - ref)
    assert (err <= bound).all(), ("outside the rounding bound", int((err > bound).sum()),
                                  float((err / np.maximum(bound, 1e-300)).max()))
    assert err.max() <= 2e-2 * np.abs(ref).max()
    return float(err.max() / np.abs(ref).max())


# (n, k, rows): K blocks of 64 -> (K parts, ring): 1 -> (1, 1), 3 -> (1, 1),
# 2 -> (2, 1), 6 -> (2, 1), 4 -> (4, 1), 8 -> (4, 2), 16 -> (4, 4), 40 -> (4, 2)
@pytest.mark.parametrize("n,k,rows", [(128, 64, 1), (256, 192, 3), (384, 128, 2),
                                      (512, 384, 5), (256, 256, 6), (640, 512, 4),
                                      (1024, 1024, 8), (2048, 2560, 7)])
def test_bf16_small_shapes(n, k, rows):
    _say(f"gemv_bf16 n={n} k={k} rows={rows}")
    w = _bf16_weights(n, k, seed=n + k + rows)
    x = S.make_x(rows, k, seed=rows + 29).cuda()
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    B.gemv_bf16(w, x, y, n, k, rows)
    torch.cuda.synchronize()
    _say("  rel", _check_bf16(w, x, y))


@pytest.mark.parametrize("rows", [1, 8])
def test_bf16_lm_head(rows):
    n, k = 151936, 6144
    _say(f"gemv_bf16 LM head [{n}, {k}] rows={rows}")
    w = _bf16_weights(n, k, seed=4400)
    x = S.make_x(rows, k, seed=4500 + rows).cuda()
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    B.gemv_bf16(w, x, y, n, k, rows)
    torch.cuda.synchronize()
    nb = n // 128
    blocks = sorted({0, 1, nb // 3, nb // 2, nb - 2, nb - 1})
    _say("  rel", _check_bf16(w, x, y, blocks))


def test_bf16_errors_and_no_ops():
    n, k = 256, 128
    w = _bf16_weights(n, k, seed=7)
    x = S.make_x(8, k, seed=8).cuda()
    y = torch.full((8, n), 3.0, dtype=torch.bfloat16, device="cuda")
    assert B.gemv_bf16_status(w, x, y, n, k, 0) == B.MOE_OK  # no-op
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    assert B.gemv_bf16_status(w, x, y, n, k, 9) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_bf16_status(w, x, y, 100, k, 1) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_bf16_status(w, x, y, n, 96, 1) == B.MOE_ERR_UNSUPPORTED
    assert B.gemv_bf16_status(None, x, y, n, k, 1) == B.MOE_ERR_INVALID_ARG
    xm = torch.empty(8 * k + 4, dtype=torch.bfloat16, device="cuda")[4:].view(8, k)  # 8 bytes in
    assert B.gemv_bf16_status(w, xm, y, n, k, 1) == B.MOE_ERR_INVALID_ARG  # misaligned
    both = torch.empty(2 * n, dtype=torch.bfloat16, device="cuda")
    assert B.gemv_bf16_status(w, both[:k].view(1, k), both[64:64 + n].view(1, n),
                              n, k, 1) == B.MOE_ERR_INVALID_ARG  # x and y overlap
