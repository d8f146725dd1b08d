"""Seeded synthetic inputs for the MoE decode step and the 1-bit GEMV.

This module only draws random numbers and stores them in the library's
canonical layouts.  It holds none of the method's arithmetic (no norm, no
routing, no GEMV, no requantisation of activations or mid); both the HIP path
and the CPU oracle consume exactly the bytes it produces.  Weight encoding
uses torch's own ``float8_e4m3fn`` conversion, and a plain nearest-value
search for E2M1; both are generator choices, not part of the method.

Canonical layouts (all row-major, stacked experts expert-major):
  FP8 matrix [N, K]:   codes uint8 [N, K], scales float32 [N/128, K/128]
  MXFP4 matrix [N, K]: codes uint8 [N, K/2] (element 2i in the low nibble),
                       scales uint8 E8M0 [N, K/32]
  Q1 routed matrix [N, K]: blocks uint8 [N, K/128, 18] (as below), no scales
  Q1 matrix [N, K]:    uint8 [N, K/128, 18] = fp16 d (little-endian) + 16 bytes
                       of sign bits, bit i of byte b is element 8b+i, 1 = minus

Workloads (sizes as the pages describe a GLM-scale layer; distributions are
synthetic stand-ins for real weights, which are not available):
  tiny:  hidden 256, 32 routed experts, intermediate 128, no shared expert,
         router ~ N(0, 0.02)
  glm:   hidden 6144, 256 routed experts, intermediate 2048, one shared expert
         of intermediate 2048, router ~ N(0, 0.01)
  x ~ N(0, 1); RMSNorm gamma ~ U(0.8, 1.2); eps 1e-6; expert weights drawn
  from N(0, 1) and encoded per block (FP8: scale amax/448 per 128x128;
  MXFP4: E8M0 exponent floor(log2 amax) - 2 per 32 along K).  Routed experts
  may instead be 1-bit (Q1_0_G128): bits Bernoulli(0.5) and group scales
  |N(0, 0.02)| in fp16, as the 1-bit GEMV's workload.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

SHAPES = {
    "tiny": dict(hidden=256, inter=128, n_experts=32, shared_inter=0, router_std=0.02),
    "glm": dict(hidden=6144, inter=2048, n_experts=256, shared_inter=2048, router_std=0.01),
}

FMT_FP8 = 1
FMT_MXFP4 = 2
FMT_Q1 = 3
Q1_D_STD = 0.02  # 1-bit group scales |N(0, 0.02)| (the 1-Bit Turbo workload's)

_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """bfloat16 tensor -> its uint16 bit patterns (as int16 storage)."""
    return t.contiguous().view(torch.int16)


def encode_fp8_blocks(w: torch.Tensor):
    """float32 [N, K] -> (uint8 codes [N, K], float32 scales [N/128, K/128]).
    Scale = amax/448 per 128x128 block, codes = torch's E4M3FN rounding of w/s."""
    n, k = w.shape
    blk = w.view(n // 128, 128, k // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    scale = amax / 448.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (blk / safe[:, None, :, None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(n, k).contiguous(), scale.float().contiguous()


def encode_mxfp4(w: torch.Tensor):
    """float32 [N, K] -> (uint8 codes [N, K/2], uint8 E8M0 scales [N, K/32]).
    Per 32 along K: X = floor(log2 amax) - 2 (largest E2M1 magnitude 6 = 1.5*2^2),
    element = nearest E2M1 value of w / 2^X (ties to the even code), saturating
    at 6; an all-zero group gets X = -127 and zero codes."""
    n, k = w.shape
    g = w.view(n, k // 32, 32)
    amax = g.abs().amax(dim=2)
    x = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    x = torch.where(amax > 0, x, torch.full_like(x, -127.0)).clamp(-127, 127)
    v = g / torch.exp2(x)[:, :, None]
    mags = torch.tensor(_E2M1_MAG, device=w.device, dtype=torch.float32)
    a = v.abs().clamp(max=6.0)
    d = (a[..., None] - mags).abs()
    best = d.argmin(dim=-1)  # first minimum = lower code on an exact tie
    dmin = d.gather(-1, best[..., None])[..., 0]
    # exact tie with the next code: take the code whose mantissa bit is 0
    nxt = (best + 1).clamp(max=7)
    tie = (d.gather(-1, nxt[..., None])[..., 0] == dmin) & (nxt != best)
    code = torch.where(tie & (best % 2 == 1), nxt, best)
    code = code | ((v < 0) & (code != 0)).to(code.dtype) << 3
    code = code.to(torch.uint8).view(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    e8m0 = (x + 127).to(torch.uint8).contiguous()
    return packed, e8m0


@dataclass
class ExpertWeights:
    """Stacked expert matrices in canonical layout (codes, scales) per matrix."""
    fmt: int
    gate: tuple
    up: tuple
    down: tuple

    def expert(self, e: int):
        """Expert e's (gate codes, gate scales, up codes, up scales, down codes,
        down scales); the scales are None for 1-bit matrices."""
        sc = lambda m: None if m[1] is None else m[1][e]
        return (self.gate[0][e], sc(self.gate), self.up[0][e], sc(self.up),
                self.down[0][e], sc(self.down))


@dataclass
class Layer:
    shape: str
    hidden: int
    inter: int
    n_experts: int
    shared_inter: int
    rms_eps: float
    gamma: torch.Tensor          # bf16 [H]
    router_w: torch.Tensor       # bf16 [E, H]
    routed: ExpertWeights        # stacked [E, ...]
    shared: Optional[ExpertWeights] = None  # stacked [1, ...]
    extra: dict = field(default_factory=dict)

    @property
    def routed_fmt(self) -> int:
        return self.routed.fmt


def _encode(fmt, w):
    return encode_fp8_blocks(w) if fmt == FMT_FP8 else encode_mxfp4(w)


def q1_blocks(bits: torch.Tensor, d16: torch.Tensor) -> torch.Tensor:
    """Q1 blocks uint8 [n, groups, 18] from sign bytes uint8 [n, groups, 16]
    and fp16 scales [n, groups] (d little-endian, then the sign bytes)."""
    n, groups = d16.shape
    blk = torch.empty(n, groups, 18, dtype=torch.uint8, device=bits.device)
    dv = d16.view(torch.int16).to(torch.int32) & 0xFFFF
    blk[..., 0] = (dv & 0xFF).to(torch.uint8)
    blk[..., 1] = (dv >> 8).to(torch.uint8)
    blk[..., 2:] = bits.to(torch.uint8)
    return blk.contiguous()


def _q1_matrix(n, k, gen, device):
    groups = k // 128
    d = (torch.randn(n, groups, generator=gen, device=device) * Q1_D_STD).abs().to(torch.float16)
    bits = torch.randint(0, 256, (n, groups, 16), generator=gen, device=device, dtype=torch.int32)
    return q1_blocks(bits, d)


def _stack(fmt, n_exp, n, k, gen, device):
    codes, scales = [], []
    for _ in range(n_exp):
        if fmt == FMT_Q1:
            codes.append(_q1_matrix(n, k, gen, device))
            continue
        w = torch.randn(n, k, generator=gen, device=device, dtype=torch.float32)
        c, s = _encode(fmt, w)
        codes.append(c)
        scales.append(s)
    return torch.stack(codes), (torch.stack(scales) if scales else None)


def make_layer(shape="tiny", routed_fmt: int = FMT_FP8, seed: int = 1000,
               device="cpu") -> Layer:
    """One MoE layer of the named shape (or a dict with the same keys as
    SHAPES' entries), drawn from ``seed`` on ``device``."""
    p = SHAPES[shape] if isinstance(shape, str) else dict(shape)
    if not isinstance(shape, str):
        shape = "custom"
    H, I, E, Is = p["hidden"], p["inter"], p["n_experts"], p["shared_inter"]
    gen = _gen(seed, device)
    gamma = (torch.rand(H, generator=gen, device=device) * 0.4 + 0.8).to(torch.bfloat16)
    router_w = (torch.randn(E, H, generator=gen, device=device) * p["router_std"]).to(torch.bfloat16)
    g = _stack(routed_fmt, E, I, H, gen, device)
    u = _stack(routed_fmt, E, I, H, gen, device)
    d = _stack(routed_fmt, E, H, I, gen, device)
    routed = ExpertWeights(routed_fmt, g, u, d)
    shared = None
    if Is > 0:
        shared = ExpertWeights(FMT_FP8, _stack(FMT_FP8, 1, Is, H, gen, device),
                               _stack(FMT_FP8, 1, Is, H, gen, device),
                               _stack(FMT_FP8, 1, H, Is, gen, device))
    return Layer(shape, H, I, E, Is, 1e-6, gamma, router_w, routed, shared)


def make_x(rows: int, hidden: int, seed: int, mode: str = "indep", device="cpu") -> torch.Tensor:
    """Token rows, bf16 [rows, hidden].  'indep': each row ~ N(0,1).
    'corr': x_0 ~ N(0,1), x_i = 0.8 x_0 + 0.6 N(0,1) (fp32, then bf16), so rows
    pick many of the same experts."""
    gen = _gen(seed, device)
    x = torch.randn(rows, hidden, generator=gen, device=device)
    if mode == "corr" and rows > 1:
        x[1:] = 0.8 * x[0:1] + 0.6 * x[1:]
    elif mode not in ("indep", "corr"):
        raise ValueError(mode)
    return x.to(torch.bfloat16).contiguous()


def make_q1(n: int, k: int, seed: int, device="cpu") -> torch.Tensor:
    """1-bit group-128 matrix: uint8 [n, k/128, 18]; bits Bernoulli(0.5),
    group scale |N(0, 0.02)| stored as fp16 (little-endian)."""
    return _q1_matrix(n, k, _gen(seed, device), device)
