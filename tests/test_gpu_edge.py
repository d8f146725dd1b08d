"""GPU parity at the method's edge cases, through the C ABI, against the fp64
oracle (same checks as tests/parity.py: bit-exact top-8 and dedup table,
bit-exact activation blocks, mid within its rounding bound and its codes
adjacent, every (row, pick) down output against the oracle's down GEMV of the
device's own mid, and the bf16 output).

Cases:
  - an all-zero token row: every logit is +0, so all experts tie and the
    picks are IDs 0..7; its activation blocks, mid blocks and output are zero;
    another row with one all-zero 128-block (activation scale 0);
  - weight rows of gate or up set to zero codes, so whole 1x128 mid blocks
    are zero (mid scale 0);
  - an exact tie across the 8th place, made by copying the router row of the
    8th pick to a lower or a higher expert ID, and a router with most rows
    zero, so that many +0 logits tie at the 8th place;
  - MXFP4 experts whose E8M0 exponents reach 0, 1, 64, 127, 180-201 and 254
    (the last on groups of zero and -0 nibbles), with -0 nibbles everywhere;
  - FP8 experts whose 128x128 block scales span 2^-30 .. 2^10, with token
    rows whose 128-blocks span 2^-20 .. 2^20.
The GPU's router sums start from +0, so a -0 logit cannot arise on the device;
the comparator's -0 == +0 rule is pinned on the CPU (tests/test_oracle_select.py).
"""
import os

import numpy as np
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S
from tests import parity as P

pytestmark = pytest.mark.gpu

NTHREADS = min(16, len(os.sched_getaffinity(0)))


def _say(*a):
    print(*a, flush=True)


def _run(layer, x, max_rows=None, cache=None):
    rows = x.shape[0]
    runner = B.LayerRunner(layer, max_rows or rows)
    out = runner.run(x.to("cuda"))
    torch.cuda.synchronize()
    gpu = runner.debug(rows)
    ref_out, ref = P.oracle_for(layer, x, gpu["logits"], nthreads=NTHREADS, host_cache=cache)
    rep = P.compare(layer, x, gpu, out, ref_out, ref)
    return out, gpu, rep


SMALL = dict(hidden=256, inter=128, n_experts=32, shared_inter=128, router_std=0.02)
MEDIUM = dict(hidden=512, inter=384, n_experts=64, shared_inter=384, router_std=0.02)


# ------------------------------------------------------------ zero inputs
@pytest.mark.parametrize("shape", [SMALL, MEDIUM], ids=["small", "medium"])
@pytest.mark.parametrize("rows", [1, 4, 8])
def test_zero_row_and_zero_activation_block(shape, rows):
    layer = S.make_layer(shape, seed=4000 + shape["hidden"], device="cuda")
    x = S.make_x(rows, shape["hidden"], seed=4100 + rows)
    x[0] = 0
    if rows > 1:
        x[1, 128:256] = 0
    _say(f"zero row, hidden={shape['hidden']} rows={rows}")
    out, gpu, rep = _run(layer, x)
    _say(rep)
    assert list(gpu["ids"][0]) == list(range(8)), gpu["ids"][0]
    assert np.all(gpu["logits"][0] == 0)
    assert np.all(gpu["gates"][0] == np.float32(0.125))
    assert not gpu["act_s"][0].any() and not gpu["act_q"][0].any()
    assert not gpu["mid"][0].any() and not gpu["midqs"][0].any()
    assert not gpu["y"][0].any()
    assert not out[0].float().abs().sum().item()
    if rows > 1:
        assert gpu["act_s"][1, 1] == 0 and not gpu["act_q"][1, 128:256].any()
        assert (gpu["act_s"][1, [0] + list(range(2, shape["hidden"] // 128))] > 0).all()


@pytest.mark.parametrize("rows", [1, 3, 8])
def test_zero_weight_rows_give_zero_mid_blocks(rows):
    """Gate rows 0..127 of every expert (routed and shared) and up rows
    128..255 are zero codes: mid blocks 0 and 1 are zero (silu(0) * up and
    silu(gate) * 0), block 2 is not."""
    layer = S.make_layer(MEDIUM, seed=4200, device="cuda")
    for ew in (layer.routed, layer.shared):
        ew.gate[0][:, 0:128, :] = 0
        ew.up[0][:, 128:256, :] = 0
    x = S.make_x(rows, MEDIUM["hidden"], seed=4300 + rows, mode="corr")
    _say(f"zero weight rows, rows={rows}")
    _, gpu, rep = _run(layer, x)
    _say(rep)
    t = gpu["grp_slot"]
    used = [(r, 8) for r in range(rows)] + [(r, int(t[g][r])) for g in range(gpu["n_groups"])
                                            for r in range(rows) if t[g][r] != 0xFF]
    for r, j in used:
        assert not gpu["midqs"][r, j, :2].any() and not gpu["midq"][r, j, :256].any()
        assert gpu["midqs"][r, j, 2] > 0


# ------------------------------------------------------------------- ties
@pytest.mark.parametrize("rows", [1, 4])
@pytest.mark.parametrize("side", ["lower", "higher"])
def test_exact_tie_across_the_eighth_place(rows, side):
    """Row 0's 8th pick a gets a twin b (a copy of its router row) that is not
    picked: the two logits are bitwise equal, and the lower ID of the two
    must hold the 8th place, the other must be left out."""
    layer = S.make_layer(SMALL, seed=4400, device="cuda")
    x = S.make_x(rows, SMALL["hidden"], seed=4500 + rows)
    runner = B.LayerRunner(layer, rows)
    runner.run(x.cuda())
    gpu = runner.debug(rows)
    ids0 = [int(e) for e in gpu["ids"][0]]
    a = ids0[7]
    rest = [e for e in range(SMALL["n_experts"]) if e not in ids0]
    cands = [e for e in rest if (e < a if side == "lower" else e > a)]
    assert cands, "no expert on that side of the 8th pick for this seed"
    b = cands[0] if side == "lower" else cands[-1]
    layer.router_w[b] = layer.router_w[a]
    _say(f"tie at the 8th place rows={rows}: pick {a}, twin {b}")
    _, gpu, rep = _run(layer, x)
    z = gpu["logits"][0]
    assert z[a] == z[b], "the twin's logit must equal the 8th pick's bit for bit"
    got = [int(e) for e in gpu["ids"][0]]
    assert got[:7] == ids0[:7]
    assert got[7] == min(a, b) and max(a, b) not in got, (got, a, b)


@pytest.mark.parametrize("rows", [1, 8])
def test_many_zero_logits_tie_at_the_eighth_place(rows):
    """All router rows but three are zero: those experts' logits are +0 and
    tie; the picks are the positive logits, then the lowest IDs among the
    zeros (the negative ones come after every zero)."""
    layer = S.make_layer(SMALL, seed=4600, device="cuda")
    keep = [5, 12, 20]
    w = layer.router_w
    mask = torch.ones(SMALL["n_experts"], dtype=torch.bool, device="cuda")
    mask[keep] = False
    w[mask] = 0
    x = S.make_x(rows, SMALL["hidden"], seed=4700 + rows)
    _say(f"zero router rows, rows={rows}")
    _, gpu, rep = _run(layer, x)
    _say(rep)
    for r in range(rows):
        z = gpu["logits"][r]
        pos = sorted([e for e in keep if z[e] > 0], key=lambda e: (-z[e], e))
        zeros = [e for e in range(SMALL["n_experts"]) if z[e] == 0]
        assert len(zeros) >= 29
        expect = (pos + zeros)[:8]
        assert [int(e) for e in gpu["ids"][r]] == expect


# --------------------------------------------------- MXFP4 exponent range
# (gate, up, down) base E8M0 codes per expert class, chosen so that every
# value the fp32 path forms stays finite: gate and up sums near 2^(c-121) at
# hidden 512, mid near their product, down outputs near 2^(cg+cu+cd-364)
MX_CLASSES = [(0, 200, 164), (64, 190, 110), (127, 127, 110), (200, 1, 163), (181, 182, 1),
              (182, 181, 0)]


def _mx_matrix(rng, n, k, base, cls_of_row):
    """MXFP4 [n, k]: uniform random nibbles (so -0, code 8, is as common as
    any other), E8M0 per (row, 32-group) = the row's base code, alternating
    with one step down (bases from 127 up) or up (below 127) from group to
    group; every 7th group (by row + group) holds only zero and -0 nibbles
    under code 254."""
    nib = rng.integers(0, 16, (n, k)).astype(np.uint8)
    g = np.arange(k // 32)[None, :]
    r = np.arange(n)[:, None]
    b = np.asarray([base[c] for c in cls_of_row])[:, None]
    step = np.where(b >= 127, -1, 1)
    e8 = (b + step * ((r + g) % 2)).astype(np.int64)
    zero = (r + g) % 7 == 3
    e8 = np.where(zero, 254, e8).astype(np.uint8)
    zmask = np.repeat(zero, 32, axis=1)
    nib = np.where(zmask, (rng.integers(0, 2, (n, k)) * 8).astype(np.uint8), nib)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, e8


def _mx_edge_layer(seed, inter):
    shape = dict(hidden=512, inter=inter, n_experts=48, shared_inter=0, router_std=0.02)
    base = S.make_layer(shape, routed_fmt=S.FMT_MXFP4, seed=seed, device="cpu")
    rng = np.random.default_rng(seed)
    E, H, I = 48, 512, inter
    mats = {"gate": [], "up": [], "down": []}
    for e in range(E):
        cg, cu, cd = MX_CLASSES[e % len(MX_CLASSES)]
        for name, (n, k), c in (("gate", (I, H), cg), ("up", (I, H), cu), ("down", (H, I), cd)):
            mats[name].append(_mx_matrix(rng, n, k, {0: c}, [0] * n))
    st = lambda name, i: torch.from_numpy(np.stack([m[i] for m in mats[name]])).cuda()
    routed = S.ExpertWeights(S.FMT_MXFP4, (st("gate", 0), st("gate", 1)), (st("up", 0), st("up", 1)),
                             (st("down", 0), st("down", 1)))
    return S.Layer("custom", H, I, E, 0, 1e-6, base.gamma.cuda(), base.router_w.cuda(), routed, None)


# intermediate 256: the down GEMV's whole-line items (I % 256 == 0); 384: its
# half-line items
@pytest.mark.parametrize("inter", [256, 384])
def test_mxfp4_exponent_range_and_negative_zero_nibbles(inter):
    layer = _mx_edge_layer(4800, inter)
    codes = set()
    for m in (layer.routed.gate, layer.routed.up, layer.routed.down):
        codes |= set(np.unique(m[1].cpu().numpy()).tolist())
    for c in (0, 1, 64, 127, 200, 254):
        assert c in codes, c
    seen = set()
    cache = {}
    for rows, mode, seed in ((8, "indep", 4900), (8, "corr", 4901), (4, "indep", 4902),
                             (1, "indep", 4903), (8, "indep", 4904)):
        x = S.make_x(rows, 512, seed=seed, mode=mode)
        _say(f"mxfp4 exponent range inter={inter} rows={rows} mode={mode}")
        _, gpu, rep = _run(layer, x, cache=cache)
        _say(rep)
        seen |= {int(e) % len(MX_CLASSES) for e in gpu["ids"].ravel()}
    assert seen == set(range(len(MX_CLASSES))), seen


# -------------------------------------------------------- FP8 scale range
def test_fp8_block_scales_and_activation_blocks_over_wide_ranges():
    layer = S.make_layer(MEDIUM, seed=5000, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(5001)
    for ew in (layer.routed, layer.shared):
        for m in (ew.gate, ew.up, ew.down):
            ex = torch.randint(-30, 11, m[1].shape, generator=g, device="cuda")
            m[1].copy_(torch.exp2(ex.float()))
    for rows in (1, 4, 8):
        x = S.make_x(rows, MEDIUM["hidden"], seed=5100 + rows).float()
        nb = MEDIUM["hidden"] // 128
        v = (torch.arange(rows * nb).view(rows, nb) * 13) % 41 - 20   # -20 .. 20
        sc = torch.exp2(v.float())
        x = (x.view(rows, -1, 128) * sc[:, :, None]).view(rows, -1).to(torch.bfloat16)
        _say(f"fp8 scale range rows={rows}")
        _, gpu, rep = _run(layer, x)
        _say(rep)
        s = gpu["act_s"][gpu["act_s"] > 0]
        assert s.max() / s.min() > 2.0 ** 20
