"""Pins for the oracle's whole-step arithmetic: hand-worked layers with closed
forms, an independent numpy pipeline built on library decoders and matmul,
invariants, the 1-bit GEMV's closed forms, and the block quantiser."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def bf(v):
    """exact bf16 bit pattern of a python float (asserts exactness)."""
    t = torch.tensor([v], dtype=torch.float64)
    b = t.to(torch.bfloat16)
    assert b.double().item() == v, v
    return int(b.view(torch.int16).item()) & 0xFFFF


# ------------------------------------------------------- hand-worked layer
H, I, E, IS = 256, 256, 9, 128


def _hand_scales():
    """Per-expert block scales chosen so that every block differs (a swapped
    or transposed scale index changes the answer) and no block's gate or up
    sum cancels to exactly zero."""
    a = {e: np.array([[(e + 1) / 256, (e % 2) / 512], [(-1) ** e / 128, 1 / 1024]]) for e in range(E)}
    b = {e: np.array([[1 / 64, -(e + 2) / 1024], [(e + 3) / 512, 5 / 2048]]) for e in range(E)}
    c = {e: np.array([[(e + 1) / 128, -1 / 256], [1 / 512, (e + 5) / 1024]]) for e in range(E)}
    sa = np.array([[1 / 32, 1 / 256]])
    sb = np.array([[-1 / 128, 1 / 64]])
    sc = np.array([[1 / 16], [-1 / 8]])
    return a, b, c, sa, sb, sc


def _hand_inputs():
    x = np.array([bf(1.0)] * 128 + [bf(-2.0)] * 128, np.uint16)[None, :]
    gamma = np.array([bf(1.0)] * H, np.uint16)
    w = np.zeros((E, H), np.uint16)
    for e in range(E):
        w[e, :128] = bf((e + 1) / 64)
        w[e, 128:] = bf((e % 3) / 128)
    return x, gamma, w


def _fp8_all_ones(n, k, scales):
    return np.full((n, k), 0x38, np.uint8), np.ascontiguousarray(scales, np.float32)


def _hand_layer_fp8():
    a, b, c, sa, sb, sc = _hand_scales()
    experts = {}
    for e in range(E):
        experts[e] = (*_fp8_all_ones(I, H, a[e]), *_fp8_all_ones(I, H, b[e]),
                      *_fp8_all_ones(H, I, c[e]))
    shared = (*_fp8_all_ones(IS, H, sa), *_fp8_all_ones(IS, H, sb), *_fp8_all_ones(H, IS, sc))
    return experts, shared


def _closed_form_fp8(act_bf16=False):
    """The step by hand.  x = 1 on block 0 and -2 on block 1, gamma = 1:
    sum x^2 = 640, rstd = 1/sqrt(640/256 + eps).  Router rows are constant per
    block, so raw_e = 128 (e+1)/64 - 256 (e%3)/128 = 2(e+1) - 2(e%3):
    experts 6,7,8 tie at 14, 3,4,5 at 8, 0,1,2 at 2 -> top-8 = 6,7,8,3,4,5,0,1.
    Activation blocks are constant: codes are all +-448 with s0 = fp32(1/448),
    s1 = fp32(2/448) = 2 s0, so h = A rstd on block 0 and -2 A rstd on block 1
    with A = 448 s0.  All weight codes are 1.0, so an output block of a matrix
    with block scales S is 128 A rstd (S[.,0] - 2 S[.,1]); mid is constant per
    block, its FP8 code is +-448 and mhat = sign(mid) 448 s_m with
    s_m = fp32(fp32|mid| / 448).  With bf16 activations the experts' input is
    u rstd itself: A = 1 exactly."""
    a, b, c, sa, sb, sc = _hand_scales()
    eps = float(F32(1e-6))
    rstd = 1.0 / np.sqrt(640.0 / 256 + eps)
    s0 = float(F32(1.0) / F32(448.0))
    A = 1.0 if act_bf16 else 448.0 * s0
    raw = np.array([2 * (e + 1) - 2 * (e % 3) for e in range(E)], float)
    z = rstd * raw
    ids = [6, 7, 8, 3, 4, 5, 0, 1]
    zs = z[ids]
    g = np.exp(zs - zs.max()) / np.exp(zs - zs.max()).sum()

    def expert_y(ga, up, dn):
        G = 128 * A * rstd * (ga[:, 0] - 2 * ga[:, 1])          # per n-block
        U = 128 * A * rstd * (up[:, 0] - 2 * up[:, 1])
        mid = G / (1 + np.exp(-G)) * U
        sm = np.array([float(F32(F32(abs(m)) / F32(448.0))) for m in mid])
        mhat = np.sign(mid) * 448.0 * sm
        y = 128 * (dn @ mhat)                                   # per h-block
        return mid, sm, y

    ys = [expert_y(a[e], b[e], c[e]) for e in ids]
    ysh = expert_y(sa, sb, sc)
    out_blocks = sum(gj * yj[2] for gj, yj in zip(g, ys)) + ysh[2]
    return dict(rstd=rstd, z=z, ids=ids, g=g, s0=s0, ys=ys, ysh=ysh, out=np.repeat(out_blocks, 128))


def test_hand_worked_layer_fp8():
    x, gamma, w = _hand_inputs()
    experts, shared = _hand_layer_fp8()
    cfg = dict(hidden=H, inter=I, n_experts=E, shared_inter=IS, rows=1, rms_eps=1e-6,
               routed_fmt=O.FMT_FP8)
    out, d = O.moe_step(cfg, x, gamma, w, experts, shared)
    cf = _closed_form_fp8()
    assert d["rstd"][0] == pytest.approx(cf["rstd"], rel=1e-15)
    assert np.allclose(d["z"][0], cf["z"], rtol=1e-14, atol=0)
    assert list(d["ids"][0]) == cf["ids"]
    assert np.allclose(d["gates"][0], cf["g"], rtol=1e-13, atol=0)
    # activation blocks: +-448 codes, scales s0 and 2 s0
    assert set(d["act_q"][0, :128]) == {0x7E} and set(d["act_q"][0, 128:]) == {0xFE}
    assert d["act_s"][0, 0] == F32(cf["s0"]) and d["act_s"][0, 1] == F32(2 * cf["s0"])
    for j in range(8):
        mid, sm, y = cf["ys"][j]
        assert np.allclose(d["mid"][0, j, :I], np.repeat(mid, 128), rtol=1e-13, atol=0)
        assert np.array_equal(d["midqs"][0, j, :2], sm.astype(F32))
        codes = d["midq"][0, j, :I].reshape(2, 128)
        for blk in range(2):
            assert set(codes[blk]) == {0x7E if mid[blk] > 0 else 0xFE}
        assert np.allclose(d["y"][0, j], np.repeat(y, 128), rtol=1e-13, atol=0)
    mid, sm, y = cf["ysh"]
    assert np.allclose(d["y"][0, 8], np.repeat(y, 128), rtol=1e-13, atol=0)
    # sums of |terms| of gate / up (used for rounding bounds): 128 A rstd (|S0| + 2|S1|)
    a, b, _, _, _, _ = _hand_scales()
    A = 448.0 * cf["s0"]
    for j, e in enumerate(cf["ids"]):
        for mats, key in ((a, "gate_abs"), (b, "up_abs")):
            blk = 128 * A * cf["rstd"] * (np.abs(mats[e][:, 0]) + 2 * np.abs(mats[e][:, 1]))
            assert np.allclose(d[key][0, j, :I], np.repeat(blk, 128), rtol=1e-13, atol=0)
            # constant terms within each group of 8: the group maxima are 1/8 of that
            gkey = key.replace("_abs", "_gmax")
            assert np.allclose(d[gkey][0, j, :I], np.repeat(blk, 128) / 8, rtol=1e-13, atol=0)
    assert np.allclose(d["out_f64"][0], cf["out"], rtol=1e-13, atol=0)
    assert np.array_equal(out[0], O.round_bf16_n(d["out_f64"][0]))


def test_hand_worked_layer_bf16_activations():
    """The same layer with the experts' input left in bf16 (no FP8 blocks):
    h = +-rstd and -+2 rstd exactly, no activation codes or scales."""
    x, gamma, w = _hand_inputs()
    experts, shared = _hand_layer_fp8()
    cfg = dict(hidden=H, inter=I, n_experts=E, shared_inter=IS, rows=1, rms_eps=1e-6,
               routed_fmt=O.FMT_FP8, act_fmt=O.ACT_BF16)
    out, d = O.moe_step(cfg, x, gamma, w, experts, shared)
    cf = _closed_form_fp8(act_bf16=True)
    assert list(d["ids"][0]) == cf["ids"]
    assert not d["act_q"].any() and not d["act_s"].any()
    for j in range(8):
        mid, sm, y = cf["ys"][j]
        assert np.allclose(d["mid"][0, j, :I], np.repeat(mid, 128), rtol=1e-13, atol=0)
        assert np.array_equal(d["midqs"][0, j, :2], sm.astype(F32))
        assert np.allclose(d["y"][0, j], np.repeat(y, 128), rtol=1e-13, atol=0)
    assert np.allclose(d["out_f64"][0], cf["out"], rtol=1e-13, atol=0)
    # the FP8 blocks' scale is not exactly 1/448 of amax in fp32, so the two
    # modes differ (a dropped or doubled activation scale would show here)
    _, d8 = O.moe_step(dict(cfg, act_fmt=O.ACT_FP8), x, gamma, w, experts, shared)
    assert not np.array_equal(d8["mid"], d["mid"])
    assert np.allclose(d8["mid"], d["mid"], rtol=1e-6, atol=0)


def test_hand_worked_layer_mxfp4():
    """MXFP4 routed experts: every E2M1 code is 1.0 (nibble 0x2), E8M0
    exponents differ per (row, 32-group), mid is not re-quantised."""
    x, gamma, w = _hand_inputs()
    rng = np.random.default_rng(5)
    experts = {}
    for e in range(E):
        mats = []
        for (n, k) in ((I, H), (I, H), (H, I)):
            codes = np.full((n, k // 2), 0x22, np.uint8)
            ex = rng.integers(123, 129, size=(n, k // 32)).astype(np.uint8)
            mats += [codes, ex]
        experts[e] = tuple(mats)
    _, shared = _hand_layer_fp8()
    cfg = dict(hidden=H, inter=I, n_experts=E, shared_inter=IS, rows=1, rms_eps=1e-6,
               routed_fmt=O.FMT_MXFP4)
    out, d = O.moe_step(cfg, x, gamma, w, experts, shared)
    cf = _closed_form_fp8()
    rstd, A = cf["rstd"], 448.0 * cf["s0"]
    h = np.concatenate([np.full(128, A * rstd), np.full(128, -2 * A * rstd)])
    acc = np.zeros(H)
    for j, e in enumerate(cf["ids"]):
        gx, ux, dx = (2.0 ** (experts[e][i].astype(float) - 127) for i in (1, 3, 5))
        # each 32-group contributes 32 * 2^(X-127) * h_group (all codes are 1.0)
        hg = h.reshape(-1, 32)[:, 0]
        G = 32 * gx @ hg
        U = 32 * ux @ hg
        mid = G / (1 + np.exp(-G)) * U
        assert np.allclose(d["mid"][0, j, :I], mid, rtol=1e-12, atol=1e-13 * np.abs(mid).max())
        y = dx @ mid.reshape(-1, 32).sum(axis=1)
        assert np.allclose(d["y"][0, j], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
        acc += cf["g"][j] * y
    acc += np.repeat(cf["ysh"][2], 128)
    assert np.allclose(d["out_f64"][0], acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())


# ------------------------------------- independent numpy pipeline (random)
def _np_fp8(codes, scales):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    return v * s


def _np_mxfp4(codes, e8m0):
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], float)
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    v = mags[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return v * np.repeat(2.0 ** (e8m0.astype(float) - 127), 32, axis=1)


def _np_step(layer, x, routed_fmt, act_fmt=0):
    """Numpy + torch-dtype reimplementation used only as a cross-check."""
    import bit_moe_decode_amd.synth as S  # generator only
    tb = lambda t: t.float().double().numpy() if t.dtype == torch.bfloat16 else t.numpy()
    xv = x.double().numpy()
    gam = layer.gamma.double().numpy()
    wr = layer.router_w.double().numpy()
    R = xv.shape[0]
    out = np.zeros((R, layer.hidden))
    for r in range(R):
        rstd = 1 / np.sqrt((xv[r] ** 2).sum() / layer.hidden + float(F32(layer.rms_eps)))
        u = torch.from_numpy(xv[r] * gam).to(torch.float32).to(torch.bfloat16).double().numpy()
        z = rstd * (wr @ u)
        ids = np.lexsort((np.arange(z.size), -z))[:8]
        g = np.exp(z[ids] - z[ids].max())
        g /= g.sum()
        ub = u.reshape(-1, 128)
        s = (np.abs(ub).max(axis=1).astype(F32) / F32(448)).astype(F32)
        q = torch.from_numpy((ub.astype(F32) / s[:, None]).astype(F32)).to(torch.float8_e4m3fn)
        h = (q.double().numpy() * s[:, None]).ravel() * rstd
        if act_fmt == O.ACT_BF16:
            h = u * rstd

        def ffn(mats, fmt):
            dec = _np_fp8 if fmt == O.FMT_FP8 else _np_mxfp4
            Wg, Wu, Wd = dec(mats[0], mats[1]), dec(mats[2], mats[3]), dec(mats[4], mats[5])
            gt, up = Wg @ h, Wu @ h
            mid = gt / (1 + np.exp(-gt)) * up
            if fmt == O.FMT_FP8:
                mb = mid.astype(F32).reshape(-1, 128)
                sm = (np.abs(mb).max(axis=1) / F32(448)).astype(F32)
                mq = torch.from_numpy((mb / sm[:, None]).astype(F32)).to(torch.float8_e4m3fn)
                mid = (mq.double().numpy() * sm[:, None]).ravel()
            return Wd @ mid

        acc = sum(g[j] * ffn([t.numpy() for t in layer.routed.expert(int(e))], routed_fmt)
                  for j, e in enumerate(ids))
        if layer.shared is not None:
            acc = acc + ffn([t.numpy() for t in layer.shared.expert(0)], O.FMT_FP8)
        out[r] = acc
    return out


def _run_oracle(layer, x, act_fmt=0, **kw):
    import bit_moe_decode_amd.synth as S
    xb = S.bf16_bits(x).numpy().view(np.uint16)
    experts = {e: tuple(None if t is None else t.numpy() for t in layer.routed.expert(e))
               for e in range(layer.n_experts)}
    shared = tuple(t.numpy() for t in layer.shared.expert(0)) if layer.shared is not None else None
    cfg = dict(hidden=layer.hidden, inter=layer.inter, n_experts=layer.n_experts,
               shared_inter=layer.shared_inter, rows=x.shape[0], rms_eps=layer.rms_eps,
               routed_fmt=layer.routed_fmt, act_fmt=act_fmt)
    return O.moe_step(cfg, xb, S.bf16_bits(layer.gamma).numpy().view(np.uint16),
                      S.bf16_bits(layer.router_w).numpy().view(np.uint16), experts, shared, **kw)


@pytest.mark.parametrize("fmt,act", [(O.FMT_FP8, O.ACT_FP8), (O.FMT_MXFP4, O.ACT_FP8),
                                     (O.FMT_FP8, O.ACT_BF16)])
def test_oracle_matches_independent_numpy_pipeline(fmt, act):
    import bit_moe_decode_amd.synth as S
    layer = S.make_layer("tiny", routed_fmt=fmt, seed=1000)
    # give the tiny layer a shared expert too, so that path is pinned as well
    layer.shared = S.make_layer("tiny", routed_fmt=S.FMT_FP8, seed=77).routed
    layer.shared = S.ExpertWeights(S.FMT_FP8, *[(m[0][:1], m[1][:1]) for m in
                                               (layer.shared.gate, layer.shared.up, layer.shared.down)])
    layer.shared_inter = layer.inter
    x = S.make_x(4, layer.hidden, seed=2000)
    out, d = _run_oracle(layer, x, act_fmt=act)
    ref = _np_step(layer, x, fmt, act)
    assert np.allclose(d["out_f64"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # the group-of-8 maxima of the gate terms, from the same decoders
    dec = _np_fp8 if fmt == O.FMT_FP8 else _np_mxfp4
    r, j = 1, 3
    e = int(d["ids"][r, j])
    m = [t.numpy() for t in layer.routed.expert(e)]
    Wg = dec(m[0], m[1])
    if act == O.ACT_BF16:
        h = O.dec_bf16_n(d["u"][r]) * d["rstd"][r]
    else:
        h = O.dec_e4m3_n(d["act_q"][r]) * np.repeat(d["act_s"][r].astype(float), 128) * d["rstd"][r]
    gm = np.abs(Wg * h[None, :]).reshape(Wg.shape[0], -1, 8).max(axis=2).sum(axis=1)
    assert np.allclose(d["gate_gmax"][r, j, :layer.inter], gm, rtol=1e-12, atol=0)


# ---------------------------------------------------------- invariants
def test_rows_are_independent_and_permutation_equivariant():
    import bit_moe_decode_amd.synth as S
    layer = S.make_layer("tiny", seed=1001)
    x = S.make_x(5, layer.hidden, seed=2001)
    out, d = _run_oracle(layer, x)
    perm = [3, 0, 4, 1, 2]
    out_p, _ = _run_oracle(layer, x[perm])
    assert np.array_equal(out_p, out[perm])
    for r in range(5):
        o1, _ = _run_oracle(layer, x[r:r + 1])
        assert np.array_equal(o1[0], out[r])
    assert np.allclose(d["gates"].sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_anchored_selection_follows_the_given_logits():
    import bit_moe_decode_amd.synth as S
    layer = S.make_layer("tiny", seed=1002)
    x = S.make_x(2, layer.hidden, seed=2002)
    _, d = _run_oracle(layer, x)
    anchor = d["z"].astype(np.float32)
    _, da = _run_oracle(layer, x, anchor_z=anchor)
    assert np.array_equal(da["ids"], d["ids"])
    # force a different choice through the anchor only
    anchor2 = anchor.copy()
    anchor2[:, 0] = 1e9
    _, db = _run_oracle(layer, x, anchor_z=anchor2)
    assert (db["ids"][:, 0] == 0).all()


# ------------------------------------------------------- block quantiser
def test_quant_blocks_properties():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(128 * 40) * np.exp2(rng.integers(-8, 8, 128 * 40))).astype(F32)
    v[128:256] = 0.0
    q, s = O.quant_blocks(v)
    assert s[1] == 0 and np.all(q[128:256] == 0)
    vals = O.dec_e4m3_n(q).reshape(-1, 128)
    vb = v.reshape(-1, 128)
    for b in range(40):
        if b == 1:
            continue
        amax = np.abs(vb[b]).max()
        assert s[b] == F32(amax) / F32(448)
        # the block maximum lands on the largest code
        assert np.abs(vals[b]).max() == 448.0
        # each code is a nearest E4M3 value: error <= half a code spacing (2^-4 relative)
        rec = vals[b] * s[b]
        big = np.abs(vb[b]) >= 2.0 ** -6 * s[b]
        assert np.all(np.abs(rec - vb[b])[big] <= np.abs(vb[b][big]) * 2.0 ** -4 + 1e-30)


def test_midq_layout_size_matches_the_pages():
    """#85 Layout: midq and midqs take 19 KB at 4 rows and 38 KB at 8 (mid
    blocks of 1x128 with one fp32 scale, 8 routed + 1 shared slot, the 4-way
    tensor-parallel share of intermediate 2048 = 512)."""
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)["midq_layout"]
    for rows, kb in ((4, facts["kb_at_4_rows"]), (8, facts["kb_at_8_rows"])):
        mid = np.ones((rows, 9, 512), F32)
        q, s = O.quant_blocks(mid.ravel())
        total = q.nbytes + s.nbytes
        assert round(total / 1000) == kb, (rows, total)


# ------------------------------------------------------------ 1-bit closed forms
def _q1_blocks(bits, d16):
    n, groups = d16.shape
    blk = np.zeros((n, groups, 18), np.uint8)
    dv = d16.view(np.uint16)
    blk[..., 0] = dv & 0xFF
    blk[..., 1] = dv >> 8
    blk[..., 2:] = bits
    return blk


def test_q1_all_plus_and_all_minus_closed_form():
    rng = np.random.default_rng(12)
    n, k = 37, 384
    d16 = np.abs(rng.standard_normal((n, k // 128)) * 0.02).astype(np.float16)
    x = torch.randn(k, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    xs = x.double().numpy().reshape(-1, 128).sum(axis=1)
    expect = d16.astype(np.float64) @ xs
    _, yp = O.lowbit_gemv_q1(_q1_blocks(np.zeros((n, k // 128, 16), np.uint8), d16), xb, n, k)
    _, ym = O.lowbit_gemv_q1(_q1_blocks(np.full((n, k // 128, 16), 255, np.uint8), d16), xb, n, k)
    assert np.allclose(yp, expect, rtol=1e-13, atol=1e-300)
    assert np.allclose(ym, -expect, rtol=1e-13, atol=1e-300)


def test_q1_single_bit_flips_one_element():
    rng = np.random.default_rng(13)
    n, k = 4, 256
    d16 = np.abs(rng.standard_normal((n, 2))).astype(np.float16) + np.float16(0.5)
    x = torch.randn(k, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    xv = x.double().numpy()
    base = np.zeros((n, 2, 16), np.uint8)
    _, y0 = O.lowbit_gemv_q1(_q1_blocks(base, d16), xb, n, k)
    for (g, byte, bit) in ((0, 0, 0), (0, 5, 3), (1, 15, 7), (1, 2, 6)):
        b = base.copy()
        b[:, g, byte] = 1 << bit
        _, y1 = O.lowbit_gemv_q1(_q1_blocks(b, d16), xb, n, k)
        elem = g * 128 + 8 * byte + bit
        assert np.allclose(y1, y0 - 2 * d16[:, g].astype(float) * xv[elem], rtol=1e-12, atol=1e-12)


def test_q1_random_against_unpackbits():
    import bit_moe_decode_amd.synth as S
    n, k = 300, 1024
    blk = S.make_q1(n, k, seed=5).numpy()
    x = S.make_x(1, k, seed=6)[0]
    xb = S.bf16_bits(x).numpy().view(np.uint16)
    y, yf = O.lowbit_gemv_q1(blk, xb, n, k, nthreads=4)
    d = blk[..., :2].copy().view(np.float16)[..., 0].astype(np.float64)
    bits = np.unpackbits(blk[..., 2:], axis=-1, bitorder="little")   # [n, g, 128]
    sign = 1.0 - 2.0 * bits
    ref = np.einsum("ng,ngk,gk->n", d, sign, x.double().numpy().reshape(-1, 128))
    assert np.allclose(yf, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(y, O.round_bf16_n(yf))


def test_q1_block_size_matches_the_pages():
    """1-Bit Turbo: 572 MB files for 4B-parameter models -> about 1.14 bits a
    weight; an 18-byte block of 128 weights is 1.125 bits a weight."""
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)["q1_size"]
    bpw = facts["file_mb"] * 1e6 * 8 / (facts["params_b"] * 1e9)
    assert abs(bpw - 18 * 8 / 128) < 0.03


# ------------------------------------------- 1-bit (Q1_0_G128) routed experts
def _q1_const(n, k, d_blocks, minus=False):
    """Q1 matrix [n, k] with every sign + (or every sign -) and group scale
    d_blocks[n // 128][g] (fp16-exact values)."""
    groups = k // 128
    d = np.repeat(np.asarray(d_blocks, np.float64), 128, axis=0)[:n, :groups].astype(np.float16)
    assert np.array_equal(d.astype(np.float64), np.repeat(np.asarray(d_blocks), 128, axis=0)[:n])
    blk = np.zeros((n, groups, 18), np.uint8)
    dv = d.view(np.uint16)
    blk[..., 0] = dv & 0xFF
    blk[..., 1] = dv >> 8
    blk[..., 2:] = 0xFF if minus else 0
    return blk


def test_hand_worked_layer_q1():
    """1-bit routed experts whose signs are all + and whose group scales d are
    the FP8 hand-worked layer's block scales: each matrix equals that layer's
    (every FP8 code there is 1.0), so the step reproduces its closed form --
    mid re-quantised to FP8 per 1x128 block as for FP8 experts.  Flipping
    every sign bit of one expert's down matrix negates its output."""
    x, gamma, w = _hand_inputs()
    a, b, c, _, _, _ = _hand_scales()
    _, shared = _hand_layer_fp8()
    experts = {e: (_q1_const(I, H, a[e]), None, _q1_const(I, H, b[e]), None,
                   _q1_const(H, I, c[e]), None) for e in range(E)}
    cfg = dict(hidden=H, inter=I, n_experts=E, shared_inter=IS, rows=1, rms_eps=1e-6,
               routed_fmt=O.FMT_Q1)
    out, d = O.moe_step(cfg, x, gamma, w, experts, shared)
    cf = _closed_form_fp8()
    assert list(d["ids"][0]) == cf["ids"]
    for j in range(8):
        mid, sm, y = cf["ys"][j]
        assert np.allclose(d["mid"][0, j, :I], np.repeat(mid, 128), rtol=1e-13, atol=0)
        assert np.array_equal(d["midqs"][0, j, :2], sm.astype(F32))
        assert np.allclose(d["y"][0, j], np.repeat(y, 128), rtol=1e-13, atol=0)
    assert np.allclose(d["out_f64"][0], cf["out"], rtol=1e-13, atol=0)
    e0 = cf["ids"][0]
    flipped = dict(experts)
    flipped[e0] = experts[e0][:4] + (_q1_const(H, I, c[e0], minus=True), None)
    _, d2 = O.moe_step(cfg, x, gamma, w, flipped, shared)
    assert np.array_equal(d2["y"][0, 0], -d["y"][0, 0])
    assert np.array_equal(d2["y"][0, 1:], d["y"][0, 1:])


def _np_q1(blocks):
    """Independent decode of Q1 blocks [n, g, 18]: d * (1 - 2 bit)."""
    n, groups, _ = blocks.shape
    d = blocks[..., :2].copy().view(np.float16)[..., 0].astype(np.float64)
    bits = np.unpackbits(blocks[..., 2:], axis=-1, bitorder="little").astype(np.float64)
    return (d[..., None] * (1.0 - 2.0 * bits)).reshape(n, groups * 128)


def test_oracle_q1_layer_matches_independent_numpy_pipeline():
    import bit_moe_decode_amd.synth as S
    shape = dict(hidden=256, inter=256, n_experts=32, shared_inter=256, router_std=0.02)
    layer = S.make_layer(shape, routed_fmt=S.FMT_Q1, seed=1020)
    x = S.make_x(3, 256, seed=2020)
    out, d = _run_oracle(layer, x)
    xv = x.double().numpy()
    gam = layer.gamma.double().numpy()
    wr = layer.router_w.double().numpy()
    for r in range(3):
        rstd = 1 / np.sqrt((xv[r] ** 2).sum() / 256 + float(F32(1e-6)))
        u = torch.from_numpy(xv[r] * gam).to(torch.float32).to(torch.bfloat16).double().numpy()
        z = rstd * (wr @ u)
        ids = np.lexsort((np.arange(z.size), -z))[:8]
        assert list(ids) == list(d["ids"][r])
        g = np.exp(z[ids] - z[ids].max())
        g /= g.sum()
        ub = u.reshape(-1, 128)
        s = (np.abs(ub).max(axis=1).astype(F32) / F32(448)).astype(F32)
        q = torch.from_numpy((ub.astype(F32) / s[:, None]).astype(F32)).to(torch.float8_e4m3fn)
        h = (q.double().numpy() * s[:, None]).ravel() * rstd

        def ffn(m, q1):
            if q1:
                Wg, Wu, Wd = _np_q1(m[0]), _np_q1(m[2]), _np_q1(m[4])
            else:
                Wg, Wu, Wd = _np_fp8(m[0], m[1]), _np_fp8(m[2], m[3]), _np_fp8(m[4], m[5])
            gt, up = Wg @ h, Wu @ h
            mid = (gt / (1 + np.exp(-gt)) * up).astype(F32).reshape(-1, 128)
            sm = (np.abs(mid).max(axis=1) / F32(448)).astype(F32)
            mq = torch.from_numpy((mid / sm[:, None]).astype(F32)).to(torch.float8_e4m3fn)
            return Wd @ (mq.double().numpy() * sm[:, None]).ravel()

        ref = sum(g[j] * ffn([None if t is None else t.numpy()
                              for t in layer.routed.expert(int(e))], True)
                  for j, e in enumerate(ids))
        ref = ref + ffn([t.numpy() for t in layer.shared.expert(0)], False)
        assert np.allclose(d["out_f64"][r], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
