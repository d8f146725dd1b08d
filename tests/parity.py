"""Comparison of the HIP path's step (outputs and intermediates) with the
oracle, shared by the GPU parity tests, the smoke check and the benchmark's
spot checks.  Test infrastructure: imports the oracle."""
import numpy as np
import torch

from oracle import oracle as O

OUT_TOL = 2e-2          # max|out - ref| <= OUT_TOL * max|ref|


def np_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def expert_host(layer, e):
    return tuple(None if t is None else t.cpu().numpy() for t in layer.routed.expert(int(e)))


def shared_host(layer):
    if layer.shared is None:
        return None
    return tuple(t.cpu().numpy() for t in layer.shared.expert(0))


def oracle_for(layer, x, gpu_logits, nthreads=1, host_cache=None, act_fmt=0):
    """Oracle step on the same inputs, selection anchored on the GPU's fp32
    logits.  Only the experts those logits pick are copied to the host."""
    R = x.shape[0]
    E = layer.n_experts
    ids = np.stack([O.top8(gpu_logits[r].astype(np.float64)) for r in range(R)])
    cache = host_cache if host_cache is not None else {}
    for e in np.unique(ids):
        if int(e) not in cache:
            cache[int(e)] = expert_host(layer, e)
    experts = {int(e): cache[int(e)] for e in np.unique(ids)}
    cfg = dict(hidden=layer.hidden, inter=layer.inter, n_experts=E,
               shared_inter=layer.shared_inter, rows=R, rms_eps=layer.rms_eps,
               routed_fmt=layer.routed_fmt, act_fmt=act_fmt)
    if "shared" not in cache:
        cache["shared"] = shared_host(layer)
    out, dbg = O.moe_step(cfg, np_u16(x), np_u16(layer.gamma), np_u16(layer.router_w), experts,
                          cache["shared"], anchor_z=gpu_logits.astype(np.float32),
                          nthreads=nthreads)
    dbg["_host"] = cache          # the host copies of the picked experts, for the down check
    dbg["_nthreads"] = nthreads
    dbg["_act_fmt"] = act_fmt
    return out, dbg


def codes_equal(a, b):
    """FP8 codes equal, +0 and -0 counted equal."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    z = ((a & 0x7F) == 0) & ((b & 0x7F) == 0)
    return (a == b) | z


def _e4m3_order(c):
    """Monotone integer position of an E4M3 code on the number line."""
    c = np.asarray(c, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


U32 = 2.0 ** -24


# The gfx950 scaled FP8 / FP4 x FP8 MFMA (16x16x128) does not sum its 128
# products as fp32 does: measured on the device with in-bounds probes (random
# codes over the whole E4M3 range, quantised N(0,1) blocks, and one large
# product beside small ones), it adds each group of 8 consecutive products
# after aligning them to the group's largest and truncating at 13 bits below
# its leading bit (a product 2^-14 below the group's largest is lost, one in
# another group is kept), then adds the group sums.  So per MFMA
#   |err| <= 7 * 2^-13 * sum over groups of the group's largest |product|
#            + 16 * 2^-23 * sum |products|,
# a bound the probes' 768K outputs met with 3x margin.  The bf16 MFMA
# (16x16x32) summed like fp32 in the same probes.
MFMA8_GROUP = 7 * 2.0 ** -13     # per group of 8, times its largest |term|
MFMA8_SUMS = 32 * U32            # the group sums, times sum |terms|


def mid_tau(gate, up, gate_abs, up_abs, nkb, gate_gmax=None, up_gmax=None):
    """Bound on |mid_gpu - mid_exact| from the kernel's arithmetic.  With FP8
    activations (gate_gmax / up_gmax given: the oracle's sums over groups of
    8 consecutive k of the largest |term|) each K block's gate / up sum is one
    scaled FP8 MFMA, bounded by the model above; with bf16 activations it is
    four 16x16x32 bf16 MFMAs, bounded as an fp32 sum with truncation
    (128 * 2^-23 * sum|terms|).  Then nkb block partials scaled and summed in
    fp32 (within K parts, then the parts in order: nkb - 1 additions in all)
    and two scale products and the rstd product rounded: (nkb + 6) * 2^-24 *
    sum|terms|.  mid = g sigma(g) u then carries |d mid/dg| dg + |d mid/du| du
    plus eight fp32 roundings of the SiLU evaluation."""
    if gate_gmax is not None:
        dg = MFMA8_GROUP * gate_gmax + (MFMA8_SUMS + (nkb + 6) * U32) * gate_abs
        du = MFMA8_GROUP * up_gmax + (MFMA8_SUMS + (nkb + 6) * U32) * up_abs
    else:
        eps = 128 * 2.0 ** -23 + (nkb + 6) * U32
        dg = eps * gate_abs
        du = eps * up_abs
    sig = 1.0 / (1.0 + np.exp(-np.clip(gate, -700, 700)))
    dmid_dg = np.abs(sig * (1.0 + gate * (1.0 - sig)) * up)
    dmid_du = np.abs(gate * sig)
    mid = gate * sig * up
    return dmid_dg * dg + dmid_du * du + 8 * U32 * np.abs(mid) + dg * du


def _window(centre, half_width, scale):
    """Number-line positions of the E4M3 roundings of the two ends of the
    interval [centre - half_width, centre + half_width] divided by `scale`
    (rounding is monotone, so they bracket every admissible code)."""
    lo = O.enc_e4m3_n(((centre - half_width) / scale).astype(np.float32))
    hi = O.enc_e4m3_n(((centre + half_width) / scale).astype(np.float32))
    return _e4m3_order(lo), _e4m3_order(hi)


def _code_in_window(codes, centre, half_width, scale):
    """True where `codes` is the E4M3 rounding of some value of the interval
    [centre - half_width, centre + half_width] divided by `scale`; +0 and -0
    sit at the same position."""
    olo, ohi = _window(centre, half_width, scale)
    c = _e4m3_order(codes)
    return (olo <= c) & (c <= ohi)


def down_bound(fmt, inter):
    """(a, b): the device's down GEMV on its own mid is within a * y_gmax +
    b * y_abs of the exact sum (y_abs = sum_k |W[n,k] mhat_k|, y_gmax = the
    sum over groups of 8 consecutive k of the largest such term), from its
    arithmetic.  FP8 (and 1-bit, whose weights enter as E4M3 +-1): per
    128-wide K block one scaled FP8 MFMA (the model above), the weight-scale
    (or group d) x mid-scale product rounded once, and inter/128 fused
    multiply-adds into the fp32 accumulator: (inter/128 + 4) * 2^-24 more.  MXFP4: the weights converted to bf16 exactly (an E2M1 value times a
    power of two), mid split into bf16 hi + lo (|mid - hi - lo| <= 2^-18
    |mid|), and 2 * inter exact fp32 products summed through the bf16 MFMA
    chain, bounded as a sequential fp32 sum with truncation."""
    if fmt in (O.FMT_FP8, O.FMT_Q1):  # 1-bit: +-1 E4M3 weights, then d x mid scale
        return MFMA8_GROUP, MFMA8_SUMS + (inter // 128 + 4) * U32
    return 0.0, 2 * inter * 2.0 ** -23 + 2.0 ** -17


def compare(layer, x, gpu, out_gpu, ref_out, ref, check_mid_codes=True):
    """All checks of one step.  gpu: LayerRunner.debug() dict; ref: oracle
    debug dict.  Returns a dict of measured errors; raises AssertionError on
    a failed check."""
    R, H = x.shape
    rep = {}
    # T1 -- selection bit-exact, anchored on the GPU's own logits
    ids_ref = np.stack([O.top8(gpu["logits"][r].astype(np.float64)) for r in range(R)])
    assert np.array_equal(gpu["ids"], ids_ref), ("top-8 differs", gpu["ids"], ids_ref)
    assert np.array_equal(ref["ids"], ids_ref)
    # router logits against the fp64 ones (selection is judged on the GPU's)
    zr = ref["z"]
    zerr = np.abs(gpu["logits"] - zr).max()
    rep["logit_err"] = float(zerr / max(np.abs(zr).max(), 1e-30))
    assert zerr <= 1e-3 * np.abs(zr).max() + 1e-6, ("router logits", zerr)
    assert np.allclose(gpu["rstd"], ref["rstd"], rtol=1e-5, atol=0)
    assert np.allclose(gpu["gates"], ref["gates"], rtol=0, atol=1e-4)
    # T2 -- dedup table bit-exact against the oracle's table of the GPU's picks
    t = O.dedup(gpu["ids"])
    assert gpu["n_groups"] == t["n"], ("group count", gpu["n_groups"], t["n"])
    assert np.array_equal(gpu["grp_expert"], t["expert"])
    assert np.array_equal(gpu["grp_owner"][:, 0], t["owner_slot"])
    assert np.array_equal(gpu["grp_owner"][:, 1], t["owner_row"])
    assert np.array_equal(gpu["grp_mask"], t["mask"])
    assert np.array_equal(gpu["grp_slot"], t["slot"])
    rep["n_groups"] = int(t["n"])
    # T3 -- activation blocks: scales and codes bit-exact
    assert np.array_equal(gpu["act_s"], ref["act_s"]), "activation scales"
    assert codes_equal(gpu["act_q"], ref["act_q"]).all(), "activation codes"
    # T4 -- mid
    tot = ndiff = n_ulp = n_tau = n_adj = 0
    worst = 0.0
    nkb = H // 128
    for slot in range(1 + t["n"]):
        if slot == 0:
            if layer.shared is None:
                continue
            users = [(r, 8) for r in range(R)]
            width, fp8 = layer.shared_inter, True
        else:
            g = slot - 1
            users = [(r, int(t["slot"][g][r])) for r in range(R) if t["slot"][g][r] != 0xFF]
            # 1-bit experts' mid is FP8 like FP8 experts'
            width, fp8 = layer.inter, layer.routed_fmt in (O.FMT_FP8, O.FMT_Q1)
        for r, j in users:
            mg = gpu["mid"][r, j, :width].astype(np.float64)
            mo = ref["mid"][r, j, :width]
            fp8_act = ref.get("_act_fmt", O.ACT_FP8) == O.ACT_FP8
            tau = mid_tau(ref["gate"][r, j, :width], ref["up"][r, j, :width],
                          ref["gate_abs"][r, j, :width], ref["up_abs"][r, j, :width], nkb,
                          ref["gate_gmax"][r, j, :width] if fp8_act else None,
                          ref["up_gmax"][r, j, :width] if fp8_act else None)
            dev = np.abs(mg - mo)
            worst = max(worst, float((dev / (tau + 1e-300)).max()))
            assert (dev <= tau).all(), ("mid outside its rounding bound", slot, r,
                                        float((dev / tau).max()))
            if not fp8 or not check_mid_codes:
                continue
            qg = gpu["midq"][r, j, :width]
            sg = gpu["midqs"][r, j, :width // 128]
            # (i) anchored: the oracle's quantiser on the GPU's fp32 mid, bit-exact
            q, s = O.quant_blocks(mg.astype(np.float32))
            assert np.array_equal(sg, s), ("midqs anchored", slot, r)
            assert codes_equal(qg, q).all(), ("midq anchored", slot, r)
            # (ii) end to end against the oracle's own codes
            qo = ref["midq"][r, j, :width]
            diff = ~codes_equal(qg, qo)
            sgx = np.repeat(sg.astype(np.float64), 128)
            # an all-zero block (scale 0) has zero codes on both sides
            zb = sgx == 0
            assert not (diff & zb).any() and not (qo[zb] & 0x7F).any(), ("zero mid block", slot, r)
            diff &= ~zb
            sgx = np.where(zb, 1.0, sgx)
            in_ulp = _code_in_window(qg, mo, np.abs(mo / sgx) * 2.0 ** -23 * sgx, sgx)
            half = tau + np.abs(mo) * 2.0 ** -23
            in_tau = _code_in_window(qg, mo, half, sgx)
            assert in_tau[diff].all(), ("mid code not a rounding of any value within tau",
                                        slot, r, int((diff & ~in_tau).sum()))
            # adjacency: where the window reaches at most one rounding boundary,
            # a differing code must be a neighbour of the oracle's
            olo, ohi = _window(mo, half, sgx)
            narrow = (ohi - olo) <= 1
            step = np.abs(_e4m3_order(qg) - _e4m3_order(qo))
            assert (step[diff & narrow] <= 1).all(), ("mid code not adjacent", slot, r)
            tot += width
            ndiff += int(diff.sum())
            n_ulp += int((diff & in_ulp).sum())
            n_tau += int((diff & in_tau).sum())
            n_adj += int((diff & narrow).sum())
    rep["mid_tau_use_max"] = worst
    rep["midq_codes"] = tot
    rep["midq_diff"] = ndiff
    rep["midq_diff_in_1ulp"] = n_ulp
    rep["midq_diff_in_tau"] = n_tau
    rep["midq_diff_adjacent_checked"] = n_adj
    # T4b -- the down GEMV judged on the GPU's own mid: every (row, pick)'s
    # fp32 down output against the oracle's down GEMV of the GPU's mid codes
    # and scales (FP8 experts) or fp32 mid (MXFP4 experts), element by element
    host = ref.get("_host")
    if host is not None and "y" in gpu:
        y_worst, n_y = 0.0, 0
        for slot in range(1 + t["n"]):
            if slot == 0:
                if layer.shared is None:
                    continue
                users = [(r, 8) for r in range(R)]
                width, fmt, mats = layer.shared_inter, O.FMT_FP8, host["shared"]
            else:
                g = slot - 1
                users = [(r, int(t["slot"][g][r])) for r in range(R) if t["slot"][g][r] != 0xFF]
                width, fmt = layer.inter, layer.routed_fmt
                mats = host[int(t["expert"][g])]
            ba, bb = down_bound(fmt, width)
            for r, j in users:
                if fmt in (O.FMT_FP8, O.FMT_Q1):
                    yref, yabs, ygm = O.expert_down(fmt, mats[4], mats[5],
                                                    midq=gpu["midq"][r, j, :width],
                                                    midqs=gpu["midqs"][r, j, :width // 128],
                                                    nthreads=ref.get("_nthreads", 1))
                else:
                    yref, yabs, ygm = O.expert_down(fmt, mats[4], mats[5],
                                                    mid32=gpu["mid"][r, j, :width],
                                                    nthreads=ref.get("_nthreads", 1))
                dev = np.abs(gpu["y"][r, j].astype(np.float64) - yref)
                lim = ba * ygm + bb * yabs
                assert (dev <= lim).all(), ("down output outside its rounding bound", slot, r, j,
                                            float((dev / np.maximum(lim, 1e-300)).max()))
                y_worst = max(y_worst, float((dev / np.maximum(lim, 1e-300)).max()))
                n_y += dev.size
        rep["y_bound_use_max"] = y_worst
        rep["y_checked"] = n_y
    # T5 -- output
    og = O.dec_bf16_n(np_u16(out_gpu))
    orf = ref["out_f64"]
    err = np.abs(og - orf).max()
    scale = np.abs(orf).max()
    rep["out_err_rel_max"] = float(err / scale) if scale > 0 else float(err)
    nrm = np.linalg.norm(orf)
    rep["out_rel_l2"] = float(np.linalg.norm(og - orf) / nrm) if nrm > 0 else float(err)
    assert err <= OUT_TOL * scale, ("output", rep)
    return rep
