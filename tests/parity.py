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
    return tuple(t.cpu().numpy() for t in layer.routed.expert(int(e)))


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


def mid_tau(gate, up, gate_abs, up_abs, nkb):
    """Bound on |mid_gpu - mid_exact| from the kernel's arithmetic: each gate /
    up output is one 128-term FP8 MFMA per K block (products exact, sum
    bounded as fp32 with truncation, 128 * 2^-23 * sum|terms|), nkb block
    partials scaled and summed in fp32 (within K parts, then the parts in
    order: nkb - 1 additions in all) and two scale products and the rstd
    product rounded: (nkb + 6) * 2^-24 * sum|terms|.
    mid = g sigma(g) u then carries |d mid/dg| dg + |d mid/du| du plus eight
    fp32 roundings of the SiLU evaluation."""
    eps = 128 * 2.0 ** -23 + (nkb + 6) * U32
    dg = eps * gate_abs
    du = eps * up_abs
    sig = 1.0 / (1.0 + np.exp(-np.clip(gate, -700, 700)))
    dmid_dg = np.abs(sig * (1.0 + gate * (1.0 - sig)) * up)
    dmid_du = np.abs(gate * sig)
    mid = gate * sig * up
    return dmid_dg * dg + dmid_du * du + 8 * U32 * np.abs(mid) + dg * du


def _code_in_window(codes, centre, half_width, scale):
    """True where `codes` is the E4M3 rounding of some value of the interval
    [centre - half_width, centre + half_width] divided by `scale` (rounding is
    monotone, so the two ends bracket every admissible code)."""
    lo = O.enc_e4m3_n(((centre - half_width) / scale).astype(np.float32))
    hi = O.enc_e4m3_n(((centre + half_width) / scale).astype(np.float32))
    c = _e4m3_order(codes)
    ok = (_e4m3_order(lo) <= c) & (c <= _e4m3_order(hi))
    zero = (np.asarray(codes) & 0x7F) == 0
    zlo = _e4m3_order(lo) <= 0
    zhi = _e4m3_order(hi) >= 0
    return ok | (zero & zlo & zhi)


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
    tot = ndiff = n_ulp = n_tau = 0
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
            width, fp8 = layer.inter, layer.routed_fmt == O.FMT_FP8
        for r, j in users:
            mg = gpu["mid"][r, j, :width].astype(np.float64)
            mo = ref["mid"][r, j, :width]
            tau = mid_tau(ref["gate"][r, j, :width], ref["up"][r, j, :width],
                          ref["gate_abs"][r, j, :width], ref["up_abs"][r, j, :width], nkb)
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
            in_ulp = _code_in_window(qg, mo, np.abs(mo / sgx) * 2.0 ** -23 * sgx, sgx)
            in_tau = _code_in_window(qg, mo, tau + np.abs(mo) * 2.0 ** -23, sgx)
            assert in_tau[diff].all(), ("mid code not a rounding of any value within tau",
                                        slot, r, int((diff & ~in_tau).sum()))
            tot += width
            ndiff += int(diff.sum())
            n_ulp += int((diff & in_ulp).sum())
            n_tau += int((diff & in_tau).sum())
    rep["mid_tau_use_max"] = worst
    rep["midq_codes"] = tot
    rep["midq_diff"] = ndiff
    rep["midq_diff_in_1ulp"] = n_ulp
    rep["midq_diff_in_tau"] = n_tau
    # T5 -- output
    og = O.dec_bf16_n(np_u16(out_gpu))
    orf = ref["out_f64"]
    err = np.abs(og - orf).max()
    scale = np.abs(orf).max()
    rep["out_err_rel_max"] = float(err / scale)
    rep["out_rel_l2"] = float(np.linalg.norm(og - orf) / np.linalg.norm(orf))
    assert err <= OUT_TOL * scale, ("output", rep)
    return rep
