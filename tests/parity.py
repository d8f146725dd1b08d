"""Comparison of the HIP path's step (outputs and intermediates) with the
oracle, shared by the GPU parity tests, the smoke check and the benchmark's
spot checks.  Test infrastructure: imports the oracle."""
import numpy as np
import torch

from oracle import oracle as O

OUT_TOL = 2e-2          # max|out - ref| <= OUT_TOL * max|ref|
MIDQ_MISMATCH_MAX = 0.01  # fraction of mid codes allowed to sit on the other side of a boundary


def np_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def expert_host(layer, e):
    return tuple(t.cpu().numpy() for t in layer.routed.expert(int(e)))


def shared_host(layer):
    if layer.shared is None:
        return None
    return tuple(t.cpu().numpy() for t in layer.shared.expert(0))


def oracle_for(layer, x, gpu_logits, nthreads=1, host_cache=None):
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
               routed_fmt=layer.routed_fmt)
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
    imax = gpu["mid"].shape[2]
    tot = mism = 0
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
            mg = gpu["mid"][slot, r, :width]
            mr = ref["mid"][r, j, :width]
            scale = max(np.abs(mr).max(), 1e-30)
            assert np.abs(mg - mr).max() <= 2e-3 * scale, ("mid", slot, r, np.abs(mg - mr).max(), scale)
            if not fp8 or not check_mid_codes:
                continue
            # (i) anchored: the oracle's quantiser on the GPU's fp32 mid
            q, s = O.quant_blocks(mg.astype(np.float32))
            assert np.array_equal(gpu["midqs"][slot, r, :width // 128], s), ("midqs", slot, r)
            assert codes_equal(gpu["midq"][slot, r, :width], q).all(), ("midq anchored", slot, r)
            # (ii) end to end: codes may move to a neighbour only
            qe = ref["midq"][r, j, :width]
            bad = ~codes_equal(gpu["midq"][slot, r, :width], qe)
            if bad.any():
                step = np.abs(_e4m3_order(gpu["midq"][slot, r, :width][bad]) - _e4m3_order(qe[bad]))
                assert (step <= 1).all(), ("mid code moved by more than one", slot, r)
            tot += width
            mism += int(bad.sum())
    rep["midq_neighbour_frac"] = mism / max(tot, 1)
    if check_mid_codes:
        assert rep["midq_neighbour_frac"] <= MIDQ_MISMATCH_MAX, rep
    # T5 -- output
    og = O.dec_bf16_n(np_u16(out_gpu))
    orf = ref["out_f64"]
    err = np.abs(og - orf).max()
    scale = np.abs(orf).max()
    rep["out_err_rel_max"] = float(err / scale)
    rep["out_rel_l2"] = float(np.linalg.norm(og - orf) / np.linalg.norm(orf))
    assert err <= OUT_TOL * scale, ("output", rep)
    return rep
