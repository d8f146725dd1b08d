"""ctypes wrapper around the fp64 CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the library.  It imports
nothing from the HIP library's package.

All arrays are numpy; codes are uint8 / uint16 bit patterns, never decoded by
numpy here (the C side decodes them bit by bit).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

FMT_FP8 = 1
FMT_MXFP4 = 2
FMT_Q1 = 3  # 1-bit group-128 routed experts: [N, K/128, 18] blocks, no separate scales
ACT_FP8, ACT_BF16 = 0, 1  # the experts' input: FP8 blocks of u (default) or u itself


class OrcMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class OrcCfg(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("rows", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("routed_fmt", ctypes.c_int32), ("nthreads", ctypes.c_int32),
        ("act_fmt", ctypes.c_int32),
    ]


class OrcDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "z", "rstd", "u", "ids", "gates", "act_q", "act_s", "mid", "midq", "midqs",
        "y", "out_f64", "gate", "up", "gate_abs", "up_abs", "gate_gmax", "up_gmax")]


def lib():
    """Load the oracle library, building it with gcc if it is not there."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = ctypes.CDLL(_build.LIB)
        _LIB.orc_dec_bf16.restype = ctypes.c_double
        _LIB.orc_dec_bf16.argtypes = [ctypes.c_uint16]
        _LIB.orc_dec_fp16.restype = ctypes.c_double
        _LIB.orc_dec_fp16.argtypes = [ctypes.c_uint16]
        _LIB.orc_dec_e4m3.restype = ctypes.c_double
        _LIB.orc_dec_e4m3.argtypes = [ctypes.c_uint8]
        _LIB.orc_dec_e2m1.restype = ctypes.c_double
        _LIB.orc_dec_e2m1.argtypes = [ctypes.c_uint8]
        _LIB.orc_dec_e8m0.restype = ctypes.c_double
        _LIB.orc_dec_e8m0.argtypes = [ctypes.c_uint8]
        _LIB.orc_enc_e4m3.restype = ctypes.c_uint8
        _LIB.orc_enc_e4m3.argtypes = [ctypes.c_float]
        _LIB.orc_round_bf16.restype = ctypes.c_uint16
        _LIB.orc_round_bf16.argtypes = [ctypes.c_double]
        _LIB.orc_moe_step.restype = ctypes.c_int
        _LIB.orc_lowbit_gemv_q1.restype = ctypes.c_int
        _LIB.orc_dedup.restype = ctypes.c_int
    return _LIB


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


# ------------------------------------------------------------------ codecs
def dec_bf16(h):
    return lib().orc_dec_bf16(int(h))


def dec_fp16(h):
    return lib().orc_dec_fp16(int(h))


def dec_e4m3(c):
    return lib().orc_dec_e4m3(int(c))


def dec_e2m1(c):
    return lib().orc_dec_e2m1(int(c))


def dec_e8m0(c):
    return lib().orc_dec_e8m0(int(c))


def enc_e4m3(v):
    return lib().orc_enc_e4m3(float(v))


def round_bf16(v):
    return lib().orc_round_bf16(float(v))


def dec_e4m3_n(codes):
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.empty(c.size, np.float64)
    lib().orc_dec_e4m3_n(_p(c), ctypes.c_int(c.size), _p(out))
    return out.reshape(np.shape(codes))


def dec_bf16_n(codes):
    c = np.ascontiguousarray(codes, dtype=np.uint16).ravel()
    out = np.empty(c.size, np.float64)
    lib().orc_dec_bf16_n(_p(c), ctypes.c_int(c.size), _p(out))
    return out.reshape(np.shape(codes))


def dec_fp16_n(codes):
    c = np.ascontiguousarray(codes, dtype=np.uint16).ravel()
    out = np.empty(c.size, np.float64)
    lib().orc_dec_fp16_n(_p(c), ctypes.c_int(c.size), _p(out))
    return out.reshape(np.shape(codes))


def enc_e4m3_n(v):
    a = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(a.size, np.uint8)
    lib().orc_enc_e4m3_n(_p(a), ctypes.c_int(a.size), _p(out))
    return out.reshape(np.shape(v))


def round_bf16_n(v):
    a = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(a.size, np.uint16)
    lib().orc_round_bf16_n(_p(a), ctypes.c_int(a.size), _p(out))
    return out.reshape(np.shape(v))


# ------------------------------------------------------------ step pieces
def top8(z):
    z = np.ascontiguousarray(z, dtype=np.float64)
    ids = np.empty(8, np.int32)
    lib().orc_top8(_p(z), ctypes.c_int(z.size), _p(ids))
    return ids


def softmax8(zsel):
    z = np.ascontiguousarray(zsel, dtype=np.float64)
    g = np.empty(8, np.float64)
    lib().orc_softmax8(_p(z), _p(g))
    return g


def dedup(ids):
    """ids int32 [R, 8] -> dict(n, expert[n], owner_slot[n], owner_row[n], mask[n], slot[n, 8])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rows = ids.shape[0]
    gmax = 8 * rows
    n = ctypes.c_int32(0)
    expert = np.zeros(gmax, np.int32)
    oslot = np.zeros(gmax, np.uint8)
    orow = np.zeros(gmax, np.uint8)
    mask = np.zeros(gmax, np.uint8)
    slot = np.zeros((gmax, 8), np.uint8)
    rc = lib().orc_dedup(_p(ids), ctypes.c_int(rows), ctypes.byref(n), _p(expert), _p(oslot),
                         _p(orow), _p(mask), _p(slot))
    if rc != 0:
        raise ValueError("orc_dedup failed")
    d = n.value
    return dict(n=d, expert=expert[:d], owner_slot=oslot[:d], owner_row=orow[:d],
                mask=mask[:d], slot=slot[:d])


def quant_blocks(v):
    """FP8 block quantiser (per 128): float32 [n] -> (codes uint8 [n], scales float32 [n/128])."""
    a = np.ascontiguousarray(v, dtype=np.float32).ravel()
    q = np.empty(a.size, np.uint8)
    s = np.empty(a.size // 128, np.float32)
    lib().orc_quant_blocks(_p(a), ctypes.c_int(a.size), _p(q), _p(s))
    return q.reshape(np.shape(v)), s


def moe_step(cfg, x, gamma, router_w, experts, shared=None, anchor_z=None, nthreads=1):
    """Run the oracle's decode step.

    cfg: dict(hidden, inter, n_experts, shared_inter, rows, rms_eps, routed_fmt, act_fmt)
         (act_fmt ACT_FP8, the default, or ACT_BF16: u itself as the experts' input)
    x: uint16 [R, H] bf16 codes; gamma: uint16 [H]; router_w: uint16 [E, H]
    experts: dict expert_id -> (gate_codes, gate_scales, up_codes, up_scales,
             down_codes, down_scales); only experts that are picked are needed
             (1-bit experts: the blocks as codes, scales None).
    shared: the same 6-tuple for the shared expert (FP8) or None.
    anchor_z: float32 [R, E] logits that decide the selection, or None.
    Returns (out uint16 [R, H], debug dict of numpy arrays).
    """
    H, I, E = cfg["hidden"], cfg["inter"], cfg["n_experts"]
    Is, R = cfg.get("shared_inter", 0), cfg["rows"]
    Imax = max(I, Is)
    c = OrcCfg(H, I, E, Is, R, float(cfg.get("rms_eps", 1e-6)),
               int(cfg.get("routed_fmt", FMT_FP8)), int(nthreads), int(cfg.get("act_fmt", ACT_FP8)))
    keep = []

    def mat(codes, scales):
        codes = np.ascontiguousarray(codes)
        keep.append(codes)
        if scales is None:
            return OrcMat(codes.ctypes.data, None)
        scales = np.ascontiguousarray(scales)
        keep.append(scales)
        return OrcMat(codes.ctypes.data, scales.ctypes.data)

    G = (OrcMat * E)()
    U = (OrcMat * E)()
    D = (OrcMat * E)()
    for e, w in experts.items():
        G[e] = mat(w[0], w[1])
        U[e] = mat(w[2], w[3])
        D[e] = mat(w[4], w[5])
    if shared is not None:
        sg, su, sd = mat(shared[0], shared[1]), mat(shared[2], shared[3]), mat(shared[4], shared[5])
        psg, psu, psd = ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd)
    else:
        psg = psu = psd = None
    x = np.ascontiguousarray(x, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    router_w = np.ascontiguousarray(router_w, dtype=np.uint16)
    az = None if anchor_z is None else np.ascontiguousarray(anchor_z, dtype=np.float32)
    out = np.zeros((R, H), np.uint16)
    dbg = dict(
        z=np.zeros((R, E)), rstd=np.zeros(R), u=np.zeros((R, H), np.uint16),
        ids=np.zeros((R, 8), np.int32), gates=np.zeros((R, 8)),
        act_q=np.zeros((R, H), np.uint8), act_s=np.zeros((R, H // 128), np.float32),
        mid=np.zeros((R, 9, Imax)), midq=np.zeros((R, 9, Imax), np.uint8),
        midqs=np.zeros((R, 9, Imax // 128), np.float32), y=np.zeros((R, 9, H)),
        out_f64=np.zeros((R, H)), gate=np.zeros((R, 9, Imax)), up=np.zeros((R, 9, Imax)),
        gate_abs=np.zeros((R, 9, Imax)), up_abs=np.zeros((R, 9, Imax)),
        gate_gmax=np.zeros((R, 9, Imax)), up_gmax=np.zeros((R, 9, Imax)))
    d = OrcDebug(**{k: v.ctypes.data for k, v in dbg.items()})
    rc = lib().orc_moe_step(ctypes.byref(c), _p(x), _p(gamma), _p(router_w), G, U, D,
                            psg, psu, psd, _p(az), _p(out), ctypes.byref(d))
    if rc != 0:
        raise ValueError("orc_moe_step failed (bad config or a picked expert is missing)")
    return out, dbg


def router(cfg, x, gamma, router_w):
    """Router stage alone: (z float64 [R, E], rstd [R], u uint16 [R, H])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, H = x.shape
    E = cfg["n_experts"]
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    router_w = np.ascontiguousarray(router_w, dtype=np.uint16)
    z = np.zeros((R, E))
    rstd = np.zeros(R)
    u = np.zeros((R, H), np.uint16)
    rc = lib().orc_router(ctypes.c_int(R), ctypes.c_int(H), ctypes.c_int(E),
                          ctypes.c_float(cfg.get("rms_eps", 1e-6)), _p(x), _p(gamma),
                          _p(router_w), _p(z), _p(rstd), _p(u))
    if rc != 0:
        raise ValueError("orc_router failed")
    return z, rstd, u


def lowbit_gemv_q1(blocks, x, n, k, nthreads=1):
    """blocks uint8 [n, k/128, 18]; x uint16 [k] bf16 -> (y uint16 [n], y_f64 [n])."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    xx = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.zeros(n, np.uint16)
    yf = np.zeros(n, np.float64)
    rc = lib().orc_lowbit_gemv_q1(_p(b), _p(xx), ctypes.c_int(n), ctypes.c_int(k),
                                  ctypes.c_int(nthreads), _p(y), _p(yf))
    if rc != 0:
        raise ValueError("orc_lowbit_gemv_q1 failed")
    return y, yf


def gemv_fp8(codes, scales, x, nthreads=1):
    """codes uint8 [n, k] (E4M3), scales float32 [n/128, k/128], x uint16 [rows, k]
    (bf16) -> (y uint16 [rows, n] bf16, y_f64 [rows, n])."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    xx = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    rows, k = xx.shape
    n = c.shape[0]
    assert c.shape == (n, k) and sc.shape == (n // 128, k // 128)
    y = np.zeros((rows, n), np.uint16)
    yf = np.zeros((rows, n), np.float64)
    rc = lib().orc_gemv_fp8(_p(c), _p(sc), _p(xx), ctypes.c_int(rows), ctypes.c_int(n),
                            ctypes.c_int(k), ctypes.c_int(nthreads), _p(y), _p(yf))
    if rc != 0:
        raise ValueError("orc_gemv_fp8 failed")
    return y, yf


def gemv_bf16(w, x, nthreads=1):
    """w uint16 [n, k] (bf16 bits), x uint16 [rows, k] (bf16 bits) ->
    (y uint16 [rows, n] bf16, y_f64 [rows, n])."""
    ww = np.ascontiguousarray(w, dtype=np.uint16)
    xx = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    rows, k = xx.shape
    n = ww.shape[0]
    assert ww.shape == (n, k)
    y = np.zeros((rows, n), np.uint16)
    yf = np.zeros((rows, n), np.float64)
    rc = lib().orc_gemv_bf16(_p(ww), _p(xx), ctypes.c_int(rows), ctypes.c_int(n),
                             ctypes.c_int(k), ctypes.c_int(nthreads), _p(y), _p(yf))
    if rc != 0:
        raise ValueError("orc_gemv_bf16 failed")
    return y, yf


def expert_down(fmt, codes, scales, midq=None, midqs=None, mid32=None, nthreads=1):
    """The down GEMV of one expert on a given mid (orc_expert_down).

    fmt FMT_FP8: codes uint8 [h, i], scales float32 [h/128, i/128], midq uint8
    [i] and midqs float32 [i/128] (the mid's FP8 codes and block scales).
    fmt FMT_MXFP4: codes uint8 [h, i/2], scales uint8 E8M0 [h, i/32], mid32
    float32 [i] (mid itself, not re-quantised).
    fmt FMT_Q1: codes uint8 [h, i/128, 18] blocks, scales None, midq/midqs as
    for FP8.
    Returns (y float64 [h], y_abs float64 [h], y_gmax float64 [h]) with y_abs =
    sum_k |W[n,k] mhat_k| and y_gmax = the sum over groups of 8 consecutive k of
    the largest |W[n,k] mhat_k| of the group."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    h = c.shape[0]
    i = {FMT_FP8: lambda: c.shape[1], FMT_MXFP4: lambda: 2 * c.shape[1],
         FMT_Q1: lambda: 128 * c.shape[1]}[fmt]()
    sc = None if fmt == FMT_Q1 else np.ascontiguousarray(
        scales, dtype=np.float32 if fmt == FMT_FP8 else np.uint8)
    q = None if midq is None else np.ascontiguousarray(midq, dtype=np.uint8).ravel()
    qs = None if midqs is None else np.ascontiguousarray(midqs, dtype=np.float32).ravel()
    m32 = None if mid32 is None else np.ascontiguousarray(mid32, dtype=np.float32).ravel()
    for a, n in ((q, i), (qs, i // 128), (m32, i)):
        assert a is None or a.size == n
    m = OrcMat(c.ctypes.data, None if sc is None else sc.ctypes.data)
    y = np.zeros(h, np.float64)
    ya = np.zeros(h, np.float64)
    yg = np.zeros(h, np.float64)
    rc = lib().orc_expert_down(ctypes.c_int(fmt), ctypes.byref(m), ctypes.c_int(h), ctypes.c_int(i),
                               _p(q), _p(qs), _p(m32), ctypes.c_int(nthreads), _p(y), _p(ya),
                               _p(yg))
    if rc != 0:
        raise ValueError("orc_expert_down failed")
    return y, ya, yg
