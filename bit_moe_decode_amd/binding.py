"""ctypes binding of the C ABI in include/moe_decode.h (argument marshalling only).

Every step of the decode path runs in the HIP library; this module only turns
torch tensors into device pointers and structs.  It raises if the built
library is missing: there is no fallback.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbit_moe_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_decode.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
FMT_FP8 = 1
FMT_MXFP4 = 2
FMT_Q1 = 3
FMT_BF16 = 4
ACT_FP8, ACT_BF16 = 0, 1  # moe_afmt
F_NO_DEDUP = 1 << 1
N_KERNELS = 5
K_UPGATE, K_DOWN = 2, 3  # kernels moe_decode_relaunch repeats
KERNEL_NAMES = ("router", "route", "upgate", "down", "combine")  # launch order


class MoeError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("max_rows", ctypes.c_int32),
        ("rms_eps", ctypes.c_float), ("routed_fmt", ctypes.c_int32), ("shared_fmt", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("act_fmt", ctypes.c_int32),
    ]


class Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [
        ("rms_gamma", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
        ("gate", Tensor), ("up", Tensor), ("down", Tensor),
        ("sh_gate", Tensor), ("sh_up", Tensor), ("sh_down", Tensor),
    ]


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "rstd", "ids", "gates", "n_groups", "grp_expert", "grp_owner", "grp_mask",
        "grp_slot", "act_q", "act_s", "mid", "midq", "midqs", "y")] + [
        ("max_groups", ctypes.c_int32), ("mid_stride", ctypes.c_int32)]


class LowbitMatrix(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_LIB = None


def lib():
    """Load the HIP library; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_decode_workspace_size.restype = ctypes.c_size_t
        L.moe_decode_workspace_size.argtypes = [ctypes.POINTER(Config)]
        L.moe_decode_init.restype = ctypes.c_int
        L.moe_decode_init.argtypes = [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        L.moe_decode_step.restype = ctypes.c_int
        L.moe_decode_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.POINTER(Weights), ctypes.c_void_p, ctypes.c_void_p]
        L.moe_decode_step_noalloc.restype = ctypes.c_int
        L.moe_decode_step_noalloc.argtypes = [ctypes.POINTER(Config), ctypes.c_void_p,
                                              ctypes.c_int32, ctypes.POINTER(Weights),
                                              ctypes.c_void_p, ctypes.c_void_p]
        L.moe_decode_debug_view.restype = ctypes.c_int
        L.moe_decode_debug_view.argtypes = [ctypes.c_void_p, ctypes.POINTER(Debug)]
        L.moe_decode_set_timing.restype = ctypes.c_int
        L.moe_decode_set_timing.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.moe_decode_relaunch.restype = ctypes.c_int
        L.moe_decode_relaunch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(Weights),
                                          ctypes.c_int32, ctypes.c_void_p]
        L.moe_decode_set_wait.restype = ctypes.c_int
        L.moe_decode_set_wait.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int32]
        L.moe_decode_wait_timeouts.restype = ctypes.c_int
        L.moe_decode_wait_timeouts.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32),
                                               ctypes.c_void_p]
        L.moe_decode_destroy.restype = None
        L.moe_decode_destroy.argtypes = [ctypes.c_void_p]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.lowbit_gemv.restype = ctypes.c_int
        L.lowbit_gemv.argtypes = [ctypes.POINTER(LowbitMatrix), ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
        _LIB = L
    return _LIB


def declared_functions():
    """Names of the functions include/moe_decode.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def status_string(s):
    return lib().moe_status_string(int(s)).decode()


def workspace_size(cfg: Config) -> int:
    return lib().moe_decode_workspace_size(ctypes.byref(cfg))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Context:
    """A decode context bound to a caller-owned device workspace."""

    def __init__(self, cfg: Config, workspace, stream=None):
        self.cfg = cfg
        self.workspace = workspace  # keep alive
        h = ctypes.c_void_p()
        nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = lib().moe_decode_init(ctypes.byref(cfg), _ptr(workspace), nbytes, _stream(stream),
                                   ctypes.byref(h))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_init")
        self.handle = h

    def step(self, x, rows, weights: Weights, out, stream=None):
        st = lib().moe_decode_step(self.handle, _ptr(x), int(rows), ctypes.byref(weights),
                                   _ptr(out), _stream(stream))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_step")

    def step_status(self, x, rows, weights, out, stream=None):
        """Like step() but returns the status instead of raising."""
        return lib().moe_decode_step(self.handle, _ptr(x), int(rows), ctypes.byref(weights),
                                     _ptr(out), _stream(stream))

    def debug_view(self) -> Debug:
        v = Debug()
        st = lib().moe_decode_debug_view(self.handle, ctypes.byref(v))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_debug_view")
        return v

    def set_timing(self, events):
        """events: list of N_KERNELS + 1 torch.cuda.Event (created with
        enable_timing=True and already recorded once), or None."""
        if events is None:
            st = lib().moe_decode_set_timing(self.handle, None)
        else:
            arr = (ctypes.c_void_p * (N_KERNELS + 1))(*[e.cuda_event for e in events])
            self._events = (events, arr)
            st = lib().moe_decode_set_timing(self.handle, ctypes.cast(arr, ctypes.c_void_p))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_set_timing")

    def relaunch_status(self, kernel, weights: Weights, reps, stream=None):
        return lib().moe_decode_relaunch(self.handle, int(kernel), ctypes.byref(weights), int(reps),
                                         _stream(stream))

    def relaunch(self, kernel, weights: Weights, reps, stream=None):
        """Enqueue `reps` more launches of one kernel of the last step (K_UPGATE
        or K_DOWN) with the weights `weights` (same experts, e.g. another copy)."""
        st = self.relaunch_status(kernel, weights, reps, stream)
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_relaunch")

    def set_wait(self, cap_ticks=0, withhold=0):
        """Cap of the routing launch's waits (100 MHz ticks, 0 = default) and
        the test-only switch that withholds the routing block's records."""
        st = lib().moe_decode_set_wait(self.handle, int(cap_ticks), int(withhold))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_set_wait")

    def wait_timeouts(self, stream=None) -> int:
        """Routed blocks that gave up waiting for their record so far."""
        n = ctypes.c_uint32()
        st = lib().moe_decode_wait_timeouts(self.handle, ctypes.byref(n), _stream(stream))
        if st != MOE_OK:
            raise MoeError(st, "moe_decode_wait_timeouts")
        return int(n.value)

    def close(self):
        if getattr(self, "handle", None):
            lib().moe_decode_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


NOALLOC_MAX_WORKSPACE = 8 << 20  # MOE_DECODE_NOALLOC_MAX_WORKSPACE


def step_noalloc_status(cfg: Config, x, rows, weights: Weights, out, stream=None):
    """moe_decode_step_noalloc: the step with the library's static device
    scratch instead of a context's workspace; returns the status."""
    return lib().moe_decode_step_noalloc(ctypes.byref(cfg), _ptr(x), int(rows),
                                         ctypes.byref(weights), _ptr(out), _stream(stream))


def make_weights(gamma, router_w, routed, shared=None) -> Weights:
    """Weights struct from device tensors: routed/shared are (gate, up, down)
    tuples of (codes, scales) tensors in canonical layout."""
    w = Weights()
    w.rms_gamma = gamma.data_ptr()
    w.router_w = router_w.data_ptr()
    for name, (c, s) in zip(("gate", "up", "down"), routed):
        setattr(w, name, Tensor(c.data_ptr(), None if s is None else s.data_ptr()))
    if shared is not None:
        for name, (c, s) in zip(("sh_gate", "sh_up", "sh_down"), shared):
            setattr(w, name, Tensor(c.data_ptr(), s.data_ptr()))
    return w


def lowbit_gemv(blocks, x, y, n, k, rows=1, stream=None, fmt=FMT_Q1):
    m = LowbitMatrix(fmt, int(n), int(k), blocks.data_ptr() if blocks is not None else None, None)
    st = lib().lowbit_gemv(ctypes.byref(m), _ptr(x), int(rows), _ptr(y), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "lowbit_gemv")


def gemv_fp8(codes, scales, x, y, n, k, rows=1, stream=None):
    """lowbit_gemv with FP8 weights: codes uint8 [n, k], scales float32
    [n/128, k/128], x bf16 [rows, k], y bf16 [rows, n] (device tensors)."""
    st = gemv_fp8_status(codes, scales, x, y, n, k, rows, stream)
    if st != MOE_OK:
        raise MoeError(st, "lowbit_gemv")


def gemv_fp8_status(codes, scales, x, y, n, k, rows=1, stream=None):
    m = LowbitMatrix(FMT_FP8, int(n), int(k), codes.data_ptr() if codes is not None else None,
                     scales.data_ptr() if scales is not None else None)
    return lib().lowbit_gemv(ctypes.byref(m), _ptr(x), int(rows), _ptr(y), _stream(stream))


def gemv_bf16(w, x, y, n, k, rows=1, stream=None):
    """lowbit_gemv with bf16 weights: w bf16 [n, k], x bf16 [rows, k], y bf16
    [rows, n] (device tensors)."""
    st = gemv_bf16_status(w, x, y, n, k, rows, stream)
    if st != MOE_OK:
        raise MoeError(st, "lowbit_gemv")


def gemv_bf16_status(w, x, y, n, k, rows=1, stream=None):
    m = LowbitMatrix(FMT_BF16, int(n), int(k), w.data_ptr() if w is not None else None, None)
    return lib().lowbit_gemv(ctypes.byref(m), _ptr(x), int(rows), _ptr(y), _stream(stream))


def lowbit_gemv_status(blocks, x, y, n, k, rows=1, stream=None, fmt=FMT_Q1):
    m = LowbitMatrix(fmt, int(n), int(k), blocks.data_ptr() if blocks is not None else None, None)
    return lib().lowbit_gemv(ctypes.byref(m), _ptr(x), int(rows), _ptr(y), _stream(stream))


class LayerRunner:
    """Plumbing for tests and the benchmark: a context, its workspace and a
    Weights struct for a synthetic layer already resident on the device.

    layer: bit_moe_decode_amd.synth.Layer whose tensors live on `device`.
    """

    def __init__(self, layer, max_rows, flags=0, device="cuda", stream=None, act_fmt=ACT_FP8):
        import torch
        self.layer = layer
        self.device = device
        self.cfg = Config(layer.hidden, layer.inter, layer.n_experts, 8, layer.shared_inter,
                          max_rows, float(layer.rms_eps), layer.routed_fmt, FMT_FP8, flags,
                          act_fmt)
        n = workspace_size(self.cfg)
        if n == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED, "moe_decode_workspace_size")
        self.ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
        off = (-self.ws.data_ptr()) % 256
        self.ws_view = self.ws[off:off + n]
        self.ctx = Context(self.cfg, self.ws_view, stream)
        self.weights = self.weights_for(layer)

    @staticmethod
    def weights_for(layer) -> Weights:
        r = layer.routed
        sh = None
        if layer.shared is not None:
            s = layer.shared
            sh = ((s.gate[0], s.gate[1]), (s.up[0], s.up[1]), (s.down[0], s.down[1]))
        return make_weights(layer.gamma, layer.router_w,
                            ((r.gate[0], r.gate[1]), (r.up[0], r.up[1]), (r.down[0], r.down[1])),
                            sh)

    def run(self, x, out=None, weights=None, stream=None):
        import torch
        rows = x.shape[0]
        if out is None:
            out = torch.empty(rows, self.layer.hidden, dtype=torch.bfloat16, device=self.device)
        self.ctx.step(x, rows, weights or self.weights, out, stream)
        return out

    def _region(self, ptr, count, dtype):
        import torch
        base = self.ws_view.data_ptr()
        off = ptr - base
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        assert 0 <= off and off + nbytes <= self.ws_view.numel(), "debug pointer outside workspace"
        return self.ws_view[off:off + nbytes].view(dtype)

    def debug(self, rows):
        """Host copies (numpy) of the last step's intermediates."""
        import torch
        v = self.ctx.debug_view()
        L, R, G = self.layer, self.cfg.max_rows, v.max_groups
        E, H, st = L.n_experts, L.hidden, v.mid_stride
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        torch.cuda.synchronize()
        g = lambda p, n, dt: self._region(p, n, dt).cpu().numpy()
        d = dict(
            logits=g(v.logits, R * E, f32).reshape(R, E)[:rows],
            rstd=g(v.rstd, R, f32)[:rows],
            ids=g(v.ids, R * 8, i32).reshape(R, 8)[:rows],
            gates=g(v.gates, R * 8, f32).reshape(R, 8)[:rows],
            n_groups=int(g(v.n_groups, 1, i32)[0]),
            grp_expert=g(v.grp_expert, G, i32),
            grp_owner=g(v.grp_owner, 2 * G, u8).reshape(G, 2),
            grp_mask=g(v.grp_mask, G, u8),
            grp_slot=g(v.grp_slot, 8 * G, u8).reshape(G, 8),
            act_q=g(v.act_q, R * H, u8).reshape(R, H)[:rows],
            act_s=g(v.act_s, R * (H // 128), f32).reshape(R, H // 128)[:rows],
            mid=g(v.mid, R * 9 * st, f32).reshape(R, 9, st)[:rows],
            midq=g(v.midq, R * 9 * st, u8).reshape(R, 9, st)[:rows],
            midqs=g(v.midqs, R * 9 * (st // 128), f32).reshape(R, 9, st // 128)[:rows],
            y=g(v.y, R * 9 * H, f32).reshape(R, 9, H)[:rows],
        )
        n = d["n_groups"]
        for k in ("grp_expert", "grp_owner", "grp_mask", "grp_slot"):
            d[k] = d[k][:n]
        return d
