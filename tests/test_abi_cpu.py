"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and its host-side validation answers as documented (no
kernel is launched by any call here)."""
import ctypes

import pytest

from bit_moe_decode_amd import binding as B


def test_library_exports_every_declared_function():
    L = B.lib()
    names = B.declared_functions()
    assert set(names) >= {"moe_decode_init", "moe_decode_step", "lowbit_gemv",
                          "moe_decode_workspace_size", "moe_decode_debug_view",
                          "moe_decode_destroy", "moe_status_string", "moe_decode_set_timing",
                          "moe_decode_relaunch", "moe_decode_set_wait",
                          "moe_decode_wait_timeouts"}
    for n in names:
        assert hasattr(L, n), n


def cfg(**kw):
    base = dict(hidden=6144, inter=2048, n_experts=256, top_k=8, shared_inter=2048, max_rows=8,
                rms_eps=1e-6, routed_fmt=B.FMT_FP8, shared_fmt=B.FMT_FP8, flags=0,
                act_fmt=B.ACT_FP8)
    base.update(kw)
    return B.Config(*base.values())


def test_one_bit_routed_experts_are_supported():
    # 1-bit steps also keep the activation codes in the 1-bit operand order
    # (max_rows x hidden bytes, a multiple of 256 here)
    assert B.workspace_size(cfg(routed_fmt=B.FMT_Q1)) == B.workspace_size(cfg()) + 8 * 6144
    assert B.workspace_size(cfg(routed_fmt=B.FMT_Q1, hidden=512, inter=256, shared_inter=0)) > 0


def test_workspace_size_supported_shapes():
    n8 = B.workspace_size(cfg())
    n1 = B.workspace_size(cfg(max_rows=1))
    assert 0 < n1 < n8 < 64 << 20
    assert B.workspace_size(cfg(hidden=256, inter=128, n_experts=32, shared_inter=0)) > 0
    # without dedup every pick is its own group: more mid slots
    assert B.workspace_size(cfg(flags=B.F_NO_DEDUP, n_experts=32)) > B.workspace_size(cfg(n_experts=32))
    # bf16 activations with FP8 experts
    assert B.workspace_size(cfg(act_fmt=B.ACT_BF16)) == n8


@pytest.mark.parametrize("kw", [dict(top_k=4), dict(hidden=6100), dict(inter=100),
                                dict(n_experts=24), dict(n_experts=2048), dict(shared_inter=64),
                                dict(routed_fmt=B.FMT_BF16), dict(shared_fmt=B.FMT_MXFP4),
                                dict(routed_fmt=B.FMT_Q1, act_fmt=B.ACT_BF16),
                                dict(routed_fmt=B.FMT_Q1, hidden=6400),
                                dict(routed_fmt=B.FMT_Q1, inter=4352, shared_inter=4352),
                                dict(routed_fmt=B.FMT_Q1, inter=384, shared_inter=384),
                                dict(shared_fmt=B.FMT_Q1),
                                dict(routed_fmt=B.FMT_MXFP4, inter=4224, shared_inter=4224),
                                dict(flags=1 << 7), dict(hidden=32768), dict(max_rows=9),
                                dict(max_rows=0), dict(act_fmt=2), dict(act_fmt=-1),
                                dict(act_fmt=B.ACT_BF16, routed_fmt=B.FMT_MXFP4)])
def test_unsupported_configs(kw):
    assert B.workspace_size(cfg(**kw)) == 0
    h = ctypes.c_void_p()
    st = B.lib().moe_decode_init(ctypes.byref(cfg(**kw)), ctypes.c_void_p(1 << 20), 1 << 30, None,
                                 ctypes.byref(h))
    assert st in (B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_INVALID_ARG)
    assert not h.value


def test_init_workspace_errors():
    L = B.lib()
    c = cfg()
    h = ctypes.c_void_p()
    assert L.moe_decode_init(ctypes.byref(c), None, 1 << 30, None, ctypes.byref(h)) == B.MOE_ERR_WORKSPACE
    # misaligned
    assert L.moe_decode_init(ctypes.byref(c), ctypes.c_void_p(4096 + 16), 1 << 30, None,
                             ctypes.byref(h)) == B.MOE_ERR_WORKSPACE
    # too small
    need = B.workspace_size(c)
    assert L.moe_decode_init(ctypes.byref(c), ctypes.c_void_p(4096), need - 1, None,
                             ctypes.byref(h)) == B.MOE_ERR_WORKSPACE
    assert L.moe_decode_init(None, ctypes.c_void_p(4096), need, None, ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_decode_init(ctypes.byref(c), ctypes.c_void_p(4096), need, None, None) == B.MOE_ERR_INVALID_ARG


def test_step_without_context():
    w = B.Weights()
    assert B.lib().moe_decode_step(None, None, 1, ctypes.byref(w), None, None) == B.MOE_ERR_INVALID_ARG
    assert B.lib().moe_decode_debug_view(None, None) == B.MOE_ERR_INVALID_ARG
    assert B.lib().moe_decode_set_wait(None, 0, 0) == B.MOE_ERR_INVALID_ARG
    n = ctypes.c_uint32()
    assert B.lib().moe_decode_wait_timeouts(None, ctypes.byref(n), None) == B.MOE_ERR_INVALID_ARG
    B.lib().moe_decode_destroy(None)


def test_lowbit_gemv_validation():
    L = B.lib()

    def call(fmt=B.FMT_Q1, n=16, k=256, rows=1, codes=4096, x=8192, y=16384, scales=None):
        m = B.LowbitMatrix(fmt, n, k, codes, scales)
        return L.lowbit_gemv(ctypes.byref(m), ctypes.c_void_p(x) if x else None, rows,
                             ctypes.c_void_p(y) if y else None, None)

    assert call(fmt=B.FMT_MXFP4) == B.MOE_ERR_UNSUPPORTED
    assert call(k=200) == B.MOE_ERR_UNSUPPORTED
    assert call(k=32768) == B.MOE_ERR_UNSUPPORTED
    assert call(rows=9) == B.MOE_ERR_UNSUPPORTED      # up to 8 rows
    assert call(rows=2, k=384) == B.MOE_ERR_UNSUPPORTED  # several rows: K in chunks of 256
    assert call(rows=-1) == B.MOE_ERR_INVALID_ARG
    # the FP8 form: N and K on the 128 grid, 1..8 rows, a scale pointer
    fp8 = dict(fmt=B.FMT_FP8, n=128, k=128, x=1 << 20, y=1 << 21, scales=1 << 22)
    assert call(**dict(fp8, n=100)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(fp8, k=200)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(fp8, rows=9)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(fp8, rows=0)) == B.MOE_OK
    assert call(**dict(fp8, scales=None)) == B.MOE_ERR_INVALID_ARG
    assert call(**dict(fp8, x=(1 << 20) + 8)) == B.MOE_ERR_INVALID_ARG  # misaligned
    assert call(**dict(fp8, y=(1 << 20) + 64)) == B.MOE_ERR_INVALID_ARG  # overlaps x
    # the bf16 form: N on the 128 grid, K on the 64 grid, 1..8 rows, no scales
    bf = dict(fmt=B.FMT_BF16, n=128, k=64, x=1 << 20, y=1 << 21)
    assert call(**dict(bf, n=100)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(bf, k=96)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(bf, rows=9)) == B.MOE_ERR_UNSUPPORTED
    assert call(**dict(bf, rows=0)) == B.MOE_OK
    assert call(**dict(bf, codes=None)) == B.MOE_ERR_INVALID_ARG
    assert call(**dict(bf, codes=4096 + 8)) == B.MOE_ERR_INVALID_ARG  # misaligned weights
    assert call(**dict(bf, x=(1 << 20) + 8)) == B.MOE_ERR_INVALID_ARG  # misaligned x
    assert call(**dict(bf, y=(1 << 21) + 1)) == B.MOE_ERR_INVALID_ARG  # odd y
    assert call(**dict(bf, y=(1 << 20) + 64)) == B.MOE_ERR_INVALID_ARG  # overlaps x
    assert call(fmt=5) == B.MOE_ERR_UNSUPPORTED
    assert call(rows=0) == B.MOE_OK                    # no-op, nothing launched
    assert call(n=0) == B.MOE_OK
    assert call(codes=None) == B.MOE_ERR_INVALID_ARG
    assert call(x=8200) == B.MOE_ERR_INVALID_ARG       # misaligned
    assert call(x=8192, y=8192) == B.MOE_ERR_INVALID_ARG  # overlap
    assert L.lowbit_gemv(None, None, 1, None, None) == B.MOE_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert B.status_string(s)
    assert "unknown" in B.status_string(99)
