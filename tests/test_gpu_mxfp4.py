"""GPU parity with MXFP4 routed experts (E2M1 pairs, one E8M0 exponent per 32
inputs; the shared expert stays FP8), through the C ABI, against the fp64
oracle: the same per-step checks as the FP8 layer (tests/parity.py), except
that an MXFP4 expert's mid is not re-quantised -- it is checked in fp32
against its rounding bound, and the down GEMV consumes it as is.
"""
import os

import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S
from tests import parity as P

pytestmark = pytest.mark.gpu

NTHREADS = min(16, len(os.sched_getaffinity(0)))


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tiny4():
    return S.make_layer("tiny", routed_fmt=S.FMT_MXFP4, seed=1200, device="cuda")


@pytest.fixture(scope="module")
def glm4():
    _say("generating the GLM-scale MXFP4 layer on the device")
    layer = S.make_layer("glm", routed_fmt=S.FMT_MXFP4, seed=1201, device="cuda")
    torch.cuda.synchronize()
    return layer


def _run(layer, x, flags=0, cache=None):
    rows = x.shape[0]
    runner = B.LayerRunner(layer, rows, flags=flags)
    out = runner.run(x.to("cuda"))
    torch.cuda.synchronize()
    gpu = runner.debug(rows)
    ref_out, ref = P.oracle_for(layer, x, gpu["logits"], nthreads=NTHREADS, host_cache=cache)
    return P.compare(layer, x, gpu, out, ref_out, ref)


@pytest.mark.parametrize("rows", [1, 4, 8])
@pytest.mark.parametrize("mode", ["indep", "corr"])
def test_tiny_mxfp4_parity(tiny4, rows, mode):
    _say(f"tiny mxfp4 rows={rows} mode={mode}")
    x = S.make_x(rows, tiny4.hidden, seed=4000 + 10 * rows + (mode == "corr"), mode=mode)
    _say(_run(tiny4, x))


@pytest.mark.parametrize("inter", [256, 384, 512, 1024])
def test_mxfp4_other_intermediate_sizes(inter):
    """MXFP4 down waves with whole-line items (256 inputs: rings of 1, 2 and 4
    items) and with half-line items (128 inputs, I = 384: a ring of 1), and
    up/gate items per K part of one and two, with a shared expert, at 1, 3
    and 8 rows."""
    shape = dict(hidden=512, inter=inter, n_experts=32, shared_inter=inter, router_std=0.02)
    layer = S.make_layer(shape, routed_fmt=S.FMT_MXFP4, seed=4200 + inter, device="cuda")
    for rows in (1, 3, 8):
        _say(f"mxfp4 inter={inter} rows={rows}")
        x = S.make_x(rows, layer.hidden, seed=4300 + rows, mode="corr")
        _say(_run(layer, x))


@pytest.mark.parametrize("hidden,inter", [(16384, 256), (512, 4096)])
def test_mxfp4_maximum_sizes(hidden, inter):
    """MXFP4 at hidden 16384 and at the largest intermediate size it accepts
    (4096: 131 KB of split mid in LDS per down block at 8 rows)."""
    shape = dict(hidden=hidden, inter=inter, n_experts=32, shared_inter=inter, router_std=0.02)
    layer = S.make_layer(shape, routed_fmt=S.FMT_MXFP4, seed=4400 + hidden, device="cuda")
    for rows in (1, 8):
        _say(f"mxfp4 hidden={hidden} inter={inter} rows={rows}")
        x = S.make_x(rows, layer.hidden, seed=4500 + rows, mode="corr")
        _say(_run(layer, x))


def test_tiny_mxfp4_dedup_off_is_bitwise_equal(tiny4):
    x = S.make_x(8, tiny4.hidden, seed=4100, mode="corr").cuda()
    on = B.LayerRunner(tiny4, 8).run(x)
    off = B.LayerRunner(tiny4, 8, flags=B.F_NO_DEDUP).run(x)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))


@pytest.mark.parametrize("rows,mode", [(1, "indep"), (2, "corr"), (4, "indep"), (6, "corr"),
                                       (8, "indep"), (8, "corr")])
def test_glm_mxfp4_parity(glm4, rows, mode):
    _say(f"glm mxfp4 rows={rows} mode={mode}")
    x = S.make_x(rows, glm4.hidden, seed=4200 + 10 * rows + (mode == "corr"), mode=mode)
    _say(_run(glm4, x, cache=glm4.extra.setdefault("host", {})))


def test_glm_mxfp4_dedup_off_is_bitwise_equal(glm4):
    x = S.make_x(8, glm4.hidden, seed=4300, mode="corr").cuda()
    on = B.LayerRunner(glm4, 8).run(x)
    off = B.LayerRunner(glm4, 8, flags=B.F_NO_DEDUP).run(x)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))
