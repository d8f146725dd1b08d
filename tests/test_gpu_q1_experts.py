"""GPU parity of the decode step with 1-bit (Q1_0_G128) routed experts,
through the C ABI, against the fp64 oracle: bit-exact top-8 and dedup table,
bit-exact activation blocks, mid within its rounding bound with its FP8 codes
reproduced by the oracle's quantiser and adjacent end to end, each (row, pick)
down output against the oracle's down GEMV of the device's own mid codes, the
bf16 output; dedup on and off bitwise equal.  The shared expert stays FP8."""
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


def _run(layer, x, cache=None, flags=0):
    rows = x.shape[0]
    runner = B.LayerRunner(layer, rows, flags=flags)
    out = runner.run(x.to("cuda"))
    torch.cuda.synchronize()
    gpu = runner.debug(rows)
    ref_out, ref = P.oracle_for(layer, x, gpu["logits"], nthreads=NTHREADS, host_cache=cache)
    return out, gpu, P.compare(layer, x, gpu, out, ref_out, ref)


@pytest.mark.parametrize("shape", [
    dict(hidden=512, inter=256, n_experts=32, shared_inter=256, router_std=0.02),
    dict(hidden=1024, inter=768, n_experts=64, shared_inter=0, router_std=0.02),
    dict(hidden=2048, inter=4096, n_experts=32, shared_inter=4096, router_std=0.02),
    # two rounds of the up/gate's block loads (hidden / 2048), one octet of the
    # down's (inter / 1024): the second octet in flight is a clamped reload
    dict(hidden=4096, inter=1024, n_experts=32, shared_inter=1024, router_std=0.02),
], ids=["h512-i256", "h1024-i768-noshared", "h2048-i4096", "h4096-i1024"])
def test_q1_experts_small(shape):
    layer = S.make_layer(shape, routed_fmt=S.FMT_Q1, seed=5300 + shape["inter"], device="cuda")
    cache = {}
    for rows, mode in ((1, "indep"), (2, "corr"), (4, "indep"), (8, "corr"), (8, "indep")):
        _say(f"q1 experts hidden={shape['hidden']} inter={shape['inter']} rows={rows} {mode}")
        x = S.make_x(rows, shape["hidden"], seed=5400 + rows + (mode == "corr"), mode=mode)
        _, _, rep = _run(layer, x, cache)
        _say(rep)


@pytest.fixture(scope="module")
def glm_q1():
    _say("generating the GLM-scale layer with 1-bit routed experts")
    return S.make_layer("glm", routed_fmt=S.FMT_Q1, seed=1004, device="cuda")


@pytest.mark.parametrize("rows,mode", [(1, "indep"), (4, "indep"), (8, "indep"), (8, "corr")])
def test_q1_experts_glm(glm_q1, rows, mode):
    _say(f"q1 experts glm rows={rows} {mode}")
    x = S.make_x(rows, glm_q1.hidden, seed=5500 + rows + (mode == "corr"), mode=mode)
    _, _, rep = _run(glm_q1, x, glm_q1.extra.setdefault("host", {}))
    _say(rep)


def test_q1_experts_dedup_off_is_bitwise_equal(glm_q1):
    x = S.make_x(8, glm_q1.hidden, seed=5600, mode="corr").cuda()
    on = B.LayerRunner(glm_q1, 8).run(x)
    off = B.LayerRunner(glm_q1, 8, flags=B.F_NO_DEDUP).run(x)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))


def test_q1_experts_unsupported_shapes():
    for kw in (dict(hidden=256, inter=256), dict(hidden=512, inter=128),
               dict(hidden=512, inter=4352)):
        c = B.Config(kw["hidden"], kw["inter"], 32, 8, 0, 4, 1e-6, B.FMT_Q1, B.FMT_FP8, 0, 0)
        assert B.workspace_size(c) == 0, kw
