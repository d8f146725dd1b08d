"""GPU parity: the HIP library's decode step, called through the C ABI,
against the fp64 oracle on the same seeded inputs.

Checks per step (see tests/parity.py): bit-exact top-8 judged on the GPU's own
fp32 logits, bit-exact dedup table, bit-exact activation scales and codes,
mid codes bit-exact when the oracle's quantiser is applied to the GPU's fp32
mid and at most one code apart end to end, and the bf16 output within
2e-2 * max|ref|.  Invariants: dedup on/off and run-to-run bitwise equality,
row permutation.
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


@pytest.fixture(scope="module")
def tiny():
    return S.make_layer("tiny", seed=1000, device="cuda")


@pytest.fixture(scope="module")
def glm():
    _say("generating the GLM-scale layer on the device")
    layer = S.make_layer("glm", seed=1001, device="cuda")
    torch.cuda.synchronize()
    return layer


def _run(layer, x, max_rows=None, flags=0, cache=None, check_mid_codes=True, act_fmt=B.ACT_FP8):
    rows = x.shape[0]
    runner = B.LayerRunner(layer, max_rows or rows, flags=flags, act_fmt=act_fmt)
    xd = x.to("cuda")
    out = runner.run(xd)
    torch.cuda.synchronize()
    gpu = runner.debug(rows)
    ref_out, ref = P.oracle_for(layer, x, gpu["logits"], nthreads=NTHREADS, host_cache=cache,
                                act_fmt=act_fmt)
    rep = P.compare(layer, x, gpu, out, ref_out, ref, check_mid_codes=check_mid_codes)
    assert runner.ctx.wait_timeouts() == 0  # every routed block got its record
    return runner, out, gpu, rep


@pytest.mark.parametrize("rows", [1, 2, 4, 8])
@pytest.mark.parametrize("mode", ["indep", "corr"])
def test_tiny_parity(tiny, rows, mode):
    _say(f"tiny rows={rows} mode={mode}")
    x = S.make_x(rows, tiny.hidden, seed=2000 + rows, mode=mode)
    _, _, _, rep = _run(tiny, x)
    _say(rep)


def test_tiny_rows_below_max_rows(tiny):
    """A context sized for 8 rows running 3-row and 1-row steps."""
    runner = B.LayerRunner(tiny, 8)
    for rows in (3, 1, 8):
        x = S.make_x(rows, tiny.hidden, seed=2100 + rows)
        out = runner.run(x.cuda())
        gpu = runner.debug(rows)
        ref_out, ref = P.oracle_for(tiny, x, gpu["logits"])
        P.compare(tiny, x, gpu, out, ref_out, ref)


def test_tiny_dedup_off_is_bitwise_equal(tiny):
    for mode in ("indep", "corr"):
        x = S.make_x(8, tiny.hidden, seed=2200, mode=mode).cuda()
        on = B.LayerRunner(tiny, 8).run(x)
        r_off = B.LayerRunner(tiny, 8, flags=B.F_NO_DEDUP)
        off = r_off.run(x)
        torch.cuda.synchronize()
        assert torch.equal(on.view(torch.int16), off.view(torch.int16))
        d = r_off.debug(8)
        assert d["n_groups"] == 64 and (d["grp_mask"] != 0).all()


def test_tiny_deterministic_and_permutation(tiny):
    x = S.make_x(8, tiny.hidden, seed=2300, mode="corr").cuda()
    r = B.LayerRunner(tiny, 8)
    a = r.run(x).clone()
    b = r.run(x).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    perm = torch.tensor([5, 2, 7, 0, 1, 6, 3, 4], device="cuda")
    c = r.run(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), a[perm].view(torch.int16))


def test_tiny_max_experts():
    """E = 1024 (the largest the router handles), 8 rows."""
    shape = dict(hidden=256, inter=128, n_experts=1024, shared_inter=128, router_std=0.02)
    layer = S.make_layer(shape, seed=1003, device="cuda")
    x = S.make_x(8, 256, seed=2400)
    _run(layer, x)


def test_tiny_tied_logits_go_to_lower_id():
    """Duplicate router rows give exactly equal logits: the lower ID must win."""
    layer = S.make_layer("tiny", seed=1004, device="cuda")
    w = layer.router_w
    for a, b in ((3, 17), (5, 6), (20, 31), (0, 9)):
        w[b] = w[a]
    x = S.make_x(4, 256, seed=2500)
    _, _, gpu, _ = _run(layer, x)
    both = 0
    for r in range(4):
        ids = list(gpu["ids"][r])
        for a, b in ((3, 17), (5, 6), (20, 31), (0, 9)):
            assert gpu["logits"][r][a] == gpu["logits"][r][b]
            assert not (b in ids and a not in ids), (r, a, b, ids)  # the higher ID never alone
            if a in ids and b in ids:
                assert ids.index(a) + 1 == ids.index(b)
                both += 1
    assert both > 0, "no duplicated pair was picked together: the order was never compared"


def test_zero_rows_is_a_noop(tiny):
    r = B.LayerRunner(tiny, 4)
    x = S.make_x(1, 256, seed=1).cuda()
    out = torch.full((1, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    assert r.ctx.step_status(x, 0, r.weights, out) == B.MOE_OK
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()


def test_step_argument_errors(tiny):
    r = B.LayerRunner(tiny, 4)
    x = S.make_x(4, 256, seed=1).cuda()
    out = torch.empty(4, 256, dtype=torch.bfloat16, device="cuda")
    assert r.ctx.step_status(x, 5, r.weights, out) == B.MOE_ERR_INVALID_ARG
    assert r.ctx.step_status(x, -1, r.weights, out) == B.MOE_ERR_INVALID_ARG
    assert r.ctx.step_status(x, 4, r.weights, x) == B.MOE_ERR_INVALID_ARG      # out aliases x
    assert r.ctx.step_status(None, 4, r.weights, out) == B.MOE_ERR_INVALID_ARG
    mis = torch.empty(4 * 256 + 4, dtype=torch.bfloat16, device="cuda")[4:].view(4, 256)
    assert r.ctx.step_status(x, 4, r.weights, mis) == B.MOE_ERR_INVALID_ARG  # not 16-B aligned
    w = B.LayerRunner.weights_for(tiny)
    w.router_w = None
    assert r.ctx.step_status(x, 4, w, out) == B.MOE_ERR_INVALID_ARG


# ------------------------------------------------------------- GLM scale
@pytest.mark.parametrize("inter", [512, 1024, 1536])
@pytest.mark.parametrize("shared", [False, True])
def test_other_intermediate_sizes(inter, shared):
    """Intermediate sizes of 4, 8 and 12 K blocks (ring depths 4, 8 and 4 in
    down), with and without a shared expert, at one and two rows (one-tile
    down waves) and at 3 and 8 rows (two-tile down waves)."""
    shape = dict(hidden=512, inter=inter, n_experts=32, shared_inter=inter if shared else 0,
                 router_std=0.02)
    layer = S.make_layer(shape, seed=3000 + inter + shared, device="cuda")
    for rows in (1, 2, 3, 8):
        _say(f"inter={inter} shared={shared} rows={rows}")
        x = S.make_x(rows, layer.hidden, seed=3100 + rows)
        _, _, _, rep = _run(layer, x)
        _say(rep)


def test_smallest_layer():
    """The smallest accepted shapes: hidden 128 (one activation block, one K
    block per up/gate slab), intermediate 128, 16 experts (8 rows then pick
    most of them), with a shared expert, at 1 to 8 rows."""
    shape = dict(hidden=128, inter=128, n_experts=16, shared_inter=128, router_std=0.05)
    layer = S.make_layer(shape, seed=3700, device="cuda")
    for rows in (1, 2, 5, 8):
        _say(f"smallest layer rows={rows}")
        x = S.make_x(rows, 128, seed=3800 + rows)
        _, _, gpu, rep = _run(layer, x)
        _say(rep)
        assert int(np.asarray(gpu["n_groups"]).ravel()[0]) <= 16


@pytest.mark.parametrize("hidden,inter", [(16384, 256), (256, 16384)])
def test_maximum_hidden_and_intermediate(hidden, inter):
    """The largest sizes the library accepts, one at a time (with a shared
    expert): hidden 16384 (two rounds of 64 activation blocks per router
    block, 32 K blocks per up/gate wave) and intermediate 16384 (a 128-block
    down ring; at 8 rows 135 KB of dynamic LDS per down block)."""
    shape = dict(hidden=hidden, inter=inter, n_experts=32, shared_inter=inter, router_std=0.02)
    layer = S.make_layer(shape, seed=3500 + hidden, device="cuda")
    for rows in (1, 8):
        _say(f"hidden={hidden} inter={inter} rows={rows}")
        x = S.make_x(rows, hidden, seed=3600 + rows, mode="corr")
        _, _, _, rep = _run(layer, x)
        _say(rep)


@pytest.mark.parametrize("rows,mode", [(1, "indep"), (2, "corr"), (4, "indep"), (4, "corr"),
                                       (8, "indep"), (8, "corr")])
def test_glm_parity(glm, rows, mode):
    _say(f"glm rows={rows} mode={mode}")
    x = S.make_x(rows, glm.hidden, seed=3000 + 10 * rows + (mode == "corr"), mode=mode)
    _, _, gpu, rep = _run(glm, x, cache=glm.extra.setdefault("host", {}))
    _say(rep)


def test_glm_zero_row_and_zero_block(glm):
    """At GLM scale, 8 rows: row 0 all zero (every logit +0, picks 0..7,
    activation, mid and output zero), row 1 with one zero 128-block."""
    x = S.make_x(8, glm.hidden, seed=3300)
    x[0] = 0
    x[1, 1024:1152] = 0
    _say("glm zero row and zero block, 8 rows")
    _, out, gpu, rep = _run(glm, x, cache=glm.extra.setdefault("host", {}))
    _say(rep)
    assert list(gpu["ids"][0]) == list(range(8))
    assert not gpu["act_q"][0].any() and not gpu["act_s"][0].any()
    assert gpu["act_s"][1, 8] == 0 and not gpu["act_q"][1, 1024:1152].any()
    assert not gpu["midqs"][0].any() and not gpu["y"][0].any()
    assert not out[0].float().abs().sum().item()


@pytest.mark.parametrize("rows", [1, 4, 8])
def test_tiny_bf16_activations(tiny, rows):
    """MOE_ACT_BF16: the experts take u itself (no FP8 activation blocks);
    the same checks against the oracle in that mode, activation codes and
    scales all zero on both sides; dedup on/off bitwise equal."""
    _say(f"tiny bf16 activations rows={rows}")
    x = S.make_x(rows, tiny.hidden, seed=2700 + rows, mode="corr")
    _, out, gpu, rep = _run(tiny, x, act_fmt=B.ACT_BF16)
    _say(rep)
    assert not np.asarray(gpu["act_q"]).any() and not np.asarray(gpu["act_s"]).any()
    off = B.LayerRunner(tiny, rows, flags=B.F_NO_DEDUP, act_fmt=B.ACT_BF16).run(x.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), off.view(torch.int16))


@pytest.mark.parametrize("rows", [1, 8])
def test_glm_bf16_activations(glm, rows):
    _say(f"glm bf16 activations rows={rows}")
    x = S.make_x(rows, glm.hidden, seed=2800 + rows, mode="corr")
    _, _, _, rep = _run(glm, x, act_fmt=B.ACT_BF16, cache=glm.extra.setdefault("host", {}))
    _say(rep)


@pytest.mark.parametrize("inter", [256, 512])
def test_glm_intermediate_shares(inter):
    """The share of the GLM-scale layer one GPU streams when the intermediate
    dimension is split over 8 or 4 GPUs (intermediate 256 or 512, the same
    hidden size, 256 experts and router, a shared expert of the same share;
    the benchmark's seed), at 1, 2, 4 and 8 rows, independent and correlated."""
    shape = dict(S.SHAPES["glm"], inter=inter, shared_inter=inter)
    layer = S.make_layer(shape, seed=1003, device="cuda")
    cache = {}
    for rows, mode in ((1, "indep"), (2, "corr"), (4, "indep"), (8, "corr")):
        _say(f"glm share inter={inter} rows={rows} mode={mode}")
        x = S.make_x(rows, layer.hidden, seed=9100 + rows, mode=mode)
        _, _, _, rep = _run(layer, x, cache=cache)
        _say(rep)


def test_glm_dedup_off_is_bitwise_equal(glm):
    x = S.make_x(8, glm.hidden, seed=3100, mode="corr").cuda()
    on = B.LayerRunner(glm, 8).run(x)
    off = B.LayerRunner(glm, 8, flags=B.F_NO_DEDUP).run(x)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))


def test_relaunch_rewrites_the_same_values(tiny):
    """moe_decode_relaunch repeats the last step's up/gate or down with
    another copy of the same weights: mid and the output are unchanged
    bitwise; without a previous step, or for another kernel, it is refused."""
    runner = B.LayerRunner(tiny, 4)
    st = runner.ctx.relaunch_status(B.K_UPGATE, runner.weights, 1)
    assert st == B.MOE_ERR_INVALID_ARG  # no step yet
    x = S.make_x(3, tiny.hidden, seed=2600).cuda()
    out = runner.run(x)
    torch.cuda.synchronize()
    before = runner.debug(3)
    copy = S.Layer(tiny.shape, tiny.hidden, tiny.inter, tiny.n_experts, tiny.shared_inter,
                   tiny.rms_eps, tiny.gamma.clone(), tiny.router_w.clone(),
                   S.ExpertWeights(tiny.routed.fmt, *[tuple(t.clone() for t in m) for m in
                                                      (tiny.routed.gate, tiny.routed.up,
                                                       tiny.routed.down)]), None)
    wc = B.LayerRunner.weights_for(copy)
    runner.ctx.relaunch(B.K_UPGATE, wc, 3)
    runner.ctx.relaunch(B.K_DOWN, wc, 2)
    torch.cuda.synchronize()
    after = runner.debug(3)
    for k in ("mid", "midq", "midqs", "ids", "gates"):
        assert np.array_equal(before[k], after[k]), k
    assert runner.ctx.relaunch_status(0, wc, 1) == B.MOE_ERR_INVALID_ARG
    assert runner.ctx.relaunch_status(B.K_UPGATE, wc, -1) == B.MOE_ERR_INVALID_ARG
    assert runner.ctx.relaunch_status(B.K_UPGATE, wc, 0) == B.MOE_OK
    out2 = runner.run(x)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert runner.ctx.wait_timeouts() == 0
