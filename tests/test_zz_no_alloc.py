"""The decode step that allocates nothing (moe_decode_step_noalloc), called
through the C ABI, against the context-based step (moe_decode_step) on the
same inputs: outputs bitwise equal (same kernels, same arithmetic), over
consecutive calls that reuse the library's static device scratch, each
later call smaller than the one before it."""
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(layer, x, max_rows, flags=0):
    """(context-based output, no-allocation output) of one step."""
    rows = x.shape[0]
    runner = B.LayerRunner(layer, max_rows, flags=flags)
    ref = runner.run(x)
    out = torch.full_like(ref, float("nan"))
    st = B.step_noalloc_status(runner.cfg, x, rows, runner.weights, out)
    assert st == B.MOE_OK, B.status_string(st)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_step_matches_the_context_step():
    _say("generating the GLM-scale layer")
    glm = S.make_layer("glm", seed=1001, device="cuda")
    tiny = S.make_layer("tiny", seed=1000, device="cuda")
    mx = S.make_layer(dict(hidden=512, inter=256, n_experts=64, shared_inter=256,
                           router_std=0.02), routed_fmt=S.FMT_MXFP4, seed=1005, device="cuda")
    # each call smaller than the previous one: stale scratch from a larger
    # step must not leak into a smaller one
    cases = [(glm, 8, "indep", 0), (glm, 2, "corr", 0), (mx, 4, "corr", 0),
             (tiny, 8, "corr", B.F_NO_DEDUP), (tiny, 1, "indep", 0)]
    for i, (layer, rows, mode, flags) in enumerate(cases):
        _say(f"no-alloc step: hidden={layer.hidden} rows={rows} mode={mode} flags={flags}")
        x = S.make_x(rows, layer.hidden, seed=6100 + i, mode=mode).cuda()
        ref, out = _both(layer, x, 8, flags)
        assert torch.equal(ref.view(torch.int16), out.view(torch.int16)), (layer.hidden, rows)
    # the same GLM-scale 8-row step again after the smaller ones
    x = S.make_x(8, glm.hidden, seed=6100, mode="indep").cuda()
    ref, out = _both(glm, x, 8)
    assert torch.equal(ref.view(torch.int16), out.view(torch.int16))


def test_noalloc_step_rejects_what_the_scratch_cannot_hold():
    big = B.Config(16384, 16384, 1024, 8, 16384, 8, 1e-6, B.FMT_FP8, B.FMT_FP8, 0, 0)
    assert B.workspace_size(big) > B.NOALLOC_MAX_WORKSPACE
    x = torch.zeros(1, 16384, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    w = B.Weights()
    assert B.step_noalloc_status(big, x, 1, w, out) == B.MOE_ERR_WORKSPACE
    tiny = S.make_layer("tiny", seed=1000, device="cuda")
    r = B.LayerRunner(tiny, 4)
    x = S.make_x(4, 256, seed=1).cuda()
    out = torch.empty(4, 256, dtype=torch.bfloat16, device="cuda")
    assert B.step_noalloc_status(r.cfg, x, 5, r.weights, out) == B.MOE_ERR_INVALID_ARG
    assert B.step_noalloc_status(r.cfg, x, 4, r.weights, x) == B.MOE_ERR_INVALID_ARG
    assert B.step_noalloc_status(r.cfg, x, 0, r.weights, out) == B.MOE_OK
