"""The routing launch's hand-off: the routing block publishes one record per
routed up/gate block of the same launch, and each of those blocks waits for
its own record (capped) before it streams its expert's weights.

Checks: consecutive steps with other token rows on one context give the same
output, bit for bit, as fresh contexts (no record of an earlier step is ever
taken); a withheld publication (the test-only switch) makes every routed
block give up at the cap, count itself and skip its work, every kernel still
ending; the next normal step is correct again with no further give-up.
Steps of more than 4 rows run the routing alone: the switch changes nothing
there.
"""
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


FUSED_MAX_ROWS = 4  # steps of up to 4 rows run their up/gate in the routing launch


def _routed_blocks(layer, rows):
    """Routed up/gate blocks of a routing launch: groups x slabs-per-group.
    K parts (FP8 experts): the largest of 4, 2, 1 dividing H/128; a block
    holds 4/ks slabs of 16 intermediate rows.  0 for steps whose up/gate runs
    in its own launch (nothing waits there)."""
    if rows > FUSED_MAX_ROWS:
        return 0
    nk = layer.hidden // 128
    ks = 4 if nk % 4 == 0 else (2 if nk % 2 == 0 else 1)
    groups = min(8 * rows, layer.n_experts)
    return groups * (layer.inter // (16 * (4 // ks)))


@pytest.fixture(scope="module")
def tiny():
    return S.make_layer("tiny", seed=1000, device="cuda")


@pytest.mark.parametrize("rows", [1, 3, 8])
def test_consecutive_steps_take_only_their_own_records(tiny, rows):
    _say(f"consecutive steps rows={rows}")
    xs = [S.make_x(rows, tiny.hidden, seed=4100 + 7 * i + rows).cuda() for i in range(4)]
    runner = B.LayerRunner(tiny, 8)
    outs = [runner.run(x).clone() for x in xs + xs[::-1]]
    torch.cuda.synchronize()
    for i, x in enumerate(xs + xs[::-1]):
        fresh = B.LayerRunner(tiny, 8).run(x)
        torch.cuda.synchronize()
        assert torch.equal(outs[i].view(torch.int16), fresh.view(torch.int16)), i
    assert runner.ctx.wait_timeouts() == 0


@pytest.mark.parametrize("rows", [1, 4, 8])
def test_withheld_records_time_out_and_every_kernel_ends(tiny, rows):
    _say(f"withheld records rows={rows}")
    x = S.make_x(rows, tiny.hidden, seed=4200 + rows).cuda()
    runner = B.LayerRunner(tiny, 8)
    good = runner.run(x).clone()
    torch.cuda.synchronize()
    assert runner.ctx.wait_timeouts() == 0
    runner.ctx.set_wait(cap_ticks=2000, withhold=1)  # 20 us cap, no records
    held = runner.run(x).clone()
    torch.cuda.synchronize()  # every kernel has ended
    n = _routed_blocks(tiny, rows)
    assert runner.ctx.wait_timeouts() == n
    if n == 0:  # the routing ran alone: nothing waited, the output is right
        assert torch.equal(held.view(torch.int16), good.view(torch.int16))
    runner.ctx.set_wait(0, 0)  # default cap, records published
    again = runner.run(x)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), good.view(torch.int16))
    assert runner.ctx.wait_timeouts() == n  # no further give-up


def test_set_wait_rejects_bad_arguments(tiny):
    runner = B.LayerRunner(tiny, 1)
    assert B.lib().moe_decode_set_wait(runner.ctx.handle, 0, 2) == B.MOE_ERR_INVALID_ARG
    assert B.lib().moe_decode_set_wait(None, 0, 0) == B.MOE_ERR_INVALID_ARG


def test_many_glm_steps_reproduce_bit_for_bit():
    """Back-to-back GLM-scale steps (the routing hand-off, and the down
    launch's combine across waves of every XCD) reproduce, bit for bit, the
    output of the same token row computed alone."""
    _say("generating the GLM-scale layer")
    glm = S.make_layer("glm", seed=1001, device="cuda")
    for rows in (1, 4):
        _say(f"many steps rows={rows}")
        xs = [S.make_x(rows, glm.hidden, seed=4300 + 11 * i + rows).cuda() for i in range(6)]
        ref = []
        for x in xs:
            ref.append(B.LayerRunner(glm, rows).run(x).clone())
        torch.cuda.synchronize()
        runner = B.LayerRunner(glm, rows)
        outs = [torch.empty_like(ref[0]) for _ in range(60)]
        for i in range(60):
            runner.run(xs[i % 6], out=outs[i])
        torch.cuda.synchronize()
        bad = [i for i in range(60)
               if not torch.equal(outs[i].view(torch.int16), ref[i % 6].view(torch.int16))]
        assert not bad, bad
        assert runner.ctx.wait_timeouts() == 0
