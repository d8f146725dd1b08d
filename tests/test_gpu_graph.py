"""The decode step captured into a HIP graph: every replay must give the same
output bits as the eager step on the same inputs.

A graph holds several steps (different token rows, row counts and weights
on one context); it is replayed several times, with eager steps of other
inputs and host synchronisations in between, and every replay's outputs are
compared bitwise with eager runs.  The eager step itself is checked against
the oracle elsewhere, so bitwise equality carries that parity over.
"""
import numpy as np
import pytest
import torch

from bit_moe_decode_amd import binding as B
from bit_moe_decode_amd import synth as S

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _graph_vs_eager(layer, row_counts, seed):
    runner = B.LayerRunner(layer, max(row_counts))
    xs = [S.make_x(r, layer.hidden, seed=seed + i, mode="corr" if i % 2 else "indep").cuda()
          for i, r in enumerate(row_counts)]
    eager = []
    for x in xs:
        eager.append(runner.run(x).clone())
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        cs = torch.cuda.current_stream()
        for x, o in zip(xs, outs):
            runner.ctx.step(x, x.shape[0], runner.weights, o, cs)
    torch.cuda.synchronize()
    other = S.make_x(max(row_counts), layer.hidden, seed=seed + 99).cuda()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), ("replay", rep, "step", i)
        runner.run(other)  # eager work between replays
        torch.cuda.synchronize()
    # the last graph step's intermediates are what the debug view shows
    g.replay()
    torch.cuda.synchronize()
    last = runner.debug(xs[-1].shape[0])
    runner.run(xs[-1])
    torch.cuda.synchronize()
    ref = runner.debug(xs[-1].shape[0])
    for k in ("ids", "gates", "n_groups", "act_q", "act_s", "mid"):
        assert np.array_equal(np.asarray(last[k]), np.asarray(ref[k])), k
    del g


def test_graph_replay_tiny():
    layer = S.make_layer("tiny", seed=1000, device="cuda")
    _graph_vs_eager(layer, [1, 8, 3, 1], seed=7100)


def test_graph_replay_glm():
    _say("generating the GLM-scale layer on the device")
    layer = S.make_layer("glm", seed=1001, device="cuda")
    _graph_vs_eager(layer, [1, 8, 4], seed=7200)


def test_graph_replay_glm_mxfp4():
    layer = S.make_layer("glm", routed_fmt=S.FMT_MXFP4, seed=1002, device="cuda")
    _graph_vs_eager(layer, [8, 1], seed=7300)
