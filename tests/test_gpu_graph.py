"""The decode step, and lowbit_gemv's forms, captured into a HIP graph: every
replay must give the same output bits as the eager calls on the same inputs.

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


def test_graph_replay_q1_experts():
    """1-bit routed experts (and the FP8 shared expert) at 1, 4 and 8 rows."""
    layer = S.make_layer(dict(hidden=1024, inter=512, n_experts=64, shared_inter=512,
                              router_std=0.02), routed_fmt=S.FMT_Q1, seed=1007, device="cuda")
    _graph_vs_eager(layer, [8, 1, 4], seed=7300)


def test_graph_replay_lowbit_gemv_forms():
    """lowbit_gemv's three forms (1-bit at 1 and 4 rows, FP8 and bf16 at 1 and
    8 rows) captured into one graph: every replay, with eager calls of other
    inputs and host synchronisations between replays, gives the eager bits."""
    n, k = 1024, 2560
    q1 = S.make_q1(n, k, seed=71, device="cuda")
    g8 = torch.Generator(device="cuda")
    g8.manual_seed(72)
    codes, scales = S.encode_fp8_blocks(torch.randn(n, k, generator=g8, device="cuda"))
    wb = (torch.randn(n, k, generator=g8, device="cuda") * 0.05).to(torch.bfloat16)

    def calls(xs, ys, stream):
        B.lowbit_gemv(q1, xs[0], ys[0], n, k, 1, stream)
        B.lowbit_gemv(q1, xs[1], ys[1], n, k, 4, stream)
        B.gemv_fp8(codes, scales, xs[2], ys[2], n, k, 1, stream)
        B.gemv_fp8(codes, scales, xs[3], ys[3], n, k, 8, stream)
        B.gemv_bf16(wb, xs[4], ys[4], n, k, 1, stream)
        B.gemv_bf16(wb, xs[5], ys[5], n, k, 8, stream)

    rows = (1, 4, 1, 8, 1, 8)
    xs = [S.make_x(r, k, seed=73 + i).cuda() for i, r in enumerate(rows)]
    eager = [torch.empty(r, n, dtype=torch.bfloat16, device="cuda") for r in rows]
    calls(xs, eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        calls(xs, outs, torch.cuda.current_stream())
    torch.cuda.synchronize()
    others = [S.make_x(r, k, seed=90 + i).cuda() for i, r in enumerate(rows)]
    scratch = [torch.empty_like(e) for e in eager]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), ("replay", rep, "call", i)
        calls(others, scratch, torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()
    del g
