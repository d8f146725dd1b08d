#!/usr/bin/env python3
"""MoE decode-step benchmark on one MI355X.

Workload: a GLM-scale MoE layer (hidden 6144, 256 routed experts of
intermediate 2048 with FP8 E4M3 weights and 128x128 fp32 block scales, top-8,
one always-on FP8 shared expert of intermediate 2048), decoded for 1 row; the
same layer is also timed at 2, 4 and 8 independent rows, at 4 and 8 correlated
rows (x_i = 0.8 x_0 + 0.6 N(0,1), so rows share experts and the dedup table is
smaller), with MXFP4 routed experts at 1 and 8 rows, and as the per-GPU share
of an 8- and a 4-way split of the intermediate dimension (intermediate 256 and
512, same hidden size, experts and router) at 1, 4 and 8 rows.  The
tail's LM-head GEMV ([151936, 6144] FP8 weights, lowbit_gemv's FP8 form) is
timed at 1 and 8 rows.  All inputs are seeded,
synthetic and already resident in HBM when the timed region starts.  Eight
copies of the layer's weights are rotated step by step so that no step finds
another step's weights in the 256 MB MALL or the L2s; a pool of 16 token rows
varies the routing.

One step = one moe_decode_step call: router, routing (up to 4 rows with the
up/gate of the shared and the routed experts, with mid, in the same launch;
else the routing alone, then the up/gate launch), down (with the mid
quantisation) and combine kernels.  Value =
algorithmic bytes of the step (each distinct expert counted once, read from
the step's own dedup table, plus the shared expert, router, gamma, x and out)
divided by the step time, timed over back-to-back steps.  The same steps are
also captured into a HIP graph (32 steps per graph) and replayed, for the
graph-replayed figure, and timed as the mean of 2 rounds of the median of 7
trials of 50 steps.  Context figures: the step with one weight copy reused
(hot), torch's copy of 2 GiB (read + write), lowbit_gemv against its VALU floor (one
lane-op per weight), and the oracle on one thread with the host CPU model.  A second pass over
the same steps has the library record HIP events around each kernel on the
step's stream.  The roofline figure is the dominant kernel's (the launch
that runs the up/gate: at 1 row the routing launch, with the routing block
and the shared and routed up/gate) algorithmic bytes over its average launch
duration, timed by HIP events around 64 back-to-back relaunches of it
(moe_decode_relaunch; a relaunched routing launch routes again from the
step's logits and its routed blocks wait for the new records) after one step,
each over another weight copy (an event pair per kernel inside a step adds
about 3-5 us).  The fp64 CPU oracle is timed on the host for a bounded sample of the
1-row workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode layer µs/step + weight-stream HBM GB/s (% of peak) at 1/4/8 rows"
PEAK_GBS = 8000.0  # MI355X HBM3E, published
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9  # fp32 lane-ops per second (157.3 TFLOP/s as FMAs)
POOL = 16
GSTEPS = 2 * POOL  # steps per captured graph
RELAUNCH = 64  # back-to-back launches of one kernel for its average duration
FUSED_MAX_ROWS = 4  # steps of up to 4 rows run their up/gate in the routing launch


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fp8_matrix_bytes(n, k):
    return n * k + (n // 128) * (k // 128) * 4


def mxfp4_matrix_bytes(n, k):
    return n * k // 2 + n * (k // 32)


def q1_matrix_bytes(n, k):
    return n * (k // 128) * 18


def routed_matrix_bytes(layer, n, k):
    return {2: mxfp4_matrix_bytes, 3: q1_matrix_bytes}.get(layer.routed_fmt, fp8_matrix_bytes)(n, k)


def step_bytes(layer, rows, d):
    H, I, E, Is = layer.hidden, layer.inter, layer.n_experts, layer.shared_inter
    expert = 2 * routed_matrix_bytes(layer, I, H) + routed_matrix_bytes(layer, H, I)
    shared = (2 * fp8_matrix_bytes(Is, H) + fp8_matrix_bytes(H, Is)) if Is else 0
    return d * expert + shared + E * H * 2 + H * 2 + 2 * rows * H * 2


def upgate_bytes(layer, rows, d):
    """Algorithmic bytes of the launch that runs the up/gate: the D distinct
    experts' gate and up matrices, the shared expert's gate and up, the
    activation codes and scales, and up to 4 rows (the routing launch) the
    router logits the routing block reads."""
    H, I, E, Is = layer.hidden, layer.inter, layer.n_experts, layer.shared_inter
    shared = 2 * fp8_matrix_bytes(Is, H) if Is else 0
    logits = rows * E * 4 if rows <= FUSED_MAX_ROWS else 0
    return (d * 2 * routed_matrix_bytes(layer, I, H) + shared + rows * H
            + rows * (H // 128) * 4 + logits)


def upgate_launch_us(kernel_us, rows):
    """In-step event span of the launch that runs the up/gate."""
    return kernel_us["route"] if rows <= FUSED_MAX_ROWS else kernel_us["upgate"]


def layer_copies(S, base, n):
    copies = [base]
    for _ in range(n - 1):
        copies.append(S.Layer(base.shape, base.hidden, base.inter, base.n_experts,
                              base.shared_inter, base.rms_eps, base.gamma.clone(),
                              base.router_w.clone(),
                              S.ExpertWeights(base.routed.fmt, *[tuple(None if t is None else
                                                                       t.clone() for t in m)
                                                                 for m in (base.routed.gate,
                                                                           base.routed.up,
                                                                           base.routed.down)]),
                              S.ExpertWeights(base.shared.fmt, *[tuple(t.clone() for t in m) for m in
                                                                 (base.shared.gate, base.shared.up,
                                                                  base.shared.down)])))
    return copies


# the sources of the routing launch's code (the counter record's hash)
TRAFFIC_SOURCES = ("route.hip", "route.h", "upgate.h", "device_common.h")


def measured_traffic():
    """HBM bytes per routing launch (routing + up/gate) at one row from the
    committed counter record, or None when the kernel source changed since it
    was taken."""
    import hashlib
    rec = os.path.join(ROOT, "profiles", "moe_route_upgate_glm_rows1_traffic.json")
    if not os.path.exists(rec):
        return None
    with open(rec) as f:
        r = json.load(f)
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "bit_moe_decode_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return int(r["traffic_bytes"]) if h.hexdigest() == r["source_sha256"] else None


def time_hot(torch, B, S, layer, rows, steps, seed_base):
    """The same step with one weight copy, reused every step (labelled hot:
    the weights partly stay in the 256 MB MALL)."""
    stream = torch.cuda.current_stream()
    runner = B.LayerRunner(layer, rows, stream=stream)
    wts = B.LayerRunner.weights_for(layer)
    pool = [S.make_x(rows, layer.hidden, seed=seed_base + t).cuda() for t in range(POOL)]
    out = torch.empty(rows, layer.hidden, dtype=torch.bfloat16, device="cuda")
    for i in range(20):
        runner.ctx.step(pool[i % POOL], rows, wts, out, stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        runner.ctx.step(pool[i % POOL], rows, wts, out, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / steps


def copy_stream_gbs(torch):
    """Context: torch's device copy of 2 GiB (read + write bytes / time), GB/s."""
    a = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    n = 10
    for _ in range(n):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * a.numel() * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def time_rows(torch, B, S, layer, copies, rows, steps, warmup, seed_base, mode="indep"):
    stream = torch.cuda.current_stream()
    runner = B.LayerRunner(layer, rows, stream=stream)
    weights = [B.LayerRunner.weights_for(c) for c in copies]
    pool = [S.make_x(rows, layer.hidden, seed=seed_base + t, mode=mode).cuda() for t in range(POOL)]
    out = torch.empty(rows, layer.hidden, dtype=torch.bfloat16, device="cuda")
    # distinct experts of each pool entry (selection does not depend on the copy)
    dvals = []
    for t in range(POOL):
        runner.ctx.step(pool[t], rows, weights[0], out, stream)
        torch.cuda.synchronize()
        dvals.append(runner.debug(rows)["n_groups"])
    for i in range(warmup):
        runner.ctx.step(pool[i % POOL], rows, weights[i % len(weights)], out, stream)
    nk = B.N_KERNELS
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # (a) the step as a caller runs it: back-to-back steps, no events between kernels
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        runner.ctx.step(pool[i % POOL], rows, weights[i % len(weights)], out, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # the pages' kernel-only protocol: mean of 2 rounds, each the median of 7
    # trials of 50 back-to-back steps
    rounds = []
    for rnd in range(2):
        trials = []
        for tr in range(7):
            torch.cuda.synchronize()
            t0.record(stream)
            for i in range(50):
                j = 50 * (7 * rnd + tr) + i
                runner.ctx.step(pool[j % POOL], rows, weights[j % len(weights)], out, stream)
            t1.record(stream)
            torch.cuda.synchronize()
            trials.append(t0.elapsed_time(t1) / 50)
        rounds.append(sorted(trials)[3])
    proto_ms = sum(rounds) / 2
    # (b) the same steps with the library's per-kernel events, for kernel durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    for row in evs:  # torch creates the HIP event on its first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        runner.ctx.set_timing(evs[i])
        runner.ctx.step(pool[i % POOL], rows, weights[i % len(weights)], out, stream)
    torch.cuda.synchronize()
    runner.ctx.set_timing(None)
    kern = [sum(evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(steps)) / steps
            for k in range(nk)]
    # (d) the up/gate and down kernels alone: after one step, back-to-back
    # relaunches over the other weight copies (the same experts at other
    # addresses, so each streams from HBM), bracketed by two events
    runner.ctx.step(pool[0], rows, weights[0], out, stream)
    alone = {}
    for name, kid in (("upgate", B.K_UPGATE), ("down", B.K_DOWN)):
        runner.ctx.relaunch(kid, weights[1 % len(weights)], 1, stream)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(RELAUNCH):
            runner.ctx.relaunch(kid, weights[(i + 2) % len(weights)], 1, stream)
        t1.record(stream)
        torch.cuda.synchronize()
        alone[name] = t0.elapsed_time(t1) * 1e3 / RELAUNCH
    ug_alone_bytes = upgate_bytes(layer, rows, dvals[0])
    # (c) the same kind of steps captured once into a HIP graph and replayed:
    # GSTEPS steps per graph (every pool entry and weight copy), replayed back to back
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        cs = torch.cuda.current_stream()
        for i in range(GSTEPS):
            runner.ctx.step(pool[i % POOL], rows, weights[i % len(weights)], out, cs)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    reps = max(1, steps // GSTEPS)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / (reps * GSTEPS)
    del g
    d_mean = sum(dvals[i % POOL] for i in range(steps)) / steps
    nbytes = sum(step_bytes(layer, rows, dvals[i % POOL]) for i in range(steps)) / steps
    ug_bytes = sum(upgate_bytes(layer, rows, dvals[i % POOL]) for i in range(steps)) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernel_us = {name: kern[k] * 1e3 for k, name in enumerate(B.KERNEL_NAMES)}
    ug_gbs = ug_bytes / (upgate_launch_us(kernel_us, rows) * 1e-6) / 1e9
    gd = sum(dvals[i % POOL] for i in range(GSTEPS)) / GSTEPS
    gbytes = sum(step_bytes(layer, rows, dvals[i % POOL]) for i in range(GSTEPS)) / GSTEPS
    graph = dict(us_per_step=graph_ms * 1e3, gbs=gbytes / (graph_ms * 1e-3) / 1e9,
                 distinct_experts=gd)
    # the protocol's steps cycle the same pool and copies, so the same mean D
    gbs_proto = nbytes / (proto_ms * 1e-3) / 1e9
    return dict(rows=rows, us_per_step=ms * 1e3, gbs=gbs, frac=gbs / PEAK_GBS, d_mean=d_mean,
                gbs_protocol=gbs_proto, frac_protocol=gbs_proto / PEAK_GBS,
                graph=graph, us_per_step_protocol=proto_ms * 1e3, alone_us=alone,
                upgate_alone_bytes=ug_alone_bytes,
                bytes_per_step=nbytes,
                kernel_us=kernel_us,
                upgate_gbs=ug_gbs, upgate_bytes=ug_bytes, runner=runner, pool=pool,
                weights=weights, dvals=dvals)


def row_summary(r):
    """The figures of one time_rows result that go into the JSON line: µs per
    step and GB/s by the pages' protocol (mean of 2 rounds of the median of 7
    trials of 50 steps), and of the plain back-to-back run."""
    return {"us_per_step": round(r["us_per_step_protocol"], 2),
            "gbs": round(r["gbs_protocol"], 1), "frac_of_peak": round(r["frac_protocol"], 4),
            "us_per_step_backtoback": round(r["us_per_step"], 2),
            "gbs_backtoback": round(r["gbs"], 1),
            "distinct_experts": r["d_mean"],
            "bytes_per_step": int(r["bytes_per_step"]),
            "kernel_us": {k: round(t, 2) for k, t in r["kernel_us"].items()},
            "kernel_alone_us": {k: round(t, 2) for k, t in r["alone_us"].items()},
            "graph_replay": {k: round(t, 2) for k, t in r["graph"].items()}}


# Per-GPU expert shares of the GLM layer when its intermediate dimension is
# split over 8 or 4 GPUs (each GPU streams 1/8 or 1/4 of every selected
# expert); same hidden size, experts and router.
TP_SHARES = (("tp8_inter256", 256), ("tp4_inter512", 512))


LOWBIT_SHAPES = (("mlp_up_gate", 9728, 2560), ("mlp_down", 2560, 9728), ("lm_head", 151936, 2560))

# The tail's LM-head GEMV in FP8 and in bf16 (lowbit_gemv's FP8 and bf16
# forms): the vocabulary of the 1-bit LM head above over the GLM hidden size.
LM_HEAD_FP8 = (151936, 6144)


def gemv_fp8_bytes(n, k, rows):
    return n * k + (n // 128) * (k // 128) * 4 + rows * k * 2 + rows * n * 2


def gemv_bf16_bytes(n, k, rows):
    return n * k * 2 + rows * k * 2 + rows * n * 2


def time_gemv_fp8(torch, B, S, n, k, rows, steps):
    """lowbit_gemv's FP8 form: back-to-back launches alternating over two
    weight copies (1.87 GB in all, past the MALL)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(79)
    w = torch.randn(n, k, generator=g, device="cuda")
    codes, scales = S.encode_fp8_blocks(w)
    del w
    mats = [(codes, scales), (codes.clone(), scales.clone())]
    x = S.make_x(rows, k, seed=80, device="cuda")
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    for i in range(10):
        B.gemv_fp8(*mats[i % 2], x, y, n, k, rows)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        B.gemv_fp8(*mats[i % 2], x, y, n, k, rows)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    nbytes = gemv_fp8_bytes(n, k, rows)
    gbs = nbytes / (us * 1e-6) / 1e9
    del mats, codes, scales
    torch.cuda.empty_cache()
    return dict(n=n, k=k, rows=rows, us=round(us, 2), gbs=round(gbs, 1),
                frac=round(gbs / PEAK_GBS, 4), bytes=nbytes)


def time_gemv_bf16(torch, B, S, n, k, rows, steps):
    """lowbit_gemv's bf16 form: back-to-back launches alternating over two
    weight copies (3.7 GB in all, past the MALL)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(81)
    mats = [(torch.randn(n, k, generator=g, device="cuda") * 0.05).to(torch.bfloat16)
            for _ in range(2)]
    x = S.make_x(rows, k, seed=82, device="cuda")
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    for i in range(10):
        B.gemv_bf16(mats[i % 2], x, y, n, k, rows)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        B.gemv_bf16(mats[i % 2], x, y, n, k, rows)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    nbytes = gemv_bf16_bytes(n, k, rows)
    gbs = nbytes / (us * 1e-6) / 1e9
    del mats
    torch.cuda.empty_cache()
    return dict(n=n, k=k, rows=rows, us=round(us, 2), gbs=round(gbs, 1),
                frac=round(gbs / PEAK_GBS, 4), bytes=nbytes)


def lowbit_bytes(n, k):
    return n * (k // 128) * 18 + k * 2 + n * 2


def time_lowbit(torch, B, S, n, k, steps, rows=1):
    """lowbit_gemv for `rows` input rows: back-to-back launches over enough
    weight copies (>= 512 MB in all) that no launch finds its matrix in the MALL."""
    size = n * (k // 128) * 18
    ncopy = max(2, -(-512 * 2 ** 20 // size))
    base = S.make_q1(n, k, seed=77, device="cuda")
    mats = [base] + [base.clone() for _ in range(ncopy - 1)]
    x = S.make_x(rows, k, seed=78, device="cuda")
    y = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    for i in range(10):
        B.lowbit_gemv(mats[i % ncopy], x, y, n, k, rows)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        B.lowbit_gemv(mats[i % ncopy], x, y, n, k, rows)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    nbytes = lowbit_bytes(n, k) + (rows - 1) * (k + n) * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    del mats
    # VALU floor at one row: one fp32 lane-op per weight at 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz
    valu_us = n * k / VALU_LANE_OPS * 1e6
    out = dict(n=n, k=k, rows=rows, us=round(us, 2), gbs=round(gbs, 1),
               frac=round(gbs / PEAK_GBS, 4), bytes=nbytes, copies=ncopy)
    if rows == 1:
        out.update(valu_floor_us=round(valu_us, 2), valu_frac=round(valu_us / us, 4))
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_threads():
    """Host threads for the oracle: every core this process may run on, but
    no more than OMP_NUM_THREADS when that is set (the GPU machine sets it to its
    CPU share per GPU)."""
    aff = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return (min(aff, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else aff), aff


def oracle_steps(torch, layer, runner, pool, weights, rows, seconds, max_steps, threads, cache):
    """The oracle (fp64, `threads` OpenMP threads) on full steps of the pool,
    anchored on the GPU's logits, until `seconds` of oracle time or
    `max_steps`; each step is also checked against the GPU's output."""
    from tests import parity as P
    done, t_used, nbytes, errs = 0, 0.0, 0.0, []
    out = torch.empty(rows, layer.hidden, dtype=torch.bfloat16, device="cuda")
    while done < max_steps and (done == 0 or t_used < seconds):
        x = pool[done % len(pool)]
        runner.ctx.step(x, rows, weights, out)
        torch.cuda.synchronize()
        gpu = runner.debug(rows)
        for e in sorted(set(int(e) for e in gpu["ids"].ravel())):
            if e not in cache:
                cache[e] = P.expert_host(layer, e)
        xc = x.cpu()
        t = time.perf_counter()
        ref_out, ref = P.oracle_for(layer, xc, gpu["logits"], nthreads=threads, host_cache=cache)
        t_used += time.perf_counter() - t
        nbytes += step_bytes(layer, rows, gpu["n_groups"])
        errs.append(P.compare(layer, xc, gpu, out, ref_out, ref)["out_err_rel_max"])
        done += 1
    return dict(ms_per_step=round(t_used / done * 1e3, 2), gbs=round(nbytes / t_used / 1e9, 3),
                steps=done, out_err_rel_max=max(errs))


def oracle_lowbit(S, n, k, threads):
    """The oracle's 1-bit GEMV at one [n, k] shape, one row."""
    from oracle import oracle as O
    blk = S.make_q1(n, k, seed=77).numpy()
    xb = S.bf16_bits(S.make_x(1, k, seed=78)[0]).numpy().view("uint16")
    t = time.perf_counter()
    O.lowbit_gemv_q1(blk, xb, n, k, nthreads=threads)
    dt = time.perf_counter() - t
    return dict(ms=round(dt * 1e3, 2), gbs=round(lowbit_bytes(n, k) / dt / 1e9, 3))


def cpu_baseline(torch, B, S, layer, results, seconds):
    """The oracle timed on the host: the headline figure on 1-row GLM-scale
    steps (about `seconds` of oracle time), then bounded samples at 4 and 8
    rows, on the tiny layer at 1/4/8 rows and the 1-bit GEMV shapes, plus 4
    one-row steps on a single thread."""
    threads, aff = oracle_threads()
    cache = {}
    m = results[1]
    main = oracle_steps(torch, layer, m["runner"], m["pool"], m["weights"][0], 1, seconds,
                        64 * POOL, threads, cache)
    per = {"glm_fp8_rows1": main}
    for rows, secs in ((4, 3.0), (8, 4.0)):
        if rows in results:
            r = results[rows]
            per[f"glm_fp8_rows{rows}"] = oracle_steps(torch, layer, r["runner"], r["pool"],
                                                     r["weights"][0], rows, secs, 4, threads,
                                                     cache)
            log(f"oracle glm rows={rows}: {per[f'glm_fp8_rows{rows}']}")
    cache.clear()
    tiny = S.make_layer("tiny", seed=1000, device="cuda")
    for rows in (1, 4, 8):
        runner = B.LayerRunner(tiny, rows)
        pool = [S.make_x(rows, tiny.hidden, seed=7500 + 10 * rows + t).cuda() for t in range(4)]
        o = oracle_steps(torch, tiny, runner, pool, runner.weights, rows, 0.5, 40, threads, {})
        per[f"tiny_rows{rows}"] = dict(us_per_step=round(o["ms_per_step"] * 1e3, 1),
                                       steps=o["steps"], out_err_rel_max=o["out_err_rel_max"])
    for name, n, k in LOWBIT_SHAPES:
        per[f"lowbit_{name}"] = oracle_lowbit(S, n, k, threads)
        log(f"oracle lowbit {name}: {per[f'lowbit_{name}']}")
    single = oracle_steps(torch, layer, m["runner"], m["pool"], m["weights"][0], 1, 1e9, 4, 1,
                          cache)
    return dict(value=main["gbs"], unit="GB/s", cores=threads, kind="oracle",
                cpu_model=cpu_model(), affinity_cores=aff,
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"),
                single_thread=dict(value=single["gbs"], unit="GB/s", cores=1,
                                   ms_per_step=single["ms_per_step"],
                                   sample=f"{single['steps']} full 1-row steps"),
                sample=f"{main['steps']} full 1-row GLM-scale steps (router, 8 routed + shared "
                       f"expert, combine; the {POOL} token rows of the timed pool, cycled), fp64, "
                       f"{threads} OpenMP threads",
                ms_per_step=main["ms_per_step"], per_config=per), main["out_err_rel_max"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rows", default="1,2,4,8")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lowbit", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true")
    ap.add_argument("--no-corr", action="store_true")
    ap.add_argument("--no-tp-share", action="store_true")
    ap.add_argument("--no-tiny", action="store_true")
    ap.add_argument("--no-q1", action="store_true")
    ap.add_argument("--counter-calibration", action="store_true",
                    help="also run torch's elementwise abs over 12,582,912 fp32 (50,331,648 B "
                         "read and written): the reference dispatch that scales HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode step has no multi-GPU path in this "
              "library (how it would shard is described in DESIGN.md); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_moe_decode_amd import binding as B
    from bit_moe_decode_amd import synth as S

    B.lib()
    torch.cuda.set_device(0)
    if args.counter_calibration:
        a = torch.randn(12582912, device="cuda")
        torch.abs(a)
        torch.cuda.synchronize()
        del a
    log("generating GLM-scale layer")
    base = S.make_layer("glm", seed=1001, device="cuda")
    copies = layer_copies(S, base, args.copies)
    ncopies = len(copies)
    torch.cuda.synchronize()
    log(f"{ncopies} layer copies resident")

    results = {}
    for rows in [int(r) for r in args.rows.split(",")]:
        log(f"timing rows={rows}")
        results[rows] = time_rows(torch, B, S, base, copies, rows, args.steps, args.warmup,
                                  seed_base=5000 + 100 * rows)
        r = results[rows]
        log(f"rows={rows}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s "
            f"({100 * r['frac']:.1f}% of peak), D={r['d_mean']:.1f}, kernels {r['kernel_us']}; "
            f"graph replay {r['graph']['us_per_step']:.1f} us/step")

    main_rows = 1 if 1 in results else min(results)
    m = results[main_rows]
    hot = {}
    for rows in results:
        hot[str(rows)] = round(time_hot(torch, B, S, base, rows, args.steps, 7000 + 100 * rows), 2)
        log(f"hot (one weight copy) rows={rows}: {hot[str(rows)]} us/step")
    tiny = None
    if not args.no_tiny:
        # the tiny layer (hidden 256, 32 experts of 128, no shared expert):
        # 0.8-3.2 MB a step, cache-resident and latency-bound, so µs only
        tiny = {}
        tl = S.make_layer("tiny", seed=1000, device="cuda")
        for rows in (1, 4, 8):
            r = time_rows(torch, B, S, tl, [tl], rows, args.steps, args.warmup,
                          seed_base=7000 + 10 * rows)
            tiny[str(rows)] = {"us_per_step": round(r["us_per_step_protocol"], 2),
                               "us_per_step_backtoback": round(r["us_per_step"], 2),
                               "graph_replay_us_per_step": round(r["graph"]["us_per_step"], 2),
                               "distinct_experts": r["d_mean"],
                               "kernel_us": {k: round(t, 2) for k, t in r["kernel_us"].items()}}
            log(f"tiny rows={rows}: {tiny[str(rows)]}")
    stream_gbs = copy_stream_gbs(torch)
    log(f"copy stream (torch copy of 2 GiB, read + write): {stream_gbs:.0f} GB/s")
    cpu, err = (None, None)
    if not args.no_cpu_baseline and main_rows == 1:
        log("timing the oracle on the host")
        cpu, err = cpu_baseline(torch, B, S, base, results, args.cpu_seconds)
    corr = None
    if not args.no_corr:
        # correlated rows (x_i = 0.8 x_0 + 0.6 N(0,1)): rows share experts, the
        # dedup table has fewer groups and each is streamed once
        corr = {}
        for rows in (4, 8):
            r = time_rows(torch, B, S, base, copies, rows, args.steps, args.warmup,
                          seed_base=8000 + 100 * rows, mode="corr")
            log(f"corr rows={rows}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s "
                f"({100 * r['frac']:.1f}% of peak), D={r['d_mean']:.1f}, kernels {r['kernel_us']}")
            corr[str(rows)] = row_summary(r)
    mx = None
    if not args.no_mxfp4:
        log("generating the GLM-scale layer with MXFP4 routed experts")
        copies = None
        torch.cuda.empty_cache()
        mbase = S.make_layer("glm", routed_fmt=S.FMT_MXFP4, seed=1002, device="cuda")
        mcopies = layer_copies(S, mbase, args.copies)
        torch.cuda.synchronize()
        mx = {}
        for rows in (1, 8):
            r = time_rows(torch, B, S, mbase, mcopies, rows, args.steps, args.warmup,
                          seed_base=6000 + 100 * rows)
            log(f"mxfp4 rows={rows}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s "
                f"({100 * r['frac']:.1f}% of peak), D={r['d_mean']:.1f}, kernels {r['kernel_us']}")
            mx[str(rows)] = row_summary(r)
            if rows == 8 and cpu is not None:
                threads, _ = oracle_threads()
                o = oracle_steps(torch, mbase, r["runner"], r["pool"], r["weights"][0], 8, 4.0,
                                 2, threads, {})
                cpu["per_config"]["glm_mxfp4_rows8"] = o
                log(f"oracle mxfp4 rows=8: {o}")
        del mcopies, mbase
        torch.cuda.empty_cache()

    q1 = None
    if not args.no_q1:
        # 1-bit (Q1_0_G128) routed experts, FP8 shared expert: 5.3 MB a routed
        # expert, so the shared expert and the router are most of a 1-row step
        log("generating the GLM-scale layer with 1-bit routed experts")
        copies = None
        torch.cuda.empty_cache()
        qbase = S.make_layer("glm", routed_fmt=S.FMT_Q1, seed=1004, device="cuda")
        qcopies = layer_copies(S, qbase, args.copies)
        torch.cuda.synchronize()
        q1 = {}
        for rows in (1, 8):
            r = time_rows(torch, B, S, qbase, qcopies, rows, args.steps, args.warmup,
                          seed_base=6500 + 100 * rows)
            log(f"q1 rows={rows}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s "
                f"({100 * r['frac']:.1f}% of peak), D={r['d_mean']:.1f}, kernels {r['kernel_us']}")
            q1[str(rows)] = row_summary(r)
        del qcopies, qbase
        torch.cuda.empty_cache()

    tp = None
    if not args.no_tp_share:
        copies = None
        torch.cuda.empty_cache()
        tp = {}
        for name, inter in TP_SHARES:
            shape = dict(S.SHAPES["glm"], inter=inter, shared_inter=inter)
            log(f"generating the {name} share of the GLM-scale layer")
            tbase = S.make_layer(shape, seed=1003, device="cuda")
            tcopies = layer_copies(S, tbase, args.copies)
            torch.cuda.synchronize()
            tp[name] = {}
            for rows in (1, 4, 8):
                r = time_rows(torch, B, S, tbase, tcopies, rows, args.steps, args.warmup,
                              seed_base=9000 + 100 * rows)
                log(f"{name} rows={rows}: {r['us_per_step']:.1f} us/step, {r['gbs']:.0f} GB/s "
                    f"({100 * r['frac']:.1f}% of peak), D={r['d_mean']:.1f}, "
                    f"kernels {r['kernel_us']}")
                tp[name][str(rows)] = row_summary(r)
            del tcopies, tbase
            torch.cuda.empty_cache()

    lowbit = None
    head = head_bf = None
    if not args.no_lowbit:
        lowbit = {}
        for name, n, k in LOWBIT_SHAPES:
            log(f"timing lowbit_gemv {name} [{n}, {k}]")
            lowbit[name] = time_lowbit(torch, B, S, n, k, steps=max(args.steps, 50))
            log(f"  {lowbit[name]}")
            lowbit[name + "_8rows"] = time_lowbit(torch, B, S, n, k, steps=max(args.steps, 50),
                                                  rows=8)
            log(f"  8 rows: {lowbit[name + '_8rows']}")
        head, head_bf = {}, {}
        for rows in (1, 8):
            n, k = LM_HEAD_FP8
            log(f"timing lowbit_gemv FP8 LM head [{n}, {k}] rows={rows}")
            head[str(rows)] = time_gemv_fp8(torch, B, S, n, k, rows, steps=max(args.steps, 50))
            log(f"  {head[str(rows)]}")
        for rows in (1, 8):
            n, k = LM_HEAD_FP8
            log(f"timing lowbit_gemv bf16 LM head [{n}, {k}] rows={rows}")
            head_bf[str(rows)] = time_gemv_bf16(torch, B, S, n, k, rows,
                                                steps=max(args.steps, 50))
            log(f"  {head_bf[str(rows)]}")

    line = {
        "metric": METRIC,
        "value": round(m["gbs_protocol"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["us_per_step_protocol"] / 1e3, 5),
        "us_per_step": round(m["us_per_step_protocol"], 2),
        "frac_of_peak": round(m["frac_protocol"], 4),
        "timing": "mean of 2 rounds of the median of 7 trials of 50 back-to-back steps; "
                  "us_per_step_backtoback = the same steps timed once over --steps",
        "us_per_step_backtoback": round(m["us_per_step"], 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"GLM-scale MoE decode layer, {main_rows} row: hidden 6144, "
                               "256 routed experts (top-8) of intermediate 2048 + 1 shared "
                               "expert of 2048, FP8 E4M3 weights with 128x128 fp32 scales, "
                               "FP8 activations and mid, bf16 in/out",
                   "rows": main_rows, "layer_copies": ncopies, "x_pool": POOL},
        "roofline": {"bound": "hbm",
                     "kernel": ("moe_route_kernel (routing block + shared and routed up/gate)"
                                if main_rows <= FUSED_MAX_ROWS else "moe_upgate_kernel"),
                     "achieved": round(m["upgate_alone_bytes"] / (m["alone_us"]["upgate"] * 1e-6) / 1e9, 1),
                     "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(m["upgate_alone_bytes"] / (m["alone_us"]["upgate"] * 1e-6) / 1e9
                                   / PEAK_GBS, 4),
                     "bytes_per_launch": int(m["upgate_alone_bytes"]),
                     "us_per_launch": round(m["alone_us"]["upgate"], 2),
                     "launches_timed": RELAUNCH,
                     "us_per_launch_in_step_events": round(upgate_launch_us(m["kernel_us"],
                                                                            main_rows), 2),
                     "traffic": measured_traffic() if main_rows == 1 else None},
        "cpu_baseline": cpu,
        "oracle_check_out_err_rel_max": err,
        "by_rows": {str(r): dict(row_summary(v),
                                 upgate_alone_gbs=round(v["upgate_alone_bytes"]
                                                        / (v["alone_us"]["upgate"] * 1e-6) / 1e9, 1))
                    for r, v in results.items()},
        "tiny_layer": tiny,
        "hot_us_per_step": hot,
        "copy_stream_gbs": round(stream_gbs, 1),
        "corr_rows": corr,
        "mxfp4_routed": mx,
        "q1_routed": q1,
        "tp_share": tp,
        "lowbit_gemv": lowbit,
        "lm_head_fp8": head,
        "lm_head_bf16": head_bf,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
