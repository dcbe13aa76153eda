"""Benchmark of the denoising-step hot path on one MI355X.

One step = one step of the denoising loop of the stack workload: 30 MoE FFN layers
(256-token canvas, d_model 2816, expert ffn 704, 128 experts top-8, W4A16 group 64,
Zipf(1.2) routing), each as route -> gate/up (GeGLU) -> down -> fixed-order combine, then the
sampler (entropy + gumbel-max over fp32 logits [256, 262144], temperature 1, then the
entropy-bound acceptance at bound 2.0), then the loop driver's update (drafts into the
canvas, the stability count, the end of the block).  A block of 48 steps starts from a
seeded random canvas and runs as one captured HIP graph whose launches are gated on the
driver's done flag; accepted positions stay frozen within a block.  All inputs are seeded
synthetic tensors resident in HBM before timing starts.

value = algorithmic bytes of the step (touched expert weights with their scales and
zero-points, activations in and out, router logits, the unfrozen logits rows; nothing for a
step after its block has ended) / time, in GB/s; ms_per_step is the latency of one step, from
one event pair around the timed steps (no other event inside);
config.step_ms_p10_p50_p90_over_blocks is the spread of the per-step time over block replays;
the gate/up roofline comes from a third pass of eager launches (see main).

Two more workloads time the parts on their own configurations (--workload):
  layer    one MoE FFN layer (route, gate/up, down, combine) at the 256-token canvas with uniform
           N(0, 1) router logits (every expert touched), two independently seeded layers in turn;
  sampler  the sampler step alone over fp32 logits [256, 262144] (every row unfrozen), two copies
           of the logits in turn;
  chain    the stack's loop with the layers chained on the device: per layer RMS norm, router
           projection, routing, FFN and combine, the output feeding the next layer (routing
           from the router itself, not given logits).
Each reports the same fields; its roofline covers its dominant launch (the chain: the step).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload stack|layer|sampler|chain] [--no-components] [--no-graph]
                       [--checkpoint-format]
                       [--eager-only]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--layers", type=int, default=None, help="MoE layers per step (default 30)")
    ap.add_argument("--workload", choices=("stack", "layer", "sampler", "chain"), default="stack",
                    help="stack (default): the whole denoising step; layer: one FFN layer at the "
                         "256-token canvas with uniform routing; sampler: the sampler alone; "
                         "chain: the denoising step with the layers chained through the RMS norm "
                         "and the router projection")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--checkpoint-format", action="store_true",
                    help="layer workload: gate/up grouped at 128 and down at 64, the format of "
                         "the model card's checkpoint")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the one-launch-at-a-time part timings (e.g. for counter runs)")
    ap.add_argument("--eager-only", action="store_true",
                    help="stack workload: run only the eager pass of pre-marshalled launches (the "
                         "gate/up roofline; value and ms_per_step are null), for counter "
                         "collection")
    ap.add_argument("--no-graph", action="store_true",
                    help="stack workload: issue each block's launches eagerly instead of replaying "
                         "its captured graph (for counter collection, which does not follow "
                         "graph launches)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(per_launch_alg_bytes):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, "gate_up_w4a16_stack_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from block_diffusion_lm_router_amd.profsum import kernel_source_hash
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


BASELINE_LAYERS = 4     # oracle sample: this many whole layers ...
BASELINE_STEPS = 2      # ... and this many whole sampler steps (about 10 s of CPU work)


def host_cores():
    """Cores this process may run on (its affinity mask), at most 16: the host share that
    comes with one GPU on the benchmark machines."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _sample_block(args):
    """Worker: the oracle's entropy and token of the given rows (their original indices keep
    the Philox counters of the full tensor)."""
    rows_x, row_ids, temperature, seed, step = args
    from oracle import sampler as osamp
    H = np.empty(len(row_ids))
    tok = np.empty(len(row_ids), dtype=np.int64)
    for i, p in enumerate(row_ids):
        H[i] = osamp.entropy(rows_x[i])
        tok[i] = (osamp.draw_token(rows_x[i], temperature, seed, step, int(p))[0]
                  if np.isfinite(H[i]) else -1)
    return H, tok


class SamplerPool:
    """The oracle's sampler over row blocks on a pool of worker processes (the oracle is plain
    Python per row, so threads would serialise on the interpreter lock).  The workers are
    fresh interpreters, started before any timing; a worker that fails raises here (the
    executor reports a broken pool) instead of being restarted."""

    def __init__(self, workers):
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        self.workers = workers
        self.pool = ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
        warm = [(np.zeros((1, 8), np.float32), [0], 1.0, 0, 0)] * workers
        list(self.pool.map(_sample_block, warm, timeout=300))

    def sample_rows(self, logits, temperature, seed, step):
        P = logits.shape[0]
        blocks = [b for b in np.array_split(np.arange(P), self.workers) if b.size]
        parts = list(self.pool.map(_sample_block, [(logits[b], b, temperature, seed, step)
                                                   for b in blocks], timeout=600))
        H = np.concatenate([h for h, _ in parts])
        tok = np.concatenate([t for _, t in parts])
        return H, tok

    def close(self):
        self.pool.shutdown(wait=True)


def cpu_baseline(shape, x, layer_inputs, logits, sampler_shape):
    """The oracle, untuned, on a bounded sample of the same workload: whole MoE layers of the
    stack (every token, every routed expert; ``layer_inputs`` = [(router, weights), ...]) and
    whole sampler steps (every row), on every core of the host share."""
    from threadpoolctl import threadpool_limits
    from oracle import moe as omoe
    from block_diffusion_lm_router_amd import workloads
    threads = host_cores()
    pool = SamplerPool(threads)
    gu, dn = workloads.expert_bytes(shape)
    T = shape.tokens
    P = logits.shape[0]
    ffn_bytes = 0
    touched = []
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        for router, w in layer_inputs:
            ids, tw = omoe.route_topk(router, shape.top_k)
            o = omoe.moe_expert_outputs(x, ids, w)
            omoe.combine(o, tw)
            touched.append(len(np.unique(ids)))
            ffn_bytes += (touched[-1] * (gu + dn) + 2 * T * shape.d_model * 2
                          + T * shape.experts * 4 + 2 * T * shape.top_k * 4)
        t1 = time.perf_counter()
        for step in range(BASELINE_STEPS):
            pool.sample_rows(logits, sampler_shape.temperature, sampler_shape.seed, step)
        t2 = time.perf_counter()
    pool.close()
    samp_bytes = BASELINE_STEPS * (P * sampler_shape.vocab * 4 + P * 4 * 4)
    secs = t2 - t0
    return {
        "value": round((ffn_bytes + samp_bytes) / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle: {len(layer_inputs)} whole MoE layers of the stack ({T} "
                   f"tokens, {touched} experts touched, {ffn_bytes / 1e6:.1f} MB) in "
                   f"{t1 - t0:.2f} s, then {BASELINE_STEPS} sampler steps (entropy + two-level "
                   f"gumbel draw) over all {P} rows ({samp_bytes / 1e6:.1f} MB) in "
                   f"{t2 - t1:.2f} s on {threads} cores (BLAS threads for the layers, worker "
                   f"processes over row blocks for the sampler); rate = algorithmic bytes / wall time, same byte "
                   f"accounting as the GPU figure"),
    }


def components(bd, workloads, layers, x, logits, sshape, ws, sws, n=50):
    """Live timings of the path's parts beside the step: n calls back to back between one
    event pair on the launch stream (an event between calls would leave the GPU idle for
    several microseconds around it), inputs alternating between two copies (or two layers) so
    the 256 MB last-level cache cannot serve a repeat; the mean time per call.

    * ffn_layer_uniform: one whole FFN layer (route, gate/up, down, combine) at the 256-token
      canvas with uniform N(0, 1) router logits (every expert touched);
    * ffn_layer_short_zipf: the same at a 64-token canvas with Zipf(1.2) routing (about 100 of
      the 128 experts touched, most with a handful of tokens: the latency-bound case);
    * sampler_entropy_bound / sampler_confidence: one sampler step over all rows unfrozen;
    * rmsnorm / router: the layer neighbours at the same shape;
    * combine / combine_rmsnorm: the fixed-order combine alone, and with the next layer's RMS
      norm in the same launch (the chain workload's form);
    * canvas_init / loop_update: the denoising-loop driver's two launches at the canvas size.
    """
    import torch
    from block_diffusion_lm_router_amd import _binding  # noqa: F401
    stream = torch.cuda.current_stream()
    shape = workloads.LAYER
    T, d, f, E, k = shape.tokens, shape.d_model, shape.d_ff, shape.experts, shape.top_k
    gu_b, dn_b = workloads.expert_bytes(shape)
    P, V = logits.shape
    out = {}

    def timed(name, fns, alg_bytes):
        for i in range(4):
            fns[i % len(fns)]()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fns[i % len(fns)]()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / n
        gbs = alg_bytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "calls": n, "alg_bytes": int(alg_bytes),
                     "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}

    router = torch.from_numpy(workloads.make_router_logits(shape)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    o = torch.empty((T, k, d), dtype=torch.float32, device="cuda")
    y = torch.empty((T, d), dtype=torch.float16, device="cuda")
    bd.moe_route_topk(layers[0][0], router, ids, tw, ws)
    touched = int(torch.unique(ids).numel())

    def layer_fn(w):
        launches = (bd.bind(bd.moe_route_topk, w, router, ids, tw, ws),
                    bd.bind(bd.moe_w4a16_gate_up, w, x, ws),
                    bd.bind(bd.moe_w4a16_down, w, T, o, ws),
                    bd.bind(bd.moe_combine_fixed_order, o, tw, y))
        return lambda: [fn() for fn in launches]

    timed("ffn_layer_uniform", [layer_fn(layers[0][0]), layer_fn(layers[1 % len(layers)][0])],
          touched * (gu_b + dn_b) + 2 * T * d * 2 + T * E * 4 + 2 * T * k * 4)
    out["ffn_layer_uniform"]["experts_touched"] = touched

    short = workloads.SHORT_LAYER
    Ts = short.tokens
    xs = x[:Ts]
    ids_s = torch.empty((Ts, k), dtype=torch.int32, device="cuda")
    tw_s = torch.empty((Ts, k), dtype=torch.float32, device="cuda")
    o_s = torch.empty((Ts, k, d), dtype=torch.float32, device="cuda")
    y_s = torch.empty((Ts, d), dtype=torch.float16, device="cuda")
    short_fns, touched_s = [], []
    for li in range(2):
        w = layers[li % len(layers)][0]
        r = torch.from_numpy(workloads.make_router_logits(short, li)).cuda()
        bd.moe_route_topk(w, r, ids_s, tw_s, ws)
        touched_s.append(int(torch.unique(ids_s).numel()))
        launches = (bd.bind(bd.moe_route_topk, w, r, ids_s, tw_s, ws),
                    bd.bind(bd.moe_w4a16_gate_up, w, xs, ws),
                    bd.bind(bd.moe_w4a16_down, w, Ts, o_s, ws),
                    bd.bind(bd.moe_combine_fixed_order, o_s, tw_s, y_s))
        short_fns.append(lambda launches=launches: [fn() for fn in launches])
    timed("ffn_layer_short_zipf", short_fns,
          float(np.mean(touched_s)) * (gu_b + dn_b) + 2 * Ts * d * 2 + Ts * E * 4 + 2 * Ts * k * 4)
    out["ffn_layer_short_zipf"]["experts_touched"] = touched_s

    logits2 = logits.clone()
    frozen = torch.zeros(P, dtype=torch.uint8, device="cuda")
    canvas = torch.zeros(P, dtype=torch.int32, device="cuda")
    # The sampler steps run with every row unfrozen and no frozen set or canvas recorded (as
    # in the sampler workload), so that every call does the same work.
    tok = torch.empty(P, dtype=torch.int32, device="cuda")
    H = torch.empty(P, dtype=torch.float32, device="cuda")
    acc = torch.empty(P, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    samp_bytes = P * V * 4 + P * (4 + 4 + 1) + 4
    timed("sampler_entropy_bound",
          [bd.bind(bd.diffusion_sample_step, lg, sshape.temperature, sshape.bound, sshape.seed, 0,
                   None, None, tok, H, acc, cnt, sws) for lg in (logits, logits2)],
          samp_bytes)
    timed("sampler_confidence",
          [bd.bind(bd.diffusion_sample_step_confidence, lg, sshape.temperature, 0.9, sshape.seed,
                   0, None, None, tok, H, acc, cnt, sws) for lg in (logits, logits2)],
          samp_bytes)
    del logits2

    h_np, wn_np, wr_np = workloads.make_norm_router(shape)
    hs = [torch.from_numpy(h_np).cuda() for _ in range(2)]
    wn = torch.from_numpy(wn_np).cuda()
    wr = torch.from_numpy(wr_np).cuda()
    xn = torch.empty((T, d), dtype=torch.float16, device="cuda")
    rl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    timed("rmsnorm", [bd.bind(bd.moe_rmsnorm, hh, wn, xn) for hh in hs], 2 * T * d * 2 + d * 2)
    timed("router", [bd.bind(bd.moe_router_logits, xn, wr, rl)], T * d * 2 + E * d * 2 + T * E * 4)
    o2 = o.clone()
    timed("combine", [bd.bind(bd.moe_combine_fixed_order, oo, tw, y) for oo in (o, o2)],
          T * k * d * 4 + T * k * 4 + T * d * 2)
    timed("combine_rmsnorm", [bd.bind(bd.moe_combine_rmsnorm, oo, tw, wn, y, xn) for oo in (o, o2)],
          T * k * d * 4 + T * k * 4 + 2 * T * d * 2 + d * 2)
    del o2

    prev = torch.empty(P, dtype=torch.int32, device="cuda")
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    timed("canvas_init", [bd.bind(bd.diffusion_canvas_init, canvas, prev, frozen, state, V, 0, 0)],
          P * (4 + 4 + 1) + 16)
    # a block that never ends inside the timed calls (threshold and budget out of reach)
    frozen.zero_()
    timed("loop_update", [bd.bind(bd.diffusion_loop_update, tok, canvas, prev, frozen, state,
                                  1 << 30, 1 << 30)], P * (4 + 4 + 4 + 4 + 1) + 32)
    return out


GU_LAUNCHES = 60
# Consecutive unchanged steps that end a block early.  The pages name the option but give no
# default; at temperature 1 with step-keyed noise the drafts change at every step, so the
# stack's blocks run the whole step budget whatever the value.
LOOP_STABILITY = 2


def gate_up_back_to_back(bd, weights, routers, x, ids, tw):
    """Average duration (us) of one gate/up launch, from a pass right after the timed region in
    which GU_LAUNCHES launches cycle back to back through the given layers, bracketed by one
    event pair.  Each layer is routed once into a workspace of its own first.  A timing
    event inside a stream of launches leaves the GPU idle for several microseconds before and
    after the next launch (the trace shows none between unmarked launches), so events around
    single launches inside the step would measure that idle time as well; spread over the
    whole pass it is a fraction of a microsecond per launch."""
    import torch
    T = x.shape[0]
    wss = [bd.moe_workspace(T, w) for w in weights]
    for w, r, ws in zip(weights, routers, wss):
        bd.moe_route_topk(w, r, ids, tw, ws)
    runs = [bd.bind(bd.moe_w4a16_gate_up, w, x, ws) for w, ws in zip(weights, wss)]
    for fn in runs:
        fn()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(GU_LAUNCHES):
        runs[i % len(runs)]()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / GU_LAUNCHES


def read_ceiling(rate_gbs):
    """The achievable HBM read rate, measured now with the library's streaming-read probe (two
    1 GiB buffers in turn, together larger than the last-level cache), and rate_gbs as a
    fraction of it."""
    from block_diffusion_lm_router_amd import hbm_probe
    log("measuring the HBM read ceiling")
    gbs = hbm_probe.read_rate(1 << 30, 10, verify=False)["read_gbs"]
    return {"GB/s": gbs, "frac": round(rate_gbs / gbs, 4),
            "probe": "bd_hbm_read, 2 x 1 GiB buffers in turn, 10 launches"}


def timed_loop(fn, steps, warmup):
    """ms per call of fn over `steps` calls after `warmup`, bracketed by synchronisation."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(warmup, warmup + steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _round(v, n):
    return None if v is None else round(v, n)


def base_record(args, value, ms, workload, extra_config):
    cfg = {"workload": workload}
    cfg.update(extra_config)
    cfg["hbm_frac_of_peak"] = round(value / HBM_PEAK_GBS, 4)
    return {
        "metric": "denoising-step MoE+sampler latency (ms) and achieved HBM GB/s vs peak, 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16-mfma/f32", "data": "synthetic",
        "config": cfg,
    }


def main_layer(args):
    """One FFN layer at the 256-token canvas, uniform routing; roofline of the gate/up launch."""
    import torch
    from block_diffusion_lm_router_amd import _binding as bd, workloads
    torch.cuda.set_device(0)
    shape = workloads.LAYER
    T, d, f, E, k = shape.tokens, shape.d_model, shape.d_ff, shape.experts, shape.top_k
    # --checkpoint-format: gate/up grouped at 128, down at 64 (the model card's checkpoint)
    groups = dict(gate_up_group=128, down_group=64) if args.checkpoint_format else {}
    gu_b, dn_b = workloads.expert_bytes(shape, **groups)
    x_np = workloads.make_activations(shape)
    r_np = workloads.make_router_logits(shape)
    x, router = torch.from_numpy(x_np).cuda(), torch.from_numpy(r_np).cuda()
    w0_np = workloads.make_weights(shape, 0, **groups)
    layers = [bd.MoeWeights.from_numpy(w0_np, k, prepare=True, drop_raw=True),
              bd.MoeWeights.from_numpy(workloads.make_weights(shape, 1, **groups), k,
                                       prepare=True, drop_raw=True)]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    o = torch.empty((T, k, d), dtype=torch.float32, device="cuda")
    y = torch.empty((T, d), dtype=torch.float16, device="cuda")
    ws = bd.moe_workspace(T, layers[0])
    bd.moe_route_topk(layers[0], router, ids, tw, ws)
    touched = int(torch.unique(ids).numel())
    launches = [(bd.bind(bd.moe_route_topk, w, router, ids, tw, ws),
                 bd.bind(bd.moe_w4a16_gate_up, w, x, ws),
                 bd.bind(bd.moe_w4a16_down, w, T, o, ws),
                 bd.bind(bd.moe_combine_fixed_order, o, tw, y)) for w in layers]

    def step(i):
        for fn in launches[i % 2]:
            fn()

    log(f"timing {args.steps} layer passes")
    ms = timed_loop(step, args.steps, args.warmup)
    alg = touched * (gu_b + dn_b) + 2 * T * d * 2 + T * E * 4 + 2 * T * k * 4
    value = alg / (ms * 1e-3) / 1e9
    # the gate/up launch alone: the two layers' launches back to back, one event pair around
    # the pass (the router logits are the same for both layers in this workload)
    gu_us = gate_up_back_to_back(bd, layers, [router, router], x, ids, tw)
    gu_alg = touched * gu_b + T * d * 2 + T * k * f * 2
    gu_gbs = gu_alg / (gu_us * 1e-6) / 1e9
    rec = base_record(args, value, ms,
                      f"layer: one MoE FFN layer (canvas {T}, d_model {d}, expert ffn {f}, {E} experts "
                      f"top-{k}, W4A16 asym "
                      + ("gate/up g128 down g64 (checkpoint format)" if args.checkpoint_format
                         else "g64")
                      + f", uniform N(0,1) router logits), route + gate/up + down + combine",
                      {"experts_touched": touched, "step_algorithmic_bytes": int(alg)})
    rec["roofline"] = {"kernel": "moe_w4a16_gate_up (w4a16_packed_kernel<true, 22, false>)", "bound": "hbm",
                       "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                       "avg_launch_us": round(gu_us, 2), "alg_bytes_per_launch": int(gu_alg),
                       "read_ceiling": read_ceiling(gu_gbs)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        from threadpoolctl import threadpool_limits
        from oracle import moe as omoe
        threads = host_cores()
        secs = 0.0
        with threadpool_limits(limits=threads):
            for l in range(BASELINE_LAYERS):
                w_np = w0_np if l == 0 else workloads.make_weights(shape, l, **groups)
                t0 = time.perf_counter()
                omoe.moe_ffn(x_np, r_np, w_np, k)
                secs += time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(BASELINE_LAYERS * alg / secs / 1e9, 4), "unit": "GB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"numpy fp64 oracle: {BASELINE_LAYERS} whole layers ({T} "
                                         f"tokens, {touched} experts each) in {secs:.2f} s "
                                         f"(weight generation not timed); same byte accounting"}
    print(json.dumps(rec), flush=True)


def main_sampler(args):
    """The sampler step alone on [256, 262144] fp32 logits; roofline of the whole call."""
    import torch
    from block_diffusion_lm_router_amd import _binding as bd, workloads
    torch.cuda.set_device(0)
    sshape = workloads.SAMPLER
    P, V = sshape.positions, sshape.vocab
    lg_np = workloads.make_logits(sshape)
    lgs = [torch.from_numpy(lg_np).cuda() for _ in range(2)]
    tok = torch.empty(P, dtype=torch.int32, device="cuda")
    H = torch.empty(P, dtype=torch.float32, device="cuda")
    acc = torch.empty(P, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    sws = bd.sample_workspace(P, V)
    calls = [[bd.bind(bd.diffusion_sample_step, lg, sshape.temperature, sshape.bound, sshape.seed,
                      s, None, None, tok, H, acc, cnt, sws) for lg in lgs] for s in range(2)]

    def step(i):
        calls[(i // 2) % 2][i % 2]()

    # One sampler step is about 55 us, so W warmup steps alone are a few milliseconds: the first
    # timed region after process start then runs about 10 % slow while the device ramps up. The
    # same step is run for a fixed 250 ms of wall time first (reported in the config).
    ramp_calls, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 0.25:
        for _ in range(64):
            step(ramp_calls)
            ramp_calls += 1
        torch.cuda.synchronize()
    log(f"timing {args.steps} sampler steps ({ramp_calls} ramp-up calls first)")
    ms = timed_loop(step, args.steps, args.warmup)
    alg = P * V * 4 + P * (4 + 4 + 1) + 4
    value = alg / (ms * 1e-3) / 1e9
    # The roofline's unit is the whole call (its three launches): its average duration is the
    # timed region's, where the calls run back to back between one event pair.
    us = ms * 1e3
    gbs = alg / (us * 1e-6) / 1e9
    rec = base_record(args, value, ms,
                      f"sampler: fp32 logits [{P}, {V}] (N(0,1) + one entry boosted U[0,12]), "
                      f"entropy + two-level gumbel-max at T=1, entropy-bound acceptance at 2.0, "
                      f"every row unfrozen", {"step_algorithmic_bytes": int(alg),
                                                     "device_rampup_calls": ramp_calls})
    rec["roofline"] = {"kernel": "diffusion_sample_step (sample_stream_kernel + sample_finish_kernel "
                                 "+ accept_kernel)", "bound": "hbm", "achieved": round(gbs, 2),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "traffic": None, "avg_launch_us": round(us, 2), "alg_bytes_per_launch": int(alg),
                       "read_ceiling": read_ceiling(gbs)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        from oracle import sampler as osamp
        n_steps = 10
        threads = host_cores()
        pool = SamplerPool(threads)
        t0 = time.perf_counter()
        for st in range(n_steps):
            H_ref, _ = pool.sample_rows(lg_np, sshape.temperature, sshape.seed, st)
            osamp.accept(H_ref.astype(np.float32), sshape.bound)
        secs = time.perf_counter() - t0
        pool.close()
        rec["cpu_baseline"] = {"value": round(n_steps * alg / secs / 1e9, 4), "unit": "GB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"numpy fp64 oracle: {n_steps} whole sampler steps over all "
                                         f"{P} rows in {secs:.2f} s (rows split over {threads} "
                                         f"worker processes); same byte accounting"}
    print(json.dumps(rec), flush=True)


def main_chain(args):
    """The denoising loop with the layers chained on the device: in every step, layer l takes
    the RMS norm of the running hidden state, projects it onto the router, routes it (top-k
    and bucketing), runs the W4A16 FFN and combines; the combined output is layer l + 1's
    hidden state, and its RMS norm is taken by the same launch as the combine
    (moe_combine_rmsnorm; layer 0 normalises the initial hidden state on its own).  Then the sampler step and the loop update, as in the stack; a block of 48
    steps is one captured graph whose launches carry the done gate.  The routing is the
    router's own (data-dependent) instead of given Zipf(1.2) logits."""
    import torch
    from block_diffusion_lm_router_amd import _binding as bd, workloads
    torch.cuda.set_device(0)
    shape = workloads.STACK_LAYER
    n_layers = args.layers or workloads.STACK_LAYERS
    sshape = workloads.SAMPLER
    T, d, f, E, k = shape.tokens, shape.d_model, shape.d_ff, shape.experts, shape.top_k
    P, V = sshape.positions, sshape.vocab
    gu_bytes, dn_bytes = workloads.expert_bytes(shape)
    log(f"generating {n_layers} chained layers")
    h0_np, _, _ = workloads.make_norm_router(shape)
    layers = []
    for l in range(n_layers):
        _, wn_np, wr_np = workloads.make_norm_router(shape, l)
        layers.append((bd.MoeWeights.from_numpy(workloads.make_weights(shape, l), k, prepare=True,
                                                drop_raw=True),
                       torch.from_numpy(wn_np).cuda(), torch.from_numpy(wr_np).cuda()))
    logits = torch.from_numpy(workloads.make_logits(sshape)).cuda()
    h0 = torch.from_numpy(h0_np).cuda()
    hs = [torch.empty((T, d), dtype=torch.float16, device="cuda") for _ in range(2)]
    xn = torch.empty((T, d), dtype=torch.float16, device="cuda")
    rl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    o = torch.empty((T, k, d), dtype=torch.float32, device="cuda")
    ws = bd.moe_workspace(T, layers[0][0])
    sws = bd.sample_workspace(P, V)
    frozen = torch.zeros(P, dtype=torch.uint8, device="cuda")
    canvas = torch.zeros(P, dtype=torch.int32, device="cuda")
    prev = torch.empty(P, dtype=torch.int32, device="cuda")
    tok = torch.empty(P, dtype=torch.int32, device="cuda")
    H = torch.empty(P, dtype=torch.float32, device="cuda")
    acc = torch.empty(P, dtype=torch.uint8, device="cuda")
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    STEPS = workloads.STACK_STEPS
    n_acc = torch.zeros(STEPS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def layer_chain(gate):
        bd.moe_rmsnorm(h0, layers[0][1], xn, loop_state=gate)
        for l, (w, wn, wr) in enumerate(layers):
            bd.moe_router_logits(xn, wr, rl, loop_state=gate)
            bd.moe_w4a16_ffn(w, xn, rl, ids, tw, o, ws, loop_state=gate)
            if l + 1 < len(layers):
                bd.moe_combine_rmsnorm(o, tw, layers[l + 1][1], hs[l % 2], xn, loop_state=gate)
            else:
                bd.moe_combine_fixed_order(o, tw, hs[l % 2], loop_state=gate)

    # Experts each layer touches (the routing is the same in every step: every step starts
    # from the same hidden state), from one eager pass of the chain.
    touched = []
    bd.moe_rmsnorm(h0, layers[0][1], xn)
    for l, (w, wn, wr) in enumerate(layers):
        bd.moe_router_logits(xn, wr, rl)
        bd.moe_w4a16_ffn(w, xn, rl, ids, tw, o, ws)
        if l + 1 < len(layers):
            bd.moe_combine_rmsnorm(o, tw, layers[l + 1][1], hs[l % 2], xn)
        else:
            bd.moe_combine_fixed_order(o, tw, hs[l % 2])
        touched.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()

    def capture(n_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            bd.diffusion_canvas_init(canvas, prev, frozen, state, V, sshape.seed, 0)
            for s in range(n_steps):
                layer_chain(state)
                bd.diffusion_sample_step(logits, sshape.temperature, sshape.bound, sshape.seed, s,
                                         frozen, canvas, tok, H, acc, n_acc[s:s + 1], sws,
                                         loop_state=state)
                bd.diffusion_loop_update(tok, canvas, prev, frozen, state, LOOP_STABILITY, STEPS)
        return g

    log(f"capturing the chained block graph ({STEPS} steps, {n_layers} layers each)")
    graphs = {STEPS: capture(STEPS)}
    for n in {args.steps % STEPS, args.warmup % STEPS} - {0}:
        graphs[n] = capture(n)

    def run_steps(n):
        for _ in range(n // STEPS):
            graphs[STEPS].replay()
        if n % STEPS:
            graphs[n % STEPS].replay()

    run_steps(max(args.warmup, 1))
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    run_steps(args.steps)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    counts = n_acc.cpu().numpy()
    steps_run = int(state.cpu().numpy()[0])
    unfrozen = np.array([P - int(counts[:s].sum()) for s in range(STEPS)], dtype=np.float64)
    live = np.arange(STEPS) < steps_run
    # Per layer: the FFN's bytes as in the stack, plus the norm (normed rows out and the
    # weight; layer 0 also reads the hidden state in, later layers take it from the combine's
    # registers) and the router projection (normed rows, router matrix, logits out).
    layer_bytes = sum(t * (gu_bytes + dn_bytes) for t in touched) + n_layers * (
        2 * T * d * 2 + T * E * 4 + 2 * T * k * 4) + T * d * 2 + n_layers * (
        T * d * 2 + d * 2 + T * d * 2 + E * d * 2 + T * E * 4)
    step_bytes_blk = np.where(live, layer_bytes + unfrozen * V * 4 + P * 4 * 4, 0.0)
    timed_steps = [i % STEPS for i in range((args.steps // STEPS) * STEPS)] + list(
        range(args.steps % STEPS))
    step_bytes = float(np.mean(step_bytes_blk[timed_steps]))
    value = step_bytes / (ms * 1e-3) / 1e9
    rec = base_record(
        args, value, ms,
        (f"chain: the denoising loop, each step {n_layers} chained MoE layers (canvas {T}, "
         f"d_model {d}, expert ffn {f}, {E} experts top-{k}, W4A16 asym g64; per layer RMS "
         f"norm, router projection, routing, FFN, combine, the output feeding the next layer; "
         f"each combine and the next layer's norm in one launch) "
         f"+ sampler fp32 [{P}, {V}] T=1 bound 2.0 + loop update; blocks of {STEPS} steps, "
         f"each one captured graph with the done gate"),
        {"steps_per_block": STEPS, "block_steps_run": steps_run,
         "experts_touched_min_max": [min(touched), max(touched)],
         "step_algorithmic_bytes": int(step_bytes)})
    rec["roofline"] = {"kernel": "whole step (every launch of the chained step)", "bound": "hbm",
                       "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                       "avg_launch_us": round(ms * 1e3, 2), "alg_bytes_per_launch": int(step_bytes),
                       "read_ceiling": read_ceiling(value)}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 2:
        print("bench.py needs --steps >= 2 (the gate/up timing pairs consecutive steps).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "layer":
        return main_layer(args)
    if args.workload == "sampler":
        return main_sampler(args)
    if args.workload == "chain":
        return main_chain(args)
    import torch
    from block_diffusion_lm_router_amd import _binding as bd, workloads

    torch.cuda.set_device(0)
    shape = workloads.STACK_LAYER
    n_layers = args.layers or workloads.STACK_LAYERS
    sshape = workloads.SAMPLER
    T, d, f, E, k = shape.tokens, shape.d_model, shape.d_ff, shape.experts, shape.top_k
    P, V = sshape.positions, sshape.vocab
    gu_bytes, dn_bytes = workloads.expert_bytes(shape)

    log(f"generating {n_layers} layers of packed weights")
    t0 = time.time()
    x_np = workloads.make_activations(shape)
    x = torch.from_numpy(x_np).cuda()
    layers = []
    baseline_layers = []
    for l in range(n_layers):
        w_np = workloads.make_weights(shape, l)
        r_np = workloads.make_router_logits(shape, l)
        layers.append((bd.MoeWeights.from_numpy(w_np, k, prepare=True, drop_raw=True),
                       torch.from_numpy(r_np).cuda()))
        if l < BASELINE_LAYERS and not args.no_cpu_baseline:
            baseline_layers.append((r_np, w_np))
        del w_np
    logits_np = workloads.make_logits(sshape)
    logits = torch.from_numpy(logits_np).cuda()
    log(f"inputs resident in HBM ({time.time() - t0:.1f} s)")

    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    o = torch.empty((T, k, d), dtype=torch.float32, device="cuda")
    y = torch.empty((T, d), dtype=torch.float16, device="cuda")
    ws = bd.moe_workspace(T, layers[0][0])
    # Experts each layer touches, from the device's own routing (for the byte accounting).
    touched = []
    for w, router in layers:
        bd.moe_route_topk(w, router, ids, tw, ws)
        touched.append(int(torch.unique(ids).numel()))
    sws = bd.sample_workspace(P, V)
    frozen = torch.zeros(P, dtype=torch.uint8, device="cuda")
    canvas = torch.zeros(P, dtype=torch.int32, device="cuda")
    tok = torch.empty(P, dtype=torch.int32, device="cuda")
    H = torch.empty(P, dtype=torch.float32, device="cuda")
    acc = torch.empty(P, dtype=torch.uint8, device="cuda")
    # The denoising loop on the device.  A block is one captured graph: the random initial
    # canvas (which also clears the frozen set and the driver state), then STACK_STEPS steps
    # of 30 layers (route, gate/up, down, combine) and the sampler step, each followed by the
    # loop driver's update; every launch but the update carries the driver state as its done
    # gate, so the steps after the block ends do no work.  K timed steps replay whole blocks
    # and, when K is not a multiple of STACK_STEPS, a graph of the first K mod STACK_STEPS
    # steps of a block.
    STEPS = workloads.STACK_STEPS
    prev = torch.empty(P, dtype=torch.int32, device="cuda")
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    n_acc = torch.zeros(STEPS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def issue(n_steps):
        """Enqueue the first n_steps steps of a block: the initial canvas, then per step the
        gated layers, the gated sampler and the loop driver's update."""
        bd.diffusion_canvas_init(canvas, prev, frozen, state, V, sshape.seed, 0)
        for s in range(n_steps):
            for w, router in layers:
                bd.moe_w4a16_ffn(w, x, router, ids, tw, o, ws, loop_state=state)
                bd.moe_combine_fixed_order(o, tw, y, loop_state=state)
            bd.diffusion_sample_step(logits, sshape.temperature, sshape.bound, sshape.seed, s,
                                     frozen, canvas, tok, H, acc, n_acc[s:s + 1], sws,
                                     loop_state=state)
            bd.diffusion_loop_update(tok, canvas, prev, frozen, state, LOOP_STABILITY, STEPS)

    def capture(n_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            issue(n_steps)
        return g

    class Eager:
        """Stands in for a block graph under --no-graph: replay() issues the launches."""

        def __init__(self, n_steps):
            self.n_steps = n_steps

        def replay(self):
            issue(self.n_steps)

    def graph_passes():
        """The timed block replays and the block-time spread; returns (ms per step, GB/s,
        steps a block ran, per-step ms of each block replay, bytes per timed step)."""
        make = Eager if args.no_graph else capture
        log(f"{'preparing eager blocks' if args.no_graph else 'capturing the block graph'} "
            f"({STEPS} steps, {n_layers} layers each)")
        graphs = {STEPS: make(STEPS)}
        for n in {args.steps % STEPS, args.warmup % STEPS} - {0}:
            graphs[n] = make(n)

        def run_steps(n):
            """Replay graphs covering n steps (whole blocks, then a partial block)."""
            for _ in range(n // STEPS):
                graphs[STEPS].replay()
            if n % STEPS:
                graphs[n % STEPS].replay()

        # Warm-up (untimed), then the timed steps between one event pair.
        run_steps(max(args.warmup, 1))
        torch.cuda.synchronize()
        log(f"warmup done; timing {args.steps} steps")
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        run_steps(args.steps)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps

        # Work done per block (every replay of a block graph does the same work): the steps
        # the block ran before it ended, and the rows each step's sampler read (unfrozen rows,
        # from the device's acceptance counts).
        counts = n_acc.cpu().numpy()
        steps_run = int(state.cpu().numpy()[0])
        unfrozen = np.array([P - int(counts[:s].sum()) for s in range(STEPS)], dtype=np.float64)
        live = np.arange(STEPS) < steps_run
        layer_bytes = sum(t * (gu_bytes + dn_bytes) for t in touched) + n_layers * (
            2 * T * d * 2 + T * E * 4 + 2 * T * k * 4)
        step_bytes_blk = np.where(live, layer_bytes + unfrozen * V * 4 + P * 4 * 4, 0.0)
        timed_steps = [i % STEPS for i in range((args.steps // STEPS) * STEPS)] + list(
            range(args.steps % STEPS))
        step_bytes = float(np.mean(step_bytes_blk[timed_steps]))
        value = step_bytes / (ms * 1e-3) / 1e9

        # A second pass: block replays with an event between consecutive blocks, the spread of
        # the block time (per step).
        n_blocks = max(3, args.steps // STEPS)
        blk_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_blocks + 1)]
        blk_ev[0].record(stream)
        for b in range(n_blocks):
            graphs[STEPS].replay()
            blk_ev[b + 1].record(stream)
        torch.cuda.synchronize()
        per_step = np.array([a.elapsed_time(b) for a, b in zip(blk_ev[:-1], blk_ev[1:])]) / STEPS
        return ms, value, steps_run, per_step, step_bytes

    if args.eager_only:
        ms = value = steps_run = per_step = step_bytes = None
    else:
        ms, value, steps_run, per_step, step_bytes = graph_passes()

    # A third pass, eager launches: the gate/up kernel's in-step duration by difference.  Step j
    # of this pass brackets with one event pair the routing and gate/up launches of layer
    # (j // 2) mod L when j is odd and the routing launch alone of the same layer when j is
    # even.  A timing event leaves the GPU idle for several microseconds around the launches
    # next to it (the trace shows no gap between unmarked launches), the same in both
    # brackets, so the median of the odd intervals minus the median of the even ones is the
    # gate/up launch as it runs inside the step.  The pass runs at least 2 L steps, so every
    # layer is bracketed both ways whatever --steps is, after one unmarked step (the first
    # interval after the switch from graph replays to eager launches carries a start-up delay
    # of tens of microseconds, which the medians would also reject).
    n_eager = max(args.steps + args.steps % 2, 2 * len(layers))
    stack = []
    for w, router in layers:
        stack.append((bd.bind(bd.moe_route_topk, w, router, ids, tw, ws),
                      bd.bind(bd.moe_w4a16_gate_up, w, x, ws),
                      bd.bind(bd.moe_w4a16_down, w, T, o, ws),
                      bd.bind(bd.moe_combine_fixed_order, o, tw, y)))
    marks = [((j // 2) % len(layers), j % 2 == 1,
              (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
             for j in range(n_eager)]
    frozen.zero_()
    for route, gate_up, down, combine in stack:   # one unmarked step first
        route()
        gate_up()
        down()
        combine()
    for j, (mli, with_gu, (a, b)) in enumerate(marks):
        for li, (route, gate_up, down, combine) in enumerate(stack):
            here = li == mli
            if here:
                a.record(stream)
            route()
            if here and not with_gu:
                b.record(stream)
            gate_up()
            if here and with_gu:
                b.record(stream)
            down()
            combine()
        bd.diffusion_sample_step(logits, sshape.temperature, sshape.bound, sshape.seed,
                                 j % STEPS, frozen, canvas, tok, H, acc, n_acc[0:1], sws)
    torch.cuda.synchronize()

    with_gu = [a.elapsed_time(b) for _, g, (a, b) in marks if g]
    route_only = [a.elapsed_time(b) for _, g, (a, b) in marks if not g]
    gu_us = (float(np.median(with_gu)) - float(np.median(route_only))) * 1e3
    gu_alg = float(np.mean([touched[li] * gu_bytes + T * d * 2 + T * k * f * 2
                            for li, g, _ in marks if g]))
    gu_gbs = gu_alg / (gu_us * 1e-6) / 1e9
    traffic = measured_traffic(gu_alg)
    parts = None
    if not args.no_components:
        log("timing the parts one launch at a time")
        parts = components(bd, workloads, layers, x, logits, sshape, ws, sws)

    result = {
        "metric": "denoising-step MoE+sampler latency (ms) and achieved HBM GB/s vs peak, 1 GPU",
        "value": _round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": _round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic",
        "config": {
            "workload": (f"stack: the denoising loop, each step {n_layers} MoE layers (canvas "
                         f"{T}, d_model {d}, expert ffn {f}, {E} experts top-{k}, W4A16 asym "
                         f"g64, Zipf(1.2) routing) + sampler fp32 [{P}, {V}] T=1 bound 2.0 + "
                         f"loop update; blocks of {STEPS} steps from a random canvas, each "
                         + ("block's launches issued eagerly (--no-graph) with the done gate"
                            if args.no_graph else
                            "block one captured graph with the done gate")),
            "steps_per_block": STEPS,
            "block_steps_run": steps_run,
            "stability_threshold": LOOP_STABILITY,
            "hbm_frac_of_peak": None if value is None else round(value / HBM_PEAK_GBS, 4),
            "step_ms_p10_p50_p90_over_blocks": (
                None if per_step is None else
                [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)]),
            "step_algorithmic_bytes": None if step_bytes is None else int(step_bytes),
            **({"eager_only": True} if args.eager_only else {}),
            **({"components": parts} if parts is not None else {}),
        },
        "roofline": {
            "kernel": "moe_w4a16_gate_up (w4a16_packed_kernel<true, 22, false>)",
            "bound": "hbm",
            "achieved": round(gu_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gu_us, 2),
            "intervals_each_way": n_eager // 2,
            "alg_bytes_per_launch": int(gu_alg),
            "read_ceiling": read_ceiling(gu_gbs),
        },
    }
    result["config"]["frac_of_read_ceiling"] = None if value is None else round(
        value / result["roofline"]["read_ceiling"]["GB/s"], 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(shape, x_np, baseline_layers, logits_np, sshape)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
