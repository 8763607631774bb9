#!/usr/bin/env python3
"""Bench of the W4A16 MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config long_prefill]

A step is one pass of the whole MoE layer (route -> permute -> expert up -> expert
down (+ the shared expert) -> combine+RMSNorm) over one batch of synthetic tokens,
inputs resident in HBM. The default workload is long prefill: 32768 tokens as 4
layer calls of 8192 (H=6144, 160 routed experts top-8 with Zipf(1.1) popularity,
plus one shared expert, I=2048), the largest configuration that fits one GPU; a
step is the 4 calls. ``--config`` selects another workload (tiny, decode_t1,
decode_t8, batched_t64, batched_t256, prefill). Weight copies are rotated so the
working set is at least 1 GiB, which keeps the 256 MB Infinity Cache from serving
the weights.

Timed passes:
  1. the headline: K steps of fused ``moe4_layer`` calls between two events on the
     launch stream (value = tokens / s, ms_per_step);
  2. the roofline: the dominant kernel (the routed expert "up" pass, W13 + SwiGLU)
     launched back to back on each chunk's plan, rotating weight copies, between two
     events on the launch stream; its algorithmic bytes (touched experts' packed
     weights + scales, activations in, h out) or flops divided by the mean launch
     duration give ``roofline.achieved``;
  3. the other expert-FFN launches of a layer call (routed down; shared up and down),
     timed the same way, reported under ``kernels`` with their sum (``ffn_total``);
  4. the other steps through their own entry points (route, permute, combine_norm),
     each call captured into a HIP graph and the graph replayed between the events (an
     eager loop of these short launches would time the host), reported under
     ``kernels`` with their algorithmic bytes.
The fp64 oracle is timed on the host (``cpu_baseline``) on a bounded sample of the
same tokens, one worker process per host core, before the GPU is touched.
Prints one JSON line.

``--op add_rmsnorm|group_rmsnorm`` times one of the neighbouring RMSNorm glue
launches instead (a step is one launch over the workload's T x H rows) and prints
its own line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s as % of peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
MALL_DEFEAT_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0 = about 2 s of GPU work)")
    ap.add_argument("--warmup", type=int, default=-1, help="untimed steps (-1 = steps / 10)")
    ap.add_argument("--config", default="long_prefill")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="oracle sample budget (per worker)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-stream", choices=["on", "off"], default="off",
                    help="routed chain on a side stream beside the shared expert (moe4_layer_side)")
    ap.add_argument("--op", choices=["layer", "add_rmsnorm", "group_rmsnorm"], default="layer",
                    help="what a step is: the MoE layer (default), or one of the neighbouring "
                         "RMSNorm glue launches over the workload's T x H rows")
    ap.add_argument("--group", type=int, default=0, help="group_rmsnorm group size (0 = H / 8)")
    ap.add_argument("--precision", choices=["w4a16", "w4a8"], default="w4a16",
                    help="expert FFN form: BF16 activations (the default), or the FP8 prefill "
                         "variant (moe4_layer_w4a8: block-scaled E4M3 activations, weights "
                         "rounded to E4M3, FP8 MFMA)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB twice with torch (a plain copy of known size, for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "bit_moe_expert_amd", "csrc")
# the source files each dominant kernel is built from
KERNEL_SOURCES = {
    "decode": [os.path.join(_CSRC, f) for f in ("ffn_decode.hip", "device.hpp")],
    "prefill": [os.path.join(_CSRC, f) for f in ("ffn_prefill.hip", "prefill_common.hpp", "device.hpp")],
    "prefill_fp8": [os.path.join(_CSRC, f) for f in ("ffn_prefill_fp8.hip", "prefill_common.hpp", "device.hpp")],
}


def source_sha(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config, kernel_sources):
    """HBM bytes per launch of the dominant kernel from a committed counter summary
    (``profiles/*_traffic.md``, its ``machine:`` line), if one was taken on this
    workload with the current kernel source; else None."""
    if not os.path.isdir(PROFILES):
        return None
    want = source_sha(kernel_sources)
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith("_traffic.md"):
            continue
        vals = {}
        for line in open(os.path.join(PROFILES, name)):
            if line.startswith("machine:"):
                for kv in line[len("machine:"):].split():
                    k, _, v = kv.partition("=")
                    vals[k] = v
        if vals.get("config") == config and vals.get("source_sha") == want:
            return int(vals["traffic_bytes"])
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ffn_work(w, T, idx, up, dense, fp8=False):
    """Algorithmic bytes and flops of one expert-FFN launch: the routed groups of the
    plan (dense False; ``idx`` the routing) or the shared expert over all T tokens.
    Bytes: the touched experts' packed codes + E4M3 scales + tensor scale, the
    activations read (x once per token for up; h rows for down), the outputs written,
    and the plan. With ``fp8`` the activations in (and h out of up) are E4M3 codes
    plus one scale byte per 32."""
    N, K = (2 * w.I, w.H) if up else (w.H, w.I)
    per_expert = N * K // 2 + N * K // 16 + 4
    if dense:
        rows, experts, plan = T, 1, 0
    else:
        rows = T * w.k
        experts = len(set(idx.reshape(-1).tolist()))
        plan = (w.E + 1) * 4 + (rows * 4 if up else 0)
    a = 1 + 1 / 32 if fp8 else 2
    act_in = int(T * w.H * a) if up else int(rows * w.I * a)
    out = int(rows * w.I * a) if up else rows * w.H * 2
    nbytes = experts * per_expert + act_in + out + plan
    flops = 2 * rows * N * K
    return nbytes, flops, experts


_CPU = {}


def _oracle_worker(wid, calls, budget_s):
    """One host core's share of the oracle baseline: layer calls on its own token
    subsets (tokens are independent) until the budget is spent."""
    from threadpoolctl import threadpool_limits

    import oracle
    inputs = _CPU["inputs"]
    fn = oracle.layer_w4a8 if _CPU["fp8"] else oracle.layer
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for chunk, tokens in calls:
            fn(inputs[chunk], tokens=tokens)
            done += len(tokens)
            if time.perf_counter() - t0 >= budget_s:
                break
    return done, time.perf_counter() - t0


def cpu_baseline(inputs, budget_s, fp8=False):
    """Time the oracle as it stands on all host cores: one worker process per core
    (forked before the GPU is initialised), each running oracle.layer (with ``fp8``
    oracle.layer_w4a8) on its own seeded subsets of the workload's tokens, BLAS one
    thread per worker."""
    import multiprocessing

    import numpy as np
    # the host cores this process may use: its affinity mask, capped by the thread
    # budget the environment sets for the job (OMP_NUM_THREADS) where it sets one
    cores = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = min(cores, cap) if cap > 0 else cores
    T, chunks = inputs[0].T, len(inputs)
    # tokens per oracle call: the whole batch split over the cores for small batches,
    # else two (a call dequantises every expert its tokens touch, seconds each)
    per_call = max(1, min(2, T // cores)) if T >= 2 * cores else max(1, -(-T // cores))
    rng = np.random.default_rng(7)
    perms = [rng.permutation(T) for _ in range(chunks)]
    cursor = [0] * chunks
    calls_per_worker = 64
    plans = []
    for w in range(cores):
        calls = []
        for i in range(calls_per_worker):
            c = (w + i) % chunks
            p = cursor[c]
            cursor[c] += per_call
            calls.append((c, np.unique(perms[c][np.arange(p, p + per_call) % T])))
        plans.append(calls)
    _CPU["inputs"] = inputs
    _CPU["fp8"] = fp8
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.starmap(_oracle_worker, [(w, plans[w], budget_s) for w in range(cores)])
    wall = time.perf_counter() - t0
    _CPU.clear()
    tokens = sum(r[0] for r in res)
    return {"value": tokens / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{tokens} token evaluations: seeded subsets of the {T * chunks}-token workload "
                      f"(all chunks, cycling), oracle {'layer_w4a8' if fp8 else 'layer'} calls of up to "
                      f"{per_call} tokens on {cores} "
                      f"worker processes (one per host core, BLAS 1 thread each), {wall:.1f} s wall"}


def glue_main(args):
    """One RMSNorm glue launch per step over the workload's T x H rows (x, residual and
    gamma drawn as for the layer); the launches run back to back between two events on
    the stream. Input copies are rotated so that at least 1 GiB is touched, up to 16
    copies: decode-sized rows then stay cache-resident, as they are after the previous
    kernel wrote them, instead of each launch paying for fresh pages."""
    # launches timed (0 = 2048: a short launch, a few ms in all) and untimed first
    args.steps = args.steps or 2048
    args.warmup = args.warmup if args.warmup >= 0 else 20
    import numpy as np
    import torch

    from bit_moe_expert_amd import binding as B
    from bit_moe_expert_amd import workloads as wl

    w = wl.workload(args.config)
    T, H = w.T * w.chunks, w.H
    G = args.group or H // 8
    rng = np.random.default_rng(0)
    x = wl.to_bf16_bits(rng.standard_normal((T, H)))
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).cuda()
    add = args.op == "add_rmsnorm"
    per_call = T * H * 2 * (4 if add else 2) + H * 2        # rows in and out, gamma
    copies = min(16, max(1, math.ceil(MALL_DEFEAT_BYTES / per_call)))
    bufs = []
    for _ in range(copies):
        bufs.append(dict(x=dev(x), r=dev(res) if add else None,
                         o=torch.empty((T, H), dtype=torch.int16, device="cuda") if add else None,
                         n=torch.empty((T, H), dtype=torch.int16, device="cuda")))
    d_g = dev(gam)

    def step(i):
        b = bufs[i % copies]
        if add:
            B.moe4_add_rmsnorm(b["x"], b["r"], d_g, b["o"], b["n"], eps=w.eps)
        else:
            B.moe4_group_rmsnorm(b["x"], G, d_g, b["n"], eps=w.eps)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_s = ev0.elapsed_time(ev1) / args.steps / 1e3
    ref_n = bufs[0]["n"].clone()
    # The same launches captured into a HIP graph and replayed: at decode sizes the eager
    # loop measures the host's launch rate, the replay the GPU's.
    per_graph = min(args.steps, 256)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(3):
            step(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            step(i)
    torch.cuda.synchronize()
    replays = max(1, args.steps // per_graph)
    graph.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(replays):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    if not torch.equal(bufs[0]["n"], ref_n):
        raise RuntimeError("graph replay output differs from the eager launch")
    mean_s = ev0.elapsed_time(ev1) / (replays * per_graph) / 1e3
    achieved = per_call / mean_s / 1e9
    log(f"{args.op}: {mean_s * 1e6:.2f} us per launch in graph replay ({eager_s * 1e6:.2f} us eager), "
        f"{achieved:.1f} GB/s, {copies} input copies")
    desc = f"group={G}" if not add else "o = x + residual"
    out = {"metric": f"{args.op} rows/s", "value": round(T / mean_s, 1), "unit": "rows/s", "n_gpus": 1,
           "steps": replays * per_graph, "warmup": args.warmup, "ms_per_step": round(mean_s * 1e3, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"{args.op} over {T} rows of H={H} BF16 ({desc}), rows of the "
                                  f"{args.config} workload; launches replayed from a HIP graph",
                      "T": T, "H": H, "group": G if not add else H, "input_copies_rotated": copies,
                      "eager_us_per_launch": round(eager_s * 1e6, 3)},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "rmsnorm_kernel", "mean_us": round(mean_s * 1e6, 3),
                        "algorithmic_bytes": per_call}}
    if not args.no_cpu_baseline:
        import oracle
        rows = min(T, 64)
        t0 = time.perf_counter()
        reps = 0
        while True:
            if add:
                oracle.add_rmsnorm(x[:rows], res[:rows], gam, w.eps)
            else:
                oracle.group_rmsnorm(x[:rows], G, gam, w.eps)
            reps += 1
            el = time.perf_counter() - t0
            if el > min(args.cpu_seconds, 5.0):
                break
        out["cpu_baseline"] = {"value": round(rows * reps / el, 1), "unit": "rows/s", "cores": 1,
                               "kind": "oracle", "sample": f"{rows} rows x {reps} repetitions"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (got --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    # counting devices does not initialise the GPU runtime (the oracle's worker
    # processes are forked before anything does)
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.op != "layer":
        torch.cuda.set_device(0)
        glue_main(args)
        return

    import numpy as np

    from bit_moe_expert_amd import binding as B
    from bit_moe_expert_amd import workloads as wl

    w = wl.workload(args.config)
    chunks = w.chunks
    log(f"generating inputs: {w}")
    t_gen = time.perf_counter()
    inputs = [wl.make_inputs(w, seed=0, chunk=0)]
    for c in range(1, chunks):
        inputs.append(wl.make_inputs(w, seed=0, chunk=c, weights_from=inputs[0]))
    inp = inputs[0]
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f} s")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on every host core for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(inputs, args.cpu_seconds, fp8=args.precision == "w4a8")
        log(f"cpu baseline: {cpu['value']:.2f} tokens/s on {cpu['cores']} cores")

    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    w13 = B.DeviceW4.from_host(inp.w13)
    w2 = B.DeviceW4.from_host(inp.w2)
    s13 = B.DeviceW4.from_host(inp.shared13) if inp.shared13 is not None else None
    s2 = B.DeviceW4.from_host(inp.shared2) if inp.shared2 is not None else None
    wr = dev(inp.w_router) if inp.w_router is not None else None
    wbytes = w13.nbytes + w2.nbytes
    copies = args.copies or max(1, math.ceil(MALL_DEFEAT_BYTES / wbytes))
    weights = [(w13, w2)] + [(w13.clone(), w2.clone()) for _ in range(copies - 1)]
    log(f"weights {wbytes / 1e6:.1f} MB x {copies} copies")

    T = inp.T
    shape = B.make_shape(T, w.H, w.E, w.k, w.I, w.n_shared, w.eps)
    per_chunk = []
    for ci in inputs:
        per_chunk.append(dict(
            x=dev(ci.x), residual=dev(ci.residual),
            logits=dev(ci.logits) if ci.logits is not None else torch.empty((T, w.E), dtype=torch.float32, device="cuda")))
    gamma = dev(inp.gamma)
    topk_idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    topk_w = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    res_out = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    norm_out = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    fp8 = args.precision == "w4a8"
    ws_n = B.moe4_w4a8_workspace_bytes(shape) if fp8 else B.moe4_layer_workspace_bytes(shape)
    if ws_n == 0:
        print(f"bench.py: {args.config} is not a valid shape for --precision {args.precision}", file=sys.stderr)
        sys.exit(2)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    if fp8 and args.side_stream == "on":
        print("bench.py: --side-stream applies to the W4A16 layer only", file=sys.stderr)
        sys.exit(2)

    use_side = args.side_stream == "on" and w.n_shared > 0
    side = torch.cuda.Stream() if use_side else None
    if use_side:
        log("routed chain on a side stream, shared expert on the launch stream")

    def layer_step(i):
        c = per_chunk[i % chunks]
        a13, a2 = weights[(i // chunks) % copies]
        if fp8:
            B.moe4_layer_w4a8(shape, c["x"], wr, c["logits"], a13, a2, s13, s2, c["residual"], gamma, topk_idx,
                              topk_w, res_out, norm_out, ws)
        else:
            B.moe4_layer(shape, c["x"], wr, c["logits"], a13, a2, s13, s2, c["residual"], gamma, topk_idx,
                         topk_w, res_out, norm_out, ws, side_stream=side)

    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    calls_per_step = chunks
    # steps: given, or about 2 s of GPU work from one timed probe step
    for i in range(calls_per_step):
        layer_step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(calls_per_step):
        layer_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    probe_s = max(ev0.elapsed_time(ev1) / 1e3, 1e-6)
    steps = args.steps or int(min(2000, max(20, 2.0 / probe_s)))
    warmup = args.warmup if args.warmup >= 0 else max(2, steps // 10)
    log(f"warmup {warmup} steps, then {steps} timed")
    for i in range(warmup * calls_per_step):
        layer_step(i)
    torch.cuda.synchronize()

    # ---- pass 1: headline ----
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps * calls_per_step):
        layer_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / steps
    tokens_per_step = T * chunks
    value = tokens_per_step * steps / (ms_total / 1e3)
    log(f"pass 1: {ms_per_step * 1e3:.2f} us/step, {value:.1f} tokens/s (wall {wall:.3f} s)")
    # the same with one weight copy ("warm": the weights may stay in the Infinity Cache
    # between steps), reported beside the headline, never as it
    warm = None
    if copies > 1:
        def warm_step(i):
            c = per_chunk[i % chunks]
            a13, a2 = weights[0]
            if fp8:
                B.moe4_layer_w4a8(shape, c["x"], wr, c["logits"], a13, a2, s13, s2, c["residual"], gamma,
                                  topk_idx, topk_w, res_out, norm_out, ws)
            else:
                B.moe4_layer(shape, c["x"], wr, c["logits"], a13, a2, s13, s2, c["residual"], gamma, topk_idx,
                             topk_w, res_out, norm_out, ws, side_stream=side)
        for i in range(warmup * calls_per_step):
            warm_step(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps * calls_per_step):
            warm_step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        warm_ms = ev0.elapsed_time(ev1) / steps
        warm = {"tokens_per_s": round(tokens_per_step * steps / (ev0.elapsed_time(ev1) / 1e3), 1),
                "ms_per_step": round(warm_ms, 6), "weight_copies": 1}
        log(f"pass 1 warm (one weight copy): {warm_ms * 1e3:.2f} us/step, {warm['tokens_per_s']:.1f} tokens/s")

    # ---- passes 2 and 3: the expert-FFN launches, each timed with events ----
    # The plan of every chunk is built first; then each launch kind runs back to back
    # (rotating weight copies as in pass 1) between two events on the launch stream,
    # so the mean is the kernel's own duration plus the gap between launches, not the
    # events' overhead. The routed up launch (pass 2) is the dominant kernel.
    pairs = T * w.k
    # where the up projections run on the GEMM, moe4_layer takes them on FP16 activations
    # (moe4_act_f16 once per call, then moe4_expert_up_f16): time the same launches
    prefill_routed = T * w.k >= 40 * w.E and w.H % 256 == 0 and w.I % 128 == 0
    prefill_dense = T >= 40 and w.H % 256 == 0 and w.I % 128 == 0
    f16_act = not fp8 and (prefill_routed or (s13 is not None and prefill_dense))

    def up_call(shp, c, offsets, perm_src, a13, h, gemm):
        if f16_act and gemm:
            B.moe4_expert_up_f16(shp, c["x16"], c["xexp"], offsets, perm_src, a13, h)
        else:
            B.moe4_expert_up(shp, c["x"], offsets, perm_src, a13, h)

    pws_n = B.moe4_permute_workspace_bytes(shape)
    pws = torch.empty(pws_n, dtype=torch.uint8, device="cuda") if pws_n else None
    plans, routing, hs, hds = [], [], [], []
    u8 = lambda *shp: torch.empty(shp, dtype=torch.uint8, device="cuda")
    # the FP8 form's halves take the activations already quantised (per chunk, once)
    fp8_h = lambda rows: (u8(rows, w.I), u8(rows, w.I // 32))
    for c in per_chunk:
        offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
        perm_src = torch.empty(pairs, dtype=torch.int32, device="cuda")
        inv = torch.empty(pairs, dtype=torch.int32, device="cuda")
        B.moe4_route(shape, c["x"] if wr is not None else None, wr, c["logits"], topk_idx, topk_w)
        B.moe4_permute(shape, topk_idx, offsets, perm_src, inv, pws)
        if fp8:
            c["x8"], c["xs"] = u8(T, w.H), u8(T, w.H // 32)
            B.moe4_quant_mxfp8(c["x"], c["x8"], c["xs"])
            h = fp8_h(pairs)
            B.moe4_expert_up_w4a8(shape, c["x8"], c["xs"], offsets, perm_src, w13, None, *h)
        else:
            h = torch.empty((pairs, w.I), dtype=torch.int16, device="cuda")
            if f16_act:  # as moe4_layer does where its up projections run on the GEMM
                c["x16"] = torch.empty((T, w.H), dtype=torch.float16, device="cuda")
                c["xexp"] = torch.empty(T, dtype=torch.int32, device="cuda")
                B.moe4_act_f16(c["x"], c["x16"], c["xexp"])
            up_call(shape, c, offsets, perm_src, w13, h, prefill_routed)
        hs.append(h)
        if s13 is not None:
            if fp8:
                hd = fp8_h(T)
                B.moe4_expert_up_w4a8(shape, c["x8"], c["xs"], None, None, s13, None, *hd)
            else:
                hd = torch.empty((T, w.I), dtype=torch.int16, device="cuda")
                up_call(shape, c, None, None, s13, hd, prefill_dense)
            hds.append(hd)
        torch.cuda.synchronize()
        routing.append(topk_idx.cpu().numpy())
        plans.append((offsets, perm_src))
    y = torch.empty((pairs, w.H), dtype=torch.int16, device="cuda")
    yd = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    h_tmp = fp8_h(pairs) if fp8 else torch.empty((pairs, w.I), dtype=torch.int16, device="cuda")
    hd_tmp = fp8_h(T) if fp8 else torch.empty((T, w.I), dtype=torch.int16, device="cuda")

    def up_routed(i):
        c = per_chunk[i % chunks]
        offsets, perm_src = plans[i % chunks]
        a13 = weights[(i // chunks) % copies][0]
        if fp8:
            B.moe4_expert_up_w4a8(shape, c["x8"], c["xs"], offsets, perm_src, a13, None, *h_tmp)
        else:
            up_call(shape, c, offsets, perm_src, a13, h_tmp, prefill_routed)

    def down_routed(i):
        offsets, _ = plans[i % chunks]
        a2 = weights[(i // chunks) % copies][1]
        if fp8:
            B.moe4_expert_down_w4a8(shape, *hs[i % chunks], offsets, a2, y)
        else:
            B.moe4_expert_down(shape, hs[i % chunks], offsets, a2, y)

    def up_shared(i):
        c = per_chunk[i % chunks]
        if fp8:
            B.moe4_expert_up_w4a8(shape, c["x8"], c["xs"], None, None, s13, None, *hd_tmp)
        else:
            up_call(shape, c, None, None, s13, hd_tmp, prefill_dense)

    def down_shared(i):
        if fp8:
            B.moe4_expert_down_w4a8(shape, *hds[i % chunks], None, s2, yd)
        else:
            B.moe4_expert_down(shape, hds[i % chunks], None, s2, yd)

    # the FP8 form always runs the tiled GEMM; the BF16 form streams below 40 rows per expert
    prefill_kind = fp8 or T * w.k >= 40 * w.E
    kind_name = "ffn_prefill_fp8_kernel" if fp8 else ("ffn_prefill_kernel" if prefill_kind else "ffn_decode_kernel")
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    launches = [("up_routed", up_routed, True, False), ("down_routed", down_routed, False, False)]
    if s13 is not None:
        launches += [("up_shared", up_shared, True, True), ("down_shared", down_shared, False, True)]
    k2 = min(steps, 400)
    kernels = {}
    for name, fn, up, dense in launches:
        for i in range(min(k2, 10) * chunks):
            fn(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(k2 * chunks):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        mean_s = ev0.elapsed_time(ev1) / (k2 * chunks) / 1e3
        nb = fl = 0
        for idx in routing:
            b, f, _ = ffn_work(w, T, idx, up, dense, fp8)
            nb += b
            fl += f
        nb /= chunks
        fl /= chunks
        if up and f16_act and (prefill_dense if dense else prefill_routed):
            kname = f"ffn_prefill_f16_kernel<{str(dense).lower()}, true>"
        elif prefill_kind:
            kname = f"{kind_name}<{str(up).lower()}, {str(dense).lower()}>"
        else:
            kname = f"{kind_name}<{str(up).lower()}, ...>"
        kernels[name] = {"kernel": kname,
                         "mean_us": round(mean_s * 1e6, 3), "launches": k2 * chunks,
                         "algorithmic_bytes": int(nb), "algorithmic_flops": int(fl),
                         "GB_s": round(nb / mean_s / 1e9, 1), "TFLOP_s": round(fl / mean_s / 1e12, 1)}
        log(f"pass {2 if name == 'up_routed' else 3}: {name} mean {mean_s * 1e6:.2f} us over {k2 * chunks} "
            f"launches; {nb / 1e6:.1f} MB, {fl / 1e9:.2f} GFLOP per launch -> {nb / mean_s / 1e9:.0f} GB/s, "
            f"{fl / mean_s / 1e12:.1f} TFLOP/s")

    # the FP16 activation rows (once per layer call, before the up GEMMs), timed the same way
    if f16_act:
        for i in range(min(k2, 10) * chunks):
            c = per_chunk[i % chunks]
            B.moe4_act_f16(c["x"], c["x16"], c["xexp"])
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(k2 * chunks):
            c = per_chunk[i % chunks]
            B.moe4_act_f16(c["x"], c["x16"], c["xexp"])
        ev1.record(stream)
        torch.cuda.synchronize()
        mean_s = ev0.elapsed_time(ev1) / (k2 * chunks) / 1e3
        nb = 2 * T * w.H * 2 + T * 4
        kernels["act_f16"] = {"kernel": "act_f16_kernel (FP16 activation rows for the up GEMMs)",
                              "mean_us": round(mean_s * 1e6, 3), "launches": k2 * chunks,
                              "algorithmic_bytes": int(nb), "GB_s": round(nb / mean_s / 1e9, 1)}
        log(f"pass 3: act_f16 mean {mean_s * 1e6:.2f} us; {nb / 1e6:.1f} MB -> {nb / mean_s / 1e9:.0f} GB/s")

    # the expert FFN as a whole: every FFN launch of a layer call (both GEMMs, routed and
    # shared, and the FP16 activation rows where the layer makes them), total work over
    # total time
    tot_us = sum(v["mean_us"] for v in kernels.values())
    tot_b = sum(v["algorithmic_bytes"] for v in kernels.values())
    tot_f = sum(v.get("algorithmic_flops", 0) for v in kernels.values())
    kernels["ffn_total"] = {"kernel": "every expert-FFN launch of a layer call", "mean_us": round(tot_us, 3),
                            "algorithmic_bytes": int(tot_b), "algorithmic_flops": int(tot_f),
                            "GB_s": round(tot_b / tot_us / 1e3, 1), "TFLOP_s": round(tot_f / tot_us / 1e6, 1)}

    # the other steps through their own entry points, timed the same way (route: the router
    # GEMV when the logits are computed, then top-k; permute; combine + RMSNorm)
    res_o = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    res_n = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
    invs = []
    for c, (offsets, perm_src) in zip(per_chunk, plans):
        inv = torch.empty(pairs, dtype=torch.int32, device="cuda")
        B.moe4_route(shape, c["x"] if wr is not None else None, wr, c["logits"], topk_idx, topk_w)
        B.moe4_permute(shape, topk_idx, offsets, perm_src, inv, pws)
        invs.append(inv)
    torch.cuda.synchronize()
    p_off = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    p_src = torch.empty(pairs, dtype=torch.int32, device="cuda")
    p_inv = torch.empty(pairs, dtype=torch.int32, device="cuda")
    glue = {
        "route": (lambda i: B.moe4_route(shape, per_chunk[i % chunks]["x"] if wr is not None else None, wr,
                                         per_chunk[i % chunks]["logits"], topk_idx, topk_w),
                  (T * w.H * 2 + w.E * w.H * 2 + T * w.E * 4 if wr is not None else T * w.E * 4) + T * w.k * 8),
        "permute": (lambda i: B.moe4_permute(shape, topk_idx, p_off, p_src, p_inv, pws),
                    T * w.k * 4 + (w.E + 1) * 4 + 2 * T * w.k * 4),
        "combine_norm": (lambda i: B.moe4_combine_norm(shape, y, invs[i % chunks], topk_w,
                                                       yd if s13 is not None else None,
                                                       per_chunk[i % chunks]["residual"], gamma, res_o, res_n),
                         pairs * w.H * 2 + (T * w.H * 2 if s13 is not None else 0) + T * w.H * 2 + w.H * 2
                         + pairs * 8 + 2 * T * w.H * 2),
    }
    # These launches are short: an eager loop would time the host's launch rate, so each
    # entry point's calls are captured into a HIP graph and replayed between the events.
    per_graph = 32 * chunks
    for name, (fn, nb) in glue.items():
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(3 * chunks):
                fn(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(per_graph):
                fn(i)
        torch.cuda.synchronize()
        replays = max(2, k2 * chunks // per_graph)
        graph.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(replays):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        mean_s = ev0.elapsed_time(ev1) / (replays * per_graph) / 1e3
        del graph
        kernels[name] = {"kernel": f"moe4_{name} (entry point, HIP graph replay)",
                         "mean_us": round(mean_s * 1e6, 3), "launches": replays * per_graph,
                         "algorithmic_bytes": int(nb), "GB_s": round(nb / mean_s / 1e9, 1)}
        log(f"pass 4: {name} mean {mean_s * 1e6:.2f} us over {replays * per_graph} calls (graph replay); "
            f"{nb / 1e6:.2f} MB -> {nb / mean_s / 1e9:.0f} GB/s")

    dom = kernels["up_routed"]
    up_mean_s = dom["mean_us"] / 1e6
    nbytes, flops = dom["algorithmic_bytes"], dom["algorithmic_flops"]
    if not prefill_kind:
        achieved = nbytes / up_mean_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = flops / up_mean_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}
    roofline["traffic"] = measured_traffic(args.config + ("_w4a8" if fp8 else ""),
                                           KERNEL_SOURCES["prefill_fp8" if fp8 else
                                                          "prefill" if prefill_kind else "decode"])
    roofline.update({"kernel": dom["kernel"] + " (routed expert up: W13 dequant-MFMA + SwiGLU)",
                     "mean_us": dom["mean_us"], "algorithmic_bytes": int(nbytes),
                     "algorithmic_flops": int(flops)})
    for v in kernels.values():
        if "TFLOP_s" in v:  # the FFN launches: against the roofline of their kind
            v["frac_of_peak"] = round(v["TFLOP_s"] / peak if prefill_kind else v["GB_s"] / HBM_PEAK_GBS, 4)
        else:               # the glue: against HBM
            v["frac_of_peak"] = round(v["GB_s"] / HBM_PEAK_GBS, 4)

    cfg = {"workload": f"{args.config}: T={T}{'x%d chunks' % chunks if chunks > 1 else ''} H={w.H} "
                       f"E={w.E}{'+%d shared' % w.n_shared if w.n_shared else ''} top-{w.k} I={w.I}, "
                       + ("W4A8 (E2M1 + E4M3/16 + FP32 weights rounded to E4M3; E4M3 activations, "
                          "E8M0 scale per 32)" if fp8 else "W4A16 (E2M1 + E4M3/16 + FP32)"),
           "T": T * chunks, "H": w.H, "E": w.E, "k": w.k, "I": w.I, "n_shared": w.n_shared,
           "weight_copies_rotated": copies, "routing": w.routing, "side_stream": use_side}
    if warm is not None:
        cfg["warm_one_weight_copy"] = warm
    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8" if fp8 else "bf16",
           "data": "synthetic", "config": cfg, "roofline": roofline, "kernels": kernels}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
