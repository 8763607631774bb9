#!/usr/bin/env python3
"""Bench of the W4A16 MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config decode_t8]

A step is one MoE layer call (route -> permute -> expert up -> expert down ->
combine+RMSNorm) over one batch of synthetic tokens, inputs resident in HBM. The
default workload is decode with T=8 tokens (H=2048, E=128 experts, top-8, I=768,
router logits computed from BF16 router weights). Weight copies are rotated so
the working set is at least 1 GiB, which keeps the 256 MB Infinity Cache from
serving the weights.

Two timed passes:
  1. the headline: K fused ``moe4_layer`` calls between two events on the launch
     stream (value = tokens / s, ms_per_step);
  2. the roofline: the dominant kernel (the expert "up" pass, W13 + SwiGLU) launched
     K times back to back on each chunk's plan, rotating weight copies, between two
     events on the launch stream; its algorithmic bytes (touched experts' packed
     weights + scales, activations in, h out) or flops divided by the mean launch
     duration give ``roofline.achieved``.
The fp64 oracle is timed on the host on a bounded sample (``cpu_baseline``).
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
MALL_DEFEAT_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="decode_t8")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-stream", choices=["on", "off"], default="off",
                    help="routed chain on a side stream beside the shared expert (moe4_layer_side)")
    ap.add_argument("--op", choices=["layer", "add_rmsnorm", "group_rmsnorm"], default="layer",
                    help="what a step is: the MoE layer (default), or one of the neighbouring "
                         "RMSNorm glue launches over the workload's T x H rows")
    ap.add_argument("--group", type=int, default=0, help="group_rmsnorm group size (0 = H / 8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB twice with torch (a plain copy of known size, for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "ffn_up_decode_t8_traffic.md")
KERNEL_SOURCES = {"decode": os.path.join(ROOT, "bit_moe_expert_amd", "csrc", "ffn_decode.hip"),
                  "prefill": os.path.join(ROOT, "bit_moe_expert_amd", "csrc", "ffn_prefill.hip")}


def source_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(config, kernel_source):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    if it was taken on this workload with the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    for line in open(TRAFFIC_SUMMARY):
        if line.startswith("machine:"):
            for kv in line[len("machine:"):].split():
                k, _, v = kv.partition("=")
                vals[k] = v
    if vals.get("config") != config or vals.get("source_sha") != source_sha(kernel_source):
        return None
    return int(vals["traffic_bytes"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def up_kernel_work(inp, idx):
    """Algorithmic bytes and flops of one expert-up launch for this routing."""
    w = inp.w
    distinct = len(set(idx.reshape(-1).tolist()))
    per_expert = 2 * w.I * w.H // 2 + 2 * w.I * w.H // 16 + 4   # nibbles + E4M3 scales + tscale
    pairs = inp.T * w.k
    act_in = inp.T * w.H * 2                                    # x, each token read once
    h_out = pairs * w.I * 2
    plan = (w.E + 1) * 4 + pairs * 4
    nbytes = distinct * per_expert + act_in + h_out + plan
    flops = 2 * pairs * w.H * (2 * w.I)
    if w.n_shared:
        nbytes += per_expert + inp.T * w.I * 2
        flops += 2 * inp.T * w.H * 2 * w.I
    return nbytes, flops, distinct


def cpu_baseline(inp, budget_s):
    """Time the oracle as it stands on the host, one thread, on a bounded sample."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    T = inp.T
    per_call = T
    sample_tokens = None
    if inp.w.T > 64:  # prefill shapes: a seeded sample of tokens
        sample_tokens = np.sort(np.random.default_rng(7).choice(inp.T, 16, replace=False))
        per_call = len(sample_tokens)
    reps, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            oracle.layer(inp, tokens=sample_tokens)
            reps += 1
            t_used = time.perf_counter() - t0
            if t_used >= budget_s or reps >= 1000:
                break
    what = (f"{reps} oracle layer calls on the same {per_call}-token batch"
            if sample_tokens is None else f"{reps} oracle calls on 16 sampled tokens of the {T}-token batch")
    return {"value": reps * per_call / t_used, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}; numpy fp64 with BLAS limited to 1 thread; {t_used:.1f} s"}


def glue_main(args):
    """One RMSNorm glue launch per step over the workload's T x H rows (x, residual and
    gamma drawn as for the layer); the launches run back to back between two events on
    the stream. Input copies are rotated so that at least 1 GiB is touched, up to 16
    copies: decode-sized rows then stay cache-resident, as they are after the previous
    kernel wrote them, instead of each launch paying for fresh pages."""
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
    if args.op != "layer":
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        torch.cuda.set_device(0)
        glue_main(args)
        return

    import numpy as np
    import torch

    from bit_moe_expert_amd import binding as B
    from bit_moe_expert_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = wl.workload(args.config)
    chunks = w.chunks
    log(f"generating inputs: {w}")
    t_gen = time.perf_counter()
    inputs = [wl.make_inputs(w, seed=0, chunk=c) for c in range(chunks)] if chunks > 1 else [wl.make_inputs(w, seed=0)]
    inp = inputs[0]
    log(f"inputs ready in {time.perf_counter() - t_gen:.1f} s")

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
    ws = torch.empty(B.moe4_layer_workspace_bytes(shape), dtype=torch.uint8, device="cuda")

    use_side = args.side_stream == "on" and w.n_shared > 0
    side = torch.cuda.Stream() if use_side else None
    if use_side:
        log("routed chain on a side stream, shared expert on the launch stream")

    def layer_step(i):
        c = per_chunk[i % chunks]
        a13, a2 = weights[(i // chunks) % copies]
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
    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup * calls_per_step):
        layer_step(i)
    torch.cuda.synchronize()

    # ---- pass 1: headline ----
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps * calls_per_step):
        layer_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    tokens_per_step = T * chunks
    value = tokens_per_step * args.steps / (ms_total / 1e3)
    log(f"pass 1: {ms_per_step * 1e3:.2f} us/step, {value:.1f} tokens/s (wall {wall:.3f} s)")

    # ---- pass 2: dominant kernel (expert up) timed with events ----
    # The plan of every chunk is built first; then K2 up launches run back to back
    # (rotating weight copies as in pass 1) between two events on the launch stream,
    # so the mean is the kernel's own duration plus the gap between launches, not the
    # events' overhead.
    pairs = T * w.k
    pws_n = B.moe4_permute_workspace_bytes(shape)
    pws = torch.empty(pws_n, dtype=torch.uint8, device="cuda") if pws_n else None
    h = torch.empty((pairs, w.I), dtype=torch.int16, device="cuda")
    plans, routing = [], []
    for c in per_chunk:
        offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
        perm_src = torch.empty(pairs, dtype=torch.int32, device="cuda")
        inv = torch.empty(pairs, dtype=torch.int32, device="cuda")
        B.moe4_route(shape, c["x"] if wr is not None else None, wr, c["logits"], topk_idx, topk_w)
        B.moe4_permute(shape, topk_idx, offsets, perm_src, inv, pws)
        torch.cuda.synchronize()
        routing.append(topk_idx.cpu().numpy())
        plans.append((offsets, perm_src))
    k2 = min(args.steps, 400)

    def up_launch(i):
        c = per_chunk[i % chunks]
        offsets, perm_src = plans[i % chunks]
        a13, _ = weights[(i // chunks) % copies]
        B.moe4_expert_up(shape, c["x"], offsets, perm_src, a13, h)

    for i in range(min(k2, 20) * chunks):
        up_launch(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(k2 * chunks):
        up_launch(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    up_mean_s = ev0.elapsed_time(ev1) / (k2 * chunks) / 1e3
    n_up = k2 * chunks
    nbytes, flops, distinct = 0, 0, []
    for ci, idx in zip(inputs, routing):
        b, f, d = up_kernel_work(ci, idx)
        nbytes += b
        flops += f
        distinct.append(d)
    nbytes /= chunks
    flops /= chunks
    log(f"pass 2: expert-up mean {up_mean_s * 1e6:.2f} us over {n_up} back-to-back launches; "
        f"{nbytes / 1e6:.1f} MB, {flops / 1e9:.2f} GFLOP per launch; distinct experts {distinct}")

    hbm_bound = flops / nbytes < 300.0
    if hbm_bound:
        achieved = nbytes / up_mean_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = flops / up_mean_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    kind = "decode" if inp.T * w.k < 64 * w.E else "prefill"
    roofline["traffic"] = measured_traffic(args.config, KERNEL_SOURCES[kind])
    roofline.update({"kernel": ("ffn_decode_kernel<true>" if kind == "decode" else "ffn_prefill_kernel<true>")
                               + " (expert up: W13 dequant-MFMA + SwiGLU)",
                     "mean_us": round(up_mean_s * 1e6, 3), "algorithmic_bytes": int(nbytes),
                     "algorithmic_flops": int(flops)})

    cfg = {"workload": f"{args.config}: T={T}{'x%d chunks' % chunks if chunks > 1 else ''} H={w.H} "
                       f"E={w.E}{'+%d shared' % w.n_shared if w.n_shared else ''} top-{w.k} I={w.I}, "
                       f"W4A16 (E2M1 + E4M3/16 + FP32)",
           "T": T * chunks, "H": w.H, "E": w.E, "k": w.k, "I": w.I, "n_shared": w.n_shared,
           "weight_copies_rotated": copies, "routing": w.routing, "side_stream": use_side}
    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": cfg, "roofline": roofline}
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
