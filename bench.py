"""Benchmark of the chunk-attention queue step on one MI355X.

One step = one queue step of the timed workload (every chunk's attention over
[predecessor K/V cache ; own K/V], all chunks x heads x query tiles in one
launch; for a workload with text tokens also the per-chunk cross-attention).
Inputs are seeded synthetic tensors already resident in HBM; the timed region
covers exactly `--steps` steps between a barrier and a device synchronisation.

Prints one JSON line with the throughput (exact FLOPs / time), queue-steps/s,
the roofline of the dominant kernel (HIP events on the stream the kernel runs
on) and, on rank 0, the CPU oracle timed on a bounded sample of the same
workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # 256 CUs x 4096 FLOP/clk x 2.4 GHz = 2516.6
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# device code of the attention kernels (the work plan and the kernel bodies);
# the host code around them does not change what the counters measure
KERNEL_SOURCES = [os.path.join(ROOT, "chunked_spatio_temporal_amd", "csrc", f)
                  for f in ("attn_kernel.h", "attn_pingpong.h", "attn_wide.h", "plan.h")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_name(block_rows: int, D: int, dtype: str) -> str:
    """The main-pass kernel a call with this work-item size runs."""
    if block_rows == 64:
        return f"chunk_attn_fwd_f32<{D}>"
    if block_rows == 384:
        return "chunk_attn_fwd_wide"
    if block_rows == 256:
        return f"chunk_attn_fwd_pingpong<{D},{dtype}>"
    return f"chunk_attn_fwd<{D},{dtype},{block_rows // 32}>"


def measure_mfma_peak(ca, ctx, synth, dev, stream, launches: int = 10) -> float:
    """Dense bf16 rate the device sustains (TFLOP/s): the library's matrix-core
    probe (one workgroup of 8 waves per CU, back-to-back 16x16x32 bf16 MFMAs,
    about 4 ms per launch), `launches` warmup launches (the clock climbs for
    about 30 ms after the attention pass), then the mean of `launches`
    launches timed with HIP events on the launch stream.  Run after the timed
    region, so its heat does not reach the measurement it is set beside."""
    import torch
    ops = synth.probe_operands(0, device=dev)
    out = torch.empty(ctx.cu_count * ca.PROBE_OUT_PER_WORKGROUP, dtype=torch.float32, device=dev)
    iters = 1 << 15
    for _ in range(launches):
        ca.mfma_probe(ops, iters, out, ctx=ctx, stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    flops = 0.0
    for _ in range(launches):
        flops += ca.mfma_probe(ops, iters, out, ctx=ctx, stream=stream)[1]
    ev[1].record(stream)
    torch.cuda.synchronize()
    return flops / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the 40-head queue); also the noise-init "
                         "workloads noise480p, noise480p_video")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-rows", type=int, default=0, choices=(0, 128, 256, 384),
                    help="query rows per work item (0: library default)")
    ap.add_argument("--item-blocks", type=int, default=0,
                    help="384-row query blocks per work item (0: chosen per call, 1..8)")
    ap.add_argument("--peaked", type=float, default=0.0,
                    help="scale Q so that the natural logits have this standard deviation "
                         "(queue workloads; 0: unit-scale inputs)")
    ap.add_argument("--exact-scale", action="store_true",
                    help="context with the exact-scale flag (scores scaled in fp32)")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the matrix-core rate probe after the timed region")
    ap.add_argument("--mfma-probe-only", action="store_true",
                    help="instead of the attention step: the matrix-core probe alone, "
                         "--warmup untimed and --steps timed launches (about 4 ms each)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (counter calibration)")
    ap.add_argument("--linearity", action="store_true",
                    help="instead of the one-workload line: queue-step time against the number "
                         "of chunks, and full attention over the same tokens against their count")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the queue step shards by head or by chunk range across GPUs, see DESIGN.md)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from chunked_spatio_temporal_amd import chunkattn as ca
    from chunked_spatio_temporal_amd import configs, synth

    if args.linearity:
        bench_linearity(args)
        return
    if args.mfma_probe_only:
        bench_mfma_probe(args)
        return
    name = args.workload or configs.BENCH_WORKLOAD
    if name in configs.NOISE_WORKLOADS:
        bench_noise(args, configs.NOISE_WORKLOADS[name])
        return
    w = configs.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ca.load_library()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    t0 = time.time()
    fifo = None
    if w.kind == "stream":
        # ring of n+1 slots; fill the queue until its head is clean (steady state)
        S = w.n + 1
        q, k, v = synth.queue_inputs(S, w.L, w.H, w.D, w.seed, device=dev, dtype=dt,
                                     k_rho=w.k_rho, v_rho=w.v_rho)
        cache = None
        out = torch.empty_like(q)
    elif w.kind in ("queue", "window"):
        q, k, v = synth.queue_inputs(w.n, w.L, w.H, w.D, w.seed, device=dev, dtype=dt,
                                     k_rho=w.k_rho, v_rho=w.v_rho)
        if args.peaked:
            q = (q.float() * args.peaked).to(dt)
        cache = synth.build_cache(k, v)
        if w.kind == "queue":
            out = torch.empty_like(q)
        else:
            out = torch.empty((w.n, 2, w.L, w.H, w.D), dtype=dt, device=dev)
        if w.n_text:
            qx = synth.cross_queries(w.n, w.L, w.H, w.D, w.seed, dev, dt)
            kt, vt = synth.text_inputs(w.n_text, w.H, w.D, w.seed, dev, dt)
            ox = torch.empty_like(qx)
    elif w.kind == "cross":
        # per-chunk queries over one shared set of text keys/values (batch stride 0)
        q = synth.cross_queries(w.n, w.L, w.H, w.D, w.seed, dev, dt)
        k, v = synth.text_inputs(w.lkv, w.H, w.D, w.seed, dev, dt)
        cache = None
        out = torch.empty_like(q)
    else:
        q = synth.normal((w.n, w.L, w.H, w.D), w.seed, synth.Q_ID, dev, dt)
        k = synth.normal((w.n, w.lkv, w.H, w.D), w.seed, synth.K_ID, dev, dt)
        v = synth.normal((w.n, w.lkv, w.H, w.D), w.seed, synth.V_ID, dev, dt)
        cache = None
        out = torch.empty_like(q)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {name} ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream(dev)
    flags = {0: 0, 128: ca.FLAG_BLOCK128, 256: ca.FLAG_BLOCK256,
             384: ca.FLAG_BLOCK384}[args.block_rows]
    if args.exact_scale:
        flags |= ca.FLAG_EXACT_SCALE
    ctx = ca.create(0, flags)
    if args.item_blocks:
        ctx = ca.Context(0, flags)
        ctx.set_item_blocks(args.item_blocks)

    if w.kind == "stream":
        fifo = ca.Fifo(w.n + 1, w.n)
        for _ in range(w.n):
            fifo.push()
            fifo.step(q, k, v, out, scale=w.scale, stream=stream, ctx=ctx)
        fifo.pop()

    def dominant():
        if w.kind == "stream":
            # steady state: a chunk enters, all n live chunks are processed, the head leaves
            fifo.push()
            fifo.step(q, k, v, out, scale=w.scale, stream=stream, ctx=ctx)
            fifo.pop()
        elif w.kind == "queue":
            ca.queue_step(q, k, v, cache, out=out, scale=w.scale, stream=stream, ctx=ctx)
        elif w.kind == "window":
            ca.window_step(q, k, v, cache, out=out, scale=w.scale, stream=stream, ctx=ctx)
        else:
            ca.full(q, k, v, out=out, scale=w.scale, stream=stream, ctx=ctx)

    def cross():
        ca.full(qx, kt, vt, out=ox, scale=w.scale, stream=stream, ctx=ctx)

    def step():
        dominant()
        if w.kind == "queue" and w.n_text:
            cross()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, events around every launch of the dominant kernel
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        dominant()
        ev[i][1].record(stream)
        if w.kind == "queue" and w.n_text:
            cross()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = total_ms / args.steps

    flops_step = w.total_flops()
    flops_dom = w.self_flops()
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    dom_avg_ms = float(launch_ms.mean())
    achieved = flops_dom / (dom_avg_ms * 1e-3) / 1e12

    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": round(BF16_PEAK_TFLOPS, 1),
        "unit": "TFLOP/s",
        "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": None,
        "kernel": kernel_name(ctx.call_block_rows(w.D, ca.BF16 if w.dtype == "bf16" else ca.F32),
                              w.D, w.dtype),
        "launch_ms_avg": round(dom_avg_ms, 4),
        "launch_ms_median": round(float(np.median(launch_ms)), 4),
        "launch_ms_min": round(float(launch_ms.min()), 4),
        "launch_ms_p90": round(float(np.percentile(launch_ms, 90)), 4),
    }
    if args.steps >= 100:
        # a long run: mean launch time over 10 consecutive segments of the timed
        # region, to show whether the rate holds as the chip heats up
        roofline["launch_ms_segments"] = [round(float(s.mean()), 4)
                                          for s in np.array_split(launch_ms, 10)]
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        entry = tr.get(name)
        if entry and entry.get("kernel_hash") == kernel_hash():
            roofline["traffic"] = entry["bytes_per_launch"]
    if not args.no_mfma_probe:
        peak = measure_mfma_peak(ca, ctx, synth, dev, stream)
        roofline["measured_peak"] = round(peak, 1)
        roofline["frac_of_measured_peak"] = round(achieved / peak, 4)

    if args.copy_calibration:
        n_bytes = 1 << 30
        a = torch.empty(n_bytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {n_bytes} bytes read + written", file=sys.stderr,
              flush=True)
        del a, b

    record = {
        "metric": "chunk-attention TFLOP/s (exact FLOPs) + queue-steps/sec; % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": name,
            "kind": w.kind,
            "n_chunks": w.n,
            "chunk_len": w.L,
            "heads": w.H,
            "head_dim": w.D,
            "lkv": w.lkv if w.kind in ("full", "cross") else None,
            "window": ("queries of chunks c and c+1; keys of chunks c-1 (cached), c, c+1"
                       if w.kind == "window" else None),
            "kv_cache": ("separate buffer" if cache is not None else
                         "predecessor read in place from its ring slot"
                         if w.kind == "stream" else None),
            "ring_slots": w.n + 1 if w.kind == "stream" else None,
            "text_tokens": w.n_text or None,
            "block_rows": ctx.call_block_rows(w.D, ca.BF16 if w.dtype == "bf16" else ca.F32),
            "item_blocks": args.item_blocks or "auto",
            "logit_std": args.peaked or 1.0,
            "scale_mode": "exact (S scaled in fp32)" if args.exact_scale else
                          "default (scaled Q rounded to bf16)",
            "flops_per_step": flops_step,
        },
        "queue_steps_per_s": round(1e3 / ms_per_step, 3),
        "pct_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": None,
    }

    if args.peaked and w.kind == "queue":
        record["recheck"] = recheck_share(w, q, k, v, cache)

    if not args.no_cpu_baseline:
        if w.kind == "stream":
            # the live chunks in processing order: chunk 0 (the tail) and its successor
            live = [s for _, s, _ in fifo.live()]
            lin = lambda t: t[live].contiguous()
            record["cpu_baseline"] = cpu_baseline(w, lin(q), lin(k), lin(v), None,
                                                  args.cpu_seconds)
        else:
            record["cpu_baseline"] = cpu_baseline(w, q, k, v, cache, args.cpu_seconds)

    print(json.dumps(record), flush=True)


def bench_mfma_probe(args):
    """The library's matrix-core probe alone: the dense bf16 rate this device
    sustains on back-to-back MFMAs (one JSON line)."""
    import numpy as np
    import torch

    from chunked_spatio_temporal_amd import chunkattn as ca
    from chunked_spatio_temporal_amd import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ca.load_library()
    ctx = ca.create(0)
    stream = torch.cuda.current_stream(dev)
    ops = synth.probe_operands(0, device=dev)
    out = torch.empty(ctx.cu_count * ca.PROBE_OUT_PER_WORKGROUP, dtype=torch.float32, device=dev)
    iters = 1 << 15
    for _ in range(args.warmup):
        ca.mfma_probe(ops, iters, out, ctx=ctx, stream=stream)
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    flops = 0.0
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        flops = ca.mfma_probe(ops, iters, out, ctx=ctx, stream=stream)[1]
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    rate = flops / (float(ms.mean()) * 1e-3) / 1e12
    record = {
        "metric": "dense bf16 MFMA rate sustained by the matrix-core probe",
        "value": round(rate, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mfma_probe", "workgroups": ctx.cu_count, "waves_per_workgroup": 8,
                   "instruction": "v_mfma_f32_16x16x32_bf16", "rounds_per_launch": iters,
                   "flops_per_launch": flops},
        "roofline": {"bound": "mfma", "achieved": round(rate, 2),
                     "peak": round(BF16_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(rate / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "mfma_peak_probe",
                     "launch_ms_min": round(float(ms.min()), 4),
                     "launch_ms_max": round(float(ms.max()), 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(record), flush=True)


def bench_linearity(args):
    """Cost against video length (DualParal write-up, section 二: with a fixed
    chunk size the per-step cost grows with the number of chunks, not with its
    square).  The 40-head 480p queue step (chunks of 6240 tokens, head dim 128,
    bf16) at 1, 2, 4, 8 and 16 chunks, and full bidirectional attention over
    the same n x 6240 tokens (one sequence, 40 heads) at n = 1, 2, 4, 8.  One
    JSON line: milliseconds per call (mean of HIP events over --steps calls
    after --warmup), FLOPs and TFLOP/s per point."""
    import torch

    from chunked_spatio_temporal_amd import chunkattn as ca
    from chunked_spatio_temporal_amd import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ca.load_library()
    L, H, D = 6240, 40, 128
    scale = D ** -0.5
    stream = torch.cuda.current_stream(dev)
    steps, warmup = max(args.steps, 1), args.warmup

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / steps

    queue, full = [], []
    for n in (1, 2, 4, 8, 16):
        q, k, v = synth.queue_inputs(n, L, H, D, 20 + n, device=dev, k_rho=0.9)
        cache = synth.build_cache(k, v)
        out = torch.empty_like(q)
        ms = timed(lambda: ca.queue_step(q, k, v, cache, out=out, scale=scale))
        flops = 4.0 * (L * L + (n - 1) * 2 * L * L) * D * H
        queue.append({"n_chunks": n, "tokens": n * L, "ms": round(ms, 4),
                      "ms_per_chunk": round(ms / n, 4), "flops": flops,
                      "tflops": round(flops / ms / 1e9, 1)})
        print(f"[bench] queue n={n}: {ms:.3f} ms", file=sys.stderr, flush=True)
        del q, k, v, cache, out
    for n in (1, 2, 4, 8):
        S = n * L
        q = synth.normal((1, S, H, D), 30 + n, synth.Q_ID, dev)
        k = synth.normal((1, S, H, D), 30 + n, synth.K_ID, dev)
        v = synth.normal((1, S, H, D), 30 + n, synth.V_ID, dev)
        out = torch.empty_like(q)
        ms = timed(lambda: ca.full(q, k, v, out=out, scale=scale))
        flops = 4.0 * S * S * D * H
        full.append({"tokens": S, "ms": round(ms, 4), "ms_per_6240_tokens": round(ms / n, 4),
                     "flops": flops, "tflops": round(flops / ms / 1e9, 1)})
        print(f"[bench] full S={S}: {ms:.3f} ms", file=sys.stderr, flush=True)
        del q, k, v, out
    print(json.dumps({"report": "linearity", "unit": "ms per call", "chunk_len": L, "heads": H,
                      "head_dim": D, "dtype": "bf16", "steps": steps, "warmup": warmup,
                      "queue_step": queue, "full_attention_same_tokens": full}), flush=True)


def bench_noise(args, w):
    """Coordinated noise initialization, chained chunk after chunk (each init
    avoids the frames the previous chunk's last `excl` frames used)."""
    import numpy as np
    import torch

    from chunked_spatio_temporal_amd import chunkattn as ca

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ca.load_library()
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(w.seed)
    pool = torch.randn((w.pool_frames,) + w.frame_shape, generator=g, device=dev).to(dt)
    n_keys = args.warmup + args.steps
    keys = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_keys, w.pool_frames), generator=g,
                         device=dev, dtype=torch.int32)
    outs = [torch.empty((w.frames,) + w.frame_shape, dtype=dt, device=dev) for _ in range(2)]
    idxs = [torch.empty(w.frames, dtype=torch.int32, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    ctx = ca.create(0)
    state = {"prev": None}

    def init(i):
        out, idx = outs[i % 2], idxs[i % 2]
        prev = state["prev"]
        ca.noise_init(pool, keys[i], w.frames, prev, w.excl if prev is not None else 0,
                      out=out, idx_out=idx, stream=stream, ctx=ctx)
        state["prev"] = idx

    for i in range(args.warmup):
        init(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for j in range(args.steps):
        ev[j][0].record(stream)
        init(args.warmup + j)
        ev[j][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    launch = np.array([a.elapsed_time(b) for a, b in ev])
    nbytes = w.bytes_per_init(pool.element_size())
    gbs = nbytes / (launch.mean() * 1e-3) / 1e9
    record = {
        "metric": "coordinated noise init: GB/s (pool frames read + chunk written)",
        "value": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "pool_frames": w.pool_frames, "frames": w.frames,
                   "excl": w.excl, "frame_shape": list(w.frame_shape),
                   "bytes_per_step": nbytes},
        "inits_per_s": round(1e3 / ms, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "noise_select + noise_gather",
                     "launch_ms_avg": round(float(launch.mean()), 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import noise as noise_sim
        pool_h = pool.cpu().numpy() if dt == torch.float32 else pool.float().cpu().numpy()
        keys_h = keys.cpu().numpy().view(np.uint32)
        t0 = time.perf_counter()
        count, prev = 0, None
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            idx = noise_sim.select(w.pool_frames, keys_h[count % n_keys], w.frames, prev,
                                   w.excl if prev is not None else 0)
            noise_sim.init_chunk(pool_h, idx)
            prev, count = idx, count + 1
        dt_cpu = time.perf_counter() - t0
        record["cpu_baseline"] = {"value": round(count * nbytes / dt_cpu / 1e9, 3), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"{count} chained chunk inits in {dt_cpu:.1f} s"}
    print(json.dumps(record), flush=True)


def recheck_share(w, q, k, v, cache):
    """Share of 384-row work items that the range recheck recomputes: items
    with a row whose sum l = sum_j 2^(S_j) (S in log2 units) leaves
    [2^-64, 2^128), computed in fp32 from the same inputs (outside the timed
    region)."""
    import math

    import torch
    c = w.scale / math.log(2.0)
    L, bm = w.L, 384
    n_items = marked = 0
    for ch in range(w.n):
        for h in range(w.H):
            # cache[ch, 0] holds the K of chunk ch - 1
            keys = k[ch, :, h] if ch == 0 else torch.cat([cache[ch, 0, :, h], k[ch, :, h]])
            s = (q[ch, :, h].float() @ keys.float().T) * c
            l2 = torch.logsumexp(s * math.log(2.0), dim=1) / math.log(2.0)
            bad = ((l2 >= 128) | (l2 < -64)).cpu()
            for t in range(0, L, bm):
                n_items += 1
                marked += int(bad[t:t + bm].any())
    return {"items": n_items, "items_rechecked": marked,
            "share": round(marked / max(n_items, 1), 5)}


def cpu_baseline(w, q, k, v, cache, seconds):
    """Times the fp64 oracle on host cores on a bounded sample of the workload.

    Sample: random query rows (all heads equally likely) of chunk 0 and of
    chunks >= 1 in their workload proportions; the oracle computes each row over
    its full key/value set.  Throughput uses the same exact FLOP count per row
    (4 * |R_c| * D), and queue-steps/s is extrapolated from it.
    """
    import numpy as np

    import oracle

    rng = np.random.default_rng(1234)
    if w.kind in ("queue", "stream"):
        chunks = [0, 1] if w.n > 1 else [0]
        lo = max(chunks[-1] - 1, 0)
        sub = lambda t: t[lo:chunks[-1] + 1].cpu()
        qs, ks, vs = sub(q), sub(k), sub(v)
        cs = None if cache is None else sub(cache)

        def rows_for(count):
            # chunk 0 carries 1 share of the work per L rows, chunks >= 1 carry 2 each
            p1 = (2 * (w.n - 1)) / (2 * (w.n - 1) + 1) if w.n > 1 else 0.0
            c = (rng.random(count) < p1).astype(np.int64)
            return np.stack([c, rng.integers(0, w.H, count), rng.integers(0, w.L, count)], 1)

        def flops(rows):
            return float(sum(4 * (2 * w.L if c >= 1 else w.L) * w.D for c in rows[:, 0]))

        run = lambda rows: oracle.queue_rows(qs, ks, vs, cs, rows, w.scale)
    elif w.kind == "window":
        # window 1 of the three-chunk sub-problem [0, 1, 2]: 2L query rows over
        # 3L keys (the shape of every interior window)
        sub = lambda t: t[0:3].cpu()
        qs, ks, vs = sub(q), sub(k), sub(v)
        cs = None if cache is None else sub(cache)

        def rows_for(count):
            return np.stack([np.ones(count, np.int64), rng.integers(0, w.H, count),
                             rng.integers(0, 2 * w.L, count)], 1)

        def flops(rows):
            return float(len(rows) * 4 * 3 * w.L * w.D)

        run = lambda rows: oracle.window_rows(qs, ks, vs, cs, rows, w.scale)
    else:
        qs, ks, vs = q.cpu(), k.cpu(), v.cpu()

        def rows_for(count):
            return np.stack([np.zeros(count, np.int64), rng.integers(0, w.H, count),
                             rng.integers(0, w.L, count)], 1)

        def flops(rows):
            return float(len(rows) * 4 * w.lkv * w.D)

        run = lambda rows: oracle.full_rows(qs, ks, vs, rows, w.scale)

    probe = rows_for(512)
    t0 = time.perf_counter()
    run(probe)
    dt = time.perf_counter() - t0
    count = int(max(512, min(400000, 512 * seconds / max(dt, 1e-6))))
    rows = rows_for(count)
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    tflops = flops(rows) / dt / 1e12
    return {
        "value": round(tflops, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{count} random query rows (all heads) of {w.name}"
                  f"{' interior windows' if w.kind == 'window' else ''}, each over its full "
                  f"key/value set; {dt:.1f} s; fp64",
        "queue_steps_per_s_extrapolated": round(tflops * 1e12 / w.self_flops(), 8),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
