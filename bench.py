#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer of one decode iteration: the new
token of every sequence is written into its slot (pa_write_kv; for the
copy-on-write workload the block copies come first, pa_copy_blocks), then
pa_decode attends over every sequence's paged context.  Inputs are resident
in HBM before timing starts.  Successive steps rotate over `--layers`
independent KV pools (one per model layer, all sharing the block tables, as
a real decode iteration does), so no step finds its K/V in the caches of the
previous one.

Decode steps are launched as HIP graph replays, one captured graph per decode
iteration of a 32-layer model (`--graph-steps`; layer i of the iteration reads
pool i % `--layers`): an eager launch from Python costs about as much host time
as the GPU work, and every graph launch adds a few microseconds of GPU idle
time, once per iteration as in a serving loop.

Prints ONE JSON line.  `value` = algorithmic bytes of the step / step time
(GB/s, decimal), tokens/s = sequences / step time.  `roofline` covers
pa_decode (its partition kernel, and the merge kernel where the merge is not
inside it), timed with HIP events
on the launch stream over graph replays of the decode alone.  `cpu_baseline` times the CPU oracle on the same
inputs (layer 0) on this host's cores.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
WARM_S = 0.1  # untimed GPU work before each timed phase (see warm_graph())

WORKLOAD_TEXT = {
    "tiny": "tiny paged decode: 1 sequence, 1 head, D 64, B 16, context 100 -> write token "
            "100 -> 101, 16 physical blocks in random order, fp32 (latency)",
    "llama3_8b": "Llama-3-8B-shaped GQA decode, one layer: 32 seqs, 32 q / 8 kv heads, D 128, "
                 "B 16, ctx ~ U{128..4096}, pool 12,000 blocks, bf16",
    "llama3_8b_table128k": "the Llama-3-8B-shaped batch with block tables of 131,072-token "
                           "capacity (8,192 entries; same lengths U{128..4096}): launch "
                           "sized by the table, not the work",
    "many_seqs": "512 sequences of U{128..600} tokens, 32 q / 8 kv heads, D 128, B 16, tables "
                 "of 40 blocks, bf16: the unit search over 8 rounds of 64 sequences",
    "opt_13b": "OPT-13B-shaped MHA decode, one layer: 64 seqs, 40 heads, D 128, B 16, "
               "ctx lognormal median 512 clipped [16, 2048], pool 10,000 blocks, fp16",
    "parallel_sampling": "parallel sampling: 16 prompts x 8 samples, 32 heads, D 128, B 16, "
                         "shared 1,024-token prompt + U{0..256} private tokens, bf16",
    "parallel_sampling_cow": "parallel sampling with copy-on-write: 16 x 8 samples, 32 heads, "
                             "1,016-token shared prompt, 112 block copies, bf16",
    "long_ctx": "long-context split decode: 4 seqs, 32 q / 8 kv heads, D 128, B 16, ctx 32K / "
                "64K / 96K / 128K, 512-token partitions, bf16",
    "prefill_llama3_8b": "paged prefill, one layer: 8 whole prompts of U{1024..4096} tokens "
                         "(21,069 tokens), 32 q / 8 kv heads, D 128, B 16, bf16",
    "prefill_chunked_llama3_8b": "chunked paged prefill, one layer: 8 sequences with cached "
                                 "prefixes of U{0..15360} tokens take 1,024-token chunks, "
                                 "32 q / 8 kv heads, D 128, B 16, bf16",
    "vattention_llama3_8b": "the Llama-3-8B-shaped decode batch (32 seqs, 32 q / 8 kv heads, "
                            "D 128, bf16) on virtual-memory KV storage: one contiguous range "
                            "per request slot (max context 4096), pages mapped on demand, "
                            "decode without a block table",
    "swap_llama3_8b": "preemption by swapping, one layer: the 8 longest sequences of the "
                      "Llama-3-8B-shaped batch (1,744 blocks of 8 kv heads x 16 tokens x D 128, "
                      "bf16) out to pinned host memory and back into other free device blocks",
}
PEAK_HOST_LINK_GBPS = 64.0  # PCIe 5.0 x16, one direction, published
PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix cores, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--layers", type=int, default=8, help="resident KV pools rotated per step")
    ap.add_argument("--graph-steps", type=int, default=32,
                    help="decode workloads: steps per captured graph, one decode iteration "
                         "of a 32-layer model (layer i on pool i %% --layers)")
    ap.add_argument("--partition", type=int, default=None,
                    help="partition tokens for pa_decode (default: the workload's, else auto)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle repetitions (0 = skip)")
    ap.add_argument("--cpu-single-reps", type=int, default=1,
                    help="decode: oracle repetitions on one thread, after the all-core ones")
    ap.add_argument("--seed", type=int, default=None,
                    help="draw of the workload (default: the workload's own seed)")
    ap.add_argument("--cascade", action="store_true",
                    help="decode with pa_decode_cascade: shared prefix blocks read once per "
                         "group of sequences (groups from the block tables)")
    ap.add_argument("--append", action="store_true",
                    help="decode workloads with one new token per sequence: the step is one "
                         "pa_decode_append call (the decode kernel stores the new tokens)")
    ap.add_argument("--warm-ms", type=float, default=WARM_S * 1e3,
                    help="untimed GPU work before each timed phase, ms (profiling runs: 0)")
    ap.add_argument("--force-valu", action="store_true",
                    help="measurement: the one-head VALU kernel on 16-bit data (PA_DECODE_FORCE_VALU)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per block for the llama3_8b workload (8, 16 or 32)")
    ap.add_argument("--page-kib", type=int, default=2048,
                    help="page size of the virtual-memory KV storage (vattention workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run torch's plain copy of a 1 GiB tensor (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counter scale)")
    return ap.parse_args()


def warm_graph(g, stream, seconds=None):
    """Untimed replays of CUDA/HIP graph g on stream for about `seconds` of GPU
    work (WARM_S by default).  Under sustained load the GPU settles at a
    faster operating point after some 15-20 ms: the Llama-3-8B decode step
    measured ~51.5 us per launch over its first 36 graph replays of 8 layers
    and 49.0 us from the 48th on (same process, back-to-back replays).  Every
    timed phase starts from that steady state, as a serving loop runs."""
    import torch
    seconds = WARM_S if seconds is None else seconds
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t0, 1e-5)
        for _ in range(max(3, int(seconds / one)) if seconds > 0 else 1):
            g.replay()
        torch.cuda.synchronize()


def calibrate_copy(reps=5):
    """Plain device copy of a known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "reps": reps}),
          flush=True)


def host_info():
    """The host's CPU model and logical CPU count (for the oracle baselines)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def raw_bits(t):
    """numpy view of a CPU tensor's element bits (the oracle's input form)."""
    import numpy as np
    import torch
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def measured_traffic(workload, part, append=False, root=ROOT, planned=False):
    """HBM bytes per pa_decode launch from the committed counter summary
    (profiles/decode_<workload>_traffic.json: rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes scaled by a plain copy's), or None when no summary exists
    for this workload and partitioning (a fixed length, "auto", or "plan" for
    pa_decode_plan's choice) or the kernel sources have changed since the
    counters were taken (the summary records their SHA-256)."""
    rel = os.path.join("profiles",
                       f"decode_{workload}{'_append' if append else ''}_traffic.json")
    path = os.path.join(root, rel)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    label = "plan" if planned else (part or "auto")
    if rec.get("workload") != workload or rec.get("partition_tokens") != label:
        return None, rel
    for src, digest in rec["sources_sha256"].items():
        with open(os.path.join(root, src), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None, rel
    return int(rec["bytes_per_launch"]), rel


def unique_decode_bytes(block_tables, ctx, S, Hq, Hkv, D, B, e):
    """decode_bytes with each physical block's tokens counted once, however
    many sequences read it: the HBM lower bound when blocks are shared."""
    used = {}
    for s in range(S):
        for i in range(-(-ctx[s] // B)):
            phys = int(block_tables[s, i])
            used[phys] = max(used.get(phys, 0), min(B, ctx[s] - i * B))
    kv = 2 * sum(used.values()) * Hkv * D * e
    return kv + 2 * S * Hq * D * e + 4 * sum(-(-c // B) for c in ctx) + 4 * S


def decode_bytes(ctx, S, Hq, Hkv, D, B, e):
    """Algorithmic bytes of one decode: K+V of every valid token, q in, out,
    the used block-table entries and the context lengths."""
    kv = sum(2 * c * Hkv * D * e for c in ctx)
    qo = 2 * S * Hq * D * e
    table = 4 * sum(-(-c // B) for c in ctx) + 4 * S
    return kv + qo + table


def main():
    args = parse()
    global WARM_S
    WARM_S = args.warm_ms * 1e-3
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-device and the benchmark measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_299_amd as pa
    from paged_kv_cache_299_amd import workloads
    from paged_kv_cache_299_amd.layout import ELEM_BYTES, kv_cache_shapes

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    pa.load_library()  # fails loudly if libpa.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload.startswith("swap_"):
        bench_swap(args, dev)
        return
    if args.workload.startswith("prefill_"):
        bench_prefill(args, dev)
        return
    if args.workload.startswith("vattention_"):
        bench_vattention(args, dev)
        return

    t_setup = time.time()
    kw = {} if args.seed is None else {"seed": args.seed}
    if args.block_size is not None:
        kw["block_size"] = args.block_size
    case = workloads.CASES[args.workload](fill=False, **kw)
    S, Hq, Hkv, D, B = case.num_seqs, case.num_heads, case.num_kv_heads, case.head_dim, \
        case.block_size
    NB, dt = case.num_blocks, case.dtype
    e = ELEM_BYTES[dt]
    part = args.partition if args.partition is not None else (case.partition_tokens or 0)
    # No length given: plan it from the batch's context lengths on the host, as
    # the scheduler that built the batch would (pa_decode_plan; 0 = automatic),
    # and time the plain pa_decode beside it: its automatic split plans the
    # length on the device from the same lengths by the same rule where it can
    # (matrix-core kernel at B = 16, fewer than 2,048 rows, at most 256
    # sequences, tables of 513 to 2^20 tokens).
    mfma = dt != torch.float32 and Hq // Hkv <= 16 and not args.force_valu
    planned = False
    if args.partition is None and not case.partition_tokens and not args.cascade \
            and not args.force_valu:
        part = pa.pa_decode_plan(case.context_lens, Hq, Hkv, B, case.max_blocks, dt)
        planned = part > 0
    device_plan = (mfma and B == 16 and S * Hkv < 2048 and S <= 256
                   and 512 < case.max_blocks * B <= (1 << 20) and not args.cascade)
    k_shape, v_shape = kv_cache_shapes(NB, Hkv, D, B, dt)
    gen = torch.Generator(device=dev)
    pools = []
    for layer in range(args.layers):
        gen.manual_seed(1000 * case.seed + layer)
        k = torch.randn(k_shape, generator=gen, device=dev, dtype=torch.float32).to(dt)
        v = torch.randn(v_shape, generator=gen, device=dev, dtype=torch.float32).to(dt)
        pools.append((k, v))
    q = case.q.to(dev)
    bt = case.block_tables.to(dev)
    cl = case.context_lens.to(dev)
    out = torch.empty_like(q)
    steps = []
    for st in case.steps:
        if isinstance(st, workloads.CopyStep):
            steps.append(("copy", st.block_mapping.to(dev)))
        else:
            steps.append(("write", st.k_new.to(dev), st.v_new.to(dev), st.slot_mapping.to(dev)))
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    ctx = case.context_lens.tolist()
    # the hint a serving system gives from its block reference counts
    shared = workloads.shares_blocks(case.block_tables, case.context_lens, B)
    gs, pb, max_group = workloads.shared_prefix_groups(case.block_tables, case.context_lens, B)
    gs_d, pb_d = gs.to(dev), pb.to(dev)
    dec_bytes = decode_bytes(ctx, S, Hq, Hkv, D, B, e)
    uniq_bytes = unique_decode_bytes(case.block_tables, ctx, S, Hq, Hkv, D, B, e)
    step_bytes = dec_bytes
    for st in case.steps:
        if isinstance(st, workloads.CopyStep):
            step_bytes += 2 * 2 * st.block_mapping.shape[0] * Hkv * B * D * e  # K+V, read+write
        else:
            T = st.slot_mapping.shape[0]
            step_bytes += 2 * 2 * T * Hkv * D * e + 8 * T

    L = len(pools)
    stream = torch.cuda.Stream()  # default priority

    # pa_decode_append: one write step of one token per sequence (its last), no copies
    append = args.append and len(steps) == 1 and steps[0][0] == "write" and \
        steps[0][1].shape[0] == S
    if args.append and not append:
        print("--append takes workloads whose step writes one token per sequence",
              file=sys.stderr)
        sys.exit(2)

    # the loads-only ceiling of the decode's access pattern (pa_read_tiles):
    # the matrix-core configuration of pa_decode only
    read_ok = (not args.cascade and not append and not shared and B == 16
               and dt != torch.float32 and Hq // Hkv <= 16 and not args.force_valu)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def enqueue(layer, write=True, decode=True, read=False, plain=False):
        k, v = pools[layer]
        if plain:  # the plain entry point pa_decode: automatic partitions, no hint
            pa.pa_decode(q, k, v, bt, cl, case.scale, out)
            return
        if read:
            pa.pa_read_tiles(k, v, bt, cl, sink, Hq, partition_tokens=part)
            return
        if append:
            if write and decode:
                pa.pa_decode_append(q, steps[0][1], steps[0][2], k, v, bt, cl, case.scale, out,
                                    partition_tokens=part)
            elif decode:
                pa.pa_decode(q, k, v, bt, cl, case.scale, out, partition_tokens=part)
            return
        if write:
            for st in steps:
                if st[0] == "copy":
                    pa.pa_copy_blocks(k, v, st[1])
                else:
                    pa.pa_write_kv(st[1], st[2], k, v, st[3])
        if decode and args.cascade:
            pa.pa_decode_cascade(q, k, v, bt, cl, gs_d, pb_d, case.scale, out,
                                 max_group_size=max_group, partition_tokens=part)
        elif decode:
            pa.pa_decode(q, k, v, bt, cl, case.scale, out, partition_tokens=part,
                         shared_blocks=shared, force_valu=args.force_valu)

    # eager warmup on the capture stream (grows the library's workspace for it;
    # the plain pa_decode phase below may need another size than `part`)
    time_plain = planned and not append
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            enqueue(i % L)
        if time_plain:
            enqueue(0, plain=True)
    torch.cuda.synchronize()

    # HIP graphs: launching a decode step from Python (ctypes marshalling of
    # two calls) takes about as long as the GPU work, and each graph launch
    # leaves the GPU idle for several microseconds, so one graph holds the
    # steps of one decode iteration of the model (--graph-steps, 32 layers as
    # in Llama-3-8B), layer i of the iteration on pool i % L -- as a serving
    # loop captures its decode iteration.  Replays are idempotent: the writes
    # store the same tokens in the same slots.
    G = max(1, args.graph_steps)

    def capture(steps, **phase):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                enqueue(i % L, **phase)
        return g

    def timed(n, **phase):
        """Runs exactly n steps of the phase as graph replays (G steps per
        graph, a shorter graph for the rest); wall seconds and GPU ms (HIP
        events on the launch stream)."""
        q_, r_ = divmod(n, G)
        g_all = capture(G, **phase) if q_ else None
        g_rest = capture(r_, **phase) if r_ else None
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        warm_graph(g_all if g_all is not None else g_rest, stream)
        with torch.cuda.stream(stream):
            if g_rest is not None:
                g_rest.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(q_):
                g_all.replay()
            if g_rest is not None:
                g_rest.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1)

    def spread(passes=25, **phase):
        """p10 / median / p90 of the per-step GPU time over graph replays of
        G steps each (events between replays)."""
        g_all = capture(G, **phase)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(passes + 1)]
        warm_graph(g_all, stream)
        with torch.cuda.stream(stream):
            ev[0].record(stream)
            for i in range(passes):
                g_all.replay()
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / G for i in range(passes))
        return {"p10": round(per[len(per) // 10], 2), "median": round(per[len(per) // 2], 2),
                "p90": round(per[(9 * len(per)) // 10], 2), "passes": passes, "steps_each": G}

    # timed region: exactly `steps` steps
    wall, step_gpu_ms = timed(args.steps)
    ms_per_step = wall * 1e3 / args.steps
    # the kernels alone, per launch: pa_decode (partition + merge kernels) and
    # the KV writes (plus block copies for copy-on-write); with --append the
    # roofline covers the fused call, which also stores the new tokens
    _, dec_ms = timed(args.steps, write=False)
    dec_avg = dec_ms / args.steps
    if append:
        wr_avg = None
        app_avg = step_gpu_ms / args.steps
    else:
        _, wr_ms = timed(args.steps, decode=False)
        wr_avg = wr_ms / args.steps
    dec_spread = spread(write=False)
    # the plain pa_decode (its automatic split) beside the host-planned length
    plain_us = None
    if time_plain:
        _, pl_ms = timed(args.steps, plain=True)
        plain_us = pl_ms / args.steps * 1e3
    read_us = None
    if read_ok:
        _, rd_ms = timed(args.steps, write=False, decode=False, read=True)
        read_us = rd_ms / args.steps * 1e3
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # roofline bytes: each physical block counted once (equal to dec_bytes
    # unless blocks are shared; then the logical rate is reported as effective)
    roof_bytes = uniq_bytes + (step_bytes - dec_bytes if append else 0)
    roof_avg = app_avg if append else dec_avg
    achieved = roof_bytes / (roof_avg * 1e-3) / 1e9
    traffic, traffic_src = ((None, None) if args.cascade or B != 16 or args.force_valu
                            else measured_traffic(args.workload, part, append,
                                                  planned=planned))

    # CPU baseline: the oracle on layer 0's pools after the steps, same inputs
    cpu = None
    if args.cpu_reps > 0:
        import oracle
        k0, v0 = pools[0]
        with torch.cuda.stream(stream):
            enqueue(0)
        torch.cuda.synchronize()
        kh, vh = raw_bits(k0.cpu()), raw_bits(v0.cpu())
        code = pa.DTYPE_CODES[dt]

        def oracle_seconds(reps):
            times = []
            for _ in range(reps):
                t = time.perf_counter()
                oracle.decode(raw_bits(case.q), kh, vh, case.block_tables.numpy(),
                              case.context_lens.numpy(), case.scale, num_kv_heads=Hkv,
                              head_dim=D, block_size=B, k_x=16 // e, dtype=code)
                times.append(time.perf_counter() - t)
            return statistics.median(times)

        t_med = oracle_seconds(args.cpu_reps)
        cpu = {"value": round(dec_bytes / t_med / 1e9, 3), "unit": "GB/s",
               "tokens_per_s": round(S / t_med, 2), "seconds": round(t_med, 3),
               "cores": oracle.num_threads(), "kind": "oracle", **host_info(),
               "sample": f"the full workload (all {S} sequences, layer 0), pa_decode only, "
                         f"median of {args.cpu_reps} runs, fp64"}
        if args.cpu_single_reps > 0:
            prev = oracle.set_num_threads(1)
            try:
                t1 = oracle_seconds(args.cpu_single_reps)
            finally:
                oracle.set_num_threads(prev)
            cpu["single_core"] = {"value": round(dec_bytes / t1 / 1e9, 3), "unit": "GB/s",
                                  "tokens_per_s": round(S / t1, 2), "seconds": round(t1, 3),
                                  "cores": 1, "runs": args.cpu_single_reps}
        del kh, vh

    rec = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and decode tokens/s "
                  "at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[dt],
        "data": "synthetic (seeded N(0,1) K/V/q, seeded block placement and context lengths)",
        "config": {"workload": WORKLOAD_TEXT[args.workload] + (
                       f" (blocks of {B} tokens)" if B != 16 else ""), "name": args.workload,
                   "num_seqs": S, "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "num_blocks": NB, "context_tokens": int(sum(ctx)),
                   "seed": case.seed, "partition_tokens": part or "auto",
                   "partition_plan": "pa_decode_plan (host context lengths)" if planned else None,
                   "shared_blocks_hint": shared, "cascade": bool(args.cascade),
                   "append": bool(append),
                   "kernel": "valu (PA_DECODE_FORCE_VALU)" if args.force_valu else None,
                   "groups": int(pb.shape[0]), "max_group_size": int(max_group),
                   "layers_rotated": args.layers, "steps_per_graph": G},
        "tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "step_bytes": int(step_bytes),
        "decode_us": round(dec_avg * 1e3, 2),
        "decode_us_spread": dec_spread,
        "append_us": round(app_avg * 1e3, 2) if append else None,
        "decode_entry": ("pa_decode_cascade" if args.cascade
                         else "pa_decode_append" if append
                         else f"pa_decode_ex (partition_tokens {part})"
                         if part or shared or args.force_valu
                         else "pa_decode"),
        "merge": (None if args.cascade else
                  {0: "none (one partition per table)", 1: "merge kernel",
                   2: "in the partition kernel"}[
                      pa.pa_decode_merge_mode(S, Hq, Hkv, D, B, case.max_blocks, dt, part,
                                              shared_blocks=shared,
                                              force_valu=args.force_valu)]),
        "logical_bytes": int(dec_bytes),
        "unique_bytes": int(uniq_bytes),
        "write_us": round(wr_avg * 1e3, 2) if wr_avg is not None else None,
        "launch": f"HIP graph replays, {G} steps per graph (one decode iteration of a "
                  f"{G}-layer model), layer pools rotated",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": ("pa_decode_cascade (unit + merge kernels)" if args.cascade
                                else "pa_decode_append (partition kernel storing the new "
                                     "tokens + merge kernel)" if append
                                else "pa_decode (partition kernel, and the merge kernel "
                                     "where the merge is not in the partition kernel)"),
                     "bytes_per_launch": int(roof_bytes)},
        "effective_GBps": round(dec_bytes / (dec_avg * 1e-3) / 1e9, 2),
        "decode_plain": None if plain_us is None else {
            "entry": "pa_decode (automatic partitions: " + (
                "length planned on the device from the context lengths)" if device_plan
                else "the library's length for the table size)"),
            "us": round(plain_us, 2),
            "GBps": round(roof_bytes / (plain_us * 1e-6) / 1e9, 2),
            "frac_of_peak": round(roof_bytes / (plain_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)},
        # the decode's K/V loads alone (pa_read_tiles: same units, load
        # instructions and look-ahead, no arithmetic), timed the same way: the
        # ceiling of this access pattern on this machine, beside the 8 TB/s peak
        "read_ceiling": None if read_us is None else {
            "kernel": "pa_read_tiles", "us": round(read_us, 2),
            "GBps": round(dec_bytes / (read_us * 1e-6) / 1e9, 2),
            "frac_of_peak": round(dec_bytes / (read_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "decode_frac_of_ceiling": round(read_us / (dec_avg * 1e3), 4)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


def contiguous_tables(case):
    """The same sequences with each one's blocks at consecutive physical ids
    (what a contiguous KV layout would read), for the paging-overhead figure."""
    import torch
    B = case.block_size
    tables = torch.zeros_like(case.block_tables)
    nxt = 0
    for s, c in enumerate(case.context_lens.tolist()):
        nb = -(-c // B)
        tables[s, :nb] = torch.arange(nxt, nxt + nb, dtype=torch.int32)
        nxt += nb
    if nxt > case.num_blocks:
        raise ValueError("pool too small for a contiguous layout")
    return tables


def bench_prefill(args, dev):
    """A step is one layer of a prefill iteration: pa_write_kv of every new
    token's K/V into its slot, then pa_prefill.  Steps rotate over `--layers`
    pool pairs and run as HIP graph replays (one graph per pass over the
    layers).  `value` = useful causal flops of the step / step time; the
    roofline covers pa_prefill alone against the dense bf16 matrix-core peak."""
    import torch

    import paged_kv_cache_299_amd as pa
    from paged_kv_cache_299_amd import workloads
    from paged_kv_cache_299_amd.layout import kv_cache_shapes

    t_setup = time.time()
    case = workloads.CASES[args.workload](
        fill=False, **({} if args.seed is None else {"seed": args.seed}))
    Hq, Hkv, D, B, NB, dt = case.num_heads, case.num_kv_heads, case.head_dim, \
        case.block_size, case.num_blocks, case.dtype
    T, S, MQ = case.q.shape[0], case.num_seqs, case.max_query_len
    flops = workloads.prefill_flops(case)
    k_shape, v_shape = kv_cache_shapes(NB, Hkv, D, B, dt)
    gen = torch.Generator(device=dev)
    pools = []
    for layer in range(args.layers):
        gen.manual_seed(3000 + 100 * case.seed + layer)
        pools.append(tuple(torch.randn(s_, generator=gen, device=dev).to(dt)
                           for s_ in (k_shape, v_shape)))
    q = case.q.to(dev)
    bt = case.block_tables.to(dev)
    bt_contig = contiguous_tables(case).to(dev)
    cl = case.context_lens.to(dev)
    qs = case.query_start.to(dev)
    out = torch.empty_like(q)
    st = case.write_step
    k_new, v_new, slots = st.k_new.to(dev), st.v_new.to(dev), st.slot_mapping.to(dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    L = len(pools)
    stream = torch.cuda.Stream()

    def enqueue(layer, write=True, attend=True, tables=bt):
        k, v = pools[layer]
        if write:
            pa.pa_write_kv(k_new, v_new, k, v, slots)
        if attend:
            pa.pa_prefill(q, k, v, tables, cl, qs, case.scale, out, max_query_len=MQ)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            enqueue(i % L)
    torch.cuda.synchronize()

    def timed(n, **phase):
        q_, r_ = divmod(n, L)
        graphs = []
        for layers in ([range(L)] * (1 if q_ else 0)) + ([range(r_)] if r_ else []):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for l in layers:
                    enqueue(l, **phase)
            graphs.append(g)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        warm_graph(graphs[0], stream)
        with torch.cuda.stream(stream):
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(q_):
                graphs[0].replay()
            if r_:
                graphs[-1].replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1)

    wall, _ = timed(args.steps)
    ms_per_step = wall * 1e3 / args.steps
    _, pf_ms = timed(args.steps, write=False)
    _, wr_ms = timed(args.steps, attend=False)
    _, pc_ms = timed(args.steps, write=False, tables=bt_contig)
    pf_avg, wr_avg, pc_avg = pf_ms / args.steps, wr_ms / args.steps, pc_ms / args.steps
    achieved = flops / (pf_avg * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12

    cpu = None
    if args.cpu_reps > 0:
        import numpy as np
        import oracle
        k0, v0 = pools[0]
        with torch.cuda.stream(stream):
            enqueue(0)
        torch.cuda.synchronize()
        kh, vh = raw_bits(k0.cpu()), raw_bits(v0.cpu())
        # sampled rows: query i of a chunk of n is the decode of position
        # ctx - n + i over its first ctx - n + i + 1 tokens
        rng = np.random.default_rng(0)
        qs_h = case.query_start.tolist()
        rows, ctx_at, seq_of = [], [], []
        for s, (c, n) in enumerate(zip(case.context_lens.tolist(), case.query_lens)):
            for i in rng.choice(n, size=min(n, 16), replace=False).tolist():
                rows.append(qs_h[s] + i)
                ctx_at.append(c - n + i + 1)
                seq_of.append(s)
        sample_flops = 4 * D * Hq * sum(ctx_at)
        times = []
        for _ in range(args.cpu_reps):
            t = time.perf_counter()
            oracle.decode(raw_bits(case.q[rows]), kh, vh, case.block_tables.numpy()[seq_of],
                          np.array(ctx_at, np.int32), case.scale, num_kv_heads=Hkv, head_dim=D,
                          block_size=B, k_x=16 // torch.tensor([], dtype=dt).element_size(),
                          dtype=pa.DTYPE_CODES[dt])
            times.append(time.perf_counter() - t)
        t_med = statistics.median(times)
        cpu = {"value": round(sample_flops / t_med / 1e12, 6), "unit": "TFLOP/s",
               "seconds": round(t_med, 3), "cores": oracle.num_threads(), "kind": "oracle", **host_info(),
               "sample": f"{len(rows)} query rows (16 per sequence, all {Hq} heads) of layer 0, "
                         f"each over its causal prefix, median of {args.cpu_reps} runs, fp64"}
        del kh, vh

    rec = {
        "metric": "paged prefill attention: useful causal TFLOP/s at 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, seeded block placement and prompt lengths)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload,
                   "num_seqs": S, "num_tokens": T, "num_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": B, "num_blocks": NB, "seed": case.seed,
                   "max_query_len": MQ, "context_tokens": int(case.context_lens.sum()),
                   "layers_rotated": L},
        "flops_per_step": int(flops),
        "prefill_us": round(pf_avg * 1e3, 2),
        "write_us": round(wr_avg * 1e3, 2),
        "prefill_contiguous_blocks_us": round(pc_avg * 1e3, 2),
        "paging_overhead_pct": round(100 * (pf_avg / pc_avg - 1), 2),
        "launch": "HIP graph replays, one graph per pass over the rotated layers",
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "pa_prefill (prefill_mfma_kernel)",
                     "flops_per_launch": int(flops)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


def bench_vattention(args, dev):
    """The Llama-3-8B-shaped decode batch stored twice per rotated layer: on
    virtual-memory storage (VirtualKV: request slot s = sequence s, pages
    mapped for its context) and in the paged pool with the workload's block
    tables.  Both decodes run as graph replays over the layers; the paging
    overhead is paged time / table-free time - 1."""
    import torch

    import paged_kv_cache_299_amd as pa
    from paged_kv_cache_299_amd import workloads
    from paged_kv_cache_299_amd.layout import kv_cache_shapes

    t_setup = time.time()
    case = workloads.llama3_8b(fill=False, **({} if args.seed is None else {"seed": args.seed}))
    S, Hq, Hkv, D, B, NB, dt = case.num_seqs, case.num_heads, case.num_kv_heads, \
        case.head_dim, case.block_size, case.num_blocks, case.dtype
    e = 2
    ctx = case.context_lens.tolist()
    max_ctx = case.max_blocks * B
    L = args.layers
    vkv = pa.VirtualKV(L, S, max_ctx, Hkv, D, dt, page_bytes=args.page_kib * 1024)  # 0 = the library default
    reqs = [vkv.alloc_reqid() for _ in range(S)]
    lens = [0] * S
    for r, c in zip(reqs, ctx):
        lens[r] = c
    t0 = time.perf_counter()
    vkv.step(lens)
    step_ms = (time.perf_counter() - t0) * 1e3
    info = vkv.info()
    # the same tokens in both layouts
    T = int(sum(ctx))
    vslots = torch.tensor([vkv.slot(r, i) for r, c in zip(reqs, ctx) for i in range(c)],
                          dtype=torch.int64, device=dev)
    bt_np = case.block_tables.numpy()
    pslots = torch.tensor([int(bt_np[s, i // B]) * B + i % B for s in range(S)
                           for i in range(ctx[s])], dtype=torch.int64, device=dev)
    k_shape, v_shape = kv_cache_shapes(NB, Hkv, D, B, dt)
    gen = torch.Generator(device=dev)
    pools = []
    for layer in range(L):
        gen.manual_seed(4000 + layer)
        kn = torch.randn((T, Hkv, D), generator=gen, device=dev).to(dt)
        vn = torch.randn((T, Hkv, D), generator=gen, device=dev).to(dt)
        vkv.write_kv(layer, kn, vn, vslots)
        kp = torch.empty(k_shape, dtype=dt, device=dev)
        vp = torch.empty(v_shape, dtype=dt, device=dev)
        pa.pa_write_kv(kn, vn, kp, vp, pslots)
        pools.append((kp, vp))
        del kn, vn
    q = case.q.to(dev)
    req_d = torch.tensor(reqs, dtype=torch.int32, device=dev)
    bt = case.block_tables.to(dev)
    cl = case.context_lens.to(dev)
    out_v = torch.empty_like(q)
    out_p = torch.empty_like(q)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    stream = torch.cuda.Stream()

    def enqueue(layer, paged):
        if paged:
            kp, vp = pools[layer]
            pa.pa_decode(q, kp, vp, bt, cl, case.scale, out_p)
        else:
            vkv.decode(layer, q, req_d, cl, case.scale, out_v)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            enqueue(i % L, False)
            enqueue(i % L, True)
    torch.cuda.synchronize()

    def timed(n, paged):
        q_, r_ = divmod(n, L)
        graphs = []
        for layers in ([range(L)] * (1 if q_ else 0)) + ([range(r_)] if r_ else []):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for l in layers:
                    enqueue(l, paged)
            graphs.append(g)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        warm_graph(graphs[0], stream)
        with torch.cuda.stream(stream):
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(q_):
                graphs[0].replay()
            if r_:
                graphs[-1].replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1)

    wall, v_ms = timed(args.steps, paged=False)
    _, p_ms = timed(args.steps, paged=True)
    v_avg, p_avg = v_ms / args.steps, p_ms / args.steps
    ms_per_step = wall * 1e3 / args.steps
    dec_bytes = decode_bytes(ctx, S, Hq, Hkv, D, B, e) - 4 * sum(-(-c // B) for c in ctx)
    identical = bool(torch.equal(out_v.view(torch.int16), out_p.view(torch.int16)))
    achieved = dec_bytes / (v_avg * 1e-3) / 1e9
    vkv.close()

    cpu = None
    if args.cpu_reps > 0:
        import oracle
        kp, vp = pools[0]
        kh, vh = raw_bits(kp.cpu()), raw_bits(vp.cpu())
        times = []
        for _ in range(args.cpu_reps):
            t = time.perf_counter()
            oracle.decode(raw_bits(case.q), kh, vh, case.block_tables.numpy(),
                          case.context_lens.numpy(), case.scale, num_kv_heads=Hkv, head_dim=D,
                          block_size=B, k_x=8, dtype=pa.DTYPE_CODES[dt])
            times.append(time.perf_counter() - t)
        t_med = statistics.median(times)
        cpu = {"value": round(dec_bytes / t_med / 1e9, 3), "unit": "GB/s",
               "seconds": round(t_med, 3), "cores": oracle.num_threads(), "kind": "oracle", **host_info(),
               "sample": f"the full batch (all {S} sequences, layer 0's tokens), median of "
                         f"{args.cpu_reps} runs, fp64"}

    rec = {
        "metric": "decode attention on virtual-memory KV storage (no block table): achieved "
                  "HBM GB/s at 1 GPU",
        "value": round(dec_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, the Llama-3-8B-shaped batch's lengths)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload,
                   "num_seqs": S, "context_tokens": T, "max_context_len": max_ctx,
                   "page_bytes": info["page_bytes"], "layers_rotated": L, "seed": case.seed},
        "vkv_decode_us": round(v_avg * 1e3, 2),
        "paged_decode_us": round(p_avg * 1e3, 2),
        "paging_overhead_pct": round(100 * (p_avg / v_avg - 1), 2),
        "outputs_bit_identical": identical,
        "mapped_bytes": info["mapped_bytes"],
        "step_map_ms": round(step_ms, 2),
        "create_us_per_page": round(info["create_us_per_page"], 2),
        "map_us_per_page": round(info["map_us_per_page"], 2),
        "launch": "HIP graph replays, one graph per pass over the rotated layers",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "pa_vkv_decode (partition + merge kernels, no block table)",
                     "bytes_per_launch": int(dec_bytes)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


def bench_swap(args, dev):
    """Swap-out then swap-in of the preempted sequences' blocks, one layer's
    pool pair per step, rotating over `--layers` device pools and as many
    pinned host pools.  Each direction is one pa_swap_blocks launch; GPU times
    come from HIP events on the launch stream, eager launches (each step is
    two launches of tens of milliseconds).  The host-link ceiling is torch's
    DMA copy of the same number of bytes as one contiguous pinned buffer."""
    import torch

    import paged_kv_cache_299_amd as pa
    from paged_kv_cache_299_amd import workloads
    from paged_kv_cache_299_amd.layout import block_bytes, kv_cache_shapes

    t_setup = time.time()
    case = workloads.llama3_8b(fill=False, **({} if args.seed is None else {"seed": args.seed}))
    plan = workloads.swap_plan(case, num_preempted=8)
    Hkv, D, B, NB, dt = case.num_kv_heads, case.head_dim, case.block_size, case.num_blocks, \
        case.dtype
    n, NH = plan.out_map.shape[0], plan.num_host_blocks
    moved = 2 * n * block_bytes(Hkv, D, B, dt)          # K and V, one direction
    k_shape, v_shape = kv_cache_shapes(NB, Hkv, D, B, dt)
    hk_shape, hv_shape = kv_cache_shapes(NH, Hkv, D, B, dt)
    gen = torch.Generator(device=dev)
    L = args.layers
    dev_pools, host_pools = [], []
    for layer in range(L):
        gen.manual_seed(2000 + layer)
        dev_pools.append(tuple(torch.randn(s_, generator=gen, device=dev).to(dt)
                               for s_ in (k_shape, v_shape)))
        host_pools.append(tuple(torch.empty(s_, dtype=dt, pin_memory=True)
                                for s_ in (hk_shape, hv_shape)))
    out_map = plan.out_map.to(dev)
    in_map = plan.in_map.to(dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    stream = torch.cuda.Stream()

    def step(layer, direction):
        (k, v), (hk, hv) = dev_pools[layer], host_pools[layer]
        if direction == "out":
            pa.pa_swap_blocks(k, v, hk, hv, out_map, stream=stream)
        else:
            pa.pa_swap_blocks(hk, hv, k, v, in_map, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i % L, "out")
            step(i % L, "in")
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i % L, "out")
            ev[i][1].record(stream)
            step(i % L, "in")
            ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out_ms = statistics.median(a.elapsed_time(b) for a, b, _ in ev)
    in_ms = statistics.median(b.elapsed_time(c) for _, b, c in ev)
    ms_per_step = wall * 1e3 / args.steps

    # host-link ceiling: one contiguous DMA copy of the same bytes each way
    dbuf = torch.empty(moved, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    d2h, h2d = [], []
    with torch.cuda.stream(stream):
        for _ in range(5):
            e0.record(stream)
            hbuf.copy_(dbuf, non_blocking=True)
            e1.record(stream)
            dbuf.copy_(hbuf, non_blocking=True)
            e2.record(stream)
            torch.cuda.synchronize()
            d2h.append(e0.elapsed_time(e1))
            h2d.append(e1.elapsed_time(e2))
    dma_out = moved / (statistics.median(d2h) * 1e-3) / 1e9
    dma_in = moved / (statistics.median(h2d) * 1e-3) / 1e9

    cpu = None
    if args.cpu_reps > 0:
        import oracle
        (k, v), (hk, hv) = dev_pools[0], host_pools[0]
        kh, vh = raw_bits(k.cpu()), raw_bits(v.cpu())
        hkh, hvh = raw_bits(hk.clone()), raw_bits(hv.clone())
        code = pa.DTYPE_CODES[dt]
        times = []
        for _ in range(args.cpu_reps):
            t = time.perf_counter()
            oracle.swap_blocks(kh, vh, hkh, hvh, plan.out_map.numpy(), num_kv_heads=Hkv,
                               head_dim=D, block_size=B, dtype=code)
            times.append(time.perf_counter() - t)
        t_med = statistics.median(times)
        cpu = {"value": round(moved / t_med / 1e9, 3), "unit": "GB/s", "seconds": round(t_med, 4),
               "cores": 1, "kind": "oracle", **host_info(),
               "sample": f"swap-out of the same {n} blocks between host arrays (memcpy per "
                         f"block, K and V), median of {args.cpu_reps} runs"}

    out_gbps = moved / (out_ms * 1e-3) / 1e9
    in_gbps = moved / (in_ms * 1e-3) / 1e9
    value = 2 * moved / (ms_per_step * 1e-3) / 1e9
    best = max(out_gbps, in_gbps)
    rec = {
        "metric": "KV block swap between HBM and pinned host memory: GB/s moved (swap-out + "
                  "swap-in) at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) pools; the seeded Llama-3-8B-shaped batch's tables)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload,
                   "blocks": n, "bytes_per_direction": int(moved), "seed": case.seed,
                   "layers_rotated": L},
        "swap_out_ms": round(out_ms, 4),
        "swap_in_ms": round(in_ms, 4),
        "swap_out_GBps": round(out_gbps, 2),
        "swap_in_GBps": round(in_gbps, 2),
        "dma_contiguous_GBps": {"device_to_host": round(dma_out, 2),
                                "host_to_device": round(dma_in, 2)},
        "launch": "eager, one pa_swap_blocks launch per direction",
        "roofline": {"bound": "host link", "achieved": round(best, 2),
                     "peak": PEAK_HOST_LINK_GBPS, "unit": "GB/s",
                     "frac": round(best / PEAK_HOST_LINK_GBPS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel ("
                               + ("swap-out" if out_gbps >= in_gbps else "swap-in") + ")",
                     "bytes_per_launch": int(moved)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
