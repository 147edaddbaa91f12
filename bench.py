#!/usr/bin/env python3
"""Decode throughput of the 4-bit paged-KV attention on one MI355X.

Workload: B=32 sequences of 4096 tokens, Hq=32, Hk=4 (GQA-8), D=256,
block_size 16 with a shuffled block table, 32 KV splits, bf16 q/k/v ~ N(0,1)
(seeded, synthetic). One step = one full uq_decode over the resident cache:
split-KV stage 1 with the query rotation and E4M3 haircut inside it, then
the stage-2 merge (at head dims 128 and 512 a separate query prologue
first).

Metric: cache bytes streamed per step (sum_b L_b * Hk * 17 D / 16; 272 bytes
per token and KV head at D = 256) / step time, in GB/s, with the fraction of
the 8 TB/s HBM peak and tokens/s (B per step). --head-dim 128 / 512 runs the
same workload at another head dim.
The 142.6 MB cache would fit the 256 MB Infinity Cache, so steps rotate over
enough stored copies of the cache that each step reads one untouched for the
last >= 768 MB of traffic.

Timing: HIP events on the stream the kernels run on. The host first queues a
spin kernel, then a few untimed steps (the first launches after the idle spin
run slower than the steady state), then all timed steps, so the GPU runs them
back to back without waiting on Python. A second pass times each kernel
alone, as back-to-back launches, which gives the dominant kernel's duration
for the roofline.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode KV-bytes GB/s (% of HBM peak) + decode tokens/s, B=32 GQA-8 D={D} 4K ctx"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps: averages over 200 steps varied by about 5% from run to run,
    # over 1000 they repeat within 1% (about 0.1 s of timed GPU work)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    help="decode (the default line), or tiny / ragged / long / mixed; mixed times a "
                         "store of one token per sequence together with the decode; prefill times "
                         "uq_continuation_prefill (a 2048-token chunk after 4096 cached tokens)")
    ap.add_argument("--queries-per-seq", type=int, default=1,
                    help="decode this many query rows per sequence (a speculative step), each "
                         "reading its own prefix, through uq_decode_ex")
    ap.add_argument("--sliding-window", type=int, default=0,
                    help="attend to the last W tokens only (uq_decode_ex); the value counts the "
                         "cache bytes inside the window")
    ap.add_argument("--sinks", action="store_true",
                    help="add seeded per-head sink logits (uq_decode_ex)")
    ap.add_argument("--head-dim", type=int, default=256, choices=(128, 256, 512),
                    help="head dim of the workload (slot 17*D/16 bytes, scale 1/sqrt(D))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run one plain streaming kernel (int32 bitwise_not) that reads and "
                         "writes this many MiB: the reference that scales the profiler's byte "
                         "counters")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def setup(w, dev):
    import numpy as np
    import torch

    import decode_attention_bit_amd as uq
    from decode_attention_bit_amd import inputs

    lay = inputs.make_layout(w)
    q = inputs.make_query(w).to(dev)
    cache = torch.zeros((lay.num_blocks, w.block_size, w.Hk, w.slot_bytes), dtype=torch.uint8, device=dev)
    for b in range(w.B):
        k, v = inputs.make_kv(w, lay, b)
        slots = inputs.slots_for(lay, b, 0, int(lay.seq_lens[b]))
        uq.store(k.to(dev), v.to(dev), cache, torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    nbytes = cache.numel()
    reps = max(2, math.ceil(768e6 / nbytes) + 1)
    caches = [cache] + [cache.clone() for _ in range(reps - 1)]
    bt = torch.from_numpy(lay.block_table).to(dev)
    sl = torch.from_numpy(lay.seq_lens).to(dev)
    torch.cuda.synchronize()
    return lay, q, caches, bt, sl


PREROLL = 10      # untimed launches between the spin and the start event


def busy(launches=200):
    """A bounded spin kernel that keeps the GPU busy while the host queues
    `launches` calls, so that they run back to back (about 60k cycles, ~25
    us, of spin per call: more than the host needs to queue one)."""
    import torch
    torch.cuda._sleep(20_000_000 + 60_000 * launches)


def serving_store(w, lay, dev):
    """The mixed serving step also stores one new token per sequence: the
    keys and values of each sequence's last token and their slots (the cache
    already holds them, so repeating the store leaves it unchanged)."""
    import numpy as np
    import torch

    from decode_attention_bit_amd import inputs

    ks, vs, slots = [], [], []
    for b in range(w.B):
        L = int(lay.seq_lens[b])
        k, v = inputs.make_kv(w, lay, b, L - 1, L)
        ks.append(k)
        vs.append(v)
        slots.append(inputs.slots_for(lay, b, L - 1, L))
    return (torch.cat(ks).to(dev), torch.cat(vs).to(dev),
            torch.from_numpy(np.concatenate(slots)).to(dev))


def multi_query(w, lay, qps, dev):
    """qps query rows per sequence, as a speculative step verifying qps
    tokens: row i of sequence b attends to L_b - qps + 1 + i tokens through
    the sequence's block-table row. Returns the queries, the row of each
    query and its length."""
    import numpy as np
    import torch

    from decode_attention_bit_amd import inputs

    rng = np.random.default_rng([w.seed, 4])
    qm = inputs.to_bf16(rng.standard_normal((w.B * qps, w.Hq, w.D), dtype=np.float32)).to(dev)
    rows = np.repeat(np.arange(w.B), qps).astype(np.int32)
    lens = (lay.seq_lens[rows].astype(np.int64) - qps + 1 + np.tile(np.arange(qps), w.B)).astype(np.int32)
    return qm, torch.from_numpy(rows).to(dev), torch.from_numpy(lens).to(dev)


def gpu_time(w, lay, q, caches, bt, sl, steps, warmup, store_args=None, multi=None, sinks=None,
             window=0):
    import torch

    import decode_attention_bit_amd as uq

    dev = q.device
    if multi is not None:                    # query rows, their table rows, their lengths
        q, rows, sl = multi
        bt_rep = bt[rows.long()].contiguous()  # the same rows repeated, for the per-kernel pass
    nq = q.shape[0]
    out = torch.empty((nq, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(uq.decode_workspace_bytes(nq, w.Hq, w.Hk, w.num_kv_splits, bt.shape[1], w.block_size, w.D),
                     dtype=torch.uint8, device=dev)
    R = len(caches)
    args = lambda i: (q, caches[i % R], bt if multi is None else bt_rep, sl, w.scale, w.num_kv_splits)

    def step(i):
        if store_args is not None:
            uq.store(store_args[0], store_args[1], caches[i % R], store_args[2])
        if multi is None and sinks is None and not window:
            uq.decode(*args(i), out=out, workspace=ws)
        else:
            uq.decode_ex(q, caches[i % R], bt, sl, w.scale, w.num_kv_splits,
                         query_row=None if multi is None else rows, sinks=sinks, sliding_window=window,
                         out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # pass 1: whole steps. The first launches after the idle spin run slower
    # than the steady state (about 1 ms per pass in all, measured), so a few
    # untimed steps are queued between the spin and the start event.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy(steps + PREROLL)                    # keep the GPU busy while the host queues the steps
    for i in range(PREROLL):
        step(i)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps

    # pass 1b: the spread of single steps, with an event recorded between
    # consecutive steps (the events add a little to each step, so the mean of
    # this pass is not the value; its percentiles show the step's spread)
    import numpy as np
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    busy(steps + PREROLL)
    for i in range(PREROLL):
        step(i)
    evs[0].record()
    for i in range(steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    spread = {f"p{p}": round(float(np.percentile(per_step, p)), 5) for p in (10, 50, 90)}

    # pass 2: each kernel on its own, `steps` back-to-back launches between two
    # events on the decode stream, so that the average is the kernel's own
    # duration (what a kernel trace reports). Stage 1 reads the prologue's
    # query codes (the same for every cache copy) and stage 2 the partials of
    # the last stage 1, so repeating one stage is well defined.
    def alone(stage):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        busy(steps + PREROLL)
        for i in range(PREROLL):
            uq.decode(*args(i), out=out, workspace=ws, stages=stage)
        a.record()
        for i in range(steps):
            uq.decode(*args(i), out=out, workspace=ws, stages=stage)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    if multi is not None or sinks is not None or window:
        return step_ms, spread, None      # the per-kernel entry points take no options
    st = {"prologue": alone(uq.STAGE_PROLOGUE), "split_kv": alone(uq.STAGE_SPLIT),
          "merge": alone(uq.STAGE_MERGE)}
    if w.D == 256:
        # the two-launch form's stage 1, which computes the query codes itself
        st["split_kv_with_query_prologue_inside"] = alone(uq.STAGE_SPLIT | uq.STAGE_FUSED_QUERY)

    # the streaming ceiling: a plain read of exactly the blocks the step
    # reads (all KV heads of every block of every sequence, in table order),
    # back to back over the same cache copies
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy(steps + PREROLL)
    for i in range(PREROLL):
        uq.stream_blocks(caches[i % R], bt, sl, sink)
    a.record()
    for i in range(steps):
        uq.stream_blocks(caches[i % R], bt, sl, sink)
    b.record()
    torch.cuda.synchronize()
    st["stream_read"] = a.elapsed_time(b) / steps
    return step_ms, spread, st


STAGE1_SOURCE = os.path.join(ROOT, "decode_attention_bit_amd", "csrc", "uq_decode.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "stage1_decode_traffic.md")
PREFILL_SOURCE = os.path.join(ROOT, "decode_attention_bit_amd", "csrc", "uq_prefill.hip")
PREFILL_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "prefill_attention_traffic.md")


def recorded_traffic(workload, record=TRAFFIC_RECORD, source=STAGE1_SOURCE):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the reference kernel), or None
    when it holds no record for this workload or the kernel source has
    changed since the counters were taken."""
    import hashlib
    import re
    if not os.path.exists(record):
        return None
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    for m in re.finditer(r"^record: workload=(\S+) source_sha256=([0-9a-f]{64}) fetch_bytes=(\d+) "
                         r"write_bytes=(\d+)$", open(record).read(), re.M):
        if m.group(1) == workload and m.group(2) == sha:
            return int(m.group(3)) + int(m.group(4))
    return None


def cpu_baseline(w, lay, seconds, wall_cap=150.0):
    """The oracle, untuned, on a bounded sample: whole (sequence, KV head)
    decodes of this workload, on every core this process may run on, one
    (sequence, KV head) pair per thread with one BLAS thread each. Sequences
    are drawn at random; each is encoded once (untimed), then all its KV
    heads are decoded concurrently with other sequences' heads, until the
    timed decodes reach `seconds` of wall time or the whole loop `wall_cap`."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    from decode_attention_bit_amd import inputs
    from oracle import uq_oracle as O

    cores = len(os.sched_getaffinity(0))
    q_bits = inputs.bf16_bits(inputs.make_query(w))
    order = np.random.default_rng(0).permutation(w.B).tolist()
    start = time.perf_counter()
    pairs, done_bytes, elapsed = 0, 0, 0.0
    with threadpool_limits(limits=1), ThreadPoolExecutor(cores) as pool:
        while order and elapsed < seconds and time.perf_counter() - start < wall_cap:
            # encode a batch of sequences (untimed), then decode all their heads at once
            batch, order = order[:max(1, cores // max(1, w.Hk))], order[max(1, cores // max(1, w.Hk)):]
            caches = {}
            for b in batch:
                L = int(lay.seq_lens[b])
                cache = np.zeros((lay.num_blocks, w.block_size, w.Hk, w.slot_bytes), dtype=np.uint8)
                k, v = inputs.make_kv(w, lay, b)
                O.store(inputs.bf16_bits(k), inputs.bf16_bits(v), cache, inputs.slots_for(lay, b, 0, L))
                caches[b] = cache
            todo = [(b, h) for b in batch for h in range(w.Hk)]
            t = time.perf_counter()
            list(pool.map(lambda bh: O.decode(q_bits, caches[bh[0]], lay.block_table, lay.seq_lens,
                                              w.scale, pairs=[bh]), todo))
            elapsed += time.perf_counter() - t
            done_bytes += sum(int(lay.seq_lens[b]) for b in batch) * w.Hk * w.slot_bytes
            pairs += len(todo)
            log(f"cpu baseline: {pairs} pairs decoded, {elapsed:.1f} s timed")
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{pairs} whole (sequence, KV head) decodes of this workload "
                      f"({done_bytes / 1e6:.1f} MB of cache), {elapsed:.1f} s wall on {cores} threads "
                      f"(one pair per thread, one BLAS thread each), cache encoding untimed"}


# Continuation prefill: one sequence of the decode workload's shape (Hq 32,
# Hk 4, D 256 unless --head-dim 128) holding 4096 cached tokens receives a
# 2048-token chunk.
PREFILL = dict(cached=4096, q_len=2048, Hq=32, Hk=4, block_size=16, seed=7)
MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(cached, q_len, Hq, D=256):
    """QK and PV multiply-adds over the visible (query, key) pairs:
    4 * D * Hq * sum_i (cached + i + 1)."""
    return 4 * D * Hq * (q_len * cached + q_len * (q_len + 1) // 2)


def time_events(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    busy(steps + PREROLL)
    for _ in range(PREROLL):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_cpu_baseline(P, q, kc, vc, cache, row, seconds, D=256):
    """The oracle, untuned, on sampled chunk positions (every key still
    dequantised and rotated), BLAS threads on every core of this process."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from decode_attention_bit_amd import inputs
    from oracle import uq_oracle as O

    qb, kb, vb = (inputs.bf16_bits(t.cpu()) for t in (q, kc, vc))
    scale = 1.0 / math.sqrt(D)
    cache_np, row_np = cache.cpu().numpy(), row.cpu().numpy()
    rng = np.random.default_rng(0)
    cores = len(os.sched_getaffinity(0))
    done, flops, elapsed = 0, 0, 0.0
    with threadpool_limits(limits=cores):
        while elapsed < seconds and done < P["q_len"]:
            rows = rng.integers(0, P["q_len"], 4)
            t = time.perf_counter()
            O.continuation_prefill(qb, kb, vb, cache_np, row_np, P["cached"], scale, rows=rows)
            elapsed += time.perf_counter() - t
            done += len(rows)
            flops += sum(4 * D * P["Hq"] * (P["cached"] + int(i) + 1) for i in rows)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} chunk positions of this workload, each call dequantising the whole "
                      f"prefix and rotating the whole chunk, {elapsed:.1f} s, BLAS on {cores} threads"}


def copy_reference(mib, dev):
    """One int32 bitwise_not over mib MiB (reads and writes mib MiB): the kernel
    of known size that HBM byte counters are scaled by."""
    import torch
    if mib <= 0:
        return
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    log(f"reference kernel bitwise_not: {n} bytes read, {n} bytes written")
    del src, dst


def prefill_main(args):
    import numpy as np
    import torch

    import decode_attention_bit_amd as uq

    P = PREFILL
    D = args.head_dim
    scale = 1.0 / math.sqrt(D)
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(P["seed"])
    bs, Hk, Hq, cached, q_len = P["block_size"], P["Hk"], P["Hq"], P["cached"], P["q_len"]
    nblk = cached // bs
    log(f"setup prefill: {cached} cached + {q_len} chunk tokens")
    cache = torch.zeros((nblk + 64, bs, Hk, D * 17 // 16), dtype=torch.uint8, device=dev)
    row = torch.randperm(nblk + 64, generator=g)[:nblk].to(torch.int32).to(dev)
    randn = lambda *shape: torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)
    k, v = randn(cached, Hk, D), randn(cached, Hk, D)
    t = torch.arange(cached, device=dev)
    uq.store(k, v, cache, row[t // bs].long() * bs + t % bs)
    q, kc, vc = randn(q_len, Hq, D), randn(q_len, Hk, D), randn(q_len, Hk, D)
    out = torch.empty((q_len, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(uq.continuation_prefill_workspace_bytes(q_len, cached + q_len, Hq, Hk, D),
                     dtype=torch.uint8, device=dev)
    copy_reference(args.copy_ref_mib, dev)
    steps = max(1, args.steps // 4)
    warmup = max(1, args.warmup // 4)
    log(f"timing {steps} calls")
    call = lambda: uq.continuation_prefill(q, kc, vc, cache, row, cached, scale, out=out, workspace=ws)
    ms = time_events(call, steps, warmup)
    # each launch of the call alone, on the workspace the whole call left
    gather = lambda: uq.continuation_prefill(q, kc, vc, cache, row, cached, scale, out=out,
                                             workspace=ws, stages=uq.PREFILL_GATHER)
    attn = lambda: uq.continuation_prefill(q, kc, vc, cache, row, cached, scale, out=out,
                                           workspace=ws, stages=uq.PREFILL_ATTEND)
    gather_ms = time_events(gather, steps, warmup)
    attn_ms = time_events(attn, steps, warmup)
    fl = prefill_flops(cached, q_len, Hq, D)
    tf = fl / (ms * 1e-3) / 1e12
    attn_tf = fl / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": f"continuation prefill TFLOP/s (16-bit MFMA), {q_len}-token chunk after {cached} cached "
                  f"tokens, GQA-8 D={D}",
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # scores on bf16 MFMAs, P.V on fp16 MFMAs over the scaled fp16 value tiles
        "dtype": "bf16+fp16-mfma",
        "data": "synthetic",
        "config": {"workload": f"prefill: cached_len={cached} q_len={q_len} Hq={Hq} Hk={Hk} D={D} "
                               f"block_size={bs} (step = one uq_continuation_prefill)",
                   "flops_per_step": fl},
        "tokens_per_s": round(q_len / (ms * 1e-3), 1),
        "stage_ms": {"whole_call": round(ms, 5), "gather_alone": round(gather_ms, 5),
                     "attention_alone": round(attn_ms, 5)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(f"prefill-D{D}", PREFILL_TRAFFIC_RECORD, PREFILL_SOURCE),
                     "kernel": "prefill_attn512_kernel" if D == 512 else "prefill_attn_kernel",
                     "flops_per_launch": fl},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = prefill_cpu_baseline(P, q, kc, vc, cache, row, args.cpu_seconds, D)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only. Every (sequence, KV head) "
                                   "unit is independent, so the path shards across GPUs by sequence "
                                   "or by KV head with no exchange; that is not run here",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload == "prefill":
        return prefill_main(args)
    import torch

    import decode_attention_bit_amd as uq
    from decode_attention_bit_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    if args.head_dim != w.D:
        import dataclasses
        w = dataclasses.replace(w, D=args.head_dim, scale=1.0 / math.sqrt(args.head_dim))
    dev = torch.device("cuda:0")
    log(f"setup {w.name}")
    lay, q, caches, bt, sl = setup(w, dev)
    kv_bytes = inputs.kv_bytes(w, lay)
    copy_reference(args.copy_ref_mib, dev)
    log(f"timing {args.steps} steps ({len(caches)} cache copies)")
    store_args = serving_store(w, lay, dev) if w.name == "mixed" else None
    multi = multi_query(w, lay, args.queries_per_seq, dev) if args.queries_per_seq > 1 else None
    # every query row of uq_decode_ex reads its own prefix: the logical
    # bytes count each read, the value counts each cache byte once
    logical_bytes = (int(multi[2].long().sum()) * w.Hk * w.slot_bytes) if multi is not None else kv_bytes
    sinks = None
    if args.sinks:
        import numpy as np
        sinks = torch.from_numpy(np.random.default_rng([w.seed, 5]).normal(0, 2, w.Hq).astype(np.float32)).to(dev)
    if args.sliding_window > 0:             # only the window's tokens are read
        import numpy as np
        kv_bytes = int(np.minimum(lay.seq_lens.astype(np.int64), args.sliding_window).sum()) * w.Hk * w.slot_bytes
        logical_bytes = kv_bytes
    step_ms, spread, st = gpu_time(w, lay, q, caches, bt, sl, args.steps, args.warmup,
                                   store_args, multi, sinks, args.sliding_window)
    gbs = kv_bytes / (step_ms * 1e-3) / 1e9
    plain = st is not None                   # no option: stage 1 timed on its own
    st1_ms = st["split_kv"] if plain else None
    st1_gbs = kv_bytes / ((st1_ms if plain else step_ms) * 1e-3) / 1e9
    parts = uq.decode_partials(w.B, w.Hq, w.Hk, w.num_kv_splits, bt.shape[1], w.block_size, w.D)
    res = {
        "metric": METRIC.format(D=w.D),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xe4m3-mfma+bf16-mfma",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} Hq={w.Hq} Hk={w.Hk} D={w.D} "
                               f"seq_len={int(lay.seq_lens.max())} block_size={w.block_size} "
                               f"num_kv_splits={w.num_kv_splits}"
                               + (" (step = store of one token per sequence + decode)"
                                  if store_args is not None else "")
                               + (f" ({args.queries_per_seq} query rows per sequence, "
                                  f"uq_decode_ex)" if multi is not None else "")
                               + (f" (sliding window {args.sliding_window})" if args.sliding_window > 0 else "")
                               + (" (with sinks)" if sinks is not None else ""),
                   "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "D": w.D, "block_size": w.block_size,
                   "num_kv_splits": w.num_kv_splits, "partials_per_row": parts,
                   "kv_bytes_per_step": kv_bytes, "logical_kv_bytes_per_step": logical_bytes},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B * max(1, args.queries_per_seq) / (step_ms * 1e-3), 1),
        "step_ms_spread": spread,
        "timing": "HIP events around back-to-back steps queued ahead of the GPU behind a spin kernel: "
                  "device time per step, host launch cost excluded",
        "stage_ms": ({k: round(v, 5) for k, v in st.items() if k != "stream_read"} if plain else None),
        "cache_copies": len(caches),
        "stream_ceiling": ({"value": round(kv_bytes / (st["stream_read"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                            "ms": round(st["stream_read"], 5),
                            "what": "uq_stream_blocks: plain 16-byte reads of exactly the blocks the step "
                                    "reads, in table order, same run"} if plain else None),
        "pct_of_stream": (round(100 * st["stream_read"] / step_ms, 2) if plain else None),
        "roofline": {"bound": "hbm", "achieved": round(st1_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(st1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name) if plain and store_args is None and w.D == 256 else None,
                     "kernel": "stage1_kernel (split-KV)" if plain else "the whole step (options on)",
                     "bytes_per_launch": kv_bytes},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(w, lay, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
