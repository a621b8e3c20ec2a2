"""Benchmark of the paged decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gqa|prefix|long|fanout|prefill]

A step is one pass of the whole hot path over one batch of synthetic
requests: ``pa_decode_step``, which makes each request's copy-on-write copy
(only the fan-out workload has any), writes its newest token at its slot
and runs decode attention over every request's paged history.  Inputs are resident in HBM
before timing starts.  Steps cycle through R replicas of the batch placed
at disjoint physical blocks, so the 256 MB Infinity Cache cannot hold the
working set between steps (every replica holds the same bytes, so every
replica gives bit-identical outputs; the benchmark checks that).

Prints one JSON line.  ``value`` is KV GB/s: algorithmic bytes of a step
(distinct KV bytes read by decode + q/out/table/length bytes + the KV write
and copy bytes) per second.  ``roofline`` is for the decode call, timed on
its own with HIP events on the stream it runs on.  ``cpu_baseline`` times
the CPU oracle on the same workload (first requests until ~10 s of work).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_kv_cache_252_amd import inputs, ops  # noqa: E402

METRIC = "paged decode attn: KV GB/s (% HBM peak) + decode tokens/s, 1x MI355X"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "gqa": dict(make=inputs.gqa, replicas=8,
                desc="GQA decode: 32 requests, context U[512,4096], 32 q / 8 KV heads, "
                     "head_dim 128, block 16, bf16, blocks shuffled in a 65536-block pool"),
    "prefix": dict(make=inputs.shared_prefix, replicas=4, runs=True,
                   desc="shared prefix: 256 requests, first 2048 tokens in the same 128 blocks, "
                        "private suffix U[64,512], 32 q / 8 KV heads, head_dim 128, block 16, bf16"),
    "long": dict(make=inputs.long_context, replicas=1,
                 desc="long context: 8 requests, context U[32768,131072], 64 q / 8 KV heads, "
                      "head_dim 128, block 16, bf16, pool sized to fit"),
    "prefill": dict(make=inputs.prefill_chunk, replicas=4,
                    desc="chunked prefill after a prefix-cache hit: 16 requests, U[1024,3072] "
                         "cached positions + 256 new query tokens each attending causally, "
                         "32 q / 8 KV heads, head_dim 128, block 16, bf16"),
    "fanout": dict(make=inputs.fanout, replicas=1,
                   desc="fan-out step: 128 prompts x 4 branches, prompt U[256,2048] with a "
                        "partial last block, copy-on-write of that block per branch, one new "
                        "token per branch, 32 q / 8 KV heads, head_dim 128, block 16, bf16"),
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def unique_kv_tokens(tables: np.ndarray, lens: np.ndarray, bs: int) -> int:
    """Distinct cached positions decode reads: per physical block, the most
    positions any request reads from it."""
    best = {}
    for t, L in zip(tables, lens):
        L = int(L)
        for j in range(-(-L // bs)):
            n = min(bs, L - j * bs)
            b = int(t[j])
            if best.get(b, 0) < n:
                best[b] = n
    return sum(best.values())


def decode_bytes(w) -> dict:
    """Algorithmic bytes of one decode call."""
    e = 2 if w.dtype == "bf16" else 4
    tables = w.block_tables.cpu().numpy()
    lens = w.context_lens.cpu().numpy()
    per_tok = w.num_kv_heads * w.head_dim * 2 * e          # K + V of one position
    uniq = unique_kv_tokens(tables, lens, w.block_size) * per_tok
    logical = int(lens.sum()) * per_tok
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * e   # q read + out written
    meta = 4 * sum(-(-int(L) // w.block_size) for L in lens) + 4 * w.num_seqs
    return dict(unique=uniq + qo + meta, logical=logical + qo + meta, kv_unique=uniq,
                kv_logical=logical)


def step_extra_bytes(w) -> int:
    """Algorithmic bytes of the KV write (read new K/V, write them, read slots)
    and of the block copies (read + write whole blocks)."""
    e = 2 if w.dtype == "bf16" else 4
    t = w.new_k.shape[0] if w.new_k is not None else 0
    write = 2 * 2 * t * w.num_kv_heads * w.head_dim * e + 8 * t
    pairs = w.cow_pairs.shape[0] if w.cow_pairs is not None else 0
    copy = pairs * (2 * 2 * w.block_elems * e + 16)
    return write + copy


def cpu_baseline(w, budget_s: float = 10.0) -> dict:
    """The CPU oracle as it stands, on the first requests of the workload."""
    from oracle import paged
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        threads = 1

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    bt = host(w.block_tables)
    lens = host(w.context_lens)
    used = np.unique(bt[bt >= 0])
    if w.cow_pairs is not None:
        used = np.union1d(used, host(w.cow_pairs)[:, 0])
    sel = torch.as_tensor(used, device=w.k_cache.device)
    kp, vp = host(w.k_cache[sel]), host(w.v_cache[sel])       # compact pool of used blocks
    remap = np.full(w.num_blocks, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    bt_c = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1)
    q = host(w.q)
    args = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim,
                dtype=w.dtype)
    new_k = host(w.new_k) if w.new_k is not None else None
    new_v = host(w.new_v) if w.new_v is not None else None
    pairs = remap[host(w.cow_pairs)] if w.cow_pairs is not None else None
    e = 2 if w.dtype == "bf16" else 4
    per_tok = w.num_kv_heads * w.head_dim * 2 * e
    done, kv_bytes, total = 0, 0, 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < budget_s:      # whole passes repeat until the budget
        if done == w.num_seqs:
            done = 0
        n = min(w.num_seqs - done, max(1, w.num_seqs // 8))
        rows = slice(done, done + n)
        k_use, v_use = kp, vp
        if pairs is not None:
            k_use, v_use = paged.copy_blocks(k_use, v_use, pairs[rows])
        if new_k is not None:
            slots = paged.slot_mapping(bt_c, np.arange(done, done + n), lens[rows] - 1,
                                       w.block_size)
            k_use, v_use = paged.write_kv(k_use, v_use, new_k[rows], new_v[rows], slots, **args)
        paged.decode(q[rows], k_use, v_use, bt_c[rows], lens[rows], w.scale, **args)
        kv_bytes += int(lens[rows].sum()) * per_tok
        done += n
        total += n
    dt = time.perf_counter() - t0
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{total} request decodes ({total / w.num_seqs:.2f} passes over the "
                      f"{w.num_seqs} requests of {w.name}, in chunks of "
                      f"{max(1, w.num_seqs // 8)}): copy/write for those requests then fp64 "
                      f"decode, {dt:.2f} s",
            "tokens_per_s": total / dt, "seconds": dt}


def measured_traffic(workload: str, part: int, stream_kv: bool):
    """HBM bytes per decode call from the committed counter summary, or None when
    there is none for this workload or the decode sources have changed since."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if (sources_digest(rec["sources"]) != rec["sources_sha256"] or rec["partition_tokens"] != part
            or rec["stream_kv"] != stream_kv):
        return None
    return int(rec["traffic_bytes_per_launch"])


def sources_digest(paths) -> str:
    """sha256 over the given source files, in order (the decode kernel's)."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(w) -> int:
    """Matrix flops of one pa_prefill call: per query row and query head, 2*D
    for the scores and 2*D for the values, times the positions it sees."""
    lens = w.context_lens.cpu().numpy()
    qs = w.q_start.cpu().numpy()
    vis = 0
    for i in range(w.num_seqs):
        n = int(qs[i + 1] - qs[i])
        L = int(lens[i])
        vis += sum(max(L - n + j + 1, 0) for j in range(n))
    return 4 * w.head_dim * w.num_q_heads * vis


def cpu_baseline_prefill(w, budget_s: float = 10.0) -> dict:
    """The CPU oracle's prefill on the first query rows of the first request."""
    from oracle import paged
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        threads = 1

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    bt = host(w.block_tables[:1])
    L = int(w.context_lens[0])
    n = int(w.q_start[1] - w.q_start[0])
    used = np.unique(bt[bt >= 0])
    sel = torch.as_tensor(used, device=w.k_cache.device)
    kp, vp = host(w.k_cache[sel]), host(w.v_cache[sel])
    remap = np.full(w.num_blocks, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    bt_c = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1)
    q = host(w.q_chunk[:n])
    args = dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim,
                dtype=w.dtype)
    done, flops = 0, 0
    t0 = time.perf_counter()
    while done < n and (time.perf_counter() - t0) < budget_s:
        k = min(16, n - done)
        # rows done .. done+k-1 of the chunk, as a chunk of their own ending at their last position
        paged.prefill(q[done:done + k], [0, k], kp, vp, bt_c, [L - n + done + k], w.scale, **args)
        flops += 4 * w.head_dim * w.num_q_heads * sum(L - n + j + 1 for j in range(done, done + k))
        done += k
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done} of {n} query rows of request 0 (context {L}), fp64, {dt:.2f} s",
            "seconds": dt}


def run_prefill(args, dev, copy_gbs) -> int:
    """``--workload prefill``: a step writes each request's new chunk of K/V
    (pa_write_kv) and runs pa_prefill for the chunk's queries."""
    cfg = WORKLOADS["prefill"]
    log("generating prefill")
    w = cfg["make"](device=dev, poison=False)
    spec = ops.CacheSpec.of(w)
    reps = args.replicas or cfg["replicas"]
    tables = inputs.replicate(w, reps) if reps > 1 else [w.block_tables]
    max_len = w.max_context_len
    qs = w.q_start.cpu().numpy()
    lens = w.context_lens.cpu().numpy()
    seq_ids, pos = [], []
    for i in range(w.num_seqs):
        n = int(qs[i + 1] - qs[i])
        seq_ids += [i] * n
        pos += list(range(int(lens[i]) - n, int(lens[i])))
    seq_ids = torch.as_tensor(seq_ids, dtype=torch.int32, device=dev)
    pos = torch.as_tensor(pos, dtype=torch.int32, device=dev)
    slots = [ops.slot_mapping(w.block_size, t, pos, seq_ids) for t in tables]
    total_q = w.q_chunk.shape[0]
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    k_new = torch.randn((total_q, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(w.k_cache.dtype)
    v_new = torch.randn((total_q, w.num_kv_heads, w.head_dim), generator=gen, device=dev).to(w.k_cache.dtype)
    part = args.partition
    need = ops.prefill_workspace_bytes(spec, w.num_seqs, total_q, w.max_q_len, w.num_q_heads,
                                       max_len, part)
    workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(w.q_chunk) for _ in tables]
    log(f"{w.num_seqs} requests, {total_q} query rows, max len {max_len}, workspace {need} B, "
        f"{reps} replicas")

    def attend(r):
        ops.prefill(spec, w.q_chunk, w.q_start, w.k_cache, w.v_cache, tables[r], w.context_lens,
                    w.max_q_len, max_len, w.scale, out=outs[r], workspace=workspace,
                    partition_tokens=part)

    def step(r):
        ops.write_kv(spec, w.k_cache, w.v_cache, k_new, v_new, slots[r])
        attend(r)

    for i in range(args.warmup):
        step(i % reps)
    for r in range(reps):
        step(r)
    torch.cuda.synchronize()
    for r in range(1, reps):
        if not torch.equal(outs[r].view(torch.int16), outs[0].view(torch.int16)):
            log("replica outputs differ")
            return 1
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % reps)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.kernel_iters):
        attend(i % reps)
    ev1.record(stream)
    ev1.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / args.kernel_iters
    flops = prefill_flops(w)
    db = decode_bytes(w)
    e = 2
    qo = 2 * total_q * w.num_q_heads * w.head_dim * e
    write = 2 * 2 * total_q * w.num_kv_heads * w.head_dim * e + 8 * total_q
    step_bytes = db["kv_unique"] + qo + write
    tflops = flops / (us * 1e-6) / 1e12
    line = {
        "metric": METRIC,
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": cfg["desc"], "name": "prefill", "requests": w.num_seqs,
                   "query_rows": total_q, "max_context_len": max_len, "replicas": reps,
                   "partition_tokens": part},
        "tokens_per_s": round(total_q / (ms * 1e-3), 1),
        "copy_probe_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_prefill", "flops_per_launch": flops,
                     "kv_bytes_per_launch": db["kv_unique"], "avg_launch_us": round(us, 3),
                     "kv_gbs": round(db["kv_unique"] / (us * 1e-6) / 1e9, 2)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(line), flush=True)
    return 0


def copy_probe(dev, mib: int) -> float:
    """Read+write GB/s of a plain device-to-device copy of ``mib`` MiB."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbs = 2 * 3 * (mib << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--partition", type=int, default=0, help="decode partition tokens (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-runs", action="store_true",
                    help="shared prefix: no cooperative shared partitions (PA_DECODE_PREFIX_RUNS off)")
    ap.add_argument("--no-group", action="store_true",
                    help="decode shared-prefix batches one request per wave")
    ap.add_argument("--stream-kv", choices=("auto", "on", "off"), default="auto",
                    help="non-temporal K/V loads: auto = on, except for shared blocks "
                         "decoded one request per wave (--no-group), whose repeat reads "
                         "must hit the caches")
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of a plain device-to-device copy timed first, as context and "
                         "as the known-size reference for traffic counters (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged decode path here runs on a single "
              "MI355X with no collectives; run it with --gpus 1.", file=sys.stderr, flush=True)
        return 2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbs = copy_probe(dev, args.copy_probe_mib) if args.copy_probe_mib > 0 else None
    if args.workload == "prefill":
        return run_prefill(args, dev, copy_gbs)
    cfg = WORKLOADS[args.workload]
    log(f"generating {args.workload}")
    w = cfg["make"](device=dev, poison=False)
    if w.new_k is None:
        inputs.add_step_tokens(w)
    spec = ops.CacheSpec.of(w)
    reps = args.replicas or cfg["replicas"]
    tables = inputs.replicate(w, reps) if reps > 1 else [w.block_tables]
    # every request appends one token at its last position, L-1
    assert torch.equal(w.new_pos, w.context_lens - 1) and torch.equal(
        w.new_seq, torch.arange(w.num_seqs, dtype=torch.int32, device=dev))
    max_len = w.max_context_len
    part = args.partition or ops.decode_partition_tokens(spec, w.num_seqs, w.num_q_heads, max_len)
    ws_bytes = ops.decode_workspace_bytes(spec, w.num_seqs, w.num_q_heads, max_len, part)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(w.q) for _ in tables]
    # sharers are consecutive requests: decode them together (each shared
    # block is then read once per group) and stream K/V
    group_shared = w.shared_blocks is not None and not args.no_group
    # one prefix shared by the whole batch: shared partitions decoded once per
    # chunk of requests (PA_DECODE_PREFIX_RUNS)
    prefix_runs = group_shared and cfg.get("runs", False) and not args.no_runs
    stream_kv = {"on": True, "off": False}.get(args.stream_kv,
                                                w.shared_blocks is None or group_shared)
    log(f"{w.num_seqs} requests, max len {max_len}, partition {part} tokens, "
        f"workspace {ws_bytes} B, {reps} replicas")

    cow_src = None
    if w.cow_pairs is not None:
        # the step's copy-on-write pairs given per request: the source of the
        # copy into the block that holds the request's newest position
        by_dst = {int(d): int(s_) for s_, d in w.cow_pairs.cpu().numpy()}
        bt0, lens0 = tables[0].cpu().numpy(), w.context_lens.cpu().numpy()
        src = [by_dst.get(int(bt0[i, (int(lens0[i]) - 1) // w.block_size]), -1)
               for i in range(w.num_seqs)]
        if reps > 1 or sum(x >= 0 for x in src) != w.cow_pairs.shape[0]:
            log("copy-on-write pairs do not map one per request")
            return 1
        cow_src = torch.as_tensor(src, dtype=torch.int32, device=dev)

    def step(r: int) -> None:
        # one call: each request's copy-on-write copy (fan-out only), the
        # append of its new token at position L-1, and decode (pa_decode_step)
        ops.decode_step(spec, w.q, w.k_cache, w.v_cache, w.new_k, w.new_v, cow_src, tables[r],
                        w.context_lens, max_len, w.scale, out=outs[r], workspace=workspace,
                        partition_tokens=part, stream_kv=stream_kv, group_shared=group_shared,
                        prefix_runs=prefix_runs)

    for i in range(args.warmup):
        step(i % reps)
    torch.cuda.synchronize()
    # every replica holds the same bytes: outputs must agree bit for bit
    for r in range(reps):
        step(r)
    torch.cuda.synchronize()
    for r in range(1, reps):
        if not torch.equal(outs[r].view(torch.int16), outs[0].view(torch.int16)):
            log("replica outputs differ")
            return 1

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % reps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # the dominant kernel: decode alone, HIP events on the stream it runs on
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.kernel_iters):
        r = i % reps
        ops.decode(spec, w.q, w.k_cache, w.v_cache, tables[r], w.context_lens, max_len, w.scale,
                   out=outs[r], workspace=workspace, partition_tokens=part, stream_kv=stream_kv,
                   group_shared=group_shared, prefix_runs=prefix_runs)
    ev1.record(stream)
    ev1.synchronize()
    dec_us = ev0.elapsed_time(ev1) * 1e3 / args.kernel_iters

    db = decode_bytes(w)
    step_bytes = db["unique"] + step_extra_bytes(w)
    value = step_bytes / (ms * 1e-3) / 1e9
    achieved = db["unique"] / (dec_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": cfg["desc"], "name": args.workload, "requests": w.num_seqs,
                   "max_context_len": max_len, "total_context_tokens": int(w.context_lens.sum()),
                   "replicas": reps, "partition_tokens": part, "stream_kv": stream_kv,
                   "group_shared": group_shared, "prefix_runs": prefix_runs,
                   "kv_layout": "one buffer [block][K|V], block_stride 2 blocks"},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w.num_seqs / (ms * 1e-3), 1),
        "kv_gbs_logical": round((db["logical"] + step_extra_bytes(w)) / (ms * 1e-3) / 1e9, 2),
        "copy_probe_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, part, stream_kv),
                     "kernel": "pa_decode", "bytes_per_launch": db["unique"],
                     "avg_launch_us": round(dec_us, 3)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
