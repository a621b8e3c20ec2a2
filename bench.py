"""Benchmark of the paged decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gqa|prefix|long|fanout|prefill|...]
                    [--extra prefix,long,fanout,prefill,...|none]

A step is one pass of the whole hot path over one batch of synthetic
requests: ``pa_decode_step``, which makes each request's copy-on-write copy
(only the fan-out workload has any), writes its newest token at its slot
and runs decode attention over every request's paged history.  Inputs are resident in HBM
before timing starts.  Steps cycle through R replicas of the batch placed
at disjoint physical blocks, so the 256 MB Infinity Cache cannot hold the
working set between steps (every replica holds the same bytes, so every
replica gives bit-identical outputs; the benchmark checks that).

Prints one JSON line for the headline workload (``--workload``, GQA decode
by default).  ``value`` is KV GB/s: algorithmic bytes of a step (distinct
KV bytes read by decode + q/out/table/length bytes + the KV write and copy
bytes) per second.  ``roofline`` is for the decode call, timed on its own
with HIP events on the stream it runs on.  ``cpu_baseline`` times the CPU
oracle on the same workload (first requests until ~10 s of work).  The
same line carries ``workloads``: every other workload (``--extra``),
measured the same way in the same run, each with a shorter oracle sample.
"""

from __future__ import annotations

import argparse
import functools
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
    "gqa_d64": dict(make=inputs.gqa_d64, replicas=8,
                    desc="GQA decode at head_dim 64: 32 requests, context U[512,4096], "
                         "32 q / 8 KV heads, block 16, bf16, blocks shuffled in a 65536-block pool"),
    "gqa_d256": dict(make=inputs.gqa_d256, replicas=8,
                     desc="GQA decode at head_dim 256: 32 requests, context U[512,4096], "
                          "32 q / 8 KV heads, block 16, bf16, blocks shuffled in a 65536-block pool"),
    "gqa_f32": dict(make=inputs.gqa_f32, replicas=8,
                    desc="GQA decode on an fp32 cache: 32 requests, context U[512,4096], "
                         "32 q / 8 KV heads, head_dim 128, block 16, blocks shuffled in a 65536-block pool"),
    "prefix": dict(make=inputs.shared_prefix, replicas=4, runs=True,
                   desc="shared prefix: 256 requests, first 2048 tokens in the same 128 blocks, "
                        "private suffix U[64,512], 32 q / 8 KV heads, head_dim 128, block 16, bf16"),
    "long": dict(make=inputs.long_context, replicas=1,
                 desc="long context: 8 requests, context U[32768,131072], 64 q / 8 KV heads, "
                      "head_dim 128, block 16, bf16, pool sized to fit"),
    "prefill": dict(make=inputs.prefill_chunk, replicas=4, prefill=True,
                    desc="chunked prefill after a prefix-cache hit: 16 requests, U[1024,3072] "
                         "cached positions + 256 new query tokens each attending causally, "
                         "32 q / 8 KV heads, head_dim 128, block 16, bf16"),
    "prefill_d64": dict(make=functools.partial(inputs.prefill_chunk, head_dim=64), replicas=4,
                        prefill=True,
                        desc="chunked prefill at head_dim 64: 16 requests, U[1024,3072] cached "
                             "positions + 256 new query tokens each attending causally, "
                             "32 q / 8 KV heads, block 16, bf16"),
    "prefill_d256": dict(make=functools.partial(inputs.prefill_chunk, head_dim=256), replicas=4,
                         prefill=True,
                         desc="chunked prefill at head_dim 256: 16 requests, U[1024,3072] cached "
                              "positions + 256 new query tokens each attending causally, "
                              "32 q / 8 KV heads, block 16, bf16"),
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


def host(t):
    """A host numpy copy of a tensor; bf16 as its raw uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def host_cores() -> dict:
    """The host cores this process may run on, and the BLAS threads numpy uses."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        blas = None
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": blas}


def cpu_baseline(w, budget_s: float = 10.0) -> dict:
    """The CPU oracle as it stands, on the first requests of the workload."""
    from oracle import paged

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
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", **host_cores(), "kind": "oracle",
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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **host_cores(), "kind": "oracle",
            "sample": f"first {done} of {n} query rows of request 0 (context {L}), fp64, {dt:.2f} s",
            "seconds": dt}


def launch_flags(name: str, w, no_group: bool = False, no_runs: bool = False,
                 stream: str = "auto") -> dict:
    """The decode flags a workload is timed with.

    Sharers are consecutive requests: decode them together (each shared block
    is then read once per group) and stream K/V.  One prefix shared by the
    whole batch: shared partitions decoded once per chunk of requests.
    """
    group_shared = w.shared_blocks is not None and not no_group
    prefix_runs = group_shared and WORKLOADS[name].get("runs", False) and not no_runs
    stream_kv = {"on": True, "off": False}.get(stream, w.shared_blocks is None or group_shared)
    return dict(stream_kv=stream_kv, group_shared=group_shared, prefix_runs=prefix_runs)


def cow_sources(w, table):
    """Per request, the source block of the copy-on-write copy into the block
    that holds its newest position (-1 = none), from the workload's pairs;
    None when the workload has no pairs."""
    if w.cow_pairs is None:
        return None
    by_dst = {int(d): int(s_) for s_, d in w.cow_pairs.cpu().numpy()}
    bt, lens = table.cpu().numpy(), w.context_lens.cpu().numpy()
    src = [by_dst.get(int(bt[i, (int(lens[i]) - 1) // w.block_size]), -1) if int(lens[i]) else -1
           for i in range(w.num_seqs)]
    if sum(x >= 0 for x in src) != w.cow_pairs.shape[0]:
        raise ValueError("copy-on-write pairs do not map one per request")
    return torch.as_tensor(src, dtype=torch.int32, device=w.q.device)


def time_calls(fn, iters: int, reps: int, dev) -> float:
    """Mean microseconds of ``fn(r)`` over ``iters`` back-to-back calls (r
    cycling over the replicas), from HIP events on the stream the library
    launches on (torch's current stream)."""
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(iters):
        fn(i % reps)
    ev1.record(stream)
    ev1.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / iters


def time_steps(fn, steps: int, reps: int) -> float:
    """Milliseconds per step by the host clock, synchronised on both sides."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i % reps)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def measure_decode(name: str, args, dev, replicas: int, partition: int, cpu_budget: float,
                   no_group=False, no_runs=False, stream="auto") -> dict:
    """Generate one decode workload, time its step and its decode call."""
    cfg = WORKLOADS[name]
    log(f"generating {name}")
    w = cfg["make"](device=dev, poison=False)
    if w.new_k is None:
        inputs.add_step_tokens(w)
    spec = ops.CacheSpec.of(w)
    reps = replicas or cfg["replicas"]
    tables = inputs.replicate(w, reps) if reps > 1 else [w.block_tables]
    # every request appends one token at its last position, L-1
    assert torch.equal(w.new_pos, w.context_lens - 1) and torch.equal(
        w.new_seq, torch.arange(w.num_seqs, dtype=torch.int32, device=dev))
    max_len = w.max_context_len
    part = partition or ops.decode_partition_tokens(spec, w.num_seqs, w.num_q_heads, max_len)
    ws_bytes = ops.decode_workspace_bytes(spec, w.num_seqs, w.num_q_heads, max_len, part)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(w.q) for _ in tables]
    flags = launch_flags(name, w, no_group, no_runs, stream)
    log(f"{name}: {w.num_seqs} requests, max len {max_len}, partition {part} tokens, "
        f"workspace {ws_bytes} B, {reps} replicas, flags {flags}")
    if reps > 1 and w.cow_pairs is not None:
        raise ValueError("copy-on-write workloads run with one replica")
    cow_src = cow_sources(w, tables[0])

    def step(r: int) -> None:
        # one call: each request's copy-on-write copy (fan-out only), the
        # append of its new token at position L-1, and decode (pa_decode_step)
        ops.decode_step(spec, w.q, w.k_cache, w.v_cache, w.new_k, w.new_v, cow_src, tables[r],
                        w.context_lens, max_len, w.scale, out=outs[r], workspace=workspace,
                        partition_tokens=part, **flags)

    def decode(r: int) -> None:
        ops.decode(spec, w.q, w.k_cache, w.v_cache, tables[r], w.context_lens, max_len, w.scale,
                   out=outs[r], workspace=workspace, partition_tokens=part, **flags)

    for i in range(args.warmup):
        step(i % reps)
    # every replica holds the same bytes: outputs must agree bit for bit
    for r in range(reps):
        step(r)
    torch.cuda.synchronize()
    for r in range(1, reps):
        if not torch.equal(outs[r].view(torch.int16), outs[0].view(torch.int16)):
            raise RuntimeError(f"{name}: replica outputs differ")
    log(f"{name}: timing {args.steps} steps")
    ms = time_steps(step, args.steps, reps)
    # the dominant kernel: decode alone, HIP events on the stream it runs on
    dec_us = time_calls(decode, args.kernel_iters, reps, dev)
    # the step once more by HIP events (its kernel time without host gaps)
    step_us = time_calls(step, args.kernel_iters, reps, dev)
    db = decode_bytes(w)
    extra = step_extra_bytes(w)
    res = {
        "name": name, "desc": cfg["desc"], "w": w, "reps": reps, "part": part, "flags": flags,
        "ms_per_step": ms, "decode_us": dec_us, "step_event_us": step_us, "bytes": db,
        "step_bytes": db["unique"] + extra, "step_bytes_logical": db["logical"] + extra,
        "traffic": measured_traffic(name, part, flags["stream_kv"]),
    }
    if cpu_budget > 0:
        log(f"{name}: timing the CPU oracle ({cpu_budget:.0f} s budget)")
        res["cpu_baseline"] = cpu_baseline(w, cpu_budget)
    del outs, workspace, tables
    return res


def measure_prefill(name, args, dev, replicas: int, partition: int, cpu_budget: float) -> dict:
    """A prefill step writes each request's new chunk of K/V (pa_write_kv) and
    runs pa_prefill for the chunk's queries."""
    cfg = WORKLOADS[name]
    log(f"generating {name}")
    w = cfg["make"](device=dev, poison=False)
    spec = ops.CacheSpec.of(w)
    reps = replicas or cfg["replicas"]
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
    part = partition
    need = ops.prefill_workspace_bytes(spec, w.num_seqs, total_q, w.max_q_len, w.num_q_heads,
                                       max_len, part)
    workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(w.q_chunk) for _ in tables]
    log(f"{name}: {w.num_seqs} requests, {total_q} query rows, max len {max_len}, "
        f"workspace {need} B, {reps} replicas")

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
            raise RuntimeError(f"{name}: replica outputs differ")
    log(f"{name}: timing {args.steps} steps")
    ms = time_steps(step, args.steps, reps)
    us = time_calls(attend, args.kernel_iters, reps, dev)
    flops = prefill_flops(w)
    db = decode_bytes(w)
    e = 2
    qo = 2 * total_q * w.num_q_heads * w.head_dim * e
    write = 2 * 2 * total_q * w.num_kv_heads * w.head_dim * e + 8 * total_q
    res = {"name": name, "prefill": True, "desc": cfg["desc"], "w": w, "reps": reps, "part": part,
           "ms_per_step": ms, "prefill_us": us, "flops": flops, "kv_unique": db["kv_unique"],
           "step_bytes": db["kv_unique"] + qo + write, "total_q": total_q}
    if cpu_budget > 0:
        log(f"{name}: timing the CPU oracle ({cpu_budget:.0f} s budget)")
        res["cpu_baseline"] = cpu_baseline_prefill(w, cpu_budget)
    del outs, workspace, tables
    return res


def decode_line(r: dict, args, copy_gbs) -> dict:
    """The JSON line of a decode workload measured by ``measure_decode``."""
    w, db, ms = r["w"], r["bytes"], r["ms_per_step"]
    value = r["step_bytes"] / (ms * 1e-3) / 1e9
    achieved = db["unique"] / (r["decode_us"] * 1e-6) / 1e9
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
        "config": {"workload": r["desc"], "name": r["name"], "requests": w.num_seqs,
                   "max_context_len": w.max_context_len,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "replicas": r["reps"], "partition_tokens": r["part"], **r["flags"],
                   "kv_layout": "one buffer [block][K|V], block_stride 2 blocks"},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w.num_seqs / (ms * 1e-3), 1),
        "kv_gbs_logical": round(r["step_bytes_logical"] / (ms * 1e-3) / 1e9, 2),
        "step_event_us": round(r["step_event_us"], 3),
        "copy_probe_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": r["traffic"], "kernel": "pa_decode",
                     "bytes_per_launch": db["unique"], "avg_launch_us": round(r["decode_us"], 3)},
    }
    if "cpu_baseline" in r:
        line["cpu_baseline"] = r["cpu_baseline"]
    return line


def prefill_line(r: dict, args, copy_gbs) -> dict:
    """The JSON line of the prefill workload measured by ``measure_prefill``."""
    w, ms, us = r["w"], r["ms_per_step"], r["prefill_us"]
    tflops = r["flops"] / (us * 1e-6) / 1e12
    line = {
        "metric": METRIC,
        "value": round(r["step_bytes"] / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": r["desc"], "name": r["name"], "requests": w.num_seqs,
                   "query_rows": r["total_q"], "max_context_len": w.max_context_len,
                   "replicas": r["reps"], "partition_tokens": r["part"]},
        "tokens_per_s": round(r["total_q"] / (ms * 1e-3), 1),
        "copy_probe_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "pa_prefill", "flops_per_launch": r["flops"],
                     "kv_bytes_per_launch": r["kv_unique"], "avg_launch_us": round(us, 3),
                     "kv_gbs": round(r["kv_unique"] / (us * 1e-6) / 1e9, 2)},
    }
    if "cpu_baseline" in r:
        line["cpu_baseline"] = r["cpu_baseline"]
    return line


def workload_entry(r: dict) -> dict:
    """The compact record of one extra workload for the ``workloads`` object."""
    w, ms = r["w"], r["ms_per_step"]
    if r.get("prefill"):
        us = r["prefill_us"]
        tflops = r["flops"] / (us * 1e-6) / 1e12
        e = {"workload": r["desc"], "prefill_us": round(us, 3), "step_us": round(ms * 1e3, 3),
             "tflops": round(tflops, 2), "roofline": {"bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS,
                                                      "unit": "TFLOP/s",
                                                      "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
             "kv_gbs": round(r["kv_unique"] / (us * 1e-6) / 1e9, 2),
             "query_tokens_per_s": round(r["total_q"] / (ms * 1e-3), 1),
             "flops_per_launch": r["flops"], "replicas": r["reps"]}
    else:
        db, us = r["bytes"], r["decode_us"]
        uniq = db["unique"] / (us * 1e-6) / 1e9
        e = {"workload": r["desc"], "requests": w.num_seqs, "decode_us": round(us, 3),
             "step_us": round(ms * 1e3, 3), "step_event_us": round(r["step_event_us"], 3),
             "step_over_decode": round(r["step_event_us"] / us, 4),
             "decode_gbs_unique": round(uniq, 2),
             "decode_gbs_logical": round(db["logical"] / (us * 1e-6) / 1e9, 2),
             "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(uniq / HBM_PEAK_GBS, 4), "traffic": r["traffic"]},
             "step_gbs": round(r["step_bytes"] / (ms * 1e-3) / 1e9, 2),
             "step_frac": round(r["step_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "tokens_per_s": round(w.num_seqs / (ms * 1e-3), 1),
             "bytes_per_launch": db["unique"], "logical_bytes_per_launch": db["logical"],
             "partition_tokens": r["part"], "replicas": r["reps"], **r["flags"]}
    if "cpu_baseline" in r:
        e["cpu_baseline"] = r["cpu_baseline"]
    return e


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
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOADS),
                    help="the headline workload of the JSON line")
    ap.add_argument("--extra", default="prefix,long,fanout,prefill,gqa_d64,gqa_d256,gqa_f32,"
                                       "prefill_d64,prefill_d256",
                    help="comma-separated workloads also measured into the line's 'workloads' "
                         "object ('none' = only the headline)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--partition", type=int, default=0, help="decode partition tokens (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the headline workload")
    ap.add_argument("--extra-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle work for each extra workload")
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
    extra = [] if args.extra in ("", "none") else args.extra.split(",")
    for e in extra:
        if e not in WORKLOADS:
            ap.error(f"unknown workload in --extra: {e}")
    extra = [e for e in extra if e != args.workload]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbs = copy_probe(dev, args.copy_probe_mib) if args.copy_probe_mib > 0 else None
    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    # Every workload's cache pool stays allocated until the run ends, as a
    # serving process keeps the pool it allocates once: measured on MI355X, a
    # pool placed in memory that an earlier pool of the same process freed
    # decodes 3-7 % slower.  (All pools together take about 40 GB of HBM.)
    pools = []
    if WORKLOADS[args.workload].get("prefill"):
        r = measure_prefill(args.workload, args, dev, args.replicas, args.partition, budget)
        line = prefill_line(r, args, copy_gbs)
    else:
        r = measure_decode(args.workload, args, dev, args.replicas, args.partition, budget,
                           args.no_group, args.no_runs, args.stream_kv)
        line = decode_line(r, args, copy_gbs)
    pools.append(r["w"])
    del r
    if extra:
        line["workloads"] = {}
        ebudget = 0.0 if args.no_cpu_baseline else args.extra_cpu_budget
        for name in extra:
            if WORKLOADS[name].get("prefill"):
                r = measure_prefill(name, args, dev, 0, 0, ebudget)
            else:
                r = measure_decode(name, args, dev, 0, 0, ebudget)
            line["workloads"][name] = workload_entry(r)
            pools.append(r["w"])
            del r
    print(json.dumps(line), flush=True)
    del pools
    return 0


if __name__ == "__main__":
    sys.exit(main())
