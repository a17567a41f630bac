"""Decode-step benchmark of the paged KV cache path on one MI355X.

One step = copy_blocks (copy-on-write pairs, when the step has any) ->
paged_kv_write (each sequence's newest token) -> paged_attention_decode, over one
synthetic batch already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload long_splitk] [--only-main]

The line of record is the largest single-GPU workload, long-context split-K (8
sequences of 32768..131072 tokens, 512-token partitions: 3.5 GB of K/V per step);
the MHA, GQA, fork/copy-on-write and tiny fp32 workloads are measured in the same
run and reported under "workloads", each with its own roofline and CPU oracle
figure.  Byte counts are algorithmic: what the method must move (K and V of
every attended position once per KV head, q, out, block-table entries, lengths, and
the written / copied rows), not what the implementation happens to move.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "paged decode attention: KV HBM GB/s (% of MI355X peak), µs/decode step"
HBM_PEAK_GBS = 8000.0
# split-context partition used per workload (0 = one work unit per (sequence, KV head); None =
# recomputed for each step by batch.balanced_partition: the fork workload's 16 sequences x 8 KV
# heads are half as many items as there are compute units)
PARTITION = {"tiny_fp32": 0, "mha7b": 0, "gqa70b": 4096, "long_splitk": 512, "fork_cow": None}
MAIN = "long_splitk"   # the line of record: the largest single-GPU workload


def partition_for(name: str, cfg, step, num_cus: int = 256) -> int:
    """The partition size bench.py times for workload `name` on this step's inputs."""
    P = PARTITION[name]
    if P is None:
        from paged_kv_cache_148_amd import batch
        P = batch.balanced_partition(cfg.num_seqs, cfg.num_kv_heads, int(step.max_context_len), cfg.block_size,
                                     num_cus)
    return P


def algorithmic_bytes(cfg, step) -> dict:
    e = cfg.elem_bytes
    S, Hq, Hkv, D, B = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    ctx = step.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * 2 * Hkv * D * e
    attn = kv + 2 * S * Hq * D * e + 4 * int(sum(-(-int(c) // B) for c in ctx)) + 4 * S
    T = len(step.slot_mapping)
    write = 4 * T * Hkv * D * e + 8 * T
    P = step.copy_pairs.shape[0]
    copy = 2 * 2 * P * B * Hkv * D * e + 16 * P
    return {"kv": kv, "attention": attn, "write": write, "copy": copy, "step": attn + write + copy}


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (the sources hold no string literal with //
    or /*): a change of comments or layout leaves the hash alone, a change of code does not."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


# the sources the attention kernels are compiled from (the counter records describe them)
ATTENTION_SOURCES = ("attention.hip", "pkv_device.h")


def kernel_source_hash() -> str:
    """sha256 over the code of the attention kernels' sources (comments and whitespace
    removed), first 16 hex digits: the key of the committed counter records."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_148_amd", "csrc")
    for f in ATTENTION_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, partition, layout: str = "scattered"):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources at this partition size (on the default shuffled pool);
    else None."""
    path = os.path.join(ROOT, "profiles", f"attention_traffic_{workload}.json")
    if layout != "scattered" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("partition_size") != partition:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_step_us(cfg, step, steps: int = 50) -> float:
    """Host time of one decode step's table work (the slot mapping of every sequence's next
    token, new blocks, the kernels' table and length arrays) with the array-held batch, on
    this workload's batch: mean over `steps` steps."""
    from paged_kv_cache_148_amd.block_manager import BlockManager, DecodeBatch
    ctx = step.context_lens.astype(np.int64)
    bm = BlockManager(int(sum(-(-int(c) // cfg.block_size) for c in ctx)) + len(ctx) * (steps // cfg.block_size + 2),
                      cfg.block_size)
    db = DecodeBatch(bm, [bm.new_sequence(int(c)) for c in ctx])
    t = time.perf_counter()
    for _ in range(steps):
        db.step()
        db.block_tables()
        db.context_lens()
    return (time.perf_counter() - t) / steps * 1e6


def block_stats(cfg, step) -> dict:
    """Internal fragmentation of the step's block allocation (slots allocated but past the
    context, over all allocated slots) and block-table length."""
    B = cfg.block_size
    ctx = step.context_lens.astype(np.int64)
    blocks = -(-ctx // B)
    return {"block_size": B, "internal_frag": float((blocks * B - ctx).sum() / max(1, int((blocks * B).sum()))),
            "table_entries_mean": float(blocks.mean()), "table_entries_max": int(blocks.max())}


def run_gpu(name: str, which: str, steps: int, warmup: int, partition: int, layout: str = "scattered",
            block_size: int | None = None, flush_mall: str | None = None, window: int = 64, keep: bool = False):
    import torch
    from paged_kv_cache_148_amd import batch, binding

    cfg = workloads.CONFIGS[name]
    if block_size is not None and block_size != cfg.block_size:
        cfg = dataclasses.replace(cfg, block_size=block_size)
    t_gen = time.time()
    wl = workloads.make_workload(cfg)
    if layout == "contiguous":
        # identity free stack: every sequence's blocks are consecutive and ascending
        wl.free_order = list(range(wl.num_blocks))
    elif layout == "windowed":
        # shuffled only within windows of `window` consecutive block ids, the windows taken in
        # ascending order: a sequence's blocks are scattered over spans of `window` blocks only
        ids = np.arange(wl.num_blocks)
        rng = np.random.default_rng(cfg.seed + 1000)
        for i in range(0, wl.num_blocks, window):
            ids[i:i + window] = rng.permutation(ids[i:i + window])
        wl.free_order = [int(x) for x in ids[::-1]]
    step = batch.step_for(wl, which)
    if partition is None:
        partition = partition_for(name, cfg, step, torch.cuda.get_device_properties(0).multi_processor_count)
    bf16 = cfg.dtype == "bf16"
    dev = "cuda"
    q = batch.to_torch(wl.q, dev, bf16)
    kc = batch.to_torch(wl.k_cache, dev, bf16)
    vc = batch.to_torch(wl.v_cache, dev, bf16)
    kn = batch.to_torch(wl.k_new, dev, bf16)
    vn = batch.to_torch(wl.v_new, dev, bf16)
    tables = batch.to_torch(step.block_tables, dev)
    ctx = batch.to_torch(step.context_lens, dev)
    slots = batch.to_torch(step.slot_mapping, dev)
    pairs = batch.to_torch(step.copy_pairs, dev)
    hm = layout == "head_major"
    if hm:
        # the same values placed head-major: k [N, Hkv, D/x, B, x], v [N, Hkv, D, B]
        kc, vc = batch.to_head_major(kc, vc)
    write = binding.paged_kv_write_head_major if hm else binding.paged_kv_write
    copy = binding.copy_blocks_head_major if hm else binding.copy_blocks
    attend = binding.paged_attention_decode_head_major if hm else binding.paged_attention_decode
    out = torch.empty_like(q)
    ws_bytes = binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim, step.max_context_len,
                                                partition)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)   # queue counters start at zero
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen
    n_pairs = step.copy_pairs.shape[0]

    def attend_once():
        attend(out, q, kc, vc, tables, ctx, step.max_context_len, wl.scale, partition, ws)

    def one_step():
        if n_pairs:
            copy(kc, vc, pairs)
        write(kn, vn, kc, vc, slots)
        attend_once()

    for _ in range(warmup):
        one_step()
    # the whole step, `steps` times, by the host clock
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / steps
    # the spread of the step: events around each whole step on the launch stream (each figure
    # includes the events' own few microseconds)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in sev:
        a.record()
        one_step()
        b.record()
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in sev)
    # the same step captured once in a HIP graph and replayed (the calls allocate and clear
    # nothing, and the queue counters return to zero inside each attention call)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_step_s = (time.perf_counter() - t0) / steps
    del graph
    # the same step through paged_attention_decode_write: the write rides in the attention
    # launch on the tile paths (row layout)
    fused_step_s = None
    if not hm:
        def fused_step():
            if n_pairs:
                copy(kc, vc, pairs)
            binding.paged_attention_decode_write(out, q, kn, vn, kc, vc, tables, ctx, step.max_context_len, wl.scale,
                                                 partition, ws)
        for _ in range(warmup):
            fused_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fused_step()
        torch.cuda.synchronize()
        fused_step_s = (time.perf_counter() - t0) / steps
    # The attention call's launch duration: the same call `steps` times back to back between one
    # pair of events on the launch stream.
    b2b = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    b2b[0].record()
    for _ in range(steps):
        attend_once()
    b2b[1].record()
    torch.cuda.synchronize()
    attn_s = b2b[0].elapsed_time(b2b[1]) / 1e3 / steps
    # and its spread: events around each launch (they add 3-9 us of their own to each figure).
    # flush_mall: 512 MB are read ("read") or written ("write") before each launch, outside its
    # events, so that no K/V byte can come from the 256 MB Infinity Cache; a written flush also
    # leaves the cache full of dirty lines that the launch's own stores then have to evict
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev) if flush_mall else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        if flush_mall == "write":
            flush.fill_(1)
        elif flush_mall == "read":
            flush.amax()
        a.record()
        attend_once()
        b.record()
    torch.cuda.synchronize()
    attn_ms = sorted(a.elapsed_time(b) for a, b in ev)
    del flush
    nb = algorithmic_bytes(cfg, step)
    res = {
        "workload": name, "step": which, "partition_size": partition, "layout": layout,
        "window_blocks": window if layout == "windowed" else None,
        "us_per_step": step_s * 1e6, "us_per_step_graph": graph_step_s * 1e6,
        "step_us_events": {"median": float(np.median(step_ms)) * 1e3, "p10": _pct(step_ms, 10) * 1e3,
                           "p90": _pct(step_ms, 90) * 1e3,
                           "timing": f"HIP events around each of {steps} whole steps (their own few us included)"},
        "us_per_step_fused": fused_step_s * 1e6 if fused_step_s else None, "attention_us_mean": attn_s * 1e6,
        "attention_us_events_mean": float(np.mean(attn_ms)) * 1e3, "mall_flushed_per_launch": flush_mall,
        "attention_us_events_median": float(np.median(attn_ms)) * 1e3,
        "attention_us_events_p10": _pct(attn_ms, 10) * 1e3,
        "attention_us_events_p90": _pct(attn_ms, 90) * 1e3,
        "step_gbs": nb["step"] / step_s / 1e9,
        "kv_gbs_attention": nb["kv"] / attn_s / 1e9,
        "attention_alg_gbs": nb["attention"] / attn_s / 1e9,
        "attention_hbm_frac": nb["attention"] / attn_s / 1e9 / HBM_PEAK_GBS,
        "seqs_per_s": cfg.num_seqs / step_s,
        "bytes": nb, "num_seqs": cfg.num_seqs, "sum_ctx": int(step.context_lens.sum()),
        "max_ctx": int(step.max_context_len), "pool_blocks": wl.num_blocks,
        "copy_pairs": int(n_pairs), "path": binding.attention_path(cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                                                                    cfg.block_size, 1 if bf16 else 0),
        "input_gen_s": gen_s,
        "host_step_us": host_step_us(cfg, step),
        **block_stats(cfg, step),
    }
    if name == "fork_cow":
        shared = (cfg.ctx[1] // cfg.block_size) * cfg.block_size
        unique_tokens = shared + int((step.context_lens.astype(np.int64) - shared).sum())
        res["unique_kv_bytes"] = unique_tokens * 2 * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
        res["note"] = "unique KV fits the 256 MB Infinity Cache: logical GB/s is not an HBM figure"
    if keep and not hm:
        # what the step left on the GPU (every timed call repeats the same step on the same state,
        # so this is one step's result): the output and both pools, as raw bits, for the parity
        # report of the CPU oracle's leg
        res["_results"] = {"out": batch.from_torch_bits(out), "k_cache": batch.from_torch_bits(kc),
                           "v_cache": batch.from_torch_bits(vc)}
    del q, kc, vc, kn, vn, out, ws
    torch.cuda.empty_cache()
    return res, wl, step


def _pct(sorted_vals, q: int) -> float:
    """q-th percentile of an ascending list (nearest rank)."""
    return float(sorted_vals[min(len(sorted_vals) - 1, max(0, -(-q * len(sorted_vals) // 100) - 1))])


KERNEL_NAMES = {1: "paged_attention_decode (attn_vec_kernel)",
                2: "paged_attention_decode (attn_tile_kernel, MFMA tiles)",
                3: "paged_attention_decode (attn_tile_kernel, VALU dots: one query head per KV head)"}


def roofline(name: str, res: dict, rd: dict | None) -> dict | None:
    """The attention call against MI355X's 8 TB/s HBM peak: algorithmic bytes per call over the
    mean duration of back-to-back calls on the launch stream.  None where the data the call reads
    fits the 256 MB Infinity Cache (fork workload) or the call is latency-bound (tiny fp32)."""
    if name in ("fork_cow", "tiny_fp32"):
        return None
    nb = res["bytes"]["attention"]
    return {
        "bound": "hbm",
        "kernel": KERNEL_NAMES.get(res["path"], "paged_attention_decode"),
        "achieved": round(res["attention_alg_gbs"], 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(res["attention_alg_gbs"] / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(name, res.get("partition_size"), res.get("layout", "scattered")),
        "algorithmic_bytes_per_launch": nb,
        "launch_us_mean": round(res["attention_us_mean"], 2),
        "timing": f"HIP events around back-to-back attention calls on the launch stream",
        "frac_of_stream_read": round(res["attention_alg_gbs"] / rd["GB/s"], 4) if rd else None,
    }


def read_probe(reps: int = 3, gib: int = 1) -> None:
    """The plain streaming read over exactly `gib` GiB, `reps` times: the read-only reference for
    scaling rocprofv3's FETCH_SIZE (a K/V stream is read-only)."""
    import torch
    from paged_kv_cache_148_amd import binding
    buf = torch.zeros(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        binding.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    print(json.dumps({"read_probe": True, "calls": reps, "bytes_read_per_call": gib << 30}), flush=True)


def copy_probe(reps: int = 3) -> None:
    """copy_blocks over a known byte count, for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE:
    16384 blocks of 32 KiB copied in each of K and V = 1 GiB read + 1 GiB written per call."""
    import torch
    from paged_kv_cache_148_amd import binding
    N, B, Hkv, D = 32768, 16, 8, 128
    kc = torch.zeros(N, B, Hkv, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    half = N // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half, N)], dim=1).to(torch.int64).cuda()
    torch.cuda.synchronize()
    for _ in range(reps):
        binding.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    nbytes = 2 * half * B * Hkv * D * 2
    print(json.dumps({"copy_probe": True, "calls": reps, "bytes_read_per_call": nbytes,
                      "bytes_written_per_call": nbytes}), flush=True)


def movers(steps: int = 20) -> dict:
    """paged_kv_write and copy_blocks at sizes where HBM bandwidth, not launch latency, bounds
    them (the decode configurations write and copy well under 1 MB per step).  Pool of 16384
    blocks of 16 slots, 8 KV heads, head_dim 128, bf16 (32 KiB per block per tensor): a write of
    131072 tokens to distinct slots scattered over the pool (256 MiB of K and V each way), and a
    copy of 8192 (src, dst) block pairs (also 256 MiB each way).  One pair of HIP events around
    `steps` back-to-back calls on the launch stream.  Beside them, torch's contiguous device copy
    of the same bytes, as the rate a copy without indirection reaches."""
    import torch
    from paged_kv_cache_148_amd import binding
    N, B, Hkv, D = 16384, 16, 8, 128
    g = torch.Generator().manual_seed(7)
    kc = torch.zeros(N, B, Hkv, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    T = N * B // 2
    kn = torch.randn(T, Hkv, D, generator=g).to(torch.bfloat16).cuda()
    vn = torch.randn(T, Hkv, D, generator=g).to(torch.bfloat16).cuda()
    slots = torch.randperm(N * B, generator=g)[:T].to(torch.int64).cuda()
    perm = torch.randperm(N, generator=g)
    pairs = torch.stack([perm[: N // 2], perm[N // 2:]], dim=1).to(torch.int64).cuda()
    row = Hkv * D * 2

    def timed(call):
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / steps

    res = {}
    for name, call, nbytes in (
            ("paged_kv_write", lambda: binding.paged_kv_write(kn, vn, kc, vc, slots), 2 * (2 * T * row) + 8 * T),
            ("copy_blocks", lambda: binding.copy_blocks(kc, vc, pairs), 2 * (2 * (N // 2) * B * row) + 16 * (N // 2))):
        t = timed(call)
        res[name] = {"us": round(t * 1e6, 2), "algorithmic_bytes": nbytes, "GB/s": round(nbytes / t / 1e9, 1),
                     "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] {name}: {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    del kc, vc, kn, vn, slots, pairs
    # Context: the runtime's own contiguous device copy of the same 512 MiB each way (no slot or
    # pair indirection): what a plain copy reaches on this machine.
    src = torch.empty(2 * T * row, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src))
    nbytes = 2 * src.numel()
    res["contiguous_device_copy"] = {"us": round(t * 1e6, 2), "algorithmic_bytes": nbytes,
                                     "GB/s": round(nbytes / t / 1e9, 1),
                                     "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
    print(f"[bench] contiguous device copy (torch copy_): {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()
    return {"results": res, "tokens_written": T, "pairs_copied": N // 2, "steps": steps,
            "timing": f"HIP events around {steps} back-to-back calls on the launch stream"}


def stream_read_ceiling(steps: int = 20, gib: int = 2) -> dict:
    """A plain streaming read of `gib` GiB (16-byte non-temporal loads, no indirection, no
    arithmetic): what this machine's HBM delivers to a read-only kernel, the context for the
    decode kernels' bandwidth.  One pair of HIP events around `steps` back-to-back reads."""
    import torch
    from paged_kv_cache_148_amd import binding
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        binding.stream_read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        binding.stream_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = gib << 30
    del buf, sink
    torch.cuda.empty_cache()
    print(f"[bench] streaming read of {gib} GiB: {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s", file=sys.stderr,
          flush=True)
    return {"bytes": nbytes, "us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
            "frac_of_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def cpu_baseline(wl, which: str, partition: int, budget_s: float = 10.0, threads: int = 0, max_reps: int = 200,
                 gpu_results: dict | None = None) -> dict:
    """The CPU oracle on the same inputs: whole decode steps (copies, write, attention) on the
    host with the oracle's own step inputs (its block model on the workload's free stack),
    `threads` OpenMP threads (0: all it may use), repeated until about budget_s seconds have been
    spent (at least once, at most max_reps times).  With gpu_results (the GPU step's output and
    pools as raw bits), the last step's results are compared with them: "parity"."""
    import oracle
    from oracle import batch as obatch
    cfg = wl.cfg
    o = obatch.step_for(wl, which)
    nb = algorithmic_bytes(cfg, _StepBytes(o))
    nt = threads if threads > 0 else oracle.max_threads()
    reps, t_total = 0, 0.0
    kc = vc = ref = None
    while reps == 0 or (t_total < budget_s and reps < max_reps):
        kc = vc = ref = None   # the previous step's pool copies go before the next are made
        kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
        t = time.perf_counter()
        oracle.copy_blocks(kc, vc, o["copy_pairs"])
        oracle.kv_write(wl.k_new, wl.v_new, kc, vc, o["slot_mapping"])
        ref = oracle.attention(wl.q, kc, vc, o["block_tables"], o["context_lens"], wl.scale, partition, num_threads=nt)
        t_total += time.perf_counter() - t
        reps += 1
    per = t_total / reps
    res = {"value": round(nb["step"] / per / 1e9, 3), "unit": "GB/s", "cores": nt, "kind": "oracle",
           "us_per_step": round(per * 1e6, 1), "steps_timed": reps, "seconds": round(t_total, 2),
           "sample": f"{reps} whole decode step(s) of the {cfg.name} workload ({cfg.num_seqs} seqs, "
                     f"{int(o['context_lens'].sum())} tokens, partition {partition}), fp64 scalar C, "
                     f"{nt} OpenMP thread(s), {t_total:.1f} s in all"}
    if gpu_results is not None:
        res["parity"] = parity(gpu_results, ref, kc, vc, cfg.dtype)
    return res


class _StepBytes:
    """The fields of a step that algorithmic_bytes reads, from the oracle's step dict."""

    def __init__(self, o):
        self.context_lens, self.block_tables = o["context_lens"], o["block_tables"]
        self.slot_mapping, self.copy_pairs = o["slot_mapping"], o["copy_pairs"]


# The parity tests' tolerance: bf16 inputs with fp32 accumulation, max |gpu - ref| <= 2e-2; fp32
# inputs, |gpu - ref| <= 1e-5 + 1e-4 |ref| per element.
BF16_MAX_ABS = 2e-2
F32_ABS, F32_REL = 1e-5, 1e-4


def parity(gpu: dict, ref, kc, vc, dtype: str) -> dict:
    """Every output element against the fp64 oracle (max-abs, max-rel, within the tolerance), and
    both pools after the step's copies and write, bit for bit."""
    import oracle
    g = oracle.widen(gpu["out"]).reshape(ref.shape)
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    if dtype == "f32":
        ok = bool((err <= F32_ABS + F32_REL * np.abs(ref)).all())
        tol = f"|gpu - ref| <= {F32_ABS:g} + {F32_REL:g} |ref| per element"
    else:
        ok = max_abs <= BF16_MAX_ABS
        tol = f"max |gpu - ref| <= {BF16_MAX_ABS:g}"
    return {"outputs_compared": int(err.size), "max_abs": float(f"{max_abs:.3e}"), "max_rel": float(f"{max_rel:.3e}"),
            "within_tolerance": bool(ok and np.isfinite(g).all()), "tolerance": tol,
            "k_cache_bit_exact": bool(np.array_equal(gpu["k_cache"], kc)),
            "v_cache_bit_exact": bool(np.array_equal(gpu["v_cache"], vc)),
            "reference": "CPU oracle (fp64), its own step inputs from the same free stack"}


def host_info() -> dict:
    """The host the CPU oracle runs on."""
    import oracle
    return {"cpu": _cpu_model(), "nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)),
            "omp_threads": oracle.max_threads(), "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=MAIN, choices=sorted(workloads.CONFIGS))
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--only-main", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--movers", action="store_true",
                    help="only time paged_kv_write and copy_blocks at HBM-bound sizes (256 MiB each way)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run copy_blocks over 1 GiB (counter calibration for rocprofv3)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the plain streaming read over 1 GiB (counter calibration for rocprofv3)")
    ap.add_argument("--layout", default="scattered", choices=["scattered", "contiguous", "windowed", "head_major"],
                    help="scattered: seeded shuffled pool (default); contiguous: identity-ordered pool; windowed: "
                         "shuffled within windows of --window blocks; head_major: the shuffled pool in the "
                         "head-major cache layout")
    ap.add_argument("--window", type=int, default=64, help="block ids per window of the windowed layout")
    ap.add_argument("--block-size", type=int, default=None,
                    help="run the workload with this block size instead of its configured one")
    ap.add_argument("--flush-mall", choices=["read", "write"], default=None,
                    help="read or write 512 MB before each per-launch-timed attention call (outside its events)")
    ap.add_argument("--sweep-block-size", action="store_true",
                    help="time the workload at block sizes 8..128 and print one JSON line of the sweep")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the decode path here has no cross-GPU step)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.read_probe:
        read_probe()
        return
    if args.movers:
        print(json.dumps({"movers": movers(), "kernel_source_hash": kernel_source_hash()}), flush=True)
        return

    main_part = PARTITION[args.workload] if args.partition is None else args.partition
    which = "steady"
    if args.sweep_block_size:
        sweep = []
        for B in (8, 16, 32, 64, 128):
            r, _, _ = run_gpu(args.workload, which, args.steps, args.warmup, main_part, args.layout, B)
            keep = ("block_size", "internal_frag", "table_entries_mean", "table_entries_max", "path", "pool_blocks",
                    "attention_us_mean", "attention_us_events_p10", "attention_us_events_p90", "us_per_step",
                    "kv_gbs_attention",
                    "attention_alg_gbs", "attention_hbm_frac")
            sweep.append({k: (round(r[k], 4) if isinstance(r[k], float) else r[k]) for k in keep})
            print(f"[bench] {args.workload} B={B}: attention {r['attention_us_mean']:.1f} us, "
                  f"{r['attention_alg_gbs']:.0f} GB/s, internal fragmentation {100 * r['internal_frag']:.2f}%",
                  file=sys.stderr, flush=True)
        print(json.dumps({"block_size_sweep": args.workload, "partition_size": main_part, "layout": args.layout,
                          "steps": args.steps, "warmup": args.warmup, "results": sweep,
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return
    res, wl, step = run_gpu(args.workload, which, args.steps, args.warmup, main_part, args.layout, args.block_size,
                            args.flush_mall, args.window, keep=not args.no_cpu)
    _say_step(args.workload, res)
    # the CPU oracle on each workload's own inputs, right after its GPU run (all host threads; the
    # line of record's for ~10 s, the others once each; one thread as well on the two smallest)
    cpu_runs = {}
    if not args.no_cpu:
        cpu_runs[args.workload] = cpu_baseline(wl, which, res["partition_size"], budget_s=10.0,
                                               gpu_results=res.pop("_results", None))
        _say_cpu(args.workload, cpu_runs[args.workload])
    del wl, step
    others = {}
    single = {}
    if not args.only_main:
        for name in OTHERS:
            if name == args.workload:
                continue
            for w in (["fork", "steady"] if name == "fork_cow" else ["steady"]):
                key = f"{name}/{w}" if name == "fork_cow" else name
                r, wl_o, step_o = run_gpu(name, w, args.steps, args.warmup, PARTITION[name], flush_mall=args.flush_mall,
                                          keep=not args.no_cpu)
                others[key] = r
                _say_step(key, r)
                if not args.no_cpu:
                    cpu_runs[key] = cpu_baseline(wl_o, w, r["partition_size"], budget_s=0.0,
                                                 gpu_results=r.pop("_results", None))
                    _say_cpu(key, cpu_runs[key])
                    if name in SINGLE_THREAD:
                        single[key] = cpu_baseline(wl_o, w, r["partition_size"], budget_s=0.0, threads=1)
                        _say_cpu(key + " (1 thread)", single[key])
                del wl_o, step_o

    # paged_kv_write and copy_blocks where HBM, not launch latency, bounds them; a plain read
    mv = None if args.only_main else movers()
    rd = None if args.only_main else stream_read_ceiling()
    cfg = workloads.CONFIGS[args.workload]
    cpu = None
    if cpu_runs:
        cpu = dict(cpu_runs[args.workload])
        cpu.pop("parity", None)
        cpu["host"] = host_info()
        cpu["per_workload"] = {k: {kk: v[kk] for kk in ("value", "unit", "us_per_step", "cores", "steps_timed")}
                               for k, v in cpu_runs.items()}
        cpu["single_thread"] = {k: {kk: v[kk] for kk in ("value", "unit", "us_per_step", "cores", "steps_timed")}
                                for k, v in single.items()}
    workloads_out = {}
    for k, v in others.items():
        e = {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
        e["roofline"] = roofline(k.split("/")[0], v, rd)
        e["parity"] = cpu_runs.get(k, {}).get("parity")
        workloads_out[k] = e
    line = {
        "metric": METRIC,
        "value": round(res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, seeded shuffled block pool)",
        "config": {"workload": f"{args.workload}: {cfg.description}", "num_seqs": cfg.num_seqs,
                   "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": res["block_size"], "partition_size": res["partition_size"], "sum_ctx": res["sum_ctx"],
                   "max_ctx": res["max_ctx"], "parallelism": "single GPU"},
        "us_per_step": round(res["us_per_step"], 2),
        "step_us_events": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in res["step_us_events"].items()},
        "us_per_step_graph": round(res["us_per_step_graph"], 2),
        "us_per_step_fused": round(res["us_per_step_fused"], 2) if res["us_per_step_fused"] else None,
        "seqs_per_s": round(res["seqs_per_s"], 1),
        "host_step_us": round(res["host_step_us"], 1),
        "hbm_frac_step": round(res["step_gbs"] / HBM_PEAK_GBS, 4),
        "roofline": roofline(args.workload, res, rd),
        "attention_us_events": {"median": round(res["attention_us_events_median"], 2),
                                "p10": round(res["attention_us_events_p10"], 2),
                                "p90": round(res["attention_us_events_p90"], 2)},
        "cpu_baseline": cpu,
        "parity": cpu_runs.get(args.workload, {}).get("parity"),
        "workloads": workloads_out,
        "movers": mv,
        "stream_read": rd,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


# the other workloads of a default run, and those the CPU oracle also runs on one thread
OTHERS = ("mha7b", "gqa70b", "long_splitk", "fork_cow", "tiny_fp32")
SINGLE_THREAD = ("tiny_fp32", "mha7b")


def _say_step(name, r):
    print(f"[bench] {name}: {r['us_per_step']:.1f} us/step ({r['us_per_step_graph']:.1f} from a graph, "
          f"{r['us_per_step_fused'] or 0:.1f} fused), attention {r['attention_us_mean']:.1f} us, "
          f"{r['attention_alg_gbs']:.0f} GB/s", file=sys.stderr, flush=True)


def _say_cpu(name, c):
    print(f"[bench] CPU oracle {name}: {c['us_per_step']:.0f} us/step, {c['value']:.2f} GB/s, {c['cores']} thread(s), "
          f"{c['steps_timed']} step(s)", file=sys.stderr, flush=True)
    pr = c.get("parity")
    if pr:
        print(f"[bench] parity {name}: {pr['outputs_compared']} outputs, max_abs {pr['max_abs']:.3e}, "
              f"max_rel {pr['max_rel']:.3e}, within tolerance {pr['within_tolerance']}, pools bit-exact "
              f"{pr['k_cache_bit_exact'] and pr['v_cache_bit_exact']}", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
