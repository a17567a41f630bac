"""CPU checks of bench.py's accounting: the algorithmic byte counts behind `value` and the
roofline, and the key that ties the committed counter records to the kernel code."""
import types

import numpy as np

import bench


def _cfg(**kw):
    base = dict(elem_bytes=2, num_seqs=2, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16)
    base.update(kw)
    return types.SimpleNamespace(**base)


def test_algorithmic_bytes_by_hand():
    # two sequences of 17 and 32 tokens (2 + 2 blocks of 16), one new token each, one copy pair
    step = types.SimpleNamespace(context_lens=np.array([17, 32]), slot_mapping=np.array([5, 40]),
                                 copy_pairs=np.array([[3, 7]]))
    nb = bench.algorithmic_bytes(_cfg(), step)
    kv = (17 + 32) * 2 * 2 * 128 * 2            # K and V rows of every attended position, per KV head
    q_out = 2 * 2 * 8 * 128 * 2                 # q read and out written, every query head
    tables = 4 * (2 + 2)                        # one int32 entry per attended block
    lengths = 4 * 2
    assert nb["kv"] == kv
    assert nb["attention"] == kv + q_out + tables + lengths
    assert nb["write"] == 2 * (2 * 2 * 128 * 2) * 2 + 8 * 2   # rows read and written, K and V, + slots
    assert nb["copy"] == 2 * 2 * 1 * 16 * 2 * 128 * 2 + 16   # a block read and written, K and V, + pair
    assert nb["step"] == nb["attention"] + nb["write"] + nb["copy"]


def test_gqa_reads_kv_once_per_kv_head():
    step = types.SimpleNamespace(context_lens=np.array([100]), slot_mapping=np.array([0]),
                                 copy_pairs=np.zeros((0, 2), np.int64))
    g8 = bench.algorithmic_bytes(_cfg(num_seqs=1, num_heads=64, num_kv_heads=8), step)
    g1 = bench.algorithmic_bytes(_cfg(num_seqs=1, num_heads=8, num_kv_heads=8), step)
    assert g8["kv"] == g1["kv"]                 # 64 query heads over 8 KV heads move no more K/V


def test_source_key_ignores_comments_and_layout():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only("/* a note */ int  f(int x)\n{ return x + 1; }")
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))
    assert len(bench.kernel_source_hash()) == 16


def test_percentiles_nearest_rank():
    v = sorted(float(x) for x in range(1, 101))     # 1 .. 100
    assert bench._pct(v, 10) == 10.0 and bench._pct(v, 90) == 90.0 and bench._pct(v, 100) == 100.0
    assert bench._pct([5.0], 10) == 5.0


def test_roofline_object():
    res = {"bytes": {"attention": 3_500_000_000}, "attention_alg_gbs": 6000.0, "attention_us_mean": 583.3, "path": 2}
    r = bench.roofline("long_splitk", res, {"GB/s": 6800.0})
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == 0.75 and r["achieved"] == 6000.0 and r["algorithmic_bytes_per_launch"] == 3_500_000_000
    assert abs(r["frac_of_stream_read"] - 6000 / 6800) < 1e-4
    assert bench.roofline("fork_cow", res, None) is None       # Infinity-Cache resident: no HBM claim


def test_host_info_names_the_cpu_model():
    h = bench.host_info()
    assert h["cpu"] not in ("", "x86_64", "unknown")            # the model name, not the ISA
    assert h["nproc"] >= 1 and h["cpus_allowed"] >= 1 and h["omp_threads"] >= 1


def test_cpu_baseline_on_the_tiny_workload():
    import workloads
    from paged_kv_cache_148_amd import batch
    wl = workloads.make_workload("tiny_fp32")
    step = batch.step_for(wl)
    c = bench.cpu_baseline(wl, step, 0, budget_s=0.0, threads=1)
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["steps_timed"] == 1 and c["value"] > 0
    assert "tiny_fp32" in c["sample"]


def _bf16_bits(x):
    """fp64 -> bf16 bit patterns, round to nearest even (finite values)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _oracle_results(wl, which, partition):
    import oracle
    from oracle import batch as obatch
    o = obatch.step_for(wl, which)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.copy_blocks(kc, vc, o["copy_pairs"])
    oracle.kv_write(wl.k_new, wl.v_new, kc, vc, o["slot_mapping"])
    ref = oracle.attention(wl.q, kc, vc, o["block_tables"], o["context_lens"], wl.scale, partition)
    return ref, kc, vc


def test_oracle_leg_reports_parity_fp32():
    import workloads
    wl = workloads.make_workload("tiny_fp32")
    ref, kc, vc = _oracle_results(wl, "steady", 0)
    good = {"out": ref.astype(np.float32), "k_cache": kc.copy(), "v_cache": vc.copy()}
    r = bench.cpu_baseline(wl, "steady", 0, budget_s=0.0, gpu_results=good)
    p = r["parity"]
    assert p["outputs_compared"] == ref.size and p["within_tolerance"]
    assert p["k_cache_bit_exact"] and p["v_cache_bit_exact"] and p["max_abs"] < 1e-6
    bad_out = dict(good, out=good["out"].copy())
    bad_out["out"].flat[7] += 1e-3                       # one element past 1e-5 + 1e-4 |ref|
    assert not bench.cpu_baseline(wl, "steady", 0, budget_s=0.0, gpu_results=bad_out)["parity"]["within_tolerance"]
    bad_pool = dict(good, v_cache=good["v_cache"].copy())
    bad_pool["v_cache"].view(np.uint32).flat[123] ^= 1   # one bit of one V element
    p = bench.cpu_baseline(wl, "steady", 0, budget_s=0.0, gpu_results=bad_pool)["parity"]
    assert p["k_cache_bit_exact"] and not p["v_cache_bit_exact"] and p["within_tolerance"]


def test_oracle_leg_reports_parity_bf16_fork_step():
    import workloads
    wl = workloads.make_workload("fork_cow")
    ref, kc, vc = _oracle_results(wl, "fork", 1024)
    good = {"out": _bf16_bits(ref), "k_cache": kc.copy(), "v_cache": vc.copy()}
    p = bench.cpu_baseline(wl, "fork", 1024, budget_s=0.0, gpu_results=good)["parity"]
    assert p["within_tolerance"] and p["k_cache_bit_exact"] and p["v_cache_bit_exact"]
    assert 0 < p["max_abs"] < 2e-2                       # the output's own bf16 rounding
    stale = dict(good, k_cache=wl.k_cache.copy())       # the pool before the step's copies and write
    p = bench.cpu_baseline(wl, "fork", 1024, budget_s=0.0, gpu_results=stale)["parity"]
    assert not p["k_cache_bit_exact"] and p["v_cache_bit_exact"]


def test_balanced_partition_by_hand():
    from paged_kv_cache_148_amd.batch import balanced_partition
    # 16 sequences x 8 KV heads = 128 items for 256 units: two pieces per sequence, whole blocks
    assert balanced_partition(16, 8, 2002, 16, 256) == 1008          # ceil(2002 / 2) = 1001 -> 1008
    assert balanced_partition(16, 8, 2513, 16, 256) == 1264          # 1257 -> 1264
    assert balanced_partition(16, 8, 2513, 32, 256) == 1280
    # enough items unsplit, or nothing to split
    assert balanced_partition(64, 32, 2048, 16, 256) == 0
    assert balanced_partition(256, 8, 8192, 16, 256) == 0
    assert balanced_partition(1, 1, 16, 16, 256) == 0
    # 8 x 8 items: four pieces; one sequence of one head: 256 pieces of 16 tokens
    assert balanced_partition(8, 8, 128737, 16, 256) == 32192
    assert balanced_partition(1, 1, 4096, 16, 256) == 16
    # a piece never reaches the whole context
    assert balanced_partition(1, 1, 20, 16, 256) == 16
    assert balanced_partition(2, 1, 17, 16, 4) == 16


def test_bench_partition_for_the_fork_workload():
    import workloads
    from paged_kv_cache_148_amd import batch
    wl = workloads.make_workload("fork_cow")
    fork, steady = batch.step_for(wl, "fork"), batch.step_for(wl, "steady")
    assert bench.partition_for("fork_cow", wl.cfg, fork) == 1008
    P = bench.partition_for("fork_cow", wl.cfg, steady)
    assert P % 16 == 0 and 2 * P >= steady.max_context_len > P    # two pieces per sequence
    assert bench.partition_for("long_splitk", wl.cfg, steady) == 512


def test_traffic_record_applies_only_where_it_was_taken(tmp_path, monkeypatch):
    import json
    (tmp_path / "profiles").mkdir()
    h = bench.kernel_source_hash()
    rec = {"kernel_source_hash": h, "partition_size": 512, "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "attention_traffic_long_splitk.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    assert bench.measured_traffic("long_splitk", 512) == 123
    assert bench.measured_traffic("long_splitk", 1024) is None            # another partition size
    assert bench.measured_traffic("long_splitk", 512, "contiguous") is None  # another pool
    assert bench.measured_traffic("mha7b", 0) is None                      # no record
    rec["kernel_source_hash"] = "0" * 16                                   # other kernel sources
    (tmp_path / "profiles" / "attention_traffic_long_splitk.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("long_splitk", 512) is None
