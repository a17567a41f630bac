"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

KV write and block copy: bit-exact over the whole pool.  Attention: within the stated
tolerance (fp32: |d| <= 1e-5 + 1e-4 |ref|; bf16: max-abs 2e-2) of the fp64 oracle, which
builds its own block tables, slots and copy pairs with its own block model.
"""
import math

import numpy as np
import pytest

import oracle
from paged_kv_cache_148_amd import batch as pbatch
from paged_kv_cache_148_amd import binding
from tests import gpu_helpers as H
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield


def _wl(name, num_seqs=None, seed=None, ctx=None):
    return workloads.make_workload(name, num_seqs=num_seqs, seed=seed, ctx_override=ctx)


# ---------------------------------------------------------------------------
# data movement: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_fp32", "mha7b", "gqa70b", "fork_cow"])
def test_kv_write_bit_exact(name):
    import torch
    wl = _wl(name, num_seqs=min(workloads.CONFIGS[name].num_seqs, 16))
    # new rows of arbitrary bits: NaN payloads, -0, infinities, subnormals must all survive
    rng = np.random.default_rng(7)
    dt = np.uint16 if wl.cfg.dtype == "bf16" else np.uint32
    wl.k_new = rng.integers(0, np.iinfo(dt).max, size=wl.k_new.shape, dtype=dt, endpoint=True)
    wl.v_new = rng.integers(0, np.iinfo(dt).max, size=wl.v_new.shape, dtype=dt, endpoint=True)
    if dt == np.uint32:
        wl.k_new, wl.v_new = wl.k_new.view(np.float32), wl.v_new.view(np.float32)
    step = pbatch.step_for(wl)
    _say("kv_write", name, wl.k_cache.shape)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_copy=False, do_attn=False)
    o, kc, vc, _ = H.oracle_step(wl, attend=False)
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
    del torch


def test_kv_write_skips_negative_slots():
    import torch
    wl = _wl("mha7b", num_seqs=4)
    step = pbatch.step_for(wl)
    step.slot_mapping[1] = -1
    _say("kv_write -1 slot")
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_copy=False, do_attn=False)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    keep = [0, 2, 3]
    oracle.kv_write(np.ascontiguousarray(wl.k_new[keep]), np.ascontiguousarray(wl.v_new[keep]), kc, vc,
                    step.slot_mapping[keep])
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
    del torch


def test_kv_write_empty_is_noop():
    wl = _wl("gqa70b", num_seqs=2)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    before = H.bits(d["k_cache"]).tobytes()
    binding.paged_kv_write(d["k_new"][:0], d["v_new"][:0], d["k_cache"], d["v_cache"], d["slot_mapping"][:0])
    import torch
    torch.cuda.synchronize()
    assert H.bits(d["k_cache"]).tobytes() == before


def test_copy_blocks_fork_step_bit_exact():
    wl = _wl("fork_cow")
    step = pbatch.step_for(wl, "fork")
    assert step.copy_pairs.shape[0] == 15
    _say("copy_blocks fork step", step.copy_pairs.shape)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_write=False, do_attn=False)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.copy_blocks(kc, vc, step.copy_pairs)
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()


@pytest.mark.parametrize("name", ["tiny_fp32", "gqa70b"])
def test_copy_blocks_random_pairs_bit_exact(name):
    import torch
    wl = _wl(name, num_seqs=8)
    step = pbatch.step_for(wl)
    rng = np.random.default_rng(3)
    N = wl.num_blocks
    perm = rng.permutation(N)
    npairs = min(N // 2, 40)
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int64)
    d = H.upload(wl, step)
    d["copy_pairs"] = pbatch.to_torch(pairs, "cuda")
    _say("copy_blocks random", name, pairs.shape)
    H.gpu_step(wl, step, d, 0, do_write=False, do_attn=False)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.copy_blocks(kc, vc, pairs)
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
    del torch


@pytest.mark.parametrize("B", [64, 128])
def test_write_and_copy_large_blocks_bit_exact(B):
    # the block-size sweep's large blocks: slot-mapped write, then random whole-block copies
    cfg = workloads.Config("bigblock", "bf16", 6, 16, 4, 128, B, ("uniform", 1, 3 * B), seed=200 + B)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    _say("write large blocks", B)
    H.gpu_step(wl, step, d, 0, do_attn=False)
    _, kc, vc, _ = H.oracle_step(wl, "steady", attend=False)   # the oracle's own slots
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
    rng = np.random.default_rng(B)
    perm = rng.permutation(wl.num_blocks)
    npairs = wl.num_blocks // 2
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int64)
    d["copy_pairs"] = pbatch.to_torch(pairs, "cuda")
    _say("copy large blocks", B, pairs.shape)
    H.gpu_step(wl, step, d, 0, do_write=False, do_attn=False)
    oracle.copy_blocks(kc, vc, pairs)
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_bulk_write_and_copy_bit_exact(dt):
    # calls that move 32 MiB or more take the non-temporal forms of both kernels; one call
    # each a little above that size and one just below, over a pool of arbitrary bit patterns
    import torch
    rng = np.random.default_rng(31)
    N, B, Hkv, D = 2048, 16, 8, 128
    udt, sdt = (np.uint16, np.int16) if dt == "bf16" else (np.uint32, np.int32)
    fdt = torch.bfloat16 if dt == "bf16" else torch.float32
    host = (lambda a: a) if dt == "bf16" else (lambda a: a.view(np.float32))   # the oracle's dtypes

    def bits(shape):
        return rng.integers(0, np.iinfo(udt).max, size=shape, dtype=udt, endpoint=True)

    def dev(a):
        return torch.from_numpy(a.view(sdt)).cuda().view(fdt)

    kc, vc = bits((N, B, Hkv, D)), bits((N, B, Hkv, D))
    dk, dv = dev(kc), dev(vc)
    row = Hkv * D * kc.itemsize
    tk = (32 << 20) // (2 * row)                       # tokens whose K and V rows make 32 MiB
    for T in (tk + 7, tk - 1):
        kn, vn = bits((T, Hkv, D)), bits((T, Hkv, D))
        slots = rng.permutation(N * B)[:T].astype(np.int64)
        _say("bulk write", dt, T)
        binding.paged_kv_write(dev(kn), dev(vn), dk, dv, torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        oracle.kv_write(host(kn), host(vn), host(kc), host(vc), slots)
        assert H.bits(dk).tobytes() == kc.tobytes()
        assert H.bits(dv).tobytes() == vc.tobytes()
    pk = (32 << 20) // (2 * B * row)                   # pairs whose K and V blocks make 32 MiB
    for P in (pk + 3, pk - 1):
        perm = rng.permutation(N)
        pairs = np.stack([perm[:P], perm[P:2 * P]], axis=1).astype(np.int64)
        _say("bulk copy", dt, P)
        binding.copy_blocks(dk, dv, torch.from_numpy(pairs).cuda())
        torch.cuda.synchronize()
        oracle.copy_blocks(host(kc), host(vc), pairs)
        assert H.bits(dk).tobytes() == kc.tobytes()
        assert H.bits(dv).tobytes() == vc.tobytes()


# ---------------------------------------------------------------------------
# attention on the configurations (sizes the oracle finishes in seconds)
# ---------------------------------------------------------------------------

SMALL = [
    # name, num_seqs, partition sizes
    ("tiny_fp32", None, [0, 8, 32]),
    ("mha7b", 6, [0, 512]),
    ("gqa70b", 12, [0, 512, 256]),
    ("fork_cow", None, [512, 0]),
]


@pytest.mark.parametrize("name,num_seqs,parts", SMALL)
def test_step_parity(name, num_seqs, parts):
    wl = _wl(name, num_seqs=num_seqs)
    whiches = ["fork", "steady"] if name == "fork_cow" else ["steady"]
    for which in whiches:
        step = pbatch.step_for(wl, which)
        for P in parts:
            _say("step", name, which, "S", wl.cfg.num_seqs, "P", P)
            d = H.upload(wl, step)
            H.gpu_step(wl, step, d, P)
            o, kc, vc, ref = H.oracle_step(wl, which, P)
            assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
            assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
            H.check_close(H.bits(d["out"]), ref, wl.cfg.dtype, f"{name}/{which}/P={P}")


def test_long_context_split_parity():
    # the long-context shape with contexts the oracle finishes quickly, spanning many partitions
    ctx = np.array([32768, 5000, 12345, 1], np.int64)
    wl = _wl("long_splitk", ctx=ctx)
    step = pbatch.step_for(wl)
    for P in (512, 2048, 0):
        _say("long split", ctx.tolist(), "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(d["out"]), ref, "bf16", f"long P={P}")


SHAPES = [
    # dtype, S, Hq, Hkv, D, B, ctx range
    ("bf16", 5, 16, 8, 128, 16, (1, 300)),    # g = 2, MFMA
    ("bf16", 5, 16, 4, 128, 16, (1, 300)),    # g = 4
    ("bf16", 3, 32, 2, 128, 16, (1, 300)),    # g = 16
    ("bf16", 4, 24, 8, 128, 32, (1, 400)),    # g = 3, B = 32
    ("bf16", 4, 8, 8, 64, 4, (1, 200)),       # vector, D = 64, B = 4
    ("bf16", 4, 16, 2, 64, 8, (1, 200)),      # vector, g = 8
    ("bf16", 4, 6, 2, 128, 8, (1, 200)),      # MFMA, g = 3, B = 8: two blocks per tile
    ("bf16", 4, 8, 2, 128, 4, (1, 200)),      # MFMA, g = 4, B = 4: four blocks per tile
    ("bf16", 4, 8, 8, 128, 32, (1, 300)),     # MHA (g = 1) on the VALU tile path, B = 32
    ("bf16", 4, 8, 8, 128, 8, (1, 300)),      # MHA on the VALU tile path, B = 8
    ("bf16", 3, 4, 4, 128, 16, (4200, 9000)), # g = 1, VALU tiles, more than 64 tiles per wave
    ("bf16", 4, 8, 8, 128, 4, (1, 300)),      # g = 1, B = 4: four blocks per tile
    ("bf16", 5, 32, 4, 128, 64, (1, 700)),    # B = 64, g = 8
    ("bf16", 4, 8, 8, 128, 128, (1, 900)),    # B = 128, g = 1
    ("bf16", 3, 16, 2, 128, 128, (1, 2600)),  # B = 128, g = 8, more than 64 tiles per wave
    ("bf16", 3, 8, 2, 128, 8, (2000, 5000)),  # MFMA, B = 8, long: the shallow ring's split partitions
    ("f32", 4, 8, 8, 128, 16, (1, 200)),      # fp32, D = 128 (32 lanes per row)
    ("f32", 4, 8, 2, 64, 8, (1, 200)),        # fp32 GQA on the vector path
    ("f32", 3, 5, 5, 64, 32, (1, 200)),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}-g{s[2]//s[3]}-D{s[4]}-B{s[5]}" for s in SHAPES])
def test_shape_sweep_parity(shape):
    dt, S, Hq, Hkv, D, B, (lo, hi) = shape
    cfg = workloads.Config("sweep", dt, S, Hq, Hkv, D, B, ("uniform", lo, hi), seed=100 + Hq + D + B)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    # below 16 slots per block also a partition that is not a multiple of the 16-token tile;
    # long contexts also split into partitions above 512 tokens (the shallow load ring)
    for P in (0, 4 * B if B >= 16 else 64) + ((3 * B,) if B < 16 else ()) + ((1024,) if hi > 2048 else ()):
        _say("sweep", shape, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(d["out"]), ref, dt, f"{shape} P={P}")


# ---------------------------------------------------------------------------
# exactness properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_fp32", "mha7b", "gqa70b"])
def test_single_token_returns_v_exactly(name):
    S = 4
    wl = _wl(name, ctx=np.ones(S, np.int64))
    step = pbatch.step_for(wl)
    _say("ctx=1", name)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0)
    g = wl.cfg.group
    out = H.bits(d["out"])
    for s in range(S):
        # the only attended row is the one just written: out = v_new exactly, per KV head
        assert out[s].tobytes() == np.repeat(wl.v_new[s], g, axis=0).tobytes()


@pytest.mark.parametrize("name,P", [("mha7b", 0), ("mha7b", 128), ("gqa70b", 0), ("gqa70b", 256),
                                    ("tiny_fp32", 8)])
def test_peaked_and_uniform_softmax(name, P):
    # scores 32 times their usual spread (near one-hot weights: the running-max rescaling does the
    # work), then q = 0 (every weight equal: the output is the mean of the attended V rows); the
    # VALU, MFMA and vector paths, unsplit and split
    for case in ("peaked", "uniform"):
        wl = _wl(name, num_seqs=6)
        if case == "peaked":   # q times 32: a power of two, so the scaled q is exact in bf16 too
            if wl.q.dtype == np.uint16:
                f = (wl.q.astype(np.uint32) << 16).view(np.float32) * np.float32(32.0)
                wl.q[...] = (f.view(np.uint32) >> 16).astype(np.uint16)
            else:
                wl.q *= np.float32(32.0)
        else:
            wl.q[...] = 0
        step = pbatch.step_for(wl)
        _say("softmax", case, name, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(d["out"]), ref, wl.cfg.dtype, f"{case} {name} P={P}")


@pytest.mark.parametrize("name,P", [("mha7b", 0), ("gqa70b", 256), ("tiny_fp32", 8)])
def test_block_permutation_invariance_bitwise(name, P):
    wl = _wl(name, num_seqs=6)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P)
    out1 = H.bits(d["out"]).copy()
    # relabel every physical block id: pool rows move, tables and slots follow
    pi = np.random.default_rng(5).permutation(wl.num_blocks)
    kc2, vc2 = np.empty_like(wl.k_cache), np.empty_like(wl.v_cache)
    kc2[pi], vc2[pi] = wl.k_cache, wl.v_cache
    wl.k_cache, wl.v_cache = kc2, vc2
    B = wl.cfg.block_size
    step.block_tables = pi[step.block_tables].astype(np.int32)
    step.slot_mapping = (pi[step.slot_mapping // B] * B + step.slot_mapping % B).astype(np.int64)
    _say("permutation", name, P)
    d2 = H.upload(wl, step)
    H.gpu_step(wl, step, d2, P)
    assert H.bits(d2["out"]).tobytes() == out1.tobytes()


@pytest.mark.parametrize("name,P", [("gqa70b", 512), ("mha7b", 0)])
def test_deterministic_across_runs(name, P):
    wl = _wl(name, num_seqs=8)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P)
    first = H.bits(d["out"]).copy()
    for _ in range(3):
        H.gpu_step(wl, step, d, P)
        assert H.bits(d["out"]).tobytes() == first.tobytes()


@pytest.mark.parametrize("name,P", [("gqa70b", 256), ("mha7b", 0), ("tiny_fp32", 0)])
def test_unread_slots_and_table_padding_never_read(name, P):
    wl = _wl(name, num_seqs=6)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P)
    clean = H.bits(d["out"]).copy()
    # poison: NaN in every slot past ctx in each last block, and a NaN block behind the padding
    B = wl.cfg.block_size
    nan = np.uint16(0x7FC1) if wl.cfg.dtype == "bf16" else np.float32("nan")
    used = set(step.block_tables[step.block_tables >= 0].ravel().tolist())
    spare = [b for b in range(wl.num_blocks) if b not in set(np.concatenate(
        [step.block_tables[s, :-(-int(c) // B)] for s, c in enumerate(step.context_lens)]).tolist())]
    assert spare, "pool has no spare block"
    poison = spare[0]
    wl.k_cache[poison] = nan
    wl.v_cache[poison] = nan
    for s, c in enumerate(step.context_lens.tolist()):
        nb = -(-c // B)
        last = step.block_tables[s, nb - 1]
        wl.k_cache[last, c - (nb - 1) * B:] = nan
        wl.v_cache[last, c - (nb - 1) * B:] = nan
        step.block_tables[s, nb:] = poison
    del used
    _say("poison", name, P)
    d2 = H.upload(wl, step)
    H.gpu_step(wl, step, d2, P)
    assert H.bits(d2["out"]).tobytes() == clean.tobytes()


@pytest.mark.parametrize("B", [4, 8])
def test_small_blocks_padding_never_read(B):
    # several blocks per 16-token tile: a tile's trailing blocks past the context are never
    # read, whatever their table entries hold (a NaN block, -1, an id past the pool)
    cfg = workloads.Config("smallblk", "bf16", 7, 16, 4, 128, B, ("uniform", 1, 90), seed=300 + B)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    for P in (0, 3 * B):
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P, do_copy=False, do_write=False)
        clean = H.bits(d["out"]).copy()
        attended = set(np.concatenate([step.block_tables[s, :-(-int(c) // B)]
                                       for s, c in enumerate(step.context_lens)]).tolist())
        poison = [b for b in range(wl.num_blocks) if b not in attended][0]
        kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
        wl.k_cache[poison] = np.uint16(0x7FC1)
        wl.v_cache[poison] = np.uint16(0x7FC1)
        for pad in (poison, -1, wl.num_blocks + 7):
            tables = step.block_tables.copy()
            for s, c in enumerate(step.context_lens.tolist()):
                tables[s, -(-c // B):] = pad
            st2 = pbatch.DecodeStep(**{**step.__dict__, "block_tables": tables})
            _say("small-block padding", B, "P", P, "pad", pad)
            d2 = H.upload(wl, st2)
            H.gpu_step(wl, st2, d2, P, do_copy=False, do_write=False)
            assert H.bits(d2["out"]).tobytes() == clean.tobytes()
        wl.k_cache[:], wl.v_cache[:] = kc, vc


# ---------------------------------------------------------------------------
# head-major cache layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,B", [("bf16", 16), ("bf16", 128), ("f32", 32)])
def test_head_major_write_and_copy_bit_exact(dt, B):
    cfg = workloads.Config("hm", dt, 6, 16, 4, 128, B, ("uniform", 1, 3 * B), seed=400 + B)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    khm, vhm = pbatch.to_head_major(d["k_cache"], d["v_cache"])
    _say("head-major write", dt, B)
    binding.paged_kv_write_head_major(d["k_new"], d["v_new"], khm, vhm, d["slot_mapping"])
    o = H.oracle_step(wl, "steady", attend=False)[0]
    rk, rv = oracle.head_major_from_rows(wl.k_cache, wl.v_cache)
    oracle.kv_write_head_major(wl.k_new, wl.v_new, rk, rv, o["slot_mapping"])
    import torch
    torch.cuda.synchronize()
    assert H.bits(khm).tobytes() == rk.tobytes() and H.bits(vhm).tobytes() == rv.tobytes()
    rng = np.random.default_rng(B)
    perm = rng.permutation(wl.num_blocks)
    npairs = wl.num_blocks // 2
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int64)
    _say("head-major copy", dt, B, pairs.shape)
    binding.copy_blocks_head_major(khm, vhm, pbatch.to_torch(pairs, "cuda"))
    torch.cuda.synchronize()
    oracle.copy_blocks(rk.reshape(rk.shape[0], -1, 1, 1), rv.reshape(rv.shape[0], -1, 1, 1), pairs)
    assert H.bits(khm).tobytes() == rk.tobytes() and H.bits(vhm).tobytes() == rv.tobytes()


HM_SHAPES = [
    # S, Hq, Hkv, B, ctx range, partition sizes
    (5, 16, 2, 16, (1, 700), (0, 64)),      # g = 8
    (4, 8, 8, 16, (1, 600), (0, 128)),      # g = 1
    (4, 24, 8, 32, (1, 500), (0, 96)),      # g = 3, B = 32
    (3, 16, 4, 128, (1, 1500), (0, 256)),   # g = 4, B = 128
    (3, 8, 2, 64, (4200, 9000), (0, 512, 1024)),  # more than 64 tiles per wave; both load rings
    (3, 4, 4, 128, (4200, 9000), (0, 512, 1024)), # g = 1 (VALU tiles), more than 64 tiles per wave
]


@pytest.mark.parametrize("shape", HM_SHAPES, ids=[f"g{s[1]//s[2]}-B{s[3]}" for s in HM_SHAPES])
def test_head_major_attention_parity(shape):
    S, Hq, Hkv, B, (lo, hi), parts = shape
    cfg = workloads.Config("hm", "bf16", S, Hq, Hkv, 128, B, ("uniform", lo, hi), seed=500 + Hq + B)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    for P in parts:
        _say("head-major attention", shape, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P, do_attn=False)        # copies and write on the row layout ...
        khm, vhm = pbatch.to_head_major(d["k_cache"], d["v_cache"])   # ... then placed head-major
        binding.paged_attention_decode_head_major(d["out"], d["q"], khm, vhm, d["block_tables"],
                                                  d["context_lens"], step.max_context_len, wl.scale, P)
        o, kc, vc, _ = H.oracle_step(wl, "steady", P, attend=False)
        rk, rv = oracle.head_major_from_rows(kc, vc)
        ref = oracle.attention_head_major(wl.q, rk, rv, o["block_tables"], o["context_lens"], wl.scale, P)
        H.check_close(H.bits(d["out"]), ref, "bf16", f"head-major {shape} P={P}")


@pytest.mark.parametrize("heads", [(32, 4), (8, 8)], ids=["g8", "g1"])
def test_head_major_unread_slots_and_padding_never_read(heads):
    cfg = workloads.Config("hm", "bf16", 6, heads[0], heads[1], 128, 16, ("uniform", 1, 200), seed=611)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    import torch
    for P in (0, 48):
        d = H.upload(wl, step)
        khm, vhm = pbatch.to_head_major(d["k_cache"], d["v_cache"])
        binding.paged_attention_decode_head_major(d["out"], d["q"], khm, vhm, d["block_tables"],
                                                  d["context_lens"], step.max_context_len, wl.scale, P)
        clean = H.bits(d["out"]).copy()
        B = cfg.block_size
        attended = set(np.concatenate([step.block_tables[s, :-(-int(c) // B)]
                                       for s, c in enumerate(step.context_lens)]).tolist())
        poison = [b for b in range(wl.num_blocks) if b not in attended][0]
        kp, vp = wl.k_cache.copy(), wl.v_cache.copy()
        kp[poison] = np.uint16(0x7FC1)
        vp[poison] = np.uint16(0x7FC1)
        tables = step.block_tables.copy()
        for s, c in enumerate(step.context_lens.tolist()):
            nb = -(-c // B)
            last = tables[s, nb - 1]
            kp[last, c - (nb - 1) * B:] = np.uint16(0x7FC1)
            vp[last, c - (nb - 1) * B:] = np.uint16(0x7FC1)
            tables[s, nb:] = poison
        _say("head-major poison", P)
        khm, vhm = pbatch.to_head_major(pbatch.to_torch(kp, "cuda", True), pbatch.to_torch(vp, "cuda", True))
        tb = pbatch.to_torch(tables, "cuda")
        binding.paged_attention_decode_head_major(d["out"], d["q"], khm, vhm, tb, d["context_lens"],
                                                  step.max_context_len, wl.scale, P)
        torch.cuda.synchronize()
        assert H.bits(d["out"]).tobytes() == clean.tobytes()


@pytest.mark.parametrize("name", ["gqa70b", "mha7b", "long_splitk"])
def test_head_major_full_size_parity(name):
    # every output element of the full-size configuration on head-major caches
    wl = _wl(name)
    step = pbatch.step_for(wl)
    for P in ((0, 2048) if name == "gqa70b" else (BENCH_PARTITION[name],)):
        _say("head-major full", name, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P, do_attn=False)
        khm, vhm = pbatch.to_head_major(d["k_cache"], d["v_cache"])
        binding.paged_attention_decode_head_major(d["out"], d["q"], khm, vhm, d["block_tables"],
                                                  d["context_lens"], step.max_context_len, wl.scale, P)
        o, kc, vc, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(d["out"]), ref, "bf16", f"head-major full {name} P={P}")
        del khm, vhm, d


@pytest.mark.parametrize("heads", [(4, 4), (8, 2)], ids=["g1", "g4"])
def test_most_partitions_per_head(heads):
    # 131072 tokens in 16-token partitions: 8192 partials per head, the most the merge stages in
    # LDS, plus a short sequence that finishes in pass 1
    Hq, Hkv = heads
    ctx = np.array([131072, 9], np.int64)
    cfg = workloads.Config("maxparts", "bf16", 2, Hq, Hkv, 128, 16, ("uniform", 1, 2), seed=71 + Hq)
    wl = workloads.make_workload(cfg, ctx_override=ctx)
    step = pbatch.step_for(wl)
    _say("most partitions", heads, ctx.tolist())
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 16)
    _, _, _, ref = H.oracle_step(wl, "steady", 16)
    H.check_close(H.bits(d["out"]), ref, "bf16", f"8192 partitions {heads}")


def test_split_matches_unsplit_within_tolerance():
    wl = _wl("gqa70b", num_seqs=10)
    step = pbatch.step_for(wl)
    outs = {}
    for P in (0, 256, 512, 1024):
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        outs[P] = H.widen(H.bits(d["out"]))
    for P in (256, 512, 1024):
        assert np.max(np.abs(outs[P] - outs[0])) <= 2 * H.BF16_MAX_ABS


# ---------------------------------------------------------------------------
# full-size configurations, in the bench's launch configuration, every output element
# ---------------------------------------------------------------------------

from bench import PARTITION as BENCH_PARTITION  # noqa: E402  (the partitions bench.py times)
from bench import partition_for as bench_partition  # noqa: E402


@pytest.mark.parametrize("name", ["tiny_fp32", "mha7b", "gqa70b", "long_splitk", "fork_cow"])
def test_full_size_parity(name):
    # the whole [S, Hq, D] output of each configuration at its full size against the fp64 oracle,
    # and both pools after the step's copies and writes bit for bit
    wl = _wl(name)
    whiches = ["fork", "steady"] if name == "fork_cow" else ["steady"]
    for which in whiches:
        step = pbatch.step_for(wl, which)
        P = bench_partition(name, wl.cfg, step)
        _say("full", name, which, "S", wl.cfg.num_seqs, "P", P, "pool", wl.k_cache.shape)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        o, kc, vc, ref = H.oracle_step(wl, which, P)
        assert np.array_equal(o["block_tables"], step.block_tables) and np.array_equal(o["copy_pairs"],
                                                                                      step.copy_pairs)
        H.check_close(H.bits(d["out"]), ref, wl.cfg.dtype, f"full {name}/{which} P={P}")
        assert np.array_equal(H.bits(d["k_cache"]), kc), f"{name}/{which}: K pool"
        assert np.array_equal(H.bits(d["v_cache"]), vc), f"{name}/{which}: V pool"
        del d, kc, vc


# ---------------------------------------------------------------------------
# device-side value handling (bounds checks in the kernels turn these into values)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_seqs,P", [(4, 0), (4, 256), (100, 0), (300, 256)])
def test_bad_device_values_give_defined_outputs(num_seqs, P):
    # the three forms of the schedule build (one wave, a wave per chunk, many chunks), split or not
    import torch
    wl = _wl("gqa70b", num_seqs=num_seqs)
    step = pbatch.step_for(wl)
    _say("bad values", num_seqs, "P", P)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P)
    good = H.bits(d["out"]).copy()
    # seq 0: context 0 -> zeros; seq 1: a table entry outside the pool -> NaN;
    # seq 2: context above the host bound -> NaN; seq 3 unaffected
    ctx = d["context_lens"].clone()
    ctx[0] = 0
    ctx[2] = step.max_context_len + 5
    bt = d["block_tables"].clone()
    bt[1, 0] = wl.num_blocks + 1000
    out = torch.empty_like(d["out"])
    binding.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], bt, ctx, step.max_context_len,
                                   wl.scale, P)
    torch.cuda.synchronize()
    o = H.widen(H.bits(out))
    assert (o[0] == 0).all()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all()
    assert H.bits(out)[3:].tobytes() == good[3:].tobytes()


# ---------------------------------------------------------------------------
# scheduling: persistent work queue and the large-batch fallback
# ---------------------------------------------------------------------------

# The merge of partial states inside the first launch (its own workgroups merging once their
# items are done, no second kernel) was built and taken out again: its first GPU run of the
# partition-64 GQA case did not finish within the test's time limit, twice (a stale poll of the
# arrival counters was found and fixed between the two runs; the second cause was not found).
# These cases stay here, skipped, for whoever takes it up again.
MERGE_INSIDE_SKIP = pytest.mark.skip(reason="merge inside the first launch: taken out after two GPU runs "
                                            "of its first case did not finish")


@pytest.mark.parametrize("name,P", [("gqa70b", 512), ("mha7b", 0), ("tiny_fp32", 8),
                                    pytest.param("gqa70b", 64, marks=MERGE_INSIDE_SKIP)])
def test_work_queue_counters_return_to_zero(name, P):
    import torch
    wl = _wl(name, num_seqs=min(12, workloads.CONFIGS[name].num_seqs))
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)          # the step's copies and write, as the oracle does
    cfg = wl.cfg
    ws = torch.zeros(binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim,
                                                      step.max_context_len, P), dtype=torch.uint8, device="cuda")
    first = None
    for _ in range(3):
        binding.paged_attention_decode(d["out"], d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                       d["context_lens"], step.max_context_len, wl.scale, P, ws)
        torch.cuda.synchronize()
        assert not ws[:8].any().item(), "work-queue counters must be zero after a call"
        got = H.bits(d["out"]).copy()
        if first is None:
            first = got
        assert got.tobytes() == first.tobytes()
    _, _, _, ref = H.oracle_step(wl, "steady", P)
    H.check_close(first, ref, cfg.dtype, f"queue {name}")


@pytest.mark.parametrize("name,P", [("mha7b", 0), ("gqa70b", 512)])
def test_back_to_back_calls_share_a_workspace(name, P):
    # calls queued on one stream with no synchronization between them, on one workspace: each
    # starts after the one before has finished and reset the queue counters, so every output
    # equals the output of a lone call
    import torch
    wl = _wl(name, num_seqs=24)
    step = pbatch.step_for(wl)
    cfg = wl.cfg
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P)
    want = H.bits(d["out"]).copy()
    ws = torch.zeros(binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim,
                                                      step.max_context_len, P), dtype=torch.uint8, device="cuda")
    outs = [torch.full_like(d["out"], float("nan")) for _ in range(6)]
    _say("back to back", name, "P", P)
    for o in outs:
        binding.paged_attention_decode(o, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                       d["context_lens"], step.max_context_len, wl.scale, P, ws)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert H.bits(o).tobytes() == want.tobytes(), f"call {i}"
    assert not ws[:8].any().item()


def test_two_streams_with_their_own_workspaces():
    # two decode steps in flight at once on two streams (default priority), each with its own
    # pool, output and workspace: the persistent launches share the CUs and nothing else
    import torch
    cases = []
    for name, P in (("mha7b", 0), ("gqa70b", 512)):
        wl = _wl(name, num_seqs=16)
        step = pbatch.step_for(wl)
        cfg = wl.cfg
        d = H.upload(wl, step)
        ws = torch.zeros(binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim,
                                                          step.max_context_len, P), dtype=torch.uint8, device="cuda")
        cases.append((wl, step, d, ws, P))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    _say("two streams")
    for (wl, step, d, ws, P), st in zip(cases, streams):
        with torch.cuda.stream(st):
            binding.paged_kv_write(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
            for _ in range(3):
                binding.paged_attention_decode(d["out"], d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                               d["context_lens"], step.max_context_len, wl.scale, P, ws)
    torch.cuda.synchronize()
    for wl, step, d, ws, P in cases:
        _, kc, _, ref = H.oracle_step(wl, "steady", P)
        assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
        H.check_close(H.bits(d["out"]), ref, wl.cfg.dtype, f"two streams {wl.cfg.name}")
        assert not ws[:8].any().item()


@pytest.mark.parametrize("as_handle", [False, True], ids=["torch-stream", "raw-handle"])
def test_explicit_stream_without_workspace(as_handle):
    # a side stream passed as `stream=` with no workspace: the binding zeroes a fresh workspace on
    # that stream and keeps it until the launch is done; torch's current stream stays idle
    import torch
    wl = _wl("gqa70b", num_seqs=12)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_attn=False)
    side = torch.cuda.Stream()
    st = side.cuda_stream if as_handle else side
    outs = []
    _say("explicit stream", "handle" if as_handle else "torch stream")
    for P in (512, 0, 512):
        o = torch.full_like(d["out"], float("nan"))
        side.wait_stream(torch.cuda.current_stream())
        binding.paged_attention_decode(o, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                       step.max_context_len, wl.scale, P, stream=st)
        outs.append((P, o))
    side.synchronize()
    for P, o in outs:
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(o), ref, "bf16", f"explicit stream P={P}")


@pytest.mark.parametrize("name,num_seqs,which,P", [("fork_cow", None, "fork", 512), ("mha7b", 6, "steady", 0)])
def test_pool_beyond_4_gib(name, num_seqs, which, P):
    # every block the step touches lies past the first 4 GiB of a pool of more than 4 GiB per
    # tensor (the oracle's pool holds the same blocks under their own ids, which relabelling does
    # not change): slots, copies and table entries address it with 64-bit offsets
    import torch
    wl = _wl(name, num_seqs=num_seqs)
    step = pbatch.step_for(wl, which)
    cfg = wl.cfg
    n_small = wl.num_blocks
    block_bytes = cfg.block_size * cfg.num_kv_heads * cfg.head_dim * cfg.elem_bytes
    first = -(-(4 << 30) // block_bytes)            # first block wholly past 4 GiB
    span = 1 << max(10, (n_small - 1).bit_length())
    n_big = first + span
    new_id = first + (np.arange(n_small, dtype=np.int64) * 7) % span   # distinct, scattered
    _say("pool beyond 4 GiB", name, "blocks", n_big, "bytes per tensor", n_big * block_bytes)
    big = {}
    for key in ("k_cache", "v_cache"):
        t = torch.empty((n_big,) + tuple(wl.k_cache.shape[1:]), dtype=torch.bfloat16, device="cuda")
        t[torch.from_numpy(new_id).cuda()] = pbatch.to_torch(getattr(wl, key), "cuda", True)
        big[key] = t
    d = H.upload(wl, step)
    del d["k_cache"], d["v_cache"]
    B = cfg.block_size
    slots = step.slot_mapping.astype(np.int64)
    slots_big = new_id[slots // B] * B + slots % B
    pairs_big = new_id[step.copy_pairs.astype(np.int64)].reshape(-1, 2) if step.copy_pairs.size else step.copy_pairs
    tables_big = new_id[np.clip(step.block_tables.astype(np.int64), 0, n_small - 1)].astype(np.int32)
    if pairs_big.size:
        binding.copy_blocks(big["k_cache"], big["v_cache"], pbatch.to_torch(np.ascontiguousarray(pairs_big), "cuda"))
    binding.paged_kv_write(d["k_new"], d["v_new"], big["k_cache"], big["v_cache"], pbatch.to_torch(slots_big, "cuda"))
    binding.paged_attention_decode(d["out"], d["q"], big["k_cache"], big["v_cache"], pbatch.to_torch(tables_big, "cuda"),
                                   d["context_lens"], step.max_context_len, wl.scale, P)
    torch.cuda.synchronize()
    _, kc, vc, ref = H.oracle_step(wl, which, P)
    idx = torch.from_numpy(new_id).cuda()
    assert H.bits(big["k_cache"][idx]).tobytes() == kc.tobytes()
    assert H.bits(big["v_cache"][idx]).tobytes() == vc.tobytes()
    H.check_close(H.bits(d["out"]), ref, cfg.dtype, f"beyond 4 GiB {name}")
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_seqs", [40, 100, 200, 300, 4096])
def test_persistent_schedule_many_sequences(num_seqs):
    # the persistent path's longest-first schedule: one wave (up to 64 sequences), one wave per
    # 64-sequence chunk (up to 256, some waves without a chunk), and many chunks up to the most
    # sequences it stages in LDS: every item exactly once, with full and last partitions mixed
    cfg = workloads.Config("chunks", "bf16", num_seqs, 8, 2, 128, 16, ("uniform", 1, 400), seed=31 + num_seqs)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    for P in (0, 128):
        _say("persistent schedule", num_seqs, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(H.bits(d["out"]), ref, "bf16", f"chunks S={num_seqs} P={P}")


def test_large_batch_uses_fallback_grid():
    # more sequences than the persistent schedule stages in LDS: one workgroup per item
    cfg = workloads.Config("many", "bf16", 4500, 8, 2, 128, 16, ("uniform", 1, 40), seed=77)
    wl = workloads.make_workload(cfg)
    step = pbatch.step_for(wl)
    rng = np.random.default_rng(1)
    items = np.unique(rng.integers(0, cfg.num_seqs * cfg.num_heads, size=200))
    for P in (0, 16):
        _say("fallback grid", cfg.num_seqs, "P", P)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P)
        _, _, _, ref = H.oracle_step(wl, "steady", P, items=items)
        got = H.bits(d["out"]).reshape(cfg.num_seqs * cfg.num_heads, -1)[items]
        H.check_close(got, ref, "bf16", f"fallback P={P}")


# ---------------------------------------------------------------------------
# the decode step replayed from a HIP graph
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,num_seqs,P,which,fused", [("mha7b", 8, 0, "steady", False),
                                                         ("gqa70b", 16, 512, "steady", False),
                                                         ("fork_cow", None, 512, "fork", False),
                                                         ("tiny_fp32", None, 8, "steady", False),
                                                         ("mha7b", 8, 0, "steady", True),
                                                         ("fork_cow", None, 1024, "fork", True)])
def test_decode_step_replays_from_a_hip_graph(name, num_seqs, P, which, fused):
    # copy_blocks -> paged_kv_write -> paged_attention_decode (or copy_blocks ->
    # paged_attention_decode_write) captured once and replayed: the calls allocate and clear
    # nothing, and each attention call leaves its queue counters at zero, so every replay -- with
    # eager calls on the same workspace and torch's own kernels in between -- gives the eager
    # step's caches and output bit for bit
    import torch
    wl = _wl(name, num_seqs=num_seqs)
    cfg = wl.cfg
    step = pbatch.step_for(wl, which)
    ws = torch.zeros(binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim,
                                                      step.max_context_len, P), dtype=torch.uint8, device="cuda")

    def run(d, out):
        if step.copy_pairs.shape[0]:
            binding.copy_blocks(d["k_cache"], d["v_cache"], d["copy_pairs"])
        if fused:
            binding.paged_attention_decode_write(out, d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                                 d["block_tables"], d["context_lens"], step.max_context_len,
                                                 wl.scale, P, ws)
            return
        binding.paged_kv_write(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
        binding.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                       d["context_lens"], step.max_context_len, wl.scale, P, ws)

    _say("graph eager", name, which, "P", P)
    d = H.upload(wl, step)
    run(d, d["out"])
    torch.cuda.synchronize()
    want_out, want_k, want_v = H.bits(d["out"]).copy(), H.bits(d["k_cache"]).copy(), H.bits(d["v_cache"]).copy()
    _, _, _, ref = H.oracle_step(wl, which, P)
    H.check_close(want_out, ref, cfg.dtype, f"graph eager {name}")

    g = H.upload(wl, step)
    other = torch.empty_like(g["out"])
    graph = torch.cuda.CUDAGraph()
    _say("graph capture", name)
    with torch.cuda.graph(graph):
        run(g, g["out"])
    for rep in range(4):
        _say("graph replay", name, rep)
        g["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert H.bits(g["out"]).tobytes() == want_out.tobytes(), f"replay {rep}: output"
        assert H.bits(g["k_cache"]).tobytes() == want_k.tobytes(), f"replay {rep}: k_cache"
        assert H.bits(g["v_cache"]).tobytes() == want_v.tobytes(), f"replay {rep}: v_cache"
        assert not ws[:8].any().item(), f"replay {rep}: queue counters"
        # eager work between replays: the same step on the same workspace into another buffer
        run(g, other)
        torch.cuda.synchronize()
        assert H.bits(other).tobytes() == want_out.tobytes(), f"eager after replay {rep}"


def test_stream_read_probe_runs():
    # the measurement-only read: it runs over a buffer that is not a multiple of its loop's
    # stride and of 16 bytes, and leaves the buffer as it was
    import torch
    buf = torch.arange((3 << 20) + 5, dtype=torch.int32, device="cuda").view(torch.uint8)[: (12 << 20) + 7]
    before = buf.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


# ---------------------------------------------------------------------------
# the write fused into the attention launch
# ---------------------------------------------------------------------------

FUSED = [
    # workload or shape, sequences, step, partition sizes
    ("mha7b", 6, "steady", (0, 512)),
    ("gqa70b", 12, "steady", (0, 256, 2048)),
    ("fork_cow", None, "fork", (512, 0)),
    ("long_splitk", None, "steady", (512,)),
    (("bf16", 4, 8, 8, 128, 4, (1, 300)), None, "steady", (0, 64)),      # g = 1, B = 4
    (("bf16", 4, 6, 2, 128, 8, (1, 200)), None, "steady", (0, 48)),      # g = 3, B = 8
    (("bf16", 4, 24, 8, 128, 32, (1, 400)), None, "steady", (0, 128)),   # g = 3, B = 32
    (("bf16", 3, 16, 2, 128, 128, (1, 2600)), None, "steady", (0, 512)), # g = 8, B = 128
    ("tiny_fp32", None, "steady", (0, 8)),                                # the vector path
    (("bf16", 4, 16, 2, 64, 8, (1, 200)), None, "steady", (0, 64)),      # vector, D = 64, g = 8
]


def _fused_wl(spec, num_seqs):
    if isinstance(spec, str):
        if spec == "long_splitk":
            return _wl(spec, ctx=np.array([5000, 12345, 1, 700], np.int64))
        return _wl(spec, num_seqs=num_seqs)
    dt, S, Hq, Hkv, D, B, (lo, hi) = spec
    return workloads.make_workload(workloads.Config("fused", dt, S, Hq, Hkv, D, B, ("uniform", lo, hi), seed=7 + Hq + B))


@pytest.mark.parametrize("spec,num_seqs,which,parts", FUSED, ids=[str(f[0]) if isinstance(f[0], str) else
                                                              f"g{f[0][2] // f[0][3]}-B{f[0][5]}" for f in FUSED])
def test_fused_write_equals_write_then_attend(spec, num_seqs, which, parts):
    # paged_attention_decode_write gives the caches and the output of paged_kv_write followed by
    # paged_attention_decode, bit for bit (the slot comes from the table, the new rows from
    # k_new / v_new), and those are the oracle's: in one launch on the tile paths, as a launch of
    # its own before the attention for short MFMA partitions and on the vector path
    import torch
    wl = _fused_wl(spec, num_seqs)
    step = pbatch.step_for(wl, which)
    for P in parts:
        _say("fused write", wl.cfg.name, which, "P", P)
        d1 = H.upload(wl, step)
        H.gpu_step(wl, step, d1, P)
        d2 = H.upload(wl, step)
        if step.copy_pairs.shape[0]:
            binding.copy_blocks(d2["k_cache"], d2["v_cache"], d2["copy_pairs"])
        binding.paged_attention_decode_write(d2["out"], d2["q"], d2["k_new"], d2["v_new"], d2["k_cache"],
                                             d2["v_cache"], d2["block_tables"], d2["context_lens"],
                                             step.max_context_len, wl.scale, P)
        torch.cuda.synchronize()
        assert H.bits(d2["k_cache"]).tobytes() == H.bits(d1["k_cache"]).tobytes()
        assert H.bits(d2["v_cache"]).tobytes() == H.bits(d1["v_cache"]).tobytes()
        assert H.bits(d2["out"]).tobytes() == H.bits(d1["out"]).tobytes()
        _, kc, vc, ref = H.oracle_step(wl, which, P)
        assert H.bits(d2["k_cache"]).tobytes() == kc.tobytes()
        assert H.bits(d2["v_cache"]).tobytes() == vc.tobytes()
        H.check_close(H.bits(d2["out"]), ref, wl.cfg.dtype, f"fused {wl.cfg.name}/{which} P={P}")


def test_fused_write_bad_values_write_nothing():
    # a sequence with context 0, one with a context above the host bound and one whose new
    # token's table entry lies outside the pool: their outputs as paged_attention_decode gives
    # them, and no byte of either pool changes for them; the others are written and attended
    import torch
    wl = _wl("gqa70b", num_seqs=6)
    step = pbatch.step_for(wl)
    B = wl.cfg.block_size
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_attn=False)
    written_k = H.bits(d["k_cache"]).copy()
    e = H.upload(wl, step)
    before_k = H.bits(e["k_cache"]).copy()
    ctx = e["context_lens"].clone()
    bt = e["block_tables"].clone()
    ctx[0] = 0
    ctx[2] = step.max_context_len + 5
    c3 = int(step.context_lens[3])
    bt[3, (c3 - 1) // B] = wl.num_blocks + 1000
    binding.paged_attention_decode_write(e["out"], e["q"], e["k_new"], e["v_new"], e["k_cache"], e["v_cache"], bt, ctx,
                                         step.max_context_len, wl.scale, 0)
    torch.cuda.synchronize()
    o = H.widen(H.bits(e["out"]))
    assert (o[0] == 0).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
    got_k = H.bits(e["k_cache"])
    slots = step.slot_mapping.tolist()
    for s_, sl in enumerate(slots):
        want = before_k if s_ in (0, 2, 3) else written_k
        assert got_k[sl // B, sl % B].tobytes() == want[sl // B, sl % B].tobytes(), f"sequence {s_}"
    H.gpu_step(wl, step, d, 0, do_copy=False, do_write=False)
    for s_ in (1, 4, 5):
        assert H.bits(e["out"])[s_].tobytes() == H.bits(d["out"])[s_].tobytes()



# ---------------------------------------------------------------------------
# wide work items: every width gives the same bits
# ---------------------------------------------------------------------------

def _attend(monkeypatch, wl, step, d, P, width):
    """paged_attention_decode with every work item `width` KV heads wide (PKV_WIDE_ITEMS; None:
    the library's own choice), on the inputs in d; returns the output's bits."""
    import torch
    if width is None:
        monkeypatch.delenv("PKV_WIDE_ITEMS", raising=False)
    else:
        monkeypatch.setenv("PKV_WIDE_ITEMS", str(width))
    out = torch.empty_like(d["q"])
    binding.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                   step.max_context_len, wl.scale, P)
    torch.cuda.synchronize()
    monkeypatch.delenv("PKV_WIDE_ITEMS", raising=False)
    return H.bits(out).copy()


@pytest.mark.parametrize("name,P,widths", [("long_splitk", 512, (1, 2, 4)), ("mha7b", 0, (1, 2, 4)),
                                           ("gqa70b", 2048, (1, 2))])
def test_wide_items_same_bits_full_size(monkeypatch, name, P, widths):
    # the library's choice (wide items for the bulk of these launches, one-head items at the
    # queue's end) and every forced width give the output of one-head items bit for bit
    wl = _wl(name)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)
    _say("wide items", name, "P", P)
    base = _attend(monkeypatch, wl, step, d, P, 1)
    for width in (None,) + widths[1:]:
        got = _attend(monkeypatch, wl, step, d, P, width)
        assert got.tobytes() == base.tobytes(), f"{name}: width {width}"
    _, _, _, ref = H.oracle_step(wl, "steady", P)
    H.check_close(got, ref, "bf16", f"{name} width {widths[-1]} P={P}")


@pytest.mark.parametrize("name,P,window", [("mha7b", 0, None), ("long_splitk", 512, None), ("long_splitk", 512, 64),
                                           ("long_splitk", 512, 1024)])
def test_near_pool_one_head_loop_same_bits(monkeypatch, name, P, window):
    # an identity-ordered pool (each sequence's blocks consecutive; window None) or one shuffled
    # only within windows of `window` block ids (2 MB or 32 MB of 32 KB blocks): the batch shape
    # picks the wide-item kernel, whose sample finds the blocks close together (identity, 2 MB:
    # the one-head item loop) or far enough apart (32 MB: wide items); either way the output is
    # the one-head kernel's bit for bit and within the oracle's tolerance
    wl = _wl(name)
    ids = np.arange(wl.num_blocks)
    if window is not None:
        rng = np.random.default_rng(7)
        for i in range(0, wl.num_blocks, window):
            ids[i:i + window] = rng.permutation(ids[i:i + window])
        ids = ids[::-1]
    wl.free_order = [int(x) for x in ids]
    step = pbatch.step_for(wl)
    if window is None:
        assert np.all(np.diff(step.block_tables[0, :8]) == 1)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)
    _say("near pool", name, "P", P, "window", window)
    base = _attend(monkeypatch, wl, step, d, P, 1)
    got = _attend(monkeypatch, wl, step, d, P, None)
    assert got.tobytes() == base.tobytes(), name
    _, _, _, ref = H.oracle_step(wl, "steady", P)
    H.check_close(got, ref, "bf16", f"{name} pool window {window} P={P}")


WIDE_SHAPES = [
    # S, Hq, Hkv, B, ctx range, partition sizes
    (5, 8, 8, 16, (1, 700), (0, 64)),        # g = 1 (VALU dots)
    (4, 16, 8, 32, (1, 900), (0, 128)),      # g = 2
    (4, 24, 8, 32, (1, 400), (0, 128)),      # g = 3: a KV head's rows straddle the waves' rows
    (6, 32, 8, 16, (1, 1300), (0, 512)),     # g = 4, the deep ring
    (3, 64, 8, 64, (1, 2600), (0, 256)),     # g = 8, B = 64, more than 64 tiles per wave
    (4, 32, 8, 128, (1, 1000), (0, 512)),    # g = 4, B = 128
    (3, 12, 4, 16, (4000, 9000), (1024,)),   # g = 3, long partitions (shallow ring)
]


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=[f"g{s[1] // s[2]}-B{s[3]}" for s in WIDE_SHAPES])
def test_wide_items_same_bits(monkeypatch, shape):
    # every item of the launch 2 or 4 KV heads wide (all that the group allows), against one-head
    # items: the same bits, ragged contexts (1 token included) and the oracle's tolerance
    S, Hq, Hkv, B, (lo, hi), parts = shape
    cfg = workloads.Config("wide", "bf16", S, Hq, Hkv, 128, B, ("uniform", lo, hi), seed=50 + Hq + B)
    wl = workloads.make_workload(cfg)
    wl.context_lens[0] = 1
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, 0, do_attn=False)
    g = Hq // Hkv
    widths = [w for w in (2, 4) if Hkv % w == 0 and w * g <= 16]
    assert widths
    for P in parts:
        _say("wide items", shape, "P", P)
        base = _attend(monkeypatch, wl, step, d, P, 1)
        for width in widths:
            got = _attend(monkeypatch, wl, step, d, P, width)
            assert got.tobytes() == base.tobytes(), f"width {width} P={P}"
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(base, ref, "bf16", f"{shape} P={P}")


@pytest.mark.parametrize("name,num_seqs,P", [("gqa70b", 12, 256), ("mha7b", 6, 0), ("long_splitk", None, 512)])
def test_wide_items_fused_write_same_bits(monkeypatch, name, num_seqs, P):
    # the fused write inside wide items: caches and output bit for bit those of one-head items
    import torch
    wl = _fused_wl(name, num_seqs)
    step = pbatch.step_for(wl)
    res = {}
    g = wl.cfg.num_heads // wl.cfg.num_kv_heads
    for width in [1] + [w for w in (2, 4) if wl.cfg.num_kv_heads % w == 0 and w * g <= 16]:
        _say("wide fused", name, "P", P, "width", width)
        monkeypatch.setenv("PKV_WIDE_ITEMS", str(width))
        d = H.upload(wl, step)
        binding.paged_attention_decode_write(d["out"], d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                             d["block_tables"], d["context_lens"], step.max_context_len, wl.scale, P)
        torch.cuda.synchronize()
        res[width] = [H.bits(d[k]).tobytes() for k in ("out", "k_cache", "v_cache")]
    monkeypatch.delenv("PKV_WIDE_ITEMS", raising=False)
    for width, r in res.items():
        assert r == res[1], f"width {width}"


@pytest.mark.parametrize("P", [0, 256])
def test_wide_items_bad_values(monkeypatch, P):
    # unusable lengths and table entries inside wide items: zeros / NaN for those sequences (every
    # KV head of them), the other sequences as with one-head items
    import torch
    wl = _wl("gqa70b", num_seqs=40)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)
    ctx = d["context_lens"].clone()
    ctx[0] = 0
    ctx[2] = step.max_context_len + 5
    d["block_tables"][1, 0] = wl.num_blocks + 1000
    d["context_lens"] = ctx
    _say("wide bad values", "P", P)
    base = _attend(monkeypatch, wl, step, d, P, 1)
    got = _attend(monkeypatch, wl, step, d, P, 2)
    o = H.widen(got)
    assert (o[0] == 0).all()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all()
    assert got.tobytes() == base.tobytes()
    del torch


# ---------------------------------------------------------------------------
# the merge of partial states inside the first launch: the same bits as the second kernel
# ---------------------------------------------------------------------------

def _attend_env(monkeypatch, wl, step, d, P, env):
    import torch
    for k in ("PKV_MERGE_PASS", "PKV_WIDE_ITEMS"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    out = torch.empty_like(d["q"])
    binding.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                   step.max_context_len, wl.scale, P)
    torch.cuda.synchronize()
    for k in env:
        monkeypatch.delenv(k, raising=False)
    return H.bits(out).copy()


MERGE_CASES = [
    # workload, sequences or contexts, partition size
    ("long_splitk", None, 512),                                   # full size: 64 .. 256 partitions
    ("long_splitk", np.array([32768, 5000, 12345, 1, 700, 513], np.int64), 256),   # ragged, single-partition ones
    ("gqa70b", 24, 64),                                           # g = 8, > 16 partitions per head
    ("mha7b", 8, 64),                                             # g = 1 (VALU dots)
]


@MERGE_INSIDE_SKIP
@pytest.mark.parametrize("name,seqs,P", MERGE_CASES, ids=[f"{c[0]}-P{c[2]}-{i}" for i, c in enumerate(MERGE_CASES)])
def test_merge_inside_launch_same_bits(monkeypatch, name, seqs, P):
    # merged by the first launch's own workgroups (the default here) against the second kernel
    # (PKV_MERGE_PASS=1), with one-head and wide items: bit for bit, and the oracle's tolerance
    if isinstance(seqs, np.ndarray):
        wl = _wl(name, ctx=seqs)
    else:
        wl = _wl(name, num_seqs=seqs)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)
    _say("merge inside", name, "P", P)
    base = _attend_env(monkeypatch, wl, step, d, P, {"PKV_MERGE_PASS": "1", "PKV_WIDE_ITEMS": "1"})
    for env in ({}, {"PKV_WIDE_ITEMS": "1"}, {"PKV_WIDE_ITEMS": "2"}, {"PKV_MERGE_PASS": "1"}):
        got = _attend_env(monkeypatch, wl, step, d, P, env)
        assert got.tobytes() == base.tobytes(), f"{env}"
    _, _, _, ref = H.oracle_step(wl, "steady", P)
    H.check_close(base, ref, "bf16", f"merge inside {name} P={P}")


@MERGE_INSIDE_SKIP
def test_merge_inside_launch_reused_workspace():
    # one workspace for calls on different inputs and shapes in a row, each merged inside the
    # launch: every output against the oracle (records of an earlier call at the same addresses
    # must not be read), and the first inputs again give the first call's bits
    import torch
    P = 256
    wla = _wl("long_splitk", ctx=np.array([9000, 5000, 12345, 700], np.int64))
    wlb = _wl("long_splitk", ctx=np.array([12000, 4100, 300, 8000, 6000], np.int64), seed=11)
    steps = [pbatch.step_for(w) for w in (wla, wlb)]
    need = max(binding.attention_workspace_size(w.cfg.num_seqs, w.cfg.num_heads, w.cfg.head_dim, st.max_context_len, P)
               for w, st in zip((wla, wlb), steps))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for wl, step in ((wla, steps[0]), (wlb, steps[1]), (wla, steps[0])):
        _say("merge inside, reused workspace", wl.cfg.num_seqs)
        d = H.upload(wl, step)
        H.gpu_step(wl, step, d, P, do_attn=False)
        binding.paged_attention_decode(d["out"], d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                       d["context_lens"], step.max_context_len, wl.scale, P, ws)
        torch.cuda.synchronize()
        assert not ws[:8].any().item()
        got = H.bits(d["out"]).copy()
        _, _, _, ref = H.oracle_step(wl, "steady", P)
        H.check_close(got, ref, "bf16", f"reused workspace S={wl.cfg.num_seqs}")
        outs.append(got)
    assert outs[2].tobytes() == outs[0].tobytes()
