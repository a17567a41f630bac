"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: values printed
on the pages (tests/golden/), a library routine (torch's scaled_dot_product_attention
in float64), 50-digit brute force (mpmath), closed forms and invariants.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import batch as obatch
from oracle.blocks import BlockModel, PrefixModel, build_tables
from tests.conftest import golden
import workloads

# ---------------------------------------------------------------------------
# small seeded inputs
# ---------------------------------------------------------------------------


def _small(seed, S, Hq, Hkv, D, B, ctx_hi, dtype="f32", extra_blocks=3, ctx=None):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, ctx_hi, size=S, endpoint=True) if ctx is None else np.asarray(ctx)
    need = sum(-(-int(c) // B) for c in ctx)
    N = need + extra_blocks
    m = BlockModel(N, B, free_order=[int(x) for x in rng.permutation(N)])
    seqs = [m.new_sequence(int(c)) for c in ctx]
    maxblk = max(len(s["table"]) for s in seqs) + 1
    bt = build_tables(seqs, maxblk)
    q = workloads.normal(S * Hq * D, seed, 11, dtype).reshape(S, Hq, D)
    kc = workloads.normal(N * B * Hkv * D, seed, 12, dtype).reshape(N, B, Hkv, D)
    vc = workloads.normal(N * B * Hkv * D, seed, 13, dtype).reshape(N, B, Hkv, D)
    return q, kc, vc, bt, ctx.astype(np.int32), m, seqs


def _sdpa(q, kc, vc, bt, ctx, scale, m):
    """torch SDPA in float64 on K/V rows fetched slot by slot through the block model."""
    torch = pytest.importorskip("torch")
    S, Hq, D = q.shape
    N, B, Hkv, _ = kc.shape
    g = Hq // Hkv
    kflat = oracle.widen(kc).reshape(N * B, Hkv, D)
    vflat = oracle.widen(vc).reshape(N * B, Hkv, D)
    out = np.empty((S, Hq, D))
    for s in range(S):
        seq = {"table": [int(x) for x in bt[s]], "len": int(ctx[s])}
        slots = [m.physical_index(seq, t) for t in range(int(ctx[s]))]
        K = torch.from_numpy(kflat[slots]).permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq, ctx, D]
        V = torch.from_numpy(vflat[slots]).permute(1, 0, 2).repeat_interleave(g, dim=0)
        Q = torch.from_numpy(oracle.widen(q[s])).unsqueeze(1)                              # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        out[s] = o[:, 0, :].numpy()
    return out


# ---------------------------------------------------------------------------
# slot formula and block model: values printed on the pages
# ---------------------------------------------------------------------------

def test_physical_index_page_examples(oracle_lib):
    for c in golden("physical_index.json")["cases"]:
        assert oracle.physical_index(c["table"], c["block_size"], c["pos"]) == c["slot"], c["cite"]
        assert c["pos"] // c["block_size"] == c["logical_block"]
        assert c["table"][c["logical_block"]] == c["physical_block"]
        assert c["pos"] % c["block_size"] == c["offset"]
        m = BlockModel(100, c["block_size"])
        assert m.physical_index({"table": c["table"]}, c["pos"]) == c["slot"]
        sl = oracle.slot_mapping(np.array([c["table"]]), [c["pos"]], c["block_size"])
        assert int(sl[0]) == c["slot"]


def test_go_scenario_block_model():
    g = golden("go_scenario.json")
    m = BlockModel(g["num_blocks"], g["block_size"])
    seqs = {k: m.new_sequence(v) for k, v in g["prompts"].items()}
    for k, t in g["tables_after_admit"].items():
        assert seqs[k]["table"] == t
    assert m.free == g["free_after_admit"]
    m.release(seqs["b"]["table"])
    m.release(seqs["d"]["table"])
    assert m.free == g["free_after_freeing_b_then_d"]
    e = m.new_sequence(g["e_prompt"])
    assert (e is not None) == g["e_succeeds"]
    assert e["table"] == g["e_table"]
    assert m.physical_index(e, 40) == g["e_physical_index_40"]
    assert oracle.physical_index(e["table"], g["block_size"], 40) == g["e_physical_index_40"]
    m.check([seqs["a"], seqs["c"], e])


def test_sharing_counts():
    cases = golden("sharing.json")["cases"]
    # nano-vLLM Ch04 section 6: 3 requests on 2 shared blocks, then one private block each
    c = cases[0]
    m = BlockModel(100, 16)
    parent = m.new_sequence(c["shared_blocks"] * 16)
    reqs = [parent] + [{"table": m.fork(parent["table"]), "len": parent["len"]} for _ in range(c["requests"] - 1)]
    assert all(m.ref[b] == c["refcount_before"] for b in parent["table"])
    assert len(m.ref) == c["blocks_before"]
    for r in reqs:
        assert m.append_token(r)
    assert len(m.ref) == c["blocks_after_one_private_each"]
    assert c["requests"] * (c["shared_blocks"] + 1) == c["blocks_without_sharing"]
    m.check(reqs)
    # PidokuInfra section 5: n = 4 on 3 prompt blocks -> 7 blocks instead of 16
    c = cases[1]
    m = BlockModel(100, 16)
    parent = m.new_sequence(c["shared_blocks"] * 16)
    reqs = [parent] + [{"table": m.fork(parent["table"]), "len": parent["len"]} for _ in range(c["requests"] - 1)]
    for r in reqs:
        assert m.append_token(r)
    used = len(m.ref)
    assert used == c["blocks_after_one_private_each"]
    assert c["requests"] * (c["shared_blocks"] + 1) == c["blocks_without_sharing"]
    assert round(100 * (1 - used / c["blocks_without_sharing"])) == c["saved_percent"]
    # quiz 2: one set of prompt blocks, refcount = number of requests
    c = cases[2]
    m = BlockModel(100, 16)
    parent = m.new_sequence(48)
    kids = [m.fork(parent["table"]) for _ in range(c["requests"] - 1)]
    assert len({tuple(parent["table"])} | {tuple(k) for k in kids}) == c["sets_of_prompt_blocks"]
    assert all(m.ref[b] == c["requests"] for b in parent["table"])


def test_block_model_oom_leaves_state_unchanged():
    m = BlockModel(4, 16)
    a = m.new_sequence(48)
    before = (list(m.free), dict(m.ref))
    assert m.new_sequence(40) is None                 # needs 3, 1 free
    assert (list(m.free), dict(m.ref)) == before
    a2 = {"table": m.fork(a["table"]), "len": a["len"]}
    b = m.new_sequence(16)
    assert b is not None and not m.free
    before = (list(m.free), dict(m.ref), list(a2["table"]))
    with pytest.raises(Exception):
        m.write_slot(a2, 47)                          # shared block, no free block for the copy
    assert (list(m.free), dict(m.ref), list(a2["table"])) == before
    assert not m.append_token(b) or True
    m.check([a, a2, b])


def test_block_model_append_growth_rule():
    # grow exactly when BlocksNeeded(len) exceeds the table (PidokuInfra section 4)
    m = BlockModel(50, 16)
    s = m.new_sequence(1)
    assert len(s["table"]) == 1
    for n in range(2, 100):
        assert m.append_token(s)
        assert s["len"] == n and len(s["table"]) == -(-n // 16)
    m.check([s])


def test_block_model_random_ops_invariants():
    rng = np.random.default_rng(7)
    m = BlockModel(64, 4, free_order=[int(x) for x in rng.permutation(64)])
    live = []
    for _ in range(2000):
        op = rng.integers(0, 5)
        if op == 0:
            s = m.new_sequence(int(rng.integers(1, 20)))
            if s is not None:
                live.append(s)
        elif op == 1 and live:
            s = live[int(rng.integers(len(live)))]
            live.append({"table": m.fork(s["table"]), "len": s["len"]})
        elif op == 2 and live:
            s = live[int(rng.integers(len(live)))]
            if m.append_token(s):
                try:
                    m.write_slot(s, s["len"] - 1)
                except Exception:
                    pass
        elif op == 3 and live:
            s = live.pop(int(rng.integers(len(live))))
            m.release(s["table"])
        m.check(live)


# ---------------------------------------------------------------------------
# prefix reuse model: the pages' ten-copies case, and scenarios worked by hand
# ---------------------------------------------------------------------------

def _prompt(n, salt=0):
    return [(7 * i + salt) % 50021 for i in range(n)]


@pytest.mark.parametrize("case", golden("prefix_sharing.json")["cases"], ids=lambda c: f"{c['prompt_tokens']}")
def test_prefix_model_ten_requests_share_one_prompt(case):
    B = golden("prefix_sharing.json")["block_size"]
    L, R = case["prompt_tokens"], case["requests"]
    plain = BlockModel(2000, B)
    copies = [plain.new_sequence(L) for _ in range(R)]
    assert len(plain.ref) == case["blocks_without_sharing"]          # ten copies
    plain.check(copies)
    m = BlockModel(2000, B)
    pm = PrefixModel(m)
    res = [pm.new_sequence(_prompt(L)) for _ in range(R)]
    assert [h for _, h in res] == case["reused_blocks_per_request"]
    assert len(m.ref) == case["blocks_with_sharing"]
    shared = res[0][0]["table"][:case["full_blocks"]]
    assert all(r["table"][:case["full_blocks"]] == shared for r, _ in res)
    assert all(m.ref[b] == case["shared_refcount"] for b in shared)
    private = [b for r, _ in res for b in r["table"][case["full_blocks"]:]]
    assert len(private) == len(set(private)) == R * case["private_blocks_per_request"]
    m.check([r for r, _ in res])


def test_prefix_model_divergent_shifted_and_released():
    # B = 4, worked by hand: a block is reused only when every token up to its end matches
    m = BlockModel(64, 4)
    pm = PrefixModel(m)
    a, ha = pm.new_sequence([1, 2, 3, 4, 5, 6, 7, 8, 9])               # 2 full blocks + 1 slot
    b, hb = pm.new_sequence([1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 12, 13])  # both full blocks reused
    c, hc = pm.new_sequence([1, 2, 3, 4, 5, 6, 0, 8])                  # diverges inside block 1
    d, hd = pm.new_sequence([9, 9, 9, 9, 5, 6, 7, 8])                  # a's block 1 ids, other prefix
    assert (ha, hb, hc, hd) == (0, 2, 1, 0)
    assert b["table"][:2] == a["table"][:2] and b["table"][2] != a["table"][2]
    assert c["table"][0] == a["table"][0] and c["table"][1] not in a["table"]
    assert not set(d["table"]) & set(a["table"] + b["table"] + c["table"])
    assert len(a["table"]) == 3 and a["table"][2] not in b["table"]     # a's partial block is private
    assert m.ref[a["table"][0]] == 3 and m.ref[a["table"][1]] == 2
    assert len(m.ref) == 3 + 1 + 1 + 2                                 # a: 3, b: +1, c: +1, d: +2
    m.check([a, b, c, d])
    for s in (a, b, c):
        pm.release(s)
    e, he = pm.new_sequence([1, 2, 3, 4, 5, 6, 7, 8])                  # every holder gone: no hit
    assert he == 0 and len(pm.by_prefix) == 4                           # d's two blocks and e's two
    f, hf = pm.new_sequence([9, 9, 9, 9, 5, 6, 7, 8, 1])                # d's prefix is still held
    assert hf == 2 and f["table"][:2] == d["table"]
    m.check([d, e, f])


def test_prefix_model_same_block_ids_under_two_prefixes():
    # block 1 of [X, C] and of [Y, C] hold the same token ids but different KV (they attend to
    # different prefixes): a third prompt [X, C] must reuse the first prompt's blocks
    X, Y, C = [1, 1, 1, 1], [2, 2, 2, 2], [3, 3, 3, 3]
    m = BlockModel(32, 4)
    pm = PrefixModel(m)
    p1, _ = pm.new_sequence(X + C)
    p2, h2 = pm.new_sequence(Y + C)
    p3, h3 = pm.new_sequence(X + C)
    assert h2 == 0 and h3 == 2
    assert p3["table"] == p1["table"] and not set(p2["table"]) & set(p1["table"])
    m.check([p1, p2, p3])


def test_prefix_model_out_of_blocks_changes_nothing():
    m = BlockModel(6, 4)
    pm = PrefixModel(m)
    a, _ = pm.new_sequence(list(range(16)))                             # 4 blocks
    before = (m.free, m.ref, dict(pm.by_prefix))
    assert pm.new_sequence(list(range(8)) + [99] * 12) is None          # 2 hits + 3 new > 2 free
    assert (m.free, m.ref, dict(pm.by_prefix)) == before
    m.check([a])


# ---------------------------------------------------------------------------
# the fork workload's step inputs: counts the workload's statement fixes
# (16 sequences on one 2000-token prompt, refcount 16; at 16-token blocks 2000 = 125 x 16,
# so the shared prompt is 125 full blocks).  Reading: the parent also holds its first
# generated token (position 2000, alone in block 125), so that block is the partly filled
# shared one whose copy-on-write the step needs; children write before the parent.
# ---------------------------------------------------------------------------

def _fork_setup(seed=5, extra=40):
    cfg = workloads.CONFIGS["fork_cow"]
    rng = np.random.default_rng(seed)
    gen = rng.integers(80, 512, size=cfg.num_seqs, endpoint=True)
    need = 126 + sum(-(-int(2001 + g) // 16) - 125 for g in gen) + extra
    return cfg, gen, need, [int(x) for x in rng.permutation(need)]


def test_oracle_fork_step_counts():
    cfg, _, N, order = _fork_setup()
    B, S = cfg.block_size, cfg.num_seqs
    o = obatch.fork_step(2000, S - 1, N, B, order)
    tb, pairs, ctx, slots = o["block_tables"], o["copy_pairs"], o["context_lens"], o["slot_mapping"]
    assert (ctx == 2002).all() and tb.shape == (S, 126)
    assert pairs.shape == (S - 1, 2)                                  # one copy per child
    parent_last = int(tb[0, 125])
    assert (pairs[:, 0] == parent_last).all()                         # all from the shared last block
    assert len(set(pairs[:, 1].tolist())) == S - 1 and parent_last not in pairs[:, 1]
    assert sorted(tb[1:, 125].tolist()) == sorted(pairs[:, 1].tolist())
    assert (tb[:, :125] == tb[0, :125]).all()                         # 125 prompt blocks shared
    assert slots.tolist() == [int(tb[s, 125]) * B + 1 for s in range(S)]   # position 2001
    h = o["holders"]
    assert (h[tb[0, :125]] == S).all() and int((h == S).sum()) == 125
    assert h[parent_last] == 1 and (h[pairs[:, 1]] == 1).all()
    assert int(h.sum()) == 125 * S + S


def test_oracle_steady_fork_step_counts():
    cfg, gen, N, order = _fork_setup()
    B, S = cfg.block_size, cfg.num_seqs
    o = obatch.steady_fork_step(2000, gen, N, B, order)
    tb, pairs, ctx, slots = o["block_tables"], o["copy_pairs"], o["context_lens"], o["slot_mapping"]
    assert ctx.tolist() == [2001 + int(g) for g in gen]
    assert pairs.shape == (0, 2)                                      # no copy left in the step
    assert (tb[:, :125] == tb[0, :125]).all()
    h = o["holders"]
    assert int((h == S).sum()) == 125 and (h[tb[0, :125]] == S).all()
    private = [int(b) for s in range(S) for b in tb[s, 125:-(-int(ctx[s]) // B)]]
    assert len(private) == len(set(private)) and all(h[b] == 1 for b in private)
    assert len(private) == sum(-(-int(c) // B) - 125 for c in ctx)
    assert slots.tolist() == [int(tb[s, (int(ctx[s]) - 1) // B]) * B + (int(ctx[s]) - 1) % B for s in range(S)]


# ---------------------------------------------------------------------------
# KV write and block copy: bytes land where the pages' examples say
# ---------------------------------------------------------------------------

def _special_rows(n_rows, row_elems, seed):
    """fp32 bit patterns including NaN payloads, -0, +-inf and subnormals."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=(n_rows, row_elems), dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF],
                        dtype=np.uint32)
    flat = bits.reshape(-1)
    flat[rng.integers(0, flat.size, size=min(flat.size, 64))] = np.resize(specials, min(flat.size, 64))
    return bits.view(np.float32)


@pytest.mark.parametrize("case", golden("physical_index.json")["cases"], ids=["slot3073", "slot3116"])
def test_kv_write_lands_at_page_slot(case):
    B, Hkv, D = case["block_size"], 1, 4
    N = max(case["table"]) + 1
    kc = _special_rows(N * B, Hkv * D, 1).reshape(N, B, Hkv, D).copy()
    vc = _special_rows(N * B, Hkv * D, 2).reshape(N, B, Hkv, D).copy()
    kn = _special_rows(1, Hkv * D, 3).reshape(1, Hkv, D)
    vn = _special_rows(1, Hkv * D, 4).reshape(1, Hkv, D)
    k0, v0 = kc.copy(), vc.copy()
    oracle.kv_write(kn, vn, kc, vc, [case["slot"]])
    pb, off = case["physical_block"], case["offset"]
    assert kc[pb, off].tobytes() == kn[0].tobytes() and vc[pb, off].tobytes() == vn[0].tobytes()
    k0[pb, off] = kn[0]
    v0[pb, off] = vn[0]
    assert kc.tobytes() == k0.tobytes() and vc.tobytes() == v0.tobytes()


def test_kv_write_then_gather_reads_back_bf16():
    # write each sequence's newest token through its slot, then the gathered view
    # (the attention side's reading of the table) returns exactly those bytes at ctx-1
    q, kc, vc, bt, ctx, m, seqs = _small(3, 5, 4, 2, 16, 4, 30, dtype="bf16")
    S, Hkv, D = len(ctx), kc.shape[2], kc.shape[3]
    kn = workloads.normal(S * Hkv * D, 99, 1, "bf16").reshape(S, Hkv, D)
    vn = workloads.normal(S * Hkv * D, 99, 2, "bf16").reshape(S, Hkv, D)
    slots = oracle.slot_mapping(bt, ctx - 1, kc.shape[1])
    k0 = kc.copy()
    oracle.kv_write(kn, vn, kc, vc, slots)
    for s in range(S):
        K = oracle.gather_sequence(kc, bt[s], int(ctx[s]))
        V = oracle.gather_sequence(vc, bt[s], int(ctx[s]))
        assert K[-1].tobytes() == kn[s].tobytes() and V[-1].tobytes() == vn[s].tobytes()
        assert K[:-1].tobytes() == oracle.gather_sequence(k0, bt[s], int(ctx[s]))[:-1].tobytes()
    changed = np.nonzero((kc != k0).any(axis=(2, 3)))
    assert set(zip(*[c.tolist() for c in changed])) <= {(int(s) // 4, int(s) % 4) for s in slots}


def test_kv_write_rejects_bad_slots():
    kc = np.zeros((4, 4, 1, 4), np.float32)
    vc = kc.copy()
    kn = np.ones((2, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(kn, kn, kc, vc, [3, 3])
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(kn, kn, kc, vc, [0, 16])
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(kn, kn, kc, vc, [-1, 2])
    oracle.kv_write(kn[:0], kn[:0], kc, vc, [])      # empty write is a no-op
    assert not kc.any()


def test_copy_on_write_keeps_parent_bytes():
    # fork a parent with a partly filled last block; every child's first write copies the
    # block first (nano-vLLM Ch04 section 6), so the parent's bytes never change
    B, Hkv, D = 4, 2, 8
    rng = np.random.default_rng(5)
    N = 40
    m = BlockModel(N, B, free_order=[int(x) for x in rng.permutation(N)])
    parent = m.new_sequence(10)                          # 3 blocks, last holds 2 of 4 slots
    kids = [{"table": m.fork(parent["table"]), "len": 10} for _ in range(3)]
    kc = _special_rows(N * B, Hkv * D, 6).reshape(N, B, Hkv, D).copy()
    vc = _special_rows(N * B, Hkv * D, 7).reshape(N, B, Hkv, D).copy()
    parent_k = [kc[b].tobytes() for b in parent["table"]]
    parent_v = [vc[b].tobytes() for b in parent["table"]]
    pairs, slots = [], []
    for kid in kids:
        assert m.append_token(kid)
        slot, pair = m.write_slot(kid, 10)
        assert pair is not None and pair[0] == parent["table"][2]
        pairs.append(pair)
        slots.append(slot)
    assert m.append_token(parent)
    slot, pair = m.write_slot(parent, 10)
    assert pair is None                                  # last holder writes in place
    slots.append(slot)
    m.check([parent] + kids)
    k_before = kc.copy()
    oracle.copy_blocks(kc, vc, pairs)
    for src, dst in pairs:
        assert kc[dst].tobytes() == kc[src].tobytes() and vc[dst].tobytes() == vc[src].tobytes()
    untouched = [b for b in range(N) if b not in {d for _, d in pairs}]
    assert kc[untouched].tobytes() == k_before[untouched].tobytes()
    kn = _special_rows(4, Hkv * D, 8).reshape(4, Hkv, D)
    oracle.kv_write(kn, kn, kc, vc, slots[:3])           # children write their own copies
    assert [kc[b].tobytes() for b in parent["table"]] == parent_k
    assert [vc[b].tobytes() for b in parent["table"]] == parent_v
    for i, kid in enumerate(kids):
        seqk = oracle.gather_sequence(kc, kid["table"], 11)
        assert seqk[10].tobytes() == kn[i].tobytes()
        assert seqk[:10].tobytes() == oracle.gather_sequence(kc, parent["table"], 10).tobytes()


def test_copy_blocks_rejects_overlap():
    kc = np.zeros((4, 2, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(kc, kc.copy(), [(0, 1), (2, 1)])      # repeated destination
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(kc, kc.copy(), [(0, 1), (1, 2)])      # destination is also a source
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(kc, kc.copy(), [(0, 4)])
    oracle.copy_blocks(kc, kc.copy(), np.zeros((0, 2), np.int64))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # seed, S, Hq, Hkv, D, B, ctx_hi, dtype
    (1, 3, 4, 4, 16, 4, 40, "f32"),
    (2, 4, 8, 2, 32, 8, 70, "bf16"),
    (3, 2, 6, 3, 8, 16, 50, "f32"),
    (4, 3, 16, 2, 64, 16, 100, "bf16"),
]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_equals_library_sdpa_and_dense(case):
    seed, S, Hq, Hkv, D, B, hi, dt = case
    q, kc, vc, bt, ctx, m, _ = _small(seed, S, Hq, Hkv, D, B, hi, dt)
    scale = 1 / math.sqrt(D)
    o1 = oracle.attention(q, kc, vc, bt, ctx, scale)
    o2 = oracle.dense_attention(q, kc, vc, bt, ctx, scale)
    o3 = _sdpa(q, kc, vc, bt, ctx, scale, m)
    assert np.max(np.abs(o1 - o3)) < 1e-12
    assert np.max(np.abs(o1 - o2)) < 1e-12


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_block_permutation_invariance(case):
    seed, S, Hq, Hkv, D, B, hi, dt = case
    q, kc, vc, bt, ctx, m, _ = _small(seed, S, Hq, Hkv, D, B, hi, dt)
    N = kc.shape[0]
    pi = np.random.default_rng(seed + 100).permutation(N)       # new id of old block b is pi[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    bt2 = pi[bt].astype(np.int32)
    o = oracle.attention(q, kc, vc, bt, ctx, 0.3)
    o2 = oracle.attention(q, kc2, vc2, bt2, ctx, 0.3)
    assert o.tobytes() == o2.tobytes()


def test_attention_single_token_returns_v():
    q, kc, vc, bt, ctx, m, _ = _small(5, 4, 8, 4, 32, 4, 1, "bf16", ctx=[1, 1, 1, 1])
    o = oracle.attention(q, kc, vc, bt, ctx, 0.2)
    for s in range(4):
        v0 = oracle.widen(vc[bt[s, 0], 0])                     # [Hkv, D]
        assert np.array_equal(o[s], np.repeat(v0, 2, axis=0))


def test_attention_uniform_weights_give_mean():
    q, kc, vc, bt, ctx, m, _ = _small(6, 3, 4, 2, 16, 4, 30, "f32")
    for qq, sc in ((np.zeros_like(q), 0.5), (q, 0.0)):
        o = oracle.attention(qq, kc, vc, bt, ctx, sc)
        for s in range(3):
            V = oracle.widen(oracle.gather_sequence(vc, bt[s], int(ctx[s])))
            mean = V.mean(axis=0)                                  # [Hkv, D]
            assert np.max(np.abs(o[s] - np.repeat(mean, 2, axis=0))) < 1e-12


def test_attention_mpmath_brute_force():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    q, kc, vc, bt, ctx, m, _ = _small(8, 2, 4, 2, 8, 4, 20, "f32")
    scale = 0.37
    o = oracle.attention(q, kc, vc, bt, ctx, scale)
    B = kc.shape[1]
    for s in range(2):
        for h in range(4):
            kvh = h // 2
            xs, vs = [], []
            for t in range(int(ctx[s])):
                b, off = int(bt[s, t // B]), t % B
                xs.append(mp.mpf(scale) * mp.fsum(mp.mpf(float(q[s, h, d])) * mp.mpf(float(kc[b, off, kvh, d]))
                                                  for d in range(8)))
                vs.append([mp.mpf(float(vc[b, off, kvh, d])) for d in range(8)])
            ws = [mp.e ** x for x in xs]
            Z = mp.fsum(ws)
            for d in range(8):
                ref = mp.fsum(w * v[d] for w, v in zip(ws, vs)) / Z
                assert abs(float(ref) - o[s, h, d]) < 1e-12


@pytest.mark.parametrize("P", [4, 8, 12, 64, 1024])
def test_split_k_equals_unsplit(P):
    q, kc, vc, bt, ctx, m, _ = _small(9, 4, 8, 2, 16, 4, 90, "bf16")
    o = oracle.attention(q, kc, vc, bt, ctx, 0.25)
    op = oracle.attention(q, kc, vc, bt, ctx, 0.25, partition_size=P)
    assert np.max(np.abs(o - op)) < 1e-12
    if P >= int(ctx.max()):
        assert o.tobytes() == op.tobytes()           # a single partition is the plain path


def test_split_k_reduce_closed_form():
    # two partitions by hand: out = (L0 e^(m0-M) o0 + L1 e^(m1-M) o1) / (L0 e^(m0-M) + L1 e^(m1-M))
    q, kc, vc, bt, ctx, m, _ = _small(10, 1, 1, 1, 4, 4, 8, "f32", ctx=[8])
    K = oracle.widen(oracle.gather_sequence(kc, bt[0], 8))[:, 0]
    V = oracle.widen(oracle.gather_sequence(vc, bt[0], 8))[:, 0]
    x = 0.5 * K @ oracle.widen(q[0, 0])
    parts = []
    for lo, hi in ((0, 4), (4, 8)):
        mp_ = x[lo:hi].max()
        w = np.exp(x[lo:hi] - mp_)
        parts.append((mp_, w.sum(), (w @ V[lo:hi]) / w.sum()))
    M = max(p[0] for p in parts)
    num = sum(L * math.exp(mm - M) * o for mm, L, o in parts)
    den = sum(L * math.exp(mm - M) for mm, L, o in parts)
    ref = num / den
    got = oracle.attention(q, kc, vc, bt, ctx, 0.5, partition_size=4)[0, 0]
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_ignores_tail_slots_and_table_padding():
    q, kc, vc, bt, ctx, m, _ = _small(11, 4, 4, 4, 16, 8, 60, "bf16", extra_blocks=1)
    o = oracle.attention(q, kc, vc, bt, ctx, 0.25)
    B = kc.shape[1]
    kp, vp = kc.copy(), vc.copy()
    poison = m.free[0]                                # a block no sequence holds
    bt2 = bt.copy()
    for s in range(4):
        c = int(ctx[s])
        nb = -(-c // B)
        bt2[s, nb:] = poison                          # padding entries point at a poisoned block
        last = bt[s, nb - 1]
        kp[last, c - (nb - 1) * B:] = 0x7FC1          # NaN bf16 in the slots past ctx
        vp[last, c - (nb - 1) * B:] = 0xFFC3
    kp[poison] = 0x7FC1
    vp[poison] = 0x7FC1
    o2 = oracle.attention(q, kp, vp, bt2, ctx, 0.25)
    assert np.isfinite(o2).all() and o.tobytes() == o2.tobytes()


def test_attention_items_subset_matches_full():
    q, kc, vc, bt, ctx, m, _ = _small(12, 3, 4, 2, 16, 4, 40, "f32")
    full = oracle.attention(q, kc, vc, bt, ctx, 0.25)
    items = [0, 5, 11, 7]
    sub = oracle.attention(q, kc, vc, bt, ctx, 0.25, items=items)
    for i, it in enumerate(items):
        assert sub[i].tobytes() == full[it // 4, it % 4].tobytes()


def test_attention_rejects_bad_inputs():
    q, kc, vc, bt, ctx, m, _ = _small(13, 2, 4, 2, 16, 4, 20, "f32")
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, kc, vc, bt, np.array([0, 3], np.int32), 0.25)          # ctx = 0
    bad = bt.copy()
    bad[0, 0] = kc.shape[0]
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, kc, vc, bad, ctx, 0.25)                                # block id out of range
    with pytest.raises(oracle.OracleError):
        oracle.attention(np.ascontiguousarray(q[:, :3]), kc, vc, bt, ctx, 0.25)                          # 3 % 2 != 0
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, kc, vc, bt, ctx, 0.25, partition_size=6)               # not a multiple of B


# ---------------------------------------------------------------------------
# head-major cache layout (PidokuInfra page, section 5 "The layout, more precisely")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,B", [("bf16", 16), ("bf16", 8), ("f32", 4), ("f32", 32)])
def test_head_major_layout_byte_properties(dt, B):
    # the page prints key_cache [N, Hkv, D/x, B, x] with x = 16 / sizeof(dtype), so 16 bytes
    # of K are x consecutive head dims of one token, and value_cache [N, Hkv, D, B], so the
    # B tokens of one head dim of V are consecutive; checked on the raw bytes
    N, Hkv, D = 5, 3, 32
    e = 2 if dt == "bf16" else 4
    x = 16 // e
    k = workloads.normal(N * B * Hkv * D, 7, 1, dt).reshape(N, B, Hkv, D)
    v = workloads.normal(N * B * Hkv * D, 7, 2, dt).reshape(N, B, Hkv, D)
    khm, vhm = oracle.head_major_from_rows(k, v)
    assert oracle.head_major_x(k.dtype) == x
    assert khm.shape == (N, Hkv, D // x, B, x) and vhm.shape == (N, Hkv, D, B)
    kb, vb = khm.tobytes(), vhm.tobytes()
    rng = np.random.default_rng(B)
    for _ in range(200):
        b, o, h, d = (int(rng.integers(n)) for n in (N, B, Hkv, D))
        j = d // x
        off = (((b * Hkv + h) * (D // x) + j) * B + o) * 16
        assert kb[off:off + 16] == k[b, o, h, j * x:(j + 1) * x].tobytes()
        off = ((b * Hkv + h) * D + d) * B * e
        assert vb[off:off + B * e] == np.ascontiguousarray(v[b, :, h, d]).tobytes()
    k2, v2 = oracle.rows_from_head_major(khm, vhm)
    assert k2.tobytes() == k.tobytes() and v2.tobytes() == v.tobytes()


def test_kv_write_head_major_matches_row_write():
    N, B, Hkv, D, T = 9, 16, 2, 64, 5
    k = _special_rows(N * B, Hkv * D, 11).reshape(N, B, Hkv, D).copy()
    v = _special_rows(N * B, Hkv * D, 12).reshape(N, B, Hkv, D).copy()
    kn = _special_rows(T, Hkv * D, 13).reshape(T, Hkv, D)
    vn = _special_rows(T, Hkv * D, 14).reshape(T, Hkv, D)
    slots = [0, 17, 143, 70, 31]
    khm, vhm = oracle.head_major_from_rows(k, v)
    oracle.kv_write(kn, vn, k, v, slots)
    oracle.kv_write_head_major(kn, vn, khm, vhm, slots)
    k2, v2 = oracle.head_major_from_rows(k, v)
    assert khm.tobytes() == k2.tobytes() and vhm.tobytes() == v2.tobytes()
    with pytest.raises(oracle.OracleError):
        oracle.kv_write_head_major(kn[:2], vn[:2], khm, vhm, [3, 3])
    with pytest.raises(oracle.OracleError):
        oracle.kv_write_head_major(kn[:1], vn[:1], khm, vhm, [N * B])


def test_attention_head_major_is_row_attention():
    q, kc, vc, bt, ctx, m, _ = _small(5, 3, 8, 2, 32, 8, 60, "bf16")
    khm, vhm = oracle.head_major_from_rows(kc, vc)
    o = oracle.attention(q, kc, vc, bt, ctx, 0.25, 16)
    o2 = oracle.attention_head_major(q, khm, vhm, bt, ctx, 0.25, 16)
    assert o.tobytes() == o2.tobytes()
