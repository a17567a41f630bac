"""paged_attention_decode_noalloc -- the entry point that allocates nothing -- against
paged_attention_decode with its own workspace: two calls in a row on the library's static
scratch, the second with a smaller input, each bit-identical to the existing entry point (the
same kernels) and within tolerance of the CPU oracle.  Collected last, so that it also runs after
every other GPU test of the process."""
import numpy as np
import pytest

from paged_kv_cache_148_amd import batch as pbatch
from paged_kv_cache_148_amd import binding
from tests import gpu_helpers as H
import workloads

pytestmark = pytest.mark.gpu


def _case(name, P, num_seqs=None):
    wl = workloads.make_workload(name, num_seqs=num_seqs)
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    H.gpu_step(wl, step, d, P, do_attn=False)        # the step's write, as the oracle's step does
    return wl, step, d


def _both(wl, step, d, P):
    import torch
    cfg = wl.cfg
    need = binding.attention_workspace_size(cfg.num_seqs, cfg.num_heads, cfg.head_dim, step.max_context_len, P)
    assert need <= binding.static_scratch_bytes()
    a = torch.full_like(d["out"], float("nan"))
    b = torch.full_like(d["out"], float("nan"))
    binding.paged_attention_decode(a, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                   step.max_context_len, wl.scale, P)
    binding.paged_attention_decode_noalloc(b, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                           d["context_lens"], step.max_context_len, wl.scale, P)
    torch.cuda.synchronize()
    return H.bits(a), H.bits(b)


@pytest.mark.parametrize("first,second", [
    (("long_splitk", 512, None), ("gqa70b", 512, 12)),     # most scratch (40 MiB of partials), then less
    (("mha7b", 0, 24), ("mha7b", 0, 5)),                    # unsplit: the work-queue header only
], ids=["split", "unsplit"])
def test_noalloc_matches_workspace_call_twice(first, second):
    for name, P, S in (first, second):
        print("[gpu case] noalloc", name, "P", P, "S", S, flush=True)
        wl, step, d = _case(name, P, S)
        want, got = _both(wl, step, d, P)
        assert got.tobytes() == want.tobytes(), f"{name}: noalloc output differs from paged_attention_decode"
        items = None
        if name == "long_splitk":
            # the longest and the shortest sequences, every head
            Hq = wl.cfg.num_heads
            ss = [int(np.argmax(step.context_lens)), int(np.argmin(step.context_lens))]
            items = np.array([s * Hq + h for s in ss for h in range(Hq)])
        _, _, _, ref = H.oracle_step(wl, "steady", P, items=items)
        g = got if items is None else got.reshape(-1, got.shape[-1])[items]
        H.check_close(g, ref, wl.cfg.dtype, f"noalloc {name} S={wl.cfg.num_seqs} P={P}")
        del d


def test_noalloc_rejects_a_call_beyond_the_scratch():
    import torch
    # 64 sequences x 64 heads x 256 partitions of partials: far beyond the static scratch
    S, Hq, Hkv, D, B = 64, 64, 8, 128, 16
    need = binding.attention_workspace_size(S, Hq, D, 131072, 512)
    assert need > binding.static_scratch_bytes()
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4, B, Hkv, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(S, 131072 // B, dtype=torch.int32, device="cuda")
    ctx = torch.ones(S, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.PkvError) as e:
        binding.paged_attention_decode_noalloc(torch.empty_like(q), q, kc, kc, bt, ctx, 131072, 0.1, 512)
    assert e.value.status == binding.PKV_ERR_SCRATCH_LIMIT


def test_noalloc_captured_in_a_hip_graph():
    # the use the entry point exists for: captured once in a HIP graph (it allocates nothing) and
    # replayed, with eager calls on the same static scratch between the replays; every replay and
    # every eager call gives paged_attention_decode's output bit for bit
    import torch
    name, P = "gqa70b", 512
    wl, step, d = _case(name, P, 16)
    want, _ = _both(wl, step, d, P)
    out = torch.full_like(d["out"], float("nan"))
    other = torch.empty_like(d["out"])
    graph = torch.cuda.CUDAGraph()
    print("[gpu case] noalloc graph capture", name, "P", P, flush=True)
    with torch.cuda.graph(graph):
        binding.paged_attention_decode_noalloc(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                               d["context_lens"], step.max_context_len, wl.scale, P)
    for rep in range(3):
        print("[gpu case] noalloc graph replay", rep, flush=True)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert H.bits(out).tobytes() == want.tobytes(), f"replay {rep}"
        binding.paged_attention_decode_noalloc(other, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                               d["context_lens"], step.max_context_len, wl.scale, P)
        torch.cuda.synchronize()
        assert H.bits(other).tobytes() == want.tobytes(), f"eager after replay {rep}"
    del graph
