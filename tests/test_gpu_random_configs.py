"""GPU parity on seeded random configurations of the supported space (tests/random_cases.py).

Each case draws the element type, head dim, block size, query heads per KV head, KV heads,
batch, context lengths (with the edge values 1, B, B + 1, P, P + 1 and the maximum mixed in),
partition size, the work-item width (on the tile paths) and whether the step goes through
paged_attention_decode_write.  The whole output is compared with the fp64 oracle within the
stated tolerance, and both pools with the oracle's bit for bit; the oracle builds its own
tables, slots and copy pairs with its own block model.
"""
import pytest

from paged_kv_cache_148_amd import batch as pbatch
from paged_kv_cache_148_amd import binding
from tests import gpu_helpers as H
from tests import random_cases as R
import workloads

pytestmark = pytest.mark.gpu

PATH = {"vector": binding.PKV_PATH_VECTOR, "mfma": binding.PKV_PATH_MFMA, "valu": binding.PKV_PATH_TILE_VALU}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield


@pytest.mark.parametrize("case", range(R.N_CASES), ids=[R.case_id(i) for i in range(R.N_CASES)])
def test_random_configuration_matches_oracle(monkeypatch, case):
    import torch
    c = R.draw(case)
    print("[gpu case] random", R.case_id(case), "ctx", c["ctx"].tolist(), flush=True)
    assert binding.attention_path(c["Hq"], c["Hkv"], c["D"], c["B"], 1 if c["dt"] == "bf16" else 0) == PATH[c["path"]]
    if c["width"]:
        monkeypatch.setenv("PKV_WIDE_ITEMS", c["width"])
    else:
        monkeypatch.delenv("PKV_WIDE_ITEMS", raising=False)
    cfg = workloads.Config("random", c["dt"], c["S"], c["Hq"], c["Hkv"], c["D"], c["B"], ("uniform", 1, 2),
                           seed=30_000 + case)
    wl = workloads.make_workload(cfg, ctx_override=c["ctx"])
    step = pbatch.step_for(wl)
    d = H.upload(wl, step)
    P = c["P"]
    if c["fused"]:
        binding.paged_attention_decode_write(d["out"], d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                             d["block_tables"], d["context_lens"], step.max_context_len, wl.scale, P)
        torch.cuda.synchronize()
    else:
        H.gpu_step(wl, step, d, P)
    _, kc, vc, ref = H.oracle_step(wl, "steady", P)
    assert H.bits(d["k_cache"]).tobytes() == kc.tobytes()
    assert H.bits(d["v_cache"]).tobytes() == vc.tobytes()
    H.check_close(H.bits(d["out"]), ref, c["dt"], f"random {R.case_id(case)}")
