"""libpkv.so loads, exports every function include/pkv.h declares, and its host-side
argument checks return status codes before anything reaches the GPU.  No kernel is
launched here: every call below is rejected (or is a declared no-op) on the host."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_148_amd import binding
from paged_kv_cache_148_amd.binding import (PKV_DTYPE_BF16, PKV_DTYPE_F32, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED,
                                            PKV_OK, PKV_PATH_MFMA, PKV_PATH_NONE, PKV_PATH_TILE_VALU,
                                            PKV_PATH_VECTOR)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from paged_kv_cache_148_amd.build import build
        build()
    return binding.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "pkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "defined"})


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert binding.status_string(PKV_OK) == "ok"
    for s in (1, 2, 3, 4):
        assert binding.status_string(s) not in ("ok", "unknown status")
    assert binding.status_string(99) == "unknown status"


def test_workspace_size(L):
    # 256-byte work-queue header + S * Hq * ceil(max_ctx / P) * (D + 32) fp32 when split:
    # D partial outputs per (sequence, head, partition) and one 128-byte (m, l) line per item
    assert binding.attention_workspace_size(8, 32, 128, 131072, 512) == 256 + 8 * 32 * 256 * 160 * 4
    assert binding.attention_workspace_size(8, 32, 128, 100, 512) == 256    # one partition
    assert binding.attention_workspace_size(8, 32, 128, 1000, 0) == 256     # no split
    assert binding.attention_workspace_size(2, 4, 64, 513, 512) == 256 + 2 * 4 * 2 * 96 * 4


def test_path_selection_head_major(L):
    assert binding.attention_path_head_major(64, 8, 128, 16, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path_head_major(32, 32, 128, 128, PKV_DTYPE_BF16) == PKV_PATH_TILE_VALU   # g = 1
    assert binding.attention_path_head_major(32, 8, 128, 8, PKV_DTYPE_BF16) == PKV_PATH_NONE    # below a tile
    assert binding.attention_path_head_major(8, 8, 128, 16, PKV_DTYPE_F32) == PKV_PATH_NONE     # bf16 only
    assert binding.attention_path_head_major(8, 8, 64, 16, PKV_DTYPE_BF16) == PKV_PATH_NONE
    assert binding.attention_path_head_major(64, 2, 128, 16, PKV_DTYPE_BF16) == PKV_PATH_NONE   # g = 32


def test_path_selection(L):
    assert binding.attention_path(64, 8, 128, 16, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path(32, 8, 128, 32, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path(32, 32, 128, 16, PKV_DTYPE_BF16) == PKV_PATH_TILE_VALU   # g = 1: no MFMA
    assert binding.attention_path(16, 1, 128, 32, PKV_DTYPE_BF16) == PKV_PATH_MFMA      # g = 16
    assert binding.attention_path(32, 32, 128, 16, PKV_DTYPE_F32) == PKV_PATH_VECTOR
    assert binding.attention_path(4, 4, 64, 4, PKV_DTYPE_F32) == PKV_PATH_VECTOR
    assert binding.attention_path(32, 8, 128, 8, PKV_DTYPE_BF16) == PKV_PATH_MFMA    # blocks below a tile
    assert binding.attention_path(32, 8, 128, 4, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path(32, 8, 64, 8, PKV_DTYPE_BF16) == PKV_PATH_VECTOR   # head_dim 64
    assert binding.attention_path(64, 4, 64, 8, PKV_DTYPE_BF16) == PKV_PATH_NONE    # g = 16 off the MFMA path
    assert binding.attention_path(64, 2, 128, 8, PKV_DTYPE_BF16) == PKV_PATH_NONE   # g = 32
    assert binding.attention_path(6, 4, 128, 16, PKV_DTYPE_BF16) == PKV_PATH_NONE   # 6 % 4 != 0
    assert binding.attention_path(8, 8, 96, 16, PKV_DTYPE_BF16) == PKV_PATH_NONE    # head_dim
    assert binding.attention_path(8, 8, 128, 64, PKV_DTYPE_BF16) == PKV_PATH_TILE_VALU   # large blocks: tile kernel
    assert binding.attention_path(16, 8, 128, 64, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path(64, 8, 128, 128, PKV_DTYPE_BF16) == PKV_PATH_MFMA
    assert binding.attention_path(8, 8, 128, 64, PKV_DTYPE_F32) == PKV_PATH_NONE    # no vector path past 32
    assert binding.attention_path(8, 8, 64, 128, PKV_DTYPE_BF16) == PKV_PATH_NONE
    assert binding.attention_path(8, 8, 128, 256, PKV_DTYPE_BF16) == PKV_PATH_NONE  # block size
    assert binding.attention_path(8, 8, 128, 16, 7) == PKV_PATH_NONE                # dtype


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: every call is refused on the host
ODD = ctypes.c_void_p((1 << 20) + 4)


def test_kv_write_host_checks(L):
    w = L.paged_kv_write
    assert w(NULL, NULL, NULL, NULL, NULL, 0, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_OK   # empty no-op
    assert w(NULL, FAKE, FAKE, FAKE, FAKE, 4, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert w(ODD, FAKE, FAKE, FAKE, FAKE, 4, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 16, 8, 96, PKV_DTYPE_BF16, NULL) == PKV_ERR_UNSUPPORTED
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 12, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_UNSUPPORTED
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 16, 8, 128, 5, NULL) == PKV_ERR_UNSUPPORTED
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG


def test_copy_blocks_host_checks(L):
    c = L.copy_blocks
    assert c(NULL, NULL, NULL, 0, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_OK
    assert c(FAKE, FAKE, NULL, 3, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert c(FAKE, ODD, FAKE, 3, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, -2, 10, 16, 8, 128, PKV_DTYPE_BF16, NULL) == PKV_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, 3, 10, 16, 8, 80, PKV_DTYPE_F32, NULL) == PKV_ERR_UNSUPPORTED


def _attn(L, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxblk=8, ctx=FAKE, maxctx=128, S=4, Hq=8, Hkv=2, D=128,
             B=16, N=100, scale=0.1, P=0, ws=NULL, wsb=0, dt=PKV_DTYPE_BF16)
    a.update(kw)
    return L.paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["maxblk"], a["ctx"], a["maxctx"],
                                    a["S"], a["Hq"], a["Hkv"], a["D"], a["B"], a["N"], a["scale"], a["P"], a["ws"],
                                    a["wsb"], a["dt"], NULL)


def test_attention_host_checks(L):
    assert _attn(L, S=0) == PKV_OK                                   # empty batch
    assert _attn(L, out=NULL) == PKV_ERR_INVALID_ARG
    assert _attn(L, q=ODD) == PKV_ERR_INVALID_ARG
    assert _attn(L, Hq=6, Hkv=4) == PKV_ERR_INVALID_ARG
    assert _attn(L, D=96) == PKV_ERR_UNSUPPORTED
    assert _attn(L, B=12) == PKV_ERR_UNSUPPORTED
    assert _attn(L, dt=9) == PKV_ERR_UNSUPPORTED
    assert _attn(L, maxctx=129) == PKV_ERR_INVALID_ARG              # exceeds max_blocks * B
    assert _attn(L, maxctx=0) == PKV_ERR_INVALID_ARG
    assert _attn(L, P=24) == PKV_ERR_INVALID_ARG                     # not a multiple of B
    assert _attn(L, P=32) == PKV_ERR_INVALID_ARG                     # needs a workspace
    assert _attn(L, P=0) == PKV_ERR_INVALID_ARG                      # the queue header is always needed
    assert _attn(L, P=0, ws=FAKE, wsb=255) == PKV_ERR_INVALID_ARG
    assert _attn(L, P=0, ws=ODD, wsb=256) == PKV_ERR_INVALID_ARG
    need = binding.attention_workspace_size(4, 8, 128, 128, 32)
    assert _attn(L, P=32, ws=FAKE, wsb=need - 4) == PKV_ERR_INVALID_ARG
    assert _attn(L, scale=float("nan")) == PKV_ERR_INVALID_ARG
    assert _attn(L, N=0) == PKV_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors(L):
    torch = pytest.importorskip("torch")
    from paged_kv_cache_148_amd import paged_kv_write
    k = torch.zeros(4, 16, 2, 64)
    with pytest.raises(ValueError):
        paged_kv_write(torch.zeros(1, 2, 64), torch.zeros(1, 2, 64), k, k.clone(), torch.zeros(1, dtype=torch.int64))


def test_stream_read_probe_rejects_bad_arguments(L):
    sink = ctypes.c_void_p(256)   # never dereferenced: every call below fails its host checks
    buf = ctypes.c_void_p(4096)
    assert L.pkv_stream_read_probe(None, 1 << 20, sink, None) == PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read_probe(buf, 1 << 20, None, None) == PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read_probe(buf, 8, sink, None) == PKV_ERR_INVALID_ARG             # under one word
    assert L.pkv_stream_read_probe(ctypes.c_void_p(4100), 1 << 20, sink, None) == PKV_ERR_INVALID_ARG
    assert L.pkv_stream_read_probe(buf, 1 << 20, ctypes.c_void_p(258), None) == PKV_ERR_INVALID_ARG


def test_noalloc_rejects_beyond_its_static_scratch_on_the_host(L):
    # the limit is checked before anything is looked up or enqueued (no GPU needed): 64 sequences
    # x 64 heads x 256 partitions of partial states are far beyond the 64 MiB array
    assert L.pkv_static_scratch_bytes() == 64 << 20
    assert binding.attention_workspace_size(64, 64, 128, 131072, 512) > L.pkv_static_scratch_bytes()
    st = L.paged_attention_decode_noalloc(None, None, None, None, None, 8192, None, 131072, 64, 64, 8, 128, 16, 4,
                                          0.1, 512, PKV_DTYPE_BF16, None)
    assert st == binding.PKV_ERR_SCRATCH_LIMIT
    assert "scratch" in binding.status_string(st)
    st = L.paged_attention_decode_noalloc(None, None, None, None, None, 8192, None, 0, 64, 64, 8, 128, 16, 4,
                                          0.1, 512, PKV_DTYPE_BF16, None)
    assert st == PKV_ERR_INVALID_ARG                                     # max_context_len 0


def test_noalloc_checks_its_arguments_before_touching_the_device(L):
    # a rejected call enqueues nothing and looks nothing up: with no GPU here, a call whose only
    # fault is a null pointer (or a bad shape) must come back INVALID_ARG / UNSUPPORTED, not a HIP
    # error from the scratch lookup; an empty batch is a no-op
    dummy = 256   # aligned, never dereferenced: the call is rejected first
    args = lambda q, S=4, B=16, Hq=8, Hkv=2: (dummy, q, dummy, dummy, dummy, 64, dummy, 1000, S, Hq, Hkv, 128, B, 100,
                                              0.1, 0, PKV_DTYPE_BF16, None)
    assert L.paged_attention_decode_noalloc(*args(None)) == PKV_ERR_INVALID_ARG
    assert L.paged_attention_decode_noalloc(*args(dummy, Hq=9, Hkv=2)) == PKV_ERR_INVALID_ARG
    assert L.paged_attention_decode_noalloc(*args(dummy, B=24)) == PKV_ERR_UNSUPPORTED
    assert L.paged_attention_decode_noalloc(*args(dummy, S=0)) == PKV_OK
