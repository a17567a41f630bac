"""CPU oracle for the paged KV cache decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may
import this package.  The GPU library never calls it; the two share no code.

Pieces:
  * ``liboracle.so`` (``pkv_oracle.c``): scalar fp64 C implementation of the KV
    write, the block copy, the slot formula and paged attention (plain and
    split-K), OpenMP over (sequence, head).  Wrapped here for numpy arrays.
  * ``dense_attention``: a numpy textbook reference -- gather each sequence's K/V
    rows through its block table into contiguous arrays, then ordinary softmax
    attention.  Paged attention computes exactly this; only the memory layout
    differs (page "nano-vLLM . Ch04 . PagedAttention", section 9, Myth 1; page
    "PagedAttention" (tokentrails), step 3 and its Code box).
  * ``oracle.blocks``: the block-manager model (free stack, refcounts, fork,
    copy-on-write) used to derive block tables, slots and copy pairs independently
    of the product's own block manager.

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
_ERRORS = {-1: "invalid argument", -2: "out of range", -3: "duplicate slot/destination", -4: "out of memory"}


class OracleError(ValueError):
    pass


def lib():
    """Load liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle.build import build
            build()
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str):
    """ctypes handle on a compiled oracle library at ``path`` with its signatures set."""
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_physical_index.restype = i64
    L.oracle_physical_index.argtypes = [p, i64, i64]
    L.oracle_slot_mapping.restype = i32
    L.oracle_slot_mapping.argtypes = [p, p, i64, p, i64, i64]
    L.oracle_kv_write.restype = i32
    L.oracle_kv_write.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32]
    L.oracle_copy_blocks.restype = i32
    L.oracle_copy_blocks.argtypes = [p, p, p, i64, i64, i64, i64, i64, i32]
    L.oracle_paged_attention.restype = i32
    L.oracle_paged_attention.argtypes = [p, p, p, p, p, i64, p, i64, i64, i64, i64, i64, i64,
                                         ctypes.c_double, i64, p, i64, i32, i32]
    L.oracle_max_threads.restype = i32
    L.oracle_max_threads.argtypes = []
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"error {rc}"))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:        # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def physical_index(table, block_size: int, pos: int) -> int:
    t = np.ascontiguousarray(table, dtype=np.int32)
    return int(lib().oracle_physical_index(_ptr(t), block_size, pos))


def slot_mapping(block_tables: np.ndarray, positions, block_size: int) -> np.ndarray:
    """slots[i] = PhysicalIndex(block_tables[i], positions[i]) (one row per token)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    out = np.empty(len(pos), dtype=np.int64)
    _check(lib().oracle_slot_mapping(_ptr(out), _ptr(bt), bt.shape[1], _ptr(pos), len(pos), block_size))
    return out


def kv_write(k_new, v_new, k_cache, v_cache, slots) -> None:
    """In place: k_cache[s // B, s % B] = k_new[i] (bytes), same for V."""
    N, B, Hkv, D = k_cache.shape
    for a in (k_new, v_new, k_cache, v_cache):
        assert a.flags.c_contiguous and a.dtype == k_cache.dtype
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    _check(lib().oracle_kv_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(sl),
                                 len(sl), N, B, Hkv, D, _dtype_code(k_cache)))


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """In place: for each (src, dst), block dst of K and V becomes a byte copy of block src."""
    N, B, Hkv, D = k_cache.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    _check(lib().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pr), pr.shape[0], N, B, Hkv, D,
                                    _dtype_code(k_cache)))


def attention(q, k_cache, v_cache, block_tables, context_lens, scale: float, partition_size: int = 0,
              items=None, num_threads: int = 0) -> np.ndarray:
    """fp64 paged attention.  Returns [S, Hq, D], or [len(items), D] for items = s * Hq + h."""
    S, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    for a in (q, k_cache, v_cache):
        assert a.flags.c_contiguous and a.dtype == q.dtype
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    it = None if items is None else np.ascontiguousarray(items, dtype=np.int64)
    n = S * Hq if it is None else len(it)
    out = np.empty((n, D), dtype=np.float64)
    _check(lib().oracle_paged_attention(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), bt.shape[1], _ptr(cl),
        S, Hq, Hkv, D, B, N, float(scale), int(partition_size),
        None if it is None else _ptr(it), 0 if it is None else len(it), _dtype_code(q), int(num_threads)))
    return out.reshape(S, Hq, D) if it is None else out


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ---------------------------------------------------------------------------
# numpy textbook reference: gather through the table, then dense attention
# ---------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """fp32 or bf16 bit patterns -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gather_sequence(cache: np.ndarray, table, ctx: int) -> np.ndarray:
    """Contiguous [ctx, Hkv, D] copy of one sequence's rows: its blocks concatenated in
    table order, cut at ctx (tokentrails page, Code box: torch.cat over the table)."""
    B = cache.shape[1]
    nblk = -(-ctx // B)
    return np.concatenate([cache[int(table[j])] for j in range(nblk)], axis=0)[:ctx]


def dense_attention(q, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """Ordinary softmax(q K^T * scale) V per (sequence, head) on gathered K/V, in float64."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    qf = widen(q)
    out = np.empty((S, Hq, D))
    for s in range(S):
        ctx = int(context_lens[s])
        K = widen(gather_sequence(k_cache, block_tables[s], ctx))     # [ctx, Hkv, D]
        V = widen(gather_sequence(v_cache, block_tables[s], ctx))
        for h in range(Hq):
            x = scale * (K[:, h // g, :] @ qf[s, h])                    # [ctx]
            w = np.exp(x - x.max())
            out[s, h] = (w @ V[:, h // g, :]) / w.sum()
    return out


# ---------------------------------------------------------------------------
# the head-major cache layout (page "PagedAttention", PidokuInfra topic 10, section 5,
# "The layout, more precisely"): per block, per KV head,
#   key_cache   [num_blocks, num_kv_heads, head_dim / x, block_size, x],  x = 16 / sizeof(dtype)
#   value_cache [num_blocks, num_kv_heads, head_dim, block_size]
# so that 16 bytes of K hold x consecutive head dims of one token and the block_size tokens
# of one V head dim are consecutive.  The values are those of the row layout
# [num_blocks, block_size, num_kv_heads, head_dim], only placed differently.
# ---------------------------------------------------------------------------

def head_major_x(dtype) -> int:
    """Elements of one 16-byte K vector: 8 for bf16, 4 for fp32."""
    return 16 // np.dtype(dtype).itemsize


def rows_from_head_major(k_hm: np.ndarray, v_hm: np.ndarray):
    """Row-layout copies: K[b, o, h, d] = K_hm[b, h, d // x, o, d % x], V[b, o, h, d] = V_hm[b, h, d, o]."""
    N, Hkv, Dx, B, x = k_hm.shape
    k = np.ascontiguousarray(k_hm.transpose(0, 3, 1, 2, 4).reshape(N, B, Hkv, Dx * x))
    v = np.ascontiguousarray(v_hm.transpose(0, 3, 1, 2))
    return k, v


def head_major_from_rows(k_rows: np.ndarray, v_rows: np.ndarray):
    """The head-major placement of row-layout K/V [N, B, Hkv, D]."""
    N, B, Hkv, D = k_rows.shape
    x = head_major_x(k_rows.dtype)
    k = np.ascontiguousarray(k_rows.reshape(N, B, Hkv, D // x, x).transpose(0, 2, 3, 1, 4))
    v = np.ascontiguousarray(v_rows.transpose(0, 2, 3, 1))
    return k, v


def kv_write_head_major(k_new, v_new, k_hm, v_hm, slots) -> None:
    """In place: token i with slot s = b * B + o lands in K_hm[b, :, :, o, :] and V_hm[b, :, :, o]."""
    N, Hkv, Dx, B, x = k_hm.shape
    sl = np.asarray(slots, dtype=np.int64)
    if len(set(sl.tolist())) != len(sl):
        raise OracleError(_ERRORS[-3])
    for i, s in enumerate(sl.tolist()):
        if s < 0 or s >= N * B:
            raise OracleError(_ERRORS[-2])
        b, o = divmod(s, B)
        k_hm[b, :, :, o, :] = k_new[i].reshape(Hkv, Dx, x)
        v_hm[b, :, :, o] = v_new[i]


def attention_head_major(q, k_hm, v_hm, block_tables, context_lens, scale: float, partition_size: int = 0,
                         items=None, num_threads: int = 0) -> np.ndarray:
    """fp64 paged attention on a head-major pool: the same attention as on the row layout."""
    k, v = rows_from_head_major(k_hm, v_hm)
    return attention(q, k, v, block_tables, context_lens, scale, partition_size, items, num_threads)
