"""Thin Python binding over libpkv.so's C ABI (include/pkv.h).

Argument marshalling only: tensors become device pointers and sizes, the launch
stream is the call's `stream` argument (a torch.cuda.Stream or a raw handle) or
else torch's current HIP stream, and a non-OK status raises PkvError.  Every step
of the computation runs in the library's HIP kernels; there is no fallback path,
so a missing or unloadable library raises immediately.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP, PKV_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
PKV_DTYPE_F32, PKV_DTYPE_BF16 = 0, 1
PKV_PATH_NONE, PKV_PATH_VECTOR, PKV_PATH_MFMA, PKV_PATH_TILE_VALU = 0, 1, 2, 3

# every symbol include/pkv.h declares
EXPORTS = ("paged_kv_write", "paged_attention_decode", "copy_blocks", "pkv_attention_workspace_size",
           "pkv_attention_path", "pkv_status_string", "paged_kv_write_head_major",
           "paged_attention_decode_head_major", "pkv_attention_path_head_major", "pkv_stream_read_probe",
           "paged_attention_decode_write", "paged_attention_decode_noalloc", "pkv_static_scratch_bytes")

_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


def lib():
    """The loaded libpkv.so with its C signatures; raises if it is not built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime: load it first so that libpkv.so binds to the same
        # runtime instance rather than pulling in a second copy from the system path
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_148_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.paged_kv_write.restype = ctypes.c_int
        L.paged_kv_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i32, ctypes.c_int, p]
        L.pkv_attention_workspace_size.restype = sz
        L.pkv_attention_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.pkv_attention_path.restype = ctypes.c_int
        L.pkv_attention_path.argtypes = [i32, i32, i32, i32, ctypes.c_int]
        L.paged_attention_decode.restype = ctypes.c_int
        L.paged_attention_decode.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.c_float, i32, p, sz, ctypes.c_int, p]
        L.paged_kv_write_head_major.restype = ctypes.c_int
        L.paged_kv_write_head_major.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i32, ctypes.c_int, p]
        L.paged_attention_decode_head_major.restype = ctypes.c_int
        L.paged_attention_decode_head_major.argtypes = L.paged_attention_decode.argtypes
        L.pkv_attention_path_head_major.restype = ctypes.c_int
        L.pkv_attention_path_head_major.argtypes = [i32, i32, i32, i32, ctypes.c_int]
        L.copy_blocks.restype = ctypes.c_int
        L.copy_blocks.argtypes = [p, p, p, i64, i32, i32, i32, i32, ctypes.c_int, p]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_status_string.argtypes = [ctypes.c_int]
        L.paged_attention_decode_write.restype = ctypes.c_int
        L.paged_attention_decode_write.argtypes = [p, p, p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i32, i32,
                                                   ctypes.c_float, i32, p, sz, ctypes.c_int, p]
        L.pkv_stream_read_probe.restype = ctypes.c_int
        L.pkv_stream_read_probe.argtypes = [p, sz, p, p]
        L.paged_attention_decode_noalloc.restype = ctypes.c_int
        L.paged_attention_decode_noalloc.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i32, i32,
                                                     ctypes.c_float, i32, ctypes.c_int, p]
        L.pkv_static_scratch_bytes.restype = sz
        L.pkv_static_scratch_bytes.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def _check(status: int, call: str):
    if status != PKV_OK:
        raise PkvError(status, call)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PKV_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    """Raw hipStream_t of the launch stream: `stream` (a torch.cuda.Stream or a raw handle), else
    torch's current stream on t's device."""
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _workspace(workspace, nbytes: int, t, stream):
    """The caller's workspace, or a fresh one whose work-queue header is zeroed on the launch
    stream itself (so the zero-fill precedes the launch) and which the caching allocator does not
    hand out again before the work queued on that stream is done."""
    if workspace is not None:
        return workspace
    torch = _torch()
    if stream is None:
        # the launch stream is torch's current stream: memory freed when this call returns is only
        # reused by work queued after the launch on that same stream
        return torch.zeros(nbytes, dtype=torch.uint8, device=t.device)
    st = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=t.device)
    with torch.cuda.stream(st):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=t.device)
    ws.record_stream(st)
    return ws


def attention_workspace_size(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                             partition_size: int) -> int:
    return int(lib().pkv_attention_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size))


def attention_path(num_heads: int, num_kv_heads: int, head_dim: int, block_size: int, dtype_code: int) -> int:
    return int(lib().pkv_attention_path(num_heads, num_kv_heads, head_dim, block_size, dtype_code))


def paged_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """k_cache[slot // B, slot % B] = k_new[i] (and V) for every token i."""
    torch = _torch()
    N, B, Hkv, D = k_cache.shape
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between k_new/v_new [T, Hkv, D], caches [N, B, Hkv, D] and slots [T]")
    dt = k_cache.dtype
    st = lib().paged_kv_write(_dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt), _dev(k_cache, "k_cache", dt),
                              _dev(v_cache, "v_cache", dt), _dev(slot_mapping, "slot_mapping", torch.int64),
                              T, N, B, Hkv, D, _dtype_code(k_cache), _stream(k_cache, stream))
    _check(st, "paged_kv_write")


def copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """For each row (src, dst) of block_mapping: block dst := block src, in both pools."""
    torch = _torch()
    N, B, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("caches must match and block_mapping must be [P, 2]")
    dt = k_cache.dtype
    st = lib().copy_blocks(_dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
                           _dev(block_mapping, "block_mapping", torch.int64), block_mapping.shape[0],
                           N, B, Hkv, D, _dtype_code(k_cache), _stream(k_cache, stream))
    _check(st, "copy_blocks")


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                           scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over each sequence's table.

    workspace: a device buffer of at least attention_workspace_size(...) bytes whose first
    256 bytes were zeroed when it was allocated (if None, a fresh one is zeroed on the launch
    stream).  stream: a torch.cuda.Stream or a raw hipStream_t handle; None = torch's current
    stream."""
    torch = _torch()
    S, Hq, D = q.shape
    N, B, Hkv, D2 = k_cache.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out [S, Hq, D] and caches [N, B, Hkv, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    # zeroed when made here: its leading work-queue counters must start at zero
    workspace = _workspace(workspace, attention_workspace_size(S, Hq, D, max_context_len, partition_size), q, stream)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = q.dtype
    st = lib().paged_attention_decode(
        _dev(out, "out", dt), _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B, N,
        float(scale), int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(q, stream))
    _check(st, "paged_attention_decode")


def static_scratch_bytes() -> int:
    """Bytes of the library's static device scratch behind paged_attention_decode_noalloc."""
    return int(lib().pkv_static_scratch_bytes())


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                                   scale: float, partition_size: int = 0, stream=None) -> None:
    """paged_attention_decode with its scratch in the library's static device array: nothing is
    allocated, here or in the library.  Calls that may overlap on one device must not be issued."""
    torch = _torch()
    S, Hq, D = q.shape
    N, B, Hkv, D2 = k_cache.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out [S, Hq, D] and caches [N, B, Hkv, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    dt = q.dtype
    st = lib().paged_attention_decode_noalloc(
        _dev(out, "out", dt), _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B, N,
        float(scale), int(partition_size), _dtype_code(q), _stream(q, stream))
    _check(st, "paged_attention_decode_noalloc")


def paged_attention_decode_write(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                 max_context_len: int, scale: float, partition_size: int = 0, workspace=None,
                                 stream=None) -> None:
    """paged_kv_write of k_new[s], v_new[s] at position context_lens[s] - 1 of each sequence
    (the slot from its table), then paged_attention_decode; one launch on the tile paths."""
    torch = _torch()
    S, Hq, D = q.shape
    N, B, Hkv, D2 = k_cache.shape
    if D2 != D or tuple(out.shape) != (S, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q/out [S, Hq, D] and caches [N, B, Hkv, D]")
    if tuple(k_new.shape) != (S, Hkv, D) or tuple(v_new.shape) != (S, Hkv, D):
        raise ValueError("k_new and v_new must be [S, Hkv, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    workspace = _workspace(workspace, attention_workspace_size(S, Hq, D, max_context_len, partition_size), q, stream)
    dt = q.dtype
    st = lib().paged_attention_decode_write(
        _dev(out, "out", dt), _dev(q, "q", dt), _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        N, float(scale), int(partition_size), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(q, stream))
    _check(st, "paged_attention_decode_write")


# ---------------------------------------------------------------------------
# head-major cache layout: k_cache [N, Hkv, D/x, B, x] (x = 16 / element bytes),
# v_cache [N, Hkv, D, B]
# ---------------------------------------------------------------------------

def _head_major_shape(k_cache, v_cache):
    N, Hkv, Dx, B, x = k_cache.shape
    D = Dx * x
    if x * k_cache.element_size() != 16 or tuple(v_cache.shape) != (N, Hkv, D, B):
        raise ValueError("head-major caches must be k [N, Hkv, D/x, B, x] with x * elem = 16 and v [N, Hkv, D, B]")
    return N, B, Hkv, D


def attention_path_head_major(num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                              dtype_code: int) -> int:
    return int(lib().pkv_attention_path_head_major(num_heads, num_kv_heads, head_dim, block_size, dtype_code))


def paged_kv_write_head_major(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """paged_kv_write into head-major caches."""
    torch = _torch()
    N, B, Hkv, D = _head_major_shape(k_cache, v_cache)
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("k_new/v_new must be [T, Hkv, D]")
    dt = k_cache.dtype
    st = lib().paged_kv_write_head_major(
        _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, N, B, Hkv, D, _dtype_code(k_cache),
        _stream(k_cache, stream))
    _check(st, "paged_kv_write_head_major")


def copy_blocks_head_major(k_cache, v_cache, block_mapping, stream=None) -> None:
    """copy_blocks on head-major caches (a block is the same bytes in either layout)."""
    torch = _torch()
    N, B, Hkv, D = _head_major_shape(k_cache, v_cache)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [P, 2]")
    dt = k_cache.dtype
    st = lib().copy_blocks(_dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
                           _dev(block_mapping, "block_mapping", torch.int64), block_mapping.shape[0],
                           N, B, Hkv, D, _dtype_code(k_cache), _stream(k_cache, stream))
    _check(st, "copy_blocks")


def paged_attention_decode_head_major(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                                      scale: float, partition_size: int = 0, workspace=None, stream=None) -> None:
    """paged_attention_decode on head-major caches."""
    torch = _torch()
    S, Hq, D = q.shape
    N, B, Hkv, D2 = _head_major_shape(k_cache, v_cache)
    if D2 != D or tuple(out.shape) != (S, Hq, D):
        raise ValueError("shape mismatch between q/out [S, Hq, D] and the caches")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    workspace = _workspace(workspace, attention_workspace_size(S, Hq, D, max_context_len, partition_size), q, stream)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = q.dtype
    st = lib().paged_attention_decode_head_major(
        _dev(out, "out", dt), _dev(q, "q", dt), _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B, N,
        float(scale), int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(q, stream))
    _check(st, "paged_attention_decode_head_major")


def stream_read_probe(buf, sink, stream=None) -> None:
    """Measurement only: one plain streaming read of the whole of `buf` (a GPU tensor), the
    bandwidth reference for the decode kernels.  `sink` is a GPU int32 tensor of at least one
    element that the kernel may write."""
    torch = _torch()
    if not buf.is_cuda or not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("stream_read_probe needs a GPU buffer and a GPU int32 sink")
    st = lib().pkv_stream_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                     ctypes.c_void_p(sink.data_ptr()), _stream(buf, stream))
    _check(st, "pkv_stream_read_probe")
