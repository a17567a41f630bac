"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and sizes buffers.  It holds none of the
paged-attention arithmetic: no slot formula, no block-table walk, no softmax.
Both the HIP path and the CPU oracle consume the bytes produced here.

Workload shapes follow the five serving-shaped decode configurations this
project is measured on (tiny fp32 check, 7B-shaped MHA layer, 70B-shaped GQA
layer, long-context split-K, shared-prefix fork with copy-on-write).  The
decode-step reading used everywhere: the newest token sits at position
``ctx - 1`` and is attended to in the same step.

Draw order for one configuration (one ``numpy.random.Generator`` seeded with
the configuration's seed): context lengths (or generated lengths for the fork
workload), then the free-list order of the pool.  The large tensors (q, K pool,
V pool, new K/V rows) are drawn from independent child streams of the same
seed, in fixed chunks, so the bytes do not depend on the thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                 # "f32" or "bf16"
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx: tuple                 # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("fork", prompt, lo, hi)
    seed: int
    num_blocks: int | None = None   # fixed pool size (tiny config); else sized from the lengths
    partition_size: int = 0         # split-K partition the configuration names (0 = none named)
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "tiny_fp32": Config(
        "tiny_fp32", "f32", 4, 4, 4, 64, 4, ("uniform", 1, 64), seed=1, num_blocks=80,
        description="4 seqs, ctx U{1..64}, B=4, 4 q = 4 kv heads, D=64, pool of 80 blocks, fp32"),
    "mha7b": Config(
        "mha7b", "bf16", 64, 32, 32, 128, 16, ("uniform", 512, 2048), seed=2,
        description="7B-shaped MHA decode layer: 64 seqs, 32/32 heads, D=128, B=16, ctx U{512..2048}, bf16"),
    "gqa70b": Config(
        "gqa70b", "bf16", 256, 64, 8, 128, 16, ("lognormal", 1024, 1.0, 16, 8192), seed=3,
        description="70B-shaped GQA decode layer: 256 seqs, 64/8 heads, D=128, B=16, "
                    "ctx log-normal median 1024 (sigma 1.0) clipped 16..8192, bf16"),
    "long_splitk": Config(
        "long_splitk", "bf16", 8, 32, 8, 128, 16, ("uniform", 32768, 131072), seed=4,
        partition_size=512,
        description="long-context split-K: 8 seqs, 32/8 heads, D=128, B=16, ctx U{32768..131072}, "
                    "512-token partitions, bf16"),
    "fork_cow": Config(
        "fork_cow", "bf16", 16, 32, 8, 128, 16, ("fork", 2000, 80, 512), seed=5,
        description="shared-prefix fork + CoW: 16 seqs forked from one 2000-token prompt, "
                    "each with 80..512 own tokens, 32/8 heads, D=128, B=16, bf16"),
}

FORK_PROMPT_TOKENS = 2000   # prompt length of the fork workload
FORK_CHILDREN = 15          # children forked from the parent (refcount 16 on the shared blocks)

# child-stream ids for the bulk tensors
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_KNEW, _STREAM_VNEW = 1, 2, 3, 4, 5
_CHUNK = 1 << 22


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# scalar draws
# ---------------------------------------------------------------------------

def draw_context_lens(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths (tokens attended, newest token included), int64 [S]."""
    kind = cfg.ctx[0]
    if kind == "uniform":
        _, lo, hi = cfg.ctx
        return rng.integers(lo, hi, size=cfg.num_seqs, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        _, median, sigma, lo, hi = cfg.ctx
        z = rng.standard_normal(cfg.num_seqs)
        return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)
    if kind == "fork":
        raise ValueError("fork workload: use draw_fork_generated")
    raise ValueError(kind)


def draw_fork_generated(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Own generated-token counts of the fork workload's 16 sequences, U{lo..hi}."""
    _, _, lo, hi = cfg.ctx
    return rng.integers(lo, hi, size=cfg.num_seqs, endpoint=True).astype(np.int64)


def pool_size(cfg: Config, tokens_per_seq_unique: np.ndarray, extra_blocks: int = 0) -> int:
    """Pool size: the configured count, else the needed blocks plus 10% free (plus extras)."""
    if cfg.num_blocks is not None:
        return cfg.num_blocks
    need = int(sum(-(-int(t) // cfg.block_size) for t in tokens_per_seq_unique))
    return int(math.ceil(1.1 * need)) + extra_blocks


def draw_free_order(num_blocks: int, rng: np.random.Generator) -> list[int]:
    """Seeded shuffled pool: the initial free stack (allocation takes from its end)."""
    return [int(x) for x in rng.permutation(num_blocks)]


# ---------------------------------------------------------------------------
# bulk normal draws (chunked, thread-count independent)
# ---------------------------------------------------------------------------

def _fill_normal_chunk(seed: int, stream: int, chunk: int, out: np.ndarray, bf16: bool) -> None:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))
    x = g.standard_normal(out.shape[0], dtype=np.float32)
    if bf16:
        u = x.view(np.uint32)
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))   # round to nearest even
        out[:] = u.view(np.uint16)[1::2]                                  # high halves (little endian)
    else:
        out[:] = x


def normal(n: int, seed: int, stream: int, dtype: str) -> np.ndarray:
    """n values ~ N(0,1): float32, or bf16 bit patterns (uint16) rounded to nearest even."""
    bf16 = dtype == "bf16"
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = -(-n // _CHUNK)
    jobs = [(seed, stream, c, out[c * _CHUNK:(c + 1) * _CHUNK], bf16) for c in range(nchunks)]
    if nchunks <= 1:
        for j in jobs:
            _fill_normal_chunk(*j)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda j: _fill_normal_chunk(*j), jobs))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bf16 is the high half of fp32)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# one workload instance
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """Host-side inputs of one decode step (numpy; bf16 held as uint16 bit patterns)."""
    cfg: Config
    context_lens: np.ndarray        # int64 [S] (for the fork workload: the steady-step lengths)
    free_order: list[int]           # initial free stack of the pool
    num_blocks: int
    q: np.ndarray                   # [S, Hq, D]
    k_cache: np.ndarray             # [N, B, Hkv, D]
    v_cache: np.ndarray
    k_new: np.ndarray               # [S, Hkv, D]  the newest token's K/V rows
    v_new: np.ndarray
    fork_generated: np.ndarray | None = None   # fork workload only: own generated tokens per seq

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.cfg.head_dim)


def make_workload(cfg: Config | str, num_seqs: int | None = None, seed: int | None = None,
                  ctx_override: np.ndarray | None = None) -> Workload:
    """Draw one decode-step workload.

    ``num_seqs`` shrinks the batch (same distributions); ``ctx_override`` replaces the drawn
    lengths (edge-case tests).  The pool is sized from the lengths actually used.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if num_seqs is not None and num_seqs != cfg.num_seqs:
        cfg = Config(**{**cfg.__dict__, "num_seqs": num_seqs})
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, D, B = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size

    fork_gen = None
    if cfg.ctx[0] == "fork":
        fork_gen = draw_fork_generated(cfg, rng)
        prompt = cfg.ctx[1]
        ctx = prompt + 1 + fork_gen                 # parent's first token, then own tokens
        # unique tokens: shared full prompt blocks once, each sequence's own tail
        shared_full = prompt // B
        unique = [shared_full * B] + [int(c) - shared_full * B for c in ctx]
        n_blocks = pool_size(cfg, np.array(unique), extra_blocks=FORK_CHILDREN)
    else:
        ctx = draw_context_lens(cfg, rng) if ctx_override is None else np.asarray(ctx_override, np.int64)
        if ctx_override is not None:
            cfg = Config(**{**cfg.__dict__, "num_seqs": len(ctx)})
            S = cfg.num_seqs
        n_blocks = pool_size(cfg, ctx)
    free_order = draw_free_order(n_blocks, rng)

    dt = cfg.dtype
    q = normal(S * Hq * D, seed, _STREAM_Q, dt).reshape(S, Hq, D)
    kc = normal(n_blocks * B * Hkv * D, seed, _STREAM_K, dt).reshape(n_blocks, B, Hkv, D)
    vc = normal(n_blocks * B * Hkv * D, seed, _STREAM_V, dt).reshape(n_blocks, B, Hkv, D)
    kn = normal(S * Hkv * D, seed, _STREAM_KNEW, dt).reshape(S, Hkv, D)
    vn = normal(S * Hkv * D, seed, _STREAM_VNEW, dt).reshape(S, Hkv, D)
    return Workload(cfg, np.asarray(ctx, np.int64), free_order, n_blocks, q, kc, vc, kn, vn, fork_gen)


def numpy_dtype(cfg: Config):
    return np.float32 if cfg.dtype == "f32" else np.uint16


# ---------------------------------------------------------------------------
# request streams for the allocator simulation: Poisson arrivals, log-normal prompt and
# output lengths (PidokuInfra page, section 10, exercise B)
# ---------------------------------------------------------------------------

@dataclass
class RequestStream:
    arrival: np.ndarray   # int64 step at which each request arrives (non-decreasing)
    prompt: np.ndarray    # int64 prompt tokens
    output: np.ndarray    # int64 tokens it will generate (>= 1)
    max_len: int          # the longest sequence a request may reach (prompt + output <= max_len)


def request_stream(seed: int, n: int, rate: float, prompt_median: float, output_median: float,
                   sigma: float = 1.0, max_len: int = 2048) -> RequestStream:
    """n requests: exponential gaps of mean 1/rate steps; prompt and output lengths
    round(median * exp(sigma * z)), z ~ N(0, 1), with 1 <= prompt <= max_len - 1 and
    1 <= output <= max_len - prompt."""
    rng = np.random.default_rng(seed)
    arrival = np.floor(np.cumsum(rng.exponential(1.0 / rate, size=n))).astype(np.int64)
    prompt = np.clip(np.round(prompt_median * np.exp(sigma * rng.standard_normal(n))), 1, max_len - 1).astype(np.int64)
    output = np.round(output_median * np.exp(sigma * rng.standard_normal(n))).astype(np.int64)
    output = np.clip(output, 1, max_len - prompt)
    return RequestStream(arrival, prompt, output, max_len)
