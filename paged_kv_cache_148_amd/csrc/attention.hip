// attention.hip -- paged decode attention for gfx950 (CDNA4).
//
// For every sequence s and query head h:
//   out[s,h] = softmax(scale * q[s,h] . K_s^T) V_s,
// K_s / V_s being the rows of positions 0..ctx-1, position t stored in physical block
// table[s][t / B] at offset t % B of the pool [N, B, Hkv, D].  The kernels walk the
// block table and accumulate with an online softmax (page "PagedAttention",
// PidokuInfra topic 10, section 5 "The kernel side"); the result is the ordinary
// attention over the gathered rows (page "PagedAttention", tokentrails, step 3).
//
// Work unit: one (KV head, context partition, sequence) item, processed by one
// workgroup of 4 waves.  An item serves every query head of the KV head's group, so each
// K/V byte is read once per group.  Without a partition size the partition is the whole
// context.  With one, an item leaves a partial state (running max m, sum l, unnormalised
// o) in the workspace and attn_reduce_kernel merges the partials by log-sum-exp;
// sequences whose context fits one partition are finished in pass 1.
//
// Scheduling: the pass-1 kernels are persistent.  As many workgroups as fit on the chip
// each build, in LDS, the prefix sum of per-sequence item counts from context_lens (so
// only non-empty items exist).  Workgroup b starts with item b and then takes items in
// order from a work-queue counter in the workspace until none are left; the kernel that
// follows (the merge, or a one-thread reset) returns the counter to zero.  A dynamic
// queue keeps every XCD busy until the end even though the XCDs do not run at identical
// speeds, and no launch slot is spent on empty partitions.  Batches too large to stage in
// LDS fall back to one workgroup per possible item.
//
// Two pass-1 kernels:
//   attn_mfma_kernel  (bf16, D = 128, B % 16 == 0, 2 <= g <= 16): a 16-token tile of
//     K times the group's Q^T on v_mfma_f32_16x16x32_bf16 gives the score tile; the
//     probabilities stay in the MFMA result layout and feed v_mfma_f32_16x16x16_bf16
//     against V^T for P.V.  The head dimension of the P.V product is permuted so that
//     each lane's V operand is one 16-byte row piece of 4 tokens, regrouped in
//     registers (no LDS round trip for V).
//   attn_vec_kernel   (everything else: g = 1, fp32, D = 64, small blocks): one token
//     row per D*e/16 lanes, 16-byte loads along head_dim, q.k as fp32 FMAs on exactly
//     widened elements, row sums by DPP.
// Scores carry scale * log2(e) so every exponential is a hardware exp2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_device.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMfmaDepth = 3;          // tiles in flight per wave on the MFMA path
constexpr int kMaxReduceParts = 8192;    // partials per (seq, head) the reduce kernel stages in LDS (32 KiB)
constexpr int kMaxSchedSeqs = 4096;     // sequences whose schedule fits in LDS (2 x 16 KiB)
constexpr size_t kQueueBytes = 256;     // work-queue header at the start of the workspace

struct AttnArgs {
  void *out;
  const void *q;
  const void *k;
  const void *v;
  const int32_t *tables;
  const int32_t *ctx;
  float *ws_o;       // [S, Hq, max_parts, D]
  float *ws_m;       // [S, Hq, max_parts]   log2-domain running max
  float *ws_l;       // [S, Hq, max_parts]
  int max_blocks;    // table row length
  int max_ctx;       // host bound on ctx
  int Hq, Hkv, g, N;
  int P;             // partition length in tokens (whole context when not splitting)
  int max_parts;
  float scale_log2;  // scale * log2(e)
  int S;             // sequences
  unsigned *queue;   // [0]: items taken beyond the grid (zero between calls)
  int persistent;    // 1: persistent workgroups + work queue; 0: one workgroup per possible item
};

// Work-item order across the chip.  Workgroups go round-robin to the 8 XCDs by their
// 1-D index.  The logical order has the KV head fastest (then partition, then sequence),
// so with Hkv a multiple of 8 each XCD receives the same KV heads of every (sequence,
// partition) -- identical amounts of work -- whatever the context-length mix.  (With the
// partition index fastest, XCD x would receive only partitions p = x mod 8, and short
// contexts would leave half the XCDs idle.)
struct WorkItem {
  int p, kvh, s;
};
__device__ __forceinline__ WorkItem work_item(int Hkv, int parts) {
  const int w = (int)blockIdx.x;
  WorkItem it;
  it.kvh = w % Hkv;
  it.p = (w / Hkv) % parts;
  it.s = w / (Hkv * parts);
  return it;
}

// Work-queue schedule.  Item counts per sequence: ceil(ctx / P) partitions times Hkv
// (one item per KV head for a sequence with an unusable length, which only writes its
// fill value).  sm_pref receives the inclusive prefix sum and sm_ctx the lengths; the
// return value is the total number of items.
__device__ int build_schedule(const AttnArgs &a, int *sm_pref, int *sm_ctx, int *sm_tmp) {
  const int S = a.S, tid = threadIdx.x;
  const int per = (S + kThreads - 1) / kThreads;
  const int lo = min(tid * per, S), hi = min(lo + per, S);
  int run = 0;
  for (int i = lo; i < hi; ++i) {
    const int c = a.ctx[i];
    sm_ctx[i] = c;
    const int np = (c >= 1 && c <= a.max_ctx) ? (c + a.P - 1) / a.P : 1;
    run += np * a.Hkv;
    sm_pref[i] = run;
  }
  int x = run;   // inclusive scan of the per-thread runs: within the wave, then across waves
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if ((tid & 63) >= off) x += y;
  }
  if ((tid & 63) == 63) sm_tmp[tid >> 6] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < (tid >> 6); ++w) before += sm_tmp[w];
  const int excl = before + x - run;
  for (int i = lo; i < hi; ++i) sm_pref[i] += excl;
  __syncthreads();
  return sm_pref[S - 1];
}

// Item w -> (sequence, partition, KV head): the first sequence whose inclusive prefix
// exceeds w, then KV head fastest within it.
__device__ __forceinline__ WorkItem decode_item(int w, const int *sm_pref, int S, int Hkv) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sm_pref[mid] > w) hi = mid; else lo = mid + 1;
  }
  const int r = w - (lo ? sm_pref[lo - 1] : 0);
  WorkItem it;
  it.s = lo;
  it.kvh = r % Hkv;
  it.p = r / Hkv;
  return it;
}

// Common driver of the pass-1 kernels: persistent work-queue loop, or one item per
// workgroup.  ITEM(s, p, kvh, ctx) processes an item (ctx < 0: read it from memory).
struct SchedSmem {
  int tmp[kWaves];
  int next;
};
template <typename Item>
__device__ __forceinline__ void run_items(const AttnArgs &a, SchedSmem &sc, int *sm_dyn, Item item) {
  if (!a.persistent) {
    const WorkItem it = work_item(a.Hkv, a.max_parts);
    item(it.s, it.p, it.kvh, -1);
    return;
  }
  const int tid = threadIdx.x;
  int *sm_pref = sm_dyn, *sm_ctx = sm_dyn + a.S;
  const int total = build_schedule(a, sm_pref, sm_ctx, sc.tmp);
  // Workgroup b starts with item b; later items come one at a time from the queue counter,
  // which counts items beyond the grid.  The next index is fetched while the current item
  // runs.
  int w = (int)blockIdx.x;
  while (w < total) {
    unsigned c = 0;
    if (tid == 0) c = atomicAdd(&a.queue[0], 1u);
    const WorkItem it = decode_item(w, sm_pref, a.S, a.Hkv);
    item(it.s, it.p, it.kvh, sm_ctx[it.s]);
    if (tid == 0) sc.next = (int)(gridDim.x + c);
    __syncthreads();
    w = sc.next;
    __syncthreads();
  }
}

// Merge weight of a partial state with max m into a combined max M (empty state -> 0).
__device__ __forceinline__ float merge_weight(float m, float M) { return m == kNegInf ? 0.f : fast_exp2(m - M); }

template <typename T>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v) {
  if constexpr (sizeof(T) == 4)
    reinterpret_cast<float *>(out)[idx] = v;
  else
    reinterpret_cast<uint16_t *>(out)[idx] = f32_to_bf16(v);
}

// Outputs of a sequence whose length is unusable: 0 for ctx <= 0, NaN for ctx above
// the host bound.
template <typename T, int D>
__device__ void fill_group(const AttnArgs &a, int s, int h0, int g, float v) {
  for (int i = threadIdx.x; i < g * D; i += blockDim.x) store_out<T>(a.out, ((size_t)s * a.Hq + h0) * D + i, v);
}

// Final phase of pass 1, shared by both kernels: the per-wave states (sm_m, sm_l,
// sm_o) are merged, then either normalised into `out` or stored as a partial.
template <typename T, int D, int GS, int OSTRIDE>
__device__ __forceinline__ void finish_group(const AttnArgs &a, int s, int kvh, int p, bool single,
                                             const float (*sm_m)[GS], const float (*sm_l)[GS],
                                             const float (*sm_o)[GS][OSTRIDE], const int *sm_bad) {
  const int g = a.g;
  const bool bad = sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3];
  for (int idx = threadIdx.x; idx < g * D; idx += kThreads) {
    const int j = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = merge_weight(sm_m[w][j], M);
      L += wt * sm_l[w][j];
      o += wt * sm_o[w][j][d];
    }
    if (bad) {
      M = 0.f;
      L = __builtin_nanf("");
      o = __builtin_nanf("");
    }
    const int h = kvh * g + j;
    if (single) {
      store_out<T>(a.out, ((size_t)s * a.Hq + h) * D + d, o / L);
    } else {
      const size_t part = ((size_t)s * a.Hq + h) * a.max_parts + p;
      a.ws_o[part * D + d] = o;
      if (d == 0) {
        a.ws_m[part] = M;
        a.ws_l[part] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA path: bf16, D = 128, B in {16, 32}, group of up to 16 query heads.
//
// Lane l of a wave: c16 = l % 16, grp = l / 16.
//   QK  (v_mfma_f32_16x16x32_bf16, A = K tile [16 tokens x 32 d], B = Q^T [32 d x 16 heads]):
//       lane l needs token c16's d-slice 32c + 8grp .. +7 for c = 0..3 and the same
//       slice of head c16's q row.  K is loaded as whole rows (like V, below) and turned
//       into this layout through a per-wave LDS staging tile.  Result S^T: lane l holds
//       tokens 4grp + r (r = 0..3) of head c16.
//   P.V (v_mfma_f32_16x16x16_bf16, A = V^T [16 d-rows x 16 tokens], B = P^T [16 tokens x
//       16 heads]): B is exactly the S^T result layout (head c16, tokens 4grp + r).  MFMA
//       number i (0..7) gives A-row c16 the head-dim index 8*c16 + i, so lane l needs
//       d = 8*c16 .. 8*c16+7 of tokens 4grp + r: one 16-byte load per token, regrouped
//       into (token pair, d) halves with byte permutes.  The accumulator of MFMA i holds,
//       in lane l, row 4grp + r' -> d = 32*grp + 8*r' + i of head c16.
//
// Loads are buffer loads through a per-tile descriptor held in SGPRs (base = the tile's
// first row, range = the tile's 16 rows), so the lane offsets are loop invariant.  A
// tile past the end gets a zero-range descriptor: its loads return zeros without a
// memory access, which keeps the number of loads in flight the same on every path.
// ---------------------------------------------------------------------------
constexpr int kBufferConfig = 0x00020000;   // buffer descriptor word 3 for gfx9-family parts
constexpr int kNontemporal = 2;             // buffer load cache-policy bit: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, (int)bytes, kBufferConfig);
}

constexpr int kMfmaOS = 128 + 4;   // padded head stride of the LDS merge buffer
struct MfmaSmem {
  float o[kWaves][16][kMfmaOS];
  float m[kWaves][16], l[kWaves][16];
  int bad[kWaves];
  u32x4 kst[kWaves][256];   // per-wave staging of one K tile (16 tokens x 16 chunks of 16 B)
};

template <int B, int NBUF>
__device__ __forceinline__ void mfma_item(const AttnArgs &a, int s, int p, int kvh, int ctx_known, MfmaSmem &sm) {
  constexpr int D = 128;
  constexpr int OS = kMfmaOS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile addresses in SGPRs
  const int c16 = lane & 15, grp = lane >> 4;
  const int g = a.g;
  float (*sm_o)[16][OS] = sm.o;
  float (*sm_m)[16] = sm.m;
  float (*sm_l)[16] = sm.l;
  int *sm_bad = sm.bad;

  // This wave's tiles are tile_lo + wave + kWaves * i.  Their block-table entries are
  // fetched 64 at a time (one per lane; the first batch together with the context length,
  // bounded by the table row rather than the context) and read back with readlane.
  const int32_t *table = a.tables + (size_t)s * a.max_blocks;
  const int tile_lo = (p * a.P) >> 4;
  auto table_chunk = [&](int i0) -> int {
    const int tok = (tile_lo + wave + kWaves * (i0 + lane)) << 4;
    const int e = tok / B;
    return e < a.max_blocks ? table[e] : 0;
  };
  int tb = table_chunk(0);
  const int ctx = ctx_known >= 0 ? ctx_known : a.ctx[s];
  if (ctx < 1 || ctx > a.max_ctx) {
    if (p == 0) fill_group<uint16_t, D>(a, s, kvh * g, g, ctx < 1 ? 0.f : __builtin_nanf(""));
    return;
  }
  const int t0 = p * a.P;
  if (t0 >= ctx) return;
  const int t1 = min(t0 + a.P, ctx);
  const bool single = ctx <= a.P;
  const int tile_hi = (t1 + 15) >> 4;
  const int n_my = tile_hi - tile_lo > wave ? (tile_hi - tile_lo - wave + kWaves - 1) / kWaves : 0;

  // Q^T operand: head c16 of the group (zero columns past g).
  bf16x8 qop[4];
  {
    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + ((size_t)s * a.Hq + kvh * g + c16) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c16 < g) v = ld16(qrow + 32 * c + 8 * grp);
      qop[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m = kNegInf, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int bad = 0;

  const uint32_t tsb = (uint32_t)a.Hkv * D * 2;           // bytes between consecutive slots
  const uint32_t tile_bytes = 16 * tsb;
  const char *kbase = reinterpret_cast<const char *>(a.k) + (size_t)kvh * D * 2;
  const char *vbase = reinterpret_cast<const char *>(a.v) + (size_t)kvh * D * 2;
  const uint32_t row_voff = 4 * grp * tsb + 16 * c16;     // tokens 4grp + r, bytes 16 c16 (whole rows)
  u32x4 *kst = sm.kst[wave];

  // issue the loads of chunk-local tile i (a zero-range descriptor past the chunk)
  auto issue = [&](int c0, int i, int cn, u32x4 *kd, u32x4 *vd) {
    const bool live = i < cn;
    int phys = __builtin_amdgcn_readlane(tb, i & 63);
    if (live && (unsigned)phys >= (unsigned)a.N) {
      bad = 1;
      phys = 0;
    }
    const int tok0 = (tile_lo + wave + kWaves * (c0 + i)) << 4;
    const size_t off = ((size_t)phys * B + (tok0 % B)) * tsb;
    const uint32_t range = live ? tile_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase + off, range);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase + off, range);
    // K and V alike: instruction r reads whole 256-byte rows (tokens 4grp + r, 16 lanes
    // per row), streamed past the caches (non-temporal).
#pragma unroll
    for (int r = 0; r < 4; ++r) kd[r] = __builtin_amdgcn_raw_buffer_load_b128(rk, row_voff, r * tsb, kNontemporal);
#pragma unroll
    for (int r = 0; r < 4; ++r) vd[r] = __builtin_amdgcn_raw_buffer_load_b128(rv, row_voff, r * tsb, kNontemporal);
  };

  auto compute = [&](int i, u32x4 *kr, u32x4 *vr) {
    const int tok0 = (tile_lo + wave + kWaves * i) << 4;
    // K tile to the MFMA A layout through the wave's LDS staging: chunk j of token t sits at
    // t*16 + (j ^ t) (16-byte units), so both the row-wise writes (fixed token, 16 chunks)
    // and the operand reads (16 tokens, fixed chunk) hit 16 distinct slots of 64 banks.
    // Lane (c16, grp) then holds token c16, chunks 4c + grp = head dims 32c + 8grp .. +7.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * grp + r;
      kst[t * 16 + (c16 ^ t)] = kr[r];
    }
    u32x4 kop[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kop[c] = kst[c16 * 16 + ((4 * c + grp) ^ c16)];
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[c]), qop[c], sc, 0, 0, 0);

    // scores of tokens tok0 + 4grp + r for head c16; positions past the end are masked
    float sv[4], mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = tok0 + 4 * grp + r < t1;
      sv[r] = ok ? sc[r] * a.scale_log2 : kNegInf;
      if (!ok) vr[r] = (u32x4){0u, 0u, 0u, 0u};   // unread slots may hold anything
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = merge_weight(m, mnew);
    float pr[4], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = sv[r] == kNegInf ? 0.f : fast_exp2(sv[r] - mnew);
      ps += pr[r];
    }
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    }
    m = mnew;

    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
    const i16x4 pop = __builtin_bit_cast(i16x4, (uint32_t __attribute__((ext_vector_type(2)))){p01, p23});
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      uint32_t a01, a23;
      if (j & 1) {
        a01 = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
        a23 = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
      } else {
        a01 = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
        a23 = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
      }
      const i16x4 aop = __builtin_bit_cast(i16x4, (uint32_t __attribute__((ext_vector_type(2)))){a01, a23});
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop, acc[j], 0, 0, 0);
    }
  };

  // NBUF-deep ring of register buffers.  Pipeline step k issues tile k into buffer k % NBUF
  // and computes tile k - (NBUF - 1); the loop is unrolled by NBUF so buffer indices are
  // compile-time constants and every load sits inside the loop.  Issues past the chunk are
  // zero-range (no memory access), computes outside [0, cn) are skipped by a wave-uniform
  // branch, so the count of loads in flight is fixed and each wait covers one tile.
  for (int c0 = 0; c0 < n_my; c0 += 64) {
    if (c0 > 0) tb = table_chunk(c0);
    const int cn = min(64, n_my - c0);
    u32x4 kbuf[NBUF][4], vbuf[NBUF][4];
    for (int k0 = 0; k0 < cn + NBUF - 1; k0 += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int k = k0 + j;
        issue(c0, k, cn, kbuf[j], vbuf[j]);
        __builtin_amdgcn_sched_barrier(0);   // keep those loads ahead of this tile's wait
        const int kc = k - (NBUF - 1);
        if (kc >= 0 && kc < cn) compute(c0 + kc, kbuf[(j + 1) % NBUF], vbuf[(j + 1) % NBUF]);
      }
    }
  }

  float lh = lsum + __shfl_xor(lsum, 16);
  lh += __shfl_xor(lh, 32);
  if (grp == 0) {
    sm_m[wave][c16] = m;
    sm_l[wave][c16] = lh;
  }
  if (lane == 0) sm_bad[wave] = bad;
  {
    float *dst = &sm_o[wave][c16][32 * grp];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[8 * r + i] = acc[i][r];
    }
  }
  __syncthreads();
  finish_group<uint16_t, D, 16, OS>(a, s, kvh, p, single, sm_m, sm_l, sm_o, sm_bad);
}

template <int B, int NBUF>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(const AttnArgs a) {
  __shared__ MfmaSmem sm;
  __shared__ SchedSmem sc;
  extern __shared__ int sm_dyn[];
  run_items(a, sc, sm_dyn, [&](int s, int p, int kvh, int ctx) { mfma_item<B, NBUF>(a, s, p, kvh, ctx, sm); });
}

// ---------------------------------------------------------------------------
// Vector path.  T = float or uint16_t (bf16).  Each token row of a KV head is
// D*sizeof(T) bytes = LPT lanes x 16 bytes; a wave covers TPW = 64 / LPT rows at once.
// Lane l: row = l / LPT, column chunk cl = l % LPT -> elements cl*EPL .. +EPL-1.
// Every row keeps its own online-softmax state; rows and waves are merged at the end.
// The wave's unit of work is CH = max(B, TPW) consecutive tokens (STEPS row steps).
// ---------------------------------------------------------------------------
template <int G, int D>
struct VecSmem {
  float o[kWaves][G][D + 4];
  float m[kWaves][G], l[kWaves][G];
  int bad[kWaves];
};

template <typename T, int D, int G, int B>
__device__ __forceinline__ void vec_item(const AttnArgs &a, int s, int p, int kvh, int ctx_known, VecSmem<G, D> &sm) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int LPT = D / EPL;
  constexpr int TPW = 64 / LPT;
  constexpr int CH = B >= TPW ? B : TPW;
  constexpr int STEPS = CH / TPW;
  constexpr int OS = D + 4;
  constexpr bool kBF16 = sizeof(T) == 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile addresses in SGPRs
  const int row = lane / LPT, cl = lane % LPT;
  const int g = a.g;
  float (*sm_o)[G][OS] = sm.o;
  float (*sm_m)[G] = sm.m;
  float (*sm_l)[G] = sm.l;
  int *sm_bad = sm.bad;

  const int ctx = ctx_known >= 0 ? ctx_known : a.ctx[s];
  if (ctx < 1 || ctx > a.max_ctx) {
    if (p == 0) fill_group<T, D>(a, s, kvh * g, g, ctx < 1 ? 0.f : __builtin_nanf(""));
    return;
  }
  const int t0 = p * a.P;
  if (t0 >= ctx) return;
  const int t1 = min(t0 + a.P, ctx);
  const bool single = ctx <= a.P;

  // this lane's slice of every query head in the group
  u32x4 qraw[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    qraw[j] = (u32x4){0u, 0u, 0u, 0u};
    if (j < g) qraw[j] = ld16(reinterpret_cast<const T *>(a.q) + ((size_t)s * a.Hq + kvh * g + j) * D + cl * EPL);
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
  }
  int bad = 0;

  const int32_t *table = a.tables + (size_t)s * a.max_blocks;
  const size_t tok_stride = (size_t)a.Hkv * D;
  const T *kpool = reinterpret_cast<const T *>(a.k) + (size_t)kvh * D + cl * EPL;
  const T *vpool = reinterpret_cast<const T *>(a.v) + (size_t)kvh * D + cl * EPL;

  // This wave's units are u_lo + wave + kWaves * i, i = 0 .. n_my - 1.  With one block per
  // unit its table entries are fetched 64 at a time (one per lane) and read back with
  // readlane; the K/V loads of unit i + 1 are issued before unit i is computed.
  const int u_lo = t0 / CH, u_hi = (t1 + CH - 1) / CH;
  const int n_my = u_hi - u_lo > wave ? (u_hi - u_lo - wave + kWaves - 1) / kWaves : 0;
  auto table_chunk = [&](int i0) -> int {
    const int i = i0 + lane;
    return i < n_my ? table[u_lo + wave + kWaves * i] : 0;
  };
  int tb = 0;
  auto issue = [&](int i, u32x4 *kd, u32x4 *vd, bool *okd) {
    const int tokc = (u_lo + wave + kWaves * i) * CH;
    int uphys = 0;
    if constexpr (B >= TPW) {
      uphys = __builtin_amdgcn_readlane(tb, i & 63);
      if ((unsigned)uphys >= (unsigned)a.N) {
        bad = 1;
        uphys = 0;
      }
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int t = tokc + st * TPW + row;
      okd[st] = t >= t0 && t < t1;
      int phys = uphys;
      if constexpr (B < TPW) {
        // the unit spans several blocks: only positions in [t0, t1) consult the table
        phys = okd[st] ? table[t / B] : 0;
        if ((unsigned)phys >= (unsigned)a.N) {
          bad = 1;
          phys = 0;
        }
      }
      const size_t off = ((size_t)phys * B + (t % B)) * tok_stride;
      kd[st] = ld16_stream(kpool + off);
      vd[st] = ld16_stream(vpool + off);
    }
  };

  // Same pipeline as the MFMA kernel: units in pairs from two register buffers, every
  // issue unconditional, a phantom (fully masked) second unit for odd counts.
  auto compute = [&](u32x4 *kr, u32x4 *vr, const bool *ok_in, bool real) {
    bool ok[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) ok[st] = ok_in[st] && real;
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
      if (!ok[st]) vr[st] = (u32x4){0u, 0u, 0u, 0u};   // unread slots may hold anything
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (j >= g) break;
      float sc[STEPS];
      float mx = kNegInf;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        float part = 0.f;
        if constexpr (kBF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            part = fmaf(bf16_lo(kr[st][w]), bf16_lo(qraw[j][w]), part);
            part = fmaf(bf16_hi(kr[st][w]), bf16_hi(qraw[j][w]), part);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) part = fmaf(__uint_as_float(kr[st][w]), __uint_as_float(qraw[j][w]), part);
        }
        part = group_sum<LPT>(part);
        sc[st] = ok[st] ? part * a.scale_log2 : kNegInf;
        mx = fmaxf(mx, sc[st]);
      }
      const float mnew = fmaxf(m[j], mx);
      const float alpha = mnew == kNegInf ? 1.f : merge_weight(m[j], mnew);
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        sc[st] = sc[st] == kNegInf ? 0.f : fast_exp2(sc[st] - mnew);
        ps += sc[st];
      }
      l[j] = l[j] * alpha + ps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        if constexpr (kBF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o[j][2 * w] = fmaf(sc[st], bf16_lo(vr[st][w]), o[j][2 * w]);
            o[j][2 * w + 1] = fmaf(sc[st], bf16_hi(vr[st][w]), o[j][2 * w + 1]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) o[j][w] = fmaf(sc[st], __uint_as_float(vr[st][w]), o[j][w]);
        }
      }
      m[j] = mnew;
    }
  };

  for (int c0 = 0; c0 < n_my; c0 += 64) {
    if constexpr (B >= TPW) tb = table_chunk(c0);
    const int cn = min(64, n_my - c0);
    u32x4 ka[STEPS], va[STEPS], kb[STEPS], vb[STEPS];
    bool oka[STEPS], okb[STEPS];
    issue(c0, ka, va, oka);
    for (int ii = 0; ii < cn; ii += 2) {
      issue(c0 + min(ii + 1, cn - 1), kb, vb, okb);
      __builtin_amdgcn_sched_barrier(0);   // keep the next unit's loads ahead of this wait
      compute(ka, va, oka, true);
      issue(c0 + min(ii + 2, cn - 1), ka, va, oka);
      __builtin_amdgcn_sched_barrier(0);
      compute(kb, vb, okb, ii + 1 < cn);
    }
  }

  // merge the TPW rows of the wave (butterfly over the row bits of the lane id)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float m2 = __shfl_xor(m[j], off), l2 = __shfl_xor(l[j], off);
      const float M = fmaxf(m[j], m2);
      const float w1 = M == kNegInf ? 0.f : merge_weight(m[j], M);
      const float w2 = M == kNegInf ? 0.f : merge_weight(m2, M);
      l[j] = w1 * l[j] + w2 * l2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[j][e], off);
        o[j][e] = w1 * o[j][e] + w2 * o2;
      }
      m[j] = M;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][j][cl * EPL + e] = o[j][e];
      if (cl == 0) {
        sm_m[wave][j] = m[j];
        sm_l[wave][j] = l[j];
      }
    }
  }
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();
  finish_group<T, D, G, OS>(a, s, kvh, p, single, sm_m, sm_l, sm_o, sm_bad);
}

template <typename T, int D, int G, int B>
__global__ __launch_bounds__(kThreads) void attn_vec_kernel(const AttnArgs a) {
  __shared__ VecSmem<G, D> sm;
  __shared__ SchedSmem sc;
  extern __shared__ int sm_dyn[];
  run_items(a, sc, sm_dyn, [&](int s, int p, int kvh, int ctx) { vec_item<T, D, G, B>(a, s, p, kvh, ctx, sm); });
}

// ---------------------------------------------------------------------------
// Pass 2: merge the partials of one (sequence, head):
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
// The partition -> thread assignment and the reduction trees are fixed, so the result
// does not depend on timing.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, bool is_max, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_reduce_kernel(const AttnArgs a) {
  constexpr int CHK = D / 4;            // float4 chunks per row
  constexpr int PL = kThreads / CHK;    // partitions processed side by side
  extern __shared__ float sm_w[];       // [max_parts] merge weights
  __shared__ f32x4 sm_acc[kThreads];
  __shared__ float red[kWaves];
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  if (h == 0 && s == 0 && tid == 0) a.queue[0] = 0u;   // pass 1 is complete: reset its work queue
  const int ctx = a.ctx[s];
  if (ctx < 1 || ctx > a.max_ctx || ctx <= a.P) return;
  const int np = (ctx + a.P - 1) / a.P;
  const size_t base = ((size_t)s * a.Hq + h) * a.max_parts;

  float mx = kNegInf;
  for (int i = tid; i < np; i += kThreads) mx = fmaxf(mx, a.ws_m[base + i]);
  const float M = block_reduce(mx, true, red);
  float ls = 0.f;
  for (int i = tid; i < np; i += kThreads) {
    const float w = merge_weight(a.ws_m[base + i], M);
    sm_w[i] = w;
    ls += w * a.ws_l[base + i];
  }
  const float L = block_reduce(ls, false, red);   // its barriers also publish sm_w

  const int c = tid % CHK, pl = tid / CHK;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 *po = reinterpret_cast<const f32x4 *>(a.ws_o + base * D) + c;
#pragma unroll 4
  for (int i = pl; i < np; i += PL) acc += sm_w[i] * po[(size_t)i * CHK];
  sm_acc[tid] = acc;
  __syncthreads();
  if (pl == 0) {
#pragma unroll
    for (int q = 1; q < PL; ++q) acc += sm_acc[q * CHK + c];
    const size_t o = ((size_t)s * a.Hq + h) * D + 4 * c;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<T>(a.out, o + e, acc[e] / L);
  }
}

// Queue reset when no merge kernel follows pass 1.
__global__ void queue_reset_kernel(unsigned *queue) {
  if (threadIdx.x == 0) queue[0] = 0u;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int vec_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 0; }

static pkv_path select_path(int Hq, int Hkv, int D, int B, pkv_dtype dt) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return PKV_PATH_NONE;
  if (dt != PKV_DTYPE_F32 && dt != PKV_DTYPE_BF16) return PKV_PATH_NONE;
  if (D != 64 && D != 128) return PKV_PATH_NONE;
  if (B != 4 && B != 8 && B != 16 && B != 32) return PKV_PATH_NONE;
  const int g = Hq / Hkv;
  if (dt == PKV_DTYPE_BF16 && D == 128 && (B == 16 || B == 32) && g >= 2 && g <= 16) return PKV_PATH_MFMA;
  return vec_group(g) ? PKV_PATH_VECTOR : PKV_PATH_NONE;
}

typedef void (*Pass1Fn)(AttnArgs);

template <typename T, int D, int G>
static Pass1Fn vec_fn_b(int B) {
  switch (B) {
    case 4: return attn_vec_kernel<T, D, G, 4>;
    case 8: return attn_vec_kernel<T, D, G, 8>;
    case 16: return attn_vec_kernel<T, D, G, 16>;
    default: return attn_vec_kernel<T, D, G, 32>;
  }
}

template <typename T, int D>
static Pass1Fn vec_fn(int g, int B) {
  switch (vec_group(g)) {
    case 1: return vec_fn_b<T, D, 1>(B);
    case 2: return vec_fn_b<T, D, 2>(B);
    case 4: return vec_fn_b<T, D, 4>(B);
    default: return vec_fn_b<T, D, 8>(B);
  }
}

static Pass1Fn pass1_fn(pkv_path path, pkv_dtype dt, int D, int B, int g) {
  if (path == PKV_PATH_MFMA) return B == 16 ? attn_mfma_kernel<16, kMfmaDepth> : attn_mfma_kernel<32, kMfmaDepth>;
  if (dt == PKV_DTYPE_BF16) return D == 128 ? vec_fn<uint16_t, 128>(g, B) : vec_fn<uint16_t, 64>(g, B);
  return D == 128 ? vec_fn<float, 128>(g, B) : vec_fn<float, 64>(g, B);
}

// Workgroups of `fn` that fit on the current device at once.
static int resident_workgroups(Pass1Fn fn, size_t dyn_lds) {
  int dev = 0, cus = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(fn), kThreads, dyn_lds) !=
      hipSuccess)
    return 0;
  return (occ > 0 ? occ : 1) * cus;
}

template <typename T, int D>
static void launch_reduce(dim3 grid, hipStream_t st, const AttnArgs &a) {
  hipLaunchKernelGGL((attn_reduce_kernel<T, D>), grid, dim3(kThreads), (size_t)a.max_parts * sizeof(float), st, a);
}

static int64_t parts_for(int64_t max_ctx, int64_t P) { return (max_ctx + P - 1) / P; }

static bool aligned(const void *p, uintptr_t al) { return ((uintptr_t)p & (al - 1)) == 0; }

}  // namespace pkv

using namespace pkv;

extern "C" pkv_path pkv_attention_path(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, pkv_dtype dtype) {
  return select_path(num_heads, num_kv_heads, head_dim, block_size, dtype);
}

extern "C" size_t pkv_attention_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0)
    return kQueueBytes;
  const int64_t np = parts_for(max_context_len, partition_size);
  if (np <= 1) return kQueueBytes;
  return kQueueBytes + (size_t)num_seqs * num_heads * np * (head_dim + 2) * sizeof(float);
}

extern "C" pkv_status paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                                             const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, float scale,
                                             int32_t partition_size, void *workspace, size_t workspace_bytes,
                                             pkv_dtype dtype, void *stream) {
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || max_context_len < 1 || partition_size < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  const pkv_path path = select_path(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (path == PKV_PATH_NONE) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_INVALID_ARG;
  if (partition_size > 0 && partition_size % block_size != 0) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return PKV_ERR_INVALID_ARG;

  const int64_t P = partition_size > 0 ? partition_size : ((int64_t)max_context_len + 15) / 16 * 16;
  const int64_t np = parts_for(max_context_len, P);
  if (np > kMaxReduceParts) return PKV_ERR_UNSUPPORTED;
  const size_t need = pkv_attention_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return PKV_ERR_INVALID_ARG;

  AttnArgs a;
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.ctx = context_lens;
  const size_t nparts_total = (size_t)num_seqs * num_heads * (size_t)np;
  a.queue = reinterpret_cast<unsigned *>(workspace);
  a.ws_o = np > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kQueueBytes) : nullptr;
  a.ws_m = np > 1 ? a.ws_o + nparts_total * head_dim : nullptr;
  a.ws_l = np > 1 ? a.ws_m + nparts_total : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.Hq = num_heads;
  a.Hkv = num_kv_heads;
  a.g = num_heads / num_kv_heads;
  a.N = num_blocks;
  a.P = (int)P;
  a.max_parts = (int)np;
  a.scale_log2 = scale * kLog2e;
  a.S = num_seqs;

  hipStream_t st = (hipStream_t)stream;
  const int64_t items = np * num_kv_heads * (int64_t)num_seqs;   // upper bound: every partition non-empty
  if (items > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const bool bf16 = dtype == PKV_DTYPE_BF16;
  const Pass1Fn fn = pass1_fn(path, dtype, head_dim, block_size, a.g);
  // persistent workgroups when the schedule fits in LDS, else one workgroup per possible item
  size_t dyn_lds = 0;
  int64_t grid = items;
  a.persistent = 0;
  if (num_seqs <= kMaxSchedSeqs) {
    dyn_lds = 2 * (size_t)num_seqs * sizeof(int);
    const int resident = resident_workgroups(fn, dyn_lds);
    if (resident > 0) {
      a.persistent = 1;
      grid = items < resident ? items : resident;
    } else {
      dyn_lds = 0;
    }
  }
  void *args[] = {&a};
  if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid), dim3(kThreads), args, dyn_lds, st) !=
      hipSuccess)
    return PKV_ERR_HIP;
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (np <= 1 && a.persistent) {
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, st, a.queue);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  if (np > 1) {
    const dim3 rgrid((unsigned)num_heads, (unsigned)num_seqs);
    if (bf16) {
      if (head_dim == 128) launch_reduce<uint16_t, 128>(rgrid, st, a);
      else launch_reduce<uint16_t, 64>(rgrid, st, a);
    } else {
      if (head_dim == 128) launch_reduce<float, 128>(rgrid, st, a);
      else launch_reduce<float, 64>(rgrid, st, a);
    }
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}
