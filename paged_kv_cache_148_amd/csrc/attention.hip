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
// K/V byte is read once per group.  On the tile paths, where the sequences' blocks lie far
// apart in the pool, the bulk of a large launch goes out in wide items of 2 or 4 adjacent KV
// heads of one (sequence, partition): the workgroup's waves then read the same blocks at the
// same time (one address translation serves several waves, which cuts the translation misses
// of a pool scattered over gigabytes more than threefold), and each head's tiles are still
// accumulated and merged exactly as in a one-head item, so the width changes no bit of the
// result.  Without a partition size the partition is the whole
// context.  With one, an item leaves a partial state (running max m, sum l, unnormalised
// o) as one contiguous record in the workspace and a second kernel merges the partials by
// log-sum-exp;
// sequences whose context fits one partition are finished in pass 1.
//
// Scheduling: the pass-1 kernels are persistent.  As many workgroups as fit on the chip
// each build the same item order in LDS from context_lens (so only non-empty items exist):
// the vector kernel in sequence order, the MFMA kernel longest first.  Workgroups take
// their first items by index and the rest from a work-queue counter in the workspace until
// none are left; the last workgroup to finish returns the counters to zero.  A dynamic
// queue keeps every XCD busy until the end even though the XCDs do not run at identical
// speeds, and no launch slot is spent on empty partitions.  Batches too large to stage in
// LDS fall back to one workgroup per possible item.
//
// Two pass-1 kernels:
//   attn_tile_kernel  (bf16, D = 128, every block size, 1 <= g <= 16): each wave streams
//     16-token tiles of K and V rows.  With a group of g >= 2 query heads (a real
//     contraction) a K tile times the group's Q^T on v_mfma_f32_16x16x32_bf16 gives the
//     score tile; the probabilities stay in the MFMA result layout and feed
//     v_mfma_f32_16x16x16_bf16 against V^T for P.V, the head dimension permuted so that
//     each lane's V operand is one 16-byte row piece of 4 tokens regrouped in registers (no
//     LDS round trip for V).  With one query head per KV head, q.k and P.V are fp32 FMAs on
//     exactly widened row pieces, q.k summed over a 16-lane row by DPP.
//   attn_vec_kernel   (everything else: fp32, D = 64): one token
//     row per D*e/16 lanes, 16-byte loads along head_dim, q.k as fp32 FMAs on exactly
//     widened elements, row sums by DPP.
// Scores carry scale * log2(e) so every exponential is a hardware exp2.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <type_traits>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
// Tile path: tiles per wave in the load ring (NB - 1 ahead).  A wave's tiles of an item are
// rounded up to a multiple of NB with empty tiles, whose slots carry no bytes at the item's
// end; one tile ahead per wave already keeps the memory system saturated and wastes the
// fewest slots.  The deep ring hides an item's merge and partial-state stores behind more
// loads in flight, which pays when items are very short partitions (at most 256 tokens: 4 tiles
// per wave), whose lengths are also whole multiples of the ring.  At 512 tokens the shallow ring,
// with its items taken just in time (attn_tile_kernel), is the faster: long contexts 548.4 ->
// 540.5 us, gqa70b split at 512 305.5 -> 304.3 us, same box; at 256 the deep ring stays ahead on
// the GQA shapes (gqa70b 538.0 against 543.1 us, the fork workload 35.6 against 37.8 us).
constexpr int kTileDepthShallow = 2;
constexpr int kTileDepthDeep = 4;
constexpr int64_t kDeepRingMaxPartition = 256;
constexpr int kMaxReduceParts = 8192;    // partials per (sequence, head) a call may have
constexpr int kMaxSchedSeqs = 4096;     // sequences whose schedule fits in LDS (up to 3 x 16 KiB)
constexpr int kClasses = 16;            // length classes of the longest-first schedule
constexpr size_t kQueueBytes = 256;     // work-queue header at the start of the workspace
// Wide work items (tile paths, row layout): at least kWideMinItems of them per workgroup, and the
// queue's last kWideReserve one-head items per workgroup stay one head wide (the finer tail).
constexpr int kWideMinItems = 4;
constexpr int kWideReserve = 2;   // with items taken just in time 2 beat 0, 4 and 8 (mha7b, gqa70b)
// ... and only where the sampled consecutive blocks of the sequences lie this far apart (in one
// pool): on pools shuffled within windows of 2 MB one-head items were faster (by 3 us on the long
// contexts' 512-token partitions), within windows of 32 MB and beyond wide ones (by 1-4 us on the
// long contexts, gqa70b and mha7b at 32 MB, 11 us on the long contexts at 256 MB).
constexpr int64_t kWideFarBytes = 4ll << 20;

struct AttnArgs {
  void *out;
  const void *q;
  const void *k;
  const void *v;
  const int32_t *tables;
  const int32_t *ctx;
  float *ws_rec;     // [S, max_parts, Hkv] records of g * D + 32 floats, one per (sequence,
                     // partition, KV head): the group's unnormalised partial rows (head j at j * D),
                     // then a 128-byte line of (m, l) pairs (head j at 2j, 2j + 1; m in the log2
                     // domain; the rest of the line unused).
                     // The KV head is fastest, as in the queue's order of full partitions, so the
                     // records written at about the same time lie side by side.
  int max_blocks;    // table row length
  int max_ctx;       // host bound on ctx
  int Hq, Hkv, g, N;
  int P;             // partition length in tokens (whole context when not splitting)
  int max_parts;
  float scale_log2;  // scale * log2(e)
  int S;             // sequences
  unsigned *queue;   // [0]: items taken beyond the grid (zero between calls)
  int persistent;    // 1: persistent workgroups + work queue; 0: one workgroup per possible item
  float cls_scale;   // length classes of the longest-first schedule: kClasses / (min(P, max_ctx) + 1)
  const void *k_new; // [S, Hkv, D]: each sequence's new K row, stored at position ctx - 1 by the
  const void *v_new; //   item that attends to it (the fused write; null otherwise)
  int hpi;           // tile path: KV heads of a wide work item (1, 2 or 4)
  int reserve;       // tile path: the queue's last `reserve` one-head items are not widened
  int far_blocks;    // tile path: block-id distance of "far apart" blocks (0: wide items regardless)
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

// End of a persistent launch for one workgroup: the last one to finish returns the queue
// counters to zero for the next call.  Every workgroup's fetches from queue[0] have
// returned before it counts itself done in queue[1], so the reset follows all of them.
__device__ __forceinline__ void queue_done(unsigned *queue) {
  if (threadIdx.x == 0 && atomicAdd(&queue[1], 1u) == gridDim.x - 1) {
    atomicExch(&queue[0], 0u);
    atomicExch(&queue[1], 0u);
  }
}

// Common driver of the vector pass-1 kernel: persistent work-queue loop, or one item per
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
  queue_done(a.queue);
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
      float *rec = a.ws_rec + (((size_t)s * a.max_parts + p) * a.Hkv + kvh) * (size_t)(g * D + 32);
      rec[j * D + d] = o;
      if (d == 0) {
        rec[g * D + 2 * j] = M;
        rec[g * D + 2 * j + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile path: bf16, D = 128, any block size (4 .. 128), a group of 1 to 16 query heads.
//
// Lane l of a wave: c16 = l % 16, grp = l / 16.  Each tile load gives lane l bytes
// 16 c16 .. + 15 (head dims 8 c16 .. + 7) of the K and V rows of tile rows 4grp + r.
// One query head per KV head (VALU): lane l's 8 dims of row 4grp + r times the same 8 dims
//   of q, summed over the 16 lanes of the row by DPP; P.V adds p(row) times the lane's 8 dims
//   of the row's V piece, and the lane groups' sums are added at the merge.
// Groups of 2..16 query heads (MFMA):
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
// Streaming.  Each wave sees one flat stream of 16-token tiles: the tiles of its share of
// the current item, then those of the next item.  Loads run NB - 1 tiles ahead of the
// compute, across the item boundary, so the first tiles of the next item are already in
// flight while the current item's states are merged.  The next item's block-table entries
// and q slice are loaded into registers one item ahead.  Every item's loop is padded to a
// multiple of NB tiles (at least NB); padded and out-of-range tiles get a zero-range
// buffer descriptor, so their loads return zeros without a memory access and every path
// through the loop issues the same loads -- the compiler's wait counts then stay exact.
// ---------------------------------------------------------------------------
constexpr int kBufferConfig = 0x00020000;   // buffer descriptor word 3 for gfx9-family parts
constexpr int kNontemporal = 2;             // buffer load cache-policy bit: non-temporal
// Store cache policy SC1: the item outputs and partial states are written through to the
// memory side.  Stored the default way, the 28 MB of partials of a 512-token split (long
// contexts) cost 40 us against no stores at all; with SC1, 22 us (non-temporal: 30 us,
// both bits: 80 us).  Measured on the long-context and GQA workloads.
constexpr int kStoreSc1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferConfig);
}

constexpr int kTileOS = 128 + 4;   // padded head stride of the LDS merge buffer
struct TileSmem {
  // per-wave states of the item being merged; two sets, alternating between items, so one
  // barrier per item separates the writes of an item from the reads of the one before
  float o[2][kWaves][16][kTileOS];
  alignas(16) float m[2][16][kWaves];   // [head][wave]: one 16-byte read per head
  alignas(16) float l[2][16][kWaves];
  int bad[2][kWaves];
  u32x4 kst[kWaves][256];   // per-wave staging of one K tile (16 tokens x 16 chunks of 16 B)
  int nextw[2];             // item indices taken from the queue, two items ahead
};

// One work item as a wave sees it.  Every field is wave-uniform.
struct MItem {
  int s, p, kvh;   // kvh: this wave's KV head
  int kvh0, u;     // the item's first KV head; kvh = kvh0 + u
  int width;       // KV heads of the item (1, 2 or 4); kWaves / width waves per KV head
  int ph0, pst;    // this wave's first tile phase and the stride between its phases
  int b1, b2, b3;  // loop indices where this wave's 2nd, 3rd, 4th phase begins (kBig: none)
  int t0, t1;    // attended token range [t0, t1)
  int tile_lo;   // first 16-token tile of the partition
  int n_my;      // this wave's live tiles (loop indices i < n_my; tile_of)
  int n_pad;     // loop length: n_my rounded up to a multiple of NB, at least NB
  int fill;      // 0 attend; 1 write zeros; 2 write NaN; 3 nothing to do
  int single;    // the partition is the whole context: normalise into out
};

// Longest-first schedule of the MFMA kernel.  The queue hands out, first, every full
// partition (P tokens) of every sequence in sequence order, then the last -- or only --
// partition of each sequence, longest first: the lengths fall into kClasses classes of
// equal width and a stable counting sort orders the sequences by class.  The longest
// items start first and the last ones to finish are short, so the workgroups run out of
// work together.  Every workgroup builds the same order from context_lens (nothing in it
// depends on timing).
// LDS (dynamic): pref[S] (inclusive prefix of full-partition items), ctx[S], order[S].
struct LptSched {
  int total_full;   // items of the full partitions
  int total;        // all items (one KV head each)
  int nwide;        // the first nwide * hpi of them go out as nwide items of hpi KV heads each
  int items;        // queue entries: nwide + total - nwide * hpi
};

// Scratch of the schedule build: sequences go in chunks of 64 (one per lane).
constexpr int kMaxChunks = kMaxSchedSeqs / 64;
struct LptSmem {
  int cnt[kMaxChunks][kClasses];   // class counts per chunk, then their exclusive prefix over chunks
  int cfull[kMaxChunks];           // full-partition items per chunk, then their exclusive prefix
  int cstart[kClasses];            // first position of each class in the order
  int total_full;
};

// Length class of a last partition: 0 for the longest lengths.  cls_scale = kClasses /
// (longest possible last partition + 1), so the product stays below kClasses.
__device__ __forceinline__ int length_class(int len, float cls_scale) {
  return kClasses - 1 - min(kClasses - 1, (int)((float)len * cls_scale));
}

// Full-partition items and length class of sequence i (class kClasses: no sequence).
__device__ __forceinline__ void classify(const AttnArgs &a, int c, bool valid, int &nfull, int &cls) {
  const bool ok = c >= 1 && c <= a.max_ctx;
  const int np = ok ? (c + a.P - 1) / a.P : 1;
  nfull = valid ? (np - 1) * a.Hkv : 0;
  cls = valid ? length_class(ok ? c - (np - 1) * a.P : 0, a.cls_scale) : kClasses;
}

// Inclusive prefix sum over the 64 lanes of a wave: within each row of 16 lanes by DPP
// shifts (zeros shifted in), then the row totals carried forward by row broadcasts
// (lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The same schedule for at most 64 sequences: one wave holds every length in a lane and
// builds it in registers (class counts by ballot, the class starts by one scan), with a single
// barrier in all.
__device__ LptSched build_lpt_schedule_one_wave(const AttnArgs &a, int *sm_pref, int *sm_ctx, int *sm_order,
                                                LptSmem &ss) {
  const int S = a.S, lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const bool valid = lane < S;
    const int c = valid ? a.ctx[lane] : 0;
    int nfull, cls;
    classify(a, c, valid, nfull, cls);
    const int incl = wave_incl_scan(nfull);
    uint64_t mine = 0ull;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kClasses; ++k) {
      const uint64_t m = __ballot(cls == k);
      if (lane == k) cnt = __popcll(m);
      if (cls == k) mine = m;
    }
    const int cincl = wave_incl_scan(cnt);   // lanes 0 .. kClasses - 1: classes; others count 0
    const int start = __shfl(cincl - cnt, cls < kClasses ? cls : 0);
    if (valid) {
      sm_ctx[lane] = c;
      sm_pref[lane] = incl;
      sm_order[start + __popcll(mine & ((1ull << lane) - 1ull))] = lane;
    }
    if (lane == 63) ss.total_full = incl;
  }
  __syncthreads();
  LptSched r;
  r.total_full = min(max(ss.total_full, 0), S * a.Hkv * (a.max_parts - 1));
  r.total = r.total_full + S * a.Hkv;
  return r;
}

// The same schedule for 65 .. 256 sequences: wave w holds chunk w (sequences 64 w .. 64 w + 63)
// in registers, publishes its class counts and full-partition count, and after one barrier
// places its own sequences using the earlier chunks' counts; two barriers in all.
__device__ LptSched build_lpt_schedule_four_waves(const AttnArgs &a, int *sm_pref, int *sm_ctx, int *sm_order,
                                                  LptSmem &ss) {
  const int S = a.S, lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int Q = (S + 63) >> 6;
  const int i = 64 * q + lane;
  const bool valid = i < S;
  const int c = valid ? a.ctx[i] : 0;
  int nfull = 0, cls = kClasses, incl = 0, cnt = 0;
  uint64_t mine = 0ull;
  if (q < Q) {
    classify(a, c, valid, nfull, cls);
    incl = wave_incl_scan(nfull);
#pragma unroll
    for (int k = 0; k < kClasses; ++k) {
      const uint64_t m = __ballot(cls == k);
      if (lane == k) cnt = __popcll(m);
      if (cls == k) mine = m;
    }
    if (lane < kClasses) ss.cnt[q][lane] = cnt;
    if (lane == 63) ss.cfull[q] = incl;
    if (valid) sm_ctx[i] = c;
  }
  __syncthreads();
  int total_full = 0, full_before = 0;
  for (int p = 0; p < Q; ++p) {
    const int f = ss.cfull[p];
    total_full += f;
    if (p < q) full_before += f;
  }
  if (q < Q) {
    // lane k: sequences of class k in the earlier chunks, and in all chunks
    int before = 0, tot = 0;
    if (lane < kClasses) {
      for (int p = 0; p < Q; ++p) {
        const int v = ss.cnt[p][lane];
        tot += v;
        if (p < q) before += v;
      }
    }
    const int cincl = wave_incl_scan(tot);
    const int start = __shfl(cincl - tot + before, cls < kClasses ? cls : 0);
    if (valid) {
      sm_pref[i] = incl + full_before;
      sm_order[start + __popcll(mine & ((1ull << lane) - 1ull))] = i;
    }
  }
  __syncthreads();
  LptSched r;
  r.total_full = min(max(total_full, 0), S * a.Hkv * (a.max_parts - 1));
  r.total = r.total_full + S * a.Hkv;
  return r;
}

// Builds the schedule; ends with a barrier.
__device__ LptSched build_lpt_schedule(const AttnArgs &a, int *sm_pref, int *sm_ctx, int *sm_order, LptSmem &ss) {
  const int S = a.S, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (S <= 64) return build_lpt_schedule_one_wave(a, sm_pref, sm_ctx, sm_order, ss);
  if (S <= 64 * kWaves) return build_lpt_schedule_four_waves(a, sm_pref, sm_ctx, sm_order, ss);
  const int Q = (S + 63) >> 6;
  constexpr int kPer = kMaxSchedSeqs / kThreads;
  {
    int cv[kPer];   // every length in flight at once
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + r * kThreads;
      cv[r] = i < S ? a.ctx[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tid + r * kThreads;
      if (i < S) sm_ctx[i] = cv[r];
    }
  }
  __syncthreads();

  // per chunk: in-chunk prefix of the full-partition items, and the class counts
  const uint64_t below = (1ull << lane) - 1ull;
  for (int q = wv; q < Q; q += kWaves) {
    const int i = 64 * q + lane;
    const bool valid = i < S;
    int nfull, cls;
    classify(a, valid ? sm_ctx[i] : 0, valid, nfull, cls);
    const int incl = wave_incl_scan(nfull);
    if (valid) sm_pref[i] = incl;
    if (lane == 63) ss.cfull[q] = incl;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kClasses; ++k) {
      const uint64_t m = __ballot(cls == k);
      if (lane == k) cnt = __popcll(m);
    }
    if (lane < kClasses) ss.cnt[q][lane] = cnt;
  }
  __syncthreads();

  // wave 0: exclusive prefixes over the chunks (lane k: class k; lane kClasses: full
  // partitions) and the first position of each class
  if (wv == 0) {
    int run = 0;
    if (lane < kClasses) {
      for (int q = 0; q < Q; ++q) {
        const int v = ss.cnt[q][lane];
        ss.cnt[q][lane] = run;
        run += v;
      }
    } else if (lane == kClasses) {
      for (int q = 0; q < Q; ++q) {
        const int v = ss.cfull[q];
        ss.cfull[q] = run;
        run += v;
      }
      ss.total_full = run;
    }
    const int tot = lane < kClasses ? run : 0;
    const int incl = wave_incl_scan(tot);
    if (lane < kClasses) ss.cstart[lane] = incl - tot;
  }
  __syncthreads();

  // per chunk: each sequence's place -- its class's start, the earlier chunks' sequences
  // of that class, then the earlier lanes' of this chunk (a stable order)
  for (int q = wv; q < Q; q += kWaves) {
    const int i = 64 * q + lane;
    const bool valid = i < S;
    int nfull, cls;
    classify(a, valid ? sm_ctx[i] : 0, valid, nfull, cls);
    uint64_t mine = 0ull;
#pragma unroll
    for (int k = 0; k < kClasses; ++k) {
      const uint64_t m = __ballot(cls == k);
      if (cls == k) mine = m;
    }
    if (valid) {
      sm_pref[i] += ss.cfull[q];
      sm_order[ss.cstart[cls] + ss.cnt[q][cls] + __popcll(mine & below)] = i;
    }
  }
  __syncthreads();
  LptSched r;
  // at most max_parts - 1 full partitions per (sequence, KV head): whatever LDS holds, the
  // item loop stays bounded
  r.total_full = min(max(ss.total_full, 0), S * a.Hkv * (a.max_parts - 1));
  r.total = r.total_full + S * a.Hkv;
  return r;
}

// Item w of the longest-first order -> (sequence, partition, KV head), KV head fastest.
__device__ __forceinline__ WorkItem decode_lpt(int w, const LptSched &sc, const int *sm_pref, const int *sm_ctx,
                                               const int *sm_order, const AttnArgs &a) {
  WorkItem it;
  if (w < sc.total_full) {
    int lo = 0, hi = a.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sm_pref[mid] > w) hi = mid; else lo = mid + 1;
    }
    const int r = w - (lo ? sm_pref[lo - 1] : 0);
    it.s = lo;
    it.kvh = r % a.Hkv;
    it.p = r / a.Hkv;
  } else {
    const int r = w - sc.total_full;
    it.s = min(max(sm_order[r / a.Hkv], 0), a.S - 1);   // in range whatever LDS holds
    it.kvh = r % a.Hkv;
    const int c = sm_ctx[it.s];
    it.p = (c >= 1 && c <= a.max_ctx) ? (c - 1) / a.P : 0;
  }
  return it;
}

constexpr int kBig = 1 << 30;   // "no such phase": past every loop index

// Tile phases: phase q of an item is its tiles q, q + 4, q + 8, ...  A one-head item gives wave w
// phase w.  A wide item (width 2 or 4 KV heads) gives each KV head kWaves / width waves, and
// each of them several phases, one after the other: wave (u, ph0) streams phases ph0,
// ph0 + pst, ... of KV head kvh0 + u, storing its state at each phase's end.  Every phase of
// every head is then accumulated exactly as in a one-head item and the merge is the same, so
// the width changes no bit of the result; it puts the waves of a workgroup on the same
// blocks at the same time.
template <int NB>
__device__ __forceinline__ MItem make_item(const AttnArgs &a, int s, int p, int kvh, int ctx, int wave,
                                           int width) {
  MItem it;
  const int lw = __builtin_ctz((unsigned)width);   // width 1, 2 or 4: shifts, not divisions
  const int wph = kWaves >> lw;
  it.s = s;
  it.p = p;
  it.kvh0 = kvh;
  it.u = (int)((unsigned)(wave * width) / kWaves);
  it.kvh = kvh + it.u;
  it.width = width;
  it.ph0 = wave & (wph - 1);
  it.pst = wph;
  it.tile_lo = (p * a.P) >> 4;
  it.t0 = p * a.P;
  it.t1 = 0;
  it.n_my = 0;
  it.single = 0;
  int nt = 0;
  if (ctx < 1 || ctx > a.max_ctx) {
    it.fill = p == 0 ? (ctx < 1 ? 1 : 2) : 3;
  } else if (p * a.P >= ctx) {
    it.fill = 3;
  } else {
    it.fill = 0;
    it.t1 = min(p * a.P + a.P, ctx);
    it.single = ctx <= a.P;
    nt = ((it.t1 + 15) >> 4) - it.tile_lo;
  }
  // tiles of phase q: nt > q ? (nt - q + 3) / 4 : 0
  int c[kWaves];
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const int q = it.ph0 + k * wph;
    c[k] = k < width && nt > q ? (nt - q + kWaves - 1) / kWaves : 0;
  }
  it.b1 = width > 1 ? c[0] : kBig;
  it.b2 = width > 2 ? c[0] + c[1] : kBig;
  it.b3 = width > 3 ? c[0] + c[1] + c[2] : kBig;
  it.n_my = c[0] + c[1] + c[2] + c[3];
  it.n_pad = max(NB, (it.n_my + NB - 1) / NB * NB);
  return it;
}

// Tile (index within the sequence) of this wave's loop index i.
template <bool WIDE>
__device__ __forceinline__ int tile_of(const MItem &it, int i) {
  if constexpr (!WIDE) return it.tile_lo + it.ph0 + kWaves * i;
  // b1 <= b2 <= b3: the phase of index i began at the largest of them not above i (selects and
  // maxima, not a branch per phase)
  const bool k1 = i >= it.b1, k2 = i >= it.b2, k3 = i >= it.b3;
  const int start = max(max(k1 ? it.b1 : 0, k2 ? it.b2 : 0), k3 ? it.b3 : 0);
  return it.tile_lo + it.ph0 + ((int)k1 + (int)k2 + (int)k3) * it.pst + kWaves * (i - start);
}

// Blocks that one 16-token tile spans: 16 / B for blocks of 4 or 8 slots, else 1.
template <int B>
constexpr int tile_blocks() { return B < 16 ? 16 / B : 1; }

// Block-table entries of tiles 64c .. 64c + 63 of an item, one per lane: entry h of each
// tile's blocks (zero past the table row or for an item with nothing to attend).
template <int B, bool WIDE>
__device__ __forceinline__ int table_chunk(const AttnArgs &a, const MItem &it, int c, int h, int lane) {
  const bool live = it.fill == 0 && 64 * c < it.n_my;
  const __amdgpu_buffer_rsrc_t r =
      buf_rsrc(a.tables + (size_t)it.s * a.max_blocks, live ? (uint32_t)a.max_blocks * 4u : 0u);
  const int tok = tile_of<WIDE>(it, 64 * c + lane) << 4;
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (tok / B + h) * 4, 0, 0);
}
template <int B, bool WIDE>
__device__ __forceinline__ void table_chunks(const AttnArgs &a, const MItem &it, int c, int lane, int *tb) {
#pragma unroll
  for (int h = 0; h < tile_blocks<B>(); ++h) tb[h] = table_chunk<B, WIDE>(a, it, c, h, lane);
}

// The Q^T operand of an item: head c16 of the KV head's group (zero columns past g).
__device__ __forceinline__ void load_q(const AttnArgs &a, const MItem &it, int c16, int grp, u32x4 *qd) {
  constexpr int D = 128;
  const bool live = it.fill == 0;
  const __amdgpu_buffer_rsrc_t r =
      buf_rsrc(reinterpret_cast<const uint16_t *>(a.q) + ((size_t)it.s * a.Hq + (size_t)it.kvh * a.g) * D,
               live ? (uint32_t)(a.g * D * 2) : 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) qd[c] = __builtin_amdgcn_raw_buffer_load_b128(r, (c16 * D + 32 * c + 8 * grp) * 2, 0, 0);
}

// The q row piece of the VALU path (one query head per KV head): lane (c16, grp) takes head
// dims 8 c16 .. 8 c16 + 7, the same piece for every grp.
__device__ __forceinline__ void load_q_row(const AttnArgs &a, const MItem &it, int c16, u32x4 *qd) {
  constexpr int D = 128;
  const __amdgpu_buffer_rsrc_t r =
      buf_rsrc(reinterpret_cast<const uint16_t *>(a.q) + ((size_t)it.s * a.Hq + it.kvh) * D,
               it.fill == 0 ? (uint32_t)(D * 2) : 0u);
  qd[0] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * c16, 0, 0);
}

// Item index -> item.  Persistent launch: from the LDS schedule; otherwise one item per
// workgroup in the fixed grid order, with the length read from memory.
// Item fields come from LDS and memory (vector registers); they are the same in every lane.
__device__ __forceinline__ MItem uniform(MItem it) {
  it.s = __builtin_amdgcn_readfirstlane(it.s);
  it.p = __builtin_amdgcn_readfirstlane(it.p);
  it.kvh = __builtin_amdgcn_readfirstlane(it.kvh);
  it.kvh0 = __builtin_amdgcn_readfirstlane(it.kvh0);
  it.u = __builtin_amdgcn_readfirstlane(it.u);
  it.width = __builtin_amdgcn_readfirstlane(it.width);
  it.ph0 = __builtin_amdgcn_readfirstlane(it.ph0);
  it.pst = __builtin_amdgcn_readfirstlane(it.pst);
  it.b1 = __builtin_amdgcn_readfirstlane(it.b1);
  it.b2 = __builtin_amdgcn_readfirstlane(it.b2);
  it.b3 = __builtin_amdgcn_readfirstlane(it.b3);
  it.t0 = __builtin_amdgcn_readfirstlane(it.t0);
  it.t1 = __builtin_amdgcn_readfirstlane(it.t1);
  it.tile_lo = __builtin_amdgcn_readfirstlane(it.tile_lo);
  it.n_my = __builtin_amdgcn_readfirstlane(it.n_my);
  it.n_pad = __builtin_amdgcn_readfirstlane(it.n_pad);
  it.fill = __builtin_amdgcn_readfirstlane(it.fill);
  it.single = __builtin_amdgcn_readfirstlane(it.single);
  return it;
}

template <int NB, bool WIDE>
__device__ __forceinline__ MItem item_at(const AttnArgs &a, int w, const LptSched &sc, const int *sm_pref,
                                         const int *sm_ctx, const int *sm_order, int wave) {
  // one make_item on every path (the item's fields stay in registers)
  int s = 0, p = 0, kvh = 0, ctx = 1, width = 1;
  const bool none = w >= sc.items;
  if (!none) {
    if (a.persistent) {
      const bool wide = w < sc.nwide;
      const int r = wide ? w * a.hpi : sc.nwide * a.hpi + (w - sc.nwide);
      const WorkItem wi = decode_lpt(r, sc, sm_pref, sm_ctx, sm_order, a);
      s = wi.s;
      p = wi.p;
      kvh = wi.kvh;
      ctx = sm_ctx[wi.s];
      width = WIDE && wide ? a.hpi : 1;
    } else {
      kvh = w % a.Hkv;
      p = (w / a.Hkv) % a.max_parts;
      s = w / (a.Hkv * a.max_parts);
      ctx = a.ctx[s];
    }
  }
  MItem it = make_item<NB>(a, s, p, kvh, ctx, wave, width);
  if (none) {   // what the stream holds past the workgroup's last item
    it.fill = 3;
    it.t1 = 0;
    it.n_my = 0;
    it.n_pad = 0;
    it.single = 0;
  }
  return uniform(it);
}

// Merge of the four phase states of each head of an item, then its output (normalised, or a
// partial state for the second pass).  Thread t covers row t / 16 of the item's query heads
// (the KV heads' groups one after the other).  It reads head dims 8l .. 8l + 7 (l = t % 16) of
// each wave's state: ten independent LDS reads, one wait, and no bank conflicts with the padded
// row stride (whereas 4 dims per lane, 16 bytes apart, left every read 2-way conflicted).  The
// merged values are then regrouped across the row's 16 lanes so that thread t holds dims
// 4l .. 4l + 3 and 64 + 4l .. + 3: each store instruction then writes whole 256-byte runs of a
// head's row (16 lanes, consecutive 16-byte pieces), so every line of the write-through partial
// states is written at once (with each lane's 8 consecutive dims an instruction left every
// 32-byte sector half written, and the memory side counted twice the records' bytes).
__device__ __forceinline__ void tile_finish(const AttnArgs &a, const MItem &it, const float (*sm_m)[kWaves],
                                            const float (*sm_l)[kWaves], const float (*sm_o)[16][kTileOS],
                                            const int *sm_bad) {
  constexpr int D = 128;
  const int t = threadIdx.x, lane = t & 63, j = t >> 4, l = t & 15, e0 = 8 * l;
  const int d0 = 4 * l, d1 = 64 + d0;   // the dims this thread stores
  // row j: query head j of the item's heads (head jj of KV head kvh0 + u)
  const int u = j / a.g, jj = j - u * a.g;
  const bool act = u < it.width;   // rows past the item's heads: their LDS rows are read, not used
  const f32x4 m4 = *reinterpret_cast<const f32x4 *>(sm_m[j]);
  const f32x4 l4 = *reinterpret_cast<const f32x4 *>(sm_l[j]);
  f32x4 oa[kWaves], ob[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    oa[w] = *reinterpret_cast<const f32x4 *>(&sm_o[w][j][e0]);
    ob[w] = *reinterpret_cast<const f32x4 *>(&sm_o[w][j][e0 + 4]);
  }
  const bool bad = sm_bad[0] | sm_bad[1] | sm_bad[2] | sm_bad[3];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m4[w]);
  float L = 0.f;
  f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};   // dims 8l .. 8l + 3, 8l + 4 .. 8l + 7
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float wt = merge_weight(m4[w], M);
    L += wt * l4[w];
    va += wt * oa[w];
    vb += wt * ob[w];
  }
  if (bad) {
    M = 0.f;
    L = __builtin_nanf("");
    va = vb = (f32x4){L, L, L, L};
  }
  // dims 4l .. 4l + 3 are lane l / 2's va (l even) or vb (l odd); dims 64 + 4l .. + 3 are lane
  // 8 + l / 2's, the same way (lanes of this row: the 16 of this thread's group in the wave)
  const int src_lo = (lane & 48) | (l >> 1), src_hi = (lane & 48) | (8 + (l >> 1));
  const bool odd = l & 1;
  f32x4 lo, hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = __shfl(va[e], src_lo), x1 = __shfl(vb[e], src_lo);
    const float y0 = __shfl(va[e], src_hi), y1 = __shfl(vb[e], src_hi);
    lo[e] = odd ? x1 : x0;
    hi[e] = odd ? y1 : y0;
  }
  // the item's first head h0: every store below goes through one wave-uniform descriptor
  // based there, with a 32-bit per-lane offset (the item's KV heads are adjacent)
  const size_t h0 = (size_t)it.s * a.Hq + (size_t)it.kvh0 * a.g;
  if (it.single) {
    if (act) {
      const u32x2 vlo = {pack_bf16x2(lo[0] / L, lo[1] / L), pack_bf16x2(lo[2] / L, lo[3] / L)};
      const u32x2 vhi = {pack_bf16x2(hi[0] / L, hi[1] / L), pack_bf16x2(hi[2] / L, hi[3] / L)};
      const __amdgpu_buffer_rsrc_t ro =
          buf_rsrc(reinterpret_cast<uint16_t *>(a.out) + h0 * D, (uint32_t)(it.width * a.g * D * 2));
      __builtin_amdgcn_raw_buffer_store_b64(vlo, ro, (uint32_t)((j * D + d0) * 2), 0, kStoreSc1);
      __builtin_amdgcn_raw_buffer_store_b64(vhi, ro, (uint32_t)((j * D + d1) * 2), 0, kStoreSc1);
    }
  } else {
    // the item's record, one contiguous piece: the group's partial rows (head j at j * D), then
    // its (m, l) line (zeros past the group).  Stored as one piece, next to the records of the
    // items the queue hands out at about the same time, rather than g rows a partition-stride
    // apart, the 28 MB of partials of the long contexts' 512-token split cost 10 us less amid
    // the K/V stream (fewer DRAM pages written).
    const size_t item = ((size_t)it.s * a.max_parts + it.p) * a.Hkv + it.kvh0;
    const uint32_t rec_bytes = (uint32_t)(a.g * D + 32) * 4;
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.ws_rec + item * (size_t)(a.g * D + 32), it.width * rec_bytes);
    const uint32_t rec = (uint32_t)u * rec_bytes;   // the record of KV head kvh0 + u
    if (act) {
      const uint32_t off = rec + (uint32_t)(jj * D) * 4;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), ro, off + d0 * 4, 0, kStoreSc1);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), ro, off + d1 * 4, 0, kStoreSc1);
      if ((t & 15) == 0) {   // the head's (m, l) pair
        const u32x2 v = {__builtin_bit_cast(uint32_t, M), __builtin_bit_cast(uint32_t, L)};
        __builtin_amdgcn_raw_buffer_store_b64(v, ro, rec + (uint32_t)(a.g * D + 2 * jj) * 4, 0, kStoreSc1);
      }
    }
  }
}

// HM: the head-major cache layout (K [N, Hkv, D/8, B, 8], V [N, Hkv, D, B]; page
// "PagedAttention", PidokuInfra topic 10, section 5 "The layout, more precisely").  One
// (block, KV head) is then a contiguous 4 KB (B = 16) of K and of V.  Lane (c16, grp) reads
// K chunk 4c + grp of token c16 straight into the QK A operand (instruction c: 16 tokens x
// 4 chunks, 1 KB contiguous at B = 16) and, for P.V MFMA i, the 4 tokens 4grp .. of head dim
// 16i + c16 (8 bytes; instruction i: 16 dims x 16 tokens, 512 B contiguous at B = 16) straight
// into its A operand: no LDS staging and no byte permutes.  The accumulator of MFMA i then
// holds dims 16i + 4grp + r.  Blocks of 16 slots or more.
// MF: q.K and P.V as MFMA tiles with the query-head group as the B operand (groups of 2 to 16
// heads, a real contraction).  !MF: one query head per KV head -- the tiles' K and V row pieces
// meet q and P in fp32 FMAs on exactly widened elements, and q.k is summed over a 16-lane row
// by DPP (an MFMA would leave 15 of its 16 columns empty).
// FUSE: the fused write of each sequence's new token (row layout only; see load_item_new).
template <int B, int NB, bool HM, bool MF, bool FUSE = false, bool WIDE = false>
__global__ __launch_bounds__(kThreads) void attn_tile_kernel(const AttnArgs a) {
  static_assert(!WIDE || (!HM && B >= 16), "wide items: row layout, blocks of 16 slots or more");
  static_assert(!HM || B >= 16, "the head-major path takes blocks of 16 slots or more");
  static_assert(!FUSE || !HM, "the fused write is built for the row layout");
  static_assert(NB >= 2, "the ring holds the tile being computed and at least one ahead");
  constexpr int D = 128;
  // How the workgroup takes its items from the queue.  With the shallow ring (items of more than
  // 256 tokens, or unsplit) it takes the next item only when the current one ends: nothing is held
  // while a slower workgroup could still start it, which shortens the launch's tail (mha7b:
  // 219 -> 211.5 us, gqa70b: 276 -> 273 us, same box), at the price of the next item's table and
  // q loads at each boundary.  With the deep ring (partitions of at most 256 tokens: many short
  // items, where those boundaries would cost more than the tail saves) it takes item k + 2 while
  // item k runs, so that the next item's table chunks, q and first tiles are in flight across
  // the boundary.
  constexpr bool kLate = NB < kTileDepthDeep;
  __shared__ TileSmem sm;
  __shared__ LptSmem sched_sm;
  extern __shared__ int sm_dyn[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile addresses in SGPRs
  const int c16 = lane & 15, grp = lane >> 4;
  int *sm_pref = sm_dyn, *sm_ctx = sm_dyn + a.S, *sm_order = sm_dyn + 2 * a.S;

  // The workgroup's items: it_0 = blockIdx.x (with the deep ring also it_1 = gridDim.x +
  // blockIdx.x: the longest items, so a fixed split costs little balance, and the launch makes
  // no queue fetch), then one index per queue fetch, counted from gridDim.x (kLate) or from
  // 2 * gridDim.x.  kLate: the fetch for it_{k+1} is made as it_k ends.  Otherwise the fetch for
  // it_{k+2} is made while it_k runs, so both the current and the next item are always known.
  // Wide items pay where the sequences' blocks lie far apart (a pool scattered over tens of MB
  // or more: address translation then weighs on the stream); on a pool whose consecutive blocks
  // lie close together one-head items stream faster.  Each wave samples 64 pairs of consecutive table
  // entries (lane l: entries l / S and l / S + 1 of sequence l % S), loaded with the lengths
  // before the schedule build, and the launch goes wide where most sampled pairs of blocks
  // that a sequence uses lie at least far_blocks apart (every workgroup sees the same bits).
  int smp_ctx = 0, smp_t0 = 0, smp_t1 = 0;
  const int smp_s = lane % a.S, smp_j = lane / a.S;
  const bool smp_in = smp_j + 1 < a.max_blocks;
  if constexpr (WIDE) {
    if (a.far_blocks > 0) {
      // (per-lane addresses: plain loads; a buffer descriptor's base must be the same in every lane)
      const int32_t *row = a.tables + (size_t)smp_s * a.max_blocks;
      if (smp_in) {
        smp_t0 = row[smp_j];
        smp_t1 = row[smp_j + 1];
      }
      smp_ctx = a.ctx[smp_s];
    }
  }
  LptSched sched;
  if (a.persistent) {
    sched = build_lpt_schedule(a, sm_pref, sm_ctx, sm_order, sched_sm);   // ends with a barrier
  } else {
    sched.total_full = 0;
    sched.total = (int)gridDim.x;
  }
  bool go_wide = WIDE && a.persistent && a.hpi > 1;
  if constexpr (WIDE) {
    if (a.far_blocks > 0) {
      const bool valid = smp_in && smp_ctx <= a.max_ctx && smp_ctx > (smp_j + 1) * B;
      const int64_t gap = (int64_t)smp_t1 - (int64_t)smp_t0;
      const bool far = valid && (gap >= a.far_blocks || gap <= -(int64_t)a.far_blocks);
      go_wide = go_wide && 2 * __popcll(__ballot(far)) > __popcll(__ballot(valid));
    }
  }
  // the queue's bulk goes out in wide items, its last `reserve` one-head items as they are
  sched.nwide = go_wide ? max(0, sched.total - a.reserve) / a.hpi : 0;
  sched.items = sched.nwide + sched.total - sched.nwide * a.hpi;
  const int total = sched.items;
  // The item loop, built twice in the wide-item kernel: a launch that hands out no wide items (a
  // pool whose blocks lie close together) runs the one-head loop, whose phase bookkeeping is
  // shorter, and so streams as the one-head kernel does; the outputs are the same bits either way.
  auto run_items = [&](auto wide_c) {
    constexpr bool WI = decltype(wide_c)::value;
    int w = (int)blockIdx.x;
    int wn = a.persistent && !kLate ? (int)(gridDim.x + blockIdx.x) : total;
    if (w < total) {
      MItem cur = item_at<NB, WI>(a, w, sched, sm_pref, sm_ctx, sm_order, wave);
      MItem nxt;

      // Token of a tile row.  Load instruction r gives lane group grp the tile token
      //   tok(grp, r) = blk * B + (4 / BPT) * grp + r % (4 / BPT),   blk = r / (4 / BPT),
      // BPT = blocks per tile: with blocks of 16 or more it is 4grp + r; with smaller blocks
      // every instruction stays inside one block (blk), so one buffer descriptor serves it.
      // The MFMA row of that token is 4grp + r throughout (K staging, scores, P, V alike), so
      // the only effect is the order of the tile's tokens in the P.V sum.
      constexpr int BPT = tile_blocks<B>();
      constexpr int RPI = 4 / BPT;   // consecutive load instructions per block
      const uint32_t tsb = (uint32_t)a.Hkv * D * 2;   // bytes between consecutive slots
      const uint32_t blk_bytes = (BPT == 1 ? 16 : B) * tsb;   // range of one descriptor
      const char *kpool = reinterpret_cast<const char *>(a.k);
      const char *vpool = reinterpret_cast<const char *>(a.v);
      const uint32_t row_voff = RPI * grp * tsb + 16 * c16;   // whole 256-byte rows, bytes 16 c16
      u32x4 *kst = sm.kst[wave];

      // registers of the stream: table chunks (current item: the chunk being issued and the
      // one after it; next item: its first two; one register per block of a tile), q operands,
      // validity flags
      int tb_cur[BPT], tb_ahead[BPT], tb_next[BPT], tb_next_ahead[BPT];
      table_chunks<B, WI>(a, cur, 0, lane, tb_cur);
      table_chunks<B, WI>(a, cur, 1, lane, tb_ahead);
      // q operands: MF, head c16 of the group in the B layout; !MF on the head-major layout, the
      // item's head at the K chunks lane group grp holds (dims 32c + 8grp); !MF on the row
      // layout, dims 8 c16 .. + 7
      auto load_item_q = [&](const MItem &it, u32x4 *qd) {
        if constexpr (MF) load_q(a, it, c16, grp, qd);
        else if constexpr (HM) load_q(a, it, 0, grp, qd);
        else load_q_row(a, it, c16, qd);
      };
      u32x4 qop[4], qnext[4];
      load_item_q(cur, qop);
      int bad_cur = 0, bad_next = 0;

      // The fused write.  The item whose partition holds a sequence's new token (position
      // ctx - 1) stores that token's K and V rows of its KV head, from k_new and v_new, into the
      // token's slot, and the wave whose tile holds the token puts the same bytes in place of the
      // (stale) row it loaded before using it: the row is used from registers, so nothing waits
      // on the store.  Lane (c16, grp) holds bytes 16 c16 .. 16 c16 + 15 of its rows, so each lane
      // loads that piece of the new rows, with the item's q.
      u32x4 kn_cur = {0u, 0u, 0u, 0u}, vn_cur = kn_cur, kn_nxt = kn_cur, vn_nxt = kn_cur;
      // the item's partition holds the context's last token
      auto is_last = [&](const MItem &it) -> bool {
        const int c = a.persistent ? sm_ctx[it.s] : a.ctx[it.s];
        return it.fill == 0 && it.t1 == __builtin_amdgcn_readfirstlane(c);
      };
      auto load_item_new = [&](const MItem &it, u32x4 &kn, u32x4 &vn) {
        if constexpr (FUSE) {
          const uint32_t range = is_last(it) ? (uint32_t)(D * 2) : 0u;
          const size_t row = ((size_t)it.s * a.Hkv + it.kvh) * D;
          kn = __builtin_amdgcn_raw_buffer_load_b128(
              buf_rsrc(reinterpret_cast<const uint16_t *>(a.k_new) + row, range), 16 * c16, 0, 0);
          vn = __builtin_amdgcn_raw_buffer_load_b128(
              buf_rsrc(reinterpret_cast<const uint16_t *>(a.v_new) + row, range), 16 * c16, 0, 0);
        }
      };
      // this wave's index of the tile holding the item's new token, or -1
      auto new_tile = [&](const MItem &it) -> int {
        if (!FUSE || !is_last(it)) return -1;
        const int rel = ((it.t1 - 1) >> 4) - it.tile_lo;
        const int q = rel & (kWaves - 1), k = q / it.pst;
        if (q - k * it.pst != it.ph0) return -1;
        return (k == 0 ? 0 : k == 1 ? it.b1 : k == 2 ? it.b2 : it.b3) + (rel >> 2);
      };
      // the table entry of the new token's block is taken when its tile is issued (-1: outside
      // the pool, so the row is not stored); hn: that block among the tile's
#define PKV_NEW_BLOCK(IT, RAW, DST)                                             \
    do {                                                                          \
      const int hn_ = BPT == 1 ? 0 : (((IT).t1 - 1) & 15) / B;                    \
      int e_ = (RAW)[0];                                                          \
      _Pragma("unroll") for (int h_ = 1; h_ < BPT; ++h_) if (h_ == hn_) e_ = (RAW)[h_]; \
      (DST) = (unsigned)e_ < (unsigned)a.N ? e_ : -1;                             \
    } while (0)
      load_item_new(cur, kn_cur, vn_cur);
      int new_i_cur = new_tile(cur), new_i_nxt = -1, new_phys_cur = -1, new_phys_nxt = -1;

      // Loads of tile i of an item (zero-range descriptors past its live tiles).
      auto load_tile = [&](const MItem &it, int i, const int *phys, u32x4 *kd, u32x4 *vd, u32x2 *vd2) {
        const bool live = i < it.n_my;
        const int tok0 = tile_of<WI>(it, i) << 4;
        if constexpr (HM) {
          constexpr uint32_t hb_bytes = D * B * 2;   // one (block, KV head) of K or of V
          const size_t off = ((size_t)phys[0] * a.Hkv + it.kvh) * hb_bytes;
          const uint32_t range = live ? hb_bytes : 0u;
          const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kpool + off, range);
          const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vpool + off, range);
          const int t0b = tok0 % B;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            kd[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, (grp * B + c16) * 16, (4 * c * B + t0b) * 16, kNontemporal);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            vd2[j] = __builtin_amdgcn_raw_buffer_load_b64(rv, (c16 * B + 4 * grp) * 2, (16 * j * B + t0b) * 2, kNontemporal);
          return;
        }
        __amdgpu_buffer_rsrc_t rk[BPT], rv[BPT];
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
          // a block of the tile that lies wholly past the range (its table entry is padding) or
          // a tile past the item's live ones: zero-range descriptor, no memory access
          const uint32_t range = live && tok0 + h * B < it.t1 ? blk_bytes : 0u;
          // the tile's rows in block h (B >= 16: the 16 rows from offset tok0 % B)
          const size_t off = ((size_t)phys[h] * B + (BPT == 1 ? tok0 % B : 0)) * tsb + (size_t)it.kvh * D * 2;
          rk[h] = buf_rsrc(kpool + off, range);
          rv[h] = buf_rsrc(vpool + off, range);
        }
        // K and V alike: instruction r reads whole 256-byte rows (16 lanes per row), streamed
        // past the caches (non-temporal).
#pragma unroll
        for (int r = 0; r < 4; ++r)
          kd[r] = __builtin_amdgcn_raw_buffer_load_b128(rk[r / RPI], row_voff, (r % RPI) * tsb, kNontemporal);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vd[r] = __builtin_amdgcn_raw_buffer_load_b128(rv[r / RPI], row_voff, (r % RPI) * tsb, kNontemporal);
      };
      // tile i of the current item
      auto issue_cur = [&](int i, u32x4 *kd, u32x4 *vd, u32x2 *vd2) {
        const bool live = i < cur.n_my;
        if (live && i > 0 && (i & 63) == 0) {   // into the next chunk of this item's table entries
#pragma unroll
          for (int h = 0; h < BPT; ++h) tb_cur[h] = tb_ahead[h];
          table_chunks<B, WI>(a, cur, (i >> 6) + 1, lane, tb_ahead);
        }
        const int tok0 = tile_of<WI>(cur, i) << 4;
        int phys[BPT];
        if constexpr (FUSE) {
#pragma unroll
          for (int h = 0; h < BPT; ++h) phys[h] = __builtin_amdgcn_readlane(tb_cur[h], i & 63);
          if (i == new_i_cur) PKV_NEW_BLOCK(cur, phys, new_phys_cur);
        }
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
          if constexpr (!FUSE) phys[h] = __builtin_amdgcn_readlane(tb_cur[h], i & 63);
          if ((unsigned)phys[h] >= (unsigned)a.N) {
            if (live && tok0 + h * B < cur.t1) bad_cur = 1;   // an entry the range reads
            phys[h] = 0;
          }
        }
        load_tile(cur, i, phys, kd, vd, vd2);
      };
      // tile i (< NB - 1) of the next item
      auto issue_next = [&](int i, const int *tb_nx, u32x4 *kd, u32x4 *vd, u32x2 *vd2) {
        const int tok0 = tile_of<WI>(nxt, i) << 4;
        int phys[BPT];
        if constexpr (FUSE) {
#pragma unroll
          for (int h = 0; h < BPT; ++h) phys[h] = __builtin_amdgcn_readlane(tb_nx[h], i);
          if (i == new_i_nxt) PKV_NEW_BLOCK(nxt, phys, new_phys_nxt);
        }
#undef PKV_NEW_BLOCK
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
          if constexpr (!FUSE) phys[h] = __builtin_amdgcn_readlane(tb_nx[h], i);
          if ((unsigned)phys[h] >= (unsigned)a.N) {
            if (i < nxt.n_my && tok0 + h * B < nxt.t1) bad_next = 1;
            phys[h] = 0;
          }
        }
        load_tile(nxt, i, phys, kd, vd, vd2);
      };

      // accumulators: MF, MFMA i's 16x16 tile; !MF, head dims 8 c16 + 4i + e of this lane group's
      // tokens (e = 0..3), summed over the lane groups at the merge
      constexpr int NACC = MF ? 8 : 2;
      float m = kNegInf, lsum = 0.f;
      f32x4 acc[NACC];
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      int mbuf = 0;   // the current item's merge buffer
      auto reset_state = [&]() {
        m = kNegInf;
        lsum = 0.f;
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      };
      // This wave's state of one phase into merge buffer mb, slot `slot`, rows of its KV head:
      // (m, l) of each head and its unnormalised rows; the item's sum is spread over the lane
      // groups except on the head-major VALU path.
      auto store_state = [&](int mb, int slot) {
        float lh = lsum;
        if constexpr (MF || !HM) {
          lh += __shfl_xor(lh, 16);
          lh += __shfl_xor(lh, 32);
        }
        const int row = WI ? cur.u * a.g + c16 : c16;     // MF: head c16 of this wave's group
        const bool own = !WI || c16 < a.g;                // (one-head items write all 16 rows)
        const int urow = WI ? cur.u : 0;                  // !MF: the wave's one head
        if constexpr (MF) {
          if (grp == 0 && own) {
            sm.m[mb][row][slot] = m;
            sm.l[mb][row][slot] = lh;
          }
        } else if (lane == 0) {   // one head: m is the same in every lane
          sm.m[mb][urow][slot] = m;
          sm.l[mb][urow][slot] = lh;
        }
        if constexpr (!MF) {   // the lane groups' sums, then dims 8 c16 .. + 7 from lane group 0
#pragma unroll
          for (int i = 0; i < NACC; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = acc[i][e];
              x += __shfl_xor(x, 16);
              x += __shfl_xor(x, 32);
              acc[i][e] = x;
            }
          }
          if (grp == 0) {
            if constexpr (HM) {   // dims 16j + c16
#pragma unroll
              for (int j = 0; j < 8; ++j) sm.o[mb][slot][urow][16 * j + c16] = acc[j >> 2][j & 3];
            } else {              // dims 8 c16 .. + 7
              *reinterpret_cast<f32x4 *>(&sm.o[mb][slot][urow][8 * c16]) = acc[0];
              *reinterpret_cast<f32x4 *>(&sm.o[mb][slot][urow][8 * c16 + 4]) = acc[1];
            }
          }
        } else if constexpr (HM) {   // MFMA i holds dims 16i + 4grp + r
          if (own) {
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4 *>(&sm.o[mb][slot][row][16 * i + 4 * grp]) = acc[i];
          }
        } else if (own) {     // MFMA i holds dims 32grp + 8r + i
          float *dst = &sm.o[mb][slot][row][32 * grp];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[8 * r + i] = acc[i][r];
          }
        }
      };

      auto compute = [&](int i, u32x4 *kr, u32x4 *vr, u32x2 *vr2) {
        if constexpr (WI) {
          if (i == cur.b1 || i == cur.b2 || i == cur.b3) {   // a phase of a wide item ends
            store_state(mbuf, cur.ph0 + (i == cur.b1 ? 0 : i == cur.b2 ? 1 : 2) * cur.pst);
            reset_state();
          }
        }
        const int tok0 = tile_of<WI>(cur, i) << 4;
        if constexpr (FUSE) {
          if (i == new_i_cur) {
            // the new token's place in the tile, and the load (lane group, instruction) of it
            const int t = (cur.t1 - 1) & 15;
            const int gn = BPT == 1 ? t >> 2 : (t % B) / RPI;
            const int rn = BPT == 1 ? (t & 3) : (t / B) * RPI + (t % B) % RPI;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool mine = grp == gn && r == rn;
              kr[r] = mine ? kn_cur : kr[r];
              vr[r] = mine ? vn_cur : vr[r];
            }
            if (new_phys_cur >= 0 && grp == 0) {
              const size_t off = ((size_t)new_phys_cur * B + (cur.t1 - 1) % B) * tsb + (size_t)cur.kvh * D * 2;
              __builtin_amdgcn_raw_buffer_store_b128(kn_cur, buf_rsrc(kpool + off, D * 2), 16 * c16, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(vn_cur, buf_rsrc(vpool + off, D * 2), 16 * c16, 0, 0);
            }
          }
        }
        if constexpr (!MF && HM) {
          // head-major, one query head: lane (c16, grp) holds K chunks 4c + grp of tile row c16
          // and the V pieces of rows 4grp .. 4grp + 3 at dims 16j + c16
          float d = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
              d = __builtin_fmaf(bf16_lo(qop[c][w2]), bf16_lo(kr[c][w2]), d);
              d = __builtin_fmaf(bf16_hi(qop[c][w2]), bf16_hi(kr[c][w2]), d);
            }
          }
          d += __shfl_xor(d, 16);   // the four lane groups' 32 dims each
          d += __shfl_xor(d, 32);
          const int tk = tok0 + c16;
          const float sv = tk >= cur.t0 && tk < cur.t1 ? d * a.scale_log2 : kNegInf;
          const float mnew = fmaxf(m, group_max16(sv));
          const float alpha = merge_weight(m, mnew);
          const float pt = sv == kNegInf ? 0.f : fast_exp2(sv - mnew);
          lsum = lsum * alpha + group_sum<16>(pt);   // the same in every lane
          if (alpha != 1.f) {
#pragma unroll
            for (int j = 0; j < NACC; ++j) acc[j] *= alpha;
          }
          m = mnew;
          if (tok0 < cur.t0 || tok0 + 16 > cur.t1) {   // unread slots may hold anything
            uint32_t keep01 = 0u, keep23 = 0u;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int tr = tok0 + 4 * grp + r;
              const uint32_t half = tr >= cur.t0 && tr < cur.t1 ? ((r & 1) ? 0xffff0000u : 0xffffu) : 0u;
              if (r < 2) keep01 |= half; else keep23 |= half;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) vr2[j] &= (u32x2){keep01, keep23};
          }
          float pr[4];   // p of rows 4grp + r, held by lane 4grp + r
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] = __shfl(pt, 4 * grp + r);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t w = vr2[j][r >> 1];
              acc[j >> 2][j & 3] = __builtin_fmaf(pr[r], (r & 1) ? bf16_hi(w) : bf16_lo(w), acc[j >> 2][j & 3]);
            }
          }
          return;
        }
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!MF) {
          // lane (c16, grp) holds dims 8 c16 .. + 7 of tile row 4 grp + r in kr[r]: a dot product
          // over its 8 dims, then the sum over the 16 lanes of the row
          float qf[8];
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            qf[2 * w2] = bf16_lo(qop[0][w2]);
            qf[2 * w2 + 1] = bf16_hi(qop[0][w2]);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float d = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
              d = __builtin_fmaf(qf[2 * w2], bf16_lo(kr[r][w2]), d);
              d = __builtin_fmaf(qf[2 * w2 + 1], bf16_hi(kr[r][w2]), d);
            }
            sc[r] = group_sum<16>(d);
          }
        } else {
          u32x4 kop[4];
          if constexpr (HM) {
#pragma unroll
            for (int c = 0; c < 4; ++c) kop[c] = kr[c];   // loaded in the A layout
          } else {
            // K tile to the MFMA A layout through the wave's LDS staging: chunk j of token t
            // sits at t*16 + (j ^ t) (16-byte units), so both the row-wise writes (fixed token,
            // 16 chunks) and the operand reads (16 tokens, fixed chunk) hit 16 distinct slots of
            // 64 banks.  Lane (c16, grp) then holds token c16, chunks 4c + grp = dims 32c + 8grp ..
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 4 * grp + r;
              kst[t * 16 + (c16 ^ t)] = kr[r];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) kop[c] = kst[c16 * 16 + ((4 * c + grp) ^ c16)];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[c]),
                                                         __builtin_bit_cast(bf16x8, qop[c]), sc, 0, 0, 0);
        }

        // scores of tile rows 4grp + r (for head c16 on the MFMA path); positions outside
        // [t0, t1) are masked
        float sv[4], mx = kNegInf;
        uint32_t keep01 = 0u, keep23 = 0u;   // head-major V: halves of the tokens in range
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tk = tok0 + (r / RPI) * B + RPI * grp + r % RPI;
          const bool ok = tk >= cur.t0 && tk < cur.t1;
          sv[r] = ok ? sc[r] * a.scale_log2 : kNegInf;
          if constexpr (HM) {
            const uint32_t half = ok ? ((r & 1) ? 0xffff0000u : 0xffffu) : 0u;
            if (r < 2) keep01 |= half; else keep23 |= half;
          } else {
            if (!ok) vr[r] = (u32x4){0u, 0u, 0u, 0u};   // unread slots may hold anything
          }
          mx = fmaxf(mx, sv[r]);
        }
        if constexpr (HM) {
          if (tok0 < cur.t0 || tok0 + 16 > cur.t1) {   // unread slots may hold anything
#pragma unroll
            for (int j = 0; j < 8; ++j) vr2[j] &= (u32x2){keep01, keep23};
          }
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
          for (int j = 0; j < NACC; ++j) acc[j] *= alpha;
        }
        m = mnew;

        if constexpr (!MF) {
          // P.V: each lane adds p(row) times its 8 dims of the row's V piece
#pragma unroll
          for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
              acc[w2 >> 1][2 * (w2 & 1)] = __builtin_fmaf(pr[r], bf16_lo(vr[r][w2]), acc[w2 >> 1][2 * (w2 & 1)]);
              acc[w2 >> 1][2 * (w2 & 1) + 1] =
                  __builtin_fmaf(pr[r], bf16_hi(vr[r][w2]), acc[w2 >> 1][2 * (w2 & 1) + 1]);
            }
          }
          return;
        }

        const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
        const i16x4 pop = __builtin_bit_cast(i16x4, (uint32_t __attribute__((ext_vector_type(2)))){p01, p23});
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (HM) {
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vr2[j]), pop, acc[j], 0, 0, 0);
            continue;
          }
          const int wd = j >> 1;
          uint32_t a01, a23;
          if (j & 1) {
            a01 = (vr[0][wd] >> 16) | (vr[1][wd] & 0xffff0000u);
            a23 = (vr[2][wd] >> 16) | (vr[3][wd] & 0xffff0000u);
          } else {
            a01 = (vr[0][wd] & 0xffffu) | (vr[1][wd] << 16);
            a23 = (vr[2][wd] & 0xffffu) | (vr[3][wd] << 16);
          }
          const i16x4 aop = __builtin_bit_cast(i16x4, (uint32_t __attribute__((ext_vector_type(2)))){a01, a23});
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop, acc[j], 0, 0, 0);
        }
      };

      // the stream's first tiles
      u32x4 kbuf[NB][4], vbuf[NB][4];
      u32x2 vbuf2[NB][HM ? 8 : 1];   // head-major V pieces (unused on the row layout)
      if constexpr (!kLate) {
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) issue_cur(j, kbuf[j], vbuf[j], vbuf2[j]);
      }

      for (int k = 0;; ++k) {
        mbuf = k & 1;
        if constexpr (kLate) {
          // this item's first NB - 1 tiles (its table chunks and q were loaded when it was taken)
#pragma unroll
          for (int j = 0; j < NB - 1; ++j) issue_cur(j, kbuf[j], vbuf[j], vbuf2[j]);
        } else {
          // The next item and its table chunks and q.  Loaded here, a whole tile loop before the
          // copies into the current item's registers at the end of this iteration, so those
          // copies never wait on memory.
          nxt = item_at<NB, WI>(a, wn, sched, sm_pref, sm_ctx, sm_order, wave);
          table_chunks<B, WI>(a, nxt, 0, lane, tb_next);
          table_chunks<B, WI>(a, nxt, 1, lane, tb_next_ahead);
          load_item_q(nxt, qnext);
          load_item_new(nxt, kn_nxt, vn_nxt);
          new_i_nxt = new_tile(nxt);
          new_phys_nxt = -1;
        }
        // Step x computes tile x and issues stream position x + NB - 1.  n_pad is a multiple
        // of NB, so (two-ahead claims) the last NB - 1 steps issue the next item's tiles
        // 0 .. NB-2 into buffers 0 .. NB-2; with kLate they issue nothing, and the next item's
        // first tiles go out at the top of its own iteration.  That last body is a separate copy,
        // so the wait on the next item's table entries sits only there.
        // The first body is a copy of its own too: its waits count the loads and stores
        // issued since this item's first tiles (the merge, the next item's table and q), so
        // it does not wait for more tiles than the one it computes.
        auto body = [&](int x) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            issue_cur(x + j + NB - 1, kbuf[(j + NB - 1) % NB], vbuf[(j + NB - 1) % NB], vbuf2[(j + NB - 1) % NB]);
            __builtin_amdgcn_sched_barrier(0);   // keep those loads ahead of this tile's wait
            if (x + j < cur.n_my) compute(x + j, kbuf[j], vbuf[j], vbuf2[j]);
          }
        };
        int x = 0;
        if (cur.n_pad > NB) {
          body(0);
          for (x = NB; x < cur.n_pad - NB; x += NB) body(x);
        }
        // Take the next item (kLate: it_{k+1}; else it_{k+2}) from the queue now, NB tiles
        // before this item ends (its index is first read at the merge below).  Taking it later
        // than at the item's start keeps a slow workgroup from claiming a long item early that a
        // faster one would finish sooner.
        const bool fetch = a.persistent && tid == 0 && (kLate || wn < total);
        unsigned fetched = 0u;
        if (fetch) fetched = atomicAdd(&a.queue[0], 1u);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (j == 0)
            issue_cur(x + NB - 1, kbuf[NB - 1], vbuf[NB - 1], vbuf2[NB - 1]);
          else if constexpr (!kLate)
            issue_next(j - 1, tb_next, kbuf[j - 1], vbuf[j - 1], vbuf2[j - 1]);
          __builtin_amdgcn_sched_barrier(0);
          if (x + j < cur.n_my) compute(x + j, kbuf[j], vbuf[j], vbuf2[j]);
        }

        // the waves' states of it_k into the merge buffer (the next item's first loads are in
        // flight): the phase in progress, then empty states for a wide item's phases with no tiles
        const int mb = k & 1;
        if constexpr (WI) {
          const int kcur = (cur.n_my > cur.b1) + (cur.n_my > cur.b2) + (cur.n_my > cur.b3);
          store_state(mb, cur.ph0 + kcur * cur.pst);
          for (int kk = kcur + 1; kk < cur.width; ++kk) {
            reset_state();
            store_state(mb, cur.ph0 + kk * cur.pst);
          }
        } else {
          store_state(mb, wave);
        }
        if (lane == 0) sm.bad[mb][wave] = bad_cur;
        if (tid == 0 && a.persistent) sm.nextw[k & 1] = fetch ? (int)((kLate ? 1 : 2) * gridDim.x + fetched) : total;
        __syncthreads();
        if (cur.fill == 0)
          tile_finish(a, cur, sm.m[mb], sm.l[mb], sm.o[mb], sm.bad[mb]);
        else if (cur.fill != 3)
          fill_group<uint16_t, D>(a, cur.s, cur.kvh0 * a.g, cur.width * a.g, cur.fill == 1 ? 0.f : __builtin_nanf(""));
        if constexpr (kLate) {
          // the item just taken: its table chunks, q and new rows
          w = a.persistent ? sm.nextw[k & 1] : total;
          if (w >= total) break;
          cur = item_at<NB, WI>(a, w, sched, sm_pref, sm_ctx, sm_order, wave);
          table_chunks<B, WI>(a, cur, 0, lane, tb_cur);
          table_chunks<B, WI>(a, cur, 1, lane, tb_ahead);
          load_item_q(cur, qop);
          load_item_new(cur, kn_cur, vn_cur);
          new_i_cur = new_tile(cur);
          new_phys_cur = -1;
          bad_cur = 0;
          reset_state();
          continue;
        }
        if (wn >= total) break;

        // advance the stream by one item
        w = wn;
        wn = a.persistent ? sm.nextw[k & 1] : total;
        cur = nxt;
        kn_cur = kn_nxt;
        vn_cur = vn_nxt;
        new_i_cur = new_i_nxt;
        new_phys_cur = new_phys_nxt;
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
          tb_cur[h] = tb_next[h];
          tb_ahead[h] = tb_next_ahead[h];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) qop[c] = qnext[c];
        bad_cur = bad_next;
        bad_next = 0;
        m = kNegInf;
        lsum = 0.f;
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  if constexpr (WIDE) {
    if (__builtin_amdgcn_readfirstlane(sched.nwide) > 0) run_items(std::true_type{});
    else run_items(std::false_type{});
  } else {
    run_items(std::false_type{});
  }
  if (a.persistent) queue_done(a.queue);
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
// Pass 2: merge the partials of one (sequence, head), written in ascending partition order p:
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
// The partition -> thread assignment and the merge order are fixed, so the result does not
// depend on timing.
// ---------------------------------------------------------------------------

// Running log-sum-exp state (max m, sum l, accumulator) merged with the state (m2, l2, o2), in
// that order: the pair's weights relative to the larger max (an empty state weighs 0).
__device__ __forceinline__ void lse_merge(float &m, float &l, f32x4 &acc, float m2, float l2, const f32x4 &o2) {
  const float mn = fmaxf(m, m2);
  const float wa = merge_weight(m, mn), wb = merge_weight(m2, mn);
  l = l * wa + l2 * wb;
  acc = acc * wa + o2 * wb;
  m = mn;
}

// One workgroup of kMergeThreads per (head, sequence), for any number of partials.  Thread
// (chunk c, lane q) takes 16-byte chunk c of the head's partial rows in partitions q, q + PL,
// q + 2 PL, ... (PL lanes) and merges them in that ascending order into a running state;
// the loads of kMergeBatch partitions are issued together, so a lane's partials arrive in one
// round trip per kMergeBatch.  The lanes' states are then merged in ascending lane order
// through LDS.  (A two-stage form -- the maxima first, then the weighted sum -- took three
// dependent rounds of loads and 8.6 us on the long contexts' 28 MB of partials.)
//
// Workgroup i of a one-dimensional grid runs on XCD i % 8 (workgroups are dealt to the eight
// XCDs in turn), and takes (sequence, head) number v, where the workgroups of one XCD take
// consecutive v: the g heads of a KV head, whose (m, l) pairs share one 128-byte line of each
// record, then read that line through one L2 instead of g.  Beyond 2^32 threads in one
// dimension the grid is (head, sequence) instead.
constexpr int kMergeThreads = 512;
constexpr int kMergeBatch = 16;
__device__ __forceinline__ int xcd_grouped(int i, int n) {
  const int x = i & 7, q8 = n >> 3, r8 = n & 7;
  return x * q8 + min(x, r8) + (i >> 3);   // a bijection of [0, n): XCD x takes a run of v
}
template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void attn_reduce_kernel(const AttnArgs a) {
  constexpr int CH = D / 4;                 // 16-byte chunks of a head's fp32 row: 32 or 16
  constexpr int PL = kMergeThreads / CH;    // partition lanes: 16 or 32
  __shared__ float sm_m[PL], sm_l[PL];
  __shared__ f32x4 sm_acc[PL][CH];
  const bool flat = gridDim.y == 1;
  const int v = flat ? xcd_grouped((int)blockIdx.x, a.Hq * a.S) : 0;
  const int h = flat ? v % a.Hq : (int)blockIdx.x, s = flat ? v / a.Hq : (int)blockIdx.y, tid = threadIdx.x;
  const int ctx = a.ctx[s];
  if (ctx < 1 || ctx > a.max_ctx || ctx <= a.P) return;
  const int np = min((ctx + a.P - 1) / a.P, a.max_parts);
  const int kvh = h / a.g, j = h % a.g, c = tid % CH, q = tid / CH;
  const size_t rs = (size_t)(a.g * D + 32);   // record stride in floats
  const float *rec = a.ws_rec + ((size_t)s * a.max_parts * a.Hkv + kvh) * rs;
  const size_t ps = (size_t)a.Hkv * rs;   // between partitions
  float m = kNegInf, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = q; p0 < np; p0 += PL * kMergeBatch) {
    float2 ml[kMergeBatch];
    f32x4 o[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int p = p0 + b * PL;
      const float *r = rec + (size_t)(p < np ? p : 0) * ps;
      ml[b] = p < np ? *reinterpret_cast<const float2 *>(r + a.g * D + 2 * j) : make_float2(kNegInf, 0.f);
      o[b] = p < np ? reinterpret_cast<const f32x4 *>(r + j * D)[c] : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) lse_merge(m, l, acc, ml[b].x, ml[b].y, o[b]);
  }
  if (c == 0) {
    sm_m[q] = m;
    sm_l[q] = l;
  }
  sm_acc[q][c] = acc;
  __syncthreads();
  if (q == 0) {
    float mt = sm_m[0], lt = sm_l[0];
    f32x4 at = sm_acc[0][c];
#pragma unroll
    for (int r = 1; r < PL; ++r) lse_merge(mt, lt, at, sm_m[r], sm_l[r], sm_acc[r][c]);
    const size_t o = ((size_t)s * a.Hq + h) * D + 4 * c;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<T>(a.out, o + e, at[e] / lt);
  }
}

// Pass 2 for at most kShortParts partials per head (the partition count is bounded by the
// host): a workgroup merges kReduceHeads heads of one sequence, a lane per 16-byte chunk of
// a head's output, with every (m, l) pair and partial of the lane loaded at once -- two
// dependent rounds of loads (the length, then the records) per workgroup.  With 8 heads (at
// head_dim 128) every wave takes two heads in one pass; 16 or more heads per workgroup, in
// passes one after the other, and 4, with waves left idle, were slower (gqa70b at 4096-token
// partitions 268.5 / 266.7 / 267.1 us for 16 / 8 / 4, fork_cow steady 25.0 / 23.8 / 23.6 us).
// The maximum first, then the weighted sums, in ascending partition order.
constexpr int kShortParts = 16;
constexpr int kReduceHeads = 8;
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_reduce_short_kernel(const AttnArgs a) {
  constexpr int CH = D / 4;      // 16-byte chunks of fp32 per head: 32 or 16
  constexpr int HPW = 64 / CH;   // heads a wave merges side by side: 2 or 4
  const int s = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ctx = a.ctx[s];
  if (ctx < 1 || ctx > a.max_ctx || ctx <= a.P) return;
  const int np = min((ctx + a.P - 1) / a.P, kShortParts);
  const int c = lane % CH;
  const int h_end = min(a.Hq, (int)(blockIdx.x + 1) * kReduceHeads);
  for (int h = (int)blockIdx.x * kReduceHeads + wv * HPW + lane / CH; h < h_end; h += kWaves * HPW) {
    const int kvh = h / a.g, j = h % a.g;
    const size_t rs = (size_t)(a.g * D + 32);
    const float *rec = a.ws_rec + ((size_t)s * a.max_parts * a.Hkv + kvh) * rs;
    const size_t ps = (size_t)a.Hkv * rs;
    const float *ml = rec + a.g * D + 2 * j;
    const f32x4 *po = reinterpret_cast<const f32x4 *>(rec + j * D) + c;
    float m[kShortParts], l[kShortParts];
    f32x4 o[kShortParts];
#pragma unroll
    for (int p = 0; p < kShortParts; ++p) {
      const bool in = p < np;
      const float2 v = in ? *reinterpret_cast<const float2 *>(ml + (size_t)p * ps) : make_float2(kNegInf, 0.f);
      m[p] = v.x;
      l[p] = v.y;
      o[p] = in ? po[(size_t)p * (ps / 4)] : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    float M = kNegInf;
#pragma unroll
    for (int p = 0; p < kShortParts; ++p) M = fmaxf(M, m[p]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kShortParts; ++p) {
      const float w = merge_weight(m[p], M);
      L += w * l[p];
      acc += w * o[p];
    }
    const size_t oi = ((size_t)s * a.Hq + h) * D + 4 * c;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + oi) = acc / L;
    } else {
      u32x2 v;
      v[0] = pack_bf16x2(acc[0] / L, acc[1] / L);
      v[1] = pack_bf16x2(acc[2] / L, acc[3] / L);
      *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + oi) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int vec_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 0; }

static pkv_path select_path(int Hq, int Hkv, int D, int B, pkv_dtype dt) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return PKV_PATH_NONE;
  if (dt != PKV_DTYPE_F32 && dt != PKV_DTYPE_BF16) return PKV_PATH_NONE;
  if (D != 64 && D != 128) return PKV_PATH_NONE;
  if (B != 4 && B != 8 && B != 16 && B != 32 && B != 64 && B != 128) return PKV_PATH_NONE;
  const int g = Hq / Hkv;
  if (dt == PKV_DTYPE_BF16 && D == 128 && g <= 16) return g == 1 ? PKV_PATH_TILE_VALU : PKV_PATH_MFMA;
  return B <= 32 && vec_group(g) ? PKV_PATH_VECTOR : PKV_PATH_NONE;
}

// Head-major layout: the MFMA kernel only (bf16, D = 128, blocks of 16 slots or more).
static pkv_path select_path_head_major(int Hq, int Hkv, int D, int B, pkv_dtype dt) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return PKV_PATH_NONE;
  if (dt != PKV_DTYPE_BF16 || D != 128 || Hq / Hkv > 16) return PKV_PATH_NONE;
  if (B != 16 && B != 32 && B != 64 && B != 128) return PKV_PATH_NONE;
  return Hq == Hkv ? PKV_PATH_TILE_VALU : PKV_PATH_MFMA;
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

template <bool MF, int NB, bool FUSE = false>
static Pass1Fn tile_fn(int B, bool wide) {
  if (wide) {
    switch (B) {
      case 16: return attn_tile_kernel<16, NB, false, MF, FUSE, true>;
      case 32: return attn_tile_kernel<32, NB, false, MF, FUSE, true>;
      case 64: return attn_tile_kernel<64, NB, false, MF, FUSE, true>;
      default: return attn_tile_kernel<128, NB, false, MF, FUSE, true>;
    }
  }
  switch (B) {
    case 4: return attn_tile_kernel<4, NB, false, MF, FUSE>;
    case 8: return attn_tile_kernel<8, NB, false, MF, FUSE>;
    case 16: return attn_tile_kernel<16, NB, false, MF, FUSE>;
    case 32: return attn_tile_kernel<32, NB, false, MF, FUSE>;
    case 64: return attn_tile_kernel<64, NB, false, MF, FUSE>;
    default: return attn_tile_kernel<128, NB, false, MF, FUSE>;
  }
}

template <bool MF, int NB>
static Pass1Fn tile_hm_fn(int B) {
  switch (B) {
    case 16: return attn_tile_kernel<16, NB, true, MF>;
    case 32: return attn_tile_kernel<32, NB, true, MF>;
    case 64: return attn_tile_kernel<64, NB, true, MF>;
    default: return attn_tile_kernel<128, NB, true, MF>;
  }
}

// deep: the MFMA tiles' deep load ring (split into partitions of at most 256 tokens).  One
// query head per KV head keeps the shallow ring: its merge and stores are a single head's.
// fuse: the fused write of the new tokens (row layout, tile paths, shallow ring: the new rows
// take the registers the deep ring would need).
static Pass1Fn pass1_fn(pkv_path path, pkv_dtype dt, int D, int B, int g, bool head_major, bool deep, bool fuse,
                        bool wide) {
  if (fuse) {
    return path == PKV_PATH_MFMA ? tile_fn<true, kTileDepthShallow, true>(B, wide)
                                 : tile_fn<false, kTileDepthShallow, true>(B, wide);
  }
  if (head_major) {
    if (path == PKV_PATH_TILE_VALU) return tile_hm_fn<false, kTileDepthShallow>(B);
    return deep ? tile_hm_fn<true, kTileDepthDeep>(B) : tile_hm_fn<true, kTileDepthShallow>(B);
  }
  if (path == PKV_PATH_MFMA)
    return deep ? tile_fn<true, kTileDepthDeep>(B, wide) : tile_fn<true, kTileDepthShallow>(B, wide);
  if (path == PKV_PATH_TILE_VALU) return tile_fn<false, kTileDepthShallow>(B, wide);
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

// KV heads per wide work item.  The widest of 4 and 2 heads that divides Hkv, whose query
// heads fit the 16 rows of the merge (width * g <= 16) and that still leaves at least
// kWideMinItems wide items per workgroup (items_ub: one-head items if every partition were
// non-empty); 1 (no wide items) otherwise.  PKV_WIDE_ITEMS=1, 2 or 4 in the environment caps the
// width instead and makes every item of the launch that wide (*forced; for tests and tuning: the
// results are the same bits at every width).
static int wide_heads(int Hkv, int g, int64_t items_ub, int64_t grid, bool *forced) {
  const char *e = getenv("PKV_WIDE_ITEMS");
  const int cap = e && *e ? atoi(e) : 0;
  *forced = cap > 0;
  for (int h = 4; h >= 2; h /= 2) {
    if (Hkv % h != 0 || h * g > 16) continue;
    if (cap > 0 ? h <= cap : items_ub / h >= kWideMinItems * grid) return h;
  }
  return 1;
}

// Pass 2: the short-count kernel when every head has at most kShortParts partials.
template <typename T, int D>
static void launch_reduce(hipStream_t st, const AttnArgs &a) {
  if (a.max_parts <= kShortParts) {
    const dim3 grid((unsigned)((a.Hq + kReduceHeads - 1) / kReduceHeads), (unsigned)a.S);
    hipLaunchKernelGGL((attn_reduce_short_kernel<T, D>), grid, dim3(kThreads), 0, st, a);
  } else {
    const int64_t n = (int64_t)a.Hq * a.S;
    const dim3 grid = n * kMergeThreads < (int64_t(1) << 32) ? dim3((unsigned)n) : dim3((unsigned)a.Hq, (unsigned)a.S);
    hipLaunchKernelGGL((attn_reduce_kernel<T, D>), grid, dim3(kMergeThreads), 0, st, a);
  }
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
  // records of S * Hkv * np items, g * D + 32 floats each: at most S * Hq * np * (D + 32) floats
  return kQueueBytes + (size_t)num_seqs * num_heads * np * (head_dim + 32) * sizeof(float);
}

// Both cache layouts: the row layout [N, B, Hkv, D] and the head-major layout.
static pkv_status decode(bool head_major, void *out, const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                         int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, int32_t partition_size,
                         void *workspace, size_t workspace_bytes, pkv_dtype dtype, void *stream,
                         const void *k_new = nullptr, const void *v_new = nullptr, bool check_only = false) {
  const bool fuse = k_new != nullptr || v_new != nullptr;
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || max_context_len < 1 || partition_size < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  const pkv_path path = head_major ? select_path_head_major(num_heads, num_kv_heads, head_dim, block_size, dtype)
                                   : select_path(num_heads, num_kv_heads, head_dim, block_size, dtype);
  if (path == PKV_PATH_NONE) return PKV_ERR_UNSUPPORTED;
  if (fuse && head_major) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_INVALID_ARG;
  if (partition_size > 0 && partition_size % block_size != 0) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  // token and table-byte offsets are 32-bit inside the kernels
  if (max_context_len > (1 << 30) || max_blocks_per_seq > (1 << 29)) return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return PKV_ERR_INVALID_ARG;
  if (fuse && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))) return PKV_ERR_INVALID_ARG;

  const int64_t P = partition_size > 0 ? partition_size : ((int64_t)max_context_len + 15) / 16 * 16;
  const int64_t np = parts_for(max_context_len, P);
  if (np > kMaxReduceParts) return PKV_ERR_UNSUPPORTED;
  const size_t need = pkv_attention_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return PKV_ERR_INVALID_ARG;
  if (check_only) return PKV_OK;

  AttnArgs a;
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.queue = reinterpret_cast<unsigned *>(workspace);
  // records of num_seqs * num_kv_heads * np items: at most what the workspace size counts
  // (num_seqs * num_heads * np * (head_dim + 32) floats)
  a.ws_rec = np > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kQueueBytes) : nullptr;
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
  a.cls_scale = (float)kClasses / (float)((P < max_context_len ? P : max_context_len) + 1);
  a.k_new = k_new;
  a.v_new = v_new;
  a.hpi = 1;
  a.reserve = 0;
  a.far_blocks = 0;

  hipStream_t st = (hipStream_t)stream;
  const int64_t items = np * num_kv_heads * (int64_t)num_seqs;   // upper bound: every partition non-empty
  if (items > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const bool bf16 = dtype == PKV_DTYPE_BF16;
  // The write rides in the attention launch on the tile paths, except where the MFMA tiles
  // want the deep ring (short partitions: the new rows would take its registers) -- there, and
  // on the vector path, the same write is a launch of its own just before the attention.
  const bool deep = path == PKV_PATH_MFMA && np > 1 && P <= kDeepRingMaxPartition;
  const bool fuse_in_tiles = fuse && !deep && (path == PKV_PATH_MFMA || path == PKV_PATH_TILE_VALU);
  if (fuse && !fuse_in_tiles) {
    // (the caches are written only when the caller passed them writable: the fused entry point)
    const pkv_status ws = launch_kv_write_last(k_new, v_new, const_cast<void *>(k_cache), const_cast<void *>(v_cache),
                                               block_tables, max_blocks_per_seq,
                                               context_lens, max_context_len, num_seqs, num_blocks, block_size,
                                               num_kv_heads, head_dim, bf16 ? 2 : 4, stream);
    if (ws != PKV_OK) return ws;
    a.k_new = a.v_new = nullptr;
  }
  // persistent workgroups when the schedule fits in LDS, else one workgroup per possible item
  Pass1Fn fn = pass1_fn(path, dtype, head_dim, block_size, a.g, head_major, deep, fuse_in_tiles, false);
  size_t dyn_lds = 0;
  int64_t grid = items;
  a.persistent = 0;
  if (num_seqs <= kMaxSchedSeqs) {
    dyn_lds = (path == PKV_PATH_VECTOR ? 2 : 3) * (size_t)num_seqs * sizeof(int);
    const int resident = resident_workgroups(fn, dyn_lds);
    if (resident > 0) {
      a.persistent = 1;
      grid = items < resident ? items : resident;
    } else {
      dyn_lds = 0;
    }
  }
  // wide work items on the tile paths of the row layout
  if (a.persistent && path != PKV_PATH_VECTOR && !head_major && block_size >= 16) {
    bool forced = false;
    a.hpi = wide_heads(num_kv_heads, a.g, items, grid, &forced);
    if (a.hpi > 1) {
      fn = pass1_fn(path, dtype, head_dim, block_size, a.g, head_major, deep, fuse_in_tiles, true);
      const int resident = resident_workgroups(fn, dyn_lds);
      if (resident > 0 && resident < grid) grid = resident;
      a.reserve = forced ? 0 : (int)(kWideReserve * grid);
      const int64_t blk_bytes = (int64_t)block_size * num_kv_heads * head_dim * (bf16 ? 2 : 4);
      a.far_blocks = forced ? 0 : (int)((kWideFarBytes + blk_bytes - 1) / blk_bytes);
    }
  }
  void *args[] = {&a};
  if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)grid), dim3(kThreads), args, dyn_lds, st) !=
      hipSuccess)
    return PKV_ERR_HIP;
  if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  if (np > 1) {
    if (bf16) {
      if (head_dim == 128) launch_reduce<uint16_t, 128>(st, a);
      else launch_reduce<uint16_t, 64>(st, a);
    } else {
      if (head_dim == 128) launch_reduce<float, 128>(st, a);
      else launch_reduce<float, 64>(st, a);
    }
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

extern "C" pkv_status paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                                             const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, float scale,
                                             int32_t partition_size, void *workspace, size_t workspace_bytes,
                                             pkv_dtype dtype, void *stream) {
  return decode(false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, workspace,
                workspace_bytes, dtype, stream);
}

extern "C" pkv_status paged_attention_decode_write(void *out, const void *q, const void *k_new, const void *v_new,
                                                   void *k_cache, void *v_cache, const int32_t *block_tables,
                                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                                   int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                   int32_t num_blocks, float scale, int32_t partition_size,
                                                   void *workspace, size_t workspace_bytes, pkv_dtype dtype,
                                                   void *stream) {
  if (!k_new || !v_new) return PKV_ERR_INVALID_ARG;
  return decode(false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, workspace,
                workspace_bytes, dtype, stream, k_new, v_new);
}

extern "C" pkv_status paged_attention_decode_head_major(
    void *out, const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void *workspace, size_t workspace_bytes, pkv_dtype dtype, void *stream) {
  return decode(true, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, workspace,
                workspace_bytes, dtype, stream);
}

extern "C" pkv_path pkv_attention_path_head_major(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t block_size, pkv_dtype dtype) {
  return select_path_head_major(num_heads, num_kv_heads, head_dim, block_size, dtype);
}

// ---------------------------------------------------------------------------
// paged_attention_decode_noalloc: the same call with the workspace in a static device array
// ---------------------------------------------------------------------------

// The work-queue header and the split's partial states of paged_attention_decode_noalloc, laid
// out as the caller's workspace is.  Every device the library runs on holds its own copy at its
// own address for the life of the process.  Host code never passes this name to a kernel or a
// copy (on the host it only stands for the symbol): it uses the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace pkv {

__global__ void clear_words_kernel(unsigned *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mutex;
static void *g_scratch[kMaxScratchDevices];

// Device address of the current device's scratch.  The first call on a device looks it up and
// clears its work-queue header with a small kernel on `st` (not a memset, so that a call under
// graph capture records a kernel node); every attention call leaves the header at zero again.
static pkv_status static_scratch(hipStream_t st, void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<unsigned *>(p),
                       (int)(kQueueBytes / sizeof(unsigned)));
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" size_t pkv_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" pkv_status paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache,
                                                     const void *v_cache, const int32_t *block_tables,
                                                     int32_t max_blocks_per_seq, const int32_t *context_lens,
                                                     int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                     int32_t num_blocks, float scale, int32_t partition_size,
                                                     pkv_dtype dtype, void *stream) {
  // the sizes decode() checks first; then the limit, before anything is looked up or enqueued
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || max_context_len < 1 || partition_size < 0)
    return PKV_ERR_INVALID_ARG;
  if (pkv_attention_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size) >
      kStaticScratchBytes)
    return PKV_ERR_SCRATCH_LIMIT;
  // every other host check of paged_attention_decode next, with an aligned stand-in for the scratch
  // that is never dereferenced: a rejected call enqueues nothing, not even the first call's clear
  void *ws = reinterpret_cast<void *>(uintptr_t{256});
  pkv_status st = decode(false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                         partition_size, ws, kStaticScratchBytes, dtype, stream, nullptr, nullptr, true);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = static_scratch((hipStream_t)stream, &ws);
  if (st != PKV_OK) return st;
  return decode(false, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, ws,
                kStaticScratchBytes, dtype, stream);
}
