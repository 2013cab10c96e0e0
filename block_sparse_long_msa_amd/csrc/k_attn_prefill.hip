// KV-block-major sparse attention for prefill, and the {q, kv block} -> {kv block, q} remap.
//
// The pages (Chinese rendering of Together AI's MiniMax-M3 write-up, section
// "KV块主序稀疏注意力减少冗余KV移动"; Russian page, third paragraph) make the KV block the outer
// loop: each selected block is moved from HBM once and attended by every query that picked
// it, and because a block only yields a partial output, a log-sum-exp reduction rescales and
// sums the partials afterwards (k_lse_merge).
//
// Remap (a counting sort):
//   bucket = (KV head g, request r, logical block b), ordered g-major.  count -> exclusive scan
//   -> scatter (t, j) into the bucket lists, plus a work list of (bucket, chunk of up to 256 query
//   tokens; smaller chunks when a launch would otherwise have too few items to fill the chip).  Order within a bucket is not fixed, but every (t, g, j) result is computed from its
//   own query row only, so outputs are exact and reproducible whatever the order.
//
// k_attn_kvbm: one workgroup per work item.  It stages block b of KV head g in LDS once -- K
// row-major and V transposed -- then streams the chunk's query rows through it in passes of
// 16*kNT rows per wave (rows = query tokens x G heads).  S^T = K Q^T on bf16 MFMA (tokens are
// M, query rows are N); P never leaves registers: its bf16 values are the B operand of
// O^T = V^T P^T because the PV contraction visits the tokens in the order the S tile already
// holds them (token 32ks + 4qd + e for e < 4, 32ks + 16 + 4qd + e - 4 after).  The causal mask
// (key s valid iff s <= q_pos[t] and s < ctx_len[r]) applies per query row.  Each (t, g, j)
// gets its normalized partial output (bf16) and natural-log LSE.
//
// Work items are mapped XCD-aware: workgroup i runs on XCD i % 8, and the items of one XCD are
// contiguous in the work list, so the items of one bucket share that XCD's L2 for the block (and,
// with the g-major order, each XCD works through about one KV head's buckets).
#include <algorithm>

#include "msa_device.h"

namespace msa {

#ifndef MSA_KVBM_WAVES
#define MSA_KVBM_WAVES 4
#endif
#ifndef MSA_KVBM_NT
#define MSA_KVBM_NT 2
#endif
#ifndef MSA_KVBM_OCC
#define MSA_KVBM_OCC 2
#endif
constexpr int kChunk = 256;               // most query tokens per work item (LDS lists)
constexpr int kMinChunk = 32;             // fewest query tokens per work item
constexpr int kTargetItems = 1024;        // work items a launch aims for (about two per workgroup slot)
constexpr int kNT = MSA_KVBM_NT;          // 16-row MFMA N tiles per wave per pass
constexpr int kWaves = MSA_KVBM_WAVES;    // waves per workgroup, sharing one staged block
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;     // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;

struct PrefillWs {
  int32_t* counts;      // [NB] rows per (KV head, request, block) bucket, all entries
  int32_t* cursor;      // [NB]
  int32_t* rcounts;     // [NB] entries left to the per-block kernel (query-tile path only)
  int32_t* hcounts;     // [NH] rows per anchor-hash bucket (query-tile path)
  int32_t* hcursor;     // [NH]
  int32_t* offsets;     // [NB + 1]
  int32_t* item_off;    // [NB + 1]; item_off[NB] = number of work items
  int32_t* entries;     // [Nq*Hkv*k] packed t * 64 + j
  int2* items;          // [max_items] (bucket, chunk)
  int32_t* hoffsets;    // [NH + 1]
  int32_t* row_key;     // [Nq*Hkv] anchor-hash bucket of the row, or -1
  int32_t* sorted_rows; // [Nq*Hkv] query rows grouped by bucket
  int2* tiles;          // [max_tiles] (bucket, chunk of rows)
  int32_t* tile_count;  // [1]
  uint16_t* dense;      // [NH * 64] each bucket's dense blocks, ascending
  int32_t* dense_n;     // [NH]
  uint64_t* cov_mask;   // [Nq*Hkv] slots j whose block is dense in the row's bucket
  int32_t* row_jt;      // [Nq*Hkv] the row's merged slot, or -1
};

static size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

// Upper bound on the work items: bucket i with c_i entries makes ceil(c_i / chunk) of them.
static int64_t max_items(int64_t total_entries, int64_t NB, int chunk) {
  return total_entries / chunk + (total_entries < NB ? total_entries : NB) + 1;
}

// Query tokens per work item: kChunk when that already makes enough items to fill the chip, else
// halved until it does, but not below one pass of the workgroup's waves (kWaves * 16 * kNT rows,
// i.e. that many / G tokens) or kMinChunk.  A row's partial does not depend on which item holds it,
// so the choice changes the work split only.
static int item_chunk(int64_t total_entries, int G) {
  const int pass = std::max(kMinChunk, kWaves * 16 * kNT / G);
  int c = kChunk;
  while (c > pass && total_entries / c < kTargetItems) c >>= 1;
  return c;
}

int tile_hash_buckets(int max_q);
size_t tile_dense_bytes(int64_t NH);
// tiles of >= 16 query rows each, plus one partial tile per non-empty bucket
static int64_t tile_bound(int64_t rows, int64_t buckets) { return rows / 16 + std::min(rows, buckets) + 1; }

struct PrefillDims {
  int64_t NB, E, R, NH, NS, max_tiles;
  int H;
};
static PrefillDims prefill_dims(int32_t Nq, int32_t Hkv, int32_t k, int32_t B, int32_t max_blocks, int32_t max_q) {
  PrefillDims d;
  d.NB = (int64_t)Hkv * B * max_blocks;
  d.E = (int64_t)Nq * Hkv * k;
  d.R = (int64_t)Nq * Hkv;
  d.NS = (int64_t)Hkv * B;
  d.H = tile_hash_buckets(max_q);
  d.NH = d.NS * d.H;
  d.max_tiles = tile_bound(d.R, d.NH);
  return d;
}

size_t prefill_workspace_bytes(int32_t Nq, int32_t Hkv, int32_t k, int32_t B, int32_t max_blocks, int32_t max_q) {
  const PrefillDims d = prefill_dims(Nq, Hkv, k, B, max_blocks, max_q);
  // the work list is sized for the smallest chunk, so it holds the list of any chunk item_chunk picks
  return a256(d.NB * 4) * 3 + a256(d.NH * 4) * 2 + a256((d.NB + 1) * 4) * 2 + a256(d.E * 4) +
         a256(max_items(d.E, d.NB, kMinChunk) * 8) + a256((d.NH + 1) * 4) + a256(d.R * 4) * 2 + a256(d.max_tiles * 8) +
         a256(4) + a256(tile_dense_bytes(d.NH)) + a256(d.NH * 4) + a256(d.R * 8) + a256(d.R * 4);
}

static PrefillWs carve(void* ws, const PrefillDims& d) {
  char* p = static_cast<char*>(ws);
  PrefillWs w;
  // the counters a launch clears come first and are adjacent: one fill clears them all
  w.counts = reinterpret_cast<int32_t*>(p); p += a256(d.NB * 4);
  w.cursor = reinterpret_cast<int32_t*>(p); p += a256(d.NB * 4);
  w.rcounts = reinterpret_cast<int32_t*>(p); p += a256(d.NB * 4);
  w.hcounts = reinterpret_cast<int32_t*>(p); p += a256(d.NH * 4);
  w.hcursor = reinterpret_cast<int32_t*>(p); p += a256(d.NH * 4);
  w.offsets = reinterpret_cast<int32_t*>(p); p += a256((d.NB + 1) * 4);
  w.item_off = reinterpret_cast<int32_t*>(p); p += a256((d.NB + 1) * 4);
  w.entries = reinterpret_cast<int32_t*>(p); p += a256(d.E * 4);
  w.items = reinterpret_cast<int2*>(p); p += a256(max_items(d.E, d.NB, kMinChunk) * 8);
  w.hoffsets = reinterpret_cast<int32_t*>(p); p += a256((d.NH + 1) * 4);
  w.row_key = reinterpret_cast<int32_t*>(p); p += a256(d.R * 4);
  w.sorted_rows = reinterpret_cast<int32_t*>(p); p += a256(d.R * 4);
  w.tiles = reinterpret_cast<int2*>(p); p += a256(d.max_tiles * 8);
  w.tile_count = reinterpret_cast<int32_t*>(p); p += a256(4);
  w.dense = reinterpret_cast<uint16_t*>(p); p += a256(tile_dense_bytes(d.NH));
  w.dense_n = reinterpret_cast<int32_t*>(p); p += a256(d.NH * 4);
  w.cov_mask = reinterpret_cast<uint64_t*>(p); p += a256(d.R * 8);
  w.row_jt = reinterpret_cast<int32_t*>(p);
  return w;
}

__global__ void k_fill_i32(int32_t* __restrict__ a, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a[i] = v;
}

// Per (t, g, j): count the entry into its bucket, or mark an empty slot's partials as absent.
__global__ __launch_bounds__(256) void k_remap_count(int64_t E, int B, int Hkv, int k, int G, int max_blocks,
                                                     const int32_t* __restrict__ cu_q, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ cnt, int32_t* __restrict__ counts,
                                                     float* __restrict__ part_lse,
                                                     const uint64_t* __restrict__ cov_mask) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= E) return;
  const int64_t tg = idx / k;
  const int j = (int)(idx % k);
  const int g = (int)(tg % Hkv);
  const int t = (int)(tg / Hkv);
  if (j < cnt[tg]) {
    const int r = request_of(cu_q, B, t);
    const int b = sel[idx];
    const int64_t bucket = ((int64_t)g * B + r) * max_blocks + b;
    if (cov_mask && ((cov_mask[tg] >> j) & 1)) return;
    atomicAdd(&counts[bucket], 1);
  } else {
    for (int h = 0; h < G; ++h) part_lse[idx * G + h] = neg_inf();
  }
}

// Exclusive scans of the bucket sizes and of their work-item counts (one workgroup), and the work
// list: bucket i's items (i, 0 .. n_i - 1) at item_off[i], item j holding its entries
// j*chunk .. j*chunk + chunk - 1.
__global__ __launch_bounds__(1024) void k_remap_scan(int64_t NB, int chunk, const int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ item_off,
                                                     int2* __restrict__ items) {
  __shared__ int32_t s_a[1024], s_b[1024];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < NB; base += 1024) {
    const int64_t i = base + tid;
    const int32_t c = i < NB ? counts[i] : 0;
    int32_t a = c, b = (c + chunk - 1) / chunk;
    s_a[tid] = a;
    s_b[tid] = b;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
      const int32_t xa = tid >= off ? s_a[tid - off] : 0;
      const int32_t xb = tid >= off ? s_b[tid - off] : 0;
      __syncthreads();
      s_a[tid] += xa;
      s_b[tid] += xb;
      __syncthreads();
    }
    const int32_t ca = carry[0], cb = carry[1];
    if (i < NB) {
      const int32_t io = cb + s_b[tid] - b;
      offsets[i] = ca + s_a[tid] - a;
      item_off[i] = io;
      for (int j = 0; j < b; ++j) items[io + j] = make_int2((int)i, j);
    }
    __syncthreads();
    if (tid == 1023) { carry[0] = ca + s_a[1023]; carry[1] = cb + s_b[1023]; }
    __syncthreads();
  }
  if (tid == 0) { offsets[NB] = carry[0]; item_off[NB] = carry[1]; }
}

__global__ __launch_bounds__(256) void k_remap_fill(int64_t E, int B, int Hkv, int k, int max_blocks,
                                                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ sel,
                                                    const int32_t* __restrict__ cnt,
                                                    const int32_t* __restrict__ offsets, int32_t* __restrict__ cursor,
                                                    int32_t* __restrict__ entries,
                                                    const uint64_t* __restrict__ cov_mask) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= E) return;
  const int64_t tg = idx / k;
  const int j = (int)(idx % k);
  if (j >= cnt[tg]) return;
  const int g = (int)(tg % Hkv);
  const int t = (int)(tg / Hkv);
  const int r = request_of(cu_q, B, t);
  const int64_t bucket = ((int64_t)g * B + r) * max_blocks + sel[idx];
  if (cov_mask && ((cov_mask[tg] >> j) & 1)) return;
  const int slot = offsets[bucket] + atomicAdd(&cursor[bucket], 1);
  entries[slot] = t * 64 + j;
}

// The same count and scatter with the atomics aggregated in LDS, when every bucket fits in one
// workgroup's histogram: a workgroup counts its run of entries into LDS and adds one total per
// touched bucket to the global counts; the scatter recounts the run, reserves one range per
// touched bucket with a single global atomic, and places its entries with LDS atomics.  The
// popular buckets (hundreds of queries picking the same block) then see one global atomic per
// workgroup instead of one per entry.
//
// Each thread takes its entries kRemapU at a time with every cnt/sel load of the batch issued
// before any is used (indices past the run are clamped and their results dropped), and finds the
// request of a row in a copy of cu_q held in LDS, so a run costs a few round trips, not one chain
// of dependent loads per entry.  Small problems use shorter runs, so that more workgroups share
// the latency.
constexpr int kLdsBuckets = 16384;  // buckets one LDS histogram holds (64 KiB)
constexpr int kRemapU = 8;          // entries per thread per batch
constexpr int kRemapMaxRun = 16384; // entries per workgroup, at most (a multiple of 256 * kRemapU)
constexpr int kLdsCu = 2048;        // requests whose cu_q fits the LDS copy

int remap_run(int64_t E) {
  int run = kRemapMaxRun;
  while (run > 256 * kRemapU && (E + run - 1) / run < 256) run >>= 1;
  return run;
}

struct RemapArgs {
  int64_t E;
  int B, Hkv, k, max_blocks;
  const int32_t* cu_q;
  const int32_t* sel;
  const int32_t* cnt;
  // when set, entry (t, g, j) with bit j of cov_mask[t*Hkv + g] is left out (the query-tile path
  // attends to it); the remap then takes the remaining entries only
  const uint64_t* cov_mask;
};

// Request of row t: binary search over cu_q[0..B], from the LDS copy when there is one.
__device__ __forceinline__ int remap_request(const RemapArgs& a, const int32_t* s_cu, int t) {
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int c = a.B <= kLdsCu ? s_cu[mid] : a.cu_q[mid];
    if (c <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void remap_load_cu(const RemapArgs& a, int32_t* s_cu) {
  if (a.B <= kLdsCu)
    for (int i = threadIdx.x; i <= a.B; i += 256) s_cu[i] = a.cu_q[i];
}

// One batch of this thread's entries base + 256*u: bucket (or -1 for an empty slot j >= cnt, or
// -2 past the run's end) and the entry's code t*64 + j.
__device__ __forceinline__ void remap_batch(const RemapArgs& a, const int32_t* s_cu, int64_t base, int64_t e1,
                                            int (&bucket)[kRemapU], int (&code)[kRemapU]) {
  // entry indices fit in int32 (the entry count is checked on the host)
  int c[kRemapU], sv[kRemapU], tg[kRemapU], ic[kRemapU];
#pragma unroll
  for (int u = 0; u < kRemapU; ++u) {
    ic[u] = (int)min(base + 256 * u, e1 - 1);
    tg[u] = ic[u] / a.k;
    c[u] = a.cnt[tg[u]];
    sv[u] = a.sel[ic[u]];
  }
#pragma unroll
  for (int u = 0; u < kRemapU; ++u) {
    const int j = ic[u] - tg[u] * a.k, t = tg[u] / a.Hkv, g = tg[u] - t * a.Hkv;
    code[u] = t * 64 + j;
    if (base + 256 * u >= e1) bucket[u] = -2;
    else if (j >= c[u]) bucket[u] = -1;
    else bucket[u] = (g * a.B + remap_request(a, s_cu, t)) * a.max_blocks + sv[u];
  }
  if (a.cov_mask) {
#pragma unroll
    for (int u = 0; u < kRemapU; ++u)
      if (bucket[u] >= 0 && ((a.cov_mask[tg[u]] >> (ic[u] - tg[u] * a.k)) & 1)) bucket[u] = -3;
  }
}

__global__ __launch_bounds__(256) void k_remap_count_lds(RemapArgs a, int run, int G, int NB,
                                                         int32_t* __restrict__ counts, float* __restrict__ part_lse) {
  __shared__ int hist[kLdsBuckets];
  __shared__ int32_t s_cu[kLdsCu + 1];
  for (int i = threadIdx.x; i < NB; i += 256) hist[i] = 0;
  remap_load_cu(a, s_cu);
  __syncthreads();
  const int64_t e0 = (int64_t)blockIdx.x * run, e1 = min(e0 + run, a.E);
  for (int64_t base = e0 + threadIdx.x; base < e1; base += 256 * kRemapU) {
    int bucket[kRemapU], code[kRemapU];
    remap_batch(a, s_cu, base, e1, bucket, code);
#pragma unroll
    for (int u = 0; u < kRemapU; ++u) {
      if (bucket[u] >= 0) {
        atomicAdd(&hist[bucket[u]], 1);
      } else if (bucket[u] == -1) {
        const int64_t idx = base + 256 * u;
        for (int h = 0; h < G; ++h) part_lse[idx * G + h] = neg_inf();
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += 256)
    if (hist[i]) atomicAdd(&counts[i], hist[i]);
}

__global__ __launch_bounds__(256) void k_remap_fill_lds(RemapArgs a, int run, int NB,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ cursor, int32_t* __restrict__ entries) {
  __shared__ int hist[kLdsBuckets];  // this run's count per bucket, then its next free slot
  __shared__ int32_t s_cu[kLdsCu + 1];
  for (int i = threadIdx.x; i < NB; i += 256) hist[i] = 0;
  remap_load_cu(a, s_cu);
  __syncthreads();
  const int64_t e0 = (int64_t)blockIdx.x * run, e1 = min(e0 + run, a.E);
  for (int64_t base = e0 + threadIdx.x; base < e1; base += 256 * kRemapU) {
    int bucket[kRemapU], code[kRemapU];
    remap_batch(a, s_cu, base, e1, bucket, code);
#pragma unroll
    for (int u = 0; u < kRemapU; ++u)
      if (bucket[u] >= 0) atomicAdd(&hist[bucket[u]], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += 256) {
    const int c = hist[i];
    if (c) hist[i] = offsets[i] + atomicAdd(&cursor[i], c);
  }
  __syncthreads();
  for (int64_t base = e0 + threadIdx.x; base < e1; base += 256 * kRemapU) {
    int bucket[kRemapU], code[kRemapU];
    remap_batch(a, s_cu, base, e1, bucket, code);
#pragma unroll
    for (int u = 0; u < kRemapU; ++u)
      if (bucket[u] >= 0) entries[atomicAdd(&hist[bucket[u]], 1)] = code[u];
  }
}

// V^T in LDS: row d holds the block's 128 tokens in 4-token (8-byte) chunks; chunk c of row d is
// stored at chunk position c ^ h(d), h(d) = ((d >> 3) & 3) * 4 + (d & 3).  The 16 lanes that read
// one chunk index from the 16 rows 8a + b (a, b < 4) of a PV tile then hit 16 distinct chunk
// positions, i.e. 16 distinct 8-byte bank pairs: no conflicts.
__device__ __forceinline__ int vt_swz(int d, int tok) {
  const int h = (((d >> 3) & 3) << 2) | (d & 3);
  return ((((tok >> 2) ^ h)) << 2) | (tok & 3);
}

template <int D>
__global__ __launch_bounds__(kThreads, MSA_KVBM_OCC) void k_attn_kvbm(
    int B, int Hkv, int G, int k, int max_blocks, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos, const bf16* __restrict__ q,
    const bf16* __restrict__ kcache, const bf16* __restrict__ vcache, int64_t kvpage,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ item_off, const int2* __restrict__ items,
    const int32_t* __restrict__ entries, int64_t NB, int chunk, float scale_log2, bf16* __restrict__ part_o,
    float* __restrict__ part_lse) {
  constexpr int KW = D / 32;        // 32-wide k windows over the head dimension
  constexpr int KS = kBlock / 32;   // 32-token k steps of the PV contraction
  constexpr int PAD = 8;            // LDS row padding (elements)
  constexpr int KST = D + PAD;      // K row stride
  constexpr int VST = kBlock;       // V^T row stride; 4-token chunks XOR-swizzled per row (vt_chunk)
  __shared__ __attribute__((aligned(16))) bf16 k_lds[kBlock * KST];
  __shared__ __attribute__((aligned(16))) bf16 vt_lds[D * VST];
  __shared__ int s_tj[kChunk], s_pos[kChunk];

  // XCD-aware item choice: the workgroups of one XCD take one contiguous run of items
  const int n_items = item_off[NB];
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + slot;
  if (slot >= per_xcd || item >= n_items) return;
  const int2 it = items[item];
  const int64_t bucket = it.x;
  const int g = (int)(bucket / ((int64_t)B * max_blocks));
  const int rb = (int)(bucket % ((int64_t)B * max_blocks));
  const int r = rb / max_blocks, b = rb % max_blocks;
  const int e_begin = offsets[bucket] + it.y * chunk;
  const int e_end = min(e_begin + chunk, offsets[bucket + 1]);  // chunk <= kChunk: fits s_tj
  const int L = ctx_len[r];
  const int page = block_table[(int64_t)r * max_blocks + b];
  const int in_block = min(kBlock, L - b * kBlock);  // tokens of the block that exist
  const int Hq = Hkv * G;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, qd = lane >> 4;

  // ---- stage K (row-major) and V (transposed) of block b, KV head g ----
  // Tokens past the block's end (the context's last, partial block) read the last token that
  // exists instead: every load is in bounds and unconditional, so all of them are in flight at
  // once, and the values are finite.  Those keys are masked for every query row (lim <= in_block),
  // so their scores never count and their V rows are weighted by exactly 0.
  const bf16* kg = kcache + (int64_t)page * kvpage + (int64_t)g * D;
  const bf16* vg = vcache + (int64_t)page * kvpage + (int64_t)g * D;
  const int tstride = Hkv * D;
  static_assert(kBlock * D / 16 % kThreads == 0, "staging assumes whole rounds of 16-byte loads");
  constexpr int NKL = kBlock * D / 8 / kThreads, NVL = kBlock * D / 16 / kThreads;
  u32x4 kst[NKL], vst[NVL][2];
#pragma unroll
  for (int c = 0; c < NKL; ++c) {
    const int idx = tid + kThreads * c, tok = min(idx / (D / 8), in_block - 1), ch = idx % (D / 8);
    kst[c] = ld16(kg + tok * tstride + ch * 8);
  }
#pragma unroll
  for (int c = 0; c < NVL; ++c) {
    const int idx = tid + kThreads * c, tp = idx % (kBlock / 2), ch = idx / (kBlock / 2);
    vst[c][0] = ld16(vg + min(2 * tp, in_block - 1) * tstride + ch * 8);
    vst[c][1] = ld16(vg + min(2 * tp + 1, in_block - 1) * tstride + ch * 8);
  }
#pragma unroll
  for (int c = 0; c < NKL; ++c) {
    const int idx = tid + kThreads * c, tok = idx / (D / 8), ch = idx % (D / 8);
    st16(&k_lds[tok * KST + ch * 8], kst[c]);
  }
#pragma unroll
  for (int c = 0; c < NVL; ++c) {  // two tokens per lane -> 32-bit transposed writes
    const int idx = tid + kThreads * c, tp = idx % (kBlock / 2), ch = idx / (kBlock / 2);
    const int t0 = 2 * tp;
    const u32x4 a = vst[c][0], bb = vst[c][1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (a[e] & 0xffffu) | (bb[e] << 16);           // d = 8ch + 2e
      const uint32_t hi = (a[e] >> 16) | (bb[e] & 0xffff0000u);       // d = 8ch + 2e + 1
      const int d0 = 8 * ch + 2 * e;
      *reinterpret_cast<uint32_t*>(&vt_lds[d0 * VST + vt_swz(d0, t0)]) = lo;
      *reinterpret_cast<uint32_t*>(&vt_lds[(d0 + 1) * VST + vt_swz(d0 + 1, t0)]) = hi;
    }
  }
  __syncthreads();

  const int rows_per_pass = 16 * kNT;          // query rows per wave per pass
  const int tpw = rows_per_pass / G;           // query tokens per wave per pass
  const int s_base = b * kBlock;               // absolute position of the block's first key
  const int n_e = e_end - e_begin;             // query tokens of this work item

  // the item's (t, j) entries and query positions, once, in LDS
  for (int i = tid; i < n_e; i += kThreads) {
    const int packed = entries[e_begin + i];
    s_tj[i] = packed;
    s_pos[i] = q_pos[packed >> 6];
  }
  __syncthreads();

  // query fragments of one pass, prefetched a pass ahead
  struct PassQ {
    u32x4 qf[kNT][KW];
    int pos[kNT], tj[kNT];
  };
  auto load_pass = [&](PassQ& P, int lb) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int rr = 16 * nt + n, sl = rr / G, h = rr % G;
      const int li = lb + sl;
      const bool ok = li < n_e;
      // a row past the chunk end reads the chunk's last query row (finite values) and gets
      // position -1, so every key is masked for it and it is never stored
      const int packed = s_tj[min(li, n_e - 1)];
      P.tj[nt] = ok ? packed : -1;
      P.pos[nt] = ok ? s_pos[li] : -1;
      const bf16* qrow = q + ((int64_t)(packed >> 6) * Hq + g * G + h) * D + 8 * qd;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) P.qf[nt][kw] = ld16(qrow + 32 * kw);
    }
  };
  PassQ nxt;
  if (w * tpw < n_e) load_pass(nxt, w * tpw);

  for (int lb = w * tpw; lb < n_e; lb += kWaves * tpw) {
    const PassQ cur = nxt;
    if (lb + kWaves * tpw < n_e) load_pass(nxt, lb + kWaves * tpw);
    const auto& qf = cur.qf;
    const int* pos = cur.pos;
    const int* tj = cur.tj;
    // S^T[token][row] for the 128 tokens of the block; K fragments read one tile ahead
    f32x4 sacc[kNT][8];
    u32x4 a_cur[KW];
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) a_cur[kw] = ld16(&k_lds[n * KST + 32 * kw + 8 * qd]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      u32x4 a_nxt[KW];
      if (mt < 7) {
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) a_nxt[kw] = ld16(&k_lds[(16 * (mt + 1) + n) * KST + 32 * kw + 8 * qd]);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        f32x4 c = fzero4();
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) c = mfma_bf16(a_cur[kw], qf[nt][kw], c);
        sacc[nt][mt] = c;
      }
      if (mt < 7) {
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) a_cur[kw] = a_nxt[kw];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // softmax statistics per row: m = max of the raw logits, p = 2^(s*scale*log2e - m*scale*log2e).
    // Rows past the chunk end have lim <= 0 and come out all-masked; they are never stored.
    int lim[kNT];
    bool full = true;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      lim[nt] = min(pos[nt] + 1, L) - s_base;  // tokens < lim are valid for this row
      full = full && lim[nt] >= kBlock;
    }
    full = __ballot(!full) == 0;  // wave-uniform: no row of this pass needs masking
    if (!full) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * mt + 4 * qd + i >= lim[nt]) sacc[nt][mt][i] = neg_inf();
    }
    float mrow[kNT], lrow[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float m = neg_inf();
#pragma unroll
      for (int mt = 0; mt < 8; mt += 2)
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(sacc[nt][mt][0], sacc[nt][mt][1]), fmaxf(sacc[nt][mt][2], sacc[nt][mt][3])),
                           fmaxf(fmaxf(sacc[nt][mt + 1][0], sacc[nt][mt + 1][1]),
                                 fmaxf(sacc[nt][mt + 1][2], sacc[nt][mt + 1][3]))));
      m = max_over_quads(m);
      const float mb = (m == neg_inf()) ? 0.f : m * scale_log2;
      float l = 0.f;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sacc[nt][mt][i], scale_log2, -mb));
          sacc[nt][mt][i] = p;
          l += p;
        }
      mrow[nt] = mb;
      lrow[nt] = sum_over_quads(l);  // fp32 sum: the LSE keeps fp32 accuracy
    }
    // P (bf16) as the B operand of the PV MFMA, in the S tile's own token order
    u32x4 pb[kNT][KS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f32x4 lo = sacc[nt][2 * ks], hi = sacc[nt][2 * ks + 1];
        u32x4 v;
        v[0] = pack_bf2(lo[0], lo[1]);
        v[1] = pack_bf2(lo[2], lo[3]);
        v[2] = pack_bf2(hi[0], hi[1]);
        v[3] = pack_bf2(hi[2], hi[3]);
        pb[nt][ks] = v;
      }
    // output slots of this lane's rows
    int64_t orow[kNT];
    float inv[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int rr = 16 * nt + n, h = rr % G;
      const int tjc = max(tj[nt], 0);  // padded rows (tj = -1) are never stored; keep their slot in range
      const int t = tjc >> 6, j = tjc & 63;
      orow[nt] = (((int64_t)t * Hkv + g) * k + j) * G + h;
      inv[nt] = __builtin_amdgcn_rcpf(lrow[nt]);
      if (tj[nt] >= 0 && qd == 0) part_lse[orow[nt]] = (mrow[nt] + fast_log2(lrow[nt])) * kLn2P;
    }
    // O^T = V^T P^T, one pair of 16-row d tiles at a time.  Tile rows are permuted so that lane
    // (n, qd) ends with d = 32u + 8qd .. 32u + 8qd + 7 of its row: row m = 4q + i of tile 2u + x
    // holds d = 32u + 8q + 4x + i.  Each lane then stores 16 contiguous bytes per pair.
#pragma unroll 1
    for (int u = 0; u < D / 32; ++u) {
      f32x4 o[kNT][2];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) { o[nt][0] = fzero4(); o[nt][1] = fzero4(); }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int drow = 32 * u + 8 * (n >> 2) + 4 * x + (n & 3);  // V^T row supplied as A row m = n
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16* vrow = &vt_lds[drow * VST];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + vt_swz(drow, 32 * ks + 4 * qd));
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + vt_swz(drow, 32 * ks + 16 + 4 * qd));
          u32x4 a;
          a[0] = lo.x; a[1] = lo.y; a[2] = hi.x; a[3] = hi.y;
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) o[nt][x] = mfma_bf16(a, pb[nt][ks], o[nt][x]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if (tj[nt] < 0) continue;
        u32x4 v;
        v[0] = pack_bf2(o[nt][0][0] * inv[nt], o[nt][0][1] * inv[nt]);
        v[1] = pack_bf2(o[nt][0][2] * inv[nt], o[nt][0][3] * inv[nt]);
        v[2] = pack_bf2(o[nt][1][0] * inv[nt], o[nt][1][1] * inv[nt]);
        v[3] = pack_bf2(o[nt][1][2] * inv[nt], o[nt][1][3] * inv[nt]);
        st16(part_o + orow[nt] * D + 32 * u + 8 * qd, v);
      }
    }
  }
}

bool tile_supported(int G, int D, int max_blocks, int k);
int tile_tokens(int G);
hipError_t launch_tile_prep(int64_t rows, int B, int Hkv, int k, int G, int max_blocks, const int32_t* cu_q,
                            const int32_t* sel, const int32_t* cnt, const int32_t* counts, int cover_min, int H,
                            int64_t NH, int TT, int32_t* hcounts, int32_t* hcursor, int32_t* row_key,
                            int32_t* hoffsets, int2* tiles, int32_t* tile_count, int32_t* sorted_rows,
                            uint16_t* dense, int32_t* dense_n, uint64_t* cov_mask, int32_t* row_jt, float* part_lse,
                            hipStream_t stream);
hipError_t launch_attn_tiles(int64_t max_tiles, int B, int Hkv, int G, int D, int k, int max_blocks, int H,
                             const int32_t* block_table, const int32_t* ctx_len, const int32_t* q_pos, const void* q,
                             const void* kcache, const void* vcache, int64_t kvpage, const int32_t* sel,
                             const int32_t* hoffsets,
                             const int32_t* sorted_rows, const uint16_t* dense, const int32_t* dense_n,
                             const uint64_t* cov_mask, const int32_t* row_jt, const int2* tiles,
                             const int32_t* tile_count, float scale_log2, void* part_o, float* part_lse,
                             hipStream_t stream);

hipError_t launch_slot_of(int64_t E, int k, const int32_t* cnt, const uint64_t* cov_mask, const int32_t* row_jt,
                          int32_t* slot_of, hipStream_t stream);

// Whether msa_sparse_attn_prefill takes the query-tile path for these shapes.
bool prefill_uses_tiles(int tile_min_rows, int G, int D, int max_blocks, int k) {
  return tile_min_rows > 0 && tile_supported(G, D, max_blocks, k);
}

hipError_t launch_attn_prefill(int B, int Nq, int Hkv, int G, int D, int max_blocks, int max_q,
                               const int32_t* block_table, const int32_t* ctx_len, const int32_t* cu_q,
                               const int32_t* q_pos, const void* q, const void* kcache, const void* vcache,
                               int64_t kvpage, const int32_t* sel, const int32_t* cnt, int k, float sm_scale,
                               int tile_min_rows, void* part_o, float* part_lse, int32_t* slot_of, void* workspace,
                               hipStream_t stream) {
  const PrefillDims d = prefill_dims(Nq, Hkv, k, B, max_blocks, max_q);
  const int64_t NB = d.NB, E = d.E;
  const bool tiles = prefill_uses_tiles(tile_min_rows, G, D, max_blocks, k) && d.NH < (int64_t(1) << 30);
  PrefillWs ws = carve(workspace, d);
  // the counters are adjacent in the workspace: one fill clears them (the tile counters only when used)
  const int64_t n_clear = (int64_t)((tiles ? ws.offsets : ws.rcounts) - ws.counts);
  const int fill_blocks = (int)((n_clear + 255) / 256 < 4096 ? (n_clear + 255) / 256 : 4096);
  hipLaunchKernelGGL(k_fill_i32, dim3(fill_blocks), dim3(256), 0, stream, ws.counts, n_clear, 0);
  const unsigned eb = (unsigned)((E + 255) / 256);
  const bool lds_remap = NB <= kLdsBuckets;
  const int run = remap_run(E);
  const unsigned rb = (unsigned)((E + run - 1) / run);
  const RemapArgs all{E, B, Hkv, k, max_blocks, cu_q, sel, cnt, nullptr};
  const RemapArgs rest{E, B, Hkv, k, max_blocks, cu_q, sel, cnt, tiles ? ws.cov_mask : nullptr};
  auto count = [&](const RemapArgs& a, int32_t* target) {
    if (lds_remap)
      hipLaunchKernelGGL(k_remap_count_lds, dim3(rb), dim3(256), 0, stream, a, run, G, (int)NB, target, part_lse);
    else
      hipLaunchKernelGGL(k_remap_count, dim3(eb), dim3(256), 0, stream, E, B, Hkv, k, G, max_blocks, cu_q, sel, cnt,
                         target, part_lse, a.cov_mask);
  };
  count(all, ws.counts);
  int32_t* bucket_counts = ws.counts;
  if (tiles) {
    // rows into anchor-hash buckets, each bucket's dense blocks, each row's dense slots; then the
    // entries left to the per-block kernel
    hipError_t e = launch_tile_prep(d.R, B, Hkv, k, G, max_blocks, cu_q, sel, cnt, ws.counts, tile_min_rows, d.H,
                                    d.NH, tile_tokens(G), ws.hcounts, ws.hcursor, ws.row_key, ws.hoffsets, ws.tiles,
                                    ws.tile_count, ws.sorted_rows, ws.dense, ws.dense_n, ws.cov_mask, ws.row_jt,
                                    part_lse, stream);
    if (e != hipSuccess) return e;
    count(rest, ws.rcounts);
    bucket_counts = ws.rcounts;
  }
  if (slot_of) {
    hipError_t e = launch_slot_of(E, k, cnt, tiles ? ws.cov_mask : nullptr, ws.row_jt, slot_of, stream);
    if (e != hipSuccess) return e;
  }
  const int chunk = item_chunk(E, G);
  hipLaunchKernelGGL(k_remap_scan, dim3(1), dim3(1024), 0, stream, NB, chunk, bucket_counts, ws.offsets, ws.item_off,
                     ws.items);
  if (lds_remap)
    hipLaunchKernelGGL(k_remap_fill_lds, dim3(rb), dim3(256), 0, stream, rest, run, (int)NB, ws.offsets, ws.cursor,
                       ws.entries);
  else
    hipLaunchKernelGGL(k_remap_fill, dim3(eb), dim3(256), 0, stream, E, B, Hkv, k, max_blocks, cu_q, sel, cnt,
                       ws.offsets, ws.cursor, ws.entries, rest.cov_mask);
  const float sl2 = sm_scale * kLog2eP;
  if (tiles) {
    hipError_t e = launch_attn_tiles(d.max_tiles, B, Hkv, G, D, k, max_blocks, d.H, block_table, ctx_len, q_pos, q,
                                     kcache, vcache, kvpage, sel, ws.hoffsets, ws.sorted_rows, ws.dense, ws.dense_n,
                                     ws.cov_mask, ws.row_jt, ws.tiles, ws.tile_count, sl2, part_o, part_lse, stream);
    if (e != hipSuccess) return e;
  }
  // upper bound on the work items, rounded up to whole XCD rounds
  const int64_t mi = max_items(E, NB, chunk);
  const unsigned grid = (unsigned)(((mi + kXcds - 1) / kXcds) * kXcds);
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kc = static_cast<const bf16*>(kcache);
  const bf16* vc = static_cast<const bf16*>(vcache);
  bf16* po = static_cast<bf16*>(part_o);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_kvbm<128>, dim3(grid), dim3(kThreads), 0, stream, B, Hkv, G, k, max_blocks, block_table,
                       ctx_len, q_pos, qq, kc, vc, kvpage, ws.offsets, ws.item_off, ws.items, ws.entries, NB, chunk,
                       sl2, po, part_lse);
  else
    hipLaunchKernelGGL(k_attn_kvbm<64>, dim3(grid), dim3(kThreads), 0, stream, B, Hkv, G, k, max_blocks, block_table,
                       ctx_len, q_pos, qq, kc, vc, kvpage, ws.offsets, ws.item_off, ws.items, ws.entries, NB, chunk,
                       sl2, po, part_lse);
  return hipGetLastError();
}

}  // namespace msa
