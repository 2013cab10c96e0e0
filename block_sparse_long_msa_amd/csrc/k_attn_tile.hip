// KV-block-major prefill attention over groups of shared blocks: the query-tile path
// (msa_sparse_attn_prefill with tile_min_rows > 0).
//
// The pages make the KV block the outer loop of prefill attention and combine the per-block
// partial outputs with a log-sum-exp reduction (Chinese rendering of Together AI's MiniMax-M3
// write-up, section "KV块主序稀疏注意力减少冗余KV移动"; Russian page, third paragraph).  One partial
// per selected (query row, block) costs a 2 KiB query read and a 2 KiB partial write per pair.
// This path merges partials on chip where many query rows share blocks:
//  - Eligible blocks are those that at least tile_min_rows rows of the request and KV head picked.
//    Each row is bucketed by a hash of its two eligible blocks with the most rows, within its
//    (KV head, request) segment.
//  - A bucket's dense blocks are the eligible blocks at least a quarter of its rows picked (at most
//    64).  The bucket's rows are cut into tiles of 256/G query tokens (eight waves of 32 rows).
//  - A tile walks the bucket's dense blocks in ascending id, staging each in two 64-key halves
//    straight from HBM into a ring of four LDS buffers, three halves ahead.  Each row keeps a running
//    softmax over the dense blocks it picked, so it writes one partial for all of them.  Its other
//    blocks keep one partial each (k_attn_kvbm), and k_lse_merge combines them.
//
// Determinism: a row's dense set depends only on which rows its bucket holds (not on their order),
// and a row takes its dense blocks in ascending id whatever tile it lands in.  A block that a row
// did not pick gets an infinite softmax base for it, so its probabilities are exactly 0 and its
// rescale exactly 1.  The order of rows inside a bucket (set with atomics) therefore changes only
// how much work is skipped, never a result bit.
#include <algorithm>
#include <type_traits>

#include "msa_device.h"

namespace msa {

constexpr int kTileWaves = 8;                 // waves per tile workgroup: two per SIMD
constexpr int kTileNT = 2;                    // 16-row MFMA tiles per wave (32 query rows)
constexpr int kTileThreads = 64 * kTileWaves;
constexpr float kTileLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;                  // log2 headroom before a row's reference max moves

// Hash of a row's two anchor blocks into one of H buckets of its segment (H a power of two).
__device__ __forceinline__ uint32_t anchor_hash(uint32_t a1, uint32_t a2, uint32_t H) {
  uint32_t x = a1 * 0x9E3779B1u ^ (a2 + 0x7F4A7C15u) * 0x85EBCA77u;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 13;
  return x & (H - 1);
}

// Request of query row t (cu_q non-decreasing, cu_q[0] = 0).
__device__ __forceinline__ int tile_request(const int32_t* __restrict__ cu_q, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Dense-set rule: a bucket's dense blocks are those that at least a quarter of its rows picked (and at
// least kDenseMinRows rows), out of the blocks with cover_min rows or more in the whole segment; at
// most kDenseMax of them, the most picked first (ties: lower id).
constexpr int kDenseMax = 64;
constexpr int kDenseMinRows = 2;
constexpr int kDenseMaxBlocks = 16384;   // LDS histogram of k_tile_dense

// Per row (t, g): its two most picked eligible blocks (bucket count >= cover_min; ties: lower id) give
// its hash bucket seg*H + hash(a1, a2), seg = g*B + r.  row_key[tg] = bucket, or -1 with no eligible
// block.
__global__ __launch_bounds__(256) void k_tile_key(int64_t rows, int B, int Hkv, int k, int max_blocks,
                                                  const int32_t* __restrict__ cu_q, const int32_t* __restrict__ sel,
                                                  const int32_t* __restrict__ cnt, const int32_t* __restrict__ counts,
                                                  int cover_min, int H, int32_t* __restrict__ hcounts,
                                                  int32_t* __restrict__ row_key) {
  const int64_t tg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tg >= rows) return;
  const int t = (int)(tg / Hkv), g = (int)(tg % Hkv);
  const int r = tile_request(cu_q, B, t);
  const int c = cnt[tg];
  const int32_t* srow = sel + tg * k;
  const int32_t* crow = counts + ((int64_t)g * B + r) * max_blocks;
  int a1 = -1, n1 = -1, a2 = -1, n2 = -1;
  for (int j = 0; j < c; ++j) {
    const int b = srow[j];
    const int n = crow[b];
    if (n < cover_min) continue;
    // blocks arrive in ascending id, so a strictly larger count is needed to displace an anchor
    if (n > n1) { a2 = a1; n2 = n1; a1 = b; n1 = n; }
    else if (n > n2) { a2 = b; n2 = n; }
  }
  if (a1 < 0) { row_key[tg] = -1; return; }
  const int64_t bucket = ((int64_t)g * B + r) * H + anchor_hash((uint32_t)a1, (uint32_t)a2, (uint32_t)H);
  row_key[tg] = (int32_t)bucket;
  atomicAdd(&hcounts[bucket], 1);
}

// One workgroup: exclusive scan of the bucket sizes (hoffsets[NH + 1]) and of their tile counts
// (ceil(rows / TT) per bucket), and the tile list: tiles[i] = (bucket, chunk of TT rows); tile_count[0]
// = number of tiles.
__global__ __launch_bounds__(1024) void k_tile_scan(int64_t NH, int TT, const int32_t* __restrict__ hcounts,
                                                    int32_t* __restrict__ hoffsets, int2* __restrict__ tiles,
                                                    int32_t* __restrict__ tile_count) {
  __shared__ int32_t s_a[1024], s_b[1024];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < NH; base += 1024) {
    const int64_t i = base + tid;
    const int32_t c = i < NH ? hcounts[i] : 0, nt = (c + TT - 1) / TT;
    s_a[tid] = c;
    s_b[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scans
      const int32_t xa = tid >= off ? s_a[tid - off] : 0;
      const int32_t xb = tid >= off ? s_b[tid - off] : 0;
      __syncthreads();
      s_a[tid] += xa;
      s_b[tid] += xb;
      __syncthreads();
    }
    const int32_t ca = carry[0], cb = carry[1];
    if (i < NH) {
      hoffsets[i] = ca + s_a[tid] - c;
      const int32_t t0 = cb + s_b[tid] - nt;
      for (int j = 0; j < nt; ++j) tiles[t0 + j] = make_int2((int)i, j);
    }
    __syncthreads();
    if (tid == 1023) { carry[0] = ca + s_a[1023]; carry[1] = cb + s_b[1023]; }
    __syncthreads();
  }
  if (tid == 0) { hoffsets[NH] = carry[0]; tile_count[0] = carry[1]; }
}

// Rows into their buckets: sorted_rows holds query row t (order inside a bucket is arbitrary and does
// not affect results).
__global__ __launch_bounds__(256) void k_tile_fill(int64_t rows, int Hkv, const int32_t* __restrict__ row_key,
                                                   const int32_t* __restrict__ hoffsets,
                                                   int32_t* __restrict__ hcursor, int32_t* __restrict__ sorted_rows) {
  const int64_t tg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tg >= rows) return;
  const int32_t bucket = row_key[tg];
  if (bucket < 0) return;
  const int pos = hoffsets[bucket] + atomicAdd(&hcursor[bucket], 1);
  sorted_rows[pos] = (int32_t)(tg / Hkv);
}

// One workgroup per bucket: histogram of its rows' eligible blocks, then its dense set (ascending ids)
// in dense[bucket * kDenseMax ...], dense_n[bucket].  The set depends only on which rows the bucket
// holds, not on their order.
__global__ __launch_bounds__(256) void k_tile_dense(int H, int B, int Hkv, int k, int max_blocks,
                                                    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
                                                    const int32_t* __restrict__ counts, int cover_min,
                                                    const int32_t* __restrict__ hoffsets,
                                                    const int32_t* __restrict__ sorted_rows,
                                                    uint16_t* __restrict__ dense, int32_t* __restrict__ dense_n) {
  __shared__ int hist[kDenseMaxBlocks];
  __shared__ int s_cand[4 * kDenseMax];  // candidates: at most 4*k <= 256 blocks reach a quarter
  __shared__ bool s_keep[4 * kDenseMax];
  __shared__ int s_nc;
  const int64_t bucket = blockIdx.x;
  const int h0 = hoffsets[bucket], n = hoffsets[bucket + 1] - h0;
  if (n == 0) {
    if (threadIdx.x == 0) dense_n[bucket] = 0;
    return;
  }
  const int seg = (int)(bucket / H);
  const int g = seg / B;
  const int32_t* crow = counts + (int64_t)seg * max_blocks;
  for (int i = threadIdx.x; i < max_blocks; i += 256) hist[i] = 0;
  if (threadIdx.x == 0) s_nc = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < n * k; e += 256) {
    const int i = e / k, j = e % k;
    const int64_t tg = (int64_t)sorted_rows[h0 + i] * Hkv + g;
    if (j < cnt[tg]) {
      const int b = sel[tg * k + j];
      if (crow[b] >= cover_min) atomicAdd(&hist[b], 1);
    }
  }
  __syncthreads();
  const int thr = max((n + 3) / 4, kDenseMinRows);
  for (int b = threadIdx.x; b < max_blocks; b += 256)
    if (hist[b] >= thr) {
      const int slot = atomicAdd(&s_nc, 1);
      if (slot < 4 * kDenseMax) s_cand[slot] = b;
    }
  __syncthreads();
  const int nc = min(s_nc, 4 * kDenseMax);
  // keep the kDenseMax candidates ranked first by (count desc, id asc), then write them in ascending id
  for (int c = threadIdx.x; c < nc; c += 256) {
    const int b = s_cand[c], hb = hist[b];
    int rank = 0;
    for (int o = 0; o < nc; ++o) {
      const int b2 = s_cand[o], h2 = hist[b2];
      rank += (h2 > hb || (h2 == hb && b2 < b)) ? 1 : 0;
    }
    s_keep[c] = rank < kDenseMax;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += 256) {
    if (!s_keep[c]) continue;
    const int b = s_cand[c];
    int pos = 0;
    for (int o = 0; o < nc; ++o) pos += (s_keep[o] && s_cand[o] < b) ? 1 : 0;
    dense[bucket * kDenseMax + pos] = (uint16_t)b;
  }
  if (threadIdx.x == 0) dense_n[bucket] = min(nc, kDenseMax);
}

// Per row (t, g): which of its selected slots are dense blocks of its bucket (cov_mask bit j), the
// lowest of them (row_jt, or -1), and lse = -inf for its other dense slots.
__global__ __launch_bounds__(256) void k_tile_entries(int64_t rows, int k, int G, const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ row_key,
                                                      const uint16_t* __restrict__ dense,
                                                      const int32_t* __restrict__ dense_n,
                                                      uint64_t* __restrict__ cov_mask, int32_t* __restrict__ row_jt,
                                                      float* __restrict__ part_lse) {
  const int64_t tg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tg >= rows) return;
  const int32_t bucket = row_key[tg];
  uint64_t m = 0;
  if (bucket >= 0) {
    const int nd = dense_n[bucket], c = cnt[tg];
    const uint16_t* dl = dense + (int64_t)bucket * kDenseMax;
    const int32_t* srow = sel + tg * k;
    int p = 0;
    for (int j = 0; j < c && p < nd; ++j) {  // both lists ascending: one merge walk
      const int b = srow[j];
      while (p < nd && dl[p] < b) ++p;
      if (p < nd && dl[p] == b) m |= 1ull << j;
    }
  }
  cov_mask[tg] = m;
  const int jt = m ? __builtin_ctzll(m) : -1;
  row_jt[tg] = jt;
  for (uint64_t rest = m & (m - 1); rest; rest &= rest - 1) {
    const int j = __builtin_ctzll(rest);
    for (int h = 0; h < G; ++h) part_lse[(tg * k + j) * G + h] = neg_inf();
  }
}

// Staged K and V rows are stored unpadded with their 16-byte chunks swizzled: logical chunk c of
// token row `row` sits at slot c ^ tile_slot(row).  D = 128 (16 chunks per row): the K operand reads
// (one chunk of 16 consecutive rows) and the transposed V reads (4 chunks of 16 consecutive rows,
// half a chunk each) both spread evenly over the 64 banks.  D = 64: rows of equal parity differ.
template <int D>
__device__ __forceinline__ int tile_slot(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

typedef short tile_v4s __attribute__((ext_vector_type(4)));

// 4 consecutive 16-bit values per lane, transposed across each group of 16 lanes (gfx950
// ds_read_b64_tr_b16): lane j of a group receives element j % 4 of the 4-element chunks that lanes
// 4v + j / 4 (v = 0..3) of the group point at, as its values v = 0..3.
__device__ __forceinline__ uint2 ld_tr4(const bf16* p) {
  const tile_v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tile_v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

// One workgroup per tile: up to TT query tokens of one bucket.  The bucket's dense blocks are walked in
// ascending id, each in two halves of 64 keys staged straight from HBM into a ring of four LDS buffers
// (K and V, three halves ahead of the one being multiplied).  A row attends to the dense blocks it
// selected: a running softmax per row, updated per half.
template <int D, int G>
__global__ __launch_bounds__(kTileThreads, 1) void k_attn_tile(
    int B, int Hkv, int k, int max_blocks, int H, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos, const bf16* __restrict__ q,
    const bf16* __restrict__ kcache, const bf16* __restrict__ vcache, int64_t kvpage, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ hoffsets, const int32_t* __restrict__ sorted_rows,
    const uint16_t* __restrict__ dense, const int32_t* __restrict__ dense_n, const uint64_t* __restrict__ cov_mask,
    const int32_t* __restrict__ row_jt, const int2* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    float scale_log2, bf16* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int TT = 256 / G;         // query tokens per tile
  constexpr int NT = kTileNT;
  constexpr int TPW = 16 * NT / G;    // query tokens per wave
  constexpr int KW = D / 32;          // 32-wide k windows of the QK^T contraction
  constexpr int CPR = D / 8;          // 16-byte chunks per staged row
  constexpr int HALF = kBlock / 2;    // keys per staged half block
  constexpr int NIH = HALF * CPR / kTileThreads;  // direct loads per wave per half and tensor
  constexpr int RING = 4;
  static_assert(NIH * kTileThreads == HALF * CPR, "whole rounds of direct loads");
  __shared__ __attribute__((aligned(16))) bf16 kb[RING][HALF * D];
  __shared__ __attribute__((aligned(16))) bf16 vb[RING][HALF * D];
  __shared__ uint16_t s_cov[TT][64];      // each token's dense blocks, ascending
  __shared__ uint16_t s_union[kDenseMax]; // the bucket's dense blocks, ascending
  __shared__ int s_ncov[TT], s_t[TT], s_jt[TT], s_pos[TT];

  // XCD-aware: the workgroups of one XCD take one contiguous run of tiles, so a bucket's tiles share
  // that XCD's L2 for the bucket's dense blocks
  const int ntile = tile_count[0];
  const int per_xcd = (ntile + 7) / 8;
  const int slot = (int)blockIdx.x / 8;
  const int item = ((int)blockIdx.x % 8) * per_xcd + slot;
  if (slot >= per_xcd || item >= ntile) return;
  const int2 tl = tiles[item];
  const int64_t bucket = tl.x;
  const int nu = dense_n[bucket];
  if (nu == 0) return;                    // the bucket's rows all go to the per-block kernel
  const int seg = (int)(bucket / H);
  const int g = seg / B, r = seg % B;
  const int row0 = hoffsets[bucket] + tl.y * TT;
  const int n_tok = min(TT, hoffsets[bucket + 1] - row0);
  const int L = ctx_len[r];
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, qd = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- the tile's tokens and the dense blocks each of them selected ----
  if (tid < kDenseMax) s_union[tid] = tid < nu ? dense[bucket * kDenseMax + tid] : 0;
  if (tid < TT) {
    if (tid < n_tok) {
      const int t = sorted_rows[row0 + tid];
      s_t[tid] = t;
      s_jt[tid] = row_jt[(int64_t)t * Hkv + g];
      s_pos[tid] = q_pos[t];
    } else {
      s_ncov[tid] = 0;
    }
  }
  __syncthreads();
  for (int tau = w; tau < n_tok; tau += kTileWaves) {
    const int64_t tg = (int64_t)s_t[tau] * Hkv + g;
    const uint64_t m = cov_mask[tg];
    const bool cov = lane < k && ((m >> lane) & 1);
    const int b = cov ? sel[tg * k + lane] : 0;
    if (cov) s_cov[tau][__popcll(m & ((1ull << lane) - 1))] = (uint16_t)b;
    if (lane == 0) s_ncov[tau] = __popcll(m);
  }

  // ---- per lane: its rows (16nt + n of the wave), their query fragments and softmax state ----
  int tau_[NT], h_[NT], pcov[NT];
  u32x4 qf[NT][KW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rr = 16 * nt + n;
    tau_[nt] = w * TPW + rr / G;
    h_[nt] = rr % G;
    pcov[nt] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tq = s_t[min(tau_[nt], n_tok - 1)];  // rows past the tile's end read a real query row
    const bf16* qrow = q + ((int64_t)tq * Hq + g * G + h_[nt]) * D + 8 * qd;
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) qf[nt][kw] = ld16(qrow + 32 * kw);
  }
  float m_run[NT], l_run[NT];
  f32x4 o[NT][D / 16];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = neg_inf();
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[nt][dt] = fzero4();
  }

  // ---- staging: half hf of dense block u, straight from HBM into ring slot s % RING (K and V) ----
  // Step s = 2u + hf.  Steps past the end re-load the last half into a slot nobody reads, so that every
  // step issues the same number of loads and the wait below counts exactly the loads behind step s.
  const int tstride = Hkv * D;
  const int nsteps = 2 * nu;
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int sc = min(s, nsteps - 1);
    // uniform block id: the page id comes from a scalar load, which the step waits do not count
    const int b = __builtin_amdgcn_readfirstlane(s_union[sc >> 1]), hf = sc & 1;
    const int page = block_table[(int64_t)r * max_blocks + b];
    const int in_block = min(kBlock, L - b * kBlock);
    const bf16* kg = kcache + (int64_t)page * kvpage + (int64_t)g * D;
    const bf16* vg = vcache + (int64_t)page * kvpage + (int64_t)g * D;
    const int buf = s % RING;
#pragma unroll
    for (int i = 0; i < NIH; ++i) {
      const int grp = kTileWaves * i + w;  // wave-uniform group of 64 chunks
      const int p = grp * 64 + lane;
      const int row = p / CPR, c = (p % CPR) ^ tile_slot<D>(row);
      // keys past a partial block's end read its last key: masked for every row
      const int srow = min(HALF * hf + row, in_block - 1);
      const bf16* ksrc = kg + (int64_t)srow * tstride + 8 * c;
      const bf16* vsrc = vg + (int64_t)srow * tstride + 8 * c;
      const uint32_t kdst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)(&kb[buf][grp * 64 * 8]));
      const uint32_t vdst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)(&vb[buf][grp * 64 * 8]));
      uint32_t m0_saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
          "s_nop 0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
          "s_nop 0\n\ts_mov_b32 m0, %0"
          : "=&s"(m0_saved)
          : "s"(kdst), "v"(ksrc), "s"(vdst), "v"(vsrc)
          : "memory");
    }
  };
  // The query fragments must be in registers before the stream starts: the compiler does not see the
  // direct loads, so a query load it still counted as outstanding inside the loop would make it wait
  // there for every load in flight.  Using them here makes it wait once, before the first step.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) asm volatile("" ::"v"(qf[nt][kw]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  issue(0);
  issue(1);
  issue(2);

  // Per-lane LDS element offsets inside a ring slot.  The key-row swizzle depends only on the row
  // mod 16, so the operand of 16-key tile mi and k window kw sits at koff[kw] + mi*16*D, and the
  // transposed V read of tile (u, x), 32-key step kk and half hh at voff[x][u] + (32kk + 16hh)*D.
  int koff[KW], voff[2][D / 32];
#pragma unroll
  for (int kw = 0; kw < KW; ++kw) koff[kw] = n * D + (((4 * kw + qd) ^ tile_slot<D>(n)) << 3);
  {
    const int c4 = n & 3, t0 = 4 * qd + (n >> 2);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int uu = 0; uu < D / 32; ++uu)
        voff[x][uu] = t0 * D + (((4 * uu + c4) ^ tile_slot<D>(t0)) << 3) + 4 * ((c4 & 1) ^ x);
  }

  bool cov[NT], need[NT];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { cov[nt] = false; need[nt] = false; lim[nt] = kBlock; }
  // One step: half hf of dense block s/2 from ring slot SLOT (a constant, so LDS addresses are
  // immediate offsets from the per-lane ones).
  auto step = [&](int s, auto slot_c) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    // this wave's loads of step s are in LDS (those of the next two steps may still be in flight)
    static_assert(NIH == 1 || NIH == 2, "wait counts below");
    if constexpr (NIH == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    __syncthreads();  // every wave's are, and no wave reads slot (s + 3) % RING any more
    issue(s + 3);
    const int hf = s & 1;
    const int b = __builtin_amdgcn_readfirstlane(s_union[s >> 1]);
    if (hf == 0) {  // which of this lane's rows picked block b; a row's dense blocks come in ascending order
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tau = tau_[nt];
        const bool ok = tau < n_tok && pcov[nt] < s_ncov[tau] && s_cov[tau][pcov[nt]] == b;
        cov[nt] = ok;
        pcov[nt] += ok ? 1 : 0;
        lim[nt] = ok ? min(s_pos[tau] + 1, L) - b * kBlock : kBlock;  // keys < lim are valid for the row
        need[nt] = __ballot(ok) != 0;
      }
    }
    if (!need[0] && !need[1]) return;
    const bf16* kbuf = kb[SLOT];
    const bf16* vbuf = vb[SLOT];
    const int k0 = HALF * hf;  // first key of the half within the block
    // keys past a picking row's causal limit exist only in its diagonal or the context's last block
    const bool cmask = __ballot(lim[0] < k0 + HALF || lim[1] < k0 + HALF) != 0;
    // The multiply-accumulate part, straight-line for each pattern of needed row tiles.
    auto body = [&](auto n0c, auto n1c) __attribute__((always_inline)) {
      constexpr bool N[2] = {decltype(n0c)::value, decltype(n1c)::value};
      // the first four waves (one per SIMD) issue first: the two waves of a SIMD leave the barrier
      // in step and would otherwise reach their MFMA and softmax phases together
      if (w < kTileWaves / 2) __builtin_amdgcn_s_setprio(1);
      // S^T[key][row] = K Q^T for the half's 64 keys
      f32x4 sacc[NT][4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        u32x4 a[KW];
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) a[kw] = ld16(&kbuf[koff[kw] + mi * 16 * D]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (!N[nt]) continue;
          f32x4 c = fzero4();
#pragma unroll
          for (int kw = 0; kw < KW; ++kw) c = mfma_bf16(a[kw], qf[nt][kw], c);
          sacc[nt][mi] = c;
        }
      }
      // Online softmax per row, in units of scale*log2(e).  The reference max of a row moves only
      // when its running max exceeds it by more than kLazy (then the accumulators are rescaled), so
      // the probabilities stay below 2^kLazy.  A row that did not pick the block gets an infinite
      // base: every probability exactly 0, rescale exactly 1, its state unchanged.
      u32x4 pb[NT][2];
      bool grow = false;
      float alpha[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        alpha[nt] = 1.f;
        if (!N[nt]) continue;
        if (cmask) {
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (k0 + 16 * mi + 4 * qd + i >= lim[nt]) sacc[nt][mi][i] = neg_inf();
        }
        float mx = fmaxf(fmaxf(sacc[nt][0][0], sacc[nt][0][1]), fmaxf(sacc[nt][0][2], sacc[nt][0][3]));
#pragma unroll
        for (int mi = 1; mi < 4; ++mi)
          mx = fmaxf(mx, fmaxf(fmaxf(sacc[nt][mi][0], sacc[nt][mi][1]), fmaxf(sacc[nt][mi][2], sacc[nt][mi][3])));
        mx = max_over_quads(mx);
        const float mb = mx * scale_log2;  // -inf when every key of the half is masked for the row
        const bool upd = cov[nt] && mb > m_run[nt] + kLazy;
        const float m_new = upd ? mb : m_run[nt];
        const float base = (cov[nt] && m_new != neg_inf()) ? m_new : __builtin_inff();
        alpha[nt] = upd ? fast_exp2(m_run[nt] - m_new) : 1.f;
        grow = grow || upd;
        float l = 0.f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(__builtin_fmaf(sacc[nt][mi][i], scale_log2, -base));
            sacc[nt][mi][i] = p;
            l += p;
          }
        l_run[nt] = l_run[nt] * alpha[nt] + sum_over_quads(l);
        m_run[nt] = m_new;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const f32x4 lo = sacc[nt][2 * kk], hi = sacc[nt][2 * kk + 1];
          u32x4 v;
          v[0] = pack_bf2(lo[0], lo[1]);
          v[1] = pack_bf2(lo[2], lo[3]);
          v[2] = pack_bf2(hi[0], hi[1]);
          v[3] = pack_bf2(hi[2], hi[3]);
          pb[nt][kk] = v;
        }
      }
      if (__ballot(grow) != 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (!N[nt]) continue;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[nt][dt][i] *= alpha[nt];
        }
      }
      // O^T += V^T P^T.  The contraction visits the keys in the order the S tile holds them (key
      // 32kk + 4qd + e for e < 4, 32kk + 16 + 4qd + e - 4 after).  Tile (u, x) row m = 4c + e holds
      // d = 32u + 8c + 4((c & 1) ^ x) + e, so that lane group qd ends with d = 32u + 8qd .. + 7 over
      // the two tiles x; the transposed read of lane (n, qd) points at key row 32kk + 16hh + 4qd + n/4,
      // d = 32u + 8(n%4) + 4((n%4 & 1) ^ x).
#pragma unroll
      for (int uu = 0; uu < D / 32; ++uu) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const uint2 lo = ld_tr4(&vbuf[voff[x][uu] + 32 * kk * D]);
            const uint2 hi = ld_tr4(&vbuf[voff[x][uu] + (32 * kk + 16) * D]);
            u32x4 a;
            a[0] = lo.x; a[1] = lo.y; a[2] = hi.x; a[3] = hi.y;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if (N[nt]) o[nt][2 * uu + x] = mfma_bf16(a, pb[nt][kk], o[nt][2 * uu + x]);
          }
        }
      }
      if (w < kTileWaves / 2) __builtin_amdgcn_s_setprio(0);
    };
    if (need[0] && need[1]) body(std::true_type{}, std::true_type{});
    else if (need[0]) body(std::true_type{}, std::false_type{});
    else body(std::false_type{}, std::true_type{});
  };
  for (int s = 0; s < nsteps; s += RING) {
    step(s, std::integral_constant<int, 0>{});
    if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
    if (s + 2 < nsteps) step(s + 2, std::integral_constant<int, 2>{});
    if (s + 3 < nsteps) step(s + 3, std::integral_constant<int, 3>{});
  }
  // no LDS write may still be in flight when the workgroup ends (the last steps re-load into the ring)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: each row's merged partial into its slot jt ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tau = tau_[nt];
    if (tau >= n_tok || s_ncov[tau] == 0) continue;
    const int t = s_t[tau], jt = s_jt[tau], h = h_[nt];
    const int64_t orow = (((int64_t)t * Hkv + g) * k + jt) * G + h;
    const float inv = __builtin_amdgcn_rcpf(l_run[nt]);
    if (qd == 0) part_lse[orow] = (m_run[nt] + fast_log2(l_run[nt])) * kTileLn2;
#pragma unroll
    for (int uu = 0; uu < D / 32; ++uu) {
      const f32x4 lo = (qd & 1) ? o[nt][2 * uu + 1] : o[nt][2 * uu];
      const f32x4 hi = (qd & 1) ? o[nt][2 * uu] : o[nt][2 * uu + 1];
      u32x4 v;
      v[0] = pack_bf2(lo[0] * inv, lo[1] * inv);
      v[1] = pack_bf2(lo[2] * inv, lo[3] * inv);
      v[2] = pack_bf2(hi[0] * inv, hi[1] * inv);
      v[3] = pack_bf2(hi[2] * inv, hi[3] * inv);
      st16(part_o + orow * D + 32 * uu + 8 * qd, v);
    }
  }
}

// slot_of[t, g, j]: the slot that holds block sel[t,g,j]'s share of the attention (-1 for j >= cnt).
__global__ __launch_bounds__(256) void k_slot_of(int64_t E, int k, const int32_t* __restrict__ cnt,
                                                 const uint64_t* __restrict__ cov_mask,
                                                 const int32_t* __restrict__ row_jt, int32_t* __restrict__ slot_of) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= E) return;
  const int64_t tg = idx / k;
  const int j = (int)(idx - tg * k);
  int v = -1;
  if (j < cnt[tg]) v = (cov_mask && ((cov_mask[tg] >> j) & 1)) ? row_jt[tg] : j;
  slot_of[idx] = v;
}

hipError_t launch_slot_of(int64_t E, int k, const int32_t* cnt, const uint64_t* cov_mask, const int32_t* row_jt,
                          int32_t* slot_of, hipStream_t stream) {
  hipLaunchKernelGGL(k_slot_of, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream, E, k, cnt, cov_mask, row_jt,
                     slot_of);
  return hipGetLastError();
}

// Hash buckets per (KV head, request) segment for a batch whose requests have at most max_q query rows.
int tile_hash_buckets(int max_q) {
  int h = 16;
  while (h < 1024 && h * 16 < max_q) h <<= 1;
  return h;
}

int tile_tokens(int G) { return 256 / G; }

bool tile_supported(int G, int D, int max_blocks, int k) {
  return (G == 4 || G == 8 || G == 16) && (D == 64 || D == 128) && max_blocks <= kDenseMaxBlocks && k <= 64;
}

size_t tile_dense_bytes(int64_t NH) { return (size_t)NH * kDenseMax * sizeof(uint16_t); }

hipError_t launch_tile_prep(int64_t rows, int B, int Hkv, int k, int G, int max_blocks, const int32_t* cu_q,
                            const int32_t* sel, const int32_t* cnt, const int32_t* counts, int cover_min, int H,
                            int64_t NH, int TT, int32_t* hcounts, int32_t* hcursor, int32_t* row_key,
                            int32_t* hoffsets, int2* tiles, int32_t* tile_count, int32_t* sorted_rows,
                            uint16_t* dense, int32_t* dense_n, uint64_t* cov_mask, int32_t* row_jt, float* part_lse,
                            hipStream_t stream) {
  const dim3 rg((unsigned)((rows + 255) / 256));
  hipLaunchKernelGGL(k_tile_key, rg, dim3(256), 0, stream, rows, B, Hkv, k, max_blocks, cu_q, sel, cnt, counts,
                     cover_min, H, hcounts, row_key);
  hipLaunchKernelGGL(k_tile_scan, dim3(1), dim3(1024), 0, stream, NH, TT, hcounts, hoffsets, tiles, tile_count);
  hipLaunchKernelGGL(k_tile_fill, rg, dim3(256), 0, stream, rows, Hkv, row_key, hoffsets, hcursor, sorted_rows);
  hipLaunchKernelGGL(k_tile_dense, dim3((unsigned)NH), dim3(256), 0, stream, H, B, Hkv, k, max_blocks, sel, cnt,
                     counts, cover_min, hoffsets, sorted_rows, dense, dense_n);
  hipLaunchKernelGGL(k_tile_entries, rg, dim3(256), 0, stream, rows, k, G, sel, cnt, row_key, dense, dense_n,
                     cov_mask, row_jt, part_lse);
  return hipGetLastError();
}

hipError_t launch_attn_tiles(int64_t max_tiles, int B, int Hkv, int G, int D, int k, int max_blocks, int H,
                             const int32_t* block_table, const int32_t* ctx_len, const int32_t* q_pos, const void* q,
                             const void* kcache, const void* vcache, int64_t kvpage, const int32_t* sel,
                             const int32_t* hoffsets, const int32_t* sorted_rows, const uint16_t* dense,
                             const int32_t* dense_n, const uint64_t* cov_mask, const int32_t* row_jt,
                             const int2* tiles, const int32_t* tile_count, float scale_log2, void* part_o,
                             float* part_lse, hipStream_t stream) {
  const unsigned grid = (unsigned)((max_tiles + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kc = static_cast<const bf16*>(kcache);
  const bf16* vc = static_cast<const bf16*>(vcache);
  bf16* po = static_cast<bf16*>(part_o);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kTileThreads), 0, stream, B, Hkv, k, max_blocks, H, block_table,
                       ctx_len, q_pos, qq, kc, vc, kvpage, sel, hoffsets, sorted_rows, dense, dense_n, cov_mask,
                       row_jt, tiles, tile_count, scale_log2, po, part_lse);
  };
  if (D == 128) {
    if (G == 4) go(k_attn_tile<128, 4>);
    else if (G == 8) go(k_attn_tile<128, 8>);
    else go(k_attn_tile<128, 16>);
  } else {
    if (G == 4) go(k_attn_tile<64, 4>);
    else if (G == 8) go(k_attn_tile<64, 8>);
    else go(k_attn_tile<64, 16>);
  }
  return hipGetLastError();
}

}  // namespace msa
