// Decode attention over the sparse per-row page table, and the log-sum-exp merge.
//
// Rows are (query row, KV head) pairs with the KV-group dimension folded into the batch;
// each row reads its selected pages through a strided view of the shared paged KV tensor
// (virtual page v at v*page_stride, tokens every token_stride elements) -- Chinese page of
// the MiniMax-M3 serving write-up, section "MSA需要新的分页注意力集成".
//
// k_attn_decode: one workgroup per (row, run of pages); the four waves take 32 tokens of every
//   page each and keep a running softmax over the run.
//   S^T = K Q^T on bf16 MFMA with the tokens as M and the G query heads padded into N.
//   P stays in the registers of the MFMA result that produced it and feeds O^T = V^T P^T as the
//   (bf16) B operand of a 16x16x32 MFMA: lane (n, q) holds P for its 8 tokens, and loads the same
//   tokens' V rows as 16 contiguous bytes each, whose element c over the 8 tokens becomes the A
//   operand of MFMA c (output row m of MFMA c is d = 8m + c).  No LDS transpose, no shuffles,
//   every V row read as whole 64-byte segments.  The four waves' (max, sum, O) are combined
//   through LDS.  A row is split over several workgroups only as far as needed to occupy the chip;
//   the last split of a row to finish combines the row's split partials (merge_row), so there is
//   no second launch, or, for rows split more than kFusedMergeMax ways, k_merge_splits does.
// k_select_attend: the top-k, the page table and k_attn_decode in one launch -- each attention
//   workgroup selects its own row's blocks from the scores (row_topk, topk_select.h) and takes the
//   chosen pages' ids from LDS instead of a page table in memory.
// k_lse_merge: LSE = log sum_j exp(lse_j); O = sum_j exp(lse_j - LSE) O_j over the parts with
//   lse_j > -inf (section "KV块主序稀疏注意力减少冗余KV移动").
#include <algorithm>
#include <mutex>

#include "msa.h"
#include "msa_device.h"
#include "topk_select.h"

namespace msa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#ifndef MSA_DECODE_TARGET_WGS
#define MSA_DECODE_TARGET_WGS 256  // workgroups a decode launch aims for (one per CU, two pages in flight each)
#endif

// One page's operands for one lane of wave w: K rows 32w + 16sub + n (16-byte chunk kw, qd of
// each) and V rows 32w + 16sub + 4qd + i (elements 8n .. 8n+7).
template <int D>
struct PageRegs {
  u32x4 k[2][D / 32];
  u32x4 v[2][4];
};

// Issue every load of one page.  A token index past the row's end is clamped to the last valid
// token, so every address stays inside the row and every loaded value is a finite cache entry;
// such tokens get probability exactly 0 below.  The loads carry no condition, so all of them are
// in flight together.  Each K load instruction covers half of every token's 128-byte line and
// the next one the other half, so K goes through L1 (ordinary loads); V rows are read as whole
// lines and stream past it (non-temporal).  (For D = 64 the lanes n >= 8 re-read chunk n - 8: same cache lines, and
// the MFMA rows they feed, d >= 64, are never stored.)
template <int D>
__device__ __forceinline__ void load_page(PageRegs<D>& r, const bf16* kb, const bf16* vb, int ts, int valid,
                                          int w, int n, int qd) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int tok = min(32 * w + 16 * sub + n, valid - 1);
#pragma unroll
    for (int kw = 0; kw < D / 32; ++kw) r.k[sub][kw] = ld16(kb + tok * ts + 32 * kw + 8 * qd);
  }
  const int dv = (8 * n) & (D - 1);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = min(32 * w + 16 * sub + 4 * qd + i, valid - 1);
      r.v[sub][i] = ld16_nt(vb + tok * ts + dv);
    }
}

// Fold one page into the wave's running (m, l, O) for head n (online softmax, base 2).
template <int D>
__device__ __forceinline__ void attend_page(const PageRegs<D>& r, const u32x4 (&qf)[D / 32], int valid, int w,
                                            int qd, float scale_log2, float& m, float& l, f32x4 (&acc)[8]) {
  f32x4 s[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = fzero4();
#pragma unroll
    for (int kw = 0; kw < D / 32; ++kw) s[sub] = mfma_bf16(r.k[sub][kw], qf[kw], s[sub]);
  }
  // s[sub][i] = S[token 32w + 16sub + 4qd + i][head n]
  float mp = neg_inf();
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 16 * sub + 4 * qd + i;
      const float x = (tok < valid) ? s[sub][i] * scale_log2 : neg_inf();
      s[sub][i] = x;
      mp = fmaxf(mp, x);
    }
  const float mn = fmaxf(m, max_over_quads(mp));
  const float alpha = (m == neg_inf()) ? 0.f : fast_exp2(m - mn);
  m = mn;
  float ls = 0.f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (mn == neg_inf()) ? 0.f : fast_exp2(s[sub][i] - mn);
      s[sub][i] = p;
      ls += p;
    }
  l = l * alpha + sum_over_quads(ls);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c][e] *= alpha;
  // O^T += V^T P^T on bf16 MFMA over the wave's 32 tokens, in the order the S tiles hold them: k slot
  // 8qd + j of lane group qd is token 4qd + j (j < 4) or 16 + 4qd + j - 4.  B = P^T: lane (n, qd)
  // already holds its 8 tokens' probabilities for head n.  A for MFMA c = V^T rows d = 8m + c: lane
  // (m, qd) loaded 8 consecutive d of each of the same 8 tokens, so its A operand is element c of those
  // 8 loads, regrouped in registers.
  u32x4 pb;
  pb[0] = pack_bf2(s[0][0], s[0][1]);
  pb[1] = pack_bf2(s[0][2], s[0][3]);
  pb[2] = pack_bf2(s[1][0], s[1][1]);
  pb[3] = pack_bf2(s[1][2], s[1][3]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e = c >> 1;
    auto pair = [&](const u32x4& x, const u32x4& y) {  // element c of x (low half), of y (high half)
      return (c & 1) ? ((x[e] >> 16) | (y[e] & 0xffff0000u)) : ((x[e] & 0xffffu) | (y[e] << 16));
    };
    u32x4 a;
    a[0] = pair(r.v[0][0], r.v[0][1]);
    a[1] = pair(r.v[0][2], r.v[0][3]);
    a[2] = pair(r.v[1][0], r.v[1][1]);
    a[3] = pair(r.v[1][2], r.v[1][3]);
    acc[c] = mfma_bf16(a, pb, acc[c]);
  }
}

// LDS of one decode attention workgroup: the four waves' (max, sum, O) for the final combine.
template <int D>
struct DecodeLds {
  static constexpr int OST = D + 4;  // padded row of the per-wave outputs
  float m[4][16], l[4][16];
  __align__(16) float o[4][16][OST];
  unsigned ticket;  // this split's place among the row's splits to finish
};

// Split partials are written by one workgroup and read by another, which may run on another XCD
// with its own L2.  They are stored and loaded as agent-scope relaxed atomics (global stores and
// loads with sc1 set), which are coherent across the XCDs by themselves, so the hand-off needs no
// device-scope fence: such a fence writes back and invalidates the whole L2 of every XCD.
__device__ __forceinline__ void store_agent(float* p, f32x4 v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(p);
  const uint64_t lo = ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]);
  const uint64_t hi = ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]);
  __hip_atomic_store(d, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_agent4(const float* p) {
  const uint64_t* s = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const f32x4 v = {__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                   __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
  return v;
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last split of row rho to finish folds the row's nsplit partials (O_j normalized, LSE_j) into
// the output: LSE = M + ln sum_j exp(LSE_j - M) with M = max_j LSE_j, O = sum_j exp(LSE_j - LSE) O_j
// (section "KV块主序稀疏注意力减少冗余KV移动").  Thread e takes the 4-float chunk e of the G x D
// output and reads the parts in batches of eight, all loads of a batch issued together.  A part with
// LSE = -inf (a split past the row's last page) has weight 0 and its O is not read.
template <int D>
__device__ __forceinline__ void merge_row(int G, int rho, int nsplit, const float* __restrict__ ws_o,
                                          const float* __restrict__ ws_lse, bf16* __restrict__ out,
                                          float* __restrict__ lse_out) {
  constexpr int kBatch = 8;
  for (int e = threadIdx.x; e < G * D / 4; e += 256) {
    const int h = (4 * e) / D, d = (4 * e) % D;
    const float* pl = ws_lse + (int64_t)rho * nsplit * G + h;
    const float* po = ws_o + ((int64_t)rho * nsplit * G + h) * D + d;
    float m = neg_inf(), sum = 0.f;
    f32x4 o = fzero4();
    for (int j0 = 0; j0 < nsplit; j0 += kBatch) {
      float x[kBatch];
      f32x4 v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) x[i] = j0 + i < nsplit ? load_agent(pl + (int64_t)(j0 + i) * G) : neg_inf();
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        v[i] = x[i] != neg_inf() ? load_agent4(po + (int64_t)(j0 + i) * G * D) : fzero4();
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (x[i] == neg_inf()) continue;
        const float mn = fmaxf(m, x[i]);
        const float a = (m == neg_inf()) ? 0.f : __expf(m - mn);
        const float wj = __expf(x[i] - mn);
        sum = sum * a + wj;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = o[t] * a + wj * v[i][t];
        m = mn;
      }
    }
    const float inv = 1.f / sum;
    uint2 pk;
    pk.x = pack_bf2(o[0] * inv, o[1] * inv);
    pk.y = pack_bf2(o[2] * inv, o[3] * inv);
    *reinterpret_cast<uint2*>(out + ((int64_t)rho * G + h) * D + d) = pk;
    if (d == 0 && lse_out) lse_out[(int64_t)rho * G + h] = m + __logf(sum);
  }
}

// Split hand-off: every thread's partial stores are complete (vmcnt(0)) before the workgroup takes
// its ticket from the row's arrival counter; the split that draws nsplit - 1 is the last, returns the
// counter to zero for the next call and merges the row.
template <int D>
__device__ __forceinline__ void finish_split(DecodeLds<D>& sm, int G, int rho, int nsplit,
                                             uint32_t* __restrict__ counters, const float* __restrict__ ws_o,
                                             const float* __restrict__ ws_lse, bf16* __restrict__ out,
                                             float* __restrict__ lse_out) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    sm.ticket = __hip_atomic_fetch_add(counters + rho, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sm.ticket != (unsigned)(nsplit - 1)) return;
  if (threadIdx.x == 0) __hip_atomic_store(counters + rho, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  merge_row<D>(G, rho, nsplit, ws_o, ws_lse, out, lse_out);
}

// Page ids of a run read from the row's page table in memory; the first two arrive with the row
// length, so the first K/V loads wait for one round trip, not two.
struct PagesInMemory {
  const int32_t* pt;
  int j0, pt0, pt1;
  __device__ int operator()(int j) const { return j == j0 ? pt0 : j == j0 + 1 ? pt1 : pt[j]; }
};
// Page ids already on chip (the fused select + attend kernel).
struct PagesInLds {
  const int* pt;
  __device__ int operator()(int j) const { return pt[j]; }
};

// Workgroup (split sp, row rho) attends to the row's pages [sp*ppw, (sp+1)*ppw) with two pages of
// loads in flight (one being consumed, the next arriving).  With nsplit = 1 it writes the final
// bf16 output and LSE; otherwise an fp32 partial and its LSE per (row, split), which the row's last
// split to finish merges.
template <int D, typename Pages>
__device__ __forceinline__ void attend_run(DecodeLds<D>& sm, int G, const bf16* __restrict__ q,
                                           const bf16* __restrict__ kview, const bf16* __restrict__ vview,
                                           int64_t page_stride, int64_t token_stride, const Pages& pages, int len,
                                           int rho, int sp, int ppw, int nsplit, float scale_log2,
                                           bf16* __restrict__ out, float* __restrict__ lse_out,
                                           float* __restrict__ ws_o, float* __restrict__ ws_lse,
                                           uint32_t* __restrict__ counters) {
  constexpr int KW = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, qd = lane >> 4;
  const int j0 = sp * ppw;
  const int npages = (len + kBlock - 1) / kBlock;
  const int j1 = min(j0 + ppw, npages);
  const int64_t part = (int64_t)rho * nsplit + sp;
  if (j0 >= j1) {  // only with nsplit > 1: a split past the row's last page
    if (tid < G) store_agent(ws_lse + part * G + tid, neg_inf());
    if (counters) finish_split<D>(sm, G, rho, nsplit, counters, ws_o, ws_lse, out, lse_out);
    return;
  }
  // Page j of the run; a prefetch past the run's end re-reads one token of its last page (valid
  // = 1: every lane of a wave hits the same two rows), so every load in the loop is unconditional
  // and the wait before each page counts exactly the page behind it.
  auto page_valid = [&](int j) { return j < j1 ? min(kBlock, len - j * kBlock) : 1; };
  auto load = [&](PageRegs<D>& r, int j) {
    const int64_t vp = pages(min(j, j1 - 1));
    load_page<D>(r, kview + vp * page_stride, vview + vp * page_stride, (int)token_stride, page_valid(j), w, n,
                 qd);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute it overlaps
  };

  u32x4 qf[KW];
  const int nq = min(n, G - 1);
#pragma unroll
  for (int kw = 0; kw < KW; ++kw) qf[kw] = ld16(q + ((int64_t)rho * G + nq) * D + 32 * kw + 8 * qd);
  PageRegs<D> ra, rb;
  load(ra, j0);
  load(rb, j0 + 1);
  if (n >= G) {
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) qf[kw] = zero4();
  }
  float m = neg_inf(), l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = fzero4();
  for (int j = j0; j < j1; j += 2) {
    attend_page<D>(ra, qf, page_valid(j), w, qd, scale_log2, m, l, acc);
    load(ra, j + 2);
    if (j + 1 < j1) attend_page<D>(rb, qf, page_valid(j + 1), w, qd, scale_log2, m, l, acc);
    load(rb, j + 3);
  }

  // acc[c][ii] = O_w[head n][d = 32qd + 8ii + c] (unnormalized); combine the four waves
  if (qd == 0) { sm.m[w][n] = m; sm.l[w][n] = l; }
  if (n < G) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int d = 32 * qd + 8 * ii;
      if (d < D) {
        const f32x4 lo = {acc[0][ii], acc[1][ii], acc[2][ii], acc[3][ii]};
        const f32x4 hi = {acc[4][ii], acc[5][ii], acc[6][ii], acc[7][ii]};
        *reinterpret_cast<f32x4*>(&sm.o[w][n][d]) = lo;
        *reinterpret_cast<f32x4*>(&sm.o[w][n][d + 4]) = hi;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D / 4; e += 256) {
    const int h = (4 * e) / D, d = (4 * e) % D;
    float M = neg_inf();
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm.m[ww][h]);
    float den = 0.f;
    f32x4 o = fzero4();
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sm.m[ww][h];
      const float f = (mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      den += f * sm.l[ww][h];
      const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.o[ww][h][d]);
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] += f * x[t];
    }
    const float inv = 1.f / den;
    const float lse = (M + fast_log2(den)) * kLn2;
    if (nsplit == 1) {
      uint2 pk;
      pk.x = pack_bf2(o[0] * inv, o[1] * inv);
      pk.y = pack_bf2(o[2] * inv, o[3] * inv);
      *reinterpret_cast<uint2*>(out + ((int64_t)rho * G + h) * D + d) = pk;
      if (d == 0 && lse_out) lse_out[(int64_t)rho * G + h] = lse;
    } else {
      f32x4 r = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      store_agent(ws_o + (part * G + h) * D + d, r);
      if (d == 0) store_agent(ws_lse + part * G + h, lse);
    }
  }
  if (nsplit > 1 && counters) finish_split<D>(sm, G, rho, nsplit, counters, ws_o, ws_lse, out, lse_out);
}

// Decode attention over a page table in memory: workgroup (split, row) = blockIdx.x as (rho*nsplit + sp).
template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_decode(
    int G, const bf16* __restrict__ q, const bf16* __restrict__ kview, const bf16* __restrict__ vview,
    int64_t page_stride, int64_t token_stride, const int32_t* __restrict__ page_table, int k,
    const int32_t* __restrict__ row_len, float scale_log2, int ppw, int nsplit, bf16* __restrict__ out,
    float* __restrict__ lse_out, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    uint32_t* __restrict__ counters) {
  __shared__ DecodeLds<D> sm;
  const int sp = (int)(blockIdx.x % (unsigned)nsplit), rho = (int)(blockIdx.x / (unsigned)nsplit);
  const int j0 = sp * ppw;
  const int32_t* pt = page_table + (int64_t)rho * k;
  // the first two page ids are read together with the row length (both in bounds of the row's k
  // entries), so the first K/V loads wait for one round trip, not two
  const int pt0 = pt[j0], pt1 = pt[min(j0 + 1, k - 1)];
  const int len = row_len[rho];
  asm volatile("" ::"s"(pt0), "s"(pt1), "s"(len));  // issue the three loads here, side by side
  const PagesInMemory pages{pt, j0, pt0, pt1};
  attend_run<D>(sm, G, q, kview, vview, page_stride, token_stride, pages, len, rho, sp, ppw, nsplit, scale_log2,
                out, lse_out, ws_o, ws_lse, counters);
}

// Top-k, page table and decode attention in one launch.  Workgroup (split sp, row rho) selects its
// row's blocks itself -- the same row_topk as the top-k kernel, over the row's scores in registers
// of its four waves -- with the block table entries of all candidate ids read beside the scores, so
// the page ids of the chosen blocks are on chip as soon as the selection is.  Split 0 also writes
// the row's selection, count, page table and row length; then every split attends to its run of
// pages exactly as k_attn_decode does.  The row's few hundred scores are read by each of its splits
// instead of once, which costs far less than the launch and the page-table round trip it saves.
// Caches of 128-token pages with Hkv*D-element token rows, page p at p*P elements: the view of KV head
// g has page stride D and token stride Hkv*D, and the virtual page of physical page p is p*vps + g
// with vps = P / D (128*Hkv for back-to-back pages).
template <int D, int R>  // R scores per thread: max_blocks <= 256*R
__global__ __launch_bounds__(256, 2) void k_select_attend(
    int B, int Hkv, int max_blocks, const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int k,
    int32_t* __restrict__ sel, int32_t* __restrict__ cnt, int32_t* __restrict__ page_table,
    int32_t* __restrict__ row_len, int vps, int G, const bf16* __restrict__ q, const bf16* __restrict__ kcache,
    const bf16* __restrict__ vcache, float scale_log2, int ppw, int nsplit, bf16* __restrict__ out,
    float* __restrict__ lse_out, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    uint32_t* __restrict__ counters) {
  constexpr int NW = 4, NT = 256;
  __shared__ DecodeLds<D> sm;
  __shared__ RowTopkLds<NW> sh;
  __shared__ int s_sel[64], s_pt[64], s_len;
  const int sp = (int)(blockIdx.x % (unsigned)nsplit), rho = (int)(blockIdx.x / (unsigned)nsplit);
  const int t = rho / Hkv, g = rho - t * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int pos = q_pos[t];
  const int n = min(pos / kBlock + 1, max_blocks);
  const float* srow = scores + (int64_t)rho * max_blocks;
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = srow[min(tid + NT * r, max_blocks - 1)];
  int r_req, L;
  request_and_len(cu_q, ctx_len, B, t, r_req, L);
  const int lim = min(pos + 1, L);  // tokens s < lim are valid
  int bt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) bt[r] = block_table[(int64_t)r_req * max_blocks + min(tid + NT * r, max_blocks - 1)];

  const int c = row_topk<NW, R>(v, n, k, sh, [&](int slot, int id, int r) {
    s_sel[slot] = id;
    s_pt[slot] = bt[r] * vps + g;
  });
  __syncthreads();
  if (wv == 0) {
    int len = lane < c ? min(kBlock, lim - s_sel[lane] * kBlock) : 0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) len += __shfl_xor(len, m, kWave);
    if (lane == 0) s_len = len;
    if (sp == 0) {
      if (lane < k) {
        sel[(int64_t)rho * k + lane] = lane < c ? s_sel[lane] : -1;
        page_table[(int64_t)rho * k + lane] = lane < c ? s_pt[lane] : -1;
      }
      if (lane == 0) {
        cnt[rho] = c;
        row_len[rho] = len;
      }
    }
  }
  __syncthreads();
  const PagesInLds pages{s_pt};
  attend_run<D>(sm, G, q, kcache, vcache, D, (int64_t)Hkv * D, pages, s_len, rho, sp, ppw, nsplit, scale_log2, out,
                lse_out, ws_o, ws_lse, counters);
}

// Merge of the decode splits: one workgroup per (row, head).  Thread (g, c) folds the parts
// g, g + NG, ... of the 4-float chunk c into a running (max, sum, O); the NG folds of each chunk
// are then combined through LDS.  Every thread's loads are independent of the other threads',
// so even a few rows with many splits spread over the whole chip.  A part whose LSE is -inf
// has weight 0 and is read from part 0 instead (split 0 always holds the row's first page).
template <int D>
__global__ __launch_bounds__(256) void k_merge_splits(int parts, int G, const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, bf16* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  constexpr int NC = D / 4;     // 4-float chunks per head
  constexpr int NG = 256 / NC;  // part groups
  __shared__ float s_m[NG][NC], s_s[NG][NC];
  __shared__ f32x4 s_o[NG][NC];
  const int64_t rh = blockIdx.x;  // row * G + head
  const int64_t row = rh / G;
  const int h = (int)(rh - row * G);
  const int c = threadIdx.x % NC, g = threadIdx.x / NC;
  const float* pl = part_lse + row * parts * G + h;
  const float* po = part_o + (row * parts * G + h) * D + 4 * c;
  float m = neg_inf(), sum = 0.f;
  f32x4 o = fzero4();
#pragma unroll 4
  for (int j = g; j < parts; j += NG) {
    const float x = pl[(int64_t)j * G];
    const bool use = x != neg_inf();
    const f32x4 v = *reinterpret_cast<const f32x4*>(po + (int64_t)(use ? j : 0) * G * D);
    const float mn = fmaxf(m, x);
    const float a = (m == neg_inf()) ? 0.f : __expf(m - mn);
    const float wj = use ? __expf(x - mn) : 0.f;
    sum = sum * a + wj;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = o[e] * a + wj * v[e];
    m = mn;
  }
  s_m[g][c] = m;
  s_s[g][c] = sum;
  s_o[g][c] = o;
  __syncthreads();
  if (g == 0) {
    float M = neg_inf();
#pragma unroll
    for (int t = 0; t < NG; ++t) M = fmaxf(M, s_m[t][c]);
    float den = 0.f;
    f32x4 acc = fzero4();
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      const float mt = s_m[t][c];
      const float f = (mt == neg_inf()) ? 0.f : __expf(mt - M);
      den += f * s_s[t][c];
      const f32x4 ot = s_o[t][c];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += f * ot[e];
    }
    const float inv = 1.f / den;
    uint2 pk;
    pk.x = pack_bf2(acc[0] * inv, acc[1] * inv);
    pk.y = pack_bf2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(out + rh * D + 4 * c) = pk;
    if (lse_out && c == 0) lse_out[rh] = M + __logf(den);
  }
}

// One wavefront per row.  Lanes 0..G-1 turn the row's parts*G log-sum-exps into normalized
// weights w[j][h] = exp(lse_j - LSE) in LDS (0 for absent parts) and note each head's first
// present part.  Then every lane combines its 8-element chunks (up to four per lane) over the
// parts in batches of eight, all of a batch's 16-byte loads issued together and streamed past
// the caches.  An absent part is read from the head's first present part instead (finite values,
// weight 0), so no load depends on a branch.
constexpr int kMergeMaxPG = 64 * 16;  // parts * G
constexpr int kMergeBatch = 8;

template <typename TIn>
__global__ __launch_bounds__(256) void k_lse_merge(int64_t rows, int parts, int G, int D,
                                                   const TIn* __restrict__ part_o, const float* __restrict__ part_lse,
                                                   bf16* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float s_w[4][kMergeMaxPG];
  __shared__ float s_lse[4][16];
  __shared__ int s_first[4][16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  const int PG = parts * G, GD = G * D, NCH = GD / 8;
  float* w = s_w[wv];
  const float* pl = part_lse + row * PG;
  if (lane < G) {  // per head: LSE, the normalized weights and the first present part
    float M = neg_inf();
    int first = -1;
    for (int j = 0; j < parts; ++j) {
      const float lj = pl[j * G + lane];
      M = fmaxf(M, lj);
      if (first < 0 && lj != neg_inf()) first = j;
    }
    float den = 0.f;
    for (int j = 0; j < parts; ++j) {
      const float lj = pl[j * G + lane];
      den += lj == neg_inf() ? 0.f : __expf(lj - M);
    }
    const float inv = 1.f / den;
    for (int j = 0; j < parts; ++j) {
      const float lj = pl[j * G + lane];
      w[j * G + lane] = lj == neg_inf() ? 0.f : __expf(lj - M) * inv;
    }
    s_lse[wv][lane] = M + __logf(den);  // -inf when no part is present
    s_first[wv][lane] = max(first, 0);  // no present part: every weight is 0, reads stay in the row
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const TIn* src = part_o + (row * parts) * (int64_t)GD;
  for (int c = lane; c < NCH; c += kWave) {
    const int h = (8 * c) / D;
    const int jp = s_first[wv][h];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int jb = 0; jb < parts; jb += kMergeBatch) {
      float wj[kMergeBatch];
      int jj[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int j = jb + u;
        wj[u] = j < parts ? w[j * G + h] : 0.f;
        jj[u] = (j < parts && wj[u] != 0.f) ? j : jp;
      }
      if constexpr (sizeof(TIn) == 2) {
        u32x4 v[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) v[u] = ld16_nt(src + (int64_t)jj[u] * GD + 8 * c);
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += wj[u] * __uint_as_float(v[u][e] << 16);
            acc[2 * e + 1] += wj[u] * __uint_as_float(v[u][e] & 0xffff0000u);
          }
      } else {
        f32x4 v0[kMergeBatch], v1[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          v0[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)jj[u] * GD + 8 * c);
          v1[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)jj[u] * GD + 8 * c + 4);
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] += wj[u] * v0[u][e];
            acc[4 + e] += wj[u] * v1[u][e];
          }
      }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf2(acc[2 * e], acc[2 * e + 1]);
    st16(out + (row * G) * (int64_t)D + 8 * c, o);
  }
  if (lse_out && lane < G) lse_out[row * G + lane] = s_lse[wv][lane];
}

#ifndef MSA_DECODE_FUSED_MERGE_MAX
#define MSA_DECODE_FUSED_MERGE_MAX 8
#endif
// Rows split at most this many ways are merged by their last split inside the attention launch (one
// batch of part loads per thread); more splits take the separate merge kernel, which spreads a row's
// merge over G workgroups instead of looping over the parts in one.
constexpr int kFusedMergeMax = MSA_DECODE_FUSED_MERGE_MAX;

int decode_splits(int rows, int k) {
  int nsplit = std::min(k, std::max(1, (MSA_DECODE_TARGET_WGS + rows - 1) / rows));
  const int ppw = (k + nsplit - 1) / nsplit;
  return (k + ppw - 1) / ppw;
}

static hipError_t launch_merge_splits(int rows, int G, int D, int nsplit, const float* ws_o, const float* ws_lse,
                                      bf16* out, float* lse, hipStream_t stream) {
  const dim3 mgrid((unsigned)((int64_t)rows * G));
  if (D == 128)
    hipLaunchKernelGGL(k_merge_splits<128>, mgrid, dim3(256), 0, stream, nsplit, G, ws_o, ws_lse, out, lse);
  else
    hipLaunchKernelGGL(k_merge_splits<64>, mgrid, dim3(256), 0, stream, nsplit, G, ws_o, ws_lse, out, lse);
  return hipGetLastError();
}

hipError_t launch_attn_decode(int rows, int G, int D, const void* q, const void* kview, const void* vview,
                              int64_t page_stride, int64_t token_stride, const int32_t* page_table, int k,
                              const int32_t* row_len, float sm_scale, void* out, float* lse, float* ws_o,
                              float* ws_lse, uint32_t* counters, hipStream_t stream) {
  const int nsplit = decode_splits(rows, k);
  const int ppw = (k + nsplit - 1) / nsplit;
  const bool fused = nsplit <= kFusedMergeMax;
  dim3 grid((unsigned)((int64_t)nsplit * rows)), block(256);
  const float sl2 = sm_scale * kLog2e;
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kk = static_cast<const bf16*>(kview);
  const bf16* vv = static_cast<const bf16*>(vview);
  bf16* oo = static_cast<bf16*>(out);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_decode<128>, grid, block, 0, stream, G, qq, kk, vv, page_stride, token_stride,
                       page_table, k, row_len, sl2, ppw, nsplit, oo, lse, ws_o, ws_lse, fused ? counters : nullptr);
  else
    hipLaunchKernelGGL(k_attn_decode<64>, grid, block, 0, stream, G, qq, kk, vv, page_stride, token_stride,
                       page_table, k, row_len, sl2, ppw, nsplit, oo, lse, ws_o, ws_lse, fused ? counters : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1 || fused) return e;
  return launch_merge_splits(rows, G, D, nsplit, ws_o, ws_lse, oo, lse, stream);
}

// Beyond 4096 blocks per row the selection repeated by every split of a row costs as much as the
// separate top-k kernel (measured on million-token rows), so those rows keep the two launches.
int select_attend_max_blocks() { return 256 * 16; }

// Top-k + page table + decode attention (split merge included) in one launch; max_blocks must be
// at most select_attend_max_blocks().  Same splits, pages and arithmetic as the separate calls.
hipError_t launch_select_attend(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                                const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const float* scores,
                                int k, int32_t* sel, int32_t* cnt, int32_t* page_table, int32_t* row_len, int vps,
                                int G, int D, const void* q, const void* kcache, const void* vcache, float sm_scale,
                                void* out, float* lse, float* ws_o, float* ws_lse, uint32_t* counters,
                                hipStream_t stream) {
  const int rows = Nq * Hkv;
  const int nsplit = decode_splits(rows, k);
  const int ppw = (k + nsplit - 1) / nsplit;
  const bool fused = nsplit <= kFusedMergeMax;
  const dim3 grid((unsigned)((int64_t)nsplit * rows)), block(256);
  const float sl2 = sm_scale * kLog2e;
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kc = static_cast<const bf16*>(kcache);
  const bf16* vc = static_cast<const bf16*>(vcache);
  bf16* oo = static_cast<bf16*>(out);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, B, Hkv, max_blocks, block_table, ctx_len, cu_q, q_pos, scores, k,
                       sel, cnt, page_table, row_len, vps, G, qq, kc, vc, sl2, ppw, nsplit, oo, lse, ws_o, ws_lse,
                       fused ? counters : nullptr);
  };
  const int r = max_blocks <= 256 ? 1 : max_blocks <= 512 ? 2 : max_blocks <= 1024 ? 4 : max_blocks <= 2048 ? 8 : 16;
  if (D == 128) {
    if (r == 1) go(k_select_attend<128, 1>);
    else if (r == 2) go(k_select_attend<128, 2>);
    else if (r == 4) go(k_select_attend<128, 4>);
    else if (r == 8) go(k_select_attend<128, 8>);
    else go(k_select_attend<128, 16>);
  } else {
    if (r == 1) go(k_select_attend<64, 1>);
    else if (r == 2) go(k_select_attend<64, 2>);
    else if (r == 4) go(k_select_attend<64, 4>);
    else if (r == 8) go(k_select_attend<64, 8>);
    else go(k_select_attend<64, 16>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1 || fused) return e;
  return launch_merge_splits(rows, G, D, nsplit, ws_o, ws_lse, oo, lse, stream);
}

// Split partials and row arrival counters of msa_topk_attn_decode_noalloc, for callers that cannot
// allocate device memory.  One copy of this array lives on every GPU the library runs on, for the life
// of the process.  It starts zeroed (static storage), every call returns the counters it used to zero,
// and every split writes its own LSE (-inf for a split past its row's last page) before the merge
// reads it, so nothing has to be cleared between calls.
constexpr size_t kDecodeScratchBytes = MSA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

// Device address of the current device's copy of `scratch`, looked up once per device with that
// device current.  In host code the array's name is only a host-side stand-in, never a device address.
hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_lse_merge_bf16(int64_t rows, int parts, int G, int D, const void* part_o, const float* part_lse,
                                 void* out, float* lse_out, hipStream_t stream) {
  const int64_t wgs = (rows + 3) / 4;
  hipLaunchKernelGGL(k_lse_merge<bf16>, dim3((unsigned)wgs), dim3(256), 0, stream, rows, parts, G, D,
                     static_cast<const bf16*>(part_o), part_lse, static_cast<bf16*>(out), lse_out);
  return hipGetLastError();
}

}  // namespace msa
