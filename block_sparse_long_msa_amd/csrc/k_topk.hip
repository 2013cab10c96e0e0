// Top-k over KV blocks per (query row, KV head), and the decode sparse page table.
//
// Top-k (Chinese page of the MiniMax-M3 serving write-up, sections "MiniMax稀疏注意力改变了服务问题"
// and "遗留问题"): the k best candidate blocks by score; equal scores prefer the lower block
// id; output in ascending block id with -1 padding.  Both kernels work on order-preserving
// 32-bit keys and end with an in-order ballot pass that writes the chosen ids, which gives
// ascending order and the lower-id tie rule for free.
//   k_topk_reg (rows of up to 16384 blocks): the row sits in registers and the k-th largest key
//     is found by bisection with ballot counts; the scores are read once.  The selection itself is
//     row_topk (topk_select.h), shared with the fused decode select + attend kernel.
//   k_topk (longer rows): radix select; it skips the bits every candidate shares, then takes
//     8-bit digits from the top with an LDS histogram per pass, stopping as soon as the boundary
//     digit's bucket is taken whole.
#include <type_traits>

#include "msa_device.h"
#include "topk_select.h"

namespace msa {

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_topk(int B, int Hkv, int max_blocks, const int32_t* __restrict__ cu_q,
                                                  const int32_t* __restrict__ q_pos, const float* __restrict__ scores,
                                                  int k, int32_t* __restrict__ sel, int32_t* __restrict__ cnt) {
  constexpr int NT = 64 * NW;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_red[2][NW];
  __shared__ uint32_t s_cnt[2][NW];
  __shared__ int s_bc[3];
  const int row = blockIdx.x;  // t*Hkv + g
  const int t = row / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = min(q_pos[t] / kBlock + 1, max_blocks);
  const float* s = scores + (int64_t)row * max_blocks;
  int32_t* out = sel + (int64_t)row * k;

  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    if (tid == 0) cnt[row] = n;
    return;
  }

  // bits shared by every candidate key need no pass
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = order_key(s[i]);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, kWave));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, kWave));
  }
  if (NW > 1) {
    if (lane == 0) { s_red[0][wv] = kmin; s_red[1][wv] = kmax; }
    __syncthreads();
    for (int x = 0; x < NW; ++x) { kmin = min(kmin, s_red[0][x]); kmax = max(kmax, s_red[1][x]); }
  }
  uint32_t prefix, mask;
  int remaining = k;
  if (kmin == kmax) {
    prefix = kmin;
    mask = 0xffffffffu;
  } else {
    const int hb = 31 - __builtin_clz(kmin ^ kmax);  // highest differing bit
    mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    prefix = kmin & mask;
    int top = hb;  // next digit covers bits [top-7, top] (clamped at bit 0)
    while (top >= 0) {
      const int lo = max(top - 7, 0);
      const int width = top - lo + 1;
      const uint32_t dmask = ((1u << width) - 1u);
      for (int i = tid; i < 256; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = order_key(s[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> lo) & dmask], 1u);
      }
      __syncthreads();
      if (wv == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending); an inclusive scan over lanes gives
        // the number of keys whose digit is at least a given value
        uint32_t c[4], local = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; local += c[j]; }
        uint32_t incl = local;
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
          const uint32_t o = (uint32_t)__shfl_up((int)incl, m, kWave);
          if (lane >= m) incl += o;
        }
        uint32_t before = incl - local;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (before < (uint32_t)remaining && before + c[j] >= (uint32_t)remaining) {
            s_bc[0] = 255 - 4 * lane - j;   // exactly one lane and digit cross the boundary
            s_bc[1] = (int)before;
            s_bc[2] = (int)c[j];
          }
          before += c[j];
        }
      }
      __syncthreads();
      const int digit = s_bc[0], gt = s_bc[1], eq = s_bc[2];
      remaining -= gt;
      prefix |= ((uint32_t)digit) << lo;
      mask |= dmask << lo;
      __syncthreads();
      if (eq == remaining) break;  // the whole boundary bucket is taken
      top = lo - 1;
    }
  }

  // emit in id order: keys above the boundary, then the first `remaining` boundary ties
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int written = 0, ties_seen = 0;
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    const uint32_t hk = (i < n) ? (order_key(s[i]) & mask) : 0u;
    const bool gt = i < n && hk > prefix;
    const bool eq = i < n && hk == prefix;
    const uint64_t eqm = __ballot(eq);
    int eq_before = ties_seen + __popcll(eqm & lt_mask);
    int eq_all = __popcll(eqm);
    if (NW > 1) {
      if (lane == 0) s_cnt[0][wv] = eq_all;
      __syncthreads();
      eq_all = 0;
      for (int x = 0; x < NW; ++x) {
        if (x < wv) eq_before += s_cnt[0][x];
        eq_all += s_cnt[0][x];
      }
    }
    const bool take = gt || (eq && eq_before < remaining);
    const uint64_t tm = __ballot(take);
    int slot = written + __popcll(tm & lt_mask);
    int take_all = __popcll(tm);
    if (NW > 1) {
      if (lane == 0) s_cnt[1][wv] = take_all;
      __syncthreads();
      take_all = 0;
      for (int x = 0; x < NW; ++x) {
        if (x < wv) slot += s_cnt[1][x];
        take_all += s_cnt[1][x];
      }
      __syncthreads();  // s_cnt is rewritten by the next chunk
    }
    if (take && slot < k) out[slot] = i;
    written += take_all;
    ties_seen += eq_all;
  }
  written = min(written, k);
  for (int i = written + tid; i < k; i += NT) out[i] = -1;
  if (tid == 0) cnt[row] = written;
}

// The same selection for rows whose candidates fit in registers (64*NW*R >= n): every lane
// reads its R scores once and row_topk (topk_select.h) finds the k-th largest key bit by bit with
// ballot counts.  Against the radix passes it saves the re-reads of the scores and the LDS
// histogram round trips.  With TL (the longest register rows) the selection is two-level
// (row_topk_two_level): each wave takes the top k of its own run of ids without a workgroup barrier
// per trial bit, and wave 0 the top k of those candidates.
//
// With page_table != NULL the same launch also writes the row's decode page table and row length
// (as k_page_table below), from the chosen ids kept in LDS; the request lookup is issued at the
// start so that it overlaps the score loads.
struct PageTableOut {
  int B;
  const int32_t* block_table;
  const int32_t* ctx_len;
  const int32_t* cu_q;
  int32_t* page_table;  // NULL: top-k only
  int32_t* row_len;
  int vps;              // virtual pages per physical page: the cache's page stride / D
};

template <int NW, int R, bool TL>
__global__ __launch_bounds__(64 * NW) void k_topk_reg(int Hkv, int max_blocks, const int32_t* __restrict__ q_pos,
                                                      const float* __restrict__ scores, int k,
                                                      int32_t* __restrict__ sel, int32_t* __restrict__ cnt,
                                                      PageTableOut pto) {
  constexpr int NT = 64 * NW;
  __shared__ std::conditional_t<TL, RowTopk2Lds<NW>, RowTopkLds<NW>> sh;
  __shared__ int s_sel[64];
  const int row = blockIdx.x;  // t*Hkv + g
  const int t = row / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int pos = q_pos[t];
  const int n = min(pos / kBlock + 1, max_blocks);
  const float* s = scores + (int64_t)row * max_blocks;
  int32_t* out = sel + (int64_t)row * k;
  // id i = tid + NT*r (TL: wv*64*R + lane + 64*r).  All R loads are unconditional (clamped to the
  // row's max_blocks entries) and go out together with the row's position and the request lookup
  // for the page table.
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = s[min(TL ? wv * 64 * R + lane + 64 * r : tid + NT * r, max_blocks - 1)];
  int r_req = 0, lim = 0;
  if (pto.page_table) {
    int L;
    request_and_len(pto.cu_q, pto.ctx_len, pto.B, t, r_req, L);
    lim = min(pos + 1, L);  // tokens s < lim are valid
  }
#pragma unroll
  for (int r = 0; r < R; ++r) asm volatile("" ::"v"(v[r]));

  auto keep = [&](int slot, int id) {
    out[slot] = id;
    s_sel[slot] = id;
  };
  int c;
  if constexpr (TL) c = row_topk_two_level<NW, R>(v, n, k, sh, keep);
  else c = row_topk<NW, R>(v, n, k, sh, [&](int slot, int id, int) { keep(slot, id); });
  for (int i = c + tid; i < k; i += NT) out[i] = -1;
  if (tid == 0) cnt[row] = c;
  if (pto.page_table) {  // the chosen ids, in ascending order, are in s_sel[0 .. c-1]
    __syncthreads();
    if (wv == 0) {
      const int g = row - t * Hkv;
      int pv = -1, len = 0;
      if (lane < c) {
        const int bl = s_sel[lane];
        pv = pto.block_table[(int64_t)r_req * max_blocks + bl] * pto.vps + g;
        len = min(kBlock, lim - bl * kBlock);
      }
      if (lane < k) pto.page_table[(int64_t)row * k + lane] = pv;
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) len += __shfl_xor(len, m, kWave);
      if (lane == 0) pto.row_len[row] = len;
    }
  }
}

// Decode sparse page table over the strided view (Chinese page, section "MSA需要新的分页注意力集成"):
// row rho = t*Hkv + g, page_table[rho, j] = block_table[r, sel[t,g,j]] * vps + g, vps = the cache's
// page stride / D (128 * Hkv for back-to-back pages).
// One wavefront per row; lane j handles slot j (k <= 64), row_len is a wave sum.
__global__ __launch_bounds__(256) void k_page_table(int rows, int B, int Hkv, int max_blocks,
                                                    const int32_t* __restrict__ block_table,
                                                    const int32_t* __restrict__ ctx_len,
                                                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
                                                    int k, int vps, int32_t* __restrict__ page_table,
                                                    int32_t* __restrict__ row_len) {
  const int rho = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int j = threadIdx.x & 63;
  if (rho >= rows) return;
  const int t = rho / Hkv, g = rho % Hkv;
  int r, L;
  request_and_len(cu_q, ctx_len, B, t, r, L);
  const int lim = min(q_pos[t] + 1, L);  // tokens s < lim are valid
  const int c = cnt[rho];
  int v = -1, len = 0;
  if (j < c) {
    const int bl = sel[(int64_t)rho * k + j];
    v = block_table[(int64_t)r * max_blocks + bl] * vps + g;
    len = min(kBlock, lim - bl * kBlock);
  }
  if (j < k) page_table[(int64_t)rho * k + j] = v;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) len += __shfl_xor(len, m, kWave);
  if (j == 0) row_len[rho] = len;
}

// Rows of 8193 to 16384 blocks (16 waves, 16 scores per lane) select in two levels: top-k plus page
// table 30.6 -> 20.5 us on two 11,719-block rows (events, bit-identical).  With 8 scores per lane the
// one-level search is as fast or faster (8192 blocks: 14.7 / 14.9 us against 14.4 / 15.6 us at one and
// four requests; 4 waves x 8: 11.6 against 12.6 us), so those layouts keep it.
template <int NW, int R>
static void launch_reg(int rows, hipStream_t stream, int Hkv, int max_blocks, const int32_t* q_pos,
                       const float* scores, int k, int32_t* sel, int32_t* cnt, const PageTableOut& pto) {
  constexpr bool TL = NW == 16 && R == 16;
  hipLaunchKernelGGL((k_topk_reg<NW, R, TL>), dim3(rows), dim3(64 * NW), 0, stream, Hkv, max_blocks, q_pos, scores,
                     k, sel, cnt, pto);
}

// Top-k, and with pto.page_table set also the decode page table.  Returns false (nothing
// launched) when the shape needs the radix kernel, which does not build page tables.
static bool launch_topk_reg(int rows, int Hkv, int max_blocks, const int32_t* q_pos, const float* scores, int k,
                            int32_t* sel, int32_t* cnt, const PageTableOut& pto, hipStream_t stream) {
  if (max_blocks > 16384) return false;
  // the smallest register layout that holds a row: 64*NW*R >= max_blocks
  auto go = [&](auto nw, auto r) {
    launch_reg<decltype(nw)::value, decltype(r)::value>(rows, stream, Hkv, max_blocks, q_pos, scores, k, sel, cnt,
                                                        pto);
  };
  using std::integral_constant;
  if (max_blocks <= 64) go(integral_constant<int, 1>(), integral_constant<int, 1>());
  else if (max_blocks <= 128) go(integral_constant<int, 1>(), integral_constant<int, 2>());
  else if (max_blocks <= 256) go(integral_constant<int, 1>(), integral_constant<int, 4>());
  else if (max_blocks <= 512) go(integral_constant<int, 1>(), integral_constant<int, 8>());
  else if (max_blocks <= 1024) go(integral_constant<int, 1>(), integral_constant<int, 16>());
  else if (max_blocks <= 2048) go(integral_constant<int, 4>(), integral_constant<int, 8>());
  else if (max_blocks <= 4096) go(integral_constant<int, 4>(), integral_constant<int, 16>());
  else if (max_blocks <= 8192) go(integral_constant<int, 16>(), integral_constant<int, 8>());
  else go(integral_constant<int, 16>(), integral_constant<int, 16>());
  return true;
}

hipError_t launch_topk(int B, int Nq, int Hkv, int max_blocks, const int32_t* cu_q, const int32_t* q_pos,
                       const float* scores, int k, int32_t* sel, int32_t* cnt, hipStream_t stream) {
  const int rows = Nq * Hkv;
  const PageTableOut none{B, nullptr, nullptr, cu_q, nullptr, nullptr, 0};
  if (launch_topk_reg(rows, Hkv, max_blocks, q_pos, scores, k, sel, cnt, none, stream)) return hipGetLastError();
  // rows longer than the register layouts: radix passes, 16 waves per row when the rows are few
  if (rows < 4096)
    hipLaunchKernelGGL(k_topk<16>, dim3(rows), dim3(1024), 0, stream, B, Hkv, max_blocks, cu_q, q_pos, scores, k,
                       sel, cnt);
  else
    hipLaunchKernelGGL(k_topk<1>, dim3(rows), dim3(64), 0, stream, B, Hkv, max_blocks, cu_q, q_pos, scores, k, sel,
                       cnt);
  return hipGetLastError();
}

hipError_t launch_page_table(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                             const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const int32_t* sel,
                             const int32_t* cnt, int k, int vps, int32_t* page_table, int32_t* row_len,
                             hipStream_t stream) {
  const int rows = Nq * Hkv;
  hipLaunchKernelGGL(k_page_table, dim3((rows + 3) / 4), dim3(256), 0, stream, rows, B, Hkv, max_blocks,
                     block_table, ctx_len, cu_q, q_pos, sel, cnt, k, vps, page_table, row_len);
  return hipGetLastError();
}

hipError_t launch_topk_page_table(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                                  const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos,
                                  const float* scores, int k, int32_t* sel, int32_t* cnt, int vps,
                                  int32_t* page_table, int32_t* row_len, hipStream_t stream) {
  const PageTableOut pto{B, block_table, ctx_len, cu_q, page_table, row_len, vps};
  if (launch_topk_reg(Nq * Hkv, Hkv, max_blocks, q_pos, scores, k, sel, cnt, pto, stream)) return hipGetLastError();
  hipError_t e = launch_topk(B, Nq, Hkv, max_blocks, cu_q, q_pos, scores, k, sel, cnt, stream);
  if (e != hipSuccess) return e;
  return launch_page_table(B, Nq, Hkv, max_blocks, block_table, ctx_len, cu_q, q_pos, sel, cnt, k, vps, page_table,
                           row_len, stream);
}

}  // namespace msa
