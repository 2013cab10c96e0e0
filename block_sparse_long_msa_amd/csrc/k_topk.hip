// Top-k over KV blocks per (query row, KV head), and the decode sparse page table.
//
// Top-k (Chinese page of the MiniMax-M3 serving write-up, sections "MiniMax稀疏注意力改变了服务问题"
// and "遗留问题"): the k best candidate blocks by score; equal scores prefer the lower block
// id; output in ascending block id with -1 padding.  One wavefront per row runs a radix
// select on order-preserving 32-bit keys: it skips the bits every candidate shares, then
// takes 8-bit digits from the top with an LDS histogram per pass, stopping as soon as the
// boundary digit's bucket is taken whole.  A final in-order ballot pass writes the chosen
// ids, which gives ascending order and the lower-id tie rule for free.
#include "msa_device.h"

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

// Decode sparse page table over the strided view (Chinese page, section "MSA需要新的分页注意力集成"):
// row rho = t*Hkv + g, page_table[rho, j] = block_table[r, sel[t,g,j]] * 128 * Hkv + g.
// One wavefront per row; lane j handles slot j (k <= 64), row_len is a wave sum.
__global__ __launch_bounds__(256) void k_page_table(int rows, int B, int Hkv, int max_blocks,
                                                    const int32_t* __restrict__ block_table,
                                                    const int32_t* __restrict__ ctx_len,
                                                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos,
                                                    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
                                                    int k, int32_t* __restrict__ page_table,
                                                    int32_t* __restrict__ row_len) {
  const int rho = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int j = threadIdx.x & 63;
  if (rho >= rows) return;
  const int t = rho / Hkv, g = rho % Hkv;
  const int r = request_of(cu_q, B, t);
  const int lim = min(q_pos[t] + 1, ctx_len[r]);  // tokens s < lim are valid
  const int c = cnt[rho];
  int v = -1, len = 0;
  if (j < c) {
    const int bl = sel[(int64_t)rho * k + j];
    v = block_table[(int64_t)r * max_blocks + bl] * (kBlock * Hkv) + g;
    len = min(kBlock, lim - bl * kBlock);
  }
  if (j < k) page_table[(int64_t)rho * k + j] = v;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) len += __shfl_xor(len, m, kWave);
  if (j == 0) row_len[rho] = len;
}

hipError_t launch_topk(int B, int Nq, int Hkv, int max_blocks, const int32_t* cu_q, const int32_t* q_pos,
                       const float* scores, int k, int32_t* sel, int32_t* cnt, hipStream_t stream) {
  // few long rows: a workgroup of up to 16 waves per row; many rows: one wave each
  const int rows = Nq * Hkv;
  const int want = rows >= 4096 ? 1 : (max_blocks >= 4096 ? 16 : (max_blocks >= 1024 ? 4 : 1));
  if (want == 16)
    hipLaunchKernelGGL(k_topk<16>, dim3(rows), dim3(1024), 0, stream, B, Hkv, max_blocks, cu_q, q_pos, scores, k,
                       sel, cnt);
  else if (want == 4)
    hipLaunchKernelGGL(k_topk<4>, dim3(rows), dim3(256), 0, stream, B, Hkv, max_blocks, cu_q, q_pos, scores, k, sel,
                       cnt);
  else
    hipLaunchKernelGGL(k_topk<1>, dim3(rows), dim3(64), 0, stream, B, Hkv, max_blocks, cu_q, q_pos, scores, k, sel,
                       cnt);
  return hipGetLastError();
}

hipError_t launch_page_table(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                             const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const int32_t* sel,
                             const int32_t* cnt, int k, int32_t* page_table, int32_t* row_len, hipStream_t stream) {
  const int rows = Nq * Hkv;
  hipLaunchKernelGGL(k_page_table, dim3((rows + 3) / 4), dim3(256), 0, stream, rows, B, Hkv, max_blocks,
                     block_table, ctx_len, cu_q, q_pos, sel, cnt, k, page_table, row_len);
  return hipGetLastError();
}

}  // namespace msa
