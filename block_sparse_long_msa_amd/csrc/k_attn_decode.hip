// Decode attention over the sparse per-row page table, and the log-sum-exp merge.
//
// Rows are (query row, KV head) pairs with the KV-group dimension folded into the batch;
// each row reads its selected pages through a strided view of the shared paged KV tensor
// (virtual page v at v*page_stride, tokens every token_stride elements) -- Chinese page of
// the MiniMax-M3 serving write-up, section "MSA需要新的分页注意力集成".
//
// k_attn_decode: one workgroup per (row, page); the four waves take 32 tokens each.
//   S^T = K Q^T on bf16 MFMA with the tokens as M and the G query heads padded into N.
//   P stays in the MFMA result registers and feeds O^T = V^T P^T directly as the B operand of
//   an fp32 16x16x4 MFMA: lane (n, q) holds P for tokens 4q+i, and loads the matching V row
//   as 16 contiguous bytes, whose 8 values become the A operand of 8 MFMAs (output row m of
//   MFMA c is d = 8m + c).  No LDS transpose, no shuffles, every V row read as whole
//   64-byte segments.  The four waves' (max, sum, O) are combined through LDS and written as
//   one fp32 partial per (row, page).
// k_lse_merge: LSE = log sum_j exp(lse_j); O = sum_j exp(lse_j - LSE) O_j over the parts with
//   lse_j > -inf (section "KV块主序稀疏注意力减少冗余KV移动").
#include "msa_device.h"

namespace msa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(256) void k_attn_decode(
    int G, const bf16* __restrict__ q, const bf16* __restrict__ kview, const bf16* __restrict__ vview,
    int64_t page_stride, int64_t token_stride, const int32_t* __restrict__ page_table, int k,
    const int32_t* __restrict__ row_len, float scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  constexpr int KW = D / 32;
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ float sm_o[4][16][D];
  const int j = blockIdx.x, rho = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, qd = lane >> 4;
  const int len = row_len[rho];
  const int npages = (len + kBlock - 1) / kBlock;
  const int64_t part = (int64_t)rho * k + j;
  if (j >= npages) {
    if (tid < G) ws_lse[part * G + tid] = neg_inf();
    return;
  }
  const int64_t vpage = page_table[part];
  const bf16* kb = kview + vpage * page_stride;
  const bf16* vb = vview + vpage * page_stride;
  const int valid = min(kBlock, len - j * kBlock);

  u32x4 qf[KW];
#pragma unroll
  for (int kw = 0; kw < KW; ++kw)
    qf[kw] = (n < G) ? ld16(q + ((int64_t)rho * G + n) * D + 32 * kw + 8 * qd) : zero4();

  // V rows this lane needs: token 32w + 16sub + 4qd + i, elements 8n .. 8n+7
  u32x4 vr[2][4];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 16 * sub + 4 * qd + i;
      vr[sub][i] = (tok < valid && 8 * n < D) ? ld16_nt(vb + (int64_t)tok * token_stride + 8 * n) : zero4();
    }

  f32x4 s[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int tok = 32 * w + 16 * sub + n;
    s[sub] = fzero4();
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) {
      const u32x4 a = (tok < valid) ? ld16_nt(kb + (int64_t)tok * token_stride + 32 * kw + 8 * qd) : zero4();
      s[sub] = mfma_bf16(a, qf[kw], s[sub]);
    }
  }
  // s[sub][i] = S[token 32w + 16sub + 4qd + i][head n]
  float m = neg_inf();
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 16 * sub + 4 * qd + i;
      const float x = (tok < valid) ? s[sub][i] * scale_log2 : neg_inf();
      s[sub][i] = x;
      m = fmaxf(m, x);
    }
  m = max_over_quads(m);
  float l = 0.f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (m == neg_inf()) ? 0.f : fast_exp2(s[sub][i] - m);
      s[sub][i] = p;
      l += p;
    }
  l = sum_over_quads(l);

  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = fzero4();
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = vr[sub][i];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t word = v[c >> 1];
        const float vf = (c & 1) ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
        acc[c] = mfma_f32(vf, s[sub][i], acc[c]);
      }
    }
  // acc[c][ii] = O_w[head n][d = 32qd + 8ii + c]
  if (qd == 0) { sm_m[w][n] = m; sm_l[w][n] = l; }
  if (n < G) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int d = 32 * qd + 8 * ii + c;
        if (d < D) sm_o[w][n][d] = acc[c][ii];
      }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e % D;
    float M = neg_inf();
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sm_m[ww][h];
      const float f = (mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      num += f * sm_o[ww][h][d];
      den += f * sm_l[ww][h];
    }
    ws_o[(part * G + h) * D + d] = num / den;
    if (d == 0) ws_lse[part * G + h] = (M + fast_log2(den)) * kLn2;
  }
}

// One wavefront per row.  The row's parts*G log-sum-exps go to LDS and become normalized
// weights w[j][h] = exp(lse_j - LSE) once; then every lane accumulates its 8-element chunks over
// the parts with independent 16-byte loads (absent parts have weight 0 and are not read).
constexpr int kMergeMaxPG = 64 * 16;  // parts * G

template <typename TIn>
__global__ __launch_bounds__(256) void k_lse_merge(int64_t rows, int parts, int G, int D,
                                                   const TIn* __restrict__ part_o, const float* __restrict__ part_lse,
                                                   bf16* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float s_w[4][kMergeMaxPG];
  __shared__ float s_lse[4][16];
  __shared__ int s_parts[4][64];
  __shared__ int s_np[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  const int PG = parts * G, GD = G * D;
  float* w = s_w[wv];
  const float* pl = part_lse + row * PG;
  for (int i = lane; i < PG; i += kWave) w[i] = pl[i];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (lane < G) {  // per head: LSE and the normalization
    float M = neg_inf();
    for (int j = 0; j < parts; ++j) M = fmaxf(M, w[j * G + lane]);
    float den = 0.f;
    for (int j = 0; j < parts; ++j) {
      const float lj = w[j * G + lane];
      den += lj == neg_inf() ? 0.f : __expf(lj - M);
    }
    const float inv = 1.f / den;
    for (int j = 0; j < parts; ++j) {
      const float lj = w[j * G + lane];
      w[j * G + lane] = lj == neg_inf() ? 0.f : __expf(lj - M) * inv;
    }
    s_lse[wv][lane] = M + __logf(den);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // compact list of the parts present for at least one head (lane j tests part j; parts <= 64)
  bool present = false;
  if (lane < parts)
    for (int h = 0; h < G; ++h) present = present || (pl[lane * G + h] != neg_inf());
  const uint64_t pm = __ballot(present);
  if (present) s_parts[wv][__popcll(pm & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))))] = lane;
  const int np = __popcll(pm);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int* plist = s_parts[wv];
  for (int c = lane; c < GD / 8; c += kWave) {
    const int h = (8 * c) / D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const TIn* src = part_o + (row * parts) * (int64_t)GD + 8 * c;
#pragma unroll 4
    for (int q = 0; q < np; ++q) {
      const int j = plist[q];
      const float wj = w[j * G + h];
      const bool use = wj != 0.f;  // a part absent for this head only: its values are never used
      if constexpr (sizeof(TIn) == 2) {
        const u32x4 v = ld16(src + (int64_t)j * GD);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += use ? wj * __uint_as_float(v[e] << 16) : 0.f;
          acc[2 * e + 1] += use ? wj * __uint_as_float(v[e] & 0xffff0000u) : 0.f;
        }
      } else {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src + (int64_t)j * GD);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + (int64_t)j * GD + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] += use ? wj * v0[e] : 0.f;
          acc[4 + e] += use ? wj * v1[e] : 0.f;
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

hipError_t launch_attn_decode(int rows, int G, int D, const void* q, const void* kview, const void* vview,
                              int64_t page_stride, int64_t token_stride, const int32_t* page_table, int k,
                              const int32_t* row_len, float sm_scale, float* ws_o, float* ws_lse,
                              hipStream_t stream) {
  dim3 grid(k, rows), block(256);
  const float sl2 = sm_scale * kLog2e;
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kk = static_cast<const bf16*>(kview);
  const bf16* vv = static_cast<const bf16*>(vview);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_decode<128>, grid, block, 0, stream, G, qq, kk, vv, page_stride, token_stride,
                       page_table, k, row_len, sl2, ws_o, ws_lse);
  else
    hipLaunchKernelGGL(k_attn_decode<64>, grid, block, 0, stream, G, qq, kk, vv, page_stride, token_stride,
                       page_table, k, row_len, sl2, ws_o, ws_lse);
  return hipGetLastError();
}

hipError_t launch_lse_merge_bf16(int64_t rows, int parts, int G, int D, const void* part_o, const float* part_lse,
                                 void* out, float* lse_out, hipStream_t stream) {
  const int64_t wgs = (rows + 3) / 4;
  hipLaunchKernelGGL(k_lse_merge<bf16>, dim3((unsigned)wgs), dim3(256), 0, stream, rows, parts, G, D,
                     static_cast<const bf16*>(part_o), part_lse, static_cast<bf16*>(out), lse_out);
  return hipGetLastError();
}

hipError_t launch_lse_merge_f32(int64_t rows, int parts, int G, int D, const float* part_o, const float* part_lse,
                                void* out, float* lse_out, hipStream_t stream) {
  const int64_t wgs = (rows + 3) / 4;
  hipLaunchKernelGGL(k_lse_merge<float>, dim3((unsigned)wgs), dim3(256), 0, stream, rows, parts, G, D, part_o,
                     part_lse, static_cast<bf16*>(out), lse_out);
  return hipGetLastError();
}

}  // namespace msa
