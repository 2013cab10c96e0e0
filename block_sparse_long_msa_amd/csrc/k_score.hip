// Stage 1 of MSA: block index scores.
//
// score[t, g, b] = max over the valid tokens s of block b of q_idx[t, g] . k_idx[s, g]
// (the max is this library's reading of "each 128-token block is reduced to one score",
// Chinese page of the MiniMax-M3 serving write-up, section "索引评分器成为解码关键路径").
//
// Kernels, picked by queries per request:
//  * decode (at most 16 queries per request): the 128-token key-index block is the MFMA M
//    dimension and the request's queries are padded only into N -- the AB-swapped layout the
//    pages describe for the decode scorer -- and each page of the key-index cache is read
//    exactly once per request.
//    - k_score_decode_lds (Hkv * Di <= 1024, the usual case): a workgroup streams consecutive
//      blocks of one request through a double-buffered LDS stage with fully coalesced loads.
//    - k_score_decode (larger rows): one workgroup per (request, block), loading straight from
//      HBM into MFMA operand registers (every 16-lane group reads whole 64-byte segments).
//  * k_score_prefill: one workgroup per (512 or 256 query rows, KV head).  A GEMM over the causal
//    range, staging each key-index block in LDS once for 256 queries whose index vectors
//    stay in registers, with the per-block max fused into the epilogue so that token-level
//    scores never reach memory.  With TOPK > 0 the same kernel keeps each row's top-k on chip
//    instead of writing scores (msa_index_topk).
#include <type_traits>

#include "msa_device.h"

#ifndef MSA_SCORE_PREFETCH
#define MSA_SCORE_PREFETCH 2
#endif
#ifndef MSA_SCORE_BPW
#define MSA_SCORE_BPW 2
#endif

namespace msa {

constexpr int kScoreBPW = MSA_SCORE_BPW;  // key-index blocks per workgroup of the staged decode scorer

// Operands of one KV head for the decode scorer: the wave's two 16-token key-index tiles and
// the (zero-padded) query index fragments.
template <int KW>
struct DecodeFrags {
  u32x4 a[2][KW];
  u32x4 b[KW];
};

template <int DI>
__device__ __forceinline__ void load_decode_frags(DecodeFrags<DI / 32>& f, const bf16* __restrict__ ka,
                                                  const bf16* __restrict__ qa, int g, int Hkv, uint32_t qmask) {
  constexpr int KW = DI / 32;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) f.a[sub][kw] = ld16_nt(ka + ((int64_t)(16 * sub) * Hkv + g) * DI + 32 * kw);
#pragma unroll
  for (int kw = 0; kw < KW; ++kw) {
    u32x4 v = ld16(qa + (int64_t)g * DI + 32 * kw);
    f.b[kw] = v & qmask;  // padded query columns contribute zeros, without a branch
  }
}

template <int DI>
__global__ __launch_bounds__(256) void k_score_decode(
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos, const bf16* __restrict__ q_idx,
    const bf16* __restrict__ kidx, int Hkv, int64_t kpage, float* __restrict__ scores) {
  constexpr int KW = DI / 32;
  constexpr int PF = MSA_SCORE_PREFETCH;  // KV heads in flight ahead of the one being multiplied
  __shared__ float red[4][64][16];
  const int b = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, qd = lane >> 4;
  const int q0 = cu_q[r], nq = cu_q[r + 1] - q0, L = ctx_len[r];

  for (int qc = 0; qc < nq; qc += 16) {
    const int nqc = min(16, nq - qc);
    const bool qvalid = n < nqc;
    const int my_t = q0 + qc + (qvalid ? n : 0);  // padded lanes read a real row, then mask it
    const int pos = qvalid ? q_pos[my_t] : -1;
    const uint32_t qmask = qvalid ? 0xffffffffu : 0u;
    int maxpos = pos;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) maxpos = max(maxpos, __shfl_xor(maxpos, m, kWave));

    if (b * kBlock > maxpos) {  // not a candidate of any query in this chunk
      for (int e = tid; e < nqc * Hkv; e += 256) {
        const int t = q0 + qc + e / Hkv, g = e % Hkv;
        scores[((int64_t)t * Hkv + g) * max_blocks + b] = neg_inf();
      }
      continue;
    }
    const int page = block_table[(int64_t)r * max_blocks + b];
    // lane (n, qd): A rows are tokens 32w + 16sub + n, k chunk 8qd within each 32-wide window
    const bf16* ka = kidx + (int64_t)page * kpage + (int64_t)(32 * w + n) * Hkv * DI + 8 * qd;
    const bf16* qa = q_idx + (int64_t)my_t * Hkv * DI + 8 * qd;
    const int tok_base = b * kBlock + 32 * w + 4 * qd;

    DecodeFrags<KW> ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < Hkv) load_decode_frags<DI>(ring[p], ka, qa, p, Hkv, qmask);

    for (int g0 = 0; g0 < Hkv; g0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int g = g0 + p;
        if (g < Hkv) {
          const DecodeFrags<KW> cur = ring[p];
          if (g + PF < Hkv) load_decode_frags<DI>(ring[p], ka, qa, g + PF, Hkv, qmask);
          float m = neg_inf();
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            f32x4 acc = fzero4();
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) acc = mfma_bf16(cur.a[sub][kw], cur.b[kw], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int s = tok_base + 16 * sub + i;
              m = (s <= pos && s < L) ? fmaxf(m, acc[i]) : m;
            }
          }
          m = max_over_quads(m);
          if (qd == 0) red[w][g][n] = m;
        }
      }
    }
    __syncthreads();
    for (int e = tid; e < nqc * Hkv; e += 256) {
      const int qq = e / Hkv, g = e % Hkv;
      const float v = fmaxf(fmaxf(red[0][g][qq], red[1][g][qq]), fmaxf(red[2][g][qq], red[3][g][qq]));
      scores[((int64_t)(q0 + qc + qq) * Hkv + g) * max_blocks + b] = v;
    }
    __syncthreads();
  }
}

// LDS-staged decode scorer, used when one 16-token slice of a page (16 * Hkv * Di * 2 bytes) fits a
// 32 KiB stage, i.e. Hkv * Di <= 1024.  A workgroup takes kScoreBPW consecutive blocks of one
// request and streams their context slices as one sequence with fully coalesced 16-byte
// non-temporal loads (each wave instruction reads 1 KiB of consecutive bytes), two slices ahead in
// registers, into a double-buffered LDS stage whose token rows are padded by 16 bytes so that the
// MFMA operand reads (16 token rows, same column) are bank-conflict free.  Every load and LDS store
// of the stream is unconditional (indices past the end are clamped to the last slice, which is then
// read again and never used), so the wait before a store covers exactly the slice being stored and
// the next slice stays in flight.  Wave w owns KV heads w, w+4, ...: it reads their operands from LDS
// and keeps their running block max in registers, so no cross-wave reduction is needed.
//
// Slices are chosen by the request's context length; token positions past a query's own position
// are masked in the max (with queries at the end of the context, as in decode, nothing is read
// that no query uses).
constexpr int kStageBytes = 32768;
constexpr int kStageLdsBytes = 16 * 16 + kStageBytes;  // + 16 B pad per token row
constexpr int kSlicesPerBlock = kBlock / 16;

template <int DI>
__global__ __launch_bounds__(256, 2) void k_score_decode_lds(
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos, const bf16* __restrict__ q_idx,
    const bf16* __restrict__ kidx, int Hkv, int64_t kpage, float* __restrict__ scores) {
  constexpr int KW = DI / 32;
  constexpr int GPW = 256 / DI;           // KV heads per wave at most (Hkv * DI <= 1024)
  constexpr int LPT = kStageBytes / 16 / 256;  // 16-byte loads per thread per slice (8)
  __shared__ __attribute__((aligned(16))) unsigned char stage[2][kStageLdsBytes];
  const int r = blockIdx.y, b0 = blockIdx.x * kScoreBPW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 15, qd = lane >> 4;
  // independent loads first: the query range, the context length and the blocks' page ids
  const int q0 = cu_q[r], nq = cu_q[r + 1] - q0, L = ctx_len[r];
  int page[kScoreBPW];
#pragma unroll
  for (int bi = 0; bi < kScoreBPW; ++bi) page[bi] = block_table[(int64_t)r * max_blocks + min(b0 + bi, max_blocks - 1)];
  const int RB = Hkv * DI * 2;            // bytes per token row (all KV heads)
  const int RBP = RB + 16;                // padded LDS row
  const int slice_bytes = 16 * RB;
  // blocks of this workgroup (nblk) and those holding context tokens (nb); slices to stream (S)
  const int nblk = min(kScoreBPW, max_blocks - b0);
  const int nb = L > 0 ? max(0, min(nblk, (L - 1) / kBlock - b0 + 1)) : 0;
  const int S = nb > 0 ? kSlicesPerBlock * (nb - 1) + min(L - 1 - (b0 + nb - 1) * kBlock, kBlock - 1) / 16 + 1 : 0;

  // this thread's 16-byte pieces of a slice: clamped offsets, so tails read (and store) the last piece again
  int soff[LPT], loff[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int off = min(16 * (tid + 256 * u), slice_bytes - 16);
    soff[u] = off;
    loff[u] = (off / RB) * RBP + off % RB;
  }
  auto slice_src = [&](int gs) {  // global slice gs (clamped by the caller) of the stream
    const int bi = gs / kSlicesPerBlock, sl = gs % kSlicesPerBlock;
    int pg = page[0];
#pragma unroll
    for (int j = 1; j < kScoreBPW; ++j) pg = bi == j ? page[j] : pg;
    return reinterpret_cast<const unsigned char*>(kidx) + ((int64_t)pg * kpage * 2 + (int64_t)sl * slice_bytes);
  };
  auto load_slice = [&](u32x4 (&reg)[LPT], int gs) {
    const unsigned char* src = slice_src(min(gs, S - 1));
#pragma unroll
    for (int u = 0; u < LPT; ++u) reg[u] = ld16_nt(src + soff[u]);
  };
  auto store_slice = [&](const u32x4 (&reg)[LPT], int buf) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) st16(&stage[buf][loff[u]], reg[u]);
  };

  for (int qc = 0; qc < nq; qc += 16) {
    const int nqc = min(16, nq - qc);
    for (int e = tid; e < (nblk - nb) * nqc * Hkv; e += 256) {  // blocks with no context token
      const int bi = nb + e / (nqc * Hkv), t = q0 + qc + (e / Hkv) % nqc, g = e % Hkv;
      scores[((int64_t)t * Hkv + g) * max_blocks + b0 + bi] = neg_inf();
    }
    if (S == 0) continue;
    const bool qvalid = n < nqc;
    const int my_t = q0 + qc + (qvalid ? n : 0);
    const uint32_t qmask = qvalid ? 0xffffffffu : 0u;

    // query operands first, so that the wait for slice 0 below also covers them
    u32x4 qf[GPW][KW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = w + 4 * gi;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw)  // unconditional loads (clamped head), zeroed by mask: no branch per load
        qf[gi][kw] = ld16(q_idx + ((int64_t)my_t * Hkv + min(g, Hkv - 1)) * DI + 32 * kw + 8 * qd) &
                     (g < Hkv ? qmask : 0u);
    }
    const int pos_t = q_pos[my_t];  // unconditional (padded lanes read a real row)
    asm volatile("" ::"v"(pos_t));
    const int pos = qvalid ? pos_t : -1;
    float mx[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) mx[gi] = neg_inf();

    u32x4 regs[2][LPT];
    load_slice(regs[0], 0);
    load_slice(regs[1], 1);
    // a request with more than 16 queries runs this loop again: the previous chunk's last slices
    // may still be read from both stage buffers by slower waves
    if (qc > 0) __syncthreads();
    store_slice(regs[0], 0);
    load_slice(regs[0], 2);
    __syncthreads();

    auto compute = [&](int gs, int buf) {  // slice gs, staged in stage[buf]
      const int bi = gs / kSlicesPerBlock, sl = gs % kSlicesPerBlock;
      const int b = b0 + bi;
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = w + 4 * gi;
        if (g < Hkv) {
          f32x4 acc = fzero4();
#pragma unroll
          for (int kw = 0; kw < KW; ++kw) {
            const u32x4 a = ld16(&stage[buf][n * RBP + g * DI * 2 + 64 * kw + 16 * qd]);
            acc = mfma_bf16(a, qf[gi][kw], acc);
          }
          const int s0 = b * kBlock + 16 * sl + 4 * qd;
#pragma unroll
          for (int i = 0; i < 4; ++i) mx[gi] = (s0 + i <= pos && s0 + i < L) ? fmaxf(mx[gi], acc[i]) : mx[gi];
        }
      }
      if (sl == kSlicesPerBlock - 1 || gs == S - 1) {  // the block's last slice: write its scores
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
          const int g = w + 4 * gi;
          const float m = max_over_quads(mx[gi]);
          if (g < Hkv && qd == 0 && qvalid) scores[((int64_t)(q0 + qc + n) * Hkv + g) * max_blocks + b] = m;
          mx[gi] = neg_inf();
        }
      }
    };
    // after compute(gs, buf): stage the next slice (held in reg) and, if asked, load slice `next` into reg
    auto advance = [&](int buf, u32x4 (&reg)[LPT], int next) {
      __syncthreads();  // stage[buf ^ 1] (slice gs - 1) is no longer read
      store_slice(reg, buf ^ 1);
      if (next >= 0) load_slice(reg, next);
      __syncthreads();
    };
    // Main loop: at the top, stage[0] holds slice gs and regs[1], regs[0] hold (or are loading)
    // slices gs + 1 and gs + 2.  Every step loads a slice that exists, so the outstanding loads are
    // in the same order on every path into the loop head.
    int gs = 0;
    for (; gs + 4 < S; gs += 2) {
      compute(gs, 0);
      advance(0, regs[1], gs + 3);
      compute(gs + 1, 1);
      advance(1, regs[0], gs + 4);
    }
    // the last R = S - gs (1..4) slices; only slice gs + 3 (if R = 4) remains to be loaded
    const int R = S - gs;
    compute(gs, 0);
    if (R > 1) advance(0, regs[1], R == 4 ? gs + 3 : -1);
    if (R > 1) compute(gs + 1, 1);
    if (R > 2) advance(1, regs[0], -1);
    if (R > 2) compute(gs + 2, 0);
    if (R > 3) advance(0, regs[1], -1);
    if (R > 3) compute(gs + 3, 1);
  }
}

// Waves per workgroup of the prefill scorer, 64 query rows each: 8 (one workgroup per CU, each staged
// block serving 512 rows) when the launch has a workgroup for every CU, else 4 (256 rows, two
// workgroups per CU), so that short prompts still spread over the chip.
constexpr int kPrefWideW = 8, kPrefNarrowW = 4;
constexpr int kPrefWideMinWgs = 256;
constexpr int kPrefSB = 16;   // blocks buffered per score flush
constexpr int kPrefTargetWgs = 512;  // a split score launch aims for two workgroups per CU
constexpr int kFusedTopK = 16;  // largest k the fused scorer + top-k keeps per row

// Slot swizzle of the staged key-index rows: logical 16-byte chunk c of token row `row` is stored at
// chunk slot c ^ kidx_slot(row).  An MFMA operand read takes the same chunk of 16 consecutive rows;
// with the swizzle those 16 reads cover all 64 LDS banks.  DI = 128 (256-byte rows, 16 slots): the
// row's low four bits.  DI = 64 (128-byte rows, two rows per bank cycle): rows of equal parity get
// distinct slots.
template <int DI>
__device__ __forceinline__ int kidx_slot(int row) {
  return DI == 128 ? (row & 15) : ((row >> 1) & 7);
}

// Bitonic networks over N (a power of two) 64-bit keys held in registers, larger keys first.
__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  const bool sw = a < b;
  const uint64_t hi = sw ? b : a, lo = sw ? a : b;
  a = hi;
  b = lo;
}
template <int N>
__device__ __forceinline__ void bitonic_merge_desc(uint64_t (&v)[N]) {  // v bitonic -> sorted
#pragma unroll
  for (int stride = N / 2; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & stride) == 0) cas_desc(v[i], v[i + stride]);
}
template <int N>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&v)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if ((i & stride) == 0) {
          if ((i & size) == 0) cas_desc(v[i], v[i + stride]);  // this run descending
          else cas_desc(v[i + stride], v[i]);                  // this run ascending
        }
}

// TOPK == 0: write the block scores.  TOPK > 0: fused top-k (k <= TOPK = 16).  Thread t of the
// workgroup adopts local row t and keeps that row's best 16 candidates in registers, as 64-bit keys
// (order-preserving score bits above the complement of the block id, so a larger key is a higher
// score or, at equal scores, a lower block id -- the library's tie rule), sorted best first.  The
// block maxima are buffered in LDS as for the score output; every 16 blocks each thread sorts its
// row's 16 new keys with a bitonic network, keeps the larger of kept[i] and new[15 - i] (the best 16
// of both lists, a bitonic sequence) and re-sorts them with a bitonic merge.  The work is the same
// for every row, so no lane waits on another's insertions.  The result equals msa_topk_blocks applied
// to the written scores.
//
// nsplit > 1 (TOPK == 0 only): the blocks a row tile needs are cut into nsplit contiguous runs, one
// workgroup per run, so that small problems still fill the chip.  A block's scores do not depend on
// the run that computes them; the first run also writes the -inf tail.
template <int DI, int TOPK, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void k_score_prefill(
    int B, int Nq, const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ q_pos, const bf16* __restrict__ q_idx,
    const bf16* __restrict__ kidx, int Hkv, int64_t kpage, float* __restrict__ scores, int k,
    int32_t* __restrict__ sel,
    int32_t* __restrict__ cnt, int nsplit) {
  constexpr int kPrefThreads = 64 * W;
  constexpr int kPrefTQ = kPrefThreads;  // query rows per workgroup (64 per wave, one per thread)
  constexpr int KW = DI / 32;
  constexpr int BLKE = kBlock * DI;  // elements of one staged key-index block
  constexpr int CPR = DI / 8;        // 16-byte chunks per token row
  constexpr int kLoadsPerWave = kBlock * CPR / 64 / W;  // 64-chunk loads per wave per block
  // Two buffers (the next block arrives while the current one is multiplied) of unpadded token rows
  // in 16-byte chunks, swizzled by kidx_slot, plus the score buffer: 96 KiB at DI = 128 with eight
  // waves (one workgroup per CU), 80 KiB with four (two per CU).  The score buffer's first words also
  // carry the position reduction.
  __shared__ __attribute__((aligned(16))) bf16 ks[2][BLKE];
  __shared__ float sbuf[kPrefTQ][kPrefSB];
  int* wred = reinterpret_cast<int*>(&sbuf[0][0]);

  const int g = blockIdx.x % Hkv;  // consecutive workgroups take consecutive KV heads
  const int split = (int)(blockIdx.x / Hkv) % nsplit;
  // Row tiles go from the last to the first: a request's later rows have longer causal ranges, so
  // the longest tiles start first and the short ones fill the end of the launch.
  const int row0 = ((int)gridDim.x / (Hkv * nsplit) - 1 - (int)blockIdx.x / (Hkv * nsplit)) * kPrefTQ;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, qd = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int last_row = min(row0 + kPrefTQ, Nq) - 1;
  const int r_first = request_of(cu_q, B, row0), r_last = request_of(cu_q, B, last_row);
  // Eight waves: waves w and w + 4 share a SIMD.  The first of each pair issues first whenever both are
  // ready, so the pair drifts out of step and one's MFMA bursts overlap the other's operand reads and
  // maxima instead of both waiting on the same LDS reads (measured: 3-5% on the long prefill; with
  // four waves per workgroup the two waves of a SIMD belong to different workgroups and it lost).
  if (W == 8 && w < 4) __builtin_amdgcn_s_setprio(1);

  for (int r = r_first; r <= r_last; ++r) {
    const int qa = max(row0, cu_q[r]), qb = min(row0 + kPrefTQ, cu_q[r + 1]);
    if (qa >= qb) continue;  // uniform across the workgroup
    const int L = ctx_len[r];

    u32x4 qf[4][KW];
    int pos[4];
    int pmax = -1, pmin = 0x7fffffff;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int row = row0 + 64 * w + 16 * nt + n;
      const bool in = row >= qa && row < qb;
      pos[nt] = in ? q_pos[row] : -1;
      if (in) { pmax = max(pmax, pos[nt]); pmin = min(pmin, pos[nt]); }
#pragma unroll
      for (int kw = 0; kw < KW; ++kw)
        qf[nt][kw] = ld16(q_idx + ((int64_t)(in ? row : qa) * Hkv + g) * DI + 32 * kw + 8 * qd) &
                     (in ? 0xffffffffu : 0u);  // rows outside the request read a valid row, zeroed
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      pmax = max(pmax, __shfl_xor(pmax, m, kWave));
      pmin = min(pmin, __shfl_xor(pmin, m, kWave));
    }
    __syncthreads();  // the previous request's flush has read sbuf, which wred overlays
    if (lane == 0) { wred[w] = pmax; wred[W + w] = pmin; }
    __syncthreads();
    pmax = wred[0];
    pmin = wred[W];
#pragma unroll
    for (int i = 1; i < W; ++i) {
      pmax = max(pmax, wred[i]);
      pmin = min(pmin, wred[W + i]);
    }
    const int nb = pmax / kBlock + 1;  // blocks needed by at least one row

    // fused top-k state (TOPK > 0) of local row tid: its last candidate block and its best keys
    const int arow = row0 + tid;
    const int my_last = (TOPK > 0 && arow >= qa && arow < qb) ? q_pos[arow] / kBlock : -1;
    constexpr int TK = TOPK > 0 ? TOPK : 1;
    uint64_t kept[TK];
#pragma unroll
    for (int j = 0; j < TK; ++j) kept[j] = 0;  // 0 ranks below every candidate key

    // Block bb goes straight from HBM into LDS buffer buf (global_load_lds_dwordx4: each lane's 16
    // bytes land at the LDS address in m0 plus 16 * lane).  Load i of wave w fills the 64 chunks of
    // group 4i + w, i.e. 64 / CPR whole token rows: lane l loads, for row grp * 64 / CPR + l / CPR, the
    // logical chunk that belongs in slot p = l % CPR, which is chunk p ^ kidx_slot(row).
    //
    // The loads are issued from inline assembly so that the compiler's wait-count pass does not see
    // them: it cannot tell the two buffers apart and would wait for these loads before the first
    // read of the buffer being multiplied.  The waits are explicit instead: a wave's loads of block
    // b are complete at the s_waitcnt that precedes the barrier opening block b, and the next block's
    // loads are issued only after that barrier, when no wave reads their buffer any more.  The LDS
    // address goes through m0, which the assembly saves and restores; s_nop 0 gives the one wait
    // state an LDS DMA needs after m0 is written, and one more before m0 is written back.
    auto issue_block = [&](int bb, int buf) {
      const int page = block_table[(int64_t)r * max_blocks + bb];
      const bf16* kb = kidx + (int64_t)page * kpage + (int64_t)g * DI;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int grp = W * i + w;                         // wave-uniform group of 64 chunks
        const int row = grp * (64 / CPR) + lane / CPR, p = lane % CPR;
        const bf16* src = kb + (int64_t)row * Hkv * DI + 8 * (p ^ kidx_slot<DI>(row));
        const uint32_t dst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)(&ks[buf][grp * 64 * 8]);
        uint32_t m0_saved;  // m0 is left as the compiler had it
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
            "s_nop 0\n\ts_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "s"(dst), "v"(src)
            : "memory");
      }
    };
    // this workgroup's run of the needed blocks (all of them unless split); uniform per workgroup
    const int per = (nb + nsplit - 1) / nsplit;
    const int lo = min(nb, split * per), hi = min(nb, lo + per);
    if (lo < hi) issue_block(lo, lo & 1);
    for (int b0 = lo; b0 < hi; b0 += kPrefSB) {
      const int b1 = min(b0 + kPrefSB, hi);
      for (int b = b0; b < b1; ++b) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of block b are in LDS
        __syncthreads();  // every wave's are, and no wave reads the other buffer any more
        if (b + 1 < hi) issue_block(b + 1, (b & 1) ^ 1);
        const bf16* kbuf = ks[b & 1];
        // operand of 16-token tile mt, k window kw for lane (n, qd): row 16mt + n, logical chunk 4kw + qd
        auto frag = [&](int mt, int kw) {
          const int row = 16 * mt + n;
          return ld16(&kbuf[row * DI + (((4 * kw + qd) ^ kidx_slot<DI>(row)) << 3)]);
        };

        // full blocks (every key valid for every row) take the unmasked body; the branch is uniform
        const bool full = (b * kBlock + kBlock - 1 <= pmin) && (b * kBlock + kBlock - 1 < L);
        float mx[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
        auto block_body = [&](auto masked) {
          constexpr bool MASKED = decltype(masked)::value;
          u32x4 a_cur[KW];
#pragma unroll
          for (int kw = 0; kw < KW; ++kw) a_cur[kw] = frag(0, kw);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            u32x4 a_nxt[KW];  // next 16-token tile's operands, read while this one multiplies
            if (mt < 7) {
#pragma unroll
              for (int kw = 0; kw < KW; ++kw) a_nxt[kw] = frag(mt + 1, kw);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              f32x4 acc = fzero4();
#pragma unroll
              for (int kw = 0; kw < KW; ++kw) acc = mfma_bf16(a_cur[kw], qf[nt][kw], acc);
              if constexpr (!MASKED) {
                mx[nt] = fmaxf(fmaxf(mx[nt], fmaxf(acc[0], acc[1])), fmaxf(acc[2], acc[3]));
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int s = b * kBlock + 16 * mt + 4 * qd + i;
                  mx[nt] = (s <= pos[nt] && s < L) ? fmaxf(mx[nt], acc[i]) : mx[nt];
                }
              }
            }
            if (mt < 7) {
#pragma unroll
              for (int kw = 0; kw < KW; ++kw) a_cur[kw] = a_nxt[kw];
            }
          }
          // Full blocks: the block's MFMAs, operand reads and maxima issue in a fixed interleave, four
          // MFMAs then one LDS read then two VALU instructions, so that every operand read and block
          // max sits between MFMAs instead of in bursts (long prefill, bit-identical scores: 5.00 ->
          // 4.82 ms alone, 5.19 -> 5.04 ms with the fused top-k; groups of 4/1/1, 2/1/1, 2/1/2, 4/1/3
          // and 8/2/4 were slower or no better).
          if constexpr (!MASKED) {
#pragma unroll
            for (int i = 0; i < 8 * 4 * KW / 4; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
            }
          }
        };
        if (full) block_body(std::false_type{});
        else block_body(std::true_type{});
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float v = max_over_quads(mx[nt]);
          if (qd == 0) sbuf[64 * w + 16 * nt + n][b - b0] = v;
        }
      }
      __syncthreads();
      if constexpr (TOPK == 0) {
        // flush: 16 consecutive threads write 16 consecutive blocks of one row
        for (int it = 0; it < kPrefTQ / (kPrefThreads / 16); ++it) {
          const int lrow = it * (kPrefThreads / 16) + (tid >> 4), bb = tid & 15, row = row0 + lrow, b = b0 + bb;
          if (row >= qa && row < qb && b < b1) scores[((int64_t)row * Hkv + g) * max_blocks + b] = sbuf[lrow][bb];
        }
      } else {
        static_assert(TOPK == kPrefSB, "one bitonic merge per flush of 16 blocks");
        uint64_t nk[TK];
#pragma unroll
        for (int j = 0; j < TK; ++j) {
          const int b = b0 + j;
          const bool cand = b < b1 && b <= my_last;
          nk[j] = cand ? ((uint64_t)order_key(sbuf[tid][j]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)b) : 0ull;
        }
        bitonic_sort_desc<TK>(nk);
#pragma unroll
        for (int j = 0; j < TK; ++j) kept[j] = kept[j] > nk[TK - 1 - j] ? kept[j] : nk[TK - 1 - j];
        bitonic_merge_desc<TK>(kept);
      }
    }
    if constexpr (TOPK == 0) {
      // non-candidate tail, written by the first run
      const int tail = split == 0 ? max_blocks - nb : 0;
      for (int e = tid; e < (qb - qa) * tail; e += kPrefThreads) {
        const int row = qa + e / tail, b = nb + e % tail;
        scores[((int64_t)row * Hkv + g) * max_blocks + b] = neg_inf();
      }
    } else if (arow >= qa && arow < qb) {
      // the first min(k, candidates) keys, as block ids in ascending order
      const int c = min(k, my_last + 1);
      int ids[TK];
#pragma unroll
      for (int j = 0; j < TK; ++j) ids[j] = j < c ? (int)(0xffffffffu - (uint32_t)kept[j]) : 0x7fffffff;
#pragma unroll
      for (int a = 0; a < TK; ++a)  // ascending block ids (odd-even transposition sort)
#pragma unroll
        for (int j = a & 1; j + 1 < TK; j += 2) {
          const int lo = min(ids[j], ids[j + 1]), hi = max(ids[j], ids[j + 1]);
          ids[j] = lo;
          ids[j + 1] = hi;
        }
      int32_t* out = sel + ((int64_t)arow * Hkv + g) * k;
#pragma unroll
      for (int j = 0; j < TK; ++j)
        if (j < k) out[j] = j < c ? ids[j] : -1;
      cnt[(int64_t)arow * Hkv + g] = c;
    }
    __syncthreads();
  }
}

hipError_t launch_score_decode(int B, int Di, const int32_t* block_table, int max_blocks, const int32_t* ctx_len,
                               const int32_t* cu_q, const int32_t* q_pos, const void* q_idx, const void* kidx,
                               int Hkv, int64_t kpage, float* scores, hipStream_t stream) {
  dim3 grid(max_blocks, B), block(256);
  const bf16* qi = static_cast<const bf16*>(q_idx);
  const bf16* ki = static_cast<const bf16*>(kidx);
  if (Hkv * Di <= 1024) {
    grid.x = (max_blocks + kScoreBPW - 1) / kScoreBPW;
    if (Di == 128)
      hipLaunchKernelGGL(k_score_decode_lds<128>, grid, block, 0, stream, block_table, max_blocks, ctx_len, cu_q,
                         q_pos, qi, ki, Hkv, kpage, scores);
    else
      hipLaunchKernelGGL(k_score_decode_lds<64>, grid, block, 0, stream, block_table, max_blocks, ctx_len, cu_q,
                         q_pos, qi, ki, Hkv, kpage, scores);
    return hipGetLastError();
  }
  if (Di == 128)
    hipLaunchKernelGGL(k_score_decode<128>, grid, block, 0, stream, block_table, max_blocks, ctx_len, cu_q, q_pos,
                       qi, ki, Hkv, kpage, scores);
  else
    hipLaunchKernelGGL(k_score_decode<64>, grid, block, 0, stream, block_table, max_blocks, ctx_len, cu_q, q_pos,
                       qi, ki, Hkv, kpage, scores);
  return hipGetLastError();
}

namespace {

// Workgroup shape and row tiles of a prefill scorer launch: eight waves when the 512-row tiles give
// every CU a workgroup, else four.
struct PrefillShape {
  int waves, tiles;
};
PrefillShape prefill_shape(int Nq, int Hkv) {
  const int wide = (Nq + 64 * kPrefWideW - 1) / (64 * kPrefWideW);
  if ((int64_t)wide * Hkv >= kPrefWideMinWgs) return {kPrefWideW, wide};
  return {kPrefNarrowW, (Nq + 64 * kPrefNarrowW - 1) / (64 * kPrefNarrowW)};
}

template <int TOPK, int W, typename... Args>
void launch_prefill(int Di, dim3 grid, hipStream_t stream, Args... args) {
  if (Di == 128)
    hipLaunchKernelGGL((k_score_prefill<128, TOPK, W>), grid, dim3(64 * W), 0, stream, args...);
  else
    hipLaunchKernelGGL((k_score_prefill<64, TOPK, W>), grid, dim3(64 * W), 0, stream, args...);
}

}  // namespace

hipError_t launch_score_prefill(int B, int Nq, int Di, const int32_t* block_table, int max_blocks,
                                const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const void* q_idx,
                                const void* kidx, int Hkv, int64_t kpage, float* scores, hipStream_t stream) {
  const PrefillShape sh = prefill_shape(Nq, Hkv);
  // Few row tiles (short prompts): cut each tile's blocks into runs, doubling the runs while the
  // launch stays within kPrefTargetWgs workgroups and there are blocks for every run.
  int nsplit = 1;
  while ((int64_t)sh.tiles * Hkv * nsplit * 2 <= kPrefTargetWgs && nsplit * 2 <= max_blocks) nsplit *= 2;
  const dim3 grid(sh.tiles * Hkv * nsplit);
  const bf16* qi = static_cast<const bf16*>(q_idx);
  const bf16* ki = static_cast<const bf16*>(kidx);
  int32_t* none = nullptr;
  if (sh.waves == kPrefWideW)
    launch_prefill<0, kPrefWideW>(Di, grid, stream, B, Nq, block_table, max_blocks, ctx_len, cu_q, q_pos, qi, ki, Hkv,
                                  kpage, scores, 0, none, none, nsplit);
  else
    launch_prefill<0, kPrefNarrowW>(Di, grid, stream, B, Nq, block_table, max_blocks, ctx_len, cu_q, q_pos, qi, ki,
                                    Hkv, kpage, scores, 0, none, none, nsplit);
  return hipGetLastError();
}

int fused_topk_capacity() { return kFusedTopK; }

hipError_t launch_score_topk_prefill(int B, int Nq, int Di, const int32_t* block_table, int max_blocks,
                                     const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos,
                                     const void* q_idx, const void* kidx, int Hkv, int64_t kpage, int k, int32_t* sel,
                                     int32_t* cnt, hipStream_t stream) {
  const PrefillShape sh = prefill_shape(Nq, Hkv);
  const dim3 grid(sh.tiles * Hkv);
  const bf16* qi = static_cast<const bf16*>(q_idx);
  const bf16* ki = static_cast<const bf16*>(kidx);
  float* none = nullptr;
  if (sh.waves == kPrefWideW)
    launch_prefill<kFusedTopK, kPrefWideW>(Di, grid, stream, B, Nq, block_table, max_blocks, ctx_len, cu_q, q_pos,
                                           qi, ki, Hkv, kpage, none, k, sel, cnt, 1);
  else
    launch_prefill<kFusedTopK, kPrefNarrowW>(Di, grid, stream, B, Nq, block_table, max_blocks, ctx_len, cu_q, q_pos,
                                             qi, ki, Hkv, kpage, none, k, sel, cnt, 1);
  return hipGetLastError();
}

}  // namespace msa
