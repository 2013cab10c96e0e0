// Top-k selection of one row held in registers by one workgroup, shared by the top-k kernel and the
// fused decode select + attend kernel.
//
// The rule is the library's: the min(n, k) highest scores among the row's n candidates, equal scores
// preferring the lower block id, chosen ids reported in ascending order.  The k-th largest key T is
// found bit by bit from the highest bit the keys do not all share, counting the keys at or above each
// trial threshold with ballots; the search stops as soon as exactly k keys clear the threshold.  T is
// then a threshold with at least k keys >= T and fewer than k keys > T, so the boundary ties are
// taken in id order.
#pragma once

#include "msa_device.h"

namespace msa {

template <int NW>
struct RowTopkLds {
  uint32_t c[2][NW];  // per-wave counts, two buffers used in turn
  uint32_t r[2][NW];  // per-wave key minimum and maximum
};

// Thread tid of the NT = 64*NW threads holds the scores of ids tid + NT*r (r < R) in v; ids >= n
// are ignored (their values may be anything).  Candidate scores must be finite.  For each chosen id,
// the thread holding it calls emit(slot, id, r) with its slot 0 .. count-1 in ascending id order.
// Returns count = min(n, k), the same in every thread.  Every thread of the workgroup must call it.
template <int NW, int R, typename Emit>
__device__ __forceinline__ int row_topk(const float (&v)[R], int n, int k, RowTopkLds<NW>& sh, Emit&& emit) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (n <= k) {  // every candidate: ids 0 .. n-1, all held in r = 0 since n <= k <= 64 <= NT
    if (tid < n) emit(tid, tid, 0);
    return n;
  }
  // ids >= n get key 0, below every candidate key
  uint32_t key[R];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool in = tid + NT * r < n;
    const uint32_t kr = order_key(v[r]);
    key[r] = in ? kr : 0u;
    kmin = min(kmin, in ? kr : 0xffffffffu);
    kmax = max(kmax, key[r]);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, kWave));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, kWave));
  }
  if (NW > 1) {
    if (lane == 0) { sh.r[0][wv] = kmin; sh.r[1][wv] = kmax; }
    __syncthreads();
    for (int x = 0; x < NW; ++x) { kmin = min(kmin, sh.r[0][x]); kmax = max(kmax, sh.r[1][x]); }
  }
  // count of keys >= thr over the whole row (uniform result)
  auto count_ge = [&](uint32_t thr, int parity) -> int {
    int c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c += __popcll(__ballot(key[r] >= thr));
    if (NW > 1) {
      if (lane == 0) sh.c[parity][wv] = c;
      __syncthreads();
      c = 0;
      for (int x = 0; x < NW; ++x) c += sh.c[parity][x];
    }
    return c;
  };
  uint32_t T = kmin;
  int parity = 0;  // buffer of the next count (alternates, so a slow wave's read is never overwritten)
  if (kmin != kmax) {
    const int hb = 31 - __builtin_clz(kmin ^ kmax);
    T = hb == 31 ? 0u : (kmin & ~((2u << hb) - 1u));
    for (int b = hb; b >= 0; --b) {  // every trial threshold is >= 1, so id slots past n never count
      const uint32_t cand = T | (1u << b);
      const int c = count_ge(cand, parity);
      parity ^= 1;
      if (c >= k) {
        T = cand;
        if (c == k) break;
      }
    }
  }
  const int remaining = k - (T == 0xffffffffu ? 0 : count_ge(T + 1u, parity));

  // emit in id order: keys above T, then the first `remaining` keys equal to T
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int written = 0, ties_seen = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid + NT * r;
    const bool gt = key[r] > T;
    const bool eq = i < n && key[r] == T;
    const uint64_t eqm = __ballot(eq);
    int eq_before = ties_seen + __popcll(eqm & lt_mask);
    int eq_all = __popcll(eqm);
    if (NW > 1) {
      __syncthreads();  // the counts of the previous use are read by every wave
      if (lane == 0) sh.c[0][wv] = eq_all;
      __syncthreads();
      eq_all = 0;
      for (int x = 0; x < NW; ++x) {
        if (x < wv) eq_before += sh.c[0][x];
        eq_all += sh.c[0][x];
      }
    }
    const bool take = gt || (eq && eq_before < remaining);
    const uint64_t tm = __ballot(take);
    int slot = written + __popcll(tm & lt_mask);
    int take_all = __popcll(tm);
    if (NW > 1) {
      if (lane == 0) sh.c[1][wv] = take_all;
      __syncthreads();
      take_all = 0;
      for (int x = 0; x < NW; ++x) {
        if (x < wv) slot += sh.c[1][x];
        take_all += sh.c[1][x];
      }
    }
    if (take && slot < k) emit(slot, i, r);
    written += take_all;
    ties_seen += eq_all;
  }
  return k;
}

// ---- two-level selection for long rows (many waves) ----
//
// Under the total order (score descending, id ascending) every member of a row's top k is also in
// the top k of any subset of the row that contains it.  So each wave first selects the top k of its
// own contiguous run of ids with ballot counts alone (no workgroup barrier per trial bit), and one
// wave then selects the row's top k from the waves' candidates, which lie in LDS in ascending id
// order.  The chosen ids are exactly those of row_topk.

// Threshold of one wave's selection: keys at position lane + 64 j (key 0 = no candidate, below every
// candidate key), at least k of them candidates.  The chosen set is the keys above T plus the first
// `remaining` keys equal to T in position order; exactly k keys.
template <int RR>
__device__ __forceinline__ void wave_threshold(const uint32_t (&key)[RR], int k, uint32_t& T, int& remaining) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < RR; ++j) {
    kmin = min(kmin, key[j] ? key[j] : 0xffffffffu);
    kmax = max(kmax, key[j]);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, kWave));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, kWave));
  }
  auto count_ge = [&](uint32_t thr) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < RR; ++j) c += __popcll(__ballot(key[j] >= thr));
    return c;
  };
  T = kmin;
  if (kmin != kmax) {
    const int hb = 31 - __builtin_clz(kmin ^ kmax);
    T = hb == 31 ? 0u : (kmin & ~((2u << hb) - 1u));
    for (int b = hb; b >= 0; --b) {  // every trial threshold is >= 1: non-candidates never count
      const uint32_t cand = T | (1u << b);
      const int c = count_ge(cand);
      if (c >= k) {
        T = cand;
        if (c == k) break;
      }
    }
  }
  remaining = k - (T == 0xffffffffu ? 0 : count_ge(T + 1u));
}

// The keys a wave selects (threshold T, `remaining` boundary ties), in position order:
// emit(slot, j) for the lane holding position lane + 64 j, slots 0, 1, ...
template <int RR, typename Emit>
__device__ __forceinline__ void wave_emit(const uint32_t (&key)[RR], uint32_t T, int remaining, Emit&& emit) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int written = 0, ties_seen = 0;
#pragma unroll
  for (int j = 0; j < RR; ++j) {
    const bool gt = key[j] > T;
    const bool eq = key[j] != 0u && key[j] == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = gt || (eq && ties_seen + __popcll(eqm & lt_mask) < remaining);
    const uint64_t tm = __ballot(take);
    if (take) emit(written + __popcll(tm & lt_mask), j);
    written += __popcll(tm);
    ties_seen += __popcll(eqm);
  }
}

template <int NW>
struct RowTopk2Lds {
  uint32_t key[NW * 64];  // wave w's candidates at [w*k, w*k + its count), ascending id
  int32_t id[NW * 64];
};

// Same contract as row_topk, for k <= 64, with ids laid out by wave: thread (wave w, lane) holds the
// scores of ids w*64*R + lane + 64*r (r < R) in v.  Every thread of the workgroup must call it; emit
// is called by wave 0 only, after one workgroup barrier.
template <int NW, int R, typename Emit>
__device__ __forceinline__ int row_topk_two_level(const float (&v)[R], int n, int k, RowTopk2Lds<NW>& sh,
                                                  Emit&& emit) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (n <= k) {  // every candidate: ids 0 .. n-1
    if (tid < n) emit(tid, tid);
    return n;
  }
  // level 1: the top k of this wave's ids [w*64R, (w+1)*64R) that are candidates (id < n)
  const int base = wv * 64 * R;
  const int nw = min(max(n - base, 0), 64 * R);  // candidates of this wave
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) key[r] = (lane + 64 * r < nw) ? order_key(v[r]) : 0u;
  if (nw <= k) {  // all of them, in id order
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane + 64 * r < nw) {
        sh.key[wv * k + lane + 64 * r] = key[r];
        sh.id[wv * k + lane + 64 * r] = base + lane + 64 * r;
      }
  } else {
    uint32_t T;
    int rem;
    wave_threshold<R>(key, k, T, rem);
    wave_emit<R>(key, T, rem, [&](int slot, int r) {
      sh.key[wv * k + slot] = key[r];
      sh.id[wv * k + slot] = base + lane + 64 * r;
    });
  }
  __syncthreads();
  // level 2 (wave 0): the waves before the one holding id n-1 each left exactly k candidates (64R >= k),
  // so the candidates fill positions [0, C) in ascending id order, C >= k
  if (wv == 0) {
    const int last = (n - 1) / (64 * R);
    const int C = last * k + min(n - last * 64 * R, k);
    uint32_t ck[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) ck[j] = (lane + 64 * j < C) ? sh.key[lane + 64 * j] : 0u;
    uint32_t T;
    int rem;
    wave_threshold<NW>(ck, k, T, rem);
    wave_emit<NW>(ck, T, rem, [&](int slot, int j) { emit(slot, sh.id[lane + 64 * j]); });
  }
  return k;
}

}  // namespace msa
