// Device-side helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;      // tokens per KV block (= page)
constexpr int kWave = 64;

typedef uint16_t bf16;           // storage type: raw bfloat16 bits
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One float -> bf16 bits (round to nearest even).
__device__ __forceinline__ uint32_t f2bf_bits(float f) { return pack_bf2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming load for data read exactly once (non-temporal hint): keeps it from displacing
// reused lines in L2 / the MALL and runs closer to the HBM peak than ordinary loads.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }
__device__ __forceinline__ f32x4 fzero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A[l%16][k in chunk l/16] and B[k in chunk l/16][l%16] (8 values each, the
// same k order on both sides); it receives D[4*(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// Reduce across the four 16-lane groups (lanes l, l^16, l^32, l^48) with gfx950's lane-swap
// instructions, which are VALU ops with no LDS round trip.  v_permlane32_swap on two copies of v
// leaves one holding the lower 32 lanes twice and the other the upper 32 lanes twice, so
// combining the two pairs every lane l with l^32; v_permlane16_swap does the same for l^16.
// Every lane ends with the same value, combined in the same order.
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_over_quads(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_over_quads(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(a + b, a, b);
  return a + b;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 2^x and log2(x) as single v_exp_f32 / v_log_f32 (results that would be denormal flush to 0,
// which softmax weights can afford; exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Order-preserving map of a float to uint32 (-0 is folded onto +0 so equal scores tie).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Request that owns query row t (cu_q is non-decreasing, cu_q[0] = 0, cu_q[B] = Nq).
__device__ __forceinline__ int request_of(const int32_t* __restrict__ cu_q, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same request index r, and ctx_len[r], found by one wavefront with one round of loads per
// 64 requests instead of a chain of dependent loads: the requests whose first query row is
// <= t form a prefix (cu_q is non-decreasing), and r is its last element.  Every lane of the
// wave must call it; the results are uniform.
__device__ __forceinline__ void request_and_len(const int32_t* __restrict__ cu_q,
                                                const int32_t* __restrict__ ctx_len, int B, int t, int& r,
                                                int& len) {
  const int lane = threadIdx.x & (kWave - 1);
  int count = 0, l_last = 0;
  for (int base = 0; base < B; base += kWave) {
    const int i = min(base + lane, B - 1);
    const int c = cu_q[i], l = ctx_len[i];
    asm volatile("" ::"v"(c), "v"(l));  // both loads in the same round trip
    const uint64_t m = __ballot(base + lane < B && c <= t);
    if (m) l_last = __shfl(l, 63 - __builtin_clzll(m), kWave);
    count += __popcll(m);
  }
  r = count - 1;
  len = __builtin_amdgcn_readfirstlane(l_last);
}

}  // namespace msa
