// Host side of the MSA C ABI: argument validation, workspace sizing and kernel launches.
// Every argument is checked before anything is enqueued; see include/msa.h for the contract.
#include "msa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

namespace msa {
hipError_t launch_score_decode(int B, int Di, const int32_t* block_table, int max_blocks, const int32_t* ctx_len,
                               const int32_t* cu_q, const int32_t* q_pos, const void* q_idx, const void* kidx,
                               int Hkv, int64_t kpage, float* scores, hipStream_t stream);
hipError_t launch_score_prefill(int B, int Nq, int Di, const int32_t* block_table, int max_blocks,
                                const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const void* q_idx,
                                const void* kidx, int Hkv, int64_t kpage, float* scores, hipStream_t stream);
int fused_topk_capacity();
hipError_t launch_score_topk_prefill(int B, int Nq, int Di, const int32_t* block_table, int max_blocks,
                                     const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos,
                                     const void* q_idx, const void* kidx, int Hkv, int64_t kpage, int k, int32_t* sel,
                                     int32_t* cnt, hipStream_t stream);
hipError_t launch_topk(int B, int Nq, int Hkv, int max_blocks, const int32_t* cu_q, const int32_t* q_pos,
                       const float* scores, int k, int32_t* sel, int32_t* cnt, hipStream_t stream);
hipError_t launch_page_table(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                             const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const int32_t* sel,
                             const int32_t* cnt, int k, int vps, int32_t* page_table, int32_t* row_len,
                             hipStream_t stream);
hipError_t launch_topk_page_table(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                                  const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos,
                                  const float* scores, int k, int32_t* sel, int32_t* cnt, int vps,
                                  int32_t* page_table, int32_t* row_len, hipStream_t stream);
int decode_splits(int rows, int k);
int select_attend_max_blocks();
hipError_t launch_select_attend(int B, int Nq, int Hkv, int max_blocks, const int32_t* block_table,
                                const int32_t* ctx_len, const int32_t* cu_q, const int32_t* q_pos, const float* scores,
                                int k, int32_t* sel, int32_t* cnt, int32_t* page_table, int32_t* row_len, int vps,
                                int G, int D, const void* q, const void* kcache, const void* vcache, float sm_scale,
                                void* out, float* lse, float* ws_o, float* ws_lse, uint32_t* counters,
                                hipStream_t stream);
hipError_t launch_attn_decode(int rows, int G, int D, const void* q, const void* kview, const void* vview,
                              int64_t page_stride, int64_t token_stride, const int32_t* page_table, int k,
                              const int32_t* row_len, float sm_scale, void* out, float* lse, float* ws_o,
                              float* ws_lse, uint32_t* counters, hipStream_t stream);
hipError_t launch_lse_merge_bf16(int64_t rows, int parts, int G, int D, const void* part_o, const float* part_lse,
                                 void* out, float* lse_out, hipStream_t stream);
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);
size_t prefill_workspace_bytes(int32_t Nq, int32_t Hkv, int32_t k, int32_t B, int32_t max_blocks, int32_t max_q);
hipError_t launch_attn_prefill(int B, int Nq, int Hkv, int G, int D, int max_blocks, int max_q,
                               const int32_t* block_table, const int32_t* ctx_len, const int32_t* cu_q,
                               const int32_t* q_pos, const void* q, const void* kcache, const void* vcache,
                               int64_t kvpage, const int32_t* sel, const int32_t* cnt, int k, float sm_scale,
                               int tile_min_rows, void* part_o, float* part_lse, int32_t* slot_of, void* workspace,
                               hipStream_t stream);
}  // namespace msa

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kMaxK = 64;
constexpr int kMaxHkv = 64;
constexpr int kMaxGridY = 65535;

#define MSA_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

msa_status check_batch(const msa_batch* b) {
  MSA_REQUIRE(b != nullptr, MSA_ERR_INVALID_ARG, "batch is NULL");
  MSA_REQUIRE(b->num_requests >= 1 && b->num_requests <= kMaxGridY, MSA_ERR_INVALID_ARG,
              "num_requests must be in [1, %d], got %d", kMaxGridY, b->num_requests);
  MSA_REQUIRE(b->num_queries >= 0, MSA_ERR_INVALID_ARG, "num_queries must be >= 0, got %d", b->num_queries);
  MSA_REQUIRE(b->max_blocks >= 1, MSA_ERR_INVALID_ARG, "max_blocks must be >= 1, got %d", b->max_blocks);
  MSA_REQUIRE(b->max_q_per_request >= 0, MSA_ERR_INVALID_ARG, "max_q_per_request must be >= 0");
  MSA_REQUIRE(b->block_table && b->ctx_len && b->cu_q, MSA_ERR_INVALID_ARG,
              "batch block_table, ctx_len and cu_q must be non-NULL");
  MSA_REQUIRE(b->num_queries == 0 || b->q_pos, MSA_ERR_INVALID_ARG, "batch q_pos is NULL");
  MSA_REQUIRE(aligned4(b->block_table) && aligned4(b->ctx_len) && aligned4(b->cu_q) && aligned4(b->q_pos),
              MSA_ERR_INVALID_ARG, "batch arrays must be 4-byte aligned");
  return MSA_OK;
}

// Elements from one page of the cache to the next.
int64_t page_elems(const msa_cache& c) {
  return c.page_stride ? c.page_stride : (int64_t)c.block_size * c.num_heads * c.head_dim;
}

// The cache's shape and page stride (data not read).
msa_status check_layout(const msa_cache& c, const char* name) {
  MSA_REQUIRE(c.num_pages >= 1, MSA_ERR_INVALID_ARG, "%s: num_pages must be >= 1", name);
  MSA_REQUIRE(c.block_size == 128, MSA_ERR_UNSUPPORTED, "%s: block_size must be 128, got %d", name, c.block_size);
  MSA_REQUIRE(c.num_heads >= 1 && c.num_heads <= kMaxHkv, MSA_ERR_UNSUPPORTED, "%s: num_heads must be in [1, %d]",
              name, kMaxHkv);
  MSA_REQUIRE(supported_dim(c.head_dim), MSA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", name,
              c.head_dim);
  const int64_t dense = (int64_t)c.block_size * c.num_heads * c.head_dim;
  MSA_REQUIRE(c.page_stride == 0 || (c.page_stride >= dense && c.page_stride % 8 == 0), MSA_ERR_INVALID_ARG,
              "%s: page_stride must be 0 or a multiple of 8 that is >= block_size*num_heads*head_dim = %lld, got %lld",
              name, (long long)dense, (long long)c.page_stride);
  return MSA_OK;
}

// A K or V cache: also the virtual page ids of the decode page table, page * (page_stride / head_dim)
// + head, must be whole and fit in int32.
msa_status check_kv_layout(const msa_cache& c, const char* name) {
  if (msa_status s = check_layout(c, name)) return s;
  MSA_REQUIRE(page_elems(c) % c.head_dim == 0, MSA_ERR_INVALID_ARG, "%s: page_stride must be a multiple of head_dim",
              name);
  MSA_REQUIRE((int64_t)c.num_pages * (page_elems(c) / c.head_dim) <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED,
              "%s: num_pages * page_stride / head_dim must fit in int32 (virtual page ids)", name);
  return MSA_OK;
}

msa_status check_cache(const msa_cache& c, const char* name) {
  MSA_REQUIRE(c.data != nullptr, MSA_ERR_INVALID_ARG, "%s: data is NULL", name);
  MSA_REQUIRE(aligned16(c.data), MSA_ERR_INVALID_ARG, "%s: data must be 16-byte aligned", name);
  if (msa_status s = check_layout(c, name)) return s;
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

int32_t msa_version(void) { return 100; }

msa_status msa_index_score(const msa_batch* batch, const void* q_idx, msa_cache k_idx, float* scores,
                           msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_cache(k_idx, "k_idx")) return s;
  MSA_REQUIRE(batch->num_queries == 0 || (q_idx && aligned16(q_idx)), MSA_ERR_INVALID_ARG,
              "q_idx must be non-NULL and 16-byte aligned");
  MSA_REQUIRE(batch->num_queries == 0 || (scores && aligned4(scores)), MSA_ERR_INVALID_ARG,
              "scores must be non-NULL and 4-byte aligned");
  if (batch->num_queries == 0) return MSA_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (batch->max_q_per_request <= 16)
    e = msa::launch_score_decode(batch->num_requests, k_idx.head_dim, batch->block_table, batch->max_blocks,
                                 batch->ctx_len, batch->cu_q, batch->q_pos, q_idx, k_idx.data, k_idx.num_heads,
                                 page_elems(k_idx), scores, st);
  else
    e = msa::launch_score_prefill(batch->num_requests, batch->num_queries, k_idx.head_dim, batch->block_table,
                                  batch->max_blocks, batch->ctx_len, batch->cu_q, batch->q_pos, q_idx, k_idx.data,
                                  k_idx.num_heads, page_elems(k_idx), scores, st);
  return from_hip(e, "msa_index_score launch");
}

static bool fused_index_topk(const msa_batch* b, int32_t k) {
  return b->max_q_per_request > 16 && k <= msa::fused_topk_capacity() && b->max_blocks <= 65536;
}

size_t msa_index_topk_workspace_size(const msa_batch* batch, int32_t num_kv_heads, int32_t k) {
  if (!batch || batch->num_queries < 0 || batch->max_blocks <= 0 || num_kv_heads <= 0 || k <= 0) return 0;
  if (fused_index_topk(batch, k)) return 0;
  return align256((size_t)batch->num_queries * num_kv_heads * batch->max_blocks * sizeof(float));
}

msa_status msa_index_topk(const msa_batch* batch, const void* q_idx, msa_cache k_idx, int32_t k, int32_t* sel,
                          int32_t* cnt, void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_cache(k_idx, "k_idx")) return s;
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(batch->num_queries == 0 || (q_idx && aligned16(q_idx) && sel && cnt), MSA_ERR_INVALID_ARG,
              "q_idx (16-byte aligned), sel and cnt must be non-NULL");
  MSA_REQUIRE(aligned4(sel) && aligned4(cnt), MSA_ERR_INVALID_ARG, "sel and cnt must be 4-byte aligned");
  MSA_REQUIRE((int64_t)batch->num_queries * k_idx.num_heads <= 0x7fffffff, MSA_ERR_UNSUPPORTED,
              "num_queries * num_kv_heads exceeds the grid limit");
  if (batch->num_queries == 0) return MSA_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (fused_index_topk(batch, k))
    return from_hip(msa::launch_score_topk_prefill(batch->num_requests, batch->num_queries, k_idx.head_dim,
                                                   batch->block_table, batch->max_blocks, batch->ctx_len,
                                                   batch->cu_q, batch->q_pos, q_idx, k_idx.data, k_idx.num_heads,
                                                   page_elems(k_idx), k, sel, cnt, st),
                    "msa_index_topk launch");
  const size_t need = msa_index_topk_workspace_size(batch, k_idx.num_heads, k);
  MSA_REQUIRE(workspace && aligned16(workspace) && workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
              "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  float* scores = static_cast<float*>(workspace);
  if (msa_status s = msa_index_score(batch, q_idx, k_idx, scores, stream)) return s;
  return msa_topk_blocks(batch, k_idx.num_heads, scores, k, sel, cnt, stream);
}

msa_status msa_topk_blocks(const msa_batch* batch, int32_t num_kv_heads, const float* scores, int32_t k,
                           int32_t* sel, int32_t* cnt, msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  MSA_REQUIRE(num_kv_heads >= 1 && num_kv_heads <= kMaxHkv, MSA_ERR_UNSUPPORTED, "num_kv_heads must be in [1, %d]",
              kMaxHkv);
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(batch->num_queries == 0 || (scores && sel && cnt), MSA_ERR_INVALID_ARG,
              "scores, sel and cnt must be non-NULL");
  MSA_REQUIRE(aligned4(scores) && aligned4(sel) && aligned4(cnt), MSA_ERR_INVALID_ARG, "arrays must be 4-byte aligned");
  MSA_REQUIRE((int64_t)batch->num_queries * num_kv_heads <= 0x7fffffff, MSA_ERR_UNSUPPORTED,
              "num_queries * num_kv_heads exceeds the grid limit");
  if (batch->num_queries == 0) return MSA_OK;
  return from_hip(msa::launch_topk(batch->num_requests, batch->num_queries, num_kv_heads, batch->max_blocks,
                                   batch->cu_q, batch->q_pos, scores, k, sel, cnt,
                                   reinterpret_cast<hipStream_t>(stream)),
                  "msa_topk_blocks launch");
}

msa_status msa_build_sparse_page_table(const msa_batch* batch, msa_cache kv_layout, const int32_t* sel,
                                       const int32_t* cnt, int32_t k, int32_t* page_table, int32_t* row_len,
                                       msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_kv_layout(kv_layout, "kv_layout")) return s;
  const int Hkv = kv_layout.num_heads;
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(batch->num_queries == 0 || (sel && cnt && page_table && row_len), MSA_ERR_INVALID_ARG,
              "sel, cnt, page_table and row_len must be non-NULL");
  MSA_REQUIRE(aligned4(sel) && aligned4(cnt) && aligned4(page_table) && aligned4(row_len), MSA_ERR_INVALID_ARG,
              "arrays must be 4-byte aligned");
  if (batch->num_queries == 0) return MSA_OK;
  return from_hip(msa::launch_page_table(batch->num_requests, batch->num_queries, Hkv, batch->max_blocks,
                                         batch->block_table, batch->ctx_len, batch->cu_q, batch->q_pos, sel, cnt, k,
                                         (int)(page_elems(kv_layout) / kv_layout.head_dim), page_table, row_len,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "msa_build_sparse_page_table launch");
}

msa_status msa_topk_page_table(const msa_batch* batch, msa_cache kv_layout, const float* scores, int32_t k,
                               int32_t* sel, int32_t* cnt, int32_t* page_table, int32_t* row_len,
                               msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_kv_layout(kv_layout, "kv_layout")) return s;
  const int Hkv = kv_layout.num_heads;
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(batch->num_queries == 0 || (scores && sel && cnt && page_table && row_len), MSA_ERR_INVALID_ARG,
              "scores, sel, cnt, page_table and row_len must be non-NULL");
  MSA_REQUIRE(aligned4(scores) && aligned4(sel) && aligned4(cnt) && aligned4(page_table) && aligned4(row_len),
              MSA_ERR_INVALID_ARG, "arrays must be 4-byte aligned");
  MSA_REQUIRE((int64_t)batch->num_queries * Hkv <= 0x7fffffff, MSA_ERR_UNSUPPORTED,
              "num_queries * num_kv_heads exceeds the grid limit");
  if (batch->num_queries == 0) return MSA_OK;
  return from_hip(msa::launch_topk_page_table(batch->num_requests, batch->num_queries, Hkv, batch->max_blocks,
                                              batch->block_table, batch->ctx_len, batch->cu_q, batch->q_pos, scores,
                                              k, sel, cnt, (int)(page_elems(kv_layout) / kv_layout.head_dim),
                                              page_table, row_len, reinterpret_cast<hipStream_t>(stream)),
                  "msa_topk_page_table launch");
}

size_t msa_sparse_attn_decode_workspace_size(int32_t rows, int32_t G, int32_t D, int32_t k) {
  if (rows <= 0 || G <= 0 || D <= 0 || k <= 0) return 0;
  const int nsplit = msa::decode_splits(rows, k);
  if (nsplit == 1) return 0;  // each row in one workgroup: outputs are written directly
  const size_t parts = (size_t)rows * nsplit * G;
  return align256((size_t)rows * sizeof(uint32_t)) + align256(parts * D * sizeof(float)) +
         align256(parts * sizeof(float));
}

namespace {

// Split workspace of the decode attention: partial O and partial LSE from the start of the buffer, one
// arrival counter per row at its end (the last 256-byte-aligned rows * 4 bytes below the buffer's
// 256-byte-aligned size).  Calls with fewer rows use a tail of the same counter region and no call's
// partials reach it, so counters that start at zero stay valid from call to call for one buffer and
// size; each call returns the counters it used to zero.
struct DecodeSplitWs {
  uint32_t* counters = nullptr;
  float* o = nullptr;
  float* lse = nullptr;
};
DecodeSplitWs decode_split_ws(void* workspace, size_t workspace_bytes, int rows, int G, int D, int k) {
  DecodeSplitWs w;
  if (msa_sparse_attn_decode_workspace_size(rows, G, D, k) == 0) return w;
  const size_t parts = (size_t)rows * msa::decode_splits(rows, k) * G;
  char* base = static_cast<char*>(workspace);
  w.o = reinterpret_cast<float*>(base);
  w.lse = reinterpret_cast<float*>(base + align256(parts * D * sizeof(float)));
  const size_t end = workspace_bytes & ~(size_t)255;
  w.counters = reinterpret_cast<uint32_t*>(base + end - align256((size_t)rows * sizeof(uint32_t)));
  return w;
}

}  // namespace

msa_status msa_sparse_attn_decode(int32_t rows, int32_t G, int32_t D, const void* q, const void* k_base,
                                  const void* v_base, int64_t page_stride, int64_t token_stride,
                                  const int32_t* page_table, int32_t k, const int32_t* row_len, float sm_scale,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  msa_stream_t stream) {
  g_last_error.clear();
  MSA_REQUIRE(rows >= 0, MSA_ERR_INVALID_ARG, "rows must be >= 0");
  MSA_REQUIRE(supported_group(G), MSA_ERR_UNSUPPORTED, "G must be 1, 2, 4, 8 or 16, got %d", G);
  MSA_REQUIRE(supported_dim(D), MSA_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(page_stride > 0 && token_stride > 0 && page_stride % 8 == 0 && token_stride % 8 == 0,
              MSA_ERR_INVALID_ARG, "page_stride and token_stride must be positive multiples of 8 elements");
  if (rows == 0) return MSA_OK;
  MSA_REQUIRE(q && k_base && v_base && page_table && row_len && out, MSA_ERR_INVALID_ARG,
              "q, k_base, v_base, page_table, row_len and out must be non-NULL");
  MSA_REQUIRE(aligned16(q) && aligned16(k_base) && aligned16(v_base) && aligned16(out) && aligned16(workspace),
              MSA_ERR_INVALID_ARG, "q, k_base, v_base, out and workspace must be 16-byte aligned");
  MSA_REQUIRE(aligned4(page_table) && aligned4(row_len) && aligned4(lse), MSA_ERR_INVALID_ARG,
              "page_table, row_len and lse must be 4-byte aligned");
  MSA_REQUIRE((int64_t)rows * k <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED, "rows*k must fit in int32");
  MSA_REQUIRE(token_stride * 128 + D <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED, "token_stride*128 must fit in int32");
  const size_t need = msa_sparse_attn_decode_workspace_size(rows, G, D, k);
  MSA_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), MSA_ERR_WORKSPACE_TOO_SMALL,
              "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  const DecodeSplitWs ws = decode_split_ws(workspace, workspace_bytes, rows, G, D, k);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return from_hip(msa::launch_attn_decode(rows, G, D, q, k_base, v_base, page_stride, token_stride, page_table, k,
                                          row_len, sm_scale, out, lse, ws.o, ws.lse, ws.counters, st),
                  "msa_sparse_attn_decode launch");
}

namespace {

// msa_topk_attn_decode and its allocation-free form: the same checks and launches; the split partials
// go to the caller's workspace, or (use_scratch) to the library's static per-device scratch.
msa_status topk_attn_decode(const msa_batch* batch, const float* scores, int32_t k, msa_cache k_cache,
                            msa_cache v_cache, int32_t G, const void* q, float sm_scale, int32_t* sel, int32_t* cnt,
                            int32_t* page_table, int32_t* row_len, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, bool use_scratch, msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_cache(k_cache, "k_cache")) return s;
  if (msa_status s = check_cache(v_cache, "v_cache")) return s;
  if (msa_status s = check_kv_layout(k_cache, "k_cache")) return s;
  MSA_REQUIRE(k_cache.num_pages == v_cache.num_pages && k_cache.num_heads == v_cache.num_heads &&
                  k_cache.head_dim == v_cache.head_dim && page_elems(k_cache) == page_elems(v_cache),
              MSA_ERR_INVALID_ARG, "k_cache and v_cache must have the same shape and page stride");
  const int Hkv = k_cache.num_heads, D = k_cache.head_dim;
  const int vps = (int)(page_elems(k_cache) / D);  // virtual pages per page of the strided views
  MSA_REQUIRE(supported_group(G), MSA_ERR_UNSUPPORTED, "G must be 1, 2, 4, 8 or 16, got %d", G);
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  const int64_t rows64 = (int64_t)batch->num_queries * Hkv;
  MSA_REQUIRE(rows64 * k <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED, "num_queries*num_heads*k must fit in int32");
  if (batch->num_queries == 0) return MSA_OK;
  MSA_REQUIRE(scores && q && sel && cnt && page_table && row_len && out, MSA_ERR_INVALID_ARG,
              "scores, q, sel, cnt, page_table, row_len and out must be non-NULL");
  MSA_REQUIRE(aligned16(q) && aligned16(out) && aligned16(workspace), MSA_ERR_INVALID_ARG,
              "q, out and workspace must be 16-byte aligned");
  MSA_REQUIRE(aligned4(scores) && aligned4(sel) && aligned4(cnt) && aligned4(page_table) && aligned4(row_len) &&
                  aligned4(lse),
              MSA_ERR_INVALID_ARG, "scores, sel, cnt, page_table, row_len and lse must be 4-byte aligned");
  const int rows = (int)rows64;
  const size_t need = msa_sparse_attn_decode_workspace_size(rows, G, D, k);
  if (use_scratch) {
    MSA_REQUIRE(need <= msa::decode_scratch_bytes(), MSA_ERR_UNSUPPORTED,
                "this batch needs %zu bytes of split scratch, more than the %zu bytes the allocation-free entry "
                "point holds; call msa_topk_attn_decode with a workspace instead",
                need, msa::decode_scratch_bytes());
    if (need > 0) {
      if (msa_status s = from_hip(msa::decode_scratch(&workspace), "msa_topk_attn_decode_noalloc scratch lookup"))
        return s;
    }
  } else {
    MSA_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), MSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  }
  const DecodeSplitWs ws =
      decode_split_ws(workspace, use_scratch ? msa::decode_scratch_bytes() : workspace_bytes, rows, G, D, k);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (batch->max_blocks <= msa::select_attend_max_blocks())
    return from_hip(msa::launch_select_attend(batch->num_requests, batch->num_queries, Hkv, batch->max_blocks,
                                              batch->block_table, batch->ctx_len, batch->cu_q, batch->q_pos, scores,
                                              k, sel, cnt, page_table, row_len, vps, G, D, q, k_cache.data,
                                              v_cache.data, sm_scale, out, lse, ws.o, ws.lse, ws.counters, st),
                    "msa_topk_attn_decode launch");
  // rows too long to select inside the attention workgroup: the two launches of the separate calls
  hipError_t e = msa::launch_topk_page_table(batch->num_requests, batch->num_queries, Hkv, batch->max_blocks,
                                             batch->block_table, batch->ctx_len, batch->cu_q, batch->q_pos, scores, k,
                                             sel, cnt, vps, page_table, row_len, st);
  if (e != hipSuccess) return from_hip(e, "msa_topk_attn_decode top-k launch");
  return from_hip(msa::launch_attn_decode(rows, G, D, q, k_cache.data, v_cache.data, D, (int64_t)Hkv * D, page_table,
                                          k, row_len, sm_scale, out, lse, ws.o, ws.lse, ws.counters, st),
                  "msa_topk_attn_decode attention launch");
}

}  // namespace

msa_status msa_topk_attn_decode(const msa_batch* batch, const float* scores, int32_t k, msa_cache k_cache,
                                msa_cache v_cache, int32_t G, const void* q, float sm_scale, int32_t* sel, int32_t* cnt,
                                int32_t* page_table, int32_t* row_len, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, msa_stream_t stream) {
  return topk_attn_decode(batch, scores, k, k_cache, v_cache, G, q, sm_scale, sel, cnt, page_table, row_len, out, lse,
                          workspace, workspace_bytes, false, stream);
}

msa_status msa_topk_attn_decode_noalloc(const msa_batch* batch, const float* scores, int32_t k, msa_cache k_cache,
                                        msa_cache v_cache, int32_t G, const void* q, float sm_scale, int32_t* sel,
                                        int32_t* cnt, int32_t* page_table, int32_t* row_len, void* out, float* lse,
                                        msa_stream_t stream) {
  return topk_attn_decode(batch, scores, k, k_cache, v_cache, G, q, sm_scale, sel, cnt, page_table, row_len, out, lse,
                          nullptr, 0, true, stream);
}

size_t msa_sparse_attn_prefill_workspace_size(const msa_batch* batch, int32_t num_kv_heads, int32_t k) {
  if (!batch || batch->num_queries < 0 || batch->num_requests <= 0 || batch->max_blocks <= 0 || num_kv_heads <= 0 ||
      k <= 0)
    return 0;
  return msa::prefill_workspace_bytes(batch->num_queries, num_kv_heads, k, batch->num_requests, batch->max_blocks,
                                      batch->max_q_per_request);
}

msa_status msa_sparse_attn_prefill(const msa_batch* batch, int32_t G, const void* q, msa_cache k_cache,
                                   msa_cache v_cache, const int32_t* sel, const int32_t* cnt, int32_t k,
                                   float sm_scale, int32_t tile_min_rows, void* part_o, float* part_lse,
                                   int32_t* slot_of, void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  if (msa_status s = check_batch(batch)) return s;
  if (msa_status s = check_cache(k_cache, "k_cache")) return s;
  if (msa_status s = check_cache(v_cache, "v_cache")) return s;
  MSA_REQUIRE(k_cache.num_pages == v_cache.num_pages && k_cache.num_heads == v_cache.num_heads &&
                  k_cache.head_dim == v_cache.head_dim && page_elems(k_cache) == page_elems(v_cache),
              MSA_ERR_INVALID_ARG, "k_cache and v_cache differ in shape or page stride");
  MSA_REQUIRE(supported_group(G), MSA_ERR_UNSUPPORTED, "G must be 1, 2, 4, 8 or 16, got %d", G);
  MSA_REQUIRE(k >= 1 && k <= kMaxK, MSA_ERR_UNSUPPORTED, "k must be in [1, %d], got %d", kMaxK, k);
  MSA_REQUIRE(tile_min_rows >= 0, MSA_ERR_INVALID_ARG, "tile_min_rows must be >= 0, got %d", tile_min_rows);
  if (batch->num_queries == 0) return MSA_OK;
  MSA_REQUIRE(q && sel && cnt && part_o && part_lse && workspace, MSA_ERR_INVALID_ARG,
              "q, sel, cnt, part_o, part_lse and workspace must be non-NULL");
  MSA_REQUIRE(aligned16(q) && aligned16(part_o) && aligned16(workspace), MSA_ERR_INVALID_ARG,
              "q, part_o and workspace must be 16-byte aligned");
  MSA_REQUIRE(aligned4(sel) && aligned4(cnt) && aligned4(part_lse) && aligned4(slot_of), MSA_ERR_INVALID_ARG,
              "sel, cnt, part_lse and slot_of must be 4-byte aligned");
  MSA_REQUIRE((int64_t)batch->num_queries * k_cache.num_heads * k <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED,
              "num_queries*Hkv*k must fit in int32");
  MSA_REQUIRE((int64_t)batch->num_queries < (1LL << 25), MSA_ERR_UNSUPPORTED, "num_queries must be < 2^25");
  MSA_REQUIRE((int64_t)k_cache.num_heads * batch->num_requests * batch->max_blocks <= 0x7fffffffLL,
              MSA_ERR_UNSUPPORTED, "num_kv_heads*num_requests*max_blocks must fit in int32");
  const size_t need = msa_sparse_attn_prefill_workspace_size(batch, k_cache.num_heads, k);
  MSA_REQUIRE(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
              workspace_bytes);
  return from_hip(msa::launch_attn_prefill(batch->num_requests, batch->num_queries, k_cache.num_heads, G,
                                           k_cache.head_dim, batch->max_blocks, batch->max_q_per_request,
                                           batch->block_table, batch->ctx_len, batch->cu_q, batch->q_pos, q,
                                           k_cache.data, v_cache.data, page_elems(k_cache), sel, cnt, k, sm_scale,
                                           tile_min_rows, part_o, part_lse, slot_of, workspace,
                                           reinterpret_cast<hipStream_t>(stream)),
                  "msa_sparse_attn_prefill launch");
}

msa_status msa_lse_merge(int64_t rows, int32_t parts, int32_t G, int32_t D, const void* part_o,
                         const float* part_lse, void* out, float* lse_out, msa_stream_t stream) {
  g_last_error.clear();
  MSA_REQUIRE(rows >= 0, MSA_ERR_INVALID_ARG, "rows must be >= 0");
  MSA_REQUIRE(parts >= 1 && parts <= kMaxK, MSA_ERR_UNSUPPORTED, "parts must be in [1, %d]", kMaxK);
  MSA_REQUIRE(supported_group(G), MSA_ERR_UNSUPPORTED, "G must be 1, 2, 4, 8 or 16, got %d", G);
  MSA_REQUIRE(supported_dim(D), MSA_ERR_UNSUPPORTED, "D must be 64 or 128, got %d", D);
  if (rows == 0) return MSA_OK;
  MSA_REQUIRE(part_o && part_lse && out, MSA_ERR_INVALID_ARG, "part_o, part_lse and out must be non-NULL");
  MSA_REQUIRE(aligned16(part_o) && aligned16(out) && aligned4(part_lse) && aligned4(lse_out), MSA_ERR_INVALID_ARG,
              "part_o and out must be 16-byte aligned, part_lse and lse_out 4-byte aligned");
  MSA_REQUIRE((rows + 3) / 4 <= 0x7fffffffLL, MSA_ERR_UNSUPPORTED, "rows exceeds the grid limit");
  return from_hip(msa::launch_lse_merge_bf16(rows, parts, G, D, part_o, part_lse, out, lse_out,
                                             reinterpret_cast<hipStream_t>(stream)),
                  "msa_lse_merge launch");
}

}  // extern "C"
