/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) hot path for AMD MI355X (gfx950).
 *
 * MSA has two stages: index scoring with a per-(request, KV group) top-k over 128-token
 * KV blocks, then dense attention from each query to the selected blocks only
 * (Together AI's MiniMax-M3 serving write-up, Chinese rendering, section
 * "MiniMax稀疏注意力改变了服务问题"; Japanese rendering, "アーキテクチャ / 特徴").
 * Prefill runs the attention KV-block-major, {kv block, q}, and combines the
 * per-block partial outputs with a log-sum-exp reduction (section
 * "KV块主序稀疏注意力减少冗余KV移动").  Decode folds the KV-group dimension into the
 * batch and gives every flattened row its own page table over a strided view of
 * the shared paged KV tensor (section "MSA需要新的分页注意力集成").
 *
 * Conventions for every call
 *  - Memory: every array argument is DEVICE memory owned by the caller (typically a
 *    PyTorch tensor's data pointer), except the msa_batch / msa_cache structs themselves,
 *    which live in host memory and are read during the call only.  The library never
 *    allocates, frees or synchronizes.  Arrays must be contiguous, 16-byte aligned.
 *  - Types: bf16 arrays hold IEEE bfloat16 bit patterns; scores, log-sum-exps and
 *    workspaces are float32; indices are int32.
 *  - Streams: work is enqueued on `stream` (NULL = the legacy default stream) and is
 *    asynchronous; results are ready when the stream reaches that point.
 *  - Errors: arguments are validated on the host before anything is launched; an invalid
 *    or unsupported argument returns MSA_ERR_INVALID_ARG / MSA_ERR_UNSUPPORTED and launches
 *    nothing.  A failed launch returns MSA_ERR_HIP.  msa_last_error() gives a message for
 *    the calling thread's last failure.  Device-side values are trusted: a block table
 *    entry, position or selection outside the documented range is undefined behaviour.
 *  - Determinism: results are bitwise reproducible for identical inputs (no float atomics).
 *  - Thread safety: stateless; calls on different streams may run concurrently.
 *  - Supported shapes: block_size = 128; D, Di in {64, 128}; G = Hq/Hkv in {1,2,4,8,16};
 *    1 <= k <= 64; 1 <= Hkv <= 64.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* msa_stream_t;

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,
  MSA_ERR_UNSUPPORTED = 2,
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4
} msa_status;

/* A batch of requests and their query rows.  Request r owns the query rows
 * cu_q[r] .. cu_q[r+1]-1; query row t sits at absolute position q_pos[t] < ctx_len[r]
 * of its request, and its own key/value/index rows are already in the caches. */
typedef struct msa_batch {
  int32_t num_requests;        /* B >= 1 */
  int32_t num_queries;         /* Nq >= 0, equals cu_q[B] */
  int32_t max_blocks;          /* columns of block_table, >= ceil(ctx_len[r] / 128) for all r */
  int32_t max_q_per_request;   /* host-side bound on cu_q[r+1]-cu_q[r]; picks the scorer shape */
  const int32_t* block_table;  /* device [B, max_blocks]: physical page of logical block b */
  const int32_t* ctx_len;      /* device [B]: L_r, tokens in the cache (current tokens included) */
  const int32_t* cu_q;         /* device [B+1]: query row offsets, cu_q[0] = 0, non-decreasing */
  const int32_t* q_pos;        /* device [Nq]: absolute position of each query row */
} msa_batch;

/* A paged cache: device bf16 pages of [block_size, num_heads, head_dim] elements (token rows of
 * num_heads*head_dim contiguous elements), page p starting at data + p*page_stride elements.
 * page_stride = 0 means block_size*num_heads*head_dim (pages back to back: [num_pages, block_size,
 * num_heads, head_dim] contiguous).  A larger stride takes pages spaced apart, e.g. the K and V halves
 * of a pool laid out [num_pages, 2, block_size, num_heads, head_dim] (both with page_stride =
 * 2*block_size*num_heads*head_dim).  A nonzero page_stride must be at least block_size*num_heads*
 * head_dim and a multiple of 8 (16-byte aligned pages); a K or V cache's must also be a multiple of
 * head_dim (virtual page ids below).  Pages must not overlap. */
typedef struct msa_cache {
  const void* data;
  int32_t num_pages;
  int32_t block_size;          /* 128 */
  int32_t num_heads;           /* Hkv */
  int32_t head_dim;            /* D (keys/values) or Di (key index) */
  int64_t page_stride;         /* elements from one page to the next; 0 = block_size*num_heads*head_dim */
} msa_cache;

/* Stage 1, index scoring (Chinese page, section "索引评分器成为解码关键路径"; Japanese page,
 * "Decode Index Scoring Kernel Optimization"): the query-side index vector of every query
 * row and KV head is dotted with the key-side index vector of every candidate token, and
 * every 128-token block is reduced to one score, the MAX over its valid tokens (the pages
 * leave the reduction open; max is this library's reading).
 *   q_idx   device bf16 [Nq, Hkv, Di]
 *   k_idx   key-index cache [pages, 128, Hkv, Di]
 *   scores  device f32 [Nq, Hkv, max_blocks], fully written: scores[t,g,b] for the candidate
 *           blocks b = 0 .. q_pos[t]/128, -inf for every other column.  A token s of a
 *           candidate block counts iff s <= q_pos[t] and s < ctx_len[r].
 * Rows of requests with at most 16 queries (batch->max_q_per_request <= 16) go to the
 * decode kernel (one pass over each page per request, queries in the MFMA N dimension);
 * larger query counts go to the prefill GEMM kernel. */
msa_status msa_index_score(const msa_batch* batch, const void* q_idx, msa_cache k_idx, float* scores,
                           msa_stream_t stream);

/* Top-k over KV blocks (Chinese page, sections "MiniMax稀疏注意力改变了服务问题" and "遗留问题"):
 * for each (query row t, KV head g) the min(k, n_cand) candidates with the highest scores,
 * n_cand = q_pos[t]/128 + 1; equal scores prefer the lower block id.
 *   scores  device f32 [Nq, Hkv, max_blocks] as written by msa_index_score
 *   sel     device i32 [Nq, Hkv, k]: selected block ids in ascending order, -1 padding
 *   cnt     device i32 [Nq, Hkv]: number of selected blocks */
msa_status msa_topk_blocks(const msa_batch* batch, int32_t num_kv_heads, const float* scores, int32_t k,
                           int32_t* sel, int32_t* cnt, msa_stream_t stream);

/* Fused index scoring + top-k.  The pages name fusing MSA's small kernels (top-k over KV blocks,
 * per-block scoring and reduction) as the open opportunity (Chinese page, section "遗留问题";
 * Japanese page, "今後の取り組み").  The result is identical to msa_index_score followed by
 * msa_topk_blocks -- same fp32 block scores, same tie rule -- but for prefill shapes
 * (batch->max_q_per_request > 16) with k <= 16 and max_blocks <= 65536 the block scores never reach
 * memory: the scoring kernel keeps every query row's running top-16 on chip.  Other shapes run the
 * two kernels through the workspace.
 *   sel, cnt   as msa_topk_blocks
 *   workspace  device, >= msa_index_topk_workspace_size(...) bytes (may be 0 / NULL) */
msa_status msa_index_topk(const msa_batch* batch, const void* q_idx, msa_cache k_idx, int32_t k, int32_t* sel,
                          int32_t* cnt, void* workspace, size_t workspace_bytes, msa_stream_t stream);
size_t msa_index_topk_workspace_size(const msa_batch* batch, int32_t num_kv_heads, int32_t k);

/* Sparse per-row page table for decode (Chinese page, section "MSA需要新的分页注意力集成"):
 * row rho = t*Hkv + g of the flattened (query row, KV head) batch gets
 *   page_table[rho, j] = block_table[r, sel[t,g,j]] * (P / D) + g   (j < cnt[t,g]; -1 after)
 * with P the cache's page stride in elements (128 * Hkv * D for back-to-back pages, which gives the
 * pages' block_table * 128 * Hkv + g): a virtual page id in the strided view of the cache whose page
 * stride is D elements and token stride Hkv*D elements, and
 *   row_len[rho] = number of valid tokens over the selected blocks (only the last,
 *                  highest block can be partial).
 * kv_layout describes the K (or V: the same layout) cache; only its shape and page stride are read
 * (data may be NULL).  Hkv = kv_layout.num_heads; num_pages * P / D must fit in int32.
 *   page_table  device i32 [Nq*Hkv, k];  row_len  device i32 [Nq*Hkv] */
msa_status msa_build_sparse_page_table(const msa_batch* batch, msa_cache kv_layout, const int32_t* sel,
                                       const int32_t* cnt, int32_t k, int32_t* page_table, int32_t* row_len,
                                       msa_stream_t stream);

/* msa_topk_blocks followed by msa_build_sparse_page_table, in one launch when the rows fit the
 * register top-k (max_blocks <= 16384), else in two.
 * Same arguments, outputs and results as the two calls; the fusion is the one the pages name as
 * open for MSA's small kernels (Chinese page, section "遗留问题"). */
msa_status msa_topk_page_table(const msa_batch* batch, msa_cache kv_layout, const float* scores, int32_t k,
                               int32_t* sel, int32_t* cnt, int32_t* page_table, int32_t* row_len,
                               msa_stream_t stream);

/* Decode attention over the sparse page table (same section): each row rho attends with its
 * G query heads q[rho*G .. rho*G+G-1] to the first row_len[rho] tokens of its virtual pages.
 * Token i of row rho is virtual page v = page_table[rho, i/128], slot s = i%128, and its
 * element d is at k_base[v*page_stride + s*token_stride + d] (same for v_base).
 * Softmax scale sm_scale, natural-log LSE.  When there are too few rows to fill the GPU, each
 * row's pages are split over several workgroups and the last of them to finish combines the parts
 * by a log-sum-exp merge through the workspace; otherwise no workspace is used (size 0, pointer may
 * be NULL).  The workspace ends in one arrival counter per row (its last 256-byte-aligned 4*rows
 * bytes): zero the whole workspace once before its first use and pass the same workspace_bytes
 * with it on every call; each call returns the counters to zero.
 * Only a row's last page may be partial, which holds for selections in ascending block order, so
 * the same call also runs prefill rows query-major (rows = Nq*Hkv, one query token per row,
 * page table from msa_topk_page_table): each row reads its own k blocks, with no partials.
 *   q        device bf16 [rows*G, D]  (= [Nq, Hq, D] when rows = Nq*Hkv)
 *   out      device bf16 [rows*G, D]
 *   lse      device f32 [rows*G] or NULL
 *   workspace  device, >= msa_sparse_attn_decode_workspace_size(rows, G, D, k) bytes, zeroed before
 *              its first use (above)
 * Rows with row_len = 0 are invalid input; rows*k must fit in int32.  Calls that share a workspace
 * must not overlap in time. */
msa_status msa_sparse_attn_decode(int32_t rows, int32_t G, int32_t D, const void* q, const void* k_base,
                                  const void* v_base, int64_t page_stride, int64_t token_stride,
                                  const int32_t* page_table, int32_t k, const int32_t* row_len,
                                  float sm_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, msa_stream_t stream);
size_t msa_sparse_attn_decode_workspace_size(int32_t rows, int32_t G, int32_t D, int32_t k);

/* msa_topk_page_table followed by msa_sparse_attn_decode on the caches' per-KV-head strided views,
 * in one launch (the split merge included).  Each attention workgroup selects its row's blocks itself,
 * so the page table never makes a round trip through memory before attention starts; the pages name
 * handing the top-k to decode attention on chip as open work for MSA's small kernels (Chinese page,
 * section "遗留问题"; Japanese page, "今後の取り組み").  Outputs and results are identical to the
 * two calls: sel, cnt, page_table and row_len as msa_topk_page_table (all four are written), out and
 * lse as msa_sparse_attn_decode with rows = Nq*Hkv, page stride D and token stride Hkv*D.  Rows of
 * more than 4096 blocks (batch->max_blocks) run the two calls' launches instead.
 *   scores            device f32 [Nq, Hkv, max_blocks] as written by msa_index_score
 *   k_cache, v_cache  [pages, 128, Hkv, D]
 *   q                 device bf16 [Nq, Hkv*G, D];  out  device bf16 [Nq, Hkv*G, D];  lse  f32 [Nq, Hkv*G] or NULL
 *   workspace         device, >= msa_sparse_attn_decode_workspace_size(Nq*Hkv, G, D, k) bytes, zeroed
 *                     before its first use, as for msa_sparse_attn_decode */
msa_status msa_topk_attn_decode(const msa_batch* batch, const float* scores, int32_t k, msa_cache k_cache,
                                msa_cache v_cache, int32_t G, const void* q, float sm_scale, int32_t* sel,
                                int32_t* cnt, int32_t* page_table, int32_t* row_len, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, msa_stream_t stream);

/* msa_topk_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, outputs and results as
 * msa_topk_attn_decode, with no workspace: when rows have to be split over several workgroups, the split
 * partials and the row arrival counters go to a static array of MSA_DECODE_NOALLOC_SCRATCH_BYTES bytes
 * (zero when the library is loaded) that the library holds on each GPU it runs on until the process
 * ends.  This call allocates nothing (no hipMalloc, no library
 * allocation).  A batch whose split partials need more than that (msa_sparse_attn_decode_workspace_size
 * of Nq*Hkv rows above the limit: at most 16 query heads per KV head, D = 128 and close to 256 rows)
 * returns MSA_ERR_UNSUPPORTED and launches nothing.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams without ordering between them) race and give
 * undefined results; calls on one stream, or ordered by events, are safe. */
#define MSA_DECODE_NOALLOC_SCRATCH_BYTES (4u << 20)
msa_status msa_topk_attn_decode_noalloc(const msa_batch* batch, const float* scores, int32_t k, msa_cache k_cache,
                                        msa_cache v_cache, int32_t G, const void* q, float sm_scale, int32_t* sel,
                                        int32_t* cnt, int32_t* page_table, int32_t* row_len, void* out, float* lse,
                                        msa_stream_t stream);

/* KV-block-major prefill attention (section "KV块主序稀疏注意力减少冗余KV移动"; Russian page,
 * third paragraph): the selection is inverted into {(KV head, request, block) -> query rows}
 * buckets, each selected KV block is staged on chip and attended by the query rows that picked
 * it, and the partial outputs are combined afterwards by a log-sum-exp reduction (msa_lse_merge).
 * Causal masking inside a block: key s counts iff s <= q_pos[t] and s < ctx_len[r].
 *
 * tile_min_rows = 0: every selected block has its own partial, slot j for block sel[t,g,j]:
 *   part_o[t,g,j,i,:] = softmax_i(scale * q[t, g*G+i] . K_b) V_b   (normalized, bf16)
 *   part_lse[t,g,j,i] = log sum exp of the same logits            (f32; -inf for j >= cnt)
 * tile_min_rows = n >= 1, with G in {4, 8, 16}, k <= 64 and max_blocks <= 16384 (otherwise as 0):
 * some blocks of a row are attended together and share one slot.  Blocks that at least n query rows
 * of the request and KV head selected are eligible; rows of the same request and KV head are grouped
 * by their two eligible blocks with the most rows; a group's dense blocks are the eligible blocks at
 * least a quarter of its rows (and two or more) selected, at most 64.  Tiles of a group's rows stage
 * each dense block once for all of their rows that picked it, and every row keeps a running softmax
 * over the dense blocks it picked.  Then for such a row
 *   the lowest of their slots holds the softmax over the valid keys of all of them (normalized
 *   output and LSE, as above), their other slots get part_lse = -inf (part_o not written),
 * and every other selected block keeps its own slot as with 0.  The grouping depends on sel and cnt
 * only, so results are deterministic; the merged output of msa_lse_merge is the same attention
 * either way, up to rounding.
 *   q        device bf16 [Nq, Hkv*G, D]
 *   k_cache, v_cache  [pages, 128, Hkv, D]
 *   sel, cnt  from msa_topk_blocks
 *   part_o   device bf16 [Nq, Hkv, k, G, D];  part_lse  device f32 [Nq, Hkv, k, G]
 *   slot_of  device i32 [Nq, Hkv, k] or NULL: for j < cnt[t,g], the slot that holds block sel[t,g,j]'s
 *            share (slot s holds the softmax over the blocks with slot_of = s); -1 for j >= cnt
 *   workspace  device, >= msa_sparse_attn_prefill_workspace_size(...) bytes
 * Combine the partials with msa_lse_merge(rows = Nq*Hkv, parts = k, ...). */
msa_status msa_sparse_attn_prefill(const msa_batch* batch, int32_t G, const void* q, msa_cache k_cache,
                                   msa_cache v_cache, const int32_t* sel, const int32_t* cnt, int32_t k,
                                   float sm_scale, int32_t tile_min_rows, void* part_o, float* part_lse,
                                   int32_t* slot_of, void* workspace, size_t workspace_bytes, msa_stream_t stream);
/* Workspace bytes for msa_sparse_attn_prefill on this batch (0 for invalid arguments). */
size_t msa_sparse_attn_prefill_workspace_size(const msa_batch* batch, int32_t num_kv_heads, int32_t k);

/* Log-sum-exp reduction of per-block partials (section "KV块主序稀疏注意力减少冗余KV移动"):
 *   LSE = log sum_j exp(lse_j),  O = sum_j exp(lse_j - LSE) * O_j, over the parts with
 *   lse_j > -inf.  A (row, head) with no such part gets O = 0 and LSE = -inf (every read stays
 *   inside the row's own parts).
 *   part_o    device bf16 [rows, parts, G, D];  part_lse  device f32 [rows, parts, G]
 *   out       device bf16 [rows, G, D];         lse_out   device f32 [rows, G] or NULL */
msa_status msa_lse_merge(int64_t rows, int32_t parts, int32_t G, int32_t D, const void* part_o,
                         const float* part_lse, void* out, float* lse_out, msa_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char* msa_status_string(msa_status status);
/* Message describing the calling thread's most recent failure ("" if none). */
const char* msa_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int32_t msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
