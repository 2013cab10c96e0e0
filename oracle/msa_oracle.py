"""CPU oracle for MiniMax Sparse Attention (MSA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it, and it shares no code with that path: it takes
plain NumPy arrays, computes in float64 from the exactly-upcast bf16 inputs, and
loops over queries the obvious way.

What it follows (the pages are the MiniMax-M3 serving write-ups: Together AI's
post and its Chinese / Russian / Japanese renderings, plus SGLang's M3.1 Flash
post):
  * Two stages: score KV blocks and keep the top-k per KV group, then run dense
    attention from the query to the selected blocks only (Chinese page, section
    "MiniMax稀疏注意力改变了服务问题"; Japanese page, "アーキテクチャ / 特徴").
  * Scoring: the query-side index vector is dotted with the key-side index
    vectors of each candidate token; every 128-token block is reduced to one
    score; each request and KV group has its own candidate range, mask and top-k
    boundary (Chinese page, "索引评分器成为解码关键路径").  The reduction op is not
    stated; this oracle takes the max over the block's valid tokens (reading R1).
  * Prefill partials: each KV block gives a partial output that a log-sum-exp
    reduction rescales and sums (Chinese page, "KV块主序稀疏注意力减少冗余KV移动").
  * Decode: the KV-group dimension is folded into the batch and a strided view
    of the KV cache (page address steps by D, tokens by Hkv*D) gives each row its
    own page table (Chinese page, "MSA需要新的分页注意力集成").

Readings of what the pages leave open (each is listed with its reason in the
design notes):
  R1 block score = max over valid tokens of q_idx . k_idx (fp64 sum, no scale);
  R2 one index vector per (token, KV group) on both sides;
  R3 candidates of a query at position p are blocks 0 .. p//128; a token s of a
     candidate block is valid iff s <= p and s < L_r;
  R4 the block holding the query is not forced in; it competes on score;
  R5 ties order by score descending, then block id ascending; selections are
     returned in ascending block id with -1 padding; k > #candidates takes all;
  R6 softmax scale 1/sqrt(D), natural exp/log; query head h uses KV head h // G;
  R7 empty partial slots carry lse = -inf and are skipped by the merge;
  R8 virtual page id of (physical page p, KV head g) in the strided view is
     p*128*Hkv + g; element (v, s, d) sits at v*D + s*Hkv*D + d.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute force, closed forms, library special cases, invariants).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(a) -> np.ndarray:
    """Exact upcast to float64 (bf16 tensors arrive as float32 or float64 arrays)."""
    return np.asarray(a, dtype=np.float64)


def num_candidates(pos: int, block: int) -> int:
    """R3: blocks 0 .. pos // block start at or before the query token."""
    return pos // block + 1


def valid_token_count(b: int, pos: int, L: int, block: int) -> int:
    """Number of tokens s in block b with s <= pos and s < L (R3)."""
    hi = min(pos + 1, L, (b + 1) * block)
    return max(0, hi - b * block)


def request_tokens(cache, block_table_row, ntok: int, block: int) -> np.ndarray:
    """Logical tokens 0..ntok-1 of one request, gathered through its block table.
    cache: [pages, block, H, D] -> returns [ntok, H, D] float64."""
    nb = -(-ntok // block)
    pages = np.asarray(block_table_row[:nb], dtype=np.int64)
    toks = _f64(cache[pages]).reshape(nb * block, *cache.shape[2:])
    return toks[:ntok]


# --- stage 1: index scores ---------------------------------------------------

def block_score(q_vec, k_rows, n_valid: int) -> float:
    """R1: the score of one block is the max over its first n_valid token rows of q_vec . k_row."""
    return float((_f64(k_rows)[:n_valid] @ _f64(q_vec)).max())


def index_scores(q_idx, kidx_cache, block_table, ctx_len, q_req, q_pos, block, max_blocks=None):
    """Block scores [Nq, Hkv, max_blocks] (float64): score[t, g, b] is the max over valid
    tokens s of block b of q_idx[t, g] . k_idx[s, g]; non-candidate blocks hold -inf."""
    q_idx = _f64(q_idx)
    Nq, Hkv, _ = q_idx.shape
    if max_blocks is None:
        max_blocks = block_table.shape[1]
    out = np.full((Nq, Hkv, max_blocks), NEG_INF)
    for t in range(Nq):
        r, p = int(q_req[t]), int(q_pos[t])
        L = int(ctx_len[r])
        for b in range(num_candidates(p, block)):
            page = int(block_table[r, b])
            n = valid_token_count(b, p, L, block)
            for g in range(Hkv):
                out[t, g, b] = block_score(q_idx[t, g], kidx_cache[page, :, g, :], n)
    return out


# --- stage 1b: top-k ---------------------------------------------------------

def topk_blocks(scores, q_pos, block, k):
    """R5: per (query, group), the min(k, n_cand) best candidates by (score desc, id asc),
    returned in ascending id order, padded with -1; plus the count."""
    Nq, Hkv, _ = scores.shape
    sel = np.full((Nq, Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((Nq, Hkv), dtype=np.int32)
    for t in range(Nq):
        n = num_candidates(int(q_pos[t]), block)
        ids = np.arange(n)
        for g in range(Hkv):
            s = np.asarray(scores[t, g, :n])
            order = np.lexsort((ids, -s))          # primary: -score, secondary: id
            chosen = np.sort(order[:min(k, n)])
            sel[t, g, :len(chosen)] = chosen
            cnt[t, g] = len(chosen)
    return sel, cnt


# --- stage 2: attention over the selected blocks ----------------------------

def attend(qv, keys, vals, scale):
    """One query head over a key set: softmax(scale * keys . qv) applied to vals -> (o [D], lse)."""
    qv, keys, vals = _f64(qv), _f64(keys), _f64(vals)
    logits = (keys @ qv) * scale
    m = logits.max()
    w = np.exp(logits - m)
    s = w.sum()
    return (w @ vals) / s, m + math.log(s)


def selected_kv(kcache, vcache, block_table_row, sel_row, cnt, g, pos, L, block):
    """Keys and values [n, D] of the valid tokens of the selected blocks of KV head g, in
    selection order (gathered page by page through the block table)."""
    ks, vs = [], []
    for b in sel_row[:cnt]:
        n = valid_token_count(int(b), pos, L, block)
        page = int(block_table_row[int(b)])
        ks.append(_f64(kcache[page, :n, g]))
        vs.append(_f64(vcache[page, :n, g]))
    return np.concatenate(ks), np.concatenate(vs)


def sparse_attention(q, kcache, vcache, block_table, ctx_len, q_req, q_pos, sel, cnt, block, scale):
    """out[t, h] = softmax(scale * q[t,h] . K_S) V_S over the union S of valid tokens of the blocks
    selected for (t, g = h // G); lse[t, h] = log sum exp of the same logits."""
    q = _f64(q)
    Nq, Hq, D = q.shape
    Hkv = sel.shape[1]
    G = Hq // Hkv
    out = np.zeros((Nq, Hq, D))
    lse = np.zeros((Nq, Hq))
    for t in range(Nq):
        r, p = int(q_req[t]), int(q_pos[t])
        L = int(ctx_len[r])
        for g in range(Hkv):
            K, V = selected_kv(kcache, vcache, block_table[r], sel[t, g], int(cnt[t, g]), g, p, L, block)
            for h in range(g * G, (g + 1) * G):
                out[t, h], lse[t, h] = attend(q[t, h], K, V, scale)
    return out, lse


def block_partials(q, kcache, vcache, block_table, ctx_len, q_req, q_pos, sel, cnt, block, scale):
    """Per selected block j: O_j = softmax within block j applied to V, lse_j = log sum exp
    within block j.  Shapes [Nq, Hkv, k, G, D] and [Nq, Hkv, k, G]; empty slots hold
    O = 0 and lse = -inf (R7)."""
    q = _f64(q)
    Nq, Hq, D = q.shape
    _, Hkv, k = sel.shape
    G = Hq // Hkv
    po = np.zeros((Nq, Hkv, k, G, D))
    pl = np.full((Nq, Hkv, k, G), NEG_INF)
    for t in range(Nq):
        r, p = int(q_req[t]), int(q_pos[t])
        L = int(ctx_len[r])
        for g in range(Hkv):
            for j in range(int(cnt[t, g])):
                b = int(sel[t, g, j])
                n = valid_token_count(b, p, L, block)
                page = int(block_table[r, b])
                K = _f64(kcache[page, :n, g])
                V = _f64(vcache[page, :n, g])
                for i in range(G):
                    po[t, g, j, i], pl[t, g, j, i] = attend(q[t, g * G + i], K, V, scale)
    return po, pl


def lse_merge(part_o, part_lse):
    """LSE = log sum_j exp(lse_j);  O = sum_j exp(lse_j - LSE) * O_j, skipping lse_j = -inf.
    part_o [..., parts, G, D], part_lse [..., parts, G] -> (O [..., G, D], LSE [..., G])."""
    po = _f64(part_o)
    pl = _f64(part_lse)
    m = pl.max(axis=-2, keepdims=True)
    w = np.where(np.isneginf(pl), 0.0, np.exp(pl - m))
    s = w.sum(axis=-2, keepdims=True)
    lse = (m + np.log(s))[..., 0, :]
    o = (w[..., None] * np.where(np.isneginf(pl)[..., None], 0.0, po)).sum(axis=-3) / s[..., 0, :, None]
    return o, lse


# --- decode: sparse per-row page table over strided views ---------------------

def sparse_page_table(sel, cnt, block_table, ctx_len, q_req, q_pos, Hkv, block):
    """R8: row rho = t*Hkv + g; page_table[rho, j] = block_table[r, sel[t,g,j]]*block*Hkv + g
    (virtual page id in the strided view), -1 past cnt; row_len[rho] = number of valid tokens
    over the selected blocks."""
    Nq = sel.shape[0]
    k = sel.shape[2]
    pt = np.full((Nq * Hkv, k), -1, dtype=np.int64)
    rl = np.zeros(Nq * Hkv, dtype=np.int64)
    for t in range(Nq):
        r, p = int(q_req[t]), int(q_pos[t])
        L = int(ctx_len[r])
        for g in range(Hkv):
            rho = t * Hkv + g
            for j in range(int(cnt[t, g])):
                b = int(sel[t, g, j])
                pt[rho, j] = int(block_table[r, b]) * block * Hkv + g
                rl[rho] += valid_token_count(b, p, L, block)
    return pt, rl


def paged_decode_attention(q, k_flat, v_flat, page_table, row_len, page_stride, token_stride,
                           block, scale):
    """Attention per flattened row read through the strided view: the token at position i of
    row rho is virtual page v = page_table[rho, i // block], slot s = i % block, and its
    element d sits at v*page_stride + s*token_stride + d of the flat cache.
    q [rows, G, D] -> (out [rows, G, D], lse [rows, G])."""
    q = _f64(q)
    rows, G, D = q.shape
    kf = _f64(k_flat).ravel()
    vf = _f64(v_flat).ravel()
    out = np.zeros((rows, G, D))
    lse = np.zeros((rows, G))
    d = np.arange(D)
    for rho in range(rows):
        n = int(row_len[rho])
        i = np.arange(n)
        v = np.asarray(page_table[rho], dtype=np.int64)[i // block]
        addr = v[:, None] * page_stride + (i % block)[:, None] * token_stride + d[None, :]
        K, V = kf[addr], vf[addr]
        for h in range(G):
            out[rho, h], lse[rho, h] = attend(q[rho, h], K, V, scale)
    return out, lse


# --- KV-block-major remap ------------------------------------------------------

def kv_block_major_lists(sel, cnt, block_table, q_req, Hkv):
    """The {kv block, q} view of a selection: for each (KV head g, physical page p), the sorted
    list of (query t, slot j) that selected it."""
    lists = {}
    for t in range(sel.shape[0]):
        r = int(q_req[t])
        for g in range(Hkv):
            for j in range(int(cnt[t, g])):
                p = int(block_table[r, int(sel[t, g, j])])
                lists.setdefault((g, p), []).append((t, j))
    return {key: sorted(v) for key, v in lists.items()}
