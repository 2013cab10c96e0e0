"""Host replay of the prefill attention kernels' index arithmetic, with every address checked
against the buffer it falls in.

The per-block kernel (k_attn_kvbm) and the query-tile kernel (k_attn_tile) form their HBM and LDS
addresses from a work list built on the GPU (bucket counts, scans, entries, tiles).  This test
rebuilds those lists on the CPU the way the remap kernels define them, walks every workgroup of the
launch grid the way the kernels do (XCD-aware item choice, passes of query rows, padded rows, staged
key rows clamped at a partial block's end, output slots), and asserts that each index lies inside
its array.  It runs on random valid selections (ascending, -1 padded) of the tiny prefill's shape and
of ragged multi-request shapes with partial last blocks, k above the candidate count and G from 1
to 16.  No GPU is used; the constants mirror the kernels' (k_attn_prefill.hip, k_attn_tile.hip).
"""
import numpy as np
import pytest

BLOCK = 128
# k_attn_prefill.hip
K_CHUNK, K_MIN_CHUNK, K_TARGET_ITEMS, K_WAVES, K_NT, K_XCDS = 256, 32, 1024, 4, 2, 8
# k_attn_tile.hip
TILE_WAVES, TILE_NT, HALF, DENSE_MAX = 8, 2, 64, 64


def item_chunk(E, G):
    pass_ = max(K_MIN_CHUNK, K_WAVES * 16 * K_NT // G)
    c = K_CHUNK
    while c > pass_ and E // c < K_TARGET_ITEMS:
        c >>= 1
    return c


def max_items(E, NB, chunk):
    return E // chunk + min(E, NB) + 1


def random_batch(rng, ctx, nq, Hkv, k):
    """Positions, block table and a random valid selection (ascending ids among each row's candidates)."""
    B = len(ctx)
    mb = max(-(-L // BLOCK) for L in ctx)
    pages = rng.permutation(sum(-(-L // BLOCK) for L in ctx))
    bt = np.zeros((B, mb), dtype=np.int64)
    o = 0
    for r, L in enumerate(ctx):
        n = -(-L // BLOCK)
        bt[r, :n] = pages[o:o + n]
        o += n
    cu = np.concatenate([[0], np.cumsum(nq)])
    pos = np.concatenate([np.arange(L - n, L) for L, n in zip(ctx, nq)])
    req = np.repeat(np.arange(B), nq)
    Nq = int(cu[-1])
    sel = np.full((Nq, Hkv, k), -1, dtype=np.int64)
    cnt = np.zeros((Nq, Hkv), dtype=np.int64)
    for t in range(Nq):
        ncand = pos[t] // BLOCK + 1
        for g in range(Hkv):
            c = min(k, ncand)
            sel[t, g, :c] = np.sort(rng.choice(ncand, size=c, replace=False))
            cnt[t, g] = c
    return dict(ctx=np.asarray(ctx), bt=bt, cu=cu, pos=pos, req=req, sel=sel, cnt=cnt, Nq=Nq, B=B, mb=mb,
                P=len(pages))


def replay_kvbm(x, Hkv, G, D, k, covered=None):
    """Remap (count, scan, fill) and every workgroup of k_attn_kvbm; covered[t, g, j] marks entries the
    tile path takes instead."""
    Nq, B, mb = x["Nq"], x["B"], x["mb"]
    NB, E = Hkv * B * mb, Nq * Hkv * k
    counts = np.zeros(NB, dtype=np.int64)
    lists = {}
    for t in range(Nq):
        r = int(x["req"][t])
        for g in range(Hkv):
            for j in range(int(x["cnt"][t, g])):
                if covered is not None and covered[t, g, j]:
                    continue
                bucket = (g * B + r) * mb + int(x["sel"][t, g, j])
                assert 0 <= bucket < NB
                counts[bucket] += 1
                lists.setdefault(bucket, []).append(t * 64 + j)
    chunk = item_chunk(E, G)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    nitems = -(-counts // chunk)
    item_off = np.concatenate([[0], np.cumsum(nitems)])
    items = [(i, c) for i in range(NB) for c in range(int(nitems[i]))]
    assert len(items) <= max_items(E, NB, chunk)
    entries = np.zeros(E, dtype=np.int64)
    for bucket, lst in lists.items():
        entries[offsets[bucket]:offsets[bucket] + len(lst)] = lst
    # the launch: grid = max_items rounded up to whole XCD rounds; workgroup -> item as in the kernel
    mi = max_items(E, NB, chunk)
    grid = -(-mi // K_XCDS) * K_XCDS
    n_items = int(item_off[NB])
    per_xcd = -(-n_items // K_XCDS)
    seen = np.zeros(n_items, dtype=np.int64)
    rows_per_pass, tpw = 16 * K_NT, 16 * K_NT // G
    stores = 0
    for wg in range(grid):
        slot = wg // K_XCDS
        item = (wg % K_XCDS) * per_xcd + slot
        if slot >= per_xcd or item >= n_items:
            continue
        seen[item] += 1
        bucket, ch = items[item]
        g, rb = bucket // (B * mb), bucket % (B * mb)
        r, b = rb // mb, rb % mb
        e_begin = int(offsets[bucket]) + ch * chunk
        e_end = min(e_begin + chunk, int(offsets[bucket + 1]))
        n_e = e_end - e_begin
        assert 0 < n_e <= K_CHUNK, "the item's entries must fit the LDS lists"
        page = int(x["bt"][r, b])
        assert 0 <= page < x["P"]
        in_block = min(BLOCK, int(x["ctx"][r]) - b * BLOCK)
        assert 1 <= in_block <= BLOCK, "a selected block has at least one existing key"
        # staging: token rows clamped to the block's existing keys
        toks = np.minimum(np.arange(BLOCK), in_block - 1)
        kv_elem = (page * BLOCK * Hkv + g) * D + toks * Hkv * D
        assert kv_elem.min() >= 0 and kv_elem.max() + D <= x["P"] * BLOCK * Hkv * D
        for w in range(K_WAVES):
            for lb in range(w * tpw, n_e, K_WAVES * tpw):
                for rr in range(rows_per_pass):
                    li, h = lb + rr // G, rr % G
                    packed = int(entries[e_begin + min(li, n_e - 1)])   # padded rows read the last entry
                    t = packed >> 6
                    assert 0 <= t < Nq
                    q_elem = (t * Hkv * G + g * G + h) * D
                    assert 0 <= q_elem and q_elem + D <= Nq * Hkv * G * D
                    tj = packed if li < n_e else -1
                    tjc = max(tj, 0)
                    orow = (((tjc >> 6) * Hkv + g) * k + (tjc & 63)) * G + h
                    assert 0 <= orow < Nq * Hkv * k * G, "output slot out of range"
                    if tj >= 0:
                        j = tj & 63
                        assert j < x["cnt"][t, g] and int(x["sel"][t, g, j]) == b
                        stores += 1
    assert np.all(seen == 1), "every work item runs exactly once"
    expect = (x["cnt"].sum() - (0 if covered is None else covered.sum())) * G
    assert stores == expect, "every uncovered (t, g, j, head) is stored exactly once"


def replay_tiles(x, Hkv, G, D, k, n_min):
    """Bucketing, dense sets and every workgroup of k_attn_tile (index ranges only); returns the
    covered entries for the per-block replay."""
    Nq, B, mb = x["Nq"], x["B"], x["mb"]
    sel, cnt, req = x["sel"], x["cnt"], x["req"]
    counts = {}
    for t in range(Nq):
        for g in range(Hkv):
            for j in range(int(cnt[t, g])):
                key = (g * B + int(req[t]), int(sel[t, g, j]))
                counts[key] = counts.get(key, 0) + 1
    # buckets: exact (segment, a1, a2) groups stand in for the hash (collisions only merge groups)
    groups = {}
    for t in range(Nq):
        seg0 = int(req[t])
        for g in range(Hkv):
            elig = [int(sel[t, g, j]) for j in range(int(cnt[t, g])) if counts[(g * B + seg0, int(sel[t, g, j]))] >= n_min]
            if not elig:
                continue
            order = sorted(elig, key=lambda b: (-counts[(g * B + seg0, b)], b))
            groups.setdefault((g * B + seg0, order[0], order[1] if len(order) > 1 else -1), []).append(t)
    TT = 256 // G
    tpw = 16 * TILE_NT // G
    # the launch: grid = a bound on the tiles rounded up to whole XCD rounds; workgroup -> tile as in the
    # kernel (each XCD takes one contiguous run of tiles), every tile exactly once
    n_tiles = sum(-(-len(rows) // TT) for rows in groups.values())
    for bound in (n_tiles, n_tiles + 5, 2 * n_tiles + 13):
        grid = -(-bound // K_XCDS) * K_XCDS
        per_xcd = -(-n_tiles // K_XCDS)
        seen = np.zeros(n_tiles, dtype=int)
        for wg in range(grid):
            slot = wg // K_XCDS
            item = (wg % K_XCDS) * per_xcd + slot
            if slot >= per_xcd or item >= n_tiles:
                continue
            seen[item] += 1
        assert np.all(seen == 1), "every tile runs exactly once"
    covered = np.zeros(sel.shape, dtype=bool)
    for (seg, _, _), rows in groups.items():
        g, r = seg // B, seg % B
        hist = {}
        for t in rows:
            for j in range(int(cnt[t, g])):
                b = int(sel[t, g, j])
                if counts[(seg, b)] >= n_min:
                    hist[b] = hist.get(b, 0) + 1
        thr = max((len(rows) + 3) // 4, 2)
        dense = sorted(sorted((b for b in hist if hist[b] >= thr), key=lambda b: (-hist[b], b))[:DENSE_MAX])
        if not dense:
            continue
        for t in rows:
            for j in range(int(cnt[t, g])):
                if int(sel[t, g, j]) in dense:
                    covered[t, g, j] = True
        L = int(x["ctx"][r])
        for c0 in range(0, len(rows), TT):
            tile = rows[c0:c0 + TT]
            n_tok = len(tile)
            for s in range(2 * len(dense) + 2):         # steps past the end re-load the last half
                sc = min(s, 2 * len(dense) - 1)
                b, hf = dense[sc >> 1], sc & 1
                page = int(x["bt"][r, b])
                in_block = min(BLOCK, L - b * BLOCK)
                assert 0 <= page < x["P"] and in_block >= 1
                srow = np.minimum(HALF * hf + np.arange(HALF), in_block - 1)
                assert srow.min() >= 0 and srow.max() < BLOCK
            for w in range(TILE_WAVES):
                for rr in range(16 * TILE_NT):
                    tau, h = w * tpw + rr // G, rr % G
                    tq = tile[min(tau, n_tok - 1)]
                    q_elem = (tq * Hkv * G + g * G + h) * D
                    assert 0 <= q_elem and q_elem + D <= Nq * Hkv * G * D
                    if tau < n_tok:
                        t = tile[tau]
                        js = [j for j in range(int(cnt[t, g])) if covered[t, g, j]]
                        if js:
                            orow = ((t * Hkv + g) * k + js[0]) * G + h
                            assert 0 <= orow < Nq * Hkv * k * G
    return covered


CASES = [  # (context lengths, query counts, Hkv, G, D, k)
    ([2048], [2048], 2, 4, 64, 4),                      # the tiny prefill's shape
    ([700, 300, 1000], [300, 300, 129], 2, 8, 128, 5),  # ragged, partial last blocks
    ([400, 129], [250, 129], 2, 2, 64, 8),              # k above the candidate count
    ([900, 520], [400, 130], 2, 16, 64, 3),
    ([640], [640], 4, 1, 128, 2),
    ([300 + 37 * i for i in range(12)], [1 + (i % 7) * 9 for i in range(12)], 4, 4, 128, 3),
    # more (KV head, request, block) buckets than one LDS histogram holds (the global-atomic remap)
    ([100000, 90000, 50000], [10, 5, 20], 8, 2, 64, 8),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_kvbm_indices_in_range(case):
    ctx, nq, Hkv, G, D, k = CASES[case]
    x = random_batch(np.random.default_rng(100 + case), ctx, nq, Hkv, k)
    replay_kvbm(x, Hkv, G, D, k)


@pytest.mark.parametrize("case", [0, 1, 3, 5])
@pytest.mark.parametrize("n_min", [1, 3])
def test_tile_and_residual_indices_in_range(case, n_min):
    ctx, nq, Hkv, G, D, k = CASES[case]
    x = random_batch(np.random.default_rng(200 + case), ctx, nq, Hkv, k)
    covered = replay_tiles(x, Hkv, G, D, k, n_min)
    replay_kvbm(x, Hkv, G, D, k, covered)


def test_long_prefill_shape_vectorized():
    """The long prefill's shape (32,768 rows over a 98,304-token prefix, 8 KV heads of 8 query heads,
    D = 128, top-16), on a random valid selection: the remap's buckets, offsets and work items, and for
    every entry the Q, output-slot, LSE and K/V element indices the per-block kernel forms, checked in
    int64 against their arrays (vectorized; the per-workgroup walk above is too slow at this size)."""
    rng = np.random.default_rng(300)
    Nq, prefix, Hkv, G, D, k = 32768, 98304, 8, 8, 128, 16
    L = prefix + Nq
    mb = L // BLOCK
    pos = np.arange(prefix, L)
    ncand = pos // BLOCK + 1
    # k distinct blocks per (row, KV head) among the row's candidates, ascending
    sel = np.empty((Nq, Hkv, k), dtype=np.int64)
    for g in range(Hkv):
        keys = rng.random((Nq, mb), dtype=np.float32)
        keys[np.arange(mb)[None, :] >= ncand[:, None]] = 2.0          # never among the k smallest
        sel[:, g, :] = np.sort(np.argpartition(keys, k, axis=1)[:, :k], axis=1)
    assert np.all(sel < ncand[:, None, None])
    bt = rng.permutation(mb)                                          # one request's pages
    P = mb
    E = Nq * Hkv * k
    t = np.repeat(np.arange(Nq), Hkv * k)
    g = np.tile(np.repeat(np.arange(Hkv), k), Nq)
    j = np.tile(np.arange(k), Nq * Hkv)
    b = sel.reshape(-1)
    NB = Hkv * 1 * mb
    bucket = g * mb + b
    assert bucket.min() >= 0 and bucket.max() < NB
    counts = np.bincount(bucket, minlength=NB)
    chunk = item_chunk(E, G)
    assert chunk <= K_CHUNK
    nitems = -(-counts // chunk)
    assert nitems.sum() <= max_items(E, NB, chunk)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    assert offsets[-1] == E and E < 2 ** 31, "entry indices fit in int32"
    code = t * 64 + j
    assert code.max() < 2 ** 31 and np.array_equal(code >> 6, t) and np.array_equal(code & 63, j)
    # per entry: Q of each of the G heads, output slot, partial and LSE elements, staged K/V rows
    Hq = Hkv * G
    for h in (0, G - 1):
        q_elem = (t * Hq + g * G + h) * D
        assert q_elem.min() >= 0 and q_elem.max() + D <= Nq * Hq * D
        orow = ((t * Hkv + g) * k + j) * G + h
        assert orow.min() >= 0 and orow.max() < Nq * Hkv * k * G
        assert orow.max() * D + D <= Nq * Hkv * k * G * D                 # part_o, indexed in int64
        assert orow.max() * D >= 2 ** 31, "this shape needs 64-bit partial offsets"
    page = bt[b]
    in_block = np.minimum(BLOCK, L - b * BLOCK)
    assert in_block.min() >= 1
    last_tok = np.minimum(BLOCK - 1, in_block - 1)
    kv_elem = (page * BLOCK * Hkv + g) * D + last_tok * Hkv * D
    assert kv_elem.min() >= 0 and kv_elem.max() + D <= P * BLOCK * Hkv * D
    # work items: every item's entries inside its bucket, at most one chunk of them
    item_bucket = np.repeat(np.arange(NB), nitems)
    first = np.concatenate([[0], np.cumsum(nitems)])[:-1]
    item_chunk_idx = np.arange(nitems.sum()) - np.repeat(first, nitems)
    e_begin = offsets[item_bucket] + item_chunk_idx * chunk
    e_end = np.minimum(e_begin + chunk, offsets[item_bucket + 1])
    assert np.all(e_end > e_begin) and np.all(e_end - e_begin <= K_CHUNK)
    assert (e_end - e_begin).sum() == E
