"""The C ABI on the CPU: libmsa.so loads, exports every function include/msa.h declares, and rejects
invalid or unsupported arguments with the documented status before anything is launched.

The argument-error cases pass fake device addresses that are never dereferenced, because host-side
validation fails first.  They are skipped when a GPU is visible, so that a validation bug could
never turn one of them into a launch with a fake pointer.
"""
import ctypes
import os
import re

import pytest
import torch

from block_sparse_long_msa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = 0x100000  # 16-byte aligned, never dereferenced

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation cases run only without a GPU")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmsa.so is not built: run `python -m block_sparse_long_msa_amd.build`")
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), "binding and header disagree"
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} not exported"


def test_status_strings_and_version(lib):
    assert lib.msa_status_string(0) == b"MSA_OK"
    assert lib.msa_status_string(3) == b"MSA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.msa_version() >= 100


def _batch(B=2, Nq=2, max_blocks=4, maxq=1, **over):
    kw = dict(num_requests=B, num_queries=Nq, max_blocks=max_blocks, max_q_per_request=maxq, block_table=FAKE,
              ctx_len=FAKE, cu_q=FAKE, q_pos=FAKE)
    kw.update(over)
    return _lib.MsaBatch(**kw)


def _cache(P=8, BS=128, H=2, D=64, data=FAKE, page_stride=0):
    return _lib.MsaCache(data, P, BS, H, D, page_stride)


@no_gpu
@pytest.mark.parametrize("batch_over,cache_kw,status", [
    (dict(num_requests=0), {}, INVALID),
    (dict(max_blocks=0), {}, INVALID),
    (dict(block_table=None), {}, INVALID),
    (dict(q_pos=FAKE + 2), {}, INVALID),          # misaligned
    ({}, dict(BS=64), UNSUPPORTED),
    ({}, dict(D=96), UNSUPPORTED),
    ({}, dict(H=65), UNSUPPORTED),
    ({}, dict(data=None), INVALID),
])
def test_index_score_rejects(lib, batch_over, cache_kw, status):
    b = _batch(**batch_over)
    st = lib.msa_index_score(ctypes.byref(b), FAKE, _cache(**cache_kw), FAKE, None)
    assert st == status
    assert lib.msa_last_error() != b""


@no_gpu
def test_index_score_null_batch(lib):
    assert lib.msa_index_score(None, FAKE, _cache(), FAKE, None) == INVALID


@no_gpu
@pytest.mark.parametrize("k,hkv,status", [(0, 2, UNSUPPORTED), (65, 2, UNSUPPORTED), (4, 0, UNSUPPORTED)])
def test_topk_rejects(lib, k, hkv, status):
    b = _batch()
    assert lib.msa_topk_blocks(ctypes.byref(b), hkv, FAKE, k, FAKE, FAKE, None) == status


@no_gpu
def test_page_table_rejects_overflowing_virtual_ids(lib):
    b = _batch()
    kv = _cache(P=1 << 22, H=8)
    assert lib.msa_build_sparse_page_table(ctypes.byref(b), kv, FAKE, FAKE, 16, FAKE, FAKE, None) == UNSUPPORTED
    # a page stride of twice the page (K and V pages interleaved) doubles the virtual ids
    kv = _cache(P=1 << 20, H=8, page_stride=2 * 128 * 8 * 64)
    assert lib.msa_build_sparse_page_table(ctypes.byref(b), kv, FAKE, FAKE, 16, FAKE, FAKE, None) == UNSUPPORTED
    kv = _cache(P=1 << 19, H=8, page_stride=2 * 128 * 8 * 64)  # fits: the call gets past its checks
    assert lib.msa_build_sparse_page_table(ctypes.byref(_batch(Nq=0)), kv, FAKE, FAKE, 16, FAKE, FAKE, None) == OK


@no_gpu
@pytest.mark.parametrize("hkv,pages,k,ps,status", [(2, 8, 0, 0, UNSUPPORTED), (2, 8, 65, 0, UNSUPPORTED),
                                                   (0, 8, 4, 0, UNSUPPORTED), (2, 0, 4, 0, INVALID),
                                                   (8, 1 << 22, 16, 0, UNSUPPORTED),
                                                   # page strides: below the page, unaligned, not whole in D
                                                   (2, 8, 4, 128 * 2 * 64 - 8, INVALID), (2, 8, 4, 128 * 2 * 64 + 4, INVALID),
                                                   (2, 8, 4, 128 * 2 * 64 + 8, INVALID)])
def test_topk_page_table_rejects(lib, hkv, pages, k, ps, status):
    b = _batch()
    kv = _cache(P=pages, H=hkv, page_stride=ps)
    assert lib.msa_topk_page_table(ctypes.byref(b), kv, FAKE, k, FAKE, FAKE, FAKE, FAKE, None) == status


@no_gpu
def test_topk_page_table_rejects_null_outputs(lib):
    b = _batch()
    assert lib.msa_topk_page_table(ctypes.byref(b), _cache(), FAKE, 4, FAKE, FAKE, None, FAKE, None) == INVALID


@no_gpu
def test_cache_page_stride_checks(lib):
    """A cache's page stride: 0 or at least one page, 16-byte aligned; K and V alike."""
    b = _batch()
    page = 128 * 2 * 64
    assert lib.msa_index_score(ctypes.byref(b), FAKE, _cache(page_stride=page - 64), FAKE, None) == INVALID
    assert lib.msa_index_score(ctypes.byref(b), FAKE, _cache(page_stride=page + 4), FAKE, None) == INVALID
    args = (FAKE, 4, _cache(page_stride=2 * page), _cache(page_stride=page), 8, FAKE, 0.1, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, 1 << 30, None)
    assert lib.msa_topk_attn_decode(ctypes.byref(b), *args) == INVALID  # K and V page strides differ


@no_gpu
@pytest.mark.parametrize("G,D,ps,ts,k,ws,status", [
    (3, 128, 128, 1024, 16, 1 << 30, UNSUPPORTED),
    (8, 96, 96, 768, 16, 1 << 30, UNSUPPORTED),
    (8, 128, 100, 1024, 16, 1 << 30, INVALID),      # page stride not a multiple of 8 elements
    (8, 128, 128, 1024, 0, 1 << 30, UNSUPPORTED),
    (8, 128, 128, 1024, 16, 64, WS_SMALL),             # 4 rows are split: a workspace is needed
    (8, 128, 128, 1 << 24, 16, 1 << 30, UNSUPPORTED),   # token_stride*128 beyond int32
])
def test_decode_attention_rejects(lib, G, D, ps, ts, k, ws, status):
    st = lib.msa_sparse_attn_decode(4, G, D, FAKE, FAKE, FAKE, ps, ts, FAKE, k, FAKE, 0.1, FAKE, FAKE, FAKE, ws, None)
    assert st == status


@no_gpu
@pytest.mark.parametrize("G,k,kc,vc,ws,status", [
    (3, 16, dict(), dict(), 1 << 30, UNSUPPORTED),                  # G not a power of two <= 16
    (8, 0, dict(), dict(), 1 << 30, UNSUPPORTED),
    (8, 65, dict(), dict(), 1 << 30, UNSUPPORTED),
    (8, 16, dict(), dict(D=128), 1 << 30, INVALID),                 # K and V caches differ
    (8, 16, dict(H=8, P=1 << 22), dict(H=8, P=1 << 22), 1 << 30, UNSUPPORTED),   # virtual page ids beyond int32
    (8, 16, dict(BS=64), dict(BS=64), 1 << 30, UNSUPPORTED),
    (8, 16, dict(), dict(), 64, WS_SMALL),                          # 4 rows are split: a workspace is needed
])
def test_topk_attn_decode_rejects(lib, G, k, kc, vc, ws, status):
    b = _batch()
    st = lib.msa_topk_attn_decode(ctypes.byref(b), FAKE, k, _cache(**kc), _cache(**vc), G, FAKE, 0.1, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, ws, None)
    assert st == status


@no_gpu
def test_topk_attn_decode_rejects_null_outputs(lib):
    b = _batch()
    assert lib.msa_topk_attn_decode(ctypes.byref(b), FAKE, 4, _cache(), _cache(), 8, FAKE, 0.1, FAKE, FAKE, None,
                                    FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID


@no_gpu
def test_topk_attn_decode_noalloc_rejects_batches_beyond_its_scratch(lib):
    # 51 queries x 5 KV heads = 255 rows of 16 query heads at D = 128, split in two: 4,210,688 bytes of
    # partials, more than the 4 MiB static scratch
    b = _batch(B=51, Nq=51)
    kc = _cache(H=5, D=128)
    assert lib.msa_sparse_attn_decode_workspace_size(255, 16, 128, 64) > (4 << 20)
    st = lib.msa_topk_attn_decode_noalloc(ctypes.byref(b), FAKE, 64, kc, kc, 16, FAKE, 0.1, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, None)
    assert st == UNSUPPORTED and b"allocation-free" in lib.msa_last_error()
    assert lib.msa_topk_attn_decode_noalloc(ctypes.byref(b), FAKE, 65, kc, kc, 16, FAKE, 0.1, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, None) == UNSUPPORTED
    e = _batch(Nq=0)
    assert lib.msa_topk_attn_decode_noalloc(ctypes.byref(e), None, 4, _cache(), _cache(), 8, None, 0.1, None, None,
                                            None, None, None, None, None) == OK


@no_gpu
def test_prefill_attention_rejects(lib):
    b = _batch(Nq=40, maxq=40)
    kc, vc = _cache(), _cache()
    assert lib.msa_sparse_attn_prefill(ctypes.byref(b), 3, FAKE, kc, vc, FAKE, FAKE, 4, 0.1, 0, FAKE, FAKE, None, FAKE,
                                       1 << 30, None) == UNSUPPORTED
    assert lib.msa_sparse_attn_prefill(ctypes.byref(b), 4, FAKE, kc, _cache(D=128), FAKE, FAKE, 4, 0.1, 0, FAKE, FAKE,
                                       None, FAKE, 1 << 30, None) == INVALID
    assert lib.msa_sparse_attn_prefill(ctypes.byref(b), 4, FAKE, kc, vc, FAKE, FAKE, 4, 0.1, 0, FAKE, FAKE, None, FAKE, 16,
                                       None) == WS_SMALL
    assert lib.msa_sparse_attn_prefill(ctypes.byref(b), 4, FAKE, kc, vc, FAKE, FAKE, 4, 0.1, -1, FAKE, FAKE, None, FAKE,
                                       1 << 30, None) == INVALID


@no_gpu
@pytest.mark.parametrize("parts,G,D,status", [(0, 8, 128, UNSUPPORTED), (4, 5, 128, UNSUPPORTED),
                                              (4, 8, 32, UNSUPPORTED)])
def test_merge_rejects(lib, parts, G, D, status):
    assert lib.msa_lse_merge(10, parts, G, D, FAKE, FAKE, FAKE, None, None) == status


def test_empty_inputs_launch_nothing(lib):
    b = _batch(Nq=0)
    assert lib.msa_index_score(ctypes.byref(b), None, _cache(), None, None) == OK
    assert lib.msa_topk_blocks(ctypes.byref(b), 2, None, 4, None, None, None) == OK
    assert lib.msa_topk_page_table(ctypes.byref(b), _cache(), None, 4, None, None, None, None, None) == OK
    assert lib.msa_topk_attn_decode(ctypes.byref(b), None, 4, _cache(), _cache(), 8, None, 0.1, None, None, None,
                                    None, None, None, None, 0, None) == OK
    assert lib.msa_lse_merge(0, 4, 8, 128, None, None, None, None, None) == OK
    assert lib.msa_sparse_attn_decode(0, 8, 128, None, None, None, 128, 1024, None, 4, None, 0.1, None, None, None,
                                      0, None) == OK


def test_workspace_sizes(lib):
    # few rows: split over page runs (here 4 runs of 4 pages), fp32 partials + LSE per run
    assert lib.msa_sparse_attn_decode_workspace_size(64, 8, 128, 16) >= 64 * 4 * 8 * 129 * 4
    # enough rows to fill the GPU one workgroup each: no workspace
    assert lib.msa_sparse_attn_decode_workspace_size(4096, 8, 128, 16) == 0
    assert lib.msa_sparse_attn_decode_workspace_size(0, 8, 128, 16) == 0
    b = _batch(B=1, Nq=32768, max_blocks=1024, maxq=32768)
    assert lib.msa_sparse_attn_prefill_workspace_size(ctypes.byref(b), 8, 16) >= 32768 * 8 * 16 * 4
    assert lib.msa_sparse_attn_prefill_workspace_size(None, 8, 16) == 0
