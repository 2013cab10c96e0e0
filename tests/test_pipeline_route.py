"""The prefill pipeline's default choice between the fused score + top-k call and the two calls, on
the CPU: the fused call runs one workgroup per (256 query rows, KV head) and cannot split a row's
blocks, so it is taken only when that launch has at least 256 workgroups."""
import pytest

from block_sparse_long_msa_amd.pipeline import MSAPrefill


@pytest.mark.parametrize("num_queries,hkv,fused", [
    (32768, 8, True),    # long prefill: 128 row tiles x 8 KV heads = 1024 workgroups
    (2048, 2, False),    # tiny prefill: 8 x 2 = 16 workgroups
    (8192, 8, True),     # 32 x 8 = 256: the threshold itself
    (7936, 8, False),    # 31 x 8 = 248
    (7937, 8, True),     # a partial last tile still counts: 32 x 8
    (1, 64, False),      # one row, the most KV heads
    (65536, 4, True),
])
def test_default_route(num_queries, hkv, fused):
    assert MSAPrefill.prefers_fused(num_queries, hkv) is fused
