"""Host-side choices the binding makes (no device, no kernel)."""

import pytest

import paged_kv_cache_253_amd as pk


@pytest.mark.parametrize("num_seqs,max_query_len,max_context_len,expect", [
    (16, 5, 4096, 1024),     # 128 units: split until 512 work units
    (32, 5, 4096, 2048),
    (48, 5, 4096, 2048),
    (64, 5, 4096, 0),        # 512 units: two per compute unit unsplit
    (128, 5, 4096, 0),
    (16, 5, 1000, 0),        # short contexts stay unsplit
    (1, 5, 100_000, 1024),   # one long sequence: 8 units x 98 partitions
    (8, 512, 8192, 0),       # chunked prefill: 64 query tiles per (sequence, KV head)
    (1, 1, 1 << 20, 4096),   # 8 units x 256 pieces of 4096 tokens
])
def test_prefill_partition(num_seqs, max_query_len, max_context_len, expect):
    got = pk.prefill_partition(num_seqs, 32, 8, 128, max_query_len, max_context_len, True,
                               compute_units=256)
    assert got == expect


def test_prefill_partition_falls_back_to_512():
    # 1 sequence, 1 KV head, one query tile, 8K context: 8 pieces of 1024 < 512 units
    assert pk.prefill_partition(1, 4, 1, 128, 1, 8192, True, compute_units=256) == 512


def test_prefill_partition_four_tiles_per_wavefront():
    # fp8 cache (four 16-column tiles): rows per tile double, units halve
    two = pk.prefill_partition(40, 32, 8, 128, 64, 4096, True, compute_units=256)
    four = pk.prefill_partition(40, 32, 8, 128, 64, 4096, False, compute_units=256)
    assert two == 0 and four == 0
    assert pk.prefill_partition(4, 32, 8, 128, 64, 4096, True, compute_units=256) == 2048
    assert pk.prefill_partition(4, 32, 8, 128, 64, 4096, False, compute_units=256) == 1024
