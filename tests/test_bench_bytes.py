"""Algorithmic byte accounting of bench.py (the roofline's numerator), against
sizes worked out by hand from the cache layout: per (b, KV head, token) the
key row, its fp16 norm, the value row and its norm, plus the key side
streams; per launch the query and the output."""
import dataclasses

import bench
import workloads as W


def test_llama7b_layer_bytes():
    by = bench.cache_bytes(W.WORKLOADS["llama7b_layer"])
    assert by["per_token_head"] == 64 + 2 + 64 + 2                      # 4-bit rows at d = 128
    assert by["cache"] == 8 * 8 * 8192 * 132 == 69_206_016
    assert by["q"] == 8 * 32 * 128 * 2 and by["out"] == 8 * 32 * 128 * 4
    assert by["append_token"] == 8 * 8 * (2 * 128 * 2 + 132)


def test_side_stream_bytes():
    wl = dataclasses.replace(W.WORKLOADS["llama7b_layer"], k_bits=3)
    # 3-bit codes + 128 sign bits + fp16 residual norm + fp16 norm: the page's 68-byte key
    assert bench.cache_bytes(wl, qjl=True)["per_token_head"] == (48 + 16 + 2 + 2) + (64 + 2)
    # outlier stream: 8 int8 codes and an fp32 scale per token
    assert bench.cache_bytes(W.WORKLOADS["llama7b_layer"], outliers=8)["per_token_head"] == 132 + 8 + 4


def test_two_tier_bytes():
    wl = W.WORKLOADS["two_tier"]
    by = bench.cache_bytes(wl)
    assert wl.near_len == 1638 and wl.far_len == 16384 - 1638
    assert by["per_token_head"] == 128 + 64 + 2                         # fp8 key (no norm), 4-bit value
    assert 14746 * 194 + 1638 * 2 * 128 * 2 == 3_699_380                  # bytes per (b, head)
    assert by["cache"] == 16 * 16 * 3_699_380
