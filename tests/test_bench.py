"""CPU checks of bench.py's contract and of the work counts its metrics divide by.

The flop count of the chunked-prefill workload is pinned to the figure derived
independently from the workload's definition (4 sequences, 4096 cached tokens
plus a 256-token chunk, 32 query heads, head_dim 128): every chunk row i sees
4096 + i + 1 keys, so the unmasked (query, key, head) triples number
4 * 32 * sum_{i<256} (4097 + i) = 138,428,416, at 4 * 128 flop each.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_gqa_slot_amd import inputs  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_flops_of_the_chunked_prefill_workload():
    w = inputs.make("qwen3_4b_b4_prefix4096_chunk256")
    triples = 4 * 32 * sum(4097 + i for i in range(256))
    assert triples == 138_428_416
    assert bench.prefill_flops(w) == triples * 4 * 128 == 70_875_348_992


def test_prefill_flops_of_ragged_chunks():
    # two sequences: 10 cached + 3 new, 0 cached + 2 new; Hq = 8
    w = inputs.custom("prefill", 2, 8, 2, [13, 2], 11, append=3, chunk=3)
    qsl = w.query_start_loc.tolist()
    lens = w.context_lens.tolist()
    visible = 0
    for b in range(2):
        C = qsl[b + 1] - qsl[b]
        visible += sum(lens[b] - C + i + 1 for i in range(C))
    assert bench.prefill_flops(w) == visible * 8 * 4 * 128
    # rows counted one by one add up to the same total
    assert sum(bench.prefill_row_flops(w, r) for r in range(qsl[-1])) == bench.prefill_flops(w)


def test_prefill_flops_rows_before_the_context_count_nothing():
    w = inputs.custom("prefill", 1, 8, 2, [40], 13, append=40, chunk=40)
    w.context_lens[0] = 37  # rows 0..2 of the chunk sit before the context
    assert bench.prefill_flops(w) == sum(range(1, 38)) * 8 * 4 * 128


def test_decode_bytes_formula():
    lens = [1, 16, 17, 300]
    w = inputs.custom("decode", 4, 16, 4, lens, 12, append=1)
    kv = sum(lens) * 4 * 128 * 2 * 2
    blocks = sum((L + 15) // 16 for L in lens)
    expect = kv + 4 * 16 * 128 * 2 * 2 + 4 * 16 * 4 + blocks * 4 + 4 * 4
    assert bench.decode_bytes(w) == expect


def test_norm_rope_bytes_formula():
    T, Hq, Hkv = 10, 32, 8
    rows = T * (Hq + 2 * Hkv)
    assert bench.norm_rope_bytes(T, Hq, Hkv) == rows * 256 * 2 + T * (128 * 4 + 8)


@pytest.mark.parametrize("n", [1, 2, 10, 11, 50])
def test_spread_picks_order_statistics(n):
    per = sorted(float(i) for i in range(n))
    s = bench.spread(per)
    assert s["p50_ms"] == per[int(0.5 * (n - 1) + 0.5)]
    assert per[0] <= s["p10_ms"] <= s["p50_ms"] <= s["p90_ms"] <= per[-1]
