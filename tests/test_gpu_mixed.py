"""GPU parity of the mixed decode/prefill launch (fe_paged_gqa_mixed) against
the fp64 oracle.

A decode row is the chunk of length one of its sequence, so the oracle's
chunked-prefill definition covers every row of a mixed batch.  Cases: small
ragged batches for several group sizes and split-K factors with NaN/large
poison (decode rows with empty, partial-block and multi-partition contexts),
batches that are all decode or all prefill, workspace reuse, and the full
Qwen3-4B mixed step on every row.  Gate: max-abs 1e-2, row-relative 1e-2,
LSE 1e-3.
"""
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs
from gpu_util import DeviceWorkload, assert_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_mixed(w, dev, parts=(0,), label="", rows=None):
    dw = DeviceWorkload(w, dev)
    rk, rv = dw.append()
    ro, rl = oracle.prefill_chunk(dw.lay.q, w.query_start_loc, rk, rv, w.block_tables, w.context_lens, w.scale,
                                  rows=rows)
    for P in parts:
        out, lse = dw.mixed(num_partitions=P)
        if rows is not None:
            idx = torch.as_tensor(rows, dtype=torch.long, device=dev)
            out, lse = out[idx], lse[idx]
        assert_attention(out, lse, ro, rl, f"{label} P={P}")
    return dw


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("poison", ["nan", "large"])
def test_mixed_small(dev, G, poison):
    # decode rows: empty, one token, a partial block, a block boundary, several
    # 64-block partitions; then prefill chunks (one of a single row)
    lens = [0, 1, 17, 32, 2100, 700, 1, 40, 300, 129]
    nd = 6
    w = inputs.custom("mixed", len(lens), 2 * G, 2, lens, 600 + G, append=64, chunk=64, num_decode=nd,
                      poison=poison)
    run_mixed(w, dev, parts=(0, 1, 3, 5), label=f"mixed G={G} {poison}")


def test_mixed_all_decode(dev):
    lens = [5, 1000, 3000, 64]
    w = inputs.custom("mixed", 4, 32, 8, lens, 611, num_decode=4)
    run_mixed(w, dev, parts=(0, 1, 4), label="all decode")


def test_mixed_all_prefill(dev):
    lens = [100, 300]
    w = inputs.custom("mixed", 2, 32, 8, lens, 612, append=90, chunk=90, num_decode=0)
    run_mixed(w, dev, parts=(0,), label="all prefill")


def test_mixed_matches_separate_calls(dev):
    """The mixed launch agrees with decode + prefill launched separately."""
    lens = [900, 2500, 400, 333]
    w = inputs.custom("mixed", 4, 32, 8, lens, 613, append=50, chunk=50, num_decode=2)
    dw = run_mixed(w, dev, parts=(0,), label="mixed vs separate")
    out, lse = dw.mixed()
    o2 = torch.empty(2, 32, 128, dtype=torch.bfloat16, device=dev)
    l2 = torch.empty(2, 32, dtype=torch.float32, device=dev)
    fe.fe_paged_gqa_decode(o2, l2, dw.q[:2].contiguous(), dw.kc, dw.vc, dw.bt[:2].contiguous(), dw.lens[:2].contiguous(),
                           w.max_context_len, w.scale)
    torch.cuda.synchronize()
    assert (o2.float() - out[:2].float()).abs().max().item() <= 2e-2
    assert (l2 - lse[:2]).abs().max().item() <= 2e-3


def test_mixed_workspace_reuse(dev):
    """One workspace, zero-filled once, serves calls with several partition
    counts; results match and its arrival counters return to zero."""
    lens = [3000, 1500, 64, 17, 700]
    w = inputs.custom("mixed", 5, 32, 8, lens, 614, append=40, chunk=40, num_decode=3)
    dw = DeviceWorkload(w, dev)
    rk, rv = dw.append()
    ro, rl = oracle.prefill_chunk(dw.lay.q, w.query_start_loc, rk, rv, w.block_tables, w.context_lens, w.scale)
    parts = (0, 4, 12, 2, 0)
    size = max(fe.fe_paged_gqa_mixed_workspace_size(3, 32, 8, 128, w.max_context_len, P) for P in parts)
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)
    for P in parts:
        out, lse = dw.mixed(num_partitions=P, workspace=ws)
        assert_attention(out, lse, ro, rl, f"reuse P={P}")
        assert int(ws[: 3 * 8 * 4].view(torch.int32).abs().sum()) == 0, "arrival counters not reset"


@pytest.mark.parametrize("seed", [7, 8, 9])
def test_mixed_qwen3_4b_step(dev, seed):
    """The full mixed step (60 decode rows of 1024..8192 tokens and 4 chunks of
    256 after 4096 cached tokens) on every row."""
    w = inputs.make("qwen3_4b_mixed_dec60_ctx1024-8192_pre4_prefix4096_chunk256", seed=seed, poison="nan")
    run_mixed(w, dev, parts=(0, 16), label=f"mixed 4b step seed {seed}")
