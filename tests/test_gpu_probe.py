"""GPU check of the HBM read probe used by bench.py as its same-run read
ceiling: every listed in-range tile is read whole (its words XOR-fold into
the wave's sink word) and out-of-range ids are skipped."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_slot_amd as fe

pytestmark = pytest.mark.gpu


def test_probe_reads_listed_tiles():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(99)
    ntiles = 300
    data = torch.randint(-(2 ** 31), 2 ** 31 - 1, (ntiles * 1024,), generator=g, dtype=torch.int64).to(torch.int32)
    n = 1000  # 62.5 waves: the last wave reads 8 tiles
    ids = torch.randint(-20, ntiles + 20, (n,), generator=g, dtype=torch.int32)
    sink = torch.full(((n + 15) // 16,), 7, dtype=torch.int32, device=dev)
    fe.fe_hbm_read_probe(data.to(dev).view(torch.uint8), ids.to(dev), sink)
    torch.cuda.synchronize()
    words = data.numpy().view(np.uint32).reshape(ntiles, 1024)
    tile_xor = np.bitwise_xor.reduce(words, axis=1)
    idn = ids.numpy()
    want = np.zeros((n + 15) // 16, np.uint32)
    for i, t in enumerate(idn):
        if 0 <= t < ntiles:
            want[i // 16] ^= tile_xor[t]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_mfma_rate_probe_sums():
    """The MFMA rate probe really multiplies its operands: each wave's sink is
    the sum of all its accumulators, which has a closed form independent of
    the output layout.  With lane l holding A[l % 32][8 (l // 32) + e] and
    B[8 (l // 32) + e][l % 32] (e < 8), sum_ij (A B)_ij = sum_k SA_k SB_k with
    SA_k, SB_k the sums of column / row k over the lanes; in every round
    accumulator j meets each of the 8 A operands once with B operand j, so a
    wave's total is R * sum_j sum_k (sum_m SA(A_m)_k) SB(B_j)_k."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(7)
    n_ops = 3000  # 16-byte entries (8 bf16 each); not a multiple of a wave's reach, so indices wrap
    ops = torch.rand(n_ops * 8, generator=g).to(torch.bfloat16)
    wgs, rounds = 3, 2
    sink = torch.full((wgs * 8,), float("nan"), dtype=torch.float32, device=dev)
    fe.fe_mfma_rate_probe(ops.to(dev), wgs, rounds, sink)
    torch.cuda.synchronize()
    vals = ops.float().numpy().astype(np.float64).reshape(n_ops, 8)
    want = np.zeros(wgs * 8)
    lanes = np.arange(64)
    for i in range(wgs * 8):
        def operand(k):  # [64 lanes][8 values] of operand slot k of wave i
            return vals[((i * 16 + k) * 64 + lanes) % n_ops]
        # column sums over the 32 lanes of each half: [2 halves][8 values] -> 16 k-indices
        sa = sum(operand(m).reshape(2, 32, 8).sum(axis=1) for m in range(8))
        total = 0.0
        for k in range(8):
            sb = operand(8 + k).reshape(2, 32, 8).sum(axis=1)
            total += float((sa * sb).sum())
        want[i] = rounds * total
    got = sink.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, want, rtol=1e-4, atol=0), (got[:4], want[:4])
