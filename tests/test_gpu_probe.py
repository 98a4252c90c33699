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
