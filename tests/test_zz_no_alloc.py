"""The allocation-free decode call (fe_paged_gqa_decode_noalloc) against
fe_paged_gqa_decode with a caller workspace: two calls in a row through the
C ABI, the second on a smaller input, must give bit-identical outputs (the
same kernels and partitioning; the scratch keeps the first call's partials,
which must not leak into the second), and both meet the oracle's gates.
A replayed HIP graph of the call (the use it exists for: no allocation
under capture) matches the eager call on every replay."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs
from gpu_util import DeviceWorkload, assert_attention, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def both(dw, P):
    w = dw.w
    res = []
    for noalloc in (False, True):
        out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=dw.dev)
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=dw.dev)
        if noalloc:
            fe.fe_paged_gqa_decode_noalloc(out, lse, dw.q, dw.kc, dw.vc, dw.bt, dw.lens, w.max_context_len, w.scale,
                                           num_partitions=P)
        else:
            fe.fe_paged_gqa_decode(out, lse, dw.q, dw.kc, dw.vc, dw.bt, dw.lens, w.max_context_len, w.scale,
                                   num_partitions=P)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def check(w, dev, parts, label):
    dw = DeviceWorkload(w, dev)
    rk, rv = dw.append()
    ro, rl = oracle.decode(dw.lay.q, rk, rv, w.block_tables, w.context_lens, w.scale)
    for P in parts:
        (o1, l1), (o2, l2) = both(dw, P)
        print(f"[{label} P={P}] partitions used: "
              f"{fe.fe_paged_gqa_decode_num_partitions(w.B, w.Hq, w.Hkv, 128, w.max_context_len, P)}", flush=True)
        assert np.array_equal(u16(o1), u16(o2)), (label, P, "out differs from fe_paged_gqa_decode")
        assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32)), (label, P, "lse")
        assert_attention(o2, l2, ro, rl, f"{label} noalloc P={P}")


def test_noalloc_two_calls_second_smaller(dev):
    print("noalloc: serving workload, 64 sequences, contexts 1024..8192", flush=True)
    check(inputs.make("qwen3_4b_b64_ctx1024-8192", seed=1, poison="nan"), dev, (0, 16), "b64")
    print("noalloc: 5 sequences, ragged contexts", flush=True)
    lens = [700, 33, 0, 1500, 16]
    check(inputs.custom("decode", len(lens), 32, 8, lens, 41, append=1, poison="nan"), dev, (0, 3, 1), "small")


def test_noalloc_too_large_is_refused(dev):
    B = 1024
    q = torch.zeros(B, 32, 128, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(4, 8, 16, 128, dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 7.0)
    bt = torch.zeros(B, 512, dtype=torch.int32, device=dev)
    lens = torch.zeros(B, dtype=torch.int32, device=dev)
    with pytest.raises(fe.binding.FeError, match="FE_ERR_WORKSPACE"):
        fe.fe_paged_gqa_decode_noalloc(out, None, q, kc, kc, bt, lens, 8192, 0.088, num_partitions=8)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must leave its output untouched"


def test_noalloc_graph_replay(dev):
    lens = [3000, 17, 900, 4096, 1]
    w = inputs.custom("decode", len(lens), 32, 8, lens, 42, append=1, poison="nan")
    dw = DeviceWorkload(w, dev)
    dw.append()
    (o_ref, l_ref), _ = both(dw, 0)
    out = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fe.fe_paged_gqa_decode_noalloc(out, lse, dw.q, dw.kc, dw.vc, dw.bt, dw.lens, w.max_context_len, w.scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fe.fe_paged_gqa_decode_noalloc(out, lse, dw.q, dw.kc, dw.vc, dw.bt, dw.lens, w.max_context_len, w.scale)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        # other work on the same GPU between replays (an eager call with a
        # different input size also uses the scratch)
        both(dw, 3)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(u16(out), u16(o_ref)), ("replay", i)
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), l_ref.cpu().numpy().view(np.uint32)), ("replay", i)
