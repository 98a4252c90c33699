"""Serving steps driven by the paged KV block allocator, on the GPU.

Requests enter (prompt appended through the allocator's slots), grow one
token per step, and leave -- finished, or cancelled midway -- releasing their
blocks, which later requests reuse.  Every step's K/V rows go through
fe_paged_kv_append at the allocator's slots, and decode (and, for prompts,
the chunked prefill) runs over the allocator's block tables; each result
matches the fp64 oracle run on a host copy of the same pools, and no KV
block is left allocated at the end.  The decode steps run either as append +
decode or as the fused fe_paged_gqa_decode_append call.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from gpu_util import assert_attention, u16

pytestmark = pytest.mark.gpu

BS, D = 16, 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("fused", [False, True])
def test_allocator_driven_serving(dev, fused):
    NB, Hq, Hkv, max_seqs, mbps = 160, 32, 8, 4, 48
    g = torch.Generator().manual_seed(900)
    alloc = fe.KVAllocator(NB, BS, max_seqs, mbps)
    kc = torch.full((NB, Hkv, BS, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    kc_h, vc_h = u16(kc), u16(vc)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    reqs = [dict(prompt=int(torch.randint(5, 300, (1,), generator=g)), gen=int(torch.randint(3, 12, (1,), generator=g)),
                 cancel=i in (1, 4)) for i in range(7)]
    waiting, running = list(range(len(reqs))), {}
    free_seqs = list(range(max_seqs))
    checked = 0

    def rows(n):
        k = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
        v = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
        return k, v

    def append(seq, n):
        nonlocal kc_h, vc_h
        slots = torch.from_numpy(alloc.append(seq, n))
        k, v = rows(n)
        fe.fe_paged_kv_append(k.to(dev), v.to(dev), slots.to(dev), kc, vc)
        kc_h, vc_h = oracle.append(k, v, slots, kc_h, vc_h)
        return k, v

    step = 0
    while waiting or running:
        # admit: the prompt is appended, then attended by a causal chunk
        while waiting and len(running) < max_seqs:
            r = waiting.pop(0)
            seq = free_seqs.pop(0)
            running[r] = dict(seq=seq, done=0)
            append(seq, reqs[r]["prompt"])
            bt, cl = alloc.batch([seq])
            C = reqs[r]["prompt"]
            q = torch.randn(C, Hq, D, generator=g).to(torch.bfloat16)
            qsl = torch.tensor([0, C], dtype=torch.int32)
            out = torch.empty(C, Hq, D, dtype=torch.bfloat16, device=dev)
            lse = torch.empty(C, Hq, dtype=torch.float32, device=dev)
            fe.fe_paged_gqa_prefill_chunk(out, lse, q.to(dev), qsl.to(dev), kc, vc, torch.from_numpy(bt).to(dev),
                                          torch.from_numpy(cl).to(dev), C, int(cl.max()), scale)
            torch.cuda.synchronize()
            ro, rl = oracle.prefill_chunk(q, qsl, kc_h, vc_h, bt, cl, scale)
            assert_attention(out, lse, ro, rl, f"step {step} prompt of request {r}")
            checked += 1
        # retire finished and cancelled requests
        for r in list(running):
            st = running[r]
            if (reqs[r]["cancel"] and st["done"] >= 2) or st["done"] >= reqs[r]["gen"]:
                alloc.release(st["seq"])
                free_seqs.append(st["seq"])
                del running[r]
        if not running:
            continue
        # one decode step for every running request
        seqs = [running[r]["seq"] for r in running]
        if fused:
            # one new row per sequence at the allocator's slot, appended by the decode call itself
            slots = torch.from_numpy(np.concatenate([alloc.append(s, 1) for s in seqs]))
            kn, vn = rows(len(seqs))
            kc_h, vc_h = oracle.append(kn, vn, slots, kc_h, vc_h)
        else:
            for s in seqs:
                append(s, 1)
        bt, cl = alloc.batch(seqs)
        q = torch.randn(len(seqs), Hq, D, generator=g).to(torch.bfloat16)
        out = torch.empty(len(seqs), Hq, D, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(len(seqs), Hq, dtype=torch.float32, device=dev)
        if fused:
            fe.fe_paged_gqa_decode_append(out, lse, q.to(dev), kn.to(dev), vn.to(dev), slots.to(dev), kc, vc,
                                          torch.from_numpy(bt).to(dev), torch.from_numpy(cl).to(dev), int(cl.max()),
                                          scale)
        else:
            fe.fe_paged_gqa_decode(out, lse, q.to(dev), kc, vc, torch.from_numpy(bt).to(dev),
                                   torch.from_numpy(cl).to(dev), int(cl.max()), scale)
        torch.cuda.synchronize()
        ro, rl = oracle.decode(q, kc_h, vc_h, bt, cl, scale)
        assert_attention(out, lse, ro, rl, f"step {step} decode of {len(seqs)}")
        checked += 1
        for r in running:
            running[r]["done"] += 1
        step += 1
    torch.cuda.synchronize()
    assert np.array_equal(u16(kc), kc_h) and np.array_equal(u16(vc), vc_h)
    assert alloc.num_allocated == 0 and alloc.num_free == NB
    assert checked > 10
