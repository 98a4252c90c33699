"""GPU parity of KV append and paged GQA decode against the fp64 oracle.

Every case goes through the C ABI (via the ctypes binding) on cuda:0.  Append
is compared byte for byte over the whole pool; attention to max-abs 1e-2,
row-relative 1e-2 and LSE 1e-3.
"""
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


def run_decode(w, dev, parts=(0,), label="", layer=0):
    dw = DeviceWorkload(w, dev, layer)
    if w.slot_mapping.numel():
        rk, rv = dw.append()
    else:
        rk, rv = dw.lay.k_cache, dw.lay.v_cache
    ro, rl = oracle.decode(dw.lay.q, rk, rv, w.block_tables, w.context_lens, w.scale)
    for P in parts:
        out, lse = dw.decode(num_partitions=P)
        assert_attention(out, lse, ro, rl, f"{label} P={P}")


# -- append -------------------------------------------------------------------

def test_append_padding_and_out_of_range_slots(dev):
    w = inputs.custom("decode", 3, 8, 2, [20, 35, 16], 7, append=5, poison="nan")
    sm = w.slot_mapping.clone()
    sm[1] = -1
    sm[3] = -7
    w.slot_mapping = sm
    dw = DeviceWorkload(w, dev)
    dw.slots[4] = w.num_blocks * 16 + 3  # beyond the pool: must be skipped on the GPU
    fe.fe_paged_kv_append(dw.k_new, dw.v_new, dw.slots, dw.kc, dw.vc)
    sm_ref = sm.clone()
    sm_ref[4] = -1
    rk, rv = oracle.append(w.layers[0].k_new, w.layers[0].v_new, sm_ref, w.layers[0].k_cache, w.layers[0].v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(u16(dw.kc), rk) and np.array_equal(u16(dw.vc), rv)


def test_append_large_batch_bit_exact(dev):
    w = inputs.make("qwen3_4b_b4_prefix4096_chunk256")  # 1024 new tokens
    DeviceWorkload(w, dev).append()


def test_append_zero_tokens_is_noop(dev):
    kc = torch.zeros(4, 8, 16, 128, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    empty = torch.zeros(0, 8, 128, dtype=torch.bfloat16, device=dev)
    fe.fe_paged_kv_append(empty, empty, torch.zeros(0, dtype=torch.int32, device=dev), kc, vc)
    torch.cuda.synchronize()
    assert not kc.any() and not vc.any()


# -- decode: small cases spanning tiles, ragged tails and edge cases ------------

@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("poison", ["nan", "large"])
def test_decode_small(dev, G, poison):
    lens = [1, 15, 16, 17, 100, 257, 0, 33]
    w = inputs.custom("decode", len(lens), 2 * G, 2, lens, 100 + G, append=1, poison=poison)
    run_decode(w, dev, parts=(1, 2, 3, 0), label=f"small G={G} {poison}")


def test_decode_spiky_keys(dev):
    lens = [700, 1500, 64, 999]
    w = inputs.custom("decode", 4, 32, 8, lens, 5, append=1, spike_frac=0.05)
    run_decode(w, dev, parts=(1, 4, 0), label="spiky")


def test_decode_all_empty(dev):
    w = inputs.custom("decode", 2, 8, 2, [0, 0], 9)
    run_decode(w, dev, parts=(1, 4, 0), label="empty")


def test_decode_context_cap(dev):
    """max_context_len smaller than a sequence's length clamps it (documented)."""
    w = inputs.custom("decode", 2, 8, 2, [40, 20], 10)
    dw = DeviceWorkload(w, dev)
    out, lse = dw.decode(num_partitions=1, max_context_len=32)
    lens = torch.tensor([32, 20], dtype=torch.int32)
    ro, rl = oracle.decode(dw.lay.q, dw.lay.k_cache, dw.lay.v_cache, w.block_tables, lens, w.scale)
    assert_attention(out, lse, ro, rl, "cap")


def test_decode_golden(dev):
    """Hand-derived examples (tests/golden) through the HIP path."""
    import json
    import os
    gdir = os.path.join(os.path.dirname(__file__), "golden")
    for name in sorted(os.listdir(gdir)):
        if not name.startswith("decode_"):
            continue
        ex = json.load(open(os.path.join(gdir, name)))
        from test_oracle import paged_from_contiguous
        ks, vs = [], []
        for seq in ex["sequences"]:
            k = torch.zeros(seq["L"], ex["Hkv"], 128)
            v = torch.zeros(seq["L"], ex["Hkv"], 128)
            for t, g, d, x in seq["k"]:
                k[t, g, d] = x
            for t, g, d, x in seq["v"]:
                v[t, g, d] = x
            ks.append(k.to(torch.bfloat16))
            vs.append(v.to(torch.bfloat16))
        kc, vc, bt = paged_from_contiguous(ks, vs, 8, ex.get("placement_seed", 1))
        q = torch.zeros(len(ex["queries"]), ex["Hq"], 128)
        for r, row in enumerate(ex["queries"]):
            for h, d, x in row:
                q[r, h, d] = x
        lens = torch.tensor([s["L"] for s in ex["sequences"]], dtype=torch.int32)
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        fe.fe_paged_gqa_decode(out, lse, q.to(torch.bfloat16).to(dev), kc.to(dev), vc.to(dev), bt.to(dev),
                               lens.to(dev), int(lens.max()), ex["scale"])
        torch.cuda.synchronize()
        for r, h, d, val in ex["expect_out"]:
            assert abs(float(out[r, h, d]) - val) <= 1e-2, (name, r, h, d)
        for r, h, val in ex["expect_lse"]:
            assert abs(float(lse[r, h]) - val) <= 1e-3, (name, r, h)


# -- decode: the five workloads at full size ---------------------------------------

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_qwen3_0_6b_b1_ctx128(dev, seed):
    w = inputs.make("qwen3_0.6b_b1_ctx128", seed=seed, poison="nan")
    run_decode(w, dev, parts=(0, 1, 2, 8), label=f"0.6b b1 seed {seed}")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_qwen3_4b_b4_36layers(dev, seed):
    w = inputs.make("qwen3_4b_b4_ctx256-2048_36layers", seed=seed, poison="nan")
    for layer in range(len(w.layers)):
        run_decode(w, dev, parts=(0,), label=f"4b b4 seed {seed} layer {layer}", layer=layer)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_qwen3_4b_b64(dev, seed):
    w = inputs.make("qwen3_4b_b64_ctx1024-8192", seed=seed, poison="nan")
    run_decode(w, dev, parts=(0, 1, 16), label=f"4b b64 seed {seed}")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_qwen3_4b_b8_ctx32768(dev, seed):
    w = inputs.make("qwen3_4b_b8_ctx32768", seed=seed, poison="nan")
    run_decode(w, dev, parts=(8, 16, 32, 0), label=f"4b b8 32k seed {seed}")


def test_decode_workspace_reuse(dev):
    """One workspace, never cleared, serves many calls with various partition
    counts; every result matches."""
    lens = [700, 1500, 64, 999, 3000, 17]
    w = inputs.custom("decode", 6, 32, 8, lens, 77, append=1)
    dw = DeviceWorkload(w, dev)
    rk, rv = dw.append()
    ro, rl = oracle.decode(dw.lay.q, rk, rv, w.block_tables, w.context_lens, w.scale)
    parts = (0, 4, 8, 2, 16, 4, 0)
    size = max(fe.fe_paged_gqa_decode_workspace_size(6, 32, 8, 128, w.max_context_len, P) for P in parts)
    ws = torch.full((size,), 0xA5, dtype=torch.uint8, device=dev)  # garbage must not matter
    for P in parts:
        out = torch.full((6, 32, 128), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((6, 32), float("nan"), dtype=torch.float32, device=dev)
        fe.fe_paged_gqa_decode(out, lse, dw.q, dw.kc, dw.vc, dw.bt, dw.lens, w.max_context_len, w.scale,
                               num_partitions=P, workspace=ws)
        torch.cuda.synchronize()
        assert_attention(out, lse, ro, rl, f"reuse P={P}")


def test_decode_negative_scale(dev):
    """A negative softmax scale is folded into q's sign bits; results follow the definition."""
    w = inputs.custom("decode", 3, 16, 4, [300, 47, 1000], 78, append=1)
    w.scale = -w.scale
    run_decode(w, dev, parts=(1, 4, 0), label="negative scale")


# -- append fused into decode (fe_paged_gqa_decode_append) ------------------------

def per_sequence_rows(w, layer=0):
    """The workload's new rows as the fused call takes them: one per sequence
    ([B][Hkv][D], slot -1 and zero rows where a sequence is empty)."""
    lay = w.layers[layer]
    lens = w.context_lens.tolist()
    kn = torch.zeros(w.B, w.Hkv, 128, dtype=torch.bfloat16)
    vn = torch.zeros_like(kn)
    slots = torch.full((w.B,), -1, dtype=torch.int32)
    i = 0
    for b, L in enumerate(lens):
        if L > 0:
            kn[b], vn[b], slots[b] = lay.k_new[i], lay.v_new[i], w.slot_mapping[i]
            i += 1
    assert i == w.slot_mapping.numel()
    return kn, vn, slots


def run_decode_append(w, dev, parts=(0,), label="", layer=0, slots_override=None, pre=None):
    """Fused append + decode against the oracle's append followed by its
    decode: the pools bit for bit after every call, attention to the gate.
    `pre` (host pools) replaces the workload's pools as the starting state."""
    lay = w.layers[layer]
    kn, vn, slots = per_sequence_rows(w, layer)
    if slots_override is not None:
        slots = slots_override
    k0, v0 = (lay.k_cache, lay.v_cache) if pre is None else pre
    # the oracle skips negative slots; slots past the pool are skipped too
    ref_slots = slots.clone()
    ref_slots[ref_slots >= w.num_blocks * 16] = -1
    rk, rv = oracle.append(kn, vn, ref_slots, k0, v0)  # uint16 images of the pools
    ro, rl = oracle.decode(lay.q, rk, rv, w.block_tables, w.context_lens, w.scale)
    q, bt, lens = lay.q.to(dev), w.block_tables.to(dev), w.context_lens.to(dev)
    kn_d, vn_d, sl_d = kn.to(dev), vn.to(dev), slots.to(dev)
    for P in parts:
        kc, vc = k0.to(dev), v0.to(dev)
        out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=dev)
        fe.fe_paged_gqa_decode_append(out, lse, q, kn_d, vn_d, sl_d, kc, vc, bt, lens, w.max_context_len, w.scale,
                                      num_partitions=P)
        torch.cuda.synchronize()
        assert np.array_equal(u16(kc), rk), (label, P, "K pool differs after the fused append")
        assert np.array_equal(u16(vc), rv), (label, P, "V pool differs after the fused append")
        assert_attention(out, lse, ro, rl, f"{label} fused P={P}")


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_append_small(dev, G):
    # full last blocks (16, 32, 256) and partial ones, a single token, an empty sequence
    lens = [1, 15, 16, 17, 100, 256, 0, 33, 32]
    w = inputs.custom("decode", len(lens), 2 * G, 2, lens, 300 + G, append=1, poison="nan")
    run_decode_append(w, dev, parts=(1, 2, 3, 0), label=f"fused small G={G}")


def test_decode_append_padding_and_out_of_range_slots(dev):
    """A padding slot (-1) and a slot past the pool write nothing; those
    sequences read their last position from the cache as it is (here: their
    rows, already written by an earlier step)."""
    lens = [40, 16, 77, 5]
    w = inputs.custom("decode", 4, 8, 2, lens, 311, append=1, poison="nan")
    kn, vn, slots = per_sequence_rows(w)
    earlier = torch.full_like(slots, -1)
    earlier[1], earlier[2] = slots[1], slots[2]
    k0, v0 = oracle.append(kn, vn, earlier, w.layers[0].k_cache, w.layers[0].v_cache)
    pre = tuple(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) for x in (k0, v0))
    slots[1] = -1
    slots[2] = w.num_blocks * 16 + 5
    run_decode_append(w, dev, parts=(1, 0), label="fused padding", slots_override=slots, pre=pre)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_append_qwen3_4b_b64(dev, seed):
    """The serving-concurrency workload, its append fused into the decode call."""
    w = inputs.make("qwen3_4b_b64_ctx1024-8192", seed=seed, poison="nan")
    run_decode_append(w, dev, parts=(0, 1, 16), label=f"fused 4b b64 seed {seed}")


def test_decode_append_qwen3_4b_b4_small_batch(dev):
    """Four sequences of the Qwen3-4B layer shape with contexts as in the
    36-layer workload (256..2048 tokens), each with a new token."""
    g = torch.Generator().manual_seed(321)
    lens = torch.randint(256, 2049, (4,), generator=g).tolist()
    w = inputs.custom("decode", 4, 32, 8, lens, 321, append=1, poison="nan")
    run_decode_append(w, dev, parts=(0, 1, 8), label="fused 4b b4")


def test_decode_append_qwen3_0_6b_b1_ctx128(dev):
    w = inputs.make("qwen3_0.6b_b1_ctx128", poison="nan")
    run_decode_append(w, dev, parts=(0, 1, 8), label="fused 0.6b b1")


def test_decode_append_random_shapes(dev):
    """Seeded random shapes for the fused call: group size, KV heads, batch,
    ragged lengths (zeros and whole blocks included) and partition counts."""
    g = torch.Generator().manual_seed(2024)
    for case in range(12):
        G = int(torch.randint(1, 9, (1,), generator=g))
        Hkv = [1, 2, 8][int(torch.randint(0, 3, (1,), generator=g))]
        B = int(torch.randint(1, 10, (1,), generator=g))
        lens = torch.randint(0, 700, (B,), generator=g)
        lens[torch.rand(B, generator=g) < 0.2] = 0
        whole = torch.rand(B, generator=g) < 0.3
        lens[whole] = (lens[whole] // 16 + 1) * 16
        lens = lens.tolist()
        if max(lens) == 0:
            lens[0] = 1
        parts = (0, 1, int(torch.randint(2, 10, (1,), generator=g)))
        w = inputs.custom("decode", B, G * Hkv, Hkv, lens, 700 + case, append=1, poison="nan")
        run_decode_append(w, dev, parts=parts, label=f"fused random #{case} G={G} Hkv={Hkv} lens={lens}")


# -- decode: sizes at the edges of the plan ----------------------------------------

def test_decode_one_very_long_sequence(dev):
    """One sequence of 131072 tokens (8192 blocks): the automatic plan (64
    partitions of 128 blocks), 40 partitions, and a request for 16 that the
    256-block limit of a partition raises to 32; the merge walks the partials
    in chunks of 16."""
    w = inputs.custom("decode", 1, 32, 8, [131072], 901, append=1, poison="nan")
    assert fe.fe_paged_gqa_decode_num_partitions(1, 32, 8, 128, w.max_context_len, 16) == 32
    run_decode(w, dev, parts=(0, 40, 16), label="1 x 131072")


def test_decode_many_partitions(dev):
    """Partition counts far above the automatic choice, down to one block per
    partition (the merge then combines up to 129 partials per row)."""
    lens = [2049, 17, 1000, 0, 512]
    w = inputs.custom("decode", len(lens), 16, 4, lens, 902, append=1, poison="nan")
    run_decode(w, dev, parts=(50, 100, 129, 1000), label="many partitions")


def test_decode_many_sequences(dev):
    """1024 sequences of short ragged contexts (0..300 tokens): a grid of
    tens of thousands of workgroups, single pass and split."""
    g = torch.Generator().manual_seed(903)
    lens = torch.randint(0, 301, (1024,), generator=g).tolist()
    w = inputs.custom("decode", 1024, 16, 8, lens, 903, append=1, poison="large")
    run_decode(w, dev, parts=(1, 0, 3), label="1024 sequences")
