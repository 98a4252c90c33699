"""Pins of the fp64 oracle against things other than itself (CPU only).

The pages print no worked example or expected tensor, so the oracle is pinned
by a library routine (torch's scaled_dot_product_attention and logsumexp in
float64 on contiguous copies), closed forms, invariants and hand-derived
examples under tests/golden/.  ``test_planted_mistakes_are_caught`` compiles
deliberately broken copies of oracle.cpp and checks that these pins fail on
each of them.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_slot_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS, D = 16, 128


# ----------------------------------------------------------------------------
# helpers (input construction and library references only)

def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def paged_from_contiguous(ks, vs, NB, seed, fill=float("nan")):
    """Scatter per-sequence contiguous K/V ([L][Hkv][D] bf16) into pools at a
    random block placement; returns (k_cache, v_cache, block_tables)."""
    Hkv = ks[0].shape[1]
    nblk = [(k.shape[0] + BS - 1) // BS for k in ks]
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(NB, generator=g)
    assert sum(nblk) < NB
    mb = max(1, max(nblk))
    bt = torch.full((len(ks), mb), int(perm[-1]), dtype=torch.int32)
    kc = torch.full((NB, Hkv, BS, D), fill, dtype=torch.bfloat16)
    vc = torch.full((NB, Hkv, BS, D), fill, dtype=torch.bfloat16)
    off = 0
    for b, (k, v) in enumerate(zip(ks, vs)):
        for j in range(nblk[b]):
            blk = int(perm[off + j])
            bt[b, j] = blk
            rows = k[j * BS:(j + 1) * BS]
            kc[blk, :, : rows.shape[0]] = rows.transpose(0, 1)
            vc[blk, :, : rows.shape[0]] = v[j * BS:(j + 1) * BS].transpose(0, 1)
        off += nblk[b]
    return kc, vc, bt


def sdpa_ref(q, k, v, scale, G):
    """torch SDPA in float64 on one sequence: q [Hq][D], k/v [L][Hkv][D]."""
    qd = q.double()[None, :, None, :]
    kd = k.double().transpose(0, 1).repeat_interleave(G, dim=0)[None]
    vd = v.double().transpose(0, 1).repeat_interleave(G, dim=0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, scale=scale)[0, :, 0]
    s = scale * torch.matmul(kd[0], q.double()[:, :, None])[..., 0]  # [Hq][L]
    lse = torch.logsumexp(s, dim=-1)
    return out.numpy(), lse.numpy()


def appended(w, layer=0):
    lay = w.layers[layer]
    return oracle.append(lay.k_new, lay.v_new, w.slot_mapping, lay.k_cache, lay.v_cache)


# ----------------------------------------------------------------------------
# pins (plain functions so the planted-mistake test can run them too)

def pin_decode_vs_sdpa():
    for G, lens, seed in [(1, [1, 17], 11), (2, [40, 16, 15], 12), (4, [33, 3], 13), (8, [64], 14)]:
        Hkv = 2
        w = inputs.custom("decode", len(lens), Hkv * G, Hkv, lens, seed, append=1, keep_contiguous=True,
                          poison="nan")
        kc, vc = appended(w)
        out, lse = oracle.decode(w.layers[0].q, kc, vc, w.block_tables, w.context_lens, w.scale)
        offs = w.seq_offsets
        for b, L in enumerate(lens):
            ro, rl = sdpa_ref(w.layers[0].q[b], w.layers[0].k_seq[offs[b]:offs[b] + L],
                              w.layers[0].v_seq[offs[b]:offs[b] + L], w.scale, G)
            np.testing.assert_allclose(out[b], ro, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b], rl, rtol=1e-12, atol=1e-13)


def pin_c1_shape_vs_sdpa():
    w = inputs.make("qwen3_0.6b_b1_ctx128", keep_contiguous=True, poison="nan")
    kc, vc = appended(w)
    out, lse = oracle.decode(w.layers[0].q, kc, vc, w.block_tables, w.context_lens, w.scale)
    ro, rl = sdpa_ref(w.layers[0].q[0], w.layers[0].k_seq, w.layers[0].v_seq, w.scale, 2)
    np.testing.assert_allclose(out[0], ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12, atol=1e-13)


def pin_block_permutation_invariance():
    w = inputs.custom("decode", 3, 8, 2, [37, 80, 5], 21, poison="nan")
    lay = w.layers[0]
    out0, lse0 = oracle.decode(lay.q, lay.k_cache, lay.v_cache, w.block_tables, w.context_lens, w.scale)
    NB = w.num_blocks
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(5))
    kc2 = torch.empty_like(lay.k_cache)
    vc2 = torch.empty_like(lay.v_cache)
    kc2[perm] = lay.k_cache
    vc2[perm] = lay.v_cache
    bt2 = perm[w.block_tables.long()].to(torch.int32)
    out1, lse1 = oracle.decode(lay.q, kc2, vc2, bt2, w.context_lens, w.scale)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def pin_weights_sum_to_one():
    w = inputs.custom("decode", 2, 8, 2, [50, 29], 31, keep_contiguous=True, spike_frac=0.2)
    lay = w.layers[0]
    out, lse = oracle.decode(lay.q, lay.k_cache, lay.v_cache, w.block_tables, w.context_lens, w.scale)
    offs = w.seq_offsets
    for b in range(2):
        k = lay.k_seq[offs[b]:offs[b + 1]].double().transpose(0, 1).repeat_interleave(4, dim=0)
        s = w.scale * torch.matmul(k, lay.q[b].double()[:, :, None])[..., 0]
        tot = torch.exp(s - torch.from_numpy(lse[b])[:, None]).sum(-1)
        np.testing.assert_allclose(tot.numpy(), 1.0, atol=1e-12)


def _single_seq(k, v, q, scale, seed=3):
    kc, vc, bt = paged_from_contiguous([k], [v], 8, seed)
    return oracle.decode(q[None], kc, vc, bt, torch.tensor([k.shape[0]], dtype=torch.int32), scale)


def pin_identical_keys_give_mean():
    g = torch.Generator().manual_seed(41)
    L, Hkv, Hq = 37, 2, 4
    k1 = torch.randn(Hkv, D, generator=g).to(torch.bfloat16)
    k = k1[None].expand(L, Hkv, D).contiguous()
    v = torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16)
    q = torch.randn(Hq, D, generator=g).to(torch.bfloat16)
    scale = inputs.fp32_scale()
    out, lse = _single_seq(k, v, q, scale)
    for h in range(Hq):
        mean = v[:, h // 2].double().mean(0).numpy()
        np.testing.assert_allclose(out[0, h], mean, rtol=1e-12, atol=1e-14)
        s = scale * float((q[h].double() * k1[h // 2].double()).sum())
        assert abs(lse[0, h] - (s + math.log(L))) < 1e-12


def pin_zero_query_uniform():
    g = torch.Generator().manual_seed(42)
    L = 19
    k = torch.randn(L, 1, D, generator=g).to(torch.bfloat16)
    v = torch.randn(L, 1, D, generator=g).to(torch.bfloat16)
    q = torch.zeros(2, D, dtype=torch.bfloat16)
    out, lse = _single_seq(k, v, q, 0.25)
    np.testing.assert_allclose(out[0, 0], v[:, 0].double().mean(0).numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(L), rtol=0, atol=1e-13)


def pin_single_token():
    g = torch.Generator().manual_seed(43)
    k = torch.randn(1, 1, D, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, D, generator=g).to(torch.bfloat16)
    q = torch.randn(1, D, generator=g).to(torch.bfloat16)
    out, lse = _single_seq(k, v, q, 0.125)
    assert np.array_equal(out[0, 0], v[0, 0].double().numpy())
    s = 0.125 * float((q[0].double() * k[0, 0].double()).sum())
    assert abs(lse[0, 0] - s) < 1e-13


def pin_dominant_key():
    g = torch.Generator().manual_seed(44)
    L, j = 40, 23
    q = torch.randn(1, D, generator=g).to(torch.bfloat16)
    k = (0.01 * torch.randn(L, 1, D, generator=g)).to(torch.bfloat16)
    k[j, 0] = (8.0 * q[0].float()).to(torch.bfloat16)  # score margin >> 50
    v = torch.randn(L, 1, D, generator=g).to(torch.bfloat16)
    out, _ = _single_seq(k, v, q, 1.0)
    np.testing.assert_allclose(out[0, 0], v[j, 0].double().numpy(), rtol=0, atol=1e-12)


def pin_equal_queries_in_group():
    w = inputs.custom("decode", 2, 16, 4, [45, 12], 45)
    lay = w.layers[0]
    q = lay.q.clone()
    q[:, 4:8] = q[:, 4:5]  # group 1 (heads 4..7) shares one query
    out, lse = oracle.decode(q, lay.k_cache, lay.v_cache, w.block_tables, w.context_lens, w.scale)
    for h in range(5, 8):
        assert np.array_equal(out[:, h], out[:, 4]) and np.array_equal(lse[:, h], lse[:, 4])
    assert not np.array_equal(out[:, 8], out[:, 4])


def pin_empty_context():
    w = inputs.custom("decode", 2, 4, 2, [0, 7], 46)
    lay = w.layers[0]
    out, lse = oracle.decode(lay.q, lay.k_cache, lay.v_cache, w.block_tables, w.context_lens, w.scale)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


def pin_prefill_rows_equal_decode():
    w = inputs.custom("prefill", 2, 8, 2, [40, 21], 51, append=9, chunk=9, poison="nan")
    lay = w.layers[0]
    kc, vc = appended(w)
    out, lse = oracle.prefill_chunk(lay.q, w.query_start_loc, kc, vc, w.block_tables, w.context_lens, w.scale)
    qsl = w.query_start_loc.tolist()
    for b in range(2):
        C = qsl[b + 1] - qsl[b]
        for i in range(C):
            r = qsl[b] + i
            L = int(w.context_lens[b]) - C + i + 1
            lens = w.context_lens.clone()
            lens[b] = L
            qd = lay.q[r][None].expand(2, -1, -1).contiguous()
            o2, l2 = oracle.decode(qd, kc, vc, w.block_tables, lens, w.scale)
            assert np.array_equal(out[r], o2[b]) and np.array_equal(lse[r], l2[b])


def pin_prefill_vs_masked_sdpa():
    w = inputs.custom("prefill", 2, 8, 2, [30, 17], 52, append=12, chunk=12, keep_contiguous=True, poison="nan")
    lay = w.layers[0]
    kc, vc = appended(w)
    out, lse = oracle.prefill_chunk(lay.q, w.query_start_loc, kc, vc, w.block_tables, w.context_lens, w.scale)
    qsl, offs = w.query_start_loc.tolist(), w.seq_offsets
    for b in range(2):
        L = int(w.context_lens[b])
        C = qsl[b + 1] - qsl[b]
        q = lay.q[qsl[b]:qsl[b + 1]].double().transpose(0, 1)[None]  # [1][Hq][C][D]
        k = lay.k_seq[offs[b]:offs[b] + L].double().transpose(0, 1).repeat_interleave(4, dim=0)[None]
        v = lay.v_seq[offs[b]:offs[b] + L].double().transpose(0, 1).repeat_interleave(4, dim=0)[None]
        allowed = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
        mask = torch.zeros(C, L, dtype=torch.float64).masked_fill(~allowed, float("-inf"))
        ro = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale)[0]
        s = w.scale * torch.matmul(q[0], k[0].transpose(1, 2)) + mask
        rl = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(out[qsl[b]:qsl[b + 1]], ro.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[qsl[b]:qsl[b + 1]], rl.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)


def pin_split_merge_identity():
    w = inputs.custom("decode", 3, 8, 2, [100, 33, 64], 61, spike_frac=0.05)
    lay = w.layers[0]
    args = (lay.q, lay.k_cache, lay.v_cache, w.block_tables, w.context_lens, w.scale)
    out, lse = oracle.decode(*args)
    for S, P in [(16, 7), (32, 4), (48, 3), (128, 1), (16, 10)]:  # P = 10 leaves empty partitions
        op, lp = oracle.decode_split(*args, S=S, P=P)
        mo, ml = oracle.merge(op, lp)
        np.testing.assert_allclose(mo, out, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ml, lse, rtol=1e-12, atol=1e-14)


def pin_merge_all_empty():
    op = np.full((2, 3, D), 7.0)
    lp = np.full((2, 3), -np.inf)
    lp[1, 1] = 0.5
    mo, ml = oracle.merge(op, lp)
    assert np.all(mo[0] == 0) and np.isneginf(ml[0])
    assert np.all(mo[1] == 7.0) and ml[1] == 0.5


def pin_append_vs_numpy_scatter():
    w = inputs.custom("decode", 3, 8, 2, [20, 35, 16], 71, append=5, poison="nan")
    lay = w.layers[0]
    sm = w.slot_mapping.clone()
    sm[1] = -1  # padding entry
    kc, vc = oracle.append(lay.k_new, lay.v_new, sm, lay.k_cache, lay.v_cache)
    ek, ev = bits(lay.k_cache).copy(), bits(lay.v_cache).copy()
    s = sm.numpy().astype(np.int64)
    keep = s >= 0
    # [NB][Hkv][BS][D] -> [NB][BS][Hkv][D] view, fancy-index assignment by (block, offset)
    ek.transpose(0, 2, 1, 3)[s[keep] // BS, s[keep] % BS] = bits(lay.k_new)[keep]
    ev.transpose(0, 2, 1, 3)[s[keep] // BS, s[keep] % BS] = bits(lay.v_new)[keep]
    assert np.array_equal(kc.view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(vc.view(np.uint8), ev.view(np.uint8))


def pin_golden_examples():
    for name in sorted(os.listdir(GOLDEN)):
        if not name.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, name)) as f:
            ex = json.load(f)
        if ex["kind"] not in ("decode", "prefill"):
            continue
        Hq, Hkv = ex["Hq"], ex["Hkv"]
        ks, vs = [], []
        for seq in ex["sequences"]:
            L = seq["L"]
            k = torch.zeros(L, Hkv, D, dtype=torch.float32)
            v = torch.zeros(L, Hkv, D, dtype=torch.float32)
            for t, g, d, x in seq["k"]:
                k[t, g, d] = x
            for t, g, d, x in seq["v"]:
                v[t, g, d] = x
            ks.append(k.to(torch.bfloat16))
            vs.append(v.to(torch.bfloat16))
        kc, vc, bt = paged_from_contiguous(ks, vs, 8, ex.get("placement_seed", 1))
        lens = torch.tensor([s["L"] for s in ex["sequences"]], dtype=torch.int32)
        rows = ex["queries"]
        q = torch.zeros(len(rows), Hq, D, dtype=torch.float32)
        for r, row in enumerate(rows):
            for h, d, x in row:
                q[r, h, d] = x
        q = q.to(torch.bfloat16)
        if ex["kind"] == "decode":
            out, lse = oracle.decode(q, kc, vc, bt, lens, ex["scale"])
        else:
            qsl = torch.tensor(ex["query_start_loc"], dtype=torch.int32)
            out, lse = oracle.prefill_chunk(q, qsl, kc, vc, bt, lens, ex["scale"])
        for r, h, d, val in ex["expect_out"]:
            assert abs(out[r, h, d] - val) <= 1e-12 * max(1.0, abs(val)), (name, r, h, d, out[r, h, d], val)
        for r, h, val in ex["expect_lse"]:
            assert abs(lse[r, h] - val) <= 1e-12 * max(1.0, abs(val)), (name, r, h, lse[r, h], val)


# ----------------------------------------------------------------------------
# the per-head RMSNorm + rotary step (f2): closed forms and invariants

HALF = D // 2


def _table(cos_first, sin_second):
    """One table row: every pair gets the same (cos, sin)."""
    t = np.zeros((1, D), np.float32)
    t[0, :HALF] = cos_first
    t[0, HALF:] = sin_second
    return t


def _nr_inputs(T=5, H=3, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, D, generator=g).to(torch.bfloat16)
    w = (1 + 0.25 * torch.randn(D, generator=g)).to(torch.bfloat16)
    return x, w


def _vals(b):
    return from_bits(b).double().numpy()


def pin_norm_rope_identity_unit_rms():
    """cos 1, sin 0 and unit weights: each row's mean square is 1 (to bf16 rounding)."""
    x, _ = _nr_inputs()
    ones = torch.ones(D, dtype=torch.bfloat16)
    y = _vals(oracle.norm_rope(x, ones, _table(1.0, 0.0), np.zeros(x.shape[0], np.int32), 0.0))
    ms = (y ** 2).mean(-1)
    assert np.all(np.abs(ms - 1.0) <= 2.0 ** -7), ms


def pin_norm_rope_quarter_and_half_turn():
    """A quarter turn maps (a, b) to (-b, a) and a half turn to (-a, -b), exactly."""
    x, w = _nr_inputs(seed=1)
    pos = np.zeros(x.shape[0], np.int32)
    ident = _vals(oracle.norm_rope(x, w, _table(1.0, 0.0), pos, 1e-6))
    quarter = _vals(oracle.norm_rope(x, w, _table(0.0, 1.0), pos, 1e-6))
    half = _vals(oracle.norm_rope(x, w, _table(-1.0, 0.0), pos, 1e-6))
    assert np.array_equal(quarter[..., :HALF], -ident[..., HALF:])
    assert np.array_equal(quarter[..., HALF:], ident[..., :HALF])
    assert np.array_equal(half, -ident)


def pin_norm_rope_scale_invariance_and_weight_linearity():
    """RMSNorm ignores a positive scale of x (eps = 0); doubling w doubles the result."""
    x, w = _nr_inputs(seed=2)
    tab = _table(0.8, 0.6)
    pos = np.zeros(x.shape[0], np.int32)
    base = oracle.norm_rope(x, w, tab, pos, 0.0)
    x2 = (x.float() * 2).to(torch.bfloat16)  # exact
    assert np.array_equal(oracle.norm_rope(x2, w, tab, pos, 0.0), base)
    w2 = (w.float() * 2).to(torch.bfloat16)  # exact
    assert np.array_equal(_vals(oracle.norm_rope(x, w2, tab, pos, 0.0)), 2 * _vals(base))


def pin_norm_rope_heads_independent():
    x, w = _nr_inputs(seed=3)
    tab = _table(0.8, 0.6)
    pos = np.zeros(x.shape[0], np.int32)
    a = oracle.norm_rope(x, w, tab, pos, 1e-6)
    x2 = x.clone()
    x2[:, 1] = (x2[:, 1].float() * -3 + 1).to(torch.bfloat16)
    b = oracle.norm_rope(x2, w, tab, pos, 1e-6)
    assert np.array_equal(a[:, [0, 2]], b[:, [0, 2]])
    assert not np.array_equal(a[:, 1], b[:, 1])


def pin_norm_rope_positions_select_rows():
    """Token t uses table row positions[t], clamped into [0, max_pos)."""
    x, w = _nr_inputs(T=5, seed=4)
    rows = [_table(1.0, 0.0), _table(0.0, 1.0), _table(-1.0, 0.0)]
    tab = np.concatenate(rows)
    pos = np.array([0, 1, 2, 7, -3], np.int32)
    got = oracle.norm_rope(x, w, tab, pos, 1e-6)
    for t, r in enumerate([0, 1, 2, 2, 0]):
        want = oracle.norm_rope(x[t:t + 1], w, rows[r], np.zeros(1, np.int32), 1e-6)
        assert np.array_equal(got[t:t + 1], want), t


def pin_norm_rope_golden():
    ex = json.load(open(os.path.join(GOLDEN, "norm_rope_one_hot.json")))
    for case in ex["cases"]:
        x = torch.zeros(1, 1, D)
        x[0, 0, 0] = case["x0"]
        out = oracle.norm_rope(x.to(torch.bfloat16), torch.ones(D, dtype=torch.bfloat16),
                               _table(ex["cos"], ex["sin"]), np.zeros(1, np.int32), case["eps"])[0, 0]
        want = np.zeros(D, np.uint16)
        for d, b in case["expect"]:
            want[d] = b
        assert np.array_equal(out, want), (case, [hex(v) for v in out[[0, 64]]])


def pin_narrow_bf16_matches_torch():
    """On float32 values (where torch's float32 -> bfloat16 conversion rounds
    once) the oracle's narrowing gives the same bits, subnormals included."""
    g = torch.Generator().manual_seed(5)
    v = torch.cat([torch.randn(3000, generator=g) * 10.0 ** torch.randint(-6, 6, (3000,), generator=g),
                   torch.randn(200, generator=g) * 1e-39,
                   torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.389e38, 3.4e38, -3.4e38])])
    want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.narrow_bf16(float(a)) for a in v.tolist()], np.uint16)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]


# ----------------------------------------------------------------------------
# the sampler's softmax / log-sum-exp / greedy argmax (f4)

def _logits(B=4, V=3000, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (3.0 * torch.randn(B, V, generator=g)).to(torch.bfloat16)


def pin_sampler_vs_torch_softmax():
    """torch's float64 softmax and logsumexp, at several temperatures."""
    x = _logits()
    it = np.array([1.0, 0.5, 1.7, 3.0], np.float32)
    p, lse, _ = oracle.sampler(x, it)
    z = x.double() * torch.from_numpy(it).double()[:, None]
    assert np.allclose(p, torch.softmax(z, -1).numpy(), rtol=1e-12, atol=1e-300)
    assert np.allclose(lse, torch.logsumexp(z, -1).numpy(), rtol=0, atol=1e-12)


def pin_sampler_argmax_first_of_ties():
    x = _logits(B=3, V=500, seed=1).float()
    x[0, 7] = x[0, 300] = x[0, 499] = 40.0       # tie at the max: lowest index wins
    x[1, :] = 2.0                                # all equal
    x[2, 499] = 50.0                             # the last entry
    x = x.to(torch.bfloat16)
    _, _, am = oracle.sampler(x, with_probs=False)
    assert am.tolist() == [7, 0, 499]
    assert am[0] == int(np.argmax(x.float().numpy()[0]))  # numpy returns the first maximum too


def pin_sampler_masked_and_uniform():
    V = 1000
    x = torch.full((3, V), 1.5)
    x[1, ::2] = float("-inf")                    # half the tokens masked
    x[2, :] = float("-inf")                      # every token masked
    p, lse, am = oracle.sampler(x.to(torch.bfloat16), np.array([2.0, 1.0, 1.0], np.float32))
    assert np.allclose(p[0], 1.0 / V, rtol=1e-14) and abs(lse[0] - (3.0 + math.log(V))) < 1e-12
    assert np.all(p[1, ::2] == 0.0) and np.allclose(p[1, 1::2], 2.0 / V, rtol=1e-14)
    assert abs(lse[1] - (1.5 + math.log(V / 2))) < 1e-12
    assert np.all(p[2] == 0.0) and lse[2] == -math.inf and am[2] == 0


def pin_sampler_temperature_scale_identity():
    """Doubling the logits (exact in bf16) at half the inverse temperature changes nothing."""
    x = _logits(B=2, V=777, seed=2)
    x2 = (x.float() * 2).to(torch.bfloat16)
    a = oracle.sampler(x, np.array([1.0, 0.8], np.float32))
    b = oracle.sampler(x2, np.array([0.5, 0.4], np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


PINS = [pin_decode_vs_sdpa, pin_c1_shape_vs_sdpa, pin_block_permutation_invariance, pin_weights_sum_to_one,
        pin_identical_keys_give_mean, pin_zero_query_uniform, pin_single_token, pin_dominant_key,
        pin_equal_queries_in_group, pin_empty_context, pin_prefill_rows_equal_decode, pin_prefill_vs_masked_sdpa,
        pin_split_merge_identity, pin_merge_all_empty, pin_append_vs_numpy_scatter, pin_golden_examples,
        pin_norm_rope_identity_unit_rms, pin_norm_rope_quarter_and_half_turn,
        pin_norm_rope_scale_invariance_and_weight_linearity, pin_norm_rope_heads_independent,
        pin_norm_rope_positions_select_rows, pin_norm_rope_golden, pin_narrow_bf16_matches_torch,
        pin_sampler_vs_torch_softmax, pin_sampler_argmax_first_of_ties, pin_sampler_masked_and_uniform,
        pin_sampler_temperature_scale_identity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail

MUTANTS = {
    "head_map_modulo": [("h / G", "h % Hkv")],
    "block_layout_transposed": [("((static_cast<size_t>(blk) * Hkv + g) * BS + off)",
                                 "((static_cast<size_t>(blk) * BS + off) * Hkv + g)")],
    "token_offset_shifted": [("const int off = t % BS;", "const int off = (t + 1) % BS;")],
    "scale_dropped": [("s[t - t0] = scale * dot;", "s[t - t0] = dot;")],
    "lse_missing_max": [("*lse = m + std::log(Z);", "*lse = std::log(Z);")],
    "value_reads_key_pool": [("const uint16_t* v = c.v + c.offset(t, g);", "const uint16_t* v = c.k + c.offset(t, g);")],
    "last_token_dropped": [("attend(out + row * D, lse + row, q + row * D, c, h / G, 0, context_lens[b], scale);",
                            "attend(out + row * D, lse + row, q + row * D, c, h / G, 0, context_lens[b] - 1, scale);")],
    "causal_off_by_one": [("h / G, 0, pos + 1, scale)", "h / G, 0, pos, scale)")],
    "merge_weight_unnormalised": [("const double w = std::exp(lp[p] - lse[r]);", "const double w = std::exp(lp[p] - M);")],
    "append_offset_reversed": [("* BS + off) * static_cast<size_t>(D);\n      const size_t src",
                                "* BS + (BS - 1 - off)) * static_cast<size_t>(D);\n      const size_t src")],
    "dot_skips_last_dim": [("for (int d = 0; d < D; ++d) dot +=", "for (int d = 0; d < D - 1; ++d) dot +=")],
    "rope_sin_sign_flipped": [("y[d] * c - y[half + d] * s", "y[d] * c + y[half + d] * s"),
                              ("y[half + d] * c + y[d] * s", "y[half + d] * c - y[d] * s")],
    "rope_cos_sin_swapped": [("const double c = cs[d], s = cs[half + d];", "const double c = cs[half + d], s = cs[d];")],
    "rope_partner_adjacent": [("y[d] * c - y[half + d] * s", "y[d] * c - y[d ^ 1] * s"),
                              ("y[half + d] * c + y[d] * s", "y[d ^ 1] * c + y[d] * s")],
    "rope_position_ignored": [("int p = positions[t];", "int p = 0;")],
    "rms_mean_over_half": [("std::sqrt(ss / D + eps)", "std::sqrt(ss / half + eps)")],
    "rms_eps_outside_sqrt": [("1.0 / std::sqrt(ss / D + eps)", "1.0 / std::sqrt(ss / D) + eps")],
    "norm_weight_dropped": [("* inv_rms * widen_bf16(w[d])", "* inv_rms")],
    "bf16_rounding_truncates": [("std::nearbyint(std::ldexp(a, shift))", "std::trunc(std::ldexp(a, shift))")],
    "argmax_takes_last_tie": [("      if (v > bestv) {", "      if (v >= bestv) {")],
    "temperature_ignored": [("const double s = inv_temp ? static_cast<double>(inv_temp[b]) : 1.0;", "const double s = 1.0;")],
    "sampler_lse_missing_max": [("lse[b] = m + std::log(Z);", "lse[b] = std::log(Z);")],
    "sampler_probs_unnormalised": [("std::exp(s * widen_bf16(x[i]) - m) / Z;", "std::exp(s * widen_bf16(x[i]) - m);")],
    "softmax_sum_skips_first_token": [("  double Z = 0.0;\n  for (int t = t0; t < t1; ++t) {\n    s[t - t0] = std::exp",
                                       "  double Z = 0.0;\n  for (int t = t0; t < t1; ++t) {\n    if (t == t0) { s[0] = std::exp(s[0] - m); continue; }\n    s[t - t0] = std::exp")],
    "value_row_one_token_late": [("const uint16_t* v = c.v + c.offset(t, g);",
                                  "const uint16_t* v = c.v + c.offset(t + 1 < t1 ? t + 1 : t, g);")],
    "prefill_top_left_alignment": [("const int pos = context_lens[b] - C + (r - query_start_loc[b]);",
                                    "const int pos = r - query_start_loc[b];")],
    "append_skips_v": [("        v_cache[dst + d] = v_new[src + d];\n", "")],
    "decode_reads_head0_query": [("attend(out + row * D, lse + row, q + row * D, c, h / G, 0, context_lens[b], scale);",
                                  "attend(out + row * D, lse + row, q + (row - h) * D, c, h / G, 0, context_lens[b], scale);")],
    "sampler_lse_base2": [("lse[b] = m + std::log(Z);", "lse[b] = m + std::log2(Z);")],
}


def _build_mutant(tmp_path, name, edits):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")).read()
    for old, new in edits:
        assert old in src, (name, old)
        src = src.replace(old, new)
    cpp = tmp_path / f"{name}.cpp"
    cpp.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-pthread", str(cpp), "-o", str(so)], check=True)
    return str(so)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(tmp_path, name):
    so = _build_mutant(tmp_path, name, MUTANTS[name])
    caught = []
    try:
        oracle.use_library(so)
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle.use_library(None)
    assert caught, f"no pin catches the planted mistake {name}"
