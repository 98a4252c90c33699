"""GPU checks of the one-launch attention step of a decode token
(fe_paged_gqa_decode_norm_rope_append): per-head QK-RMSNorm + rotary
embedding of q and of the new k rows, the append, and decode.

(1) Bit for bit against the same step built from the other calls.
fe_qk_norm_rope_append writes q_out and the normalised, rotated k rows into
a copy of the pools; those k rows, read back from their slots, and q_out go
into fe_paged_gqa_decode_append on a fresh copy.  The fused call must give
the same out, lse and pools, bit for bit: it runs the same arithmetic with
the same bf16 roundings.
(2) Against the fp64 oracle (its norm/rotary step, then its decode), with
the V pool bit for bit.  The q rows and the appended k rows are held to the
norm/rotary gate (each within one bf16 step of the oracle's, few differing).
The output and LSE are held to the attention gate (max-abs 1e-2,
row-relative 1e-2, LSE 1e-3), widened row by row by the exact effect of
those rows' differences: a q element that rounds to the other neighbouring
bf16 value shifts every score of its row, and where the softmax is peaked
one such flip alone moves the LSE by several 1e-4 (on the 64-sequence step
below, 8 of 262144 q elements differ and one of them moves a row's LSE by
5.6e-4; an fp32 emulation of the rows on the CPU gives the same figure).
Rows whose q and keys equal the oracle's get no allowance.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs
from gpu_util import assert_attention, assert_rope_close, norm_only_rows, rope_term, rounding_allowance, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def per_sequence(w, c):
    """The norm/rotary case with one row per sequence, as the fused call
    takes it: an empty sequence gets zero rows, slot -1 and position 0."""
    B = w.B
    q = torch.zeros((B, w.Hq, 128), dtype=torch.bfloat16)
    k = torch.zeros((B, w.Hkv, 128), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    pos = torch.zeros(B, dtype=torch.int32)
    sm = torch.full((B,), -1, dtype=torch.int32)
    i = 0
    for b, L in enumerate(w.context_lens.tolist()):
        if L > 0:
            q[b], k[b], v[b], pos[b], sm[b] = c.q[i], c.k[i], c.v[i], c.positions[i], c.slot_mapping[i]
            i += 1
    assert i == c.q.shape[0]
    c.q, c.k, c.v, c.positions, c.slot_mapping = q, k, v, pos, sm
    return c


def run(w, c, dev, P, label, oracle_check=True):
    B, Hq, Hkv = w.B, w.Hq, w.Hkv
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    qw, kw, cs = c.q_norm_w.to(dev), c.k_norm_w.to(dev), c.cos_sin.to(dev)
    pos, sm = c.positions.to(dev), c.slot_mapping.to(dev)
    bt, lens = w.block_tables.to(dev), w.context_lens.to(dev)
    mcl = w.max_context_len
    kc0, vc0 = c.k_cache.to(dev), c.v_cache.to(dev)

    # the step from the other calls
    kc_a, vc_a = kc0.clone(), vc0.clone()
    q_out = torch.empty_like(q)
    fe.fe_qk_norm_rope_append(q_out, q, k, v, qw, kw, cs, pos, sm, kc_a, vc_a, c.eps)
    nslots = kc0.shape[0] * 16
    s_ok = (sm >= 0) & (sm < nslots)
    s_c = torch.where(s_ok, sm, torch.zeros_like(sm)).long()
    k_rows = kc_a[s_c // 16, :, s_c % 16, :].contiguous()  # [B][Hkv][D]; rows of skipped slots are not used
    kc_b, vc_b = kc0.clone(), vc0.clone()
    out_b = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lse_b = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    fe.fe_paged_gqa_decode_append(out_b, lse_b, q_out, k_rows, v, sm, kc_b, vc_b, bt, lens, mcl, w.scale,
                                  num_partitions=P)

    # the fused call
    kc_c, vc_c = kc0.clone(), vc0.clone()
    out_c = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lse_c = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    fe.fe_paged_gqa_decode_norm_rope_append(out_c, lse_c, q, k, v, qw, kw, cs, pos, sm, kc_c, vc_c, bt, lens, mcl,
                                            w.scale, c.eps, num_partitions=P)
    torch.cuda.synchronize()
    # bit patterns throughout (the pools hold NaN poison where nothing is read)
    ka, va = u16(kc_a), u16(vc_a)
    assert np.array_equal(u16(kc_c), ka) and np.array_equal(u16(vc_c), va), (label, "pools differ from the norm/rotary call's")
    assert np.array_equal(u16(kc_b), ka) and np.array_equal(u16(vc_b), va), (label, "append-decode pools differ")
    assert np.array_equal(u16(out_c), u16(out_b)), (label, "out differs from the composed step")
    assert np.array_equal(lse_c.cpu().numpy().view(np.uint32), lse_b.cpu().numpy().view(np.uint32)), (
        label, "lse differs from the composed step")

    if oracle_check:
        rq, rk, rkc, rvc = oracle.qk_norm_rope_append(c.q, c.k, c.v, c.q_norm_w, c.k_norm_w, c.cos_sin, c.positions,
                                                      c.slot_mapping, c.k_cache, c.v_cache, c.eps)
        assert np.array_equal(va, rvc), (label, "V pool differs from the oracle's")
        gq = u16(q_out)
        assert_rope_close(gq, rq, rope_term(norm_only_rows(c.q, c.q_norm_w, c.eps), c.cos_sin, c.positions),
                          f"{label} q rows")
        sm_h = c.slot_mapping.numpy().astype(np.int64)
        ok = (sm_h >= 0) & (sm_h < nslots)
        kt = rope_term(norm_only_rows(c.k, c.k_norm_w, c.eps), c.cos_sin, c.positions)
        assert_rope_close(ka[sm_h[ok] // 16, :, sm_h[ok] % 16, :], rk[ok], kt[ok], f"{label} k rows")
        written = np.zeros(ka.shape[:1] + ka.shape[2:3], bool)
        written[sm_h[ok] // 16, sm_h[ok] % 16] = True
        outside = np.broadcast_to(~written[:, None, :, None], ka.shape)
        assert np.array_equal(ka[outside], rkc[outside]), (label, "K pool changed outside the written slots")
        ro, rl = oracle.decode(rq, rkc, rvc, w.block_tables, w.context_lens, w.scale)
        allow = rounding_allowance(gq, rq, ka, rkc, rvc, w.block_tables.numpy(), w.context_lens.numpy(), w.scale,
                                      ro)
        assert_attention(out_c, lse_c, ro, rl, f"{label} P={P}", allowance=allow)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8])
def test_decode_norm_rope_small(dev, G):
    # empty context, one token, partial and full last blocks, several partitions
    lens = [0, 1, 17, 32, 300, 2100]
    w = inputs.custom("decode", len(lens), 2 * G, 2, lens, 900 + G, append=1, poison="nan")
    c = per_sequence(w, inputs.norm_rope_case(w, 900 + G))
    for P in (0, 1, 3):
        run(w, c, dev, P, f"G={G}")


def test_decode_norm_rope_skipped_slots(dev):
    """A padding slot (-1) and an out-of-pool slot write nothing: that
    sequence's last position is read from the cache as it is (here: rows an
    earlier step wrote there), and q is still normalised."""
    lens = [40, 64, 33, 500]
    w = inputs.custom("decode", 4, 32, 8, lens, 910, append=1, poison="nan")
    c = per_sequence(w, inputs.norm_rope_case(w, 910))
    earlier = torch.full_like(c.slot_mapping, -1)
    earlier[1], earlier[2] = c.slot_mapping[1], c.slot_mapping[2]
    k0, v0 = oracle.append(c.k, c.v, earlier, c.k_cache, c.v_cache)
    c.k_cache = torch.from_numpy(k0.view(np.int16)).view(torch.bfloat16)
    c.v_cache = torch.from_numpy(v0.view(np.int16)).view(torch.bfloat16)
    sm = c.slot_mapping.clone()
    sm[1], sm[2] = -1, w.num_blocks * 16 + 3
    c.slot_mapping = sm
    run(w, c, dev, 0, "skipped slots")


def test_decode_norm_rope_positions_outside_the_table(dev):
    """Positions below 0 or past the table use its first or last row, as in
    fe_qk_norm_rope_append."""
    lens = [90, 200, 16]
    w = inputs.custom("decode", 3, 32, 8, lens, 911, append=1)
    c = per_sequence(w, inputs.norm_rope_case(w, 911, max_pos=100))
    p = c.positions.clone()
    p[0], p[1] = -3, 5000
    c.positions = p
    run(w, c, dev, 0, "positions outside the table")


def test_decode_norm_rope_qwen3_4b_b64(dev):
    """One decode step of the 64-sequence workload (contexts 1024-8192,
    positions up to 8191), every row against the oracle."""
    w = inputs.make("qwen3_4b_b64_ctx1024-8192", poison="nan")
    c = per_sequence(w, inputs.norm_rope_case(w, 12, max_pos=40960))
    run(w, c, dev, 0, "b64 decode step")


def test_decode_norm_rope_qwen3_4b_b4(dev):
    """Four sequences of the Qwen3-4B layer shape with contexts as in the
    36-layer workload (256..2048 tokens), with explicit partitions."""
    w = inputs.custom("decode", 4, 32, 8, [256, 700, 1500, 2048], 13, append=1, poison="nan")
    c = per_sequence(w, inputs.norm_rope_case(w, 13))
    for P in (0, 8, 16):
        run(w, c, dev, P, "b4 layer", oracle_check=P == 0)
