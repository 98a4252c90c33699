"""GPU parity of the fused per-head QK-RMSNorm + rotary + append step
(fe_qk_norm_rope_append) against the fp64 oracle.

Gate, from the arithmetic: the kernel computes in fp32 and the oracle in
fp64, each rounding once to bf16.  Before that rounding the fp32 result of
out = y_d c - y_p s (p the rotation partner of d) carries an absolute error
of a few units of 2^-24 (|y_d c| + |y_p s|), from the rounding of y and of
the two products; where the products do not cancel that is far below one
bf16 ulp, where they do it can be several ulps of the small result.  So each
element must satisfy |gpu - oracle| <= ulp_bf16(oracle) + 2^-20 (|y_d c| +
|y_p s|) (|y| from the oracle's norm-only result), and fewer than 1% of all
elements may differ at all.  V rows are a bit copy (exact), and every pool
byte the step does not write must keep its value (exact).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs
from gpu_util import assert_rope_close, norm_only_rows, rope_term, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_case(c: inputs.NormRopeCase, dev, label, in_place=False):
    q = c.q.to(dev)
    q_out = q if in_place else torch.full_like(q, float("nan"))
    kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
    fe.fe_qk_norm_rope_append(q_out, q, c.k.to(dev), c.v.to(dev), c.q_norm_w.to(dev), c.k_norm_w.to(dev),
                              c.cos_sin.to(dev), c.positions.to(dev), c.slot_mapping.to(dev), kc, vc, c.eps)
    torch.cuda.synchronize()
    rq, rk_rows, rkc, rvc = oracle.qk_norm_rope_append(c.q, c.k, c.v, c.q_norm_w, c.k_norm_w, c.cos_sin,
                                                       c.positions, c.slot_mapping, c.k_cache, c.v_cache, c.eps)
    # |y| of the bound: the oracle's norm-only rows (a table whose every row is cos 1, sin 0)
    yq = norm_only_rows(c.q, c.q_norm_w, c.eps)
    yk = norm_only_rows(c.k, c.k_norm_w, c.eps)
    assert_rope_close(u16(q_out), rq, rope_term(yq, c.cos_sin, c.positions), f"{label} q")
    gk, gv = u16(kc), u16(vc)
    assert np.array_equal(gv, rvc), f"{label}: V pool differs"
    # K pool: bytes outside the written slots exact; each written slot holds
    # its token's k rows (the last token written to a slot wins)
    sm = c.slot_mapping.numpy()
    nslots = gk.shape[0] * gk.shape[2]
    written = np.zeros((gk.shape[0], gk.shape[2]), bool)
    token_of = {}
    for t, slot in enumerate(sm):
        if 0 <= slot < nslots:
            written[slot // 16, slot % 16] = True
            token_of[int(slot)] = t
    mask = np.broadcast_to(written[:, None, :, None], gk.shape)
    assert np.array_equal(gk[~mask], rkc[~mask]), f"{label}: K pool changed outside the written slots"
    toks = np.array(sorted(token_of.values()), dtype=np.int64)
    slots = np.array([sm[t] for t in toks], dtype=np.int64)
    got_rows = gk[slots // 16, :, slots % 16, :]
    want_rows = rkc[slots // 16, :, slots % 16, :]
    assert np.array_equal(want_rows, rk_rows[toks]), f"{label}: oracle pool/rows disagree"
    term_k = rope_term(yk, c.cos_sin, c.positions)[toks]
    assert_rope_close(got_rows, want_rows, term_k, f"{label} k")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (16, 8), (8, 8), (4, 1)])
def test_norm_rope_small(dev, Hq, Hkv):
    w = inputs.custom("prefill", 3, Hq, Hkv, [40, 17, 200], 700 + Hq, append=17, chunk=17, poison="nan")
    c = inputs.norm_rope_case(w, 700 + Hq)
    run_case(c, dev, f"small {Hq}/{Hkv}")


def test_norm_rope_edge_slots_and_positions(dev):
    """Padding and out-of-pool slots write nothing (q_out still written);
    positions outside the table use its first or last row."""
    w = inputs.custom("prefill", 2, 32, 8, [64, 30], 710, append=12, chunk=12, poison="large")
    c = inputs.norm_rope_case(w, 710, max_pos=50)
    sm = c.slot_mapping.clone()
    sm[0], sm[5] = -1, w.num_blocks * 16 + 7
    c.slot_mapping = sm
    pos = c.positions.clone()
    pos[1], pos[2], pos[3] = -5, 50, 10_000
    c.positions = pos
    run_case(c, dev, "edge slots/positions")


def test_norm_rope_in_place(dev):
    w = inputs.custom("prefill", 2, 32, 8, [100, 90], 711, append=33, chunk=33)
    run_case(inputs.norm_rope_case(w, 711), dev, "in place", in_place=True)


def test_norm_rope_prefill_chunk_workload(dev):
    """The 4 x 256 appended tokens of the chunked-prefill workload (positions 4096..4351)."""
    w = inputs.make("qwen3_4b_b4_prefix4096_chunk256", poison="nan")
    run_case(inputs.norm_rope_case(w, 5), dev, "prefill chunk 1024 tokens")


def test_norm_rope_decode_step_workload(dev):
    """One decode step of the 64-sequence workload (positions up to 8191)."""
    w = inputs.make("qwen3_4b_b64_ctx1024-8192", poison="nan")
    run_case(inputs.norm_rope_case(w, 6, max_pos=40960), dev, "decode step 64 tokens")
