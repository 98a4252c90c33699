"""GPU parity of the sampler step (fe_sampler_softmax_argmax) against the
fp64 oracle.

Gate, from the arithmetic: the kernel evaluates 2^(s x log2 e - m) in fp32;
the exponent argument carries an absolute error of about |s x log2 e| 2^-23
(at most ~70 here, so ~1e-5 relative on a probability after exp2), the sum
of ~150k terms a relative error of a few 1e-6, and exp2 and the final
product one ulp each: about 2e-5 relative in all.  Probabilities must be
within 1e-4 relative (plus 1e-37 absolute, for values fp32 flushes or
underflows), the LSE within 1e-4, and the argmax -- an exact comparison of
the bf16 logits on both sides -- must be identical.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs

pytestmark = pytest.mark.gpu

REL, ABS, LSE_ABS = 1e-4, 1e-37, 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(c: inputs.SamplerCase, dev, label, with_probs=True, temps=True, form=0):
    B, V = c.logits.shape
    x = c.logits.to(dev)
    it = c.inv_temperature.to(dev) if temps else None
    probs = torch.full((B, V), float("nan"), dtype=torch.float32, device=dev) if with_probs else None
    lse = torch.full((B,), float("nan"), dtype=torch.float32, device=dev)
    am = torch.full((B,), -1, dtype=torch.int32, device=dev)
    fe.fe_sampler_softmax_argmax_ex(probs, lse, am, x, it, form)
    torch.cuda.synchronize()
    rp, rl, ra = oracle.sampler(c.logits, c.inv_temperature if temps else None, with_probs=with_probs)
    assert np.array_equal(am.cpu().numpy(), ra), (label, "argmax")
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), (label, "lse -inf pattern")
    fin = ~np.isneginf(rl)
    lerr = float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0
    assert lerr <= LSE_ABS, (label, "lse", lerr)
    if with_probs:
        gp = probs.cpu().numpy().astype(np.float64)
        err = np.abs(gp - rp)
        ok = err <= REL * rp + ABS
        worst = float((err / (REL * rp + ABS)).max())
        print(f"[{label}] worst err/bound {worst:.3f}, lse err {lerr:.2e}", flush=True)
        assert ok.all(), (label, "probs", worst)


# form 1: ranges (two launches); form 2: one workgroup per row (one launch)
FORMS = [1, 2]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("B,V", [(1, 8), (3, 16), (5, 1000), (64, 4104), (2, 40000), (3, 163840)])
def test_sampler_small(dev, B, V, form):
    run(inputs.sampler_case(B, V, seed=B + V, peaks=min(5, V)), dev, f"B={B} V={V} form {form}", form=form)


@pytest.mark.parametrize("form", FORMS)
def test_sampler_masked_rows_and_ties(dev, form):
    c = inputs.sampler_case(4, 4096, seed=3)
    x = c.logits.float()
    x[0, ::3] = float("-inf")                  # a third of the tokens masked
    x[1, :] = float("-inf")                    # every token masked
    x[2, [5, 900, 4095]] = 60.0                # three-way tie at the max: the lowest index wins
    x[3, :] = 1.25                             # all equal: index 0, uniform probabilities
    c.logits = x.to(torch.bfloat16)
    run(c, dev, f"masked / ties, form {form}", form=form)


@pytest.mark.parametrize("form", FORMS)
def test_sampler_no_temperature_and_no_probs(dev, form):
    c = inputs.sampler_case(6, 12000, seed=4)
    run(c, dev, f"no temperature, form {form}", temps=False, form=form)
    run(c, dev, f"argmax and lse only, form {form}", with_probs=False, form=form)


@pytest.mark.parametrize("form", [0, 2])
def test_sampler_qwen3_vocab_batch64(dev, form):
    """The sampler step of the 64-sequence decode batch over the full Qwen3
    vocabulary (automatic: the ranges form at 64 rows; and one workgroup per row)."""
    run(inputs.sampler_case(64, inputs.QWEN3_VOCAB, seed=5), dev, f"Qwen3 vocab B=64 form {form}", form=form)


@pytest.mark.parametrize("form", [0, 1])
def test_sampler_qwen3_vocab_batch256(dev, form):
    """256 rows of the full vocabulary: the automatic choice is one workgroup
    per row from 192 rows on; the ranges form beside it."""
    assert fe.fe_sampler_form(256, inputs.QWEN3_VOCAB) == 2
    c = inputs.sampler_case(256, inputs.QWEN3_VOCAB, seed=6)
    x, it = c.logits.to(dev), c.inv_temperature.to(dev)
    probs = torch.empty((256, inputs.QWEN3_VOCAB), dtype=torch.float32, device=dev)
    lse = torch.empty((256,), dtype=torch.float32, device=dev)
    am = torch.empty((256,), dtype=torch.int32, device=dev)
    fe.fe_sampler_softmax_argmax_ex(probs, lse, am, x, it, form)
    torch.cuda.synchronize()
    rows = list(range(0, 256, 17)) + [255]
    rp, rl, ra = oracle.sampler(c.logits[rows], c.inv_temperature[rows])
    assert np.array_equal(am.cpu().numpy()[rows], ra), "argmax"
    assert float(np.abs(lse.cpu().numpy()[rows].astype(np.float64) - rl).max()) <= LSE_ABS, "lse"
    gp = probs.cpu().numpy()[rows].astype(np.float64)
    assert (np.abs(gp - rp) <= REL * rp + ABS).all(), "probs"


def test_sampler_masked_rows_in_the_automatic_row_form(dev):
    """Masked rows and ties in a batch of 200 rows, which the automatic choice
    runs one workgroup per row."""
    assert fe.fe_sampler_form(200, 2048) == 2
    c = inputs.sampler_case(200, 2048, seed=8)
    x = c.logits.float()
    x[7, :] = float("-inf")
    x[8, ::2] = float("-inf")
    x[9, [3, 1000, 2047]] = 50.0
    x[199, :] = -3.5
    c.logits = x.to(torch.bfloat16)
    run(c, dev, "B=200 automatic (one workgroup per row)", form=0)


def test_sampler_workspace_reused(dev):
    """One workspace of the largest size serves calls of different shapes in
    turn (each call's partials overwrite the previous call's; the 256-row
    call runs one workgroup per row and leaves the workspace alone)."""
    V = inputs.QWEN3_VOCAB
    ws = torch.empty(fe.fe_sampler_workspace_size(256, V), dtype=torch.uint8, device=dev)
    for B, seed in [(64, 21), (8, 22), (256, 23), (64, 24)]:
        c = inputs.sampler_case(B, V, seed=seed)
        x, it = c.logits.to(dev), c.inv_temperature.to(dev)
        probs = torch.empty((B, V), dtype=torch.float32, device=dev)
        lse = torch.empty((B,), dtype=torch.float32, device=dev)
        am = torch.empty((B,), dtype=torch.int32, device=dev)
        fe.fe_sampler_softmax_argmax(probs, lse, am, x, it, workspace=ws)
        torch.cuda.synchronize()
        rows = sorted({0, B // 3, B - 1})
        rp, rl, ra = oracle.sampler(c.logits[rows], c.inv_temperature[rows])
        assert np.array_equal(am.cpu().numpy()[rows], ra), (B, "argmax")
        assert float(np.abs(lse.cpu().numpy()[rows].astype(np.float64) - rl).max()) <= LSE_ABS, (B, "lse")
        gp = probs.cpu().numpy()[rows].astype(np.float64)
        assert (np.abs(gp - rp) <= REL * rp + ABS).all(), (B, "probs")


@pytest.mark.parametrize("form", [0, 1])
def test_sampler_more_rows_than_resident_workgroups(dev, form):
    """1024 rows of the full vocabulary: four rounds of one workgroup per row
    (the automatic choice), or ten ranges per row, ten times more workgroups
    than the GPU holds at once.  Sampled rows against the oracle."""
    B, V = 1024, inputs.QWEN3_VOCAB
    assert fe.fe_sampler_form(B, V) == 2
    c = inputs.sampler_case(B, V, seed=31)
    x, it = c.logits.to(dev), c.inv_temperature.to(dev)
    probs = torch.empty((B, V), dtype=torch.float32, device=dev)
    lse = torch.empty((B,), dtype=torch.float32, device=dev)
    am = torch.empty((B,), dtype=torch.int32, device=dev)
    fe.fe_sampler_softmax_argmax_ex(probs, lse, am, x, it, form)
    torch.cuda.synchronize()
    rows = list(range(0, B, 97)) + [B - 1]
    rp, rl, ra = oracle.sampler(c.logits[rows], c.inv_temperature[rows])
    assert np.array_equal(am.cpu().numpy()[rows], ra), "argmax"
    assert float(np.abs(lse.cpu().numpy()[rows].astype(np.float64) - rl).max()) <= LSE_ABS, "lse"
    gp = probs.cpu().numpy()[rows].astype(np.float64)
    assert (np.abs(gp - rp) <= REL * rp + ABS).all(), "probs"
