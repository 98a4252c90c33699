"""CPU checks of tests/gpu_util.rounding_allowance, the per-row widening of
the attention gate for inputs that a fused step rounds itself: with q rows
and cached k rows altered by one bf16 step in a few elements, the allowance
must equal the change those alterations make to the oracle's own LSE and
output, row by row, and be zero on untouched rows.  Both sides here are the
oracle (no GPU)."""
import numpy as np
import torch

import oracle
from paged_kv_gqa_slot_amd import inputs
from gpu_util import rounding_allowance, u16


def _bits_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)


def test_rounding_allowance_is_the_exact_shift():
    w = inputs.custom("decode", 4, 8, 2, [5, 40, 17, 0], 4242, poison="nan")
    lay = w.layers[0]
    qr, kr, vr = u16(lay.q), u16(lay.k_cache), u16(lay.v_cache)
    bt, lens = w.block_tables.numpy(), w.context_lens.numpy()
    qa, ka = qr.copy(), kr.copy()
    qa[1, 3, 7] += 1          # one bf16 step up (same sign, same binade for these values)
    qa[2, 5, 100] -= 1
    blk = int(bt[1, 1])       # a key of sequence 1, KV head 0, inside its 40 tokens
    ka[blk, 0, 4, 17] += 1
    ro, rl = oracle.decode(_bits_tensor(qr), _bits_tensor(kr), _bits_tensor(vr), w.block_tables, w.context_lens,
                           w.scale)
    ao, al = oracle.decode(_bits_tensor(qa), _bits_tensor(ka), _bits_tensor(vr), w.block_tables, w.context_lens,
                           w.scale)
    d_lse, d_abs, d_rel = rounding_allowance(qa, qr, ka, kr, vr, bt, lens, w.scale, ro)
    fin = np.isfinite(rl)
    assert np.allclose(np.abs(al[fin] - rl[fin]), d_lse[fin], rtol=1e-6, atol=1e-12)
    assert np.allclose(np.abs(ao - ro).max(axis=-1), d_abs, rtol=1e-6, atol=1e-12)
    rn = np.linalg.norm(ro, axis=-1)
    want_rel = np.where(rn > 0, np.linalg.norm(ao - ro, axis=-1) / np.where(rn > 0, rn, 1), 0)
    assert np.allclose(want_rel, d_rel, rtol=1e-6, atol=1e-12)
    # rows touched: (1, 3) and every head of sequence 1's KV head 0 (its k row changed), (2, 5); others exact 0
    touched = np.zeros_like(d_lse, dtype=bool)
    touched[1, 0:4] = True
    touched[2, 5] = True
    assert np.all(d_lse[~touched] == 0) and np.all(d_abs[~touched] == 0)
    assert np.all(d_lse[touched] > 0)
