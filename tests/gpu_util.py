"""Helpers for the GPU parity tests: run a workload through libfe.so and
compare with the oracle to the stated gates."""
import json
import os

import numpy as np
import torch

import oracle
import paged_kv_gqa_slot_amd as fe

# Gates: append bit-exact; attention max-abs 1e-2, row-relative L2 1e-2,
# LSE absolute 1e-3 (natural log).
MAX_ABS = 1e-2
ROW_REL = 1e-2
LSE_ABS = 1e-3


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def attention_row_errors(out_bf16: torch.Tensor, lse: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray):
    """Per (row, head): max |out - ref|, relative L2 error ||out - ref|| / ||ref||
    (0 for an empty row, which must be exactly zero) and |LSE - ref| (0 where
    both are -inf, which must coincide)."""
    o = out_bf16.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    diff = o - ref_out
    abs_row = np.abs(diff).max(axis=-1) if diff.size else np.zeros(diff.shape[:-1])
    rn = np.linalg.norm(ref_out, axis=-1)
    dn = np.linalg.norm(diff, axis=-1)
    empty = rn == 0
    assert np.all(dn[empty] == 0), "empty rows must be exactly zero"
    rel_row = np.where(empty, 0.0, dn / np.where(empty, 1.0, rn))
    ninf = np.isneginf(lg)
    assert np.array_equal(ninf, np.isneginf(ref_lse)), "lse -inf pattern differs"
    with np.errstate(invalid="ignore"):
        lse_row = np.where(ninf, 0.0, np.abs(lg - ref_lse))
    return abs_row, rel_row, lse_row


def _top(a: np.ndarray) -> float:
    return float(a.max()) if a.size else 0.0


def attention_errors(out_bf16: torch.Tensor, lse: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray):
    return tuple(_top(a) for a in attention_row_errors(out_bf16, lse, ref_out, ref_lse))


def beyond_output_rounding(out_bf16: torch.Tensor, ref_out: np.ndarray) -> float:
    """Largest |gpu - ref| minus the error that rounding ref itself to bf16
    (nearest even) already makes: the arithmetic error of the kernel beyond
    what any bf16 output must carry.  Reported beside the gates, not gated."""
    o = out_bf16.float().cpu().numpy().astype(np.float64)
    r = torch.from_numpy(ref_out.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    if not o.size:
        return 0.0
    return float((np.abs(o - ref_out) - np.abs(r - ref_out)).max())


def log_margins(label, max_abs, row_rel, lse_err, rows, beyond=None, row_rounding_lse=None):
    """Append one parity record to the JSON-lines file named by the
    FE_PARITY_LOG environment variable (when set), so the margins against the
    gates are kept, not only asserted."""
    path = os.environ.get("FE_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    rec = {"test": test, "label": label, "max_abs": max_abs, "row_rel": row_rel, "lse_abs": lse_err, "rows": rows,
           "max_abs_beyond_rounding": beyond}
    if row_rounding_lse is not None:
        rec["row_rounding_lse"] = row_rounding_lse
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def assert_attention(out_bf16, lse, ref_out, ref_lse, label="", allowance=None):
    """The attention gate.  `allowance`, from rounding_allowance, widens it
    row by row by the exact effect of inputs that the two sides rounded
    differently (a fused step's own bf16 rows)."""
    a, r, l = attention_row_errors(out_bf16, lse, ref_out, ref_lse)
    max_abs, row_rel, lse_err = _top(a), _top(r), _top(l)
    shift = None if allowance is None else _top(allowance[0])
    extra = "" if shift is None else f" (rounding of the rows moves lse by up to {shift:.3e})"
    print(f"[{label}] max_abs {max_abs:.3e} row_rel {row_rel:.3e} lse_abs {lse_err:.3e}{extra}", flush=True)
    if os.environ.get("FE_PARITY_LOG"):
        log_margins(label, max_abs, row_rel, lse_err, int(np.prod(ref_lse.shape)),
                    beyond_output_rounding(out_bf16, ref_out), shift)
    if allowance is None:
        assert max_abs <= MAX_ABS, (label, "max_abs", max_abs)
        assert row_rel <= ROW_REL, (label, "row_rel", row_rel)
        assert lse_err <= LSE_ABS, (label, "lse", lse_err)
    else:
        lse_extra, abs_extra, rel_extra = allowance
        assert np.all(a <= MAX_ABS + abs_extra), (label, "max_abs", max_abs, "allowance", _top(abs_extra))
        assert np.all(r <= ROW_REL + rel_extra), (label, "row_rel", row_rel, "allowance", _top(rel_extra))
        assert np.all(l <= LSE_ABS + lse_extra), (label, "lse", lse_err, "allowance", shift)


# ----------------------------------------------------------------------------
# Rows of the norm/rotary step.  Its gate (stated with its tests): each element
# within one bf16 step of the oracle's, plus 2^-20 (|y_d c| + |y_p s|) where the
# two rotation products cancel, and fewer than MISMATCH_FRAC of them differing.

MISMATCH_FRAC = 1e-2


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (2^-133 below the normal range)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def norm_only_rows(x: torch.Tensor, w: torch.Tensor, eps: float) -> np.ndarray:
    """The oracle's RMSNorm-only rows (its norm/rotary step over a one-row
    table of cos 1, sin 0), bits [T][H][D]."""
    ident = torch.zeros(1, 128)
    ident[0, :64] = 1.0
    zero = torch.zeros(x.shape[0], dtype=torch.int32)
    return oracle.norm_rope(x, w, ident, zero, eps)


def rope_term(y_bits: np.ndarray, cos_sin: torch.Tensor, positions: torch.Tensor) -> np.ndarray:
    """|y_d c| + |y_p s| per element of [T][H][D] rows (p = partner of d)."""
    y = bf16_values(y_bits)
    T, H, Dm = y.shape
    half = Dm // 2
    cs = cos_sin.numpy().astype(np.float64)
    pos = np.clip(positions.numpy(), 0, cs.shape[0] - 1)
    c = np.abs(np.concatenate([cs[pos, :half], cs[pos, :half]], axis=1))[:, None, :]
    s = np.abs(np.concatenate([cs[pos, half:], cs[pos, half:]], axis=1))[:, None, :]
    partner = np.concatenate([y[..., half:], y[..., :half]], axis=-1)
    return np.abs(y) * c + np.abs(partner) * s


def assert_rope_close(got: np.ndarray, want: np.ndarray, term: np.ndarray, label: str):
    assert got.shape == want.shape == term.shape, label
    g, w = bf16_values(got), bf16_values(want)
    err = np.abs(g - w)
    bound = ulp_bf16(w) + 2.0 ** -20 * term
    frac = float((got != want).mean()) if got.size else 0.0
    worst = float((err / bound).max()) if got.size else 0.0
    print(f"[{label}] worst err/bound {worst:.3f}, differing {frac:.2e}", flush=True)
    assert np.all(err <= bound), (label, "bound", worst)
    assert frac <= MISMATCH_FRAC, (label, "fraction", frac)


def rounding_allowance(q_gpu, q_ref, kp_gpu, kp_ref, vp, block_tables, context_lens, scale, ref_out):
    """Per-row allowance for a decode whose q rows and cached k rows came out
    of a rounding step on each side (the norm/rotary step: bf16 rows that may
    differ by the one-step flips its gate admits, where the fp32 and the fp64
    result straddle a rounding boundary).

    For row (b, h) with keys j: the oracle's scores s_j = scale q_r . k_r,j and
    weights p = softmax(s), and the score shifts d_j = scale (q_g . k_g,j -
    q_r . k_r,j) that the GPU's rows make, all in fp64.  Over the GPU's rows
    the exact LSE is the oracle's plus log sum_j p_j e^(d_j), and the exact
    output the oracle's plus sum_j (p'_j - p_j) v_j with p' = softmax(s + d).
    A kernel within the gate of the exact decode over its own rows is, by the
    triangle inequality, within the gate plus these shifts of the oracle's.
    The expected values stay the oracle's: the GPU's rows only size the
    allowance, and they are held to the norm/rotary gate themselves.  All rows
    are bits: q [B][Hq][D], pools [NB][Hkv][16][D].  Returns the allowance on
    LSE, max-abs and row-relative error, each [B][Hq]; rows whose q and keys
    match the oracle's exactly get 0."""
    B, Hq, Dm = q_ref.shape
    Hkv = kp_ref.shape[1]
    G = Hq // Hkv
    bt = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    q_diff = np.any(q_gpu != q_ref, axis=-1)
    blk_diff = np.any(kp_gpu != kp_ref, axis=(2, 3))
    d_lse = np.zeros((B, Hq))
    d_abs = np.zeros((B, Hq))
    d_rel = np.zeros((B, Hq))
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        blocks = bt[b, :(L + 15) // 16].astype(np.int64)
        for kh in range(Hkv):
            k_changed = bool(blk_diff[blocks, kh].any())
            heads = [h for h in range(kh * G, (kh + 1) * G) if k_changed or q_diff[b, h]]
            if not heads:
                continue
            kg = bf16_values(kp_gpu[blocks, kh].reshape(-1, Dm)[:L])
            kr = bf16_values(kp_ref[blocks, kh].reshape(-1, Dm)[:L])
            v = bf16_values(vp[blocks, kh].reshape(-1, Dm)[:L])
            for h in heads:
                s_r = scale * (kr @ bf16_values(q_ref[b, h]))
                d = scale * (kg @ bf16_values(q_gpu[b, h])) - s_r
                p = np.exp(s_r - s_r.max())
                p /= p.sum()
                e = p * np.exp(d - d.max())
                d_lse[b, h] = abs(d.max() + np.log(e.sum()))
                dout = (e / e.sum() - p) @ v
                d_abs[b, h] = float(np.abs(dout).max())
                rn = float(np.linalg.norm(ref_out[b, h]))
                d_rel[b, h] = float(np.linalg.norm(dout)) / rn if rn > 0 else 0.0
    return d_lse, d_abs, d_rel


class DeviceWorkload:
    """A workload's tensors on the GPU plus its oracle-side appended pools."""

    def __init__(self, w, dev, layer=0):
        self.w = w
        lay = w.layers[layer]
        self.lay = lay
        self.kc = lay.k_cache.to(dev)
        self.vc = lay.v_cache.to(dev)
        self.q = lay.q.to(dev)
        self.k_new = lay.k_new.to(dev)
        self.v_new = lay.v_new.to(dev)
        self.slots = w.slot_mapping.to(dev)
        self.bt = w.block_tables.to(dev)
        self.lens = w.context_lens.to(dev)
        self.qsl = w.query_start_loc.to(dev) if w.query_start_loc is not None else None
        self.dev = dev

    def append(self, check=True):
        fe.fe_paged_kv_append(self.k_new, self.v_new, self.slots, self.kc, self.vc)
        rk, rv = oracle.append(self.lay.k_new, self.lay.v_new, self.w.slot_mapping, self.lay.k_cache,
                               self.lay.v_cache)
        if check:
            torch.cuda.synchronize()
            assert np.array_equal(u16(self.kc), rk), "K pool differs after append"
            assert np.array_equal(u16(self.vc), rv), "V pool differs after append"
        return rk, rv

    def decode(self, num_partitions=0, max_context_len=None):
        w = self.w
        out = torch.full((w.B, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=self.dev)
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=self.dev)
        mcl = w.max_context_len if max_context_len is None else max_context_len
        fe.fe_paged_gqa_decode(out, lse, self.q, self.kc, self.vc, self.bt, self.lens, mcl, w.scale,
                               num_partitions=num_partitions)
        torch.cuda.synchronize()
        return out, lse

    def prefill(self, max_q_len=None, key_groups=None, split_weights=0):
        """fe_paged_gqa_prefill_chunk, or fe_paged_gqa_prefill_chunk_ex with
        the given tile shape (key_groups 0, 1, 2 or 3) and weight precision
        (split_weights 0 or 1)."""
        w = self.w
        total_q = self.q.shape[0]
        out = torch.full((total_q, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=self.dev)
        lse = torch.full((total_q, w.Hq), float("nan"), dtype=torch.float32, device=self.dev)
        qsl = w.query_start_loc.tolist()
        mql = max(b - a for a, b in zip(qsl[:-1], qsl[1:])) if max_q_len is None else max_q_len
        if key_groups is None and not split_weights:
            fe.fe_paged_gqa_prefill_chunk(out, lse, self.q, self.qsl, self.kc, self.vc, self.bt, self.lens, mql,
                                          w.max_context_len, w.scale)
        else:
            fe.fe_paged_gqa_prefill_chunk_ex(out, lse, self.q, self.qsl, self.kc, self.vc, self.bt, self.lens, mql,
                                             w.max_context_len, w.scale, key_groups or 0, split_weights)
        torch.cuda.synchronize()
        return out, lse

    def mixed(self, num_partitions=0, workspace=None):
        """Decode rows (the first spec.num_decode sequences) and prefill chunks in one launch."""
        w = self.w
        nd = w.spec.num_decode
        total_q = self.q.shape[0]
        out = torch.full((total_q, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=self.dev)
        lse = torch.full((total_q, w.Hq), float("nan"), dtype=torch.float32, device=self.dev)
        qsl = w.query_start_loc.tolist()
        chunks = [b - a for a, b in zip(qsl[:-1], qsl[1:])]
        mql = max(chunks[nd:], default=0)
        fe.fe_paged_gqa_mixed(out, lse, self.q, self.qsl, self.kc, self.vc, self.bt, self.lens, nd, mql,
                              w.max_context_len, w.scale, num_partitions=num_partitions, workspace=workspace)
        torch.cuda.synchronize()
        return out, lse
