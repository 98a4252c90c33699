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


def attention_errors(out_bf16: torch.Tensor, lse: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray):
    o = out_bf16.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    diff = o - ref_out
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rn = np.linalg.norm(ref_out, axis=-1)
    dn = np.linalg.norm(diff, axis=-1)
    empty = rn == 0
    assert np.all(dn[empty] == 0), "empty rows must be exactly zero"
    row_rel = float((dn[~empty] / rn[~empty]).max()) if np.any(~empty) else 0.0
    both_ninf = np.isneginf(lg) & np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse)), "lse -inf pattern differs"
    lse_err = float(np.abs(lg[~both_ninf] - ref_lse[~both_ninf]).max()) if np.any(~both_ninf) else 0.0
    return max_abs, row_rel, lse_err


def beyond_output_rounding(out_bf16: torch.Tensor, ref_out: np.ndarray) -> float:
    """Largest |gpu - ref| minus the error that rounding ref itself to bf16
    (nearest even) already makes: the arithmetic error of the kernel beyond
    what any bf16 output must carry.  Reported beside the gates, not gated."""
    o = out_bf16.float().cpu().numpy().astype(np.float64)
    r = torch.from_numpy(ref_out.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    if not o.size:
        return 0.0
    return float((np.abs(o - ref_out) - np.abs(r - ref_out)).max())


def log_margins(label, max_abs, row_rel, lse_err, rows, beyond=None):
    """Append one parity record to the JSON-lines file named by the
    FE_PARITY_LOG environment variable (when set), so the margins against the
    gates are kept, not only asserted."""
    path = os.environ.get("FE_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps({"test": test, "label": label, "max_abs": max_abs, "row_rel": row_rel, "lse_abs": lse_err,
                            "rows": rows, "max_abs_beyond_rounding": beyond}) + "\n")


def assert_attention(out_bf16, lse, ref_out, ref_lse, label=""):
    max_abs, row_rel, lse_err = attention_errors(out_bf16, lse, ref_out, ref_lse)
    print(f"[{label}] max_abs {max_abs:.3e} row_rel {row_rel:.3e} lse_abs {lse_err:.3e}", flush=True)
    if os.environ.get("FE_PARITY_LOG"):
        log_margins(label, max_abs, row_rel, lse_err, int(np.prod(ref_lse.shape)),
                    beyond_output_rounding(out_bf16, ref_out))
    assert max_abs <= MAX_ABS, (label, "max_abs", max_abs)
    assert row_rel <= ROW_REL, (label, "row_rel", row_rel)
    assert lse_err <= LSE_ABS, (label, "lse", lse_err)


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

    def prefill(self, max_q_len=None, key_groups=None):
        """fe_paged_gqa_prefill_chunk, or fe_paged_gqa_prefill_chunk_ex with
        the given tile shape (key_groups 0, 1, 2 or 3)."""
        w = self.w
        total_q = self.q.shape[0]
        out = torch.full((total_q, w.Hq, 128), float("nan"), dtype=torch.bfloat16, device=self.dev)
        lse = torch.full((total_q, w.Hq), float("nan"), dtype=torch.float32, device=self.dev)
        qsl = w.query_start_loc.tolist()
        mql = max(b - a for a, b in zip(qsl[:-1], qsl[1:])) if max_q_len is None else max_q_len
        if key_groups is None:
            fe.fe_paged_gqa_prefill_chunk(out, lse, self.q, self.qsl, self.kc, self.vc, self.bt, self.lens, mql,
                                          w.max_context_len, w.scale)
        else:
            fe.fe_paged_gqa_prefill_chunk_ex(out, lse, self.q, self.qsl, self.kc, self.vc, self.bt, self.lens, mql,
                                             w.max_context_len, w.scale, key_groups)
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
