"""Seeded synthetic workloads for paged GQA attention.

This module only builds inputs: sequence lengths, block placement in a shared
pool, bf16 query/key/value values, slot mappings and poison fill.  It holds
none of the attention arithmetic and imports neither the HIP binding nor the
oracle, so both sides can be fed the same bytes.

The shapes are the Qwen3 layer shapes of the two models the pages run --
Qwen3-0.6B in "Make the Engine Talk" section 1.1, Qwen3-4B-Instruct-2507 in
the ForgeEngine README -- at head_dim 128 and 16-token KV blocks.  The pages
name no benchmark data set; values are N(0, 1) drawn from torch's CPU
generator and rounded to bf16 (round to nearest even).

Layout (shared by every workload):
  * K and V pools: bf16 [num_blocks][Hkv][16][128], head-major inside a block;
  * block_tables: int32 [B][max_blocks_per_seq]; entries past a sequence's
    last block point at a dedicated poisoned block;
  * slot = block * 16 + offset (int32); context_lens[b] counts the tokens
    appended this step;
  * every pool slot that holds no token -- unused blocks, tail slots of a
    sequence's last block, the slots appended tokens will fill -- holds poison
    (a large finite bf16 value, or NaN).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

D = 128
BS = 16
POISON_LARGE = 30000.0


def fp32_scale(head_dim: int = D) -> float:
    """1/sqrt(head_dim) rounded to fp32 (the value every call receives)."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


# Stream ids: every random quantity gets its own generator so that changing
# one size does not shift the others.
_LEN, _PERM, _Q, _K, _V, _SPIKE = 1, 2, 3, 4, 5, 6
_NR_Q, _NR_K, _NR_V, _NR_W = 7, 8, 9, 10  # inputs of the norm/rotary step
_SM_X, _SM_PEAK = 11, 12                   # inputs of the sampler step


def _gen(seed: int, stream: int, layer: int = 0) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 100003 + layer * 101 + stream)


@dataclass
class Spec:
    """Shape recipe of one workload."""

    name: str
    kind: str  # "decode", "prefill" or "mixed"
    B: int
    Hq: int
    Hkv: int
    len_lo: int  # context length range (inclusive), counting appended tokens
    len_hi: int
    append: int = 0  # tokens appended per sequence before attention
    layers: int = 1  # independent pools (one decode call each)
    pool_blocks: Optional[int] = None  # fixed pool size, else 1.125 x needed
    spike_frac: float = 0.0  # fraction of token positions whose K is x spike_mul
    spike_mul: float = 3.0
    chunk: int = 0  # prefill query chunk per sequence (bottom-right causal)
    # "mixed": sequences [0, num_decode) are decode rows (1 token appended, 1
    # query row, lengths drawn from [len_lo, len_hi]); the others are prefill
    # chunks of `chunk` rows (`append` tokens appended) with length pre_len.
    num_decode: int = 0
    pre_len: int = 0


# The five workloads.  Names state the model shape and the sizes.
SPECS = {
    # Qwen3-0.6B layer (16 q heads, 8 KV heads, G = 2): one sequence of 128
    # tokens in 8 blocks of a 64-block pool; 1 token appended first.
    "qwen3_0.6b_b1_ctx128": Spec("qwen3_0.6b_b1_ctx128", "decode", 1, 16, 8, 128, 128, append=1,
                                 pool_blocks=64),
    # Qwen3-4B layer (32/8, G = 4), 4 sequences of 256..2048 tokens, 36 layers
    # with independent pools sharing one block table: one step = 36 calls.
    "qwen3_4b_b4_ctx256-2048_36layers": Spec("qwen3_4b_b4_ctx256-2048_36layers", "decode", 4, 32, 8, 256,
                                             2048, layers=36),
    # Qwen3-4B, 64 sequences of 1024..8192 tokens; K x3 on 1% of positions;
    # 1 token appended per sequence first.
    "qwen3_4b_b64_ctx1024-8192": Spec("qwen3_4b_b64_ctx1024-8192", "decode", 64, 32, 8, 1024, 8192,
                                      append=1, spike_frac=0.01),
    # Qwen3-4B long context: 8 sequences of 32768 tokens (split-K).
    "qwen3_4b_b8_ctx32768": Spec("qwen3_4b_b8_ctx32768", "decode", 8, 32, 8, 32768, 32768),
    # Qwen3-4B chunked prefill: 4 sequences of 4096 cached + 256 new tokens;
    # the 256-token chunks are appended, then attend causally.
    "qwen3_4b_b4_prefix4096_chunk256": Spec("qwen3_4b_b4_prefix4096_chunk256", "prefill", 4, 32, 8, 4352,
                                            4352, append=256, chunk=256),
}
# A mixed step of a token-budgeted batcher (decode rows and prefill chunks in
# one launch): 60 decode rows over 1024..8192 tokens and 4 chunks of 256 new
# tokens after 4096 cached ones, at the Qwen3-4B layer shape.
SPECS["qwen3_4b_mixed_dec60_ctx1024-8192_pre4_prefix4096_chunk256"] = Spec(
    "qwen3_4b_mixed_dec60_ctx1024-8192_pre4_prefix4096_chunk256", "mixed", 64, 32, 8, 1024, 8192, append=256,
    chunk=256, num_decode=60, pre_len=4352)
# A larger chunked-prefill step (64 chunks of 256 new tokens after 1024 cached
# ones, 16384 appended tokens): the token set on which the norm/rotary/append
# step's streaming rate is measured.
SPECS["qwen3_4b_b64_prefix1024_chunk256"] = Spec("qwen3_4b_b64_prefix1024_chunk256", "prefill", 64, 32, 8, 1280, 1280,
                                                 append=256, chunk=256)
ORDER = list(SPECS)  # default seed of SPECS[ORDER[i]] is i + 1


@dataclass
class Layer:
    k_cache: torch.Tensor  # bf16 [NB][Hkv][BS][D], before the append
    v_cache: torch.Tensor
    q: torch.Tensor  # bf16 [B][Hq][D] (decode) or [total_q][Hq][D] (prefill)
    k_new: torch.Tensor  # bf16 [T][Hkv][D]
    v_new: torch.Tensor
    k_seq: Optional[torch.Tensor] = None  # bf16 [sum L][Hkv][D], contiguous copy
    v_seq: Optional[torch.Tensor] = None


@dataclass
class Workload:
    spec: Spec
    seed: int
    scale: float
    num_blocks: int
    context_lens: torch.Tensor  # int32 [B]
    block_tables: torch.Tensor  # int32 [B][max_blocks_per_seq]
    slot_mapping: torch.Tensor  # int32 [T]
    query_start_loc: Optional[torch.Tensor]  # int32 [B+1] (prefill)
    poison_block: int
    layers: list = field(default_factory=list)

    @property
    def B(self):
        return self.spec.B

    @property
    def Hq(self):
        return self.spec.Hq

    @property
    def Hkv(self):
        return self.spec.Hkv

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.context_lens.numel() else 0

    @property
    def kv_tokens(self) -> int:
        return int(self.context_lens.sum().item())

    @property
    def seq_offsets(self) -> list:
        lens = self.context_lens.tolist()
        return [0] + list(np.cumsum(lens))


def _poison_value(poison: str) -> float:
    if poison == "large":
        return POISON_LARGE
    if poison == "nan":
        return float("nan")
    raise ValueError(poison)


def build(spec: Spec, seed: int, poison: str = "large", keep_contiguous: bool = False,
          lens: Optional[list] = None, layers: Optional[int] = None) -> Workload:
    """Generate one workload.  ``lens`` overrides the drawn context lengths
    (tests use it for edge cases); ``layers`` limits the number of pools."""
    B = spec.B
    if lens is None:
        if spec.len_lo == spec.len_hi:
            lens_t = torch.full((B,), spec.len_lo, dtype=torch.int64)
        else:
            lens_t = torch.randint(spec.len_lo, spec.len_hi + 1, (B,), generator=_gen(seed, _LEN))
        if spec.kind == "mixed":
            lens_t[spec.num_decode:] = spec.pre_len
    else:
        lens_t = torch.tensor(list(lens), dtype=torch.int64)
        assert lens_t.numel() == B
    lens_l = [int(x) for x in lens_t.tolist()]
    nd = spec.num_decode if spec.kind == "mixed" else 0
    appends = [1 if b < nd else spec.append for b in range(B)]
    nblk = [(L + BS - 1) // BS for L in lens_l]
    need = sum(nblk)
    if spec.pool_blocks is not None:
        NB = spec.pool_blocks
    else:
        NB = max(math.ceil(1.125 * need), need + 1)
    assert NB >= need + 1, "pool must keep one block for poison"
    perm = torch.randperm(NB, generator=_gen(seed, _PERM))
    max_blocks = max(1, max(nblk) if nblk else 1)
    poison_block = int(perm[need])
    bt = torch.full((B, max_blocks), poison_block, dtype=torch.int64)
    off = 0
    for b in range(B):
        bt[b, : nblk[b]] = perm[off : off + nblk[b]]
        off += nblk[b]

    # slot of every token, in sequence order; the last `append` tokens of each
    # sequence are the new ones (clamped for sequences shorter than that)
    tok_b = torch.repeat_interleave(torch.arange(B), torch.tensor(lens_l, dtype=torch.int64))
    tok_t = torch.cat([torch.arange(L) for L in lens_l]) if lens_l and sum(lens_l) else torch.zeros(0, dtype=torch.int64)
    tok_blk = bt[tok_b, tok_t // BS] if tok_t.numel() else tok_t
    tok_off = tok_t % BS
    is_new = torch.zeros(tok_t.shape, dtype=torch.bool)
    for b in range(B):
        a = min(appends[b], lens_l[b])
        if a:
            start = sum(lens_l[:b])
            is_new[start + lens_l[b] - a : start + lens_l[b]] = True
    slot_mapping = (tok_blk * BS + tok_off)[is_new].to(torch.int32)

    qsl = None
    total_q = B
    if spec.kind in ("prefill", "mixed"):
        chunks = [1 if b < nd else min(spec.chunk, L) for b, L in enumerate(lens_l)]
        qsl = torch.tensor([0] + list(np.cumsum(chunks)), dtype=torch.int32)
        total_q = int(qsl[-1])

    pv = _poison_value(poison)
    n_layers = spec.layers if layers is None else layers
    out_layers = []
    n_tok = tok_t.numel()
    for layer in range(n_layers):
        k = torch.randn((n_tok, spec.Hkv, D), generator=_gen(seed, _K, layer), dtype=torch.float32)
        if spec.spike_frac > 0 and n_tok:
            spike = torch.rand((n_tok,), generator=_gen(seed, _SPIKE, layer)) < spec.spike_frac
            k[spike] *= spec.spike_mul
        k = k.to(torch.bfloat16)
        v = torch.randn((n_tok, spec.Hkv, D), generator=_gen(seed, _V, layer), dtype=torch.float32).to(
            torch.bfloat16)
        q = torch.randn((total_q, spec.Hq, D), generator=_gen(seed, _Q, layer), dtype=torch.float32).to(
            torch.bfloat16)
        kc = torch.full((NB, spec.Hkv, BS, D), pv, dtype=torch.bfloat16)
        vc = torch.full((NB, spec.Hkv, BS, D), pv, dtype=torch.bfloat16)
        old = ~is_new
        # [NB][Hkv][BS][D] viewed as [NB][BS][Hkv][D] so (block, offset) indexes a token row
        kc.permute(0, 2, 1, 3)[tok_blk[old], tok_off[old]] = k[old]
        vc.permute(0, 2, 1, 3)[tok_blk[old], tok_off[old]] = v[old]
        out_layers.append(Layer(
            k_cache=kc, v_cache=vc, q=q,
            k_new=k[is_new].contiguous(), v_new=v[is_new].contiguous(),
            k_seq=k if keep_contiguous else None, v_seq=v if keep_contiguous else None))
        del k, v
    return Workload(spec=spec, seed=seed, scale=fp32_scale(D), num_blocks=NB,
                    context_lens=torch.tensor(lens_l, dtype=torch.int32),
                    block_tables=bt.to(torch.int32), slot_mapping=slot_mapping, query_start_loc=qsl,
                    poison_block=poison_block, layers=out_layers)


def make(name: str, seed: Optional[int] = None, **kw) -> Workload:
    """Workload by name; the default seed is the workload's 1-based position."""
    if seed is None:
        seed = ORDER.index(name) + 1
    return build(SPECS[name], seed, **kw)


def custom(kind: str, B: int, Hq: int, Hkv: int, lens, seed: int, append: int = 0, chunk: int = 0,
           spike_frac: float = 0.0, pool_blocks: Optional[int] = None, layers: int = 1, num_decode: int = 0,
           **kw) -> Workload:
    """Ad-hoc workload with explicit lengths (edge cases, small parity sizes).
    For kind "mixed", lens lists every sequence; the first num_decode are
    decode rows."""
    lens = list(lens)
    spec = Spec(f"custom_{kind}_b{B}_h{Hq}x{Hkv}", kind, B, Hq, Hkv, min(lens) if lens else 0,
                max(lens) if lens else 0, append=append, layers=layers, pool_blocks=pool_blocks,
                spike_frac=spike_frac, chunk=chunk, num_decode=num_decode)
    return build(spec, seed, lens=lens, **kw)


# ----------------------------------------------------------------------------
# Inputs of the per-head QK-RMSNorm + rotary + append step.

ROPE_BASE = 1_000_000.0  # Qwen3's rotary base
NORM_EPS = 1e-6          # Qwen3's RMSNorm epsilon


def appended_positions(w: Workload) -> torch.Tensor:
    """Positions of the appended tokens, in slot_mapping order (the last
    `append` tokens of each sequence; one for a mixed batch's decode rows)."""
    spec = w.spec
    nd = spec.num_decode if spec.kind == "mixed" else 0
    pos = []
    for b, L in enumerate(w.context_lens.tolist()):
        a = min(1 if b < nd else spec.append, L)
        pos.extend(range(L - a, L))
    return torch.tensor(pos, dtype=torch.int32)


def rope_table(max_pos: int, head_dim: int = D, base: float = ROPE_BASE) -> torch.Tensor:
    """The rotary table a caller keeps, fp32 [max_pos][head_dim]: for position
    p and pair d < head_dim / 2 the angle p * base^(-2d / head_dim) (in
    float64), its cosine at [p][d] and its sine at [p][head_dim / 2 + d]."""
    half = head_dim // 2
    inv = base ** (-torch.arange(half, dtype=torch.float64) * 2.0 / head_dim)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).contiguous()


@dataclass
class NormRopeCase:
    q: torch.Tensor         # bf16 [T][Hq][D], projected, before norm and rotation
    k: torch.Tensor         # bf16 [T][Hkv][D]
    v: torch.Tensor         # bf16 [T][Hkv][D]
    q_norm_w: torch.Tensor  # bf16 [D]
    k_norm_w: torch.Tensor  # bf16 [D]
    cos_sin: torch.Tensor   # fp32 [max_pos][D]
    positions: torch.Tensor  # int32 [T]
    slot_mapping: torch.Tensor  # int32 [T]
    k_cache: torch.Tensor   # bf16 pools, before the append
    v_cache: torch.Tensor
    eps: float = NORM_EPS


def norm_rope_case(w: Workload, seed: int, max_pos: Optional[int] = None) -> NormRopeCase:
    """The norm/rotary/append step of workload w's appended tokens: fresh
    projected rows (randn, bf16), norm weights 1 + 0.1 randn (bf16), the
    workload's slots and pools, and a rotary table covering its positions."""
    T = int(w.slot_mapping.numel())
    pos = appended_positions(w)
    assert pos.numel() == T
    if max_pos is None:
        max_pos = int(pos.max().item()) + 1 if T else 1
    q = torch.randn((T, w.Hq, D), generator=_gen(seed, _NR_Q), dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((T, w.Hkv, D), generator=_gen(seed, _NR_K), dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((T, w.Hkv, D), generator=_gen(seed, _NR_V), dtype=torch.float32).to(torch.bfloat16)
    ww = 1.0 + 0.1 * torch.randn((2, D), generator=_gen(seed, _NR_W), dtype=torch.float32)
    return NormRopeCase(q=q, k=k, v=v, q_norm_w=ww[0].to(torch.bfloat16), k_norm_w=ww[1].to(torch.bfloat16),
                        cos_sin=rope_table(max_pos), positions=pos, slot_mapping=w.slot_mapping.clone(),
                        k_cache=w.layers[0].k_cache, v_cache=w.layers[0].v_cache)


# ----------------------------------------------------------------------------
# Inputs of the sampler step (softmax / argmax over the vocabulary).

QWEN3_VOCAB = 151936
TEMPERATURES = (0.6, 0.7, 1.0, 1.3)  # cycled over the rows


@dataclass
class SamplerCase:
    logits: torch.Tensor           # bf16 [B][V]
    inv_temperature: torch.Tensor  # fp32 [B]


def sampler_case(B: int, V: int = QWEN3_VOCAB, seed: int = 1, peaks: int = 5) -> SamplerCase:
    """Language-model-like logits: 2.5 * randn, plus `peaks` tokens per row
    raised by 8..16 (the likely next tokens); rows cycle through TEMPERATURES."""
    g = _gen(seed, _SM_X)
    x = 2.5 * torch.randn((B, V), generator=g, dtype=torch.float32)
    if peaks and V:
        gp = _gen(seed, _SM_PEAK)
        idx = torch.randint(0, V, (B, peaks), generator=gp)
        x.scatter_add_(1, idx, 8.0 + 8.0 * torch.rand((B, peaks), generator=gp))
    it = torch.tensor([1.0 / TEMPERATURES[b % len(TEMPERATURES)] for b in range(B)], dtype=torch.float32)
    return SamplerCase(logits=x.to(torch.bfloat16), inv_temperature=it)
