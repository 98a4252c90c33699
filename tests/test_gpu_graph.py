"""The calls captured in a HIP graph (the way a serving loop replays its
step): every replay, with other GPU work run eagerly in between, must give
exactly the results of the same calls launched eagerly (the kernels reduce in
a fixed order, so the outputs are bit-identical).  Covers KV append + split-K
decode (pass 1 + merge), the mixed launch (in-kernel merge through the
workspace counters), append fused into decode, the fused norm/rotary/append step,
append + prefill (both weight forms) and the sampler."""
import pytest
import torch

import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def replay_matches(step, outputs, dev, replays=3, updated=()):
    """Run step eagerly, capture it, then replay it several times; after each
    replay the outputs must equal the eager ones bit for bit.  `outputs` are
    fully written by the step (poisoned before each replay); `updated` are
    tensors it changes in part (reset to their state before the step)."""
    before = [u.clone() for u in updated]
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in list(outputs) + list(updated)]
    for u, b in zip(updated, before):
        u.copy_(b)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    noise = torch.randn(1 << 20, device=dev)
    for r in range(replays):
        for o in outputs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(-1)
        for u, b in zip(updated, before):
            u.copy_(b)
        torch.cuda.synchronize()
        g.replay()
        noise.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        for o, w in zip(list(outputs) + list(updated), want):
            assert torch.equal(o, w) or (o.is_floating_point() and torch.equal(o.isnan(), w.isnan())
                                         and torch.equal(torch.nan_to_num(o), torch.nan_to_num(w))), r


def test_graph_append_and_split_decode(dev):
    w = inputs.custom("decode", 6, 32, 8, [700, 1500, 64, 999, 3000, 17], 801, append=1)
    lay = w.layers[0]
    kc, vc = lay.k_cache.to(dev), lay.v_cache.to(dev)
    kn, vn, sm = lay.k_new.to(dev), lay.v_new.to(dev), w.slot_mapping.to(dev)
    q, bt, cl = lay.q.to(dev), w.block_tables.to(dev), w.context_lens.to(dev)
    out = torch.empty(6, 32, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(6, 32, dtype=torch.float32, device=dev)
    ws = torch.zeros(fe.fe_paged_gqa_decode_workspace_size(6, 32, 8, 128, w.max_context_len, 8), dtype=torch.uint8,
                     device=dev)

    def step():
        fe.fe_paged_kv_append(kn, vn, sm, kc, vc)
        fe.fe_paged_gqa_decode(out, lse, q, kc, vc, bt, cl, w.max_context_len, w.scale, num_partitions=8,
                               workspace=ws)

    replay_matches(step, [out, lse], dev, updated=[kc, vc])


def test_graph_mixed(dev):
    w = inputs.custom("mixed", 5, 32, 8, [3000, 1500, 64, 17, 700], 802, append=40, chunk=40, num_decode=3)
    lay = w.layers[0]
    kc, vc = lay.k_cache.to(dev), lay.v_cache.to(dev)
    kn, vn, sm = lay.k_new.to(dev), lay.v_new.to(dev), w.slot_mapping.to(dev)
    q, qsl = lay.q.to(dev), w.query_start_loc.to(dev)
    bt, cl = w.block_tables.to(dev), w.context_lens.to(dev)
    total_q = q.shape[0]
    out = torch.empty(total_q, 32, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(total_q, 32, dtype=torch.float32, device=dev)
    ws = torch.zeros(fe.fe_paged_gqa_mixed_workspace_size(3, 32, 8, 128, w.max_context_len, 6), dtype=torch.uint8,
                     device=dev)

    def step():
        fe.fe_paged_kv_append(kn, vn, sm, kc, vc)
        fe.fe_paged_gqa_mixed(out, lse, q, qsl, kc, vc, bt, cl, 3, 40, w.max_context_len, w.scale, num_partitions=6,
                              workspace=ws)

    replay_matches(step, [out, lse], dev, updated=[kc, vc])
    assert int(ws[: 3 * 8 * 4].view(torch.int32).abs().sum()) == 0


def test_graph_norm_rope(dev):
    w = inputs.custom("prefill", 3, 32, 8, [100, 40, 300], 803, append=33, chunk=33)
    c = inputs.norm_rope_case(w, 803)
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    qw, kw, cs = c.q_norm_w.to(dev), c.k_norm_w.to(dev), c.cos_sin.to(dev)
    pos, sm = c.positions.to(dev), c.slot_mapping.to(dev)
    kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
    q_out = torch.empty_like(q)

    def step():
        fe.fe_qk_norm_rope_append(q_out, q, k, v, qw, kw, cs, pos, sm, kc, vc, c.eps)

    replay_matches(step, [q_out], dev, updated=[kc, vc])


def test_graph_decode_append(dev):
    """Append fused into split-K decode (pass 1 writes the new rows, pass 2
    merges) as a replayed graph."""
    lens = [700, 1500, 64, 999, 16, 1]
    w = inputs.custom("decode", 6, 32, 8, lens, 81, append=1)
    lay = w.layers[0]
    kn, vn = lay.k_new.to(dev), lay.v_new.to(dev)  # every sequence has one new token
    slots = w.slot_mapping.to(dev)
    kc, vc = lay.k_cache.to(dev), lay.v_cache.to(dev)
    q, bt, cl = lay.q.to(dev), w.block_tables.to(dev), w.context_lens.to(dev)
    out = torch.empty(6, 32, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(6, 32, dtype=torch.float32, device=dev)
    ws = torch.empty(fe.fe_paged_gqa_decode_workspace_size(6, 32, 8, 128, w.max_context_len, 4), dtype=torch.uint8,
                     device=dev)

    def step():
        fe.fe_paged_gqa_decode_append(out, lse, q, kn, vn, slots, kc, vc, bt, cl, w.max_context_len, w.scale,
                                      num_partitions=4, workspace=ws)

    replay_matches(step, [out, lse], dev, updated=[kc, vc])


def test_graph_decode_norm_rope_append(dev):
    """The one-launch attention step (norm/rotary of q and the new k, the
    append, split-K decode) as a replayed graph."""
    lens = [700, 1500, 64, 999, 16, 1]
    w = inputs.custom("decode", 6, 32, 8, lens, 82, append=1)
    c = inputs.norm_rope_case(w, 82)  # every sequence has one new token
    q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
    qw, kw, cs = c.q_norm_w.to(dev), c.k_norm_w.to(dev), c.cos_sin.to(dev)
    pos, slots = c.positions.to(dev), c.slot_mapping.to(dev)
    kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
    bt, cl = w.block_tables.to(dev), w.context_lens.to(dev)
    out = torch.empty(6, 32, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(6, 32, dtype=torch.float32, device=dev)
    ws = torch.empty(fe.fe_paged_gqa_decode_workspace_size(6, 32, 8, 128, w.max_context_len, 4), dtype=torch.uint8,
                     device=dev)

    def step():
        fe.fe_paged_gqa_decode_norm_rope_append(out, lse, q, k, v, qw, kw, cs, pos, slots, kc, vc, bt, cl,
                                                w.max_context_len, w.scale, c.eps, num_partitions=4, workspace=ws)

    replay_matches(step, [out, lse], dev, updated=[kc, vc])


@pytest.mark.parametrize("B", [64, 256])
def test_graph_sampler(dev, B):
    """The sampler step as a replayed graph, the way the vocabulary
    benchmark launches it: two passes through a caller-owned workspace at 64
    rows, one workgroup per row at 256."""
    c = inputs.sampler_case(B, inputs.QWEN3_VOCAB, seed=11)
    x, it = c.logits.to(dev), c.inv_temperature.to(dev)
    B, V = c.logits.shape
    probs = torch.empty(B, V, dtype=torch.float32, device=dev)
    lse = torch.empty(B, dtype=torch.float32, device=dev)
    am = torch.empty(B, dtype=torch.int32, device=dev)
    ws = torch.empty(max(fe.fe_sampler_workspace_size(B, V), 1), dtype=torch.uint8, device=dev)

    def step():
        fe.fe_sampler_softmax_argmax(probs, lse, am, x, it, workspace=ws)

    replay_matches(step, [probs, lse, am], dev)


@pytest.mark.parametrize("split", [0, 1])
def test_graph_prefill(dev, split):
    """KV append of the chunks, then the prefill call (split_weights 0 and 1)."""
    w = inputs.custom("prefill", 3, 32, 8, [300, 90, 1100], 806, append=70, chunk=70)
    lay = w.layers[0]
    kc, vc = lay.k_cache.to(dev), lay.v_cache.to(dev)
    kn, vn, sm = lay.k_new.to(dev), lay.v_new.to(dev), w.slot_mapping.to(dev)
    q, qsl, bt, cl = lay.q.to(dev), w.query_start_loc.to(dev), w.block_tables.to(dev), w.context_lens.to(dev)
    out = torch.empty(q.shape[0], 32, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[0], 32, dtype=torch.float32, device=dev)

    def step():
        fe.fe_paged_kv_append(kn, vn, sm, kc, vc)
        fe.fe_paged_gqa_prefill_chunk_ex(out, lse, q, qsl, kc, vc, bt, cl, 70, w.max_context_len, w.scale, 0, split)

    replay_matches(step, [out, lse], dev, updated=[kc, vc])
