"""C-ABI checks that need no GPU: libfe.so loads, exports every function
include/fe.h declares, and rejects bad arguments synchronously (before any
HIP call) with the documented status codes.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import paged_kv_gqa_slot_amd as fe
from paged_kv_gqa_slot_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fe.h")

OK, NULL, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3, -4
P = 0x1000  # a non-NULL placeholder pointer: never dereferenced on these paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libfe.so not built")
    return fe.load_library()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("fe_paged_kv_append", "fe_paged_gqa_decode", "fe_paged_gqa_prefill_chunk",
              "fe_paged_gqa_decode_workspace_size", "fe_status_string", "fe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libfe.so does not export {name}"


def test_python_binding_has_same_names():
    for name in declared_functions():
        assert hasattr(fe, name) or hasattr(binding, name), name


def test_status_strings(lib):
    assert fe.fe_status_string(0) == "FE_OK"
    assert fe.fe_status_string(-4) == "FE_ERR_WORKSPACE"
    assert fe.fe_status_string(12345) == "FE_ERR_UNKNOWN"


def dec(lib, **kw):
    a = dict(out=P, lse=None, q=P, k=P, v=P, bt=P, mb=8, cl=P, B=2, Hq=32, Hkv=8, D=128, BS=16, NB=64, mcl=128,
             scale=0.088, parts=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_decode(a["out"], a["lse"], a["q"], a["k"], a["v"], a["bt"], a["mb"], a["cl"], a["B"],
                                   a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"], a["mcl"], a["scale"], a["parts"],
                                   a["ws"], a["wsb"], a["stream"])


def test_decode_argument_errors(lib):
    assert dec(lib, q=None) == NULL
    assert dec(lib, out=None) == NULL
    assert dec(lib, bt=None) == NULL
    assert dec(lib, Hq=30) == INVALID  # not a multiple of Hkv
    assert dec(lib, Hkv=0) == INVALID
    assert dec(lib, B=-1) == INVALID
    assert dec(lib, NB=0) == INVALID
    assert dec(lib, mcl=-5) == INVALID
    assert dec(lib, parts=-1) == INVALID
    assert dec(lib, scale=float("nan")) == INVALID
    assert dec(lib, scale=float("inf")) == INVALID
    assert dec(lib, D=64) == UNSUPPORTED
    assert dec(lib, BS=32) == UNSUPPORTED
    assert dec(lib, Hq=72, Hkv=8) == UNSUPPORTED  # G = 9
    assert "head_dim" in fe.fe_last_error() or dec(lib, D=64) == UNSUPPORTED
    assert dec(lib, D=64) == UNSUPPORTED and "head_dim 128" in fe.fe_last_error()
    # split-K needs a workspace of the queried size
    need = lib.fe_paged_gqa_decode_workspace_size(2, 32, 8, 128, 4096, 8)
    assert need > 0
    assert dec(lib, mcl=4096, mb=256, parts=8) == WORKSPACE
    assert dec(lib, mcl=4096, mb=256, parts=8, ws=P, wsb=need - 1) == WORKSPACE
    assert "workspace" in fe.fe_last_error()


def test_decode_batch_zero_is_noop(lib):
    assert dec(lib, B=0) == OK


def dec_append(lib, **kw):
    a = dict(out=P, lse=None, q=P, kn=P, vn=P, sm=P, k=P, v=P, bt=P, mb=8, cl=P, B=2, Hq=32, Hkv=8, D=128, BS=16,
             NB=64, mcl=128, scale=0.088, parts=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_decode_append(a["out"], a["lse"], a["q"], a["kn"], a["vn"], a["sm"], a["k"], a["v"],
                                          a["bt"], a["mb"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["BS"],
                                          a["NB"], a["mcl"], a["scale"], a["parts"], a["ws"], a["wsb"], a["stream"])


def test_decode_append_argument_errors(lib):
    # the fused call checks everything the decode call does ...
    assert dec_append(lib, q=None) == NULL
    assert dec_append(lib, bt=None) == NULL
    assert dec_append(lib, Hq=30) == INVALID
    assert dec_append(lib, scale=float("nan")) == INVALID
    assert dec_append(lib, D=64) == UNSUPPORTED
    assert dec_append(lib, BS=32) == UNSUPPORTED
    need = lib.fe_paged_gqa_decode_workspace_size(2, 32, 8, 128, 4096, 8)
    assert dec_append(lib, mcl=4096, mb=256, parts=8, ws=P, wsb=need - 1) == WORKSPACE
    # ... and the new rows and their slots
    for name in ("kn", "vn", "sm"):
        assert dec_append(lib, **{name: None}) == NULL
        assert "slot_mapping" in fe.fe_last_error()
    assert dec_append(lib, kn=P + 4) == INVALID
    assert dec_append(lib, vn=P + 8) == INVALID
    assert "16-byte" in fe.fe_last_error()
    assert dec_append(lib, B=0) == OK


def dec_norm_rope(lib, **kw):
    a = dict(out=P, lse=None, q=P, kn=P, vn=P, qw=P, kw=P, cs=P, mp=4096, pos=P, sm=P, k=P, v=P, bt=P, mb=8, cl=P,
             B=2, Hq=32, Hkv=8, D=128, BS=16, NB=64, mcl=128, scale=0.088, eps=1e-6, parts=1, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_decode_norm_rope_append(
        a["out"], a["lse"], a["q"], a["kn"], a["vn"], a["qw"], a["kw"], a["cs"], a["mp"], a["pos"], a["sm"], a["k"],
        a["v"], a["bt"], a["mb"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"], a["mcl"], a["scale"],
        a["eps"], a["parts"], a["ws"], a["wsb"], a["stream"])


def test_decode_norm_rope_append_argument_errors(lib):
    # everything the fused append + decode call checks ...
    assert dec_norm_rope(lib, q=None) == NULL
    assert dec_norm_rope(lib, sm=None) == NULL
    assert dec_norm_rope(lib, Hq=30) == INVALID
    assert dec_norm_rope(lib, D=64) == UNSUPPORTED
    assert dec_norm_rope(lib, kn=P + 4) == INVALID
    need = lib.fe_paged_gqa_decode_workspace_size(2, 32, 8, 128, 4096, 8)
    assert dec_norm_rope(lib, mcl=4096, mb=256, parts=8, ws=P, wsb=need - 1) == WORKSPACE
    # ... and the norm/rotary inputs
    for name in ("qw", "kw", "cs", "pos"):
        assert dec_norm_rope(lib, **{name: None}) == NULL
        assert "positions" in fe.fe_last_error()
    assert dec_norm_rope(lib, mp=0) == INVALID and "max_pos" in fe.fe_last_error()
    assert dec_norm_rope(lib, eps=-1e-6) == INVALID
    assert dec_norm_rope(lib, eps=float("nan")) == INVALID
    assert dec_norm_rope(lib, cs=P + 4) == INVALID
    assert dec_norm_rope(lib, qw=P + 2) == INVALID and "16-byte" in fe.fe_last_error()
    assert dec_norm_rope(lib, B=0, qw=None, kw=None, cs=None, pos=None) == OK


def test_workspace_and_partition_queries(lib):
    ws = lib.fe_paged_gqa_decode_workspace_size
    npart = lib.fe_paged_gqa_decode_num_partitions
    assert ws(2, 32, 8, 128, 4096, 1) == 0
    assert npart(2, 32, 8, 128, 4096, 1) == 1
    assert npart(8, 32, 8, 128, 32768, 8) == 8
    assert npart(8, 32, 8, 128, 32768, 16) == 16
    assert npart(8, 32, 8, 128, 32768, 32) == 32
    # partitions never outnumber KV blocks
    assert npart(1, 16, 8, 128, 40, 100) == 3
    # the automatic choice depends only on the arguments and needs the queried workspace
    p = npart(64, 32, 8, 128, 8192, 0)
    assert p >= 1 and npart(64, 32, 8, 128, 8192, 0) == p
    if p > 1:
        assert ws(64, 32, 8, 128, 8192, 0) >= 64 * 32 * p * (128 + 1) * 4
    assert ws(2, 32, 8, 64, 4096, 1) == ctypes.c_size_t(-1).value
    assert npart(2, 30, 8, 128, 4096, 1) == -1
    assert ws(2, 32, 8, 128, 0, 0) == 0


def app(lib, **kw):
    a = dict(kn=P, vn=P, sm=P, kc=P, vc=P, T=4, NB=64, Hkv=8, D=128, BS=16, stream=None)
    a.update(kw)
    return lib.fe_paged_kv_append(a["kn"], a["vn"], a["sm"], a["kc"], a["vc"], a["T"], a["NB"], a["Hkv"], a["D"],
                                  a["BS"], a["stream"])


def test_append_argument_errors(lib):
    assert app(lib, kn=None) == NULL
    assert app(lib, kc=None) == NULL
    assert app(lib, sm=None) == NULL
    assert app(lib, T=-1) == INVALID
    assert app(lib, NB=0) == INVALID
    assert app(lib, D=256) == UNSUPPORTED
    assert app(lib, BS=8) == UNSUPPORTED
    assert app(lib, T=0, kn=None, vn=None, sm=None) == OK  # nothing to do


def pre(lib, **kw):
    a = dict(out=P, lse=None, q=P, qsl=P, k=P, v=P, bt=P, mb=8, cl=P, B=2, tq=16, mql=8, Hq=32, Hkv=8, D=128, BS=16,
             NB=64, mcl=128, scale=0.088, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_prefill_chunk(a["out"], a["lse"], a["q"], a["qsl"], a["k"], a["v"], a["bt"], a["mb"],
                                          a["cl"], a["B"], a["tq"], a["mql"], a["Hq"], a["Hkv"], a["D"], a["BS"],
                                          a["NB"], a["mcl"], a["scale"], a["stream"])


def pre_ex(lib, key_groups, **kw):
    a = dict(out=P, lse=None, q=P, qsl=P, k=P, v=P, bt=P, mb=8, cl=P, B=2, tq=16, mql=8, Hq=32, Hkv=8, D=128, BS=16,
             NB=64, mcl=128, scale=0.088, split=0, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_prefill_chunk_ex(a["out"], a["lse"], a["q"], a["qsl"], a["k"], a["v"], a["bt"], a["mb"],
                                             a["cl"], a["B"], a["tq"], a["mql"], a["Hq"], a["Hkv"], a["D"], a["BS"],
                                             a["NB"], a["mcl"], a["scale"], key_groups, a["split"], a["stream"])


def test_prefill_ex_key_groups_checks(lib):
    # checked before anything is enqueued; B = 0 makes every valid call a no-op
    for kg in (0, 1, 2, 3):
        assert pre_ex(lib, kg, B=0) == OK
    assert pre_ex(lib, 4, B=0) == INVALID
    assert pre_ex(lib, -1, B=0) == INVALID
    assert pre_ex(lib, 2, B=0, Hq=40, Hkv=8) == UNSUPPORTED  # two groups exist only for Hq/Hkv <= 4
    assert pre_ex(lib, 3, B=0, Hq=40, Hkv=8) == UNSUPPORTED
    assert pre_ex(lib, 3, B=0, Hq=24, Hkv=8) == UNSUPPORTED  # Hq/Hkv = 3 runs groups of 3 waves
    assert pre_ex(lib, 3, B=0, Hq=16, Hkv=8) == OK
    assert pre_ex(lib, 1, B=0, Hq=64, Hkv=8) == OK
    assert pre_ex(lib, 2, B=0, Hq=24, Hkv=8) == OK
    # the other checks are those of fe_paged_gqa_prefill_chunk
    assert pre_ex(lib, 1, qsl=None) == NULL
    assert pre_ex(lib, 2, D=96) == UNSUPPORTED
    assert pre_ex(lib, 5, B=0) == INVALID
    assert "key_groups" in fe.fe_last_error()


def test_prefill_ex_split_weights_checks(lib):
    for kg in (0, 1, 3):
        assert pre_ex(lib, kg, B=0, split=1) == OK
    for bad in (-1, 2, 7):
        assert pre_ex(lib, 0, B=0, split=bad) == INVALID
        assert "split_weights" in fe.fe_last_error()
    assert pre_ex(lib, 1, qsl=None, split=1) == NULL


def test_prefill_argument_errors(lib):
    assert pre(lib, qsl=None) == NULL
    assert pre(lib, q=None) == NULL
    assert pre(lib, Hq=12) == INVALID
    assert pre(lib, tq=-1) == INVALID
    assert pre(lib, mql=-1) == INVALID
    assert pre(lib, scale=float("nan")) == INVALID
    assert pre(lib, D=96) == UNSUPPORTED
    assert pre(lib, B=0) == OK
    assert pre(lib, tq=0) == OK


def test_binding_refuses_host_tensors(lib):
    import torch
    q = torch.zeros(1, 16, 128, dtype=torch.bfloat16)
    kc = torch.zeros(4, 8, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        fe.fe_paged_gqa_decode(torch.empty_like(q), None, q, kc, kc, torch.zeros(1, 4, dtype=torch.int32),
                               torch.ones(1, dtype=torch.int32), 16, 0.088, num_partitions=1)


def mix(lib, **kw):
    a = dict(out=P, lse=None, q=P, qsl=P, k=P, v=P, bt=P, mb=8, cl=P, B=3, nd=2, tq=18, mql=16, Hq=32, Hkv=8, D=128,
             BS=16, NB=64, mcl=128, scale=0.088, parts=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_mixed(a["out"], a["lse"], a["q"], a["qsl"], a["k"], a["v"], a["bt"], a["mb"], a["cl"],
                                  a["B"], a["nd"], a["tq"], a["mql"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"],
                                  a["mcl"], a["scale"], a["parts"], a["ws"], a["wsb"], a["stream"])


def test_mixed_argument_errors(lib):
    assert mix(lib, qsl=None) == NULL
    assert mix(lib, out=None) == NULL
    assert mix(lib, nd=-1) == INVALID
    assert mix(lib, nd=4) == INVALID  # more decode rows than sequences
    assert mix(lib, nd=3, tq=2) == INVALID  # fewer query rows than decode rows
    assert mix(lib, Hq=12) == INVALID
    assert mix(lib, parts=-1) == INVALID
    assert mix(lib, scale=float("inf")) == INVALID
    assert mix(lib, D=64) == UNSUPPORTED
    assert mix(lib, Hq=72) == UNSUPPORTED
    need = lib.fe_paged_gqa_mixed_workspace_size(2, 32, 8, 128, 4096, 4)
    assert need > 0
    assert mix(lib, mcl=4096, mb=256, parts=4) == WORKSPACE
    assert mix(lib, mcl=4096, mb=256, parts=4, ws=P, wsb=need - 1) == WORKSPACE
    assert "workspace" in fe.fe_last_error()
    assert mix(lib, B=0, nd=0) == OK
    assert mix(lib, tq=0, nd=0) == OK


def test_mixed_workspace_plan(lib):
    ws = lib.fe_paged_gqa_mixed_workspace_size
    assert ws(0, 32, 8, 128, 8192, 0) == 0          # no decode rows: nothing to split
    assert ws(4, 32, 8, 128, 1024, 0) == 0          # 64 blocks: one automatic partition
    # 8192 tokens = 512 blocks: automatic ranges of 64 blocks -> 8 partitions;
    # counters + fp32 partials + their LSEs
    need = ws(4, 32, 8, 128, 8192, 0)
    assert need >= 4 * 8 * 4 + 4 * 32 * 8 * (128 + 1) * 4
    # 60 decode rows x 8 KV heads: about 6 items per compute unit -> 3 partitions of 160 blocks
    need60 = ws(60, 32, 8, 128, 7665, 0)
    assert 60 * 32 * 3 * (128 + 1) * 4 <= need60 < 60 * 32 * 4 * (128 + 1) * 4
    assert ws(4, 32, 8, 128, 4096, 1) == 0          # one range of 256 blocks
    assert ws(4, 32, 8, 128, 8192, 1) > 0           # a range holds at most 256 blocks: raised to 2
    assert ws(4, 30, 8, 128, 8192, 0) == ctypes.c_size_t(-1).value


def nr(lib, **kw):
    a = dict(qo=P, q=P, k=P, v=P, qw=P, kw=P, cs=P, mp=64, pos=P, sm=P, kc=P, vc=P, T=4, Hq=32, Hkv=8, D=128, BS=16,
             NB=64, eps=1e-6, stream=None)
    a.update(kw)
    return lib.fe_qk_norm_rope_append(a["qo"], a["q"], a["k"], a["v"], a["qw"], a["kw"], a["cs"], a["mp"], a["pos"],
                                      a["sm"], a["kc"], a["vc"], a["T"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"],
                                      a["eps"], a["stream"])


def test_norm_rope_argument_errors(lib):
    assert nr(lib, cs=None) == NULL
    assert nr(lib, qo=None) == NULL
    assert nr(lib, T=-1) == INVALID
    assert nr(lib, mp=0) == INVALID
    assert nr(lib, eps=-1.0) == INVALID
    assert nr(lib, eps=float("nan")) == INVALID
    assert nr(lib, D=64) == UNSUPPORTED
    assert nr(lib, BS=32) == UNSUPPORTED
    assert nr(lib, cs=P + 4) == INVALID and "aligned" in fe.fe_last_error()
    assert nr(lib, T=0, q=None, k=None, v=None, qo=None) == OK


def test_misaligned_pointers_rejected(lib):
    assert app(lib, kn=P + 2) == INVALID
    assert dec(lib, q=P + 8) == INVALID
    assert pre(lib, out=P + 2) == INVALID
    assert mix(lib, k=P + 4) == INVALID


def smp(lib, **kw):
    a = dict(probs=P, lse=P, am=P, x=P, it=None, B=4, V=1024, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fe_sampler_softmax_argmax(a["probs"], a["lse"], a["am"], a["x"], a["it"], a["B"], a["V"], a["ws"],
                                         a["wsb"], a["stream"])


def test_sampler_argument_errors(lib):
    assert smp(lib, am=None) == NULL
    assert smp(lib, x=None) == NULL
    assert smp(lib, B=-1) == INVALID
    assert smp(lib, V=0) == INVALID
    assert smp(lib, V=1001) == UNSUPPORTED
    assert smp(lib, ws=None) == WORKSPACE
    need = lib.fe_sampler_workspace_size(4, 151936)
    assert need > 0 and smp(lib, V=151936, wsb=need - 1) == WORKSPACE
    assert smp(lib, x=P + 2) == INVALID
    assert smp(lib, B=0, x=None, am=None) == OK
    assert lib.fe_sampler_workspace_size(4, 1001) == ctypes.c_size_t(-1).value


def smp_ex(lib, form, **kw):
    a = dict(probs=P, lse=P, am=P, x=P, it=None, B=4, V=1024, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fe_sampler_softmax_argmax_ex(a["probs"], a["lse"], a["am"], a["x"], a["it"], a["B"], a["V"], form,
                                            a["ws"], a["wsb"], a["stream"])


def test_sampler_form_argument_errors(lib):
    """form must be 0, 1 or 2; the one-workgroup-per-row form holds rows of
    at most 1024 threads x 20 units x 8 logits; every form needs the
    workspace the size query gives."""
    assert smp_ex(lib, 3) == INVALID and "form" in fe.fe_last_error()
    assert smp_ex(lib, -1) == INVALID
    assert smp_ex(lib, 2, V=163840 + 8) == UNSUPPORTED and "163,840" in fe.fe_last_error()
    assert smp_ex(lib, 2, ws=None) == WORKSPACE
    assert smp_ex(lib, 0, B=256, V=151936, ws=None) == WORKSPACE
    assert smp_ex(lib, 2, B=0, x=None, am=None) == OK
    assert smp_ex(lib, 1, V=1001) == UNSUPPORTED


def test_sampler_automatic_form():
    """One workgroup per row (form 2) once every round of 256 workgroups holds
    at least 160 rows and the row fits 1024 threads x 20 units; ranges (form
    1) otherwise."""
    V = 151936
    assert [fe.fe_sampler_form(B, V) for B in (1, 64, 128, 159)] == [1, 1, 1, 1]
    assert [fe.fe_sampler_form(B, V) for B in (160, 192, 256, 512, 1024, 416)] == [2, 2, 2, 2, 2, 2]
    assert [fe.fe_sampler_form(B, V) for B in (300, 384, 512 + 159)] == [1, 1, 1]
    assert fe.fe_sampler_form(256, 163840) == 2 and fe.fe_sampler_form(256, 163848) == 1
    assert fe.fe_sampler_form(0, V) == 1
    with pytest.raises(ValueError):
        fe.fe_sampler_form(4, 1001)


def test_oversized_launches_rejected(lib):
    """Sizes whose launch would reach 2^32 work-items are refused on the host."""
    assert app(lib, T=1 << 30, NB=1 << 20) == UNSUPPORTED
    assert pre(lib, mql=1 << 30, B=1 << 10, tq=1 << 30) == UNSUPPORTED
    assert nr(lib, T=1 << 28) == UNSUPPORTED
    assert "2^32" in fe.fe_last_error()


# -- host-side shape checks of the Python binding: a mis-shaped tensor is
# rejected before any pointer reaches the library (CPU tensors suffice, since
# the shape check comes before the device check) ------------------------------

def _bf(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _i32(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.int32)


def _f32(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.float32)


def _decode_args(B=2, Hq=8, Hkv=2, NB=16, mb=4):
    return dict(out=_bf(B, Hq, 128), lse=_f32(B, Hq), q=_bf(B, Hq, 128), k_cache=_bf(NB, Hkv, 16, 128),
                v_cache=_bf(NB, Hkv, 16, 128), block_tables=_i32(B, mb), context_lens=_i32(B))


@pytest.mark.parametrize("bad, pattern", [
    (dict(out=_bf(2, 8, 64)), "out"),
    (dict(out=_bf(3, 8, 128)), "out"),
    (dict(lse=_f32(2, 4)), "lse"),
    (dict(context_lens=_i32(3)), "context_lens"),
    (dict(block_tables=_i32(1, 4)), "block_tables"),
    (dict(block_tables=_i32(8)), "block_tables"),
    (dict(v_cache=_bf(8, 2, 16, 128)), "v_cache"),
    (dict(k_cache=_bf(16, 2, 16, 64), v_cache=_bf(16, 2, 16, 64)), "head_dim"),
])
def test_binding_rejects_misshaped_decode(lib, bad, pattern):
    a = _decode_args()
    a.update(bad)
    with pytest.raises(ValueError, match=pattern):
        fe.fe_paged_gqa_decode(a["out"], a["lse"], a["q"], a["k_cache"], a["v_cache"], a["block_tables"],
                               a["context_lens"], 64, 0.088, num_partitions=1)


@pytest.mark.parametrize("bad, pattern", [
    (dict(out=_bf(2, 4, 128)), "out"),
    (dict(context_lens=_i32(1)), "context_lens"),
    (dict(v_cache=_bf(16, 1, 16, 128)), "v_cache"),
    (dict(k_new=_bf(2, 1, 128)), "k_new"),
    (dict(v_new=_bf(3, 2, 128)), "v_new"),
    (dict(slot_mapping=_i32(5)), "slot_mapping"),
])
def test_binding_rejects_misshaped_decode_append(lib, bad, pattern):
    a = _decode_args()
    a.update(k_new=_bf(2, 2, 128), v_new=_bf(2, 2, 128), slot_mapping=_i32(2))
    a.update(bad)
    with pytest.raises(ValueError, match=pattern):
        fe.fe_paged_gqa_decode_append(a["out"], a["lse"], a["q"], a["k_new"], a["v_new"], a["slot_mapping"],
                                      a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 64, 0.088,
                                      num_partitions=1)


def _packed_args(B=2, tq=10, Hq=8, Hkv=2, NB=16, mb=4):
    return dict(out=_bf(tq, Hq, 128), lse=_f32(tq, Hq), q=_bf(tq, Hq, 128), qsl=_i32(B + 1),
                k_cache=_bf(NB, Hkv, 16, 128), v_cache=_bf(NB, Hkv, 16, 128), block_tables=_i32(B, mb),
                context_lens=_i32(B))


@pytest.mark.parametrize("bad, pattern", [
    (dict(out=_bf(9, 8, 128)), "out"),
    (dict(lse=_f32(10, 2)), "lse"),
    (dict(qsl=_i32(2)), "query_start_loc"),
    (dict(block_tables=_i32(3, 4)), "block_tables"),
    (dict(v_cache=_bf(16, 2, 8, 128)), "v_cache"),
])
@pytest.mark.parametrize("call", ["prefill", "prefill_ex", "mixed"])
def test_binding_rejects_misshaped_packed(lib, bad, pattern, call):
    a = _packed_args()
    a.update(bad)
    args = (a["out"], a["lse"], a["q"], a["qsl"], a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"])
    with pytest.raises(ValueError, match=pattern):
        if call == "prefill":
            fe.fe_paged_gqa_prefill_chunk(*args, 8, 64, 0.088)
        elif call == "prefill_ex":
            fe.fe_paged_gqa_prefill_chunk_ex(*args, 8, 64, 0.088, 1)
        else:
            fe.fe_paged_gqa_mixed(*args, 1, 8, 64, 0.088, num_partitions=1, workspace=torch_uint8(16))


def torch_uint8(n):
    import torch
    return torch.zeros(n, dtype=torch.uint8)


@pytest.mark.parametrize("bad, pattern", [
    (dict(probs=_f32(4, 1000)), "probs"),
    (dict(lse=_f32(3)), "lse"),
    (dict(argmax=_i32(5)), "argmax"),
    (dict(inv_temperature=_f32(2)), "inv_temperature"),
])
def test_binding_rejects_misshaped_sampler(lib, bad, pattern):
    a = dict(probs=_f32(4, 1024), lse=_f32(4), argmax=_i32(4), logits=_bf(4, 1024), inv_temperature=_f32(4))
    a.update(bad)
    with pytest.raises(ValueError, match=pattern):
        fe.fe_sampler_softmax_argmax(a["probs"], a["lse"], a["argmax"], a["logits"], a["inv_temperature"],
                                     workspace=torch_uint8(1 << 16))


@pytest.mark.parametrize("bad, pattern", [
    (dict(q_out=_bf(2, 8, 128)), "q_out"),
    (dict(positions=_i32(2)), "positions"),
    (dict(slot_mapping=_i32(4)), "slot_mapping"),
    (dict(q_norm_w=_bf(64)), "q_norm_w"),
    (dict(cos_sin=_f32(32, 64)), "cos_sin"),
    (dict(v_cache=_bf(8, 2, 16, 128)), "v_cache"),
])
def test_binding_rejects_misshaped_norm_rope(lib, bad, pattern):
    a = dict(q_out=_bf(3, 8, 128), q=_bf(3, 8, 128), k=_bf(3, 2, 128), v=_bf(3, 2, 128), q_norm_w=_bf(128),
             k_norm_w=_bf(128), cos_sin=_f32(32, 128), positions=_i32(3), slot_mapping=_i32(3),
             k_cache=_bf(16, 2, 16, 128), v_cache=_bf(16, 2, 16, 128))
    a.update(bad)
    with pytest.raises(ValueError, match=pattern):
        fe.fe_qk_norm_rope_append(a["q_out"], a["q"], a["k"], a["v"], a["q_norm_w"], a["k_norm_w"], a["cos_sin"],
                                  a["positions"], a["slot_mapping"], a["k_cache"], a["v_cache"], 1e-6)


def test_binding_rejects_misshaped_append(lib):
    with pytest.raises(ValueError, match="k_new"):
        fe.fe_paged_kv_append(_bf(3, 1, 128), _bf(3, 2, 128), _i32(3), _bf(16, 2, 16, 128), _bf(16, 2, 16, 128))
    with pytest.raises(ValueError, match="v_cache"):
        fe.fe_paged_kv_append(_bf(3, 2, 128), _bf(3, 2, 128), _i32(3), _bf(16, 2, 16, 128), _bf(16, 4, 16, 128))
    with pytest.raises(ValueError, match="slot_mapping"):
        fe.fe_paged_kv_append(_bf(3, 2, 128), _bf(3, 2, 128), _i32(3, 1), _bf(16, 2, 16, 128), _bf(16, 2, 16, 128))


def test_decode_append_slot_precondition_check():
    """check_decode_append_slots (the validate=True path of
    fe_paged_gqa_decode_append) accepts the slot of each sequence's last
    position, padding, out-of-pool slots and empty sequences, and names the
    first sequence whose in-pool slot is anywhere else."""
    import numpy as np
    bt = np.array([[5, 2, 9], [7, 1, 0], [3, 4, 6]], np.int32)
    lens = np.array([20, 16, 0], np.int32)  # positions 19 (block 2, row 3) and 15 (block 7, row 15)
    good = np.array([2 * 16 + 3, 7 * 16 + 15, 123], np.int32)
    binding.check_decode_append_slots(good, bt, lens, 10, 16, 48)
    binding.check_decode_append_slots(np.array([-1, 7 * 16 + 15, 0], np.int32), bt, lens, 10, 16, 48)
    binding.check_decode_append_slots(np.array([10 * 16, -5, 0], np.int32), bt, lens, 10, 16, 48)  # past the pool
    with pytest.raises(ValueError, match=r"slot_mapping\[0\]"):
        binding.check_decode_append_slots(np.array([2 * 16 + 2, 7 * 16 + 15, 0], np.int32), bt, lens, 10, 16, 48)
    with pytest.raises(ValueError, match=r"slot_mapping\[1\]"):
        binding.check_decode_append_slots(np.array([2 * 16 + 3, 1 * 16, 0], np.int32), bt, lens, 10, 16, 48)
    # the context is clamped as the kernel clamps it: max_context_len 16 puts
    # sequence 0's last position at 15 (block 5, row 15)
    binding.check_decode_append_slots(np.array([5 * 16 + 15, 7 * 16 + 15, 0], np.int32), bt, lens, 10, 16, 16)


def dec_noalloc(lib, **kw):
    a = dict(out=P, lse=None, q=P, k=P, v=P, bt=P, mb=8, cl=P, B=2, Hq=32, Hkv=8, D=128, BS=16, NB=64, mcl=128,
             scale=0.088, parts=1, stream=None)
    a.update(kw)
    return lib.fe_paged_gqa_decode_noalloc(a["out"], a["lse"], a["q"], a["k"], a["v"], a["bt"], a["mb"], a["cl"],
                                           a["B"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"], a["mcl"], a["scale"],
                                           a["parts"], a["stream"])


def test_decode_noalloc_argument_errors(lib):
    """The allocation-free decode checks what fe_paged_gqa_decode checks and
    refuses, before anything is enqueued, sizes whose split-K partials do not
    fit its 32 MiB of device scratch."""
    assert dec_noalloc(lib, q=None) == NULL
    assert dec_noalloc(lib, Hq=30) == INVALID
    assert dec_noalloc(lib, scale=float("nan")) == INVALID
    assert dec_noalloc(lib, D=64) == UNSUPPORTED
    assert dec_noalloc(lib, q=P + 8) == INVALID
    assert dec_noalloc(lib, B=0) == OK
    ws = lib.fe_paged_gqa_decode_workspace_size
    # 1024 sequences x 32 heads x 8 partitions of fp32 partials: 128 MiB
    assert ws(1024, 32, 8, 128, 8192, 8) > (32 << 20)
    assert dec_noalloc(lib, B=1024, mcl=8192, mb=512, parts=8) == WORKSPACE
    assert "32" in fe.fe_last_error() and "scratch" in fe.fe_last_error()
    # the gate-sized call fits (64 x 32 heads x 8 partitions: ~8.5 MB)
    assert ws(64, 32, 8, 128, 8192, 0) <= (32 << 20)


def test_mfma_rate_probe_argument_errors(lib):
    f = lib.fe_mfma_rate_probe
    assert f(P, 16, 0, 4, P, None) == OK  # nothing to launch
    assert f(None, 16, 2, 4, P, None) == NULL
    assert f(P, 16, 2, 4, None, None) == NULL
    assert f(P, 0, 2, 4, P, None) == INVALID
    assert f(P, 16, -1, 4, P, None) == INVALID
    assert f(P, 16, 2, -1, P, None) == INVALID
    assert f(P + 4, 16, 2, 4, P, None) == INVALID
    assert f(P, 16, 1 << 23, 4, P, None) == UNSUPPORTED


def test_hbm_read_probe_argument_errors(lib):
    f = lib.fe_hbm_read_probe
    assert f(P, 16, P, 0, P, None) == OK  # nothing to read
    assert f(None, 16, P, 4, P, None) == NULL
    assert f(P, 16, None, 4, P, None) == NULL
    assert f(P, 16, P, 4, None, None) == NULL
    assert f(P, 0, P, 4, P, None) == INVALID
    assert f(P, 16, P, -1, P, None) == INVALID
    assert f(P + 4, 16, P, 4, P, None) == INVALID
