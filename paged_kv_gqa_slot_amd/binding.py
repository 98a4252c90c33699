"""ctypes binding of libfe.so -- argument marshalling only.

Each function has the name of the C entry point it calls (declared in
``include/fe.h``), takes torch tensors, checks dtype/device/contiguity,
passes ``data_ptr()`` and the current HIP stream, and raises
:class:`FeError` on a non-zero status.  All arithmetic happens in the HIP
kernels; if the library is not built this module raises instead of computing
anything itself.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfe.so"
_lib = None


class FeError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed: {fe_status_string(status)} ({status}): {detail}")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libfe.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fe_paged_kv_append.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
    lib.fe_paged_kv_append.restype = I
    lib.fe_paged_gqa_decode_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.fe_paged_gqa_decode_workspace_size.restype = Z
    lib.fe_paged_gqa_decode_num_partitions.argtypes = [I, I, I, I, I, I]
    lib.fe_paged_gqa_decode_num_partitions.restype = I
    lib.fe_paged_gqa_decode.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fe_paged_gqa_decode.restype = I
    lib.fe_paged_gqa_decode_noalloc.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P]
    lib.fe_paged_gqa_decode_noalloc.restype = I
    lib.fe_paged_gqa_decode_append.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fe_paged_gqa_decode_append.restype = I
    lib.fe_paged_gqa_decode_norm_rope_append.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, P, P, I, P, I, I, I, I,
                                                         I, I, I, F, F, I, P, Z, P]
    lib.fe_paged_gqa_decode_norm_rope_append.restype = I
    lib.fe_paged_gqa_prefill_chunk.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, F, P]
    lib.fe_paged_gqa_prefill_chunk.restype = I
    lib.fe_paged_gqa_prefill_chunk_ex.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, F, I, I, P]
    lib.fe_paged_gqa_prefill_chunk_ex.restype = I
    lib.fe_paged_gqa_mixed_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.fe_paged_gqa_mixed_workspace_size.restype = Z
    lib.fe_paged_gqa_mixed.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, I, F, I, P, Z, P]
    lib.fe_paged_gqa_mixed.restype = I
    lib.fe_qk_norm_rope_append.argtypes = [P, P, P, P, P, P, P, I, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.fe_qk_norm_rope_append.restype = I
    H = ctypes.c_void_p  # fe_kv_allocator*
    lib.fe_kv_allocator_create.argtypes = [I, I, I, I]
    lib.fe_kv_allocator_create.restype = H
    lib.fe_kv_allocator_destroy.argtypes = [H]
    lib.fe_kv_allocator_destroy.restype = None
    lib.fe_kv_allocator_append.argtypes = [H, I, I, P]
    lib.fe_kv_allocator_append.restype = I
    lib.fe_kv_allocator_release.argtypes = [H, I]
    lib.fe_kv_allocator_release.restype = I
    for name in ("fe_kv_allocator_num_free", "fe_kv_allocator_num_allocated"):
        getattr(lib, name).argtypes = [H]
        getattr(lib, name).restype = I
    lib.fe_kv_allocator_seq_len.argtypes = [H, I]
    lib.fe_kv_allocator_seq_len.restype = I
    lib.fe_kv_allocator_batch.argtypes = [H, P, I, P, I, ctypes.c_int32, P]
    lib.fe_kv_allocator_batch.restype = I
    lib.fe_sampler_workspace_size.argtypes = [I, I]
    lib.fe_sampler_workspace_size.restype = Z
    lib.fe_sampler_softmax_argmax.argtypes = [P, P, P, P, P, I, I, P, Z, P]
    lib.fe_sampler_softmax_argmax.restype = I
    lib.fe_sampler_softmax_argmax_ex.argtypes = [P, P, P, P, P, I, I, I, P, Z, P]
    lib.fe_sampler_softmax_argmax_ex.restype = I
    lib.fe_sampler_form.argtypes = [I, I]
    lib.fe_sampler_form.restype = I
    lib.fe_hbm_read_probe.argtypes = [P, ctypes.c_int64, P, I, P, P]
    lib.fe_hbm_read_probe.restype = I
    lib.fe_mfma_rate_probe.argtypes = [P, I, I, I, P, P]
    lib.fe_mfma_rate_probe.restype = I
    lib.fe_status_string.argtypes = [I]
    lib.fe_status_string.restype = ctypes.c_char_p
    lib.fe_last_error.argtypes = []
    lib.fe_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fe_status_string(status: int) -> str:
    return load_library().fe_status_string(int(status)).decode()


def fe_last_error() -> str:
    return load_library().fe_last_error().decode()


def _check(rc: int, func: str):
    if rc != 0:
        raise FeError(rc, func, fe_last_error())


# torch's raw current-stream query (a plain int, no Stream object): about
# 0.1 us against ~2.7 us for torch.cuda.current_stream() per call
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> Optional[int]:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: Optional[torch.Tensor], dtype, name: str, ndim: Optional[int] = None):
    """Device pointer of t after checking dtype, device, contiguity and rank
    (one combined test on the common path; the error names the failure)."""
    if t is None:
        return None
    if t.dtype is not dtype or not t.is_cuda or not t.is_contiguous() or (ndim is not None and t.dim() != ndim):
        if t.dtype != dtype:
            raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name}: expected a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous tensor")
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], name: str, *dims):
    """Raise ValueError unless t (if given) has exactly len(dims) dimensions
    whose sizes equal dims (None matches any size).  Runs before any pointer
    is passed on, so a mis-shaped tensor never reaches a kernel."""
    if t is None:
        return
    shape = t.shape
    if len(shape) == len(dims):
        for s, d in zip(shape, dims):
            if d is not None and s != d:
                break
        else:
            return
    want = "[" + "][".join("*" if d is None else str(d) for d in dims) + "]"
    raise ValueError(f"{name}: expected shape {want}, got {list(shape)}")


def _pools(k_cache, v_cache):
    """(NB, Hkv, BS, D) of the K/V pools; both must be [NB][Hkv][BS][D] alike."""
    _shape(k_cache, "k_cache", None, None, None, None)
    _shape(v_cache, "v_cache", *k_cache.shape)
    return tuple(k_cache.shape)


def fe_paged_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Scatter k_new/v_new [T][Hkv][D] into the pools [NB][Hkv][BS][D] by slot."""
    NB, Hkv, BS, D = _pools(k_cache, v_cache)
    _shape(slot_mapping, "slot_mapping", None)
    T = slot_mapping.shape[0]
    if T:
        _shape(k_new, "k_new", T, Hkv, D)
        _shape(v_new, "v_new", T, Hkv, D)
    rc = load_library().fe_paged_kv_append(
        _dev(k_new, torch.bfloat16, "k_new"), _dev(v_new, torch.bfloat16, "v_new"),
        _dev(slot_mapping, torch.int32, "slot_mapping", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), T, NB, Hkv, D, BS, _stream(stream))
    _check(rc, "fe_paged_kv_append")


@functools.lru_cache(maxsize=256)
def fe_paged_gqa_decode_workspace_size(B, Hq, Hkv, D, max_context_len, num_partitions=0) -> int:
    n = load_library().fe_paged_gqa_decode_workspace_size(B, Hq, Hkv, D, max_context_len, num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("fe_paged_gqa_decode_workspace_size: invalid sizes")
    return int(n)


@functools.lru_cache(maxsize=256)
def fe_paged_gqa_decode_num_partitions(B, Hq, Hkv, D, max_context_len, num_partitions=0) -> int:
    n = load_library().fe_paged_gqa_decode_num_partitions(B, Hq, Hkv, D, max_context_len, num_partitions)
    if n < 0:
        raise ValueError("fe_paged_gqa_decode_num_partitions: invalid sizes")
    return int(n)


def _decode_shapes(out, lse, q, k_cache, block_tables, context_lens):
    B, Hq, D = q.shape
    _shape(out, "out", B, Hq, D)
    _shape(lse, "lse", B, Hq)
    _shape(block_tables, "block_tables", B, None)
    _shape(context_lens, "context_lens", B)
    if k_cache.shape[3] != D:
        raise ValueError(f"q's head_dim {D} differs from the pools' {k_cache.shape[3]}")


def fe_paged_gqa_decode(out, lse, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                        scale: float, num_partitions: int = 0, workspace=None, stream=None) -> None:
    """Decode attention.  ``workspace`` is a uint8 device tensor of at least
    fe_paged_gqa_decode_workspace_size() bytes; one is allocated when not given."""
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _decode_shapes(out, lse, q, k_cache, block_tables, context_lens)
    ws_bytes = fe_paged_gqa_decode_workspace_size(B, Hq, Hkv, D, max_context_len, num_partitions)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_have = workspace.numel() if workspace is not None else 0
    rc = load_library().fe_paged_gqa_decode(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(k_cache, torch.bfloat16, "k_cache", 4), _dev(v_cache, torch.bfloat16, "v_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), B, Hq, Hkv, D, BS, NB, int(max_context_len),
        float(scale), int(num_partitions), ws_ptr, ws_have, _stream(stream))
    _check(rc, "fe_paged_gqa_decode")


def fe_paged_gqa_decode_noalloc(out, lse, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                                scale: float, num_partitions: int = 0, stream=None) -> None:
    """fe_paged_gqa_decode with no workspace and no allocation: the split-K
    partials live in the library's per-GPU device scratch (32 MiB).  Calls
    that may overlap in time on one GPU race on that scratch."""
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _decode_shapes(out, lse, q, k_cache, block_tables, context_lens)
    rc = load_library().fe_paged_gqa_decode_noalloc(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(k_cache, torch.bfloat16, "k_cache", 4), _dev(v_cache, torch.bfloat16, "v_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), B, Hq, Hkv, D, BS, NB, int(max_context_len),
        float(scale), int(num_partitions), _stream(stream))
    _check(rc, "fe_paged_gqa_decode_noalloc")


def check_decode_append_slots(slot_mapping, block_tables, context_lens, num_blocks: int, block_size: int,
                              max_context_len: int) -> None:
    """Host-side check of fe_paged_gqa_decode_append's precondition: for
    every sequence b with L = min(context_lens[b], max_context_len,
    block_tables row length * block_size) > 0 whose slot lies in the pool,
    slot_mapping[b] == block_tables[b][(L-1) // BS] * BS + (L-1) % BS.
    Raises ValueError naming the first offending sequence.  Takes torch
    tensors (device or host) or arrays; device ones are copied to the host."""
    sm = np.asarray(slot_mapping.cpu() if hasattr(slot_mapping, "cpu") else slot_mapping, dtype=np.int64)
    bt = np.asarray(block_tables.cpu() if hasattr(block_tables, "cpu") else block_tables, dtype=np.int64)
    cl = np.asarray(context_lens.cpu() if hasattr(context_lens, "cpu") else context_lens, dtype=np.int64)
    cap = min(int(max_context_len), bt.shape[1] * block_size)
    for b in range(sm.shape[0]):
        L = min(max(int(cl[b]), 0), cap)
        s = int(sm[b])
        if L == 0 or s < 0 or s >= num_blocks * block_size:
            continue
        want = int(bt[b, (L - 1) // block_size]) * block_size + (L - 1) % block_size
        if s != want:
            raise ValueError(f"slot_mapping[{b}] = {s} is not the slot of position {L - 1} "
                             f"(block_tables gives {want})")


def fe_paged_gqa_decode_append(out, lse, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                               max_context_len: int, scale: float, num_partitions: int = 0, workspace=None,
                               stream=None, validate: bool = False) -> None:
    """Append of one new K/V row per sequence (into slot_mapping[b], the
    slot of position context_lens[b] - 1) fused into decode attention.
    Same workspace as fe_paged_gqa_decode; one is allocated when not given.

    validate=True first checks the call's precondition on host copies (a
    device synchronisation): every in-pool slot_mapping[b] must be the slot
    of position context_lens[b] - 1 in row b of block_tables."""
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _decode_shapes(out, lse, q, k_cache, block_tables, context_lens)
    _shape(k_new, "k_new", B, Hkv, D)
    _shape(v_new, "v_new", B, Hkv, D)
    _shape(slot_mapping, "slot_mapping", B)
    if validate:
        check_decode_append_slots(slot_mapping, block_tables, context_lens, NB, BS, max_context_len)
    ws_bytes = fe_paged_gqa_decode_workspace_size(B, Hq, Hkv, D, max_context_len, num_partitions)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_have = workspace.numel() if workspace is not None else 0
    rc = load_library().fe_paged_gqa_decode_append(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(k_new, torch.bfloat16, "k_new", 3), _dev(v_new, torch.bfloat16, "v_new", 3),
        _dev(slot_mapping, torch.int32, "slot_mapping", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens", 1), B, Hq, Hkv, D, BS, NB,
        int(max_context_len), float(scale), int(num_partitions), ws_ptr, ws_have, _stream(stream))
    _check(rc, "fe_paged_gqa_decode_append")


def fe_paged_gqa_decode_norm_rope_append(out, lse, q, k_new, v_new, q_norm_w, k_norm_w, cos_sin, positions,
                                         slot_mapping, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len: int, scale: float, eps: float, num_partitions: int = 0,
                                         workspace=None, stream=None, validate: bool = False) -> None:
    """Per-head RMSNorm + rotary embedding of q and of the new k rows, the
    append of the new K/V rows and decode, in one launch: the same result as
    fe_qk_norm_rope_append followed by fe_paged_gqa_decode on its q_out.
    Same workspace as fe_paged_gqa_decode; one is allocated when not given.
    validate=True checks slot_mapping on host copies as
    fe_paged_gqa_decode_append does."""
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _decode_shapes(out, lse, q, k_cache, block_tables, context_lens)
    _shape(k_new, "k_new", B, Hkv, D)
    _shape(v_new, "v_new", B, Hkv, D)
    _shape(slot_mapping, "slot_mapping", B)
    _shape(positions, "positions", B)
    _shape(cos_sin, "cos_sin", None, D)
    _shape(q_norm_w, "q_norm_w", D)
    _shape(k_norm_w, "k_norm_w", D)
    if validate:
        check_decode_append_slots(slot_mapping, block_tables, context_lens, NB, BS, max_context_len)
    ws_bytes = fe_paged_gqa_decode_workspace_size(B, Hq, Hkv, D, max_context_len, num_partitions)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_have = workspace.numel() if workspace is not None else 0
    rc = load_library().fe_paged_gqa_decode_norm_rope_append(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(k_new, torch.bfloat16, "k_new", 3), _dev(v_new, torch.bfloat16, "v_new", 3),
        _dev(q_norm_w, torch.bfloat16, "q_norm_w", 1), _dev(k_norm_w, torch.bfloat16, "k_norm_w", 1),
        _dev(cos_sin, torch.float32, "cos_sin", 2), cos_sin.shape[0], _dev(positions, torch.int32, "positions", 1),
        _dev(slot_mapping, torch.int32, "slot_mapping", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens", 1), B, Hq, Hkv, D, BS, NB,
        int(max_context_len), float(scale), float(eps), int(num_partitions), ws_ptr, ws_have, _stream(stream))
    _check(rc, "fe_paged_gqa_decode_norm_rope_append")


def _packed_shapes(out, lse, q, query_start_loc, k_cache, block_tables, B):
    total_q, Hq, D = q.shape
    _shape(out, "out", total_q, Hq, D)
    _shape(lse, "lse", total_q, Hq)
    _shape(query_start_loc, "query_start_loc", B + 1)
    _shape(block_tables, "block_tables", B, None)
    if k_cache.shape[3] != D:
        raise ValueError(f"q's head_dim {D} differs from the pools' {k_cache.shape[3]}")


def fe_paged_gqa_prefill_chunk(out, lse, q, query_start_loc, k_cache, v_cache, block_tables, context_lens,
                               max_q_len: int, max_context_len: int, scale: float, stream=None) -> None:
    """Chunked prefill attention over the paged cache (bottom-right causal)."""
    _shape(q, "q", None, None, None)
    total_q, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _shape(context_lens, "context_lens", None)
    B = context_lens.shape[0]
    _packed_shapes(out, lse, q, query_start_loc, k_cache, block_tables, B)
    rc = load_library().fe_paged_gqa_prefill_chunk(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(query_start_loc, torch.int32, "query_start_loc", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens", 1), B, total_q, int(max_q_len),
        Hq, Hkv, D, BS, NB, int(max_context_len), float(scale), _stream(stream))
    _check(rc, "fe_paged_gqa_prefill_chunk")


def fe_paged_gqa_prefill_chunk_ex(out, lse, q, query_start_loc, k_cache, v_cache, block_tables, context_lens,
                                  max_q_len: int, max_context_len: int, scale: float, key_groups: int,
                                  split_weights: int = 0, stream=None) -> None:
    """fe_paged_gqa_prefill_chunk with the tile shape chosen by the caller
    (key_groups 0 automatic, 1 or 2 wave groups over the keys, 3 two query
    tiles over one K/V stream) and the precision of the softmax weights in
    the PV product (split_weights 0: rounded to bf16; 1: a bf16 value and
    its bf16 remainder)."""
    _shape(q, "q", None, None, None)
    total_q, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _shape(context_lens, "context_lens", None)
    B = context_lens.shape[0]
    _packed_shapes(out, lse, q, query_start_loc, k_cache, block_tables, B)
    rc = load_library().fe_paged_gqa_prefill_chunk_ex(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(query_start_loc, torch.int32, "query_start_loc", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens", 1), B, total_q, int(max_q_len),
        Hq, Hkv, D, BS, NB, int(max_context_len), float(scale), int(key_groups), int(split_weights),
        _stream(stream))
    _check(rc, "fe_paged_gqa_prefill_chunk_ex")


@functools.lru_cache(maxsize=256)
def fe_paged_gqa_mixed_workspace_size(num_decode, Hq, Hkv, D, max_context_len, num_partitions=0) -> int:
    n = load_library().fe_paged_gqa_mixed_workspace_size(num_decode, Hq, Hkv, D, max_context_len, num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("fe_paged_gqa_mixed_workspace_size: invalid sizes")
    return int(n)


def fe_paged_gqa_mixed(out, lse, q, query_start_loc, k_cache, v_cache, block_tables, context_lens, num_decode: int,
                       max_q_len: int, max_context_len: int, scale: float, num_partitions: int = 0, workspace=None,
                       stream=None) -> None:
    """Decode rows (sequences [0, num_decode), one query row each) and prefill
    chunks (the rest) in one launch.  ``workspace``: uint8 device tensor of at
    least fe_paged_gqa_mixed_workspace_size() bytes, zero-filled before its
    first use; one is allocated (zeroed) when not given."""
    _shape(q, "q", None, None, None)
    total_q, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _shape(context_lens, "context_lens", None)
    B = context_lens.shape[0]
    _packed_shapes(out, lse, q, query_start_loc, k_cache, block_tables, B)
    ws_bytes = fe_paged_gqa_mixed_workspace_size(num_decode, Hq, Hkv, D, max_context_len, num_partitions)
    if workspace is None and ws_bytes:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
    ws_have = workspace.numel() if workspace is not None else 0
    rc = load_library().fe_paged_gqa_mixed(
        _dev(out, torch.bfloat16, "out", 3), _dev(lse, torch.float32, "lse", 2), _dev(q, torch.bfloat16, "q", 3),
        _dev(query_start_loc, torch.int32, "query_start_loc", 1), _dev(k_cache, torch.bfloat16, "k_cache", 4),
        _dev(v_cache, torch.bfloat16, "v_cache", 4), _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], _dev(context_lens, torch.int32, "context_lens", 1), B, int(num_decode), total_q,
        int(max_q_len), Hq, Hkv, D, BS, NB, int(max_context_len), float(scale), int(num_partitions), ws_ptr, ws_have,
        _stream(stream))
    _check(rc, "fe_paged_gqa_mixed")


def fe_qk_norm_rope_append(q_out, q, k, v, q_norm_w, k_norm_w, cos_sin, positions, slot_mapping, k_cache, v_cache,
                           eps: float, stream=None) -> None:
    """Per-head RMSNorm + rotary embedding of q and k, then append of k and v
    into the pools; q_out may be q (in place)."""
    _shape(q, "q", None, None, None)
    T, Hq, D = q.shape
    NB, Hkv, BS, _ = _pools(k_cache, v_cache)
    _shape(q_out, "q_out", T, Hq, D)
    _shape(k, "k", T, Hkv, D)
    _shape(v, "v", T, Hkv, D)
    _shape(cos_sin, "cos_sin", None, D)
    _shape(q_norm_w, "q_norm_w", D)
    _shape(k_norm_w, "k_norm_w", D)
    _shape(positions, "positions", T)
    _shape(slot_mapping, "slot_mapping", T)
    rc = load_library().fe_qk_norm_rope_append(
        _dev(q_out, torch.bfloat16, "q_out", 3), _dev(q, torch.bfloat16, "q", 3), _dev(k, torch.bfloat16, "k", 3),
        _dev(v, torch.bfloat16, "v", 3), _dev(q_norm_w, torch.bfloat16, "q_norm_w", 1),
        _dev(k_norm_w, torch.bfloat16, "k_norm_w", 1), _dev(cos_sin, torch.float32, "cos_sin", 2), cos_sin.shape[0],
        _dev(positions, torch.int32, "positions", 1), _dev(slot_mapping, torch.int32, "slot_mapping", 1),
        _dev(k_cache, torch.bfloat16, "k_cache", 4), _dev(v_cache, torch.bfloat16, "v_cache", 4), T, Hq, Hkv, D, BS,
        NB, float(eps), _stream(stream))
    _check(rc, "fe_qk_norm_rope_append")


@functools.lru_cache(maxsize=256)
def fe_sampler_workspace_size(B: int, V: int) -> int:
    n = load_library().fe_sampler_workspace_size(int(B), int(V))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("fe_sampler_workspace_size: invalid sizes")
    return int(n)


@functools.lru_cache(maxsize=256)
def fe_sampler_form(B: int, V: int) -> int:
    """The sampler form the automatic choice runs: 1 ranges, 2 one workgroup per row."""
    f = load_library().fe_sampler_form(int(B), int(V))
    if f < 0:
        raise ValueError("fe_sampler_form: invalid sizes")
    return int(f)


def fe_sampler_softmax_argmax(probs, lse, argmax, logits, inv_temperature=None, workspace=None, stream=None) -> None:
    """fp32 softmax (probs may be None), LSE (may be None) and greedy argmax of bf16 logits [B][V]."""
    fe_sampler_softmax_argmax_ex(probs, lse, argmax, logits, inv_temperature, 0, workspace, stream)


def fe_sampler_softmax_argmax_ex(probs, lse, argmax, logits, inv_temperature=None, form: int = 0, workspace=None,
                                 stream=None) -> None:
    """fe_sampler_softmax_argmax with the kernel form chosen: 0 automatic, 1
    ranges (two launches), 2 one workgroup per row (one launch)."""
    _shape(logits, "logits", None, None)
    B, V = logits.shape
    _shape(probs, "probs", B, V)
    _shape(lse, "lse", B)
    _shape(argmax, "argmax", B)
    _shape(inv_temperature, "inv_temperature", B)
    ws_bytes = fe_sampler_workspace_size(B, V)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=logits.device)
    rc = load_library().fe_sampler_softmax_argmax_ex(
        _dev(probs, torch.float32, "probs", 2), _dev(lse, torch.float32, "lse", 1),
        _dev(argmax, torch.int32, "argmax", 1), _dev(logits, torch.bfloat16, "logits", 2),
        _dev(inv_temperature, torch.float32, "inv_temperature", 1), B, V, int(form),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(rc, "fe_sampler_softmax_argmax")


def fe_hbm_read_probe(base, tile_ids, sink, stream=None) -> None:
    """Read the 4 KiB tiles of uint8 device buffer ``base`` listed in int32
    ``tile_ids`` with the decode kernel's load form (a read-rate probe);
    ``sink`` is an int32 device tensor of ceil(n / 16) words."""
    _shape(base, "base", None)
    _shape(tile_ids, "tile_ids", None)
    n = tile_ids.shape[0]
    _shape(sink, "sink", (n + 15) // 16)
    rc = load_library().fe_hbm_read_probe(
        _dev(base, torch.uint8, "base", 1), base.numel() // 4096, _dev(tile_ids, torch.int32, "tile_ids", 1), n,
        _dev(sink, torch.int32, "sink", 1), _stream(stream))
    _check(rc, "fe_hbm_read_probe")


def fe_mfma_rate_probe(operands, workgroups: int, rounds: int, sink, stream=None) -> None:
    """Issue workgroups * 8 waves * rounds * 64 bf16 MFMAs (32x32x16) on
    operands from the bfloat16 device tensor ``operands`` (a multiple of 8
    elements); ``sink`` is a float32 device tensor of workgroups * 8 sums."""
    _shape(operands, "operands", None)
    if operands.numel() % 8:
        raise ValueError("fe_mfma_rate_probe: operands must hold a multiple of 8 bf16 values")
    _shape(sink, "sink", int(workgroups) * 8)
    rc = load_library().fe_mfma_rate_probe(
        _dev(operands, torch.bfloat16, "operands", 1), operands.numel() // 8, int(workgroups), int(rounds),
        _dev(sink, torch.float32, "sink", 1), _stream(stream))
    _check(rc, "fe_mfma_rate_probe")


# ----------------------------------------------------------------------------
# paged KV block allocator (host)

def fe_kv_allocator_create(num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int) -> int:
    h = load_library().fe_kv_allocator_create(num_blocks, block_size, max_seqs, max_blocks_per_seq)
    if not h:
        raise ValueError("fe_kv_allocator_create: invalid sizes")
    return h


def fe_kv_allocator_destroy(h) -> None:
    load_library().fe_kv_allocator_destroy(h)


def fe_kv_allocator_append(h, seq: int, n: int) -> np.ndarray:
    """Slots (int32 [n]) of n new tokens at the end of sequence seq."""
    out = np.zeros(max(int(n), 0), np.int32)
    _check(load_library().fe_kv_allocator_append(h, int(seq), int(n), out.ctypes.data_as(ctypes.c_void_p)),
           "fe_kv_allocator_append")
    return out


def fe_kv_allocator_release(h, seq: int) -> None:
    _check(load_library().fe_kv_allocator_release(h, int(seq)), "fe_kv_allocator_release")


def fe_kv_allocator_seq_len(h, seq: int) -> int:
    n = load_library().fe_kv_allocator_seq_len(h, int(seq))
    _check(min(n, 0), "fe_kv_allocator_seq_len")
    return n


def fe_kv_allocator_num_free(h) -> int:
    return load_library().fe_kv_allocator_num_free(h)


def fe_kv_allocator_num_allocated(h) -> int:
    return load_library().fe_kv_allocator_num_allocated(h)


def fe_kv_allocator_batch(h, seqs, row_len: int, pad_block: int = 0):
    """(block_tables int32 [n][row_len], context_lens int32 [n]) of the listed sequences."""
    s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
    bt = np.zeros((s.shape[0], row_len), np.int32)
    cl = np.zeros(s.shape[0], np.int32)
    _check(load_library().fe_kv_allocator_batch(h, s.ctypes.data_as(ctypes.c_void_p), s.shape[0],
                                                bt.ctypes.data_as(ctypes.c_void_p), int(row_len), int(pad_block),
                                                cl.ctypes.data_as(ctypes.c_void_p)), "fe_kv_allocator_batch")
    return bt, cl


class KVAllocator:
    """Owning wrapper of an fe_kv_allocator handle (same calls, as methods)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int):
        self.handle = None
        self.handle = fe_kv_allocator_create(num_blocks, block_size, max_seqs, max_blocks_per_seq)
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq

    def append(self, seq, n):
        return fe_kv_allocator_append(self.handle, seq, n)

    def release(self, seq):
        fe_kv_allocator_release(self.handle, seq)

    def seq_len(self, seq):
        return fe_kv_allocator_seq_len(self.handle, seq)

    @property
    def num_free(self):
        return fe_kv_allocator_num_free(self.handle)

    @property
    def num_allocated(self):
        return fe_kv_allocator_num_allocated(self.handle)

    def batch(self, seqs, row_len=None, pad_block=0):
        return fe_kv_allocator_batch(self.handle, seqs, row_len or self.max_blocks_per_seq, pad_block)

    def close(self):
        if getattr(self, "handle", None):
            fe_kv_allocator_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()
