"""CPU fp64 oracle for paged grouped-query attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (built from
``oracle.cpp`` by g++, see :func:`build`) with NumPy marshalling.  It shares no
code with the HIP library and never imports it.

What each function computes, and the passage it follows, is documented in
``oracle.cpp``.  Inputs are torch CPU tensors or NumPy arrays; bf16 tensors are
passed by their bit patterns.  Results come back as float64 NumPy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (no GPU code)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           _SRC, "-o", _LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def use_library(path=None):
    """Point the wrappers at another build of oracle.cpp (tests load deliberately
    broken copies to show the pins catch them); ``None`` restores the default."""
    global _lib, _lib_override
    _lib = None
    _lib_override = path


_lib_override = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_override or _LIB_PATH
    if _lib_override is None and (not os.path.exists(_LIB_PATH)
                                  or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    Dd = ctypes.c_double
    lib.oracle_append.argtypes = [P, P, P, I, P, P, I, I, I, I]
    lib.oracle_append.restype = None
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, Dd, I]
    lib.oracle_decode.restype = I
    lib.oracle_decode_split.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, Dd, I, I, I]
    lib.oracle_decode_split.restype = I
    lib.oracle_merge.argtypes = [P, P, P, P, I, I, I]
    lib.oracle_merge.restype = None
    lib.oracle_prefill_chunk.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, Dd, P, I, I]
    lib.oracle_prefill_chunk.restype = I
    lib.oracle_qk_norm_rope.argtypes = [P, P, P, P, I, P, I, I, I, Dd, I]
    lib.oracle_qk_norm_rope.restype = I
    lib.oracle_sampler.argtypes = [P, P, P, P, P, I, I, I]
    lib.oracle_sampler.restype = I
    lib.oracle_narrow_bf16.argtypes = [Dd]
    lib.oracle_narrow_bf16.restype = ctypes.c_uint16
    _lib = lib
    return lib


def _bits(x) -> np.ndarray:
    """bf16 tensor/array -> contiguous uint16 bit pattern array."""
    if hasattr(x, "view") and hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch  # local: only needed for torch inputs

        return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    a = np.asarray(x)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bits (uint16), got {a.dtype}")
    return np.ascontiguousarray(a)


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


def append(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Bit-copy append.  Returns new (k_cache, v_cache) uint16 arrays."""
    kn, vn, sm = _bits(k_new), _bits(v_new), _i32(slot_mapping)
    kc, vc = _bits(k_cache).copy(), _bits(v_cache).copy()
    NB, Hkv, BS, D = kc.shape
    T = sm.shape[0]
    assert kn.shape == (T, Hkv, D) and vn.shape == (T, Hkv, D) and vc.shape == kc.shape
    _load().oracle_append(_ptr(kn), _ptr(vn), _ptr(sm), T, _ptr(kc), _ptr(vc), NB, Hkv, D, BS)
    return kc, vc


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, nthreads=None):
    """fp64 decode attention.  Returns (out [B][Hq][D], lse [B][Hq])."""
    qb, kc, vc = _bits(q), _bits(k_cache), _bits(v_cache)
    bt, cl = _i32(block_tables), _i32(context_lens)
    B, Hq, D = qb.shape
    NB, Hkv, BS, D2 = kc.shape
    assert D2 == D and vc.shape == kc.shape and bt.shape[0] == B and cl.shape == (B,)
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = _load().oracle_decode(_ptr(out), _ptr(lse), _ptr(qb), _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1],
                               _ptr(cl), B, Hq, Hkv, D, BS, float(scale), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_decode rejected the shapes (status {rc})")
    return out, lse


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, S, P, nthreads=None):
    """Per-partition partials over token ranges [p*S, (p+1)*S) clipped to L."""
    qb, kc, vc = _bits(q), _bits(k_cache), _bits(v_cache)
    bt, cl = _i32(block_tables), _i32(context_lens)
    B, Hq, D = qb.shape
    NB, Hkv, BS, _ = kc.shape
    out = np.zeros((B, Hq, P, D), np.float64)
    lse = np.zeros((B, Hq, P), np.float64)
    rc = _load().oracle_decode_split(_ptr(out), _ptr(lse), _ptr(qb), _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1],
                                     _ptr(cl), B, Hq, Hkv, D, BS, float(scale), int(S), int(P),
                                     _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_decode_split rejected the arguments (status {rc})")
    return out, lse


def merge(out_part, lse_part):
    """Log-sum-exp merge over the partition axis: [..., P, D], [..., P]."""
    op = np.ascontiguousarray(out_part, dtype=np.float64)
    lp = np.ascontiguousarray(lse_part, dtype=np.float64)
    *lead, P, D = op.shape
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros((*lead, D), np.float64)
    lse = np.zeros(tuple(lead), np.float64)
    _load().oracle_merge(_ptr(out), _ptr(lse), _ptr(op), _ptr(lp), rows, P, D)
    return out, lse


def prefill_chunk(q, query_start_loc, k_cache, v_cache, block_tables, context_lens, scale, rows=None,
                  nthreads=None):
    """fp64 chunked-prefill attention (bottom-right causal).

    Returns (out [n][Hq][D], lse [n][Hq]) for every packed row, or only for the
    packed row indices in ``rows``.
    """
    qb, kc, vc = _bits(q), _bits(k_cache), _bits(v_cache)
    qsl, bt, cl = _i32(query_start_loc), _i32(block_tables), _i32(context_lens)
    total_q, Hq, D = qb.shape
    NB, Hkv, BS, _ = kc.shape
    B = cl.shape[0]
    assert qsl.shape == (B + 1,)
    if rows is None:
        rr, n = None, total_q
    else:
        rr = _i32(rows)
        n = rr.shape[0]
    out = np.zeros((n, Hq, D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    rc = _load().oracle_prefill_chunk(_ptr(out), _ptr(lse), _ptr(qb), _ptr(qsl), _ptr(kc), _ptr(vc), _ptr(bt),
                                      bt.shape[1], _ptr(cl), B, total_q, Hq, Hkv, D, BS, float(scale),
                                      _ptr(rr) if rr is not None else None, n, _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_prefill_chunk rejected the shapes (status {rc})")
    return out, lse


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def norm_rope(x, w, cos_sin, positions, eps, nthreads=None):
    """Per-head RMSNorm + rotary embedding of x [T][H][D] (bf16).  Returns the
    bf16 result as uint16 bits [T][H][D]."""
    xb, wb, cs, pos = _bits(x), _bits(w), _f32(cos_sin), _i32(positions)
    T, H, D = xb.shape
    assert wb.shape == (D,) and cs.ndim == 2 and cs.shape[1] == D and pos.shape == (T,)
    out = np.zeros((T, H, D), np.uint16)
    rc = _load().oracle_qk_norm_rope(_ptr(out), _ptr(xb), _ptr(wb), _ptr(cs), cs.shape[0], _ptr(pos), T, H, D,
                                     float(eps), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_qk_norm_rope rejected the arguments (status {rc})")
    return out


def qk_norm_rope_append(q, k, v, q_norm_w, k_norm_w, cos_sin, positions, slot_mapping, k_cache, v_cache, eps):
    """The fused step: normed + rotated q (bits [T][Hq][D]), and the pools after
    appending normed + rotated k and the unchanged v at the slots."""
    q_out = norm_rope(q, q_norm_w, cos_sin, positions, eps)
    k_rows = norm_rope(k, k_norm_w, cos_sin, positions, eps)
    kc, vc = append(k_rows, v, slot_mapping, k_cache, v_cache)
    return q_out, k_rows, kc, vc


def narrow_bf16(v: float) -> int:
    """Nearest-even bf16 bits of a double (the oracle's own rounding)."""
    return int(_load().oracle_narrow_bf16(float(v)))


def sampler(logits, inv_temp=None, with_probs=True, nthreads=None):
    """fp64 softmax / log-sum-exp / greedy argmax of bf16 logits [B][V] at
    per-row inverse temperatures.  Returns (probs [B][V] or None, lse [B], argmax [B] int32)."""
    x = _bits(logits)
    B, V = x.shape
    it = None if inv_temp is None else _f32(inv_temp)
    probs = np.zeros((B, V), np.float64) if with_probs else None
    lse = np.zeros(B, np.float64)
    am = np.zeros(B, np.int32)
    rc = _load().oracle_sampler(_ptr(probs) if probs is not None else None, _ptr(lse), _ptr(am), _ptr(x),
                                _ptr(it) if it is not None else None, B, V, _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_sampler rejected the sizes (status {rc})")
    return probs, lse, am
