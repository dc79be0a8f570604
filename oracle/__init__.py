"""CPU oracle for paged-attention decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It is the plain, slow fp64 reference the GPU library is checked against and
shares no code with it: the arithmetic lives in ``pkv_oracle.c`` (built with gcc into
``liboracle.so`` next to it) and in ``sizing.py``.

The wrappers take numpy arrays (or CPU torch tensors) of 16-bit words — the raw bits of bf16 or
fp16 values — and return float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP16 = 1

_lib = None


def build() -> str:
    """Compile pkv_oracle.c with gcc (fp64, IEEE semantics, OpenMP) into liboracle.so."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i = ctypes.c_int
    lg = ctypes.c_long
    lib.oracle_pool_index.argtypes = [i, lg, i, i, i, i, i, i]
    lib.oracle_pool_index.restype = lg
    lib.oracle_gather.argtypes = [p, p, p, p, i, p, i, i, i, i, i, lg]
    lib.oracle_gather.restype = i
    lib.oracle_paged_decode.argtypes = [p, p, p, p, i, p, p, i, i, i, i, i, lg, i,
                                        ctypes.c_float, p, i, i]
    lib.oracle_paged_decode.restype = i
    lib.oracle_reshape_and_cache.argtypes = [p, p, p, p, p, i, i, i, i, lg]
    lib.oracle_reshape_and_cache.restype = i
    lib.oracle_e4m3_value.argtypes = [i]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = i
    lib.oracle_pool_index8.argtypes = [i, lg, i, i, i, i, i, i]
    lib.oracle_pool_index8.restype = lg
    f = ctypes.c_float
    lib.oracle_paged_decode8.argtypes = [p, p, p, p, f, f, i, p, p, i, i, i, i, i, lg, i, f, p, i,
                                         i]
    lib.oracle_paged_decode8.restype = i
    lib.oracle_reshape_and_cache8.argtypes = [p, p, p, p, i, f, f, p, i, i, i, i, lg]
    lib.oracle_reshape_and_cache8.restype = i
    lib.oracle_dead_slot_indices.argtypes = [i, i, p, p, i, i, i, i, i, p, lg]
    lib.oracle_dead_slot_indices.restype = lg
    lib.oracle_slot_indices.argtypes = [i, i, p, i, i, i, i, p, lg]
    lib.oracle_slot_indices.restype = lg
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    _lib = lib
    return lib


def _words(a) -> np.ndarray:
    """Raw 16-bit words of a numpy array or CPU torch tensor (bf16/fp16/int16/uint16)."""
    if not isinstance(a, np.ndarray):  # torch tensor
        import torch
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.view(torch.int16)
        a = a.contiguous().numpy()
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit words, got {a.dtype}")
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    if not isinstance(a, np.ndarray):
        a = a.contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def pool_index(is_v: bool, block: int, kv_head: int, slot: int, dim: int,
               num_kv_heads: int, block_size: int, head_dim: int) -> int:
    """Element index of (block, kv head, token slot, dim) in one layer's K or V pool."""
    return int(_load().oracle_pool_index(int(bool(is_v)), block, kv_head, slot, dim,
                                         num_kv_heads, block_size, head_dim))


def dead_slot_indices(is_v: bool, fp8: bool, block_tables, context_lens, num_kv_heads: int,
                      block_size: int, head_dim: int) -> np.ndarray:
    """int64 pool indices (pool_index / pool_index8) of every dead slot: slots n mod B .. B-1
    of each sequence's partly filled last block, all kv heads and dims."""
    bt, cl = _i32(block_tables), _i32(context_lens)
    S = cl.shape[0]
    mb = bt.shape[1] if bt.ndim == 2 else 0
    args = (int(bool(is_v)), int(bool(fp8)), _ptr(bt), _ptr(cl), S, mb, num_kv_heads, block_size,
            head_dim)
    n = int(_load().oracle_dead_slot_indices(*args, None, 0))
    out = np.zeros(max(n, 1), np.int64)
    _load().oracle_dead_slot_indices(*args, _ptr(out), n)
    return out[:n]


def slot_indices(is_v: bool, fp8: bool, slot_mapping, num_kv_heads: int, block_size: int,
                 head_dim: int) -> np.ndarray:
    """int64 pool indices (pool_index / pool_index8) of the whole token rows named by the
    non-negative slots (all kv heads and dims)."""
    sm = slot_mapping
    if not isinstance(sm, np.ndarray):
        sm = sm.contiguous().numpy()
    sm = np.ascontiguousarray(sm, dtype=np.int64)
    args = (int(bool(is_v)), int(bool(fp8)), _ptr(sm), sm.shape[0], num_kv_heads, block_size,
            head_dim)
    n = int(_load().oracle_slot_indices(*args, None, 0))
    out = np.zeros(max(n, 1), np.int64)
    _load().oracle_slot_indices(*args, _ptr(out), n)
    return out[:n]


def gather(k_pool, v_pool, dtype: int, table, n: int, kv_head: int, num_kv_heads: int,
           head_dim: int, block_size: int, num_blocks: int):
    """Contiguous fp64 K_c[n][D], V_c[n][D] of one sequence's first n tokens for one kv head."""
    kp, vp, tb = _words(k_pool), _words(v_pool), _i32(table)
    K = np.zeros((max(n, 1), head_dim), np.float64)
    V = np.zeros((max(n, 1), head_dim), np.float64)
    rc = _load().oracle_gather(_ptr(K), _ptr(V), _ptr(kp), _ptr(vp), dtype, _ptr(tb), n, kv_head,
                               num_kv_heads, head_dim, block_size, num_blocks)
    if rc != 0:
        raise ValueError("block table entry out of range")
    return K[:n], V[:n]


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, block_size: int, num_blocks: int, dtype: int,
                 pairs=None, threads: int = 0) -> np.ndarray:
    """fp64 decode attention. Returns [S][Hq][D], or [len(pairs)][D] for a list of (s, h)."""
    qw, kp, vp = _words(q), _words(k_pool), _words(v_pool)
    bt, cl = _i32(block_tables), _i32(context_lens)
    S = cl.shape[0]
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0
    if pairs is None:
        out = np.zeros((S, num_q_heads, head_dim), np.float64)
        pp, npairs = None, 0
    else:
        pa = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((pa.shape[0], head_dim), np.float64)
        pp, npairs = _ptr(pa), pa.shape[0]
    rc = _load().oracle_paged_decode(_ptr(out), _ptr(qw), _ptr(kp), _ptr(vp), dtype, _ptr(bt),
                                     _ptr(cl), S, num_q_heads, num_kv_heads, head_dim, block_size,
                                     num_blocks, max_blocks, ctypes.c_float(scale), pp, npairs,
                                     threads)
    if rc != 0:
        raise ValueError(f"oracle_paged_decode failed ({rc})")
    return out


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key, value, slot_mapping,
                      num_kv_heads: int, head_dim: int, block_size: int, num_blocks: int) -> None:
    """In-place host scatter of new tokens into numpy uint16 copies of one layer's pools."""
    if k_pool.dtype != np.uint16 or v_pool.dtype != np.uint16:
        raise TypeError("pools must be uint16 numpy arrays (modified in place)")
    if not (k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
        raise ValueError("pools must be contiguous")
    kw, vw = _words(key), _words(value)
    sm = slot_mapping
    if not isinstance(sm, np.ndarray):
        sm = sm.contiguous().numpy()
    sm = np.ascontiguousarray(sm, dtype=np.int64)
    rc = _load().oracle_reshape_and_cache(_ptr(k_pool), _ptr(v_pool), _ptr(kw), _ptr(vw),
                                          _ptr(sm), sm.shape[0], num_kv_heads, head_dim,
                                          block_size, num_blocks)
    if rc != 0:
        raise ValueError("slot out of range")


# ---- fp8 (OCP E4M3) KV pools: one fp32 scale per pool; value = e4m3_value(code) * scale ----

def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code (from the format's definition)."""
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode(y: float) -> int:
    """Nearest E4M3 code to the fp32 value y (ties to even, saturating, NaN kept)."""
    return int(_load().oracle_e4m3_encode(ctypes.c_float(y)))


def pool_index8(is_v: bool, block: int, kv_head: int, slot: int, dim: int, num_kv_heads: int,
                block_size: int, head_dim: int) -> int:
    """Byte index of (block, kv head, token slot, dim) in one layer's fp8 K or V pool."""
    return int(_load().oracle_pool_index8(int(bool(is_v)), block, kv_head, slot, dim,
                                          num_kv_heads, block_size, head_dim))


def _bytes(a) -> np.ndarray:
    if not isinstance(a, np.ndarray):
        import torch
        if a.dtype != torch.uint8:
            a = a.view(torch.uint8)
        a = a.contiguous().numpy()
    if a.dtype != np.uint8:
        a = a.view(np.uint8)
    return np.ascontiguousarray(a)


def paged_decode8(q, k_pool, v_pool, k_scale: float, v_scale: float, block_tables, context_lens,
                  scale: float, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  block_size: int, num_blocks: int, dtype: int, pairs=None,
                  threads: int = 0) -> np.ndarray:
    """fp64 decode attention over fp8 pools (q 16-bit). Returns [S][Hq][D] or [len(pairs)][D]."""
    qw, kp, vp = _words(q), _bytes(k_pool), _bytes(v_pool)
    bt, cl = _i32(block_tables), _i32(context_lens)
    S = cl.shape[0]
    max_blocks = bt.shape[1] if bt.ndim == 2 else 0
    if pairs is None:
        out = np.zeros((S, num_q_heads, head_dim), np.float64)
        pp, npairs = None, 0
    else:
        pa = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((pa.shape[0], head_dim), np.float64)
        pp, npairs = _ptr(pa), pa.shape[0]
    f = ctypes.c_float
    rc = _load().oracle_paged_decode8(_ptr(out), _ptr(qw), _ptr(kp), _ptr(vp), f(k_scale),
                                      f(v_scale), dtype, _ptr(bt), _ptr(cl), S, num_q_heads,
                                      num_kv_heads, head_dim, block_size, num_blocks, max_blocks,
                                      f(scale), pp, npairs, threads)
    if rc != 0:
        raise ValueError(f"oracle_paged_decode8 failed ({rc})")
    return out


def reshape_and_cache8(k_pool: np.ndarray, v_pool: np.ndarray, key, value, dtype: int,
                       k_scale: float, v_scale: float, slot_mapping, num_kv_heads: int,
                       head_dim: int, block_size: int, num_blocks: int) -> None:
    """In-place host scatter of 16-bit new tokens, quantized to E4M3, into numpy uint8 copies of
    one layer's fp8 pools."""
    if k_pool.dtype != np.uint8 or v_pool.dtype != np.uint8:
        raise TypeError("pools must be uint8 numpy arrays (modified in place)")
    if not (k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
        raise ValueError("pools must be contiguous")
    kw, vw = _words(key), _words(value)
    sm = slot_mapping
    if not isinstance(sm, np.ndarray):
        sm = sm.contiguous().numpy()
    sm = np.ascontiguousarray(sm, dtype=np.int64)
    f = ctypes.c_float
    rc = _load().oracle_reshape_and_cache8(_ptr(k_pool), _ptr(v_pool), _ptr(kw), _ptr(vw), dtype,
                                           f(k_scale), f(v_scale), _ptr(sm), sm.shape[0],
                                           num_kv_heads, head_dim, block_size, num_blocks)
    if rc != 0:
        raise ValueError("slot out of range")
