"""PagedAttention decode for AMD Instinct MI355X (gfx950): Python binding of libpagedkv.

Every entry point has the name of the C function it wraps (include/pagedkv.h) and only marshals
arguments: tensors become device pointers, the current torch stream becomes the hipStream_t,
a non-OK status becomes a PagedKVError. All computation happens in the HIP library; there is no
fallback path. The library is loaded from this package directory (libpagedkv.so, built by
``python -m paged_kv_cache_452_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_BF16 = 0
PKV_FP16 = 1
PKV_FP8_E4M3 = 2
PKV_SWAP_OUT = 0
PKV_SWAP_IN = 1

EXPORTED = ("kv_pool_bytes", "kv_pool_create", "kv_pool_layer", "kv_pool_destroy",
            "reshape_and_cache", "paged_attention_num_workgroups",
            "paged_attention_workspace_bytes", "paged_attention_decode", "copy_blocks",
            "reshape_and_cache_fp8", "paged_attention_decode_fp8", "swap_blocks", "swap_blocks_dma",
            "paged_attention_decode_append", "paged_attention_decode_append_fp8",
            "kv_block_manager_create", "kv_block_manager_destroy", "kv_block_manager_num_free",
            "kv_block_manager_allocate", "kv_block_manager_fork", "kv_block_manager_append",
            "kv_block_manager_release", "kv_block_manager_tables", "kv_block_manager_num_free_host",
            "kv_block_manager_swap_out", "kv_block_manager_swap_in", "pkv_status_string",
            "paged_attention_check_inputs",
            "paged_attention_decode_noalloc")

PKV_NOALLOC_SCRATCH_BYTES = 17043456  # include/pagedkv.h

PKV_ERR_NO_BLOCKS = -6


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} ({status})")
        self.status = status


_lib = None


def load_library(build_if_missing: bool = True):
    """Load libpagedkv.so (building it first only when it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is not built")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.kv_pool_bytes.argtypes = [i, i, i, i, i, i]
    lib.kv_pool_bytes.restype = sz
    lib.kv_pool_create.argtypes = [ctypes.POINTER(vp), vp, sz, i, i, i, i, i, i]
    lib.kv_pool_create.restype = i
    lib.kv_pool_layer.argtypes = [vp, i, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.kv_pool_layer.restype = i
    lib.kv_pool_destroy.argtypes = [vp]
    lib.kv_pool_destroy.restype = None
    lib.reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.reshape_and_cache.restype = i
    lib.paged_attention_num_workgroups.argtypes = [i, i, i, i, i]
    lib.paged_attention_num_workgroups.restype = i
    lib.paged_attention_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.paged_attention_workspace_bytes.restype = sz
    lib.paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, i,
                                           vp, sz, vp]
    lib.paged_attention_decode.restype = i
    lib.reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, vp]
    lib.reshape_and_cache_fp8.restype = i
    lib.paged_attention_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, f, f, f, i, i, i, i, i, i,
                                               i, i, i, vp, sz, vp]
    lib.paged_attention_decode_fp8.restype = i
    lib.paged_attention_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f, i, i, i, i, i,
                                                  i, i, i, i, vp, sz, vp]
    lib.paged_attention_decode_append.restype = i
    lib.paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, f, i, i, i, i, i, i, i,
                                                   i, i, vp]
    lib.paged_attention_decode_noalloc.restype = i
    lib.paged_attention_check_inputs.argtypes = [vp, vp, i, i, i, i, i, vp, i, vp, vp]
    lib.paged_attention_check_inputs.restype = i
    lib.paged_attention_decode_append_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f, f, f, i,
                                                      i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.paged_attention_decode_append_fp8.restype = i
    lib.copy_blocks.argtypes = [vp, vp, vp, i, vp]
    lib.swap_blocks.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.swap_blocks.restype = i
    lib.swap_blocks_dma.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.swap_blocks_dma.restype = i
    lib.copy_blocks.restype = i
    i64 = ctypes.c_int64
    lib.kv_block_manager_create.argtypes = [ctypes.POINTER(vp), i, i, i]
    lib.kv_block_manager_create.restype = i
    lib.kv_block_manager_destroy.argtypes = [vp]
    lib.kv_block_manager_destroy.restype = None
    lib.kv_block_manager_num_free.argtypes = [vp]
    lib.kv_block_manager_num_free.restype = i
    lib.kv_block_manager_num_free_host.argtypes = [vp]
    lib.kv_block_manager_num_free_host.restype = i
    for fn in (lib.kv_block_manager_swap_out, lib.kv_block_manager_swap_in):
        fn.argtypes = [vp, vp, i, vp, vp, i, ctypes.POINTER(i)]
        fn.restype = i
    lib.kv_block_manager_allocate.argtypes = [vp, i64, i64]
    lib.kv_block_manager_allocate.restype = i
    lib.kv_block_manager_fork.argtypes = [vp, i64, i64]
    lib.kv_block_manager_fork.restype = i
    lib.kv_block_manager_append.argtypes = [vp, vp, i, vp, vp, vp, ctypes.POINTER(i)]
    lib.kv_block_manager_append.restype = i
    lib.kv_block_manager_release.argtypes = [vp, i64]
    lib.kv_block_manager_release.restype = i
    lib.kv_block_manager_tables.argtypes = [vp, vp, i, i, vp, vp]
    lib.kv_block_manager_tables.restype = i
    lib.pkv_status_string.argtypes = [i]
    lib.pkv_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().pkv_status_string(status).decode()
        raise PagedKVError(fn, status, msg)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float16:
        return PKV_FP16
    raise TypeError(f"unsupported element type {t.dtype} (bf16 or fp16)")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require_cuda(*tensors) -> None:
    for t in tensors:
        if t is not None and not isinstance(t, int) and not t.is_cuda:
            raise ValueError("device tensors required (the library runs on the GPU only)")


# Argument checks of the bindings. The kernels take raw addresses and trust the element types,
# shapes and the dense row-major layout of what they index: an int64 block table or a sliced view
# read as int32 would send table padding or the wrong rows into the pool walk. Every check runs
# before any launch and raises ValueError.

def _int_tensor(name: str, t, dtype, ndim: int, rows: Optional[int] = None,
                address_ok: bool = False):
    import torch
    if isinstance(t, int) and address_ok:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor or a device address")
    if t.dtype != dtype:
        raise ValueError(f"{name}: element type {t.dtype}, expected {dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {ndim}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name}: {t.shape[0]} rows, expected {rows}")


def _rows(name: str, t, shape, dtype=None):
    """A dense [..] tensor of 16-bit elements with exactly `shape` (and `dtype`, when given)."""
    import torch
    if isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor or a device address")
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"{name}: element type {t.dtype}, expected bfloat16 or float16")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: element type {t.dtype}, expected {dtype} (as q / key)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _disjoint(name: str, t, others) -> None:
    """The output tensor `t` shares no byte with any of `others` ((name, tensor) pairs; device
    addresses and None are skipped). The kernels read their inputs while they write the output,
    so an output that overlaps an input is refused rather than left to the order of the writes."""
    if not hasattr(t, "data_ptr"):
        return
    a0 = t.data_ptr()
    a1 = a0 + t.numel() * t.element_size()
    for other_name, o in others:
        if not hasattr(o, "data_ptr") or o.numel() == 0 or t.numel() == 0:
            continue
        b0 = o.data_ptr()
        b1 = b0 + o.numel() * o.element_size()
        if a0 < b1 and b0 < a1:
            raise ValueError(f"{name}: must not overlap {other_name}")


def _plane(name: str, t, dtype, tile: int = 0, tiles: Optional[int] = None):
    """A pool plane: a view whose last dimension is dense (the K or V tiles of one layer), of the
    pool's element type. The K and V tiles of a (block, kv head) alternate in the pool, so the
    kernels address the n tiles of a plane across 2n - 1 tiles of memory from its first element:
    with `tile` (elements per tile) given, the tensor's storage must hold that span from the view
    on. n is `tiles` when the caller knows it (num_blocks * num_kv_heads), else the tiles the view
    itself covers. A compact copy of a plane (half that span) is refused here, before any launch
    could write or read past its end."""
    import torch
    if isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor or a device address")
    if t.dtype != dtype:
        raise ValueError(f"{name}: element type {t.dtype}, expected {dtype}")
    if t.dim() == 0 or (t.shape[-1] > 1 and t.stride(-1) != 1):
        raise ValueError(f"{name}: the last dimension must be dense")
    if tile > 0:
        n = tiles if tiles is not None else t.numel() // tile
        span = (2 * n - 1) * tile if n > 0 else 0
        held = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
        if held < span:
            raise ValueError(
                f"{name}: its storage holds {held} elements from this view, but the {n} tiles of "
                f"a plane span {span} (K and V tiles alternate): pass a plane of the pool "
                "(a view), not a copy")


def _workspace(t):
    import torch
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor")


def _decode_args(name, out, q, k_pool, v_pool, block_tables, context_lens, num_q_heads,
                 head_dim, block_size, pool_dtype=None):
    """Checks shared by the decode bindings. Returns the number of sequences."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError(f"{name}: q must be a tensor [num_seqs][num_q_heads][head_dim]")
    S = q.shape[0]
    _rows("q", q, (S, num_q_heads, head_dim))
    _rows("out", out, (S, num_q_heads, head_dim), q.dtype)
    _disjoint("out", out, (("q", q),))
    pd = q.dtype if pool_dtype is None else pool_dtype
    _plane("k_pool", k_pool, pd, block_size * head_dim)
    _plane("v_pool", v_pool, pd, block_size * head_dim)
    _int_tensor("block_tables", block_tables, torch.int32, 2, S)
    _int_tensor("context_lens", context_lens, torch.int32, 1, S)
    return S


def pkv_status_string(status: int) -> str:
    return load_library().pkv_status_string(status).decode()


def kv_pool_bytes(num_layers: int, num_blocks: int, num_kv_heads: int, head_dim: int,
                  block_size: int, dtype: int) -> int:
    return int(load_library().kv_pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim,
                                            block_size, dtype))


class KVPool:
    """Host-side geometry of a caller-owned KV pool (kv_pool_create / kv_pool_destroy): one
    allocation of [layer][block][kv_head][K tile, V tile]."""

    def __init__(self, base, nbytes: int, num_layers: int, num_blocks: int, num_kv_heads: int,
                 head_dim: int, block_size: int, dtype: int):
        lib = load_library()
        h = ctypes.c_void_p()
        _check("kv_pool_create", lib.kv_pool_create(ctypes.byref(h), _ptr(base), nbytes,
                                                    num_layers, num_blocks, num_kv_heads,
                                                    head_dim, block_size, dtype))
        self._h = h
        self._keep = base
        self.num_layers = num_layers

    def layer(self, layer: int) -> Tuple[int, int]:
        return kv_pool_layer(self, layer)

    def destroy(self) -> None:
        if self._h is not None and self._h.value:
            load_library().kv_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def kv_pool_create(base, nbytes: int, num_layers: int, num_blocks: int, num_kv_heads: int,
                   head_dim: int, block_size: int, dtype: int) -> KVPool:
    return KVPool(base, nbytes, num_layers, num_blocks, num_kv_heads, head_dim, block_size, dtype)


def kv_pool_layer(pool: KVPool, layer: int) -> Tuple[int, int]:
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check("kv_pool_layer", load_library().kv_pool_layer(pool._h, layer, ctypes.byref(k),
                                                         ctypes.byref(v)))
    return int(k.value or 0), int(v.value or 0)


def kv_pool_destroy(pool: KVPool) -> None:
    pool.destroy()


def reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, num_blocks: int,
                      block_size: int = 16, stream=None) -> None:
    """Scatter key/value [T][Hkv][D] into the pool slots named by slot_mapping (int64 [T]).
    k_pool / v_pool: one layer's K and V planes, as tensors (views) or device addresses."""
    import torch
    if not isinstance(key, torch.Tensor) or key.dim() != 3:
        raise ValueError("key must be a tensor [num_tokens][num_kv_heads][head_dim]")
    T, Hkv, D = key.shape
    _rows("key", key, (T, Hkv, D))
    _rows("value", value, (T, Hkv, D), key.dtype)
    _plane("k_pool", k_pool, key.dtype, block_size * D, num_blocks * Hkv)
    _plane("v_pool", v_pool, key.dtype, block_size * D, num_blocks * Hkv)
    _int_tensor("slot_mapping", slot_mapping, torch.int64, 1, T, address_ok=True)
    _require_cuda(key, value, k_pool, v_pool, slot_mapping)
    _check("reshape_and_cache", load_library().reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping), T, Hkv, D,
        block_size, num_blocks, _dtype_code(key), _stream(stream)))


def paged_attention_num_workgroups(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                   max_context_len: int, block_size: int = 16) -> int:
    return int(load_library().paged_attention_num_workgroups(
        num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size))


def paged_attention_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, block_size: int, max_context_len: int,
                                    num_workgroups: int = 0) -> int:
    r = int(load_library().paged_attention_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
        num_workgroups))
    if r == ctypes.c_size_t(-1).value:
        raise PagedKVError("paged_attention_workspace_bytes", -1, "PKV_ERR_INVALID_ARG")
    return r


def new_workspace(num_bytes: int, device="cuda"):
    """A decode workspace of at least num_bytes, zero-filled (its counters must start at zero;
    every completed call leaves them zero). None when no workspace is needed."""
    import torch
    if num_bytes <= 0:
        return None
    return torch.zeros((num_bytes + 3) // 4, dtype=torch.int32, device=device)


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale: float,
                           num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                           max_context_len: int, num_workgroups: int = 0, workspace=None,
                           stream=None) -> None:
    """out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s over each sequence's paged K/V."""
    S = _decode_args("paged_attention_decode", out, q, k_pool, v_pool, block_tables,
                     context_lens, num_q_heads, head_dim, block_size)
    _workspace(workspace)
    _require_cuda(out, q, k_pool, v_pool, block_tables, context_lens, workspace)
    max_blocks = block_tables.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attention_decode", load_library().paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
        float(scale), num_q_heads, num_kv_heads, head_dim, block_size, S, max_blocks,
        max_context_len, num_workgroups, _dtype_code(q), _ptr(workspace), ws_bytes,
        _stream(stream)))


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens,
                                   scale: float, num_q_heads: int, num_kv_heads: int,
                                   head_dim: int, block_size: int, max_context_len: int,
                                   num_workgroups: int = 0, stream=None) -> None:
    """paged_attention_decode without a workspace: the library's own per-device scratch holds the
    split-stream state, so the call allocates nothing. Calls that overlap in time on one device
    race (they share that scratch); calls ordered on one stream are safe."""
    S = _decode_args("paged_attention_decode_noalloc", out, q, k_pool, v_pool, block_tables,
                     context_lens, num_q_heads, head_dim, block_size)
    _require_cuda(out, q, k_pool, v_pool, block_tables, context_lens)
    _check("paged_attention_decode_noalloc", load_library().paged_attention_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
        float(scale), num_q_heads, num_kv_heads, head_dim, block_size, S,
        block_tables.shape[1], max_context_len, num_workgroups, _dtype_code(q),
        _stream(stream)))


def paged_attention_check_inputs(block_tables, context_lens, num_blocks: int,
                                 block_size: int = 16, max_context_len: Optional[int] = None,
                                 slot_mapping=None, stream=None) -> dict:
    """Debug check of a step's index inputs on the device (never reads the pool). Waits for the
    device and returns the counts: bad_table_entries (used entries outside [0, num_blocks)),
    bad_context_lens, repeated_slots and slots_past_pool (slot_mapping, when given)."""
    import torch
    _int_tensor("block_tables", block_tables, torch.int32, 2)
    S, max_blocks = block_tables.shape
    _int_tensor("context_lens", context_lens, torch.int32, 1, S)
    T = 0
    if slot_mapping is not None:
        _int_tensor("slot_mapping", slot_mapping, torch.int64, 1)
        T = slot_mapping.shape[0]
    _require_cuda(block_tables, context_lens, slot_mapping)
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    result = torch.empty(4, dtype=torch.int32, device=block_tables.device)
    _check("paged_attention_check_inputs", load_library().paged_attention_check_inputs(
        _ptr(block_tables), _ptr(context_lens), S, max_blocks, max_context_len, block_size,
        num_blocks, _ptr(slot_mapping), T, _ptr(result), _stream(stream)))
    torch.cuda.synchronize(result.device)
    c = result.cpu().tolist()
    return dict(bad_table_entries=c[0], bad_context_lens=c[1], repeated_slots=c[2],
                slots_past_pool=c[3])


def reshape_and_cache_fp8(key, value, k_pool, v_pool, slot_mapping, num_blocks: int,
                          k_scale: float, v_scale: float, block_size: int = 16,
                          stream=None) -> None:
    """Quantize key/value [T][Hkv][D] (bf16/fp16) to E4M3 and scatter them into one layer's fp8
    pools (uint8 tensors or device addresses) at the slots named by slot_mapping."""
    import torch
    if not isinstance(key, torch.Tensor) or key.dim() != 3:
        raise ValueError("key must be a tensor [num_tokens][num_kv_heads][head_dim]")
    T, Hkv, D = key.shape
    _rows("key", key, (T, Hkv, D))
    _rows("value", value, (T, Hkv, D), key.dtype)
    _plane("k_pool", k_pool, torch.uint8, block_size * D, num_blocks * Hkv)
    _plane("v_pool", v_pool, torch.uint8, block_size * D, num_blocks * Hkv)
    _int_tensor("slot_mapping", slot_mapping, torch.int64, 1, T, address_ok=True)
    _require_cuda(key, value, k_pool, v_pool, slot_mapping)
    _check("reshape_and_cache_fp8", load_library().reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping), T, Hkv, D,
        block_size, num_blocks, _dtype_code(key), float(k_scale), float(v_scale),
        _stream(stream)))


def paged_attention_decode_fp8(out, q, k_pool, v_pool, block_tables, context_lens, scale: float,
                               k_scale: float, v_scale: float, num_q_heads: int,
                               num_kv_heads: int, head_dim: int, block_size: int,
                               max_context_len: int, num_workgroups: int = 0, workspace=None,
                               stream=None) -> None:
    """paged_attention_decode over fp8 (E4M3) pools with per-pool scales."""
    import torch
    S = _decode_args("paged_attention_decode_fp8", out, q, k_pool, v_pool, block_tables,
                     context_lens, num_q_heads, head_dim, block_size, pool_dtype=torch.uint8)
    _workspace(workspace)
    _require_cuda(out, q, k_pool, v_pool, block_tables, context_lens, workspace)
    max_blocks = block_tables.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attention_decode_fp8", load_library().paged_attention_decode_fp8(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
        float(scale), float(k_scale), float(v_scale), num_q_heads, num_kv_heads, head_dim,
        block_size, S, max_blocks, max_context_len, num_workgroups, _dtype_code(q),
        _ptr(workspace), ws_bytes, _stream(stream)))


def swap_blocks(device_pool: "KVPool", host_pool: "KVPool", src_blocks, dst_blocks,
                direction: int, stream=None) -> None:
    """Copy whole blocks between a device pool and a pinned host pool of the same geometry
    (PKV_SWAP_OUT: device -> host, PKV_SWAP_IN: host -> device). src_blocks, dst_blocks: int32
    tensors on the device or in pinned host memory."""
    import torch
    for t in (src_blocks, dst_blocks):
        if isinstance(t, torch.Tensor):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("block ids must be contiguous int32")
            if not t.is_cuda and not t.is_pinned():
                raise ValueError("block ids must be on the device or in pinned host memory")
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _check("swap_blocks", load_library().swap_blocks(device_pool._h, host_pool._h,
                                                     _ptr(src_blocks), _ptr(dst_blocks), n,
                                                     int(direction), _stream(stream)))


def swap_blocks_dma(device_pool: "KVPool", host_pool: "KVPool", src_blocks, dst_blocks,
                    direction: int, stream=None) -> None:
    """swap_blocks on the GPU's copy engines: the same copies, for swaps that run beside a decode
    on another stream, which they barely slow. src_blocks, dst_blocks: int32 ids in host memory
    (1-D numpy arrays or CPU tensors), read during the call; an id outside its pool refuses the
    whole call."""
    import numpy as np
    import torch
    ptrs = []
    for name, t in (("src_blocks", src_blocks), ("dst_blocks", dst_blocks)):
        if isinstance(t, torch.Tensor):
            if t.is_cuda:
                raise ValueError(f"{name}: must be in host memory (the host reads it)")
            if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
                raise ValueError(f"{name}: must be a contiguous 1-D int32 tensor")
            ptrs.append((t.data_ptr(), t.numel()))
        elif isinstance(t, np.ndarray):
            if t.dtype != np.int32 or t.ndim != 1 or not t.flags.c_contiguous:
                raise ValueError(f"{name}: must be a contiguous 1-D int32 array")
            ptrs.append((t.ctypes.data, t.size))
        else:
            raise ValueError(f"{name}: expected an int32 numpy array or CPU tensor")
    n = ptrs[0][1]
    if ptrs[1][1] != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _check("swap_blocks_dma", load_library().swap_blocks_dma(
        device_pool._h, host_pool._h, ptrs[0][0] if n else None, ptrs[1][0] if n else None, n,
        int(direction), _stream(stream)))


def paged_attention_decode_append(out, q, key, value, k_pool, v_pool, block_tables, context_lens,
                                  scale: float, num_q_heads: int, num_kv_heads: int,
                                  head_dim: int, block_size: int, max_context_len: int,
                                  num_workgroups: int = 0, workspace=None, stream=None,
                                  kv_scales=None) -> None:
    """One fused decode step: each sequence's newest token (key/value [S][Hkv][D], at position
    context_lens[s] - 1) is written into the pool and attended to with the rest of the context.
    kv_scales=(k_scale, v_scale) for fp8 pools."""
    import torch
    S = _decode_args("paged_attention_decode_append", out, q, k_pool, v_pool, block_tables,
                     context_lens, num_q_heads, head_dim, block_size,
                     pool_dtype=None if kv_scales is None else torch.uint8)
    _rows("key", key, (S, num_kv_heads, head_dim), q.dtype)
    _rows("value", value, (S, num_kv_heads, head_dim), q.dtype)
    _disjoint("out", out, (("key", key), ("value", value)))
    _workspace(workspace)
    _require_cuda(out, q, key, value, k_pool, v_pool, block_tables, context_lens, workspace)
    max_blocks = block_tables.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    if kv_scales is None:
        rc = lib.paged_attention_decode_append(
            _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), _ptr(context_lens), float(scale), num_q_heads, num_kv_heads,
            head_dim, block_size, S, max_blocks, max_context_len, num_workgroups,
            _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream))
        _check("paged_attention_decode_append", rc)
    else:
        rc = lib.paged_attention_decode_append_fp8(
            _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), _ptr(context_lens), float(scale), float(kv_scales[0]),
            float(kv_scales[1]), num_q_heads, num_kv_heads, head_dim, block_size, S, max_blocks,
            max_context_len, num_workgroups, _dtype_code(q), _ptr(workspace), ws_bytes,
            _stream(stream))
        _check("paged_attention_decode_append_fp8", rc)


def copy_blocks(pool: "KVPool", src_blocks, dst_blocks, stream=None) -> None:
    """Copy blocks src_blocks[i] -> dst_blocks[i] (device int32 tensors) in every layer of the
    pool's K and V (the device half of copy-on-write)."""
    import torch
    for name, t in (("src_blocks", src_blocks), ("dst_blocks", dst_blocks)):
        _int_tensor(name, t, torch.int32, 1, address_ok=True)
    _require_cuda(src_blocks, dst_blocks)
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _check("copy_blocks", load_library().copy_blocks(pool._h, _ptr(src_blocks) if n else None,
                                                     _ptr(dst_blocks) if n else None, n,
                                                     _stream(stream) if n else None))


class BlockManager:
    """Host block manager (kv_block_manager_*): blocks of one pool, per-sequence tables, fork,
    copy-on-write, and swapping to num_host_blocks host blocks. Plain numpy in and out; no device
    work."""

    def __init__(self, num_blocks: int, block_size: int = 16, num_host_blocks: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        _check("kv_block_manager_create", lib.kv_block_manager_create(
            ctypes.byref(h), num_blocks, num_host_blocks, block_size))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        try:
            if self._h is not None and self._h.value:
                load_library().kv_block_manager_destroy(self._h)
            self._h = None
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(load_library().kv_block_manager_num_free(self._h))

    @property
    def num_free_host(self) -> int:
        return int(load_library().kv_block_manager_num_free_host(self._h))

    def _move(self, name: str, seq_ids, capacity: int):
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        src = np.zeros(max(capacity, 1), np.int32)
        dst = np.zeros(max(capacity, 1), np.int32)
        k = ctypes.c_int(0)
        vp = ctypes.c_void_p
        _check(name, getattr(load_library(), name)(
            self._h, ids.ctypes.data_as(vp), ids.shape[0], src.ctypes.data_as(vp),
            dst.ctypes.data_as(vp), capacity, ctypes.byref(k)))
        return np.stack([src[:k.value], dst[:k.value]], axis=1)

    def swap_out(self, seq_ids):
        """Move the group to host blocks. Returns int32 [k][2] (device block, host block) pairs
        for swap_blocks(PKV_SWAP_OUT)."""
        return self._move("kv_block_manager_swap_out", seq_ids, self.num_blocks)

    def swap_in(self, seq_ids):
        """Bring the group back. Returns int32 [k][2] (host block, device block) pairs for
        swap_blocks(PKV_SWAP_IN)."""
        return self._move("kv_block_manager_swap_in", seq_ids, self.num_blocks)

    def allocate(self, seq_id: int, num_tokens: int) -> None:
        _check("kv_block_manager_allocate",
               load_library().kv_block_manager_allocate(self._h, seq_id, num_tokens))

    def fork(self, src_seq_id: int, dst_seq_id: int) -> None:
        _check("kv_block_manager_fork",
               load_library().kv_block_manager_fork(self._h, src_seq_id, dst_seq_id))

    def release(self, seq_id: int) -> None:
        _check("kv_block_manager_release", load_library().kv_block_manager_release(self._h, seq_id))

    def append(self, seq_ids):
        """One new token per listed sequence. Returns (slot_mapping int64 [n],
        copies int32 [k][2] of (shared block, fresh block))."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        n = ids.shape[0]
        slots = np.zeros(n, np.int64)
        src = np.zeros(max(n, 1), np.int32)
        dst = np.zeros(max(n, 1), np.int32)
        k = ctypes.c_int(0)
        vp = ctypes.c_void_p
        _check("kv_block_manager_append", load_library().kv_block_manager_append(
            self._h, ids.ctypes.data_as(vp), n, slots.ctypes.data_as(vp), src.ctypes.data_as(vp),
            dst.ctypes.data_as(vp), ctypes.byref(k)))
        return slots, np.stack([src[:k.value], dst[:k.value]], axis=1)

    def tables(self, seq_ids, max_blocks_per_seq: int):
        """(block_tables int32 [n][max_blocks_per_seq] padded with -1, context_lens int32 [n])."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        n = ids.shape[0]
        bt = np.zeros((n, max_blocks_per_seq), np.int32)
        cl = np.zeros(n, np.int32)
        vp = ctypes.c_void_p
        _check("kv_block_manager_tables", load_library().kv_block_manager_tables(
            self._h, ids.ctypes.data_as(vp), n, max_blocks_per_seq, bt.ctypes.data_as(vp),
            cl.ctypes.data_as(vp)))
        return bt, cl


class Decoder:
    """Convenience holder of a zero-initialised workspace sized for one decode shape (allocated
    once, reused by every call on one stream)."""

    def __init__(self, num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_context_len: int, block_size: int = 16, num_workgroups: int = 0,
                 device="cuda"):
        self.args = (num_q_heads, num_kv_heads, head_dim, block_size)
        self.max_context_len = max_context_len
        self.num_workgroups = num_workgroups
        nbytes = paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_context_len, num_workgroups)
        self.workspace = new_workspace(nbytes, device)

    def __call__(self, out, q, k_pool, v_pool, block_tables, context_lens, scale, stream=None):
        Hq, Hkv, D, B = self.args
        paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale, Hq, Hkv,
                               D, B, self.max_context_len, self.num_workgroups, self.workspace,
                               stream)
