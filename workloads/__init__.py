"""Seeded synthetic decode batches (shared input source for tests, smoke check and benchmark).

This module draws random numbers and builds host-side block tables; it performs none of the
attention or scatter arithmetic. Everything is seeded, so a (workload, seed) pair names one input.

Shapes follow the five decode workloads this library is measured on:
  1. tiny MHA       S=4, context {1,15,16,41}, 4/4 heads, d64, bf16, pool of 64 blocks
  2. 13B-shaped     S=32, context U{128..2048}, 40/40 heads, d128, fp16, pool 1.5x needed
  3. 8B-shaped GQA  S=64, context U{1024..8192}, 32/8 heads, d128, bf16, pool 1.5x needed
  4. 70B-shaped GQA S=64 x 4096 tokens, 64/8 heads, d128, bf16, 80 layers, 16384 blocks/layer
  5. shared prefix  50 x (800-token shared prefix + U{16..512}), 1 x 32768, 15 x U{64..256},
                    32/8 heads, d128, bf16, pool 1.5x the unique blocks
Block size 16 everywhere. Values are N(0,1) rounded to the element type (round to nearest even).

Block allocation mirrors a paged block manager (host side, for building inputs only): a free list
in seeded random order, blocks popped from its front; a sequence of n tokens owns ceil(n/16)
blocks; the token at position n-1 is the step's new token, written by reshape_and_cache to slot
table[(n-1)//16]*16 + (n-1)%16 — a fresh block when n-1 starts a block.
Blocks no table references are filled with NaN so a stray read shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Spec:
    index: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str              # "bf16" | "fp16"
    num_layers: int
    seed: int
    block_size: int = BLOCK_SIZE

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


SPECS = {
    1: Spec(1, "tiny MHA decode (4 seqs, ctx {1,15,16,41}, 4/4 heads, d64, bf16)",
            4, 4, 4, 64, "bf16", 1, seed=1001),
    2: Spec(2, "13B-shaped MHA decode (32 seqs, ctx U{128..2048}, 40/40 heads, d128, fp16)",
            32, 40, 40, 128, "fp16", 1, seed=2002),
    3: Spec(3, "Llama-3-8B-shaped GQA decode (64 seqs, ctx U{1024..8192}, 32/8 heads, d128, bf16)",
            64, 32, 8, 128, "bf16", 1, seed=3003),
    4: Spec(4, "Llama-3-70B-shaped GQA decode (64 seqs x 4096, 64/8 heads, d128, bf16, 80 layers)",
            64, 64, 8, 128, "bf16", 80, seed=4004),
    5: Spec(5, "shared-prefix + skew GQA decode (50x(800+U{16..512}), 1x32768, 15xU{64..256}, "
               "32/8 heads, d128, bf16)", 66, 32, 8, 128, "bf16", 1, seed=5005),
}


@dataclasses.dataclass
class Tables:
    """Host-side structure of one decode step (no K/V values)."""
    context_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray        # int32 [S][max_blocks], padding -1
    num_blocks: int                 # physical blocks per layer in the pool
    slot_mapping: np.ndarray        # int64 [T], the step's new tokens
    used_blocks: np.ndarray         # bool [num_blocks], referenced by some table
    shared_prefix_blocks: int = 0   # shared-prefix batch: leading table entries shared by its first 50 seqs
    free_list: Optional[List[int]] = None  # remaining free blocks, front first


class FreeList:
    """Physical blocks in seeded random order; pop from the front (host block manager)."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.blocks = [int(b) for b in rng.permutation(num_blocks)]
        self.pos = 0

    def pop(self) -> int:
        if self.pos >= len(self.blocks):
            raise MemoryError("no free physical blocks")
        b = self.blocks[self.pos]
        self.pos += 1
        return b

    def remaining(self) -> List[int]:
        return self.blocks[self.pos:]


def _lens(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    i = spec.index
    if i == 1:
        return np.array([1, 15, 16, 41], np.int32)
    if i == 2:
        return rng.integers(128, 2048, size=32, endpoint=True).astype(np.int32)
    if i == 3:
        return rng.integers(1024, 8192, size=64, endpoint=True).astype(np.int32)
    if i == 4:
        return np.full(64, 4096, np.int32)
    if i == 5:
        suffix = rng.integers(16, 512, size=50, endpoint=True)
        short = rng.integers(64, 256, size=15, endpoint=True)
        return np.concatenate([800 + suffix, [32768], short]).astype(np.int32)
    raise ValueError(i)


def make_tables(spec: Spec, lens: Optional[np.ndarray] = None, pool_factor: float = 1.5,
                num_blocks: Optional[int] = None, seed: Optional[int] = None) -> Tables:
    """Block tables, context lengths and the step's slot mapping for a workload (seeded)."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    B = spec.block_size
    if lens is None:
        lens = _lens(spec, rng)
    lens = np.asarray(lens, np.int32)
    S = lens.shape[0]
    need = [-(-int(n) // B) for n in lens]
    prefix_blocks = 800 // B if spec.index == 5 else 0
    n_prefix_users = 50 if spec.index == 5 else 0
    unique = sum(need) - prefix_blocks * max(n_prefix_users - 1, 0)
    if num_blocks is None:
        if spec.index == 1:
            num_blocks = 64
        elif spec.index == 4:
            num_blocks = unique
        else:
            num_blocks = int(math.ceil(unique * pool_factor))
    free = FreeList(num_blocks, rng)
    max_blocks = max(max(need), 1)
    tables = np.full((S, max_blocks), -1, np.int32)
    prefix = [free.pop() for _ in range(prefix_blocks)]
    for s in range(S):
        row = []
        if s < n_prefix_users:
            row.extend(prefix)
        while len(row) < need[s]:
            row.append(free.pop())
        tables[s, :len(row)] = row
    used = np.zeros(num_blocks, bool)
    for s in range(S):
        used[tables[s, :need[s]]] = True
    slots = []
    for s in range(S):
        n = int(lens[s])
        if n == 0:
            slots.append(-1)
            continue
        p = n - 1
        slots.append(int(tables[s, p // B]) * B + p % B)
    return Tables(lens, tables, num_blocks, np.array(slots, np.int64), used,
                  prefix_blocks, free.remaining())


def append_step(tables: Tables, block_size: int = BLOCK_SIZE) -> Tables:
    """Next decode step: every sequence gains one token at position n (boundary allocation pops
    a fresh block from the free list when n is a multiple of the block size)."""
    lens = tables.context_lens.copy()
    free = list(tables.free_list or [])
    S = lens.shape[0]
    need_more = [int(n) % block_size == 0 for n in lens]
    extra = max(int(np.max([-(-(int(n) + 1) // block_size) for n in lens])) -
                tables.block_tables.shape[1], 0)
    bt = np.concatenate([tables.block_tables, np.full((S, extra), -1, np.int32)], axis=1)
    used = tables.used_blocks.copy()
    slots = []
    for s in range(S):
        n = int(lens[s])
        if need_more[s]:
            if not free:
                raise MemoryError("no free physical blocks")
            b = free.pop(0)
            bt[s, n // block_size] = b
            used[b] = True
        slots.append(int(bt[s, n // block_size]) * block_size + n % block_size)
        lens[s] = n + 1
    return Tables(lens, bt, tables.num_blocks, np.array(slots, np.int64), used,
                  tables.shared_prefix_blocks, free)


@dataclasses.dataclass
class Batch:
    spec: Spec
    tables: Tables
    q: torch.Tensor            # [S][Hq][D]
    k_pool: torch.Tensor       # [L][NB][Hkv][B*D]: the K plane of kv_pool (a strided view)
    v_pool: torch.Tensor       # the V plane
    new_key: torch.Tensor      # [T][Hkv][D]
    new_value: torch.Tensor
    block_tables: torch.Tensor  # int32, on device
    context_lens: torch.Tensor  # int32, on device
    slot_mapping: torch.Tensor  # int64, on device
    kv_pool: Optional[torch.Tensor] = None  # [L][NB][Hkv][2][B*D], the one allocation

    @property
    def scale(self) -> float:
        return self.spec.scale

    @property
    def max_context_len(self) -> int:
        return int(self.tables.context_lens.max()) if self.tables.context_lens.size else 0


def randn(shape, dtype, generator: torch.Generator, device) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to `dtype` (round to nearest even)."""
    return torch.randn(shape, generator=generator, dtype=torch.float32,
                       device=device).to(dtype)


def new_pool(num_layers: int, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
             dtype, device, pin_memory: bool = False) -> torch.Tensor:
    """An uninitialised KV pool in the library's layout: [layer][block][kv_head][K tile, V tile],
    as a tensor [L][NB][Hkv][2][B*D] (one allocation; see planes)."""
    return torch.empty((num_layers, num_blocks, num_kv_heads, 2, block_size * head_dim),
                       dtype=dtype, device=device, pin_memory=pin_memory)


def planes(pool: torch.Tensor):
    """The K and V planes of a pool from new_pool: views [L][NB][Hkv][B*D] whose layer slices
    have the addresses kv_pool_layer gives."""
    return pool.select(-2, 0), pool.select(-2, 1)


def fill_pool_(pool: torch.Tensor, generator: torch.Generator, chunk_elems: int = 1 << 28):
    """Fill a [..] 16-bit pool with N(0,1) in chunks (bounded fp32 temporaries)."""
    flat = pool.view(-1)
    for start in range(0, flat.numel(), chunk_elems):
        stop = min(start + chunk_elems, flat.numel())
        flat[start:stop] = randn((stop - start,), pool.dtype, generator, pool.device)
    return pool


E4M3_NAN = 0x7F   # the NaN code of OCP E4M3, written into unused fp8 pool blocks


def random_e4m3_codes(n: int, generator: torch.Generator, device) -> torch.Tensor:
    """n random 8-bit E4M3 codes (uint8): random sign, exponent field uniform in 0..8, mantissa
    uniform in 0..7, so the magnitudes lie in [0, 3.75] and no code is NaN."""
    kw = dict(generator=generator, device=device, dtype=torch.uint8)
    sign = torch.randint(0, 2, (n,), **kw)
    expo = torch.randint(0, 9, (n,), **kw)
    mant = torch.randint(0, 8, (n,), **kw)
    return (sign << 7) | (expo << 3) | mant


def fill_pool_fp8_(pool: torch.Tensor, generator: torch.Generator, chunk: int = 1 << 30):
    """Fill a uint8 pool with random_e4m3_codes in chunks."""
    flat = pool.view(-1)
    for start in range(0, flat.numel(), chunk):
        stop = min(start + chunk, flat.numel())
        flat[start:stop] = random_e4m3_codes(stop - start, generator, pool.device)
    return pool


def make_batch_fp8(spec: Spec, device="cpu", tables: Optional[Tables] = None,
                   seed: Optional[int] = None) -> Batch:
    """As make_batch, with fp8 pools: uint8 [L][NB][Hkv][B*D] of random E4M3 codes and the NaN
    code in blocks no table references. q, new_key and new_value stay 16-bit."""
    if tables is None:
        tables = make_tables(spec)
    Hq, Hkv, D, B = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    S = tables.context_lens.shape[0]
    L, NB = spec.num_layers, tables.num_blocks
    g = torch.Generator(device=device)
    g.manual_seed((spec.seed if seed is None else seed) * 7919 + 23)
    dt = spec.torch_dtype
    q = randn((S, Hq, D), dt, g, device)
    kv = fill_pool_fp8_(new_pool(L, NB, Hkv, B, D, torch.uint8, device), g)
    k_pool, v_pool = planes(kv)
    if not tables.used_blocks.all():
        unused = torch.from_numpy(np.nonzero(~tables.used_blocks)[0]).to(device)
        k_pool[:, unused] = E4M3_NAN
        v_pool[:, unused] = E4M3_NAN
    T = tables.slot_mapping.shape[0]
    new_key = randn((T, Hkv, D), dt, g, device)
    new_value = randn((T, Hkv, D), dt, g, device)
    return Batch(spec, tables, q, k_pool, v_pool, new_key, new_value,
                 torch.from_numpy(tables.block_tables).to(device),
                 torch.from_numpy(tables.context_lens).to(device),
                 torch.from_numpy(tables.slot_mapping).to(device), kv)


def make_batch(spec: Spec, device="cpu", tables: Optional[Tables] = None,
               poison_unused: bool = True, seed: Optional[int] = None) -> Batch:
    """Full seeded input of one decode step: q, both pools (all layers), new K/V, tables."""
    if tables is None:
        tables = make_tables(spec)
    S, Hq, Hkv, D, B = (spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                        spec.block_size)
    S = tables.context_lens.shape[0]
    L, NB = spec.num_layers, tables.num_blocks
    g = torch.Generator(device=device)
    g.manual_seed((spec.seed if seed is None else seed) * 7919 + 17)
    dt = spec.torch_dtype
    q = randn((S, Hq, D), dt, g, device)
    kv = fill_pool_(new_pool(L, NB, Hkv, B, D, dt, device), g)
    k_pool, v_pool = planes(kv)
    if poison_unused and not tables.used_blocks.all():
        unused = torch.from_numpy(np.nonzero(~tables.used_blocks)[0]).to(device)
        k_pool[:, unused] = float("nan")
        v_pool[:, unused] = float("nan")
    T = tables.slot_mapping.shape[0]
    new_key = randn((T, Hkv, D), dt, g, device)
    new_value = randn((T, Hkv, D), dt, g, device)
    return Batch(spec, tables, q, k_pool, v_pool, new_key, new_value,
                 torch.from_numpy(tables.block_tables).to(device),
                 torch.from_numpy(tables.context_lens).to(device),
                 torch.from_numpy(tables.slot_mapping).to(device), kv)
