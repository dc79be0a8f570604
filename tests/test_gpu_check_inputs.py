"""GPU: paged_attention_check_inputs, the debug check of a step's index inputs. Its four counts
(used table entries outside the pool, context lengths out of range, repeated slots, slots past
the pool) must equal a host count of the same rules exactly: on clean batches (all zero), on
planted errors, and on seeded random corruption. It never reads the pool, so the planted errors
cannot fault the device."""
import numpy as np
import pytest
import torch

import paged_kv_cache_452_amd as pkv
import workloads
from helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
KEYS = ("bad_table_entries", "bad_context_lens", "repeated_slots", "slots_past_pool")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def host_counts(tables, lens, max_ctx, B, NB, slots):
    """The header's rules, counted on the host."""
    S, max_blocks = tables.shape
    row = max_blocks * B
    bad_lens = sum(1 for n in lens if n < 0 or n > min(max_ctx, row))
    bad_entries = 0
    for s, n in enumerate(lens):
        used = -(-min(max(int(n), 0), row) // B)
        e = tables[s, :used]
        bad_entries += int(((e < 0) | (e >= NB)).sum())
    seen, repeats, past = set(), 0, 0
    for x in (slots if slots is not None else []):
        x = int(x)
        past += x >= NB * B
        if x >= 0:
            repeats += x in seen
            seen.add(x)
    return dict(zip(KEYS, (bad_entries, bad_lens, repeats, past)))


def gpu_counts(tables, lens, NB, B, max_ctx, slots):
    return pkv.paged_attention_check_inputs(
        torch.from_numpy(np.ascontiguousarray(tables, np.int32)).to(DEV),
        torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(DEV), NB, B, max_ctx,
        None if slots is None else torch.from_numpy(np.ascontiguousarray(slots, np.int64)).to(DEV))


def test_clean_batches_have_no_violations():
    for idx in (1, 3, 5):
        spec = workloads.SPECS[idx]
        t = workloads.make_tables(spec)
        max_ctx = int(t.context_lens.max())
        got = gpu_counts(t.block_tables, t.context_lens, t.num_blocks, spec.block_size, max_ctx,
                         t.slot_mapping)
        say("check inputs, clean", spec.name, got)
        assert got == dict.fromkeys(KEYS, 0)


def test_planted_violations_are_counted():
    spec = workloads.SPECS[3]
    t = workloads.make_tables(spec)
    B, NB = spec.block_size, t.num_blocks
    tables, lens, slots = t.block_tables.copy(), t.context_lens.copy(), t.slot_mapping.copy()
    max_ctx = int(lens.max())
    tables[0, 0] = NB              # used entries outside the pool
    tables[1, 3] = -1
    tables[2, 5] = 2 ** 31 - 1
    used7 = -(-int(lens[7]) // B)
    if used7 < tables.shape[1]:
        tables[7, used7] = NB + 5  # past the used entries: not counted
    lens[10] = -3                  # out-of-range lengths
    lens[11] = max_ctx + 1
    slots[4] = slots[9]            # two repeats of one slot, one of another
    slots[5] = slots[9]
    slots[20] = slots[21]
    slots[30] = NB * B + 7         # past the pool
    slots[31] = -1                 # skipped: neither repeated nor past
    want = host_counts(tables, lens, max_ctx, B, NB, slots)
    assert want["bad_table_entries"] >= 3 and want["bad_context_lens"] == 2
    assert want["repeated_slots"] == 3 and want["slots_past_pool"] == 1
    got = gpu_counts(tables, lens, NB, B, max_ctx, slots)
    say("check inputs, planted", got)
    assert got == want


@pytest.mark.parametrize("seed", range(12))
def test_random_corruption_counts_match_the_host(seed):
    rng = np.random.default_rng(4200 + seed)
    S = int(rng.choice([1, 7, 64, 300, 2048]))
    B = int(rng.choice([16, 32]))
    NB = int(rng.integers(16, 5000))
    max_blocks = int(rng.integers(1, 40))
    max_ctx = int(rng.integers(0, max_blocks * B + 1))
    lens = rng.integers(-2, max_blocks * B + 3, size=S).astype(np.int32)
    tables = rng.integers(0, NB, size=(S, max_blocks)).astype(np.int32)
    bad = rng.random(tables.shape) < 0.02
    tables[bad] = rng.choice([-1, NB, NB + 1, -(2 ** 31), 2 ** 31 - 1], size=int(bad.sum()))
    T = int(rng.integers(0, 3000))
    slots = rng.integers(-1, NB * B + 10, size=T).astype(np.int64) if T else None
    want = host_counts(tables, lens, max_ctx, B, NB, slots)
    got = gpu_counts(tables, lens, NB, B, max_ctx, slots)
    say("check inputs, random", seed, f"S={S} B={B} NB={NB} T={T}", got)
    assert got == want


def test_prefill_sized_slot_mapping():
    """20,000 slots of one long sequence (the search runs over LDS tiles of 256 earlier slots):
    repeats planted across tile edges, far apart and at the very end, plus skipped and
    past-the-pool slots, counted exactly as the host counts them."""
    T, B = 20000, 16
    NB = T // B + 4
    lens = np.array([T], np.int32)
    tables = np.arange(NB - 4, dtype=np.int32)[None]
    slots = np.arange(T, dtype=np.int64)
    for dst, src in ((256, 255), (512, 0), (4096, 4095), (19999, 7), (12345, 12344),
                     (767, 511)):
        slots[dst] = slots[src]
    slots[100] = -1
    slots[300] = NB * B + 3
    slots[301] = NB * B + 3  # past the pool and a repeat
    want = host_counts(tables, lens, T, B, NB, slots)
    assert want["repeated_slots"] == 7 and want["slots_past_pool"] == 2
    got = gpu_counts(tables, lens, NB, B, T, slots)
    say("check inputs, prefill-sized", got)
    assert got == want


def test_empty_inputs():
    got = gpu_counts(np.zeros((0, 4), np.int32), np.zeros(0, np.int32), 10, 16, 64, None)
    assert got == dict.fromkeys(KEYS, 0)
    # zero-width tables: only the lengths are checked
    got = gpu_counts(np.zeros((3, 0), np.int32), np.array([0, 1, 0], np.int32), 10, 16, 0, None)
    assert got == dict(bad_table_entries=0, bad_context_lens=1, repeated_slots=0,
                       slots_past_pool=0)
