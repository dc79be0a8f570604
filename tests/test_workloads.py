"""Host-side invariants of the seeded decode inputs (no GPU needed)."""
import numpy as np
import pytest
import torch

import workloads
from workloads import SPECS, append_step, make_tables


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_tables_are_valid_block_maps(idx):
    spec = SPECS[idx]
    t = make_tables(spec)
    B = spec.block_size
    S = t.context_lens.shape[0]
    assert S == spec.num_seqs
    owners = {}
    for s in range(S):
        n = int(t.context_lens[s])
        nb = -(-n // B)
        row = t.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < t.num_blocks)
        assert np.all(row[nb:] == -1)                      # padding never names a block
        waste = nb * B - n
        assert 0 <= waste <= B - 1                         # at most B-1 empty slots
        for j, b in enumerate(row[:nb]):
            owners.setdefault(int(b), []).append((s, j))
    shared = [b for b, o in owners.items() if len(o) > 1]
    if idx == 5:
        # 50 requests share the same 50 blocks (800-token prefix) at logical blocks 0..49
        assert len(shared) == 50
        for b in shared:
            o = owners[b]
            assert len(o) == 50 and len({j for _, j in o}) == 1 and {s for s, _ in o} == set(range(50))
    else:
        assert shared == []
    # slots: one per sequence at position n-1, distinct, inside the sequence's own block
    slots = t.slot_mapping
    assert len(set(slots.tolist())) == len(slots)
    for s in range(S):
        n = int(t.context_lens[s])
        assert slots[s] == t.block_tables[s, (n - 1) // B] * B + (n - 1) % B
    used = np.zeros(t.num_blocks, bool)
    used[list(owners)] = True
    assert np.array_equal(used, t.used_blocks)


def test_workload_shapes():
    t1 = make_tables(SPECS[1])
    assert t1.context_lens.tolist() == [1, 15, 16, 41] and t1.num_blocks == 64
    t2 = make_tables(SPECS[2])
    assert t2.context_lens.min() >= 128 and t2.context_lens.max() <= 2048
    need2 = sum(-(-int(n) // 16) for n in t2.context_lens)
    assert t2.num_blocks == int(np.ceil(need2 * 1.5))
    t3 = make_tables(SPECS[3])
    assert t3.context_lens.min() >= 1024 and t3.context_lens.max() <= 8192
    t4 = make_tables(SPECS[4])
    assert t4.num_blocks == 16384 and t4.used_blocks.all()
    assert np.array_equal(np.sort(t4.block_tables.ravel()), np.arange(16384))
    t5 = make_tables(SPECS[5])
    lens = t5.context_lens
    assert lens[50] == 32768 and np.all((lens[:50] >= 816) & (lens[:50] <= 1312))
    assert np.all((lens[51:] >= 64) & (lens[51:] <= 256))


def test_seeded_and_reproducible():
    a = make_tables(SPECS[3])
    b = make_tables(SPECS[3])
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.context_lens, b.context_lens)
    c = make_tables(SPECS[3], seed=1)
    assert not np.array_equal(a.block_tables, c.block_tables)


def test_append_step_allocates_on_block_boundary():
    t = make_tables(SPECS[1])
    used_before = int(t.used_blocks.sum())
    t2 = append_step(t)
    assert t2.context_lens.tolist() == [2, 16, 17, 42]
    # only the 16-token sequence crossed into a new block
    assert int(t2.used_blocks.sum()) == used_before + 1
    assert t2.block_tables[2, 1] >= 0 and t.block_tables[2, 1] == -1
    assert t2.slot_mapping[2] == t2.block_tables[2, 1] * 16 + 0
    assert t2.slot_mapping[0] == t.block_tables[0, 0] * 16 + 1
    assert len(set(t2.slot_mapping.tolist())) == 4


def test_free_list_exhaustion_raises_memory_error():
    rng = np.random.default_rng(0)
    fl = workloads.FreeList(2, rng)
    fl.pop()
    fl.pop()
    with pytest.raises(MemoryError):
        fl.pop()


def test_make_batch_cpu_small():
    spec = SPECS[1]
    b = workloads.make_batch(spec)
    assert b.k_pool.shape == (1, 64, 4, 16 * 64)
    assert b.q.shape == (4, 4, 64)
    unused = ~b.tables.used_blocks
    assert b.k_pool[0, unused].isnan().all() and not b.k_pool[0, ~unused].isnan().any()
    b2 = workloads.make_batch(spec)
    assert b.q.equal(b2.q) and b.new_key.equal(b2.new_key)


def test_random_e4m3_codes_are_finite_and_bounded():
    import oracle
    g = torch.Generator().manual_seed(3)
    c = workloads.random_e4m3_codes(1 << 16, g, "cpu").numpy()
    assert c.dtype == np.uint8
    assert not np.any((c & 0x7F) == 0x7F), "NaN code drawn"
    vals = np.array([oracle.e4m3_value(int(x)) for x in range(256)])
    v = vals[c]
    assert np.all(np.isfinite(v)) and np.max(np.abs(v)) <= 3.75
    assert len(np.unique(c)) == 2 * 9 * 8      # every sign / exponent 0..8 / mantissa drawn
