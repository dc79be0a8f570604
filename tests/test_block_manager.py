"""Block manager: the oracle model against the pages' printed allocator run and invariants; the
native library's block manager against the model (host code, runs without a GPU)."""
import json
import os
import random

import pytest

from oracle.block_manager import BlockManagerModel, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "allocator_run.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_model_reproduces_the_printed_allocator_run():
    g = _golden()
    m = BlockManagerModel(g["num_blocks"], g["block_size"])
    assert g["num_blocks"] * g["block_size"] == g["capacity_tokens"]
    A, B = 0, 1
    s = g["steps"]
    assert m.allocate(A, s[0]["num_tokens"]) == s[0]["table_A"]
    assert m.num_free() == s[0]["free"]
    assert m.fork(A, B) == s[1]["table_B"]
    assert m.num_free() == s[1]["free"]
    slot, copy = m.append(A)
    assert m.table(A) == s[2]["table_A"] and m.table(B) == s[2]["table_B"]
    assert m.num_free() == s[2]["free"]
    # the 7th token of A (position 6) lands in slot 2 of the copied block; block 1 -> block 2
    assert copy == (1, 2) and slot == 2 * 4 + 2
    m.release(A)
    m.release(B)
    assert m.num_free() == s[3]["free"] == g["num_blocks"]


def test_on_demand_and_boundary_allocation_examples():
    # "a 25-token prompt with B = 16 allocates exactly 2 physical blocks"
    m = BlockManagerModel(8, 16)
    assert len(m.allocate(0, 25)) == 2
    # tokens 26..32 stay in block 1; the 33rd token crosses the boundary and pops block 2
    for _ in range(7):
        m.append(0)
    assert len(m.table(0)) == 2 and m.num_tokens(0) == 32
    slot, copy = m.append(0)
    assert m.table(0) == [0, 1, 2] and slot == 32 and copy is None


def test_full_shared_block_is_not_copied():
    m = BlockManagerModel(6, 4)
    m.allocate(0, 8)              # two full blocks
    m.fork(0, 1)
    slot, copy = m.append(0)      # position 8 opens a new block; nothing shared is modified
    assert copy is None and m.table(0) == [0, 1, 2] and m.table(1) == [0, 1] and slot == 8
    assert m.ref[0] == 2 and m.ref[1] == 2


def test_out_of_blocks_changes_nothing():
    m = BlockManagerModel(3, 4)
    m.allocate(0, 9)              # 3 blocks: pool exhausted
    before = (list(m.free), list(m.ref), m.table(0), m.num_tokens(0))
    with pytest.raises(OutOfBlocks):
        m.allocate(1, 1)
    for _ in range(3):
        m.append(0)               # positions 9..11 fit in block 2
    with pytest.raises(OutOfBlocks):
        m.append_batch([0])       # position 12 needs a fourth block
    assert m.table(0) == before[2] and m.num_tokens(0) == 12


def _check_invariants(m: BlockManagerModel):
    refs = [0] * m.num_blocks
    for s, t in m.tables.items():
        assert len(t) == -(-m.tokens[s] // m.block_size)           # exactly ceil(n/B) blocks
        assert len(t) * m.block_size - m.tokens[s] <= m.block_size - 1   # waste <= B - 1
        for b in t:
            refs[b] += 1
    assert refs == m.ref                                            # counts = table references
    assert sorted(m.free) == [b for b in range(m.num_blocks) if refs[b] == 0]


def _random_ops(seed, n_ops=400, num_blocks=64, block_size=4):
    rng = random.Random(seed)
    ops, live, nxt = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.15 or not live:
            ops.append(("allocate", nxt, rng.randint(0, 3 * block_size))); live.append(nxt); nxt += 1
        elif r < 0.25:
            ops.append(("fork", rng.choice(live), nxt)); live.append(nxt); nxt += 1
        elif r < 0.35:
            s = rng.choice(live); ops.append(("release", s)); live.remove(s)
        else:
            ops.append(("append", [rng.choice(live) for _ in range(rng.randint(1, 4))]))
    return ops


def _live(m, op):
    """False when the op names a sequence an earlier failed operation never created."""
    if op[0] == "allocate":
        return True
    if op[0] in ("fork", "release"):
        return op[1] in m.tables
    return all(s in m.tables for s in op[1])


def _apply(m, op):
    if not _live(m, op):
        return None
    kind = op[0]
    if kind == "allocate":
        return m.allocate(op[1], op[2])
    if kind == "fork":
        return m.fork(op[1], op[2])
    if kind == "release":
        return m.release(op[1])
    return m.append_batch(op[1])


@pytest.mark.parametrize("seed", range(6))
def test_model_invariants_under_random_operations(seed):
    m = BlockManagerModel(64, 4)
    for op in _random_ops(seed):
        try:
            _apply(m, op)
        except OutOfBlocks:
            pass
        _check_invariants(m)


@pytest.mark.parametrize("seed", range(6))
def test_copy_on_write_never_changes_what_other_sequences_read(seed):
    """Replaying the slot writes and block copies on a token-id 'pool' gives every sequence
    exactly its own token history (what the device pool must hold after reshape_and_cache and
    copy_blocks)."""
    B = 4
    m = BlockManagerModel(64, B)
    pool = {}            # slot -> token id
    history = {}         # seq -> token ids
    tok = 1000
    for op in _random_ops(seed):
        if not _live(m, op):
            continue
        try:
            if op[0] == "allocate":
                m.allocate(op[1], op[2])
                history[op[1]] = list(range(tok, tok + op[2]))
                for i, t in enumerate(history[op[1]]):
                    pool[m.table(op[1])[i // B] * B + i % B] = t
                tok += op[2]
            elif op[0] == "fork":
                m.fork(op[1], op[2])
                history[op[2]] = list(history[op[1]])
            elif op[0] == "release":
                m.release(op[1])
                del history[op[1]]
            else:
                slots, copies = m.append_batch(op[1])
                for src, dst in copies:         # device copies happen before the token writes
                    for i in range(B):
                        if src * B + i in pool:
                            pool[dst * B + i] = pool[src * B + i]
                for s, slot in zip(op[1], slots):
                    pool[slot] = tok
                    history[s].append(tok)
                    tok += 1
        except OutOfBlocks:
            continue
        for s, h in history.items():
            t = m.table(s)
            assert [pool[t[i // B] * B + i % B] for i in range(len(h))] == h


# ---- the library's native block manager against the model (host code, no GPU needed) ----

import numpy as np  # noqa: E402

import paged_kv_cache_452_amd as pkv  # noqa: E402


def test_native_reproduces_the_printed_allocator_run():
    g = _golden()
    bm = pkv.BlockManager(g["num_blocks"], g["block_size"])
    bm.allocate(0, 6)
    assert bm.tables([0], 4)[0][0, :2].tolist() == [0, 1] and bm.num_free == 8
    bm.fork(0, 1)
    assert bm.tables([1], 4)[0][0, :2].tolist() == [0, 1] and bm.num_free == 8
    slots, copies = bm.append([0])
    bt, cl = bm.tables([0, 1], 4)
    assert bt[0, :2].tolist() == [0, 2] and bt[1, :2].tolist() == [0, 1]
    assert bt[0, 2:].tolist() == [-1, -1] and cl.tolist() == [7, 6]
    assert copies.tolist() == [[1, 2]] and slots.tolist() == [10] and bm.num_free == 7
    bm.release(0)
    bm.release(1)
    assert bm.num_free == 10


def _native_apply(bm, op):
    kind = op[0]
    if kind == "allocate":
        return bm.allocate(op[1], op[2])
    if kind == "fork":
        return bm.fork(op[1], op[2])
    if kind == "release":
        return bm.release(op[1])
    return bm.append(op[1])


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("block_size", [4, 16])
def test_native_matches_model_on_random_operations(seed, block_size):
    """Same operations on both: identical slots, copies, tables, lengths, free counts and
    refusals."""
    m = BlockManagerModel(64, block_size)
    bm = pkv.BlockManager(64, block_size)
    for op in _random_ops(seed + 100 * block_size, block_size=block_size):
        if not _live(m, op):
            continue
        try:
            want = _apply(m, op)
            want_err = None
        except OutOfBlocks:
            want, want_err = None, pkv.PKV_ERR_NO_BLOCKS
        try:
            got = _native_apply(bm, op)
            got_err = None
        except pkv.PagedKVError as e:
            got, got_err = None, e.status
        assert got_err == want_err, op
        if op[0] == "append" and want_err is None:
            assert got[0].tolist() == want[0], op
            assert [tuple(c) for c in got[1].tolist()] == want[1], op
        assert bm.num_free == m.num_free()
        seqs = sorted(m.tables)
        if seqs:
            mb = max(1, max(len(t) for t in m.tables.values()))
            bt, cl = bm.tables(seqs, mb)
            for i, s in enumerate(seqs):
                t = m.table(s)
                assert bt[i].tolist() == t + [-1] * (mb - len(t))
                assert cl[i] == m.num_tokens(s)


def test_native_argument_errors():
    bm = pkv.BlockManager(8, 4)
    bm.allocate(5, 3)
    for fn, args in [(bm.allocate, (5, 1)), (bm.fork, (9, 10)), (bm.fork, (5, 5)),
                     (bm.release, (42,)), (bm.append, ([5, 77],))]:
        with pytest.raises(pkv.PagedKVError) as e:
            fn(*args)
        assert e.value.status == -1
    with pytest.raises(pkv.PagedKVError):
        bm.tables([5], 0)                 # table longer than the row
    with pytest.raises(pkv.PagedKVError):
        pkv.BlockManager(0, 4)
    assert bm.num_free == 7               # failed calls changed nothing
    lib = pkv.load_library()
    assert lib.kv_block_manager_num_free(None) == -1
    lib.kv_block_manager_destroy(None)
