"""GPU invariants that must hold bit for bit: nothing in the result may depend on where blocks sit
in the pool, on whether prefix blocks are shared, on what dead slots or table padding hold, or on
the run."""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close, gpu_decode, oracle_decode, poison_dead_slots_, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def _case(lens, Hq=32, Hkv=8, seed=21, extra=50):
    lens = np.asarray(lens, np.int32)
    spec = workloads.Spec(0, "invariants", len(lens), Hq, Hkv, 128, "bf16", 1, seed=seed)
    need = sum(-(-int(n) // 16) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + extra, seed=seed)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    return spec, t, b


def _run(spec, b, k, v, tables, pt=0):
    return gpu_decode(b.q, k, v, tables, b.context_lens, spec.scale, spec.num_q_heads,
                      spec.num_kv_heads, int(b.tables.context_lens.max()), pt)


def test_physical_block_permutation_gives_identical_output():
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 3000, size=12)
    spec, t, b = _case(lens)
    k, v = b.k_pool[0], b.v_pool[0]
    base = _run(spec, b, k, v, b.block_tables)
    perm = torch.from_numpy(rng.permutation(t.num_blocks)).to(DEV)
    kv2 = torch.empty_like(b.kv_pool[0])     # [blocks][kv heads][K, V][tile]
    kv2[perm] = b.kv_pool[0]
    k2, v2 = kv2.select(-2, 0), kv2.select(-2, 1)
    bt = b.block_tables.clone()
    valid = bt >= 0
    bt[valid] = perm[bt[valid].long()].int()
    say("permuted blocks")
    moved = _run(spec, b, k2, v2, bt)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_shared_prefix_equals_private_copies():
    spec = workloads.SPECS[5]
    t = workloads.make_tables(spec)
    P = t.shared_prefix_blocks
    extra = 49 * P
    b = workloads.make_batch(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    say("shared prefix")
    shared = _run(spec, b, k, v, b.block_tables)
    prefix = torch.from_numpy(t.block_tables[0, :P].astype(np.int64)).to(DEV)
    kv = b.kv_pool[0]
    kv2 = torch.cat([kv, kv[prefix].repeat(49, 1, 1, 1)])
    k2, v2 = kv2.select(-2, 0), kv2.select(-2, 1)
    bt = b.block_tables.clone()
    for s in range(1, 50):
        base = t.num_blocks + (s - 1) * P
        bt[s, :P] = torch.arange(base, base + P, dtype=torch.int32, device=DEV)
    assert k2.shape[0] == t.num_blocks + extra
    say("private copies")
    private = _run(spec, b, k2, v2, bt)
    torch.cuda.synchronize()
    assert torch.equal(shared.view(torch.int16), private.view(torch.int16))
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, spec.num_q_heads,
                        spec.num_kv_heads, t.num_blocks)
    assert_close(shared, ref, "shared-prefix batch")


def test_dead_slots_and_table_padding_are_never_read():
    rng = np.random.default_rng(41)
    lens = [17, 33, 250, 1, 1023]
    spec, t, b = _case(lens, extra=64)
    k, v = b.k_pool[0], b.v_pool[0]
    clean = _run(spec, b, k, v, b.block_tables)
    # NaN into every dead slot of every last block
    poison_dead_slots_(k, v, t.block_tables, t.context_lens, spec.num_kv_heads, spec.head_dim)
    # table padding -> ids of unused (NaN-filled) blocks: in range, so a stray read cannot fault
    unused = np.nonzero(~t.used_blocks)[0]
    bt = t.block_tables.copy()
    pad = bt < 0
    bt[pad] = rng.choice(unused, size=int(pad.sum()))
    say("poisoned dead slots + garbage padding")
    dirty = _run(spec, b, k, v, torch.from_numpy(bt).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16))


def test_repeat_runs_are_bit_identical():
    rng = np.random.default_rng(51)
    spec, t, b = _case(rng.integers(1, 5000, size=16))
    k, v = b.k_pool[0], b.v_pool[0]
    outs = [_run(spec, b, k, v, b.block_tables) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))
