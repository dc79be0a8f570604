"""GPU parity: the HIP path against the fp64 oracle on the five decode workloads and edge cases.

Bar: reshape_and_cache and all indexing bit-exact (whole-pool word compare); attention outputs
within max-abs 1e-2 and relative L2 2e-3 of the oracle.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import helpers
import oracle
import paged_kv_cache_452_amd as pkv
import workloads
from helpers import (LayerHost, assert_close, gpu_decode, oracle_decode, poison_dead_slots_, say,
                     set_plane_, words)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def _layer(batch, L=0):
    return batch.k_pool[L], batch.v_pool[L]


def _step(batch, layer=0, poison=True):
    """One decode step on one layer: reshape_and_cache of the new tokens, then decode.
    Returns (gpu_out, oracle_out, pools bit-exact flag)."""
    spec, t = batch.spec, batch.tables
    k, v = _layer(batch, layer)
    if poison:
        poison_dead_slots_(k, v, t.block_tables, t.context_lens, spec.num_kv_heads, spec.head_dim)
    kw, vw = words(k), words(v)
    # oracle side: host scatter on the host copy
    oracle.reshape_and_cache(kw, vw, batch.new_key.cpu(), batch.new_value.cpu(), t.slot_mapping,
                             spec.num_kv_heads, spec.head_dim, 16, t.num_blocks)
    say("reshape_and_cache", spec.name, "layer", layer)
    pkv.reshape_and_cache(batch.new_key, batch.new_value, k, v, batch.slot_mapping, t.num_blocks)
    torch.cuda.synchronize()
    assert np.array_equal(words(k), kw), "K pool differs after reshape_and_cache"
    assert np.array_equal(words(v), vw), "V pool differs after reshape_and_cache"
    say("decode", spec.name, "layer", layer)
    out = gpu_decode(batch.q, k, v, batch.block_tables, batch.context_lens, spec.scale,
                     spec.num_q_heads, spec.num_kv_heads, batch.max_context_len)
    torch.cuda.synchronize()
    ref = oracle_decode(batch.q, k, v, t.block_tables, t.context_lens, spec.scale,
                        spec.num_q_heads, spec.num_kv_heads, t.num_blocks, k_words=kw, v_words=vw)
    return out, ref


@pytest.mark.parametrize("idx", [1, 2, 3, 5])
def test_decode_step_matches_oracle(idx):
    spec = workloads.SPECS[idx]
    batch = workloads.make_batch(spec, device=DEV)
    out, ref = _step(batch)
    assert_close(out, ref, spec.name)


def test_tiny_batch_two_steps_cross_block_boundary():
    spec = workloads.SPECS[1]
    batch = workloads.make_batch(spec, device=DEV)
    out, ref = _step(batch)
    assert_close(out, ref, "step 1")
    t2 = workloads.append_step(batch.tables)
    assert t2.context_lens.tolist() == [2, 16, 17, 42]
    g = torch.Generator(device=DEV).manual_seed(99)
    b2 = dataclasses.replace(
        batch, tables=t2,
        q=workloads.randn(batch.q.shape, batch.q.dtype, g, DEV),
        new_key=workloads.randn(batch.new_key.shape, batch.q.dtype, g, DEV),
        new_value=workloads.randn(batch.new_value.shape, batch.q.dtype, g, DEV),
        block_tables=torch.from_numpy(t2.block_tables).to(DEV),
        context_lens=torch.from_numpy(t2.context_lens).to(DEV),
        slot_mapping=torch.from_numpy(t2.slot_mapping).to(DEV))
    out2, ref2 = _step(b2, poison=False)
    assert_close(out2, ref2, "step 2")


LAYER_CHUNK = 10   # layers per test of the full-size checks (each test stays well under a minute)


@pytest.fixture(scope="module")
def batch70():
    """The 70B-shaped batch (64 x 4096 tokens, 64/8 heads, d128, bf16, 80 layers in one 80 GiB
    pool), built once for the full-size checks of this module."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    spec = workloads.SPECS[4]
    t = workloads.make_tables(spec)
    say("70B-shaped batch: allocating and filling 2 x 40 GiB")
    batch = workloads.make_batch(spec, device=DEV, tables=t)
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(S, Hq, Hkv, D, 16, 4096), DEV)
    yield spec, t, batch, LayerHost(batch.kv_pool[0]), ws
    del batch, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("first", range(0, 80, LAYER_CHUNK))
def test_70b_shaped_step_every_layer_and_row(batch70, first):
    """The benchmark's workload and step, checked in full (10 layers per test, all 80 over the
    set): for each layer, reshape_and_cache of the 64 new tokens (the whole layer's K and V planes
    equal the oracle's scatter word for word) then decode (every (sequence, head) row against the
    oracle)."""
    spec, t, batch, host, ws = batch70
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    out = torch.empty_like(batch.q)
    key, value = batch.new_key.cpu(), batch.new_value.cpu()
    for L in range(first, first + LAYER_CHUNK):
        kw, vw = host.planes(batch.kv_pool[L])
        oracle.reshape_and_cache(kw, vw, key, value, t.slot_mapping, Hkv, D, 16, t.num_blocks)
        say("70B-shaped step, layer", L)
        k, v = _layer(batch, L)
        pkv.reshape_and_cache(batch.new_key, batch.new_value, k, v, batch.slot_mapping,
                              t.num_blocks)
        pkv.paged_attention_decode(out, batch.q, k, v, batch.block_tables, batch.context_lens,
                                   spec.scale, Hq, Hkv, D, 16, 4096, 0, ws)
        torch.cuda.synchronize()
        assert host.equals(batch.kv_pool[L], kw, vw), f"layer {L}: pool differs after reshape"
        ref = oracle_decode(batch.q, None, None, t.block_tables, t.context_lens, spec.scale, Hq,
                            Hkv, t.num_blocks, k_words=kw, v_words=vw)
        assert_close(out, ref, f"layer {L}")


@pytest.mark.parametrize("first", range(0, 80, LAYER_CHUNK))
def test_fused_append_70b_shaped_every_layer_and_row(batch70, first):
    """The fused step on the 70B-shaped batch, checked in full (10 layers per test): the new
    tokens' slots are NaN before each launch; after it, the layer's K and V planes equal the
    oracle's scatter word for word and every (sequence, head) row matches the oracle."""
    spec, t, batch, host, ws = batch70
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    out = torch.empty_like(batch.q)
    key, value = batch.new_key.cpu(), batch.new_value.cpu()
    for L in range(first, first + LAYER_CHUNK):
        _poison_new_slots_(batch.k_pool[L], batch.v_pool[L], t, Hkv, D, 16)
        kw, vw = host.planes(batch.kv_pool[L])
        oracle.reshape_and_cache(kw, vw, key, value, t.slot_mapping, Hkv, D, 16, t.num_blocks)
        say("fused step, 70B-shaped batch, layer", L)
        pkv.paged_attention_decode_append(out, batch.q, batch.new_key, batch.new_value,
                                          batch.k_pool[L], batch.v_pool[L], batch.block_tables,
                                          batch.context_lens, spec.scale, Hq, Hkv, D, 16, 4096, 0,
                                          ws)
        torch.cuda.synchronize()
        assert host.equals(batch.kv_pool[L], kw, vw), f"layer {L}: pool differs"
        ref = oracle_decode(batch.q, None, None, t.block_tables, t.context_lens, spec.scale, Hq,
                            Hkv, t.num_blocks, k_words=kw, v_words=vw)
        assert_close(out, ref, f"fused layer {L}")


def _random_case(Hq, Hkv, D, lens, dtype=torch.bfloat16, seed=0, extra_blocks=7, block_size=16):
    """A small paged batch with NaN-poisoned unused blocks and dead slots."""
    lens = np.asarray(lens, np.int32)
    spec = workloads.Spec(0, f"case Hq={Hq} Hkv={Hkv} D={D} B={block_size} lens={lens.tolist()}",
                          len(lens), Hq, Hkv, D, "bf16" if dtype == torch.bfloat16 else "fp16", 1,
                          seed=seed, block_size=block_size)
    need = sum(-(-int(n) // block_size) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=max(need + extra_blocks, 1), seed=seed)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    k, v = _layer(b)
    poison_dead_slots_(k, v, t.block_tables, t.context_lens, Hkv, D, block_size)
    return spec, t, b


@pytest.mark.parametrize("Hq,Hkv,D,dtype,lens", [
    (8, 8, 128, torch.bfloat16, [1, 2, 15, 16, 17, 31, 32, 33]),       # MHA, ragged tails
    (32, 8, 128, torch.float16, [100, 257, 1000]),                      # GQA fp16
    (12, 4, 64, torch.bfloat16, [5, 64, 65, 300]),                      # group of 3, d64
    (64, 2, 128, torch.bfloat16, [40, 513]),                            # group of 32: 2 head tiles
    (16, 1, 64, torch.float16, [2049]),                                 # MQA, many blocks
    (4, 4, 64, torch.bfloat16, [0, 3, 0, 16]),                          # empty sequences
])
def test_edge_shapes(Hq, Hkv, D, dtype, lens):
    spec, t, b = _random_case(Hq, Hkv, D, lens, dtype, seed=len(lens) * 7 + Hq)
    k, v = _layer(b)
    say("edge", spec.name)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv,
                     max(int(max(lens)), 1))
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks)
    assert_close(out, ref, spec.name)
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[s]).item() == 0


@pytest.mark.parametrize("num_workgroups", [1, 2, 3, 7, 64, 500, 2000, 0])
def test_workgroup_counts_agree_with_oracle(num_workgroups):
    """Any number of workgroups gives the oracle's result: 1 (no stream split), a few (long
    ranges crossing many streams), many more than positions (most streams cut into one-block
    pieces merged by the last arriver)."""
    spec, t, b = _random_case(32, 8, 128, [1, 255, 256, 257, 1500, 4000], seed=11)
    k, v = _layer(b)
    say("workgroups", num_workgroups)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, 4000,
                     num_workgroups)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 32, 8,
                        t.num_blocks)
    assert_close(out, ref, f"{num_workgroups} workgroups")


def test_workspace_counters_return_to_zero_and_reuse():
    """The arrival counters are left zero by every call, so one workspace serves call after call
    (different batches, different workgroup counts) with identical results."""
    spec, t, b = _random_case(32, 8, 128, [3000, 17, 900, 4096, 1], seed=14)
    k, v = _layer(b)
    G = 300
    nbytes = pkv.paged_attention_workspace_bytes(5, 32, 8, 128, 16, 4096, G)
    ws = pkv.new_workspace(nbytes, DEV)
    counters = ws[-G:]   # the last G words; calls with fewer workgroups use a suffix of them
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 32, 8,
                        t.num_blocks)
    first = None
    for rep, g in enumerate([G, G, 77, G]):
        say("reuse", rep, g)
        out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, 4096, g,
                         workspace=ws)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(counters).item()) == 0, "counters not reset"
        assert_close(out, ref, f"reuse {rep}")
        if g == G:
            if first is None:
                first = out.clone()
            else:
                assert torch.equal(first.view(torch.int16), out.view(torch.int16))


def test_long_sequence_spread_over_workgroups():
    spec, t, b = _random_case(32, 8, 128, [32768, 100], seed=12)
    k, v = _layer(b)
    for g in (1, 16, 0):
        say("long sequence, workgroups", g)
        out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, 32768, g)
        torch.cuda.synchronize()
        ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 32, 8,
                            t.num_blocks)
        assert_close(out, ref, f"32k, {g} workgroups")


def test_max_context_fills_block_table():
    lens = [64 * 16, 64 * 16 - 1]
    spec, t, b = _random_case(8, 2, 128, lens, seed=13)
    assert t.block_tables.shape[1] == 64
    k, v = _layer(b)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 8, 2, 64 * 16)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 8, 2,
                        t.num_blocks)
    assert_close(out, ref, "max context")


@pytest.mark.parametrize("Hq,Hkv,D,dtype,lens,nwg", [
    (32, 8, 128, torch.bfloat16, [1, 16, 17, 31, 32, 33, 500, 4097], 0),   # ragged sub-tiles
    (8, 8, 64, torch.float16, [63, 64, 65, 1000], 0),
    (32, 8, 128, torch.bfloat16, [3000, 7, 32 * 40], 200),                 # many split streams
    (64, 2, 128, torch.bfloat16, [33, 2049], 3),
])
def test_block_size_32_decode(Hq, Hkv, D, dtype, lens, nwg):
    """Block size 32: a block holds two 16-token sub-tiles; decode walks them through the table."""
    spec, t, b = _random_case(Hq, Hkv, D, lens, dtype, seed=len(lens) + D, block_size=32)
    k, v = _layer(b)
    say("block size 32", spec.name, nwg)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv,
                     int(max(lens)), nwg, block_size=32)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks, block_size=32)
    assert_close(out, ref, spec.name)


@pytest.mark.parametrize("D", [64, 128])
def test_block_size_32_reshape_and_cache_bit_exact(D):
    lens = [1, 16, 17, 32, 33, 64, 90]
    spec, t, b = _random_case(8, 4, D, lens, seed=D, block_size=32)
    k, v = _layer(b)
    kw, vw = words(k), words(v)
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), t.slot_mapping, 4, D, 32,
                             t.num_blocks)
    say("reshape block size 32", D)
    pkv.reshape_and_cache(b.new_key, b.new_value, k, v, b.slot_mapping, t.num_blocks, 32)
    torch.cuda.synchronize()
    assert np.array_equal(words(k), kw) and np.array_equal(words(v), vw)


def test_reshape_and_cache_skips_negative_and_past_pool_slots():
    spec, t, b = _random_case(4, 2, 128, [5, 9, 20, 33], seed=31)
    k, v = _layer(b)
    sm = b.slot_mapping.clone()
    sm[0] = -1
    sm[2] = t.num_blocks * 16      # first slot past the sub-pool: skipped
    kw, vw = words(k), words(v)
    sm_oracle = sm.cpu().clone()
    sm_oracle[2] = -1
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), sm_oracle, 2, 128, 16,
                             t.num_blocks)
    say("reshape negative and past-pool slots")
    pkv.reshape_and_cache(b.new_key, b.new_value, k, v, sm, t.num_blocks)
    torch.cuda.synchronize()
    assert np.array_equal(words(k), kw) and np.array_equal(words(v), vw)


# ---- One fused step: paged_attention_decode_append = reshape_and_cache + decode ----

def _new_slots(t, B):
    """Slot of each sequence's newest token (position n - 1), -1 for empty sequences."""
    return np.array([int(t.block_tables[s][(int(n) - 1) // B]) * B + (int(n) - 1) % B if n > 0
                     else -1 for s, n in enumerate(t.context_lens)], np.int64)


def _poison_new_slots_(k, v, t, Hkv, D, B):
    """NaN into the slot each sequence's new token goes to: the fused launch must write the token
    there before it reads the slot's tile, or the NaN reaches the output."""
    slots = _new_slots(t, B)
    for plane, is_v in ((k, False), (v, True)):
        idx = oracle.slot_indices(is_v, False, slots, Hkv, B, D)
        set_plane_(plane, torch.from_numpy(idx).to(plane.device), float("nan"))


@pytest.mark.parametrize("Hq,Hkv,D,dtype,lens,B,nwg", [
    (8, 8, 128, torch.bfloat16, [1, 2, 15, 16, 17, 31, 32, 33], 16, 0),   # n = 1: only the new token
    (32, 8, 128, torch.float16, [100, 257, 1000], 16, 0),
    (12, 4, 64, torch.bfloat16, [5, 64, 65, 300], 16, 0),
    (64, 2, 128, torch.bfloat16, [40, 513], 16, 3),                        # 2 head tiles, split
    (4, 4, 64, torch.bfloat16, [0, 3, 0, 1, 16], 16, 0),                   # empty sequences
    (32, 8, 128, torch.bfloat16, [3000, 7, 32 * 40 + 1, 17], 16, 200),     # many split streams
    (32, 8, 128, torch.bfloat16, [1, 16, 17, 32, 33, 500, 4097], 32, 0),
    (16, 1, 64, torch.float16, [2049, 2], 32, 5),
])
def test_fused_append_decode_matches_oracle(Hq, Hkv, D, dtype, lens, B, nwg):
    spec, t, b = _random_case(Hq, Hkv, D, lens, dtype, seed=len(lens) * 3 + Hq + B, block_size=B)
    k, v = _layer(b)
    _poison_new_slots_(k, v, t, Hkv, D, B)
    kw, vw = words(k), words(v)
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), t.slot_mapping, Hkv, D, B,
                             t.num_blocks)
    ref = oracle_decode(b.q, None, None, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks, k_words=kw, v_words=vw, block_size=B)
    maxc = max(int(max(lens)), 1)
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(len(lens), Hq, Hkv, D, B, maxc,
                                                               nwg), DEV)
    out = torch.empty_like(b.q)
    say("fused append", spec.name, nwg)
    pkv.paged_attention_decode_append(out, b.q, b.new_key, b.new_value, k, v, b.block_tables,
                                      b.context_lens, spec.scale, Hq, Hkv, D, B, maxc, nwg, ws)
    torch.cuda.synchronize()
    assert_close(out, ref, spec.name)
    assert np.array_equal(words(k), kw), "K pool differs from reshape_and_cache's"
    assert np.array_equal(words(v), vw), "V pool differs from reshape_and_cache's"
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[s]).item() == 0
        if n == 1:   # softmax over one token: the output is its value row, exactly
            g = torch.arange(Hq, device=DEV) // (Hq // Hkv)
            assert torch.equal(out[s].view(torch.int16), b.new_value[s][g].view(torch.int16))


@pytest.mark.parametrize("table,n", [
    ([7, 3, 9], 41),    # tokens 0..40 in physical blocks 7, 3, 9; the last block 9/16 full
    ([7, 2, 19], 48),   # tokens 0..47 in physical blocks 7, 2, 19; every block full
])
def test_block_tables_of_the_pages(table, n):
    """The two block tables the pages draw ("KV-Cache Management and PagedAttention", section
    "PagedAttention: treat the cache like virtual memory": tokens 0..40 in blocks [7, 3, 9];
    "PagedAttention and KV Cache Management", section "PagedAttention: OS Virtual Memory
    Architecture for GPUs": logical blocks 0, 1, 2 in physical blocks 7, 2, 19), in a 64-block
    pool with NaN in every other block and in the dead slots of the last block. The step's token
    (position n - 1) goes in by reshape_and_cache, checked against the oracle's scatter over the
    whole pool, then the decode is checked against the oracle (4/4 heads, d64, bf16)."""
    Hq = Hkv = 4
    D, NB, B = 64, 64, 16
    spec = workloads.Spec(0, f"page table {table}, {n} tokens", 1, Hq, Hkv, D, "bf16", 1,
                          seed=sum(table) + n)
    bt = np.array([table], np.int32)
    lens = np.array([n], np.int32)
    used = np.zeros(NB, bool)
    used[table] = True
    slot = np.array([table[(n - 1) // B] * B + (n - 1) % B], np.int64)
    t = workloads.Tables(lens, bt, NB, slot, used)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    assert torch.isnan(b.k_pool[0][~torch.from_numpy(used).to(DEV)]).all()
    k, v = _layer(b)
    poison_dead_slots_(k, v, bt, lens, Hkv, D)
    kw, vw = words(k), words(v)
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), slot, Hkv, D, B, NB)
    say("page table", table, n)
    pkv.reshape_and_cache(b.new_key, b.new_value, k, v, b.slot_mapping, NB)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv, n)
    torch.cuda.synchronize()
    assert np.array_equal(words(k), kw) and np.array_equal(words(v), vw)
    ref = oracle_decode(b.q, None, None, bt, lens, spec.scale, Hq, Hkv, NB, k_words=kw,
                        v_words=vw)
    assert_close(out, ref, spec.name)


def test_max_sequences_per_launch():
    """2048 sequences (the most one launch plans for), ragged short contexts, some empty."""
    rng = np.random.default_rng(2048)
    lens = rng.integers(0, 70, size=2048).astype(np.int32)
    lens[::97] = 0
    spec, t, b = _random_case(8, 2, 64, lens, seed=77, extra_blocks=3)
    k, v = _layer(b)
    say("2048 sequences")
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 8, 2, int(lens.max()))
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 8, 2, t.num_blocks)
    assert_close(out, ref, "2048 sequences")
    assert torch.count_nonzero(out[lens == 0]).item() == 0


@pytest.mark.parametrize("nwg", [0, 5])
def test_wide_group_many_head_tiles(nwg):
    """128 query heads on one kv head: 8 head tiles per (sequence, kv head), each its own stream
    over the same tiles."""
    spec, t, b = _random_case(128, 1, 128, [300, 17, 1024], seed=128)
    k, v = _layer(b)
    say("128/1 heads", nwg)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 128, 1, 1024, nwg)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 128, 1,
                        t.num_blocks)
    assert_close(out, ref, spec.name)


@pytest.mark.parametrize("num_workgroups", [0, 37, 300])
def test_split_streams_are_deterministic(num_workgroups):
    """Split streams are merged by whichever of their workgroups arrives last (directly from its
    combine buffer when all others are in, else after storing its own part): repeated launches,
    whose arrival orders differ, must give bit-identical outputs, and the oracle's values."""
    spec, t, b = _random_case(32, 8, 128, [4000, 17, 900, 2500, 1, 333], seed=91)
    k, v = _layer(b)
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(6, 32, 8, 128, 16, 4000,
                                                               num_workgroups), DEV)
    say("determinism", num_workgroups)
    first = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, 4000,
                       num_workgroups, workspace=ws).clone()
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 32, 8,
                        t.num_blocks)
    assert_close(first, ref, f"{num_workgroups} workgroups")
    for rep in range(12):
        out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, 4000,
                         num_workgroups, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"rep {rep}"


def test_default_grid_halves_for_few_uneven_streams():
    """128 (sequence, kv head) streams of uneven lengths, enough blocks for the full default grid
    (two workgroups per compute unit): the kernel runs them on the first half of that grid. The
    result must match the oracle and equal, bit for bit, an explicit grid of that half size."""
    lens = np.random.default_rng(31).integers(2000, 8001, size=16)
    spec, t, b = _random_case(32, 8, 128, lens.tolist(), seed=31)
    k, v = _layer(b)
    S, maxc = len(lens), int(lens.max())
    full = pkv.paged_attention_num_workgroups(S, 32, 8, maxc, 16)
    assert full == 2 * torch.cuda.get_device_properties(0).multi_processor_count
    say("halved default grid", full)
    out_default = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, maxc)
    out_half = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 32, 8, maxc,
                          full // 2)
    torch.cuda.synchronize()
    assert torch.equal(out_default.view(torch.int16), out_half.view(torch.int16))
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, 32, 8,
                        t.num_blocks)
    assert_close(out_default, ref, "halved default grid")


def test_fused_append_on_halved_default_grid():
    """The fused step on a batch that runs on half of the default grid: outputs match the oracle
    and the pools equal the oracle's scatter word for word (the exiting half writes nothing, the
    working half writes every new token)."""
    lens = np.random.default_rng(37).integers(2000, 8001, size=16)
    spec, t, b = _random_case(32, 8, 128, lens.tolist(), seed=37)
    k, v = _layer(b)
    _poison_new_slots_(k, v, t, 8, 128, 16)
    kw, vw = words(k), words(v)
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), t.slot_mapping, 8, 128,
                             16, t.num_blocks)
    ref = oracle_decode(b.q, None, None, t.block_tables, t.context_lens, spec.scale, 32, 8,
                        t.num_blocks, k_words=kw, v_words=vw)
    maxc = int(lens.max())
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(len(lens), 32, 8, 128, 16, maxc),
                           DEV)
    out = torch.empty_like(b.q)
    say("fused append on the halved default grid")
    pkv.paged_attention_decode_append(out, b.q, b.new_key, b.new_value, k, v, b.block_tables,
                                      b.context_lens, spec.scale, 32, 8, 128, 16, maxc, 0, ws)
    torch.cuda.synchronize()
    assert_close(out, ref, "fused append, halved grid")
    assert np.array_equal(words(k), kw), "K pool differs from reshape_and_cache's"
    assert np.array_equal(words(v), vw), "V pool differs from reshape_and_cache's"


@pytest.mark.parametrize("num_workgroups", [0, 1, 600])
def test_all_sequences_empty(num_workgroups):
    """Every context empty: no block positions at all. Each output row is zero (written over a
    non-zero fill), and the call completes with the default grid, one workgroup or many."""
    spec, t, b = _random_case(16, 4, 128, [0, 0, 0, 0, 0], seed=43)
    k, v = _layer(b)
    out = torch.full_like(b.q, 7.0)
    say("all sequences empty", num_workgroups)
    gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, 16, 4, 1, num_workgroups,
               out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("fp8", [False, True])
def test_70b_shaped_block_size_32_step_every_row(fp8):
    """The benchmark's block-size-32 workload (bench.py --block-size 32, with or without
    --kv-dtype fp8): the 70B-shaped batch with 8,192 blocks of 32 tokens per layer, two layers.
    For each layer, the step's scatter (whole K and V planes equal the oracle's, word for word or
    byte for byte) then decode (every (sequence, head) row against the oracle)."""
    spec = dataclasses.replace(workloads.SPECS[4], num_layers=2, block_size=32)
    t = workloads.make_tables(spec)
    B = 32
    say("70B-shaped batch, block size 32, fp8" if fp8 else "70B-shaped batch, block size 32")
    b = (workloads.make_batch_fp8 if fp8 else workloads.make_batch)(spec, device=DEV, tables=t)
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    ks, vs = 0.5, 0.5
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(S, Hq, Hkv, D, B, 4096), DEV)
    out = torch.empty_like(b.q)
    host = LayerHost(b.kv_pool[0])
    key, value = b.new_key.cpu(), b.new_value.cpu()
    for L in range(spec.num_layers):
        kw, vw = host.planes(b.kv_pool[L])
        if fp8:
            oracle.reshape_and_cache8(kw, vw, key, value, oracle.BF16, ks, vs, t.slot_mapping,
                                      Hkv, D, B, t.num_blocks)
            pkv.reshape_and_cache_fp8(b.new_key, b.new_value, b.k_pool[L], b.v_pool[L],
                                      b.slot_mapping, t.num_blocks, ks, vs, B)
            pkv.paged_attention_decode_fp8(out, b.q, b.k_pool[L], b.v_pool[L], b.block_tables,
                                           b.context_lens, spec.scale, ks, vs, Hq, Hkv, D, B,
                                           4096, 0, ws)
        else:
            oracle.reshape_and_cache(kw, vw, key, value, t.slot_mapping, Hkv, D, B, t.num_blocks)
            pkv.reshape_and_cache(b.new_key, b.new_value, b.k_pool[L], b.v_pool[L],
                                  b.slot_mapping, t.num_blocks, B)
            pkv.paged_attention_decode(out, b.q, b.k_pool[L], b.v_pool[L], b.block_tables,
                                       b.context_lens, spec.scale, Hq, Hkv, D, B, 4096, 0, ws)
        torch.cuda.synchronize()
        assert host.equals(b.kv_pool[L], kw, vw), f"layer {L}: pool differs after the scatter"
        if fp8:
            ref = helpers.oracle_decode8(b.q, kw, vw, t.block_tables, t.context_lens, spec.scale,
                                         ks, vs, Hq, Hkv, t.num_blocks, block_size=B)
        else:
            ref = oracle_decode(b.q, None, None, t.block_tables, t.context_lens, spec.scale, Hq,
                                Hkv, t.num_blocks, k_words=kw, v_words=vw, block_size=B)
        assert_close(out, ref, f"block size 32, layer {L}")
    del b, host, ws
    torch.cuda.empty_cache()


def test_planes_given_as_device_addresses():
    """The bindings take a layer's planes as tensors or as the device addresses kv_pool_layer
    gives. Both forms reach the same kernels: reshape_and_cache then decode on the last layer of
    a three-layer pool, once each way from the same starting pool, leave the same pool and give
    the same outputs bit for bit, and those match the oracle."""
    L, S, Hq, Hkv, D, B = 3, 6, 16, 4, 128, 16
    lens = np.array([1, 15, 16, 17, 300, 1000], np.int32)
    spec = workloads.Spec(0, "planes as addresses", S, Hq, Hkv, D, "bf16", L, seed=61)
    t = workloads.make_tables(spec, lens=lens, seed=61)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    for layer in range(L):
        poison_dead_slots_(b.k_pool[layer], b.v_pool[layer], t.block_tables, lens, Hkv, D)
    pool = pkv.kv_pool_create(b.kv_pool, b.kv_pool.numel() * 2, L, t.num_blocks, Hkv, D, B,
                              pkv.PKV_BF16)
    try:
        ka, va = pkv.kv_pool_layer(pool, L - 1)
    finally:
        pkv.kv_pool_destroy(pool)
    k, v = b.k_pool[L - 1], b.v_pool[L - 1]
    assert (ka, va) == (k.data_ptr(), v.data_ptr())
    start = b.kv_pool.clone()
    results = []
    for kk, vv in ((k, v), (ka, va)):
        b.kv_pool.copy_(start)
        say("planes as", "addresses" if isinstance(kk, int) else "views")
        pkv.reshape_and_cache(b.new_key, b.new_value, kk, vv, b.slot_mapping, t.num_blocks, B)
        out = torch.full_like(b.q, 3.0)
        ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(S, Hq, Hkv, D, B,
                                                                   int(lens.max()), 0), DEV)
        pkv.paged_attention_decode(out, b.q, kk, vv, b.block_tables, b.context_lens, spec.scale,
                                   Hq, Hkv, D, B, int(lens.max()), 0, ws)
        torch.cuda.synchronize()
        results.append((out, b.kv_pool.clone()))
    (o1, p1), (o2, p2) = results
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1.view(torch.int16), p2.view(torch.int16))
    ref = oracle_decode(b.q, k, v, t.block_tables, lens, spec.scale, Hq, Hkv, t.num_blocks)
    assert_close(o2, ref, "planes as device addresses")


def test_context_lengths_are_clamped_to_the_table_row():
    """The decode clamps each context length to [0, max_blocks_per_seq * block_size]: a negative
    length decodes like an empty sequence (zeros), and a length past the table row like the full
    row (here a row of full blocks). max_context_len only sizes the grid: lengths above it still
    decode to the oracle's result."""
    spec, t, b = _random_case(16, 4, 128, [304, 80, 40], seed=29)
    assert t.block_tables.shape[1] * 16 == 304          # sequence 0 fills its whole row
    k, v = _layer(b)
    given = torch.tensor([10000, 80, -7], dtype=torch.int32, device=DEV)
    meant = np.array([304, 80, 0], np.int32)
    say("clamped context lengths")
    got = gpu_decode(b.q, k, v, b.block_tables, given, spec.scale, 16, 4, 304)
    want = gpu_decode(b.q, k, v, b.block_tables, torch.from_numpy(meant).to(DEV), spec.scale, 16,
                      4, 304)
    small_hint = gpu_decode(b.q, k, v, b.block_tables, given, spec.scale, 16, 4, 16)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert not got[2].float().abs().any()
    ref = oracle_decode(b.q, k, v, t.block_tables, meant, spec.scale, 16, 4, t.num_blocks)
    assert_close(got, ref, "clamped lengths")
    assert_close(small_hint, ref, "lengths above max_context_len")
