"""GPU parity on seeded random shapes: sequence counts, GQA groups (including several head tiles
per kv head), head dims, block sizes, element types, context-length mixes with empty, short and
long sequences, and workgroup counts from 1 to many more than the chip holds. Each case is
checked against the fp64 oracle to the same bar as the fixed cases (max-abs 1e-2, relative L2
2e-3), with NaN in every unused block and dead slot. The same draws also run over fp8 (E4M3)
pools with random per-pool scales, and through the fused append step (whose pools must equal the
oracle's scatter, word for word)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_452_amd as pkv
import workloads
from helpers import (assert_close, gpu_decode, gpu_decode8, oracle_decode, oracle_decode8,
                     codes, poison_dead_slots_, poison_dead_slots8_, say, set_plane_, words)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def random_shape(seed: int):
    """One case's shape and lengths from its seed (no arithmetic of the method here)."""
    rng = np.random.default_rng(9000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16, 24, 32]))
    while Hkv * G > 64:
        Hkv //= 2
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    S = int(rng.integers(1, 49))
    kind = rng.choice(4, size=S, p=[0.15, 0.35, 0.35, 0.15])
    lo = np.array([0, 1, 41, 601])[kind]
    hi = np.array([0, 40, 600, 3000])[kind]
    lens = [int(rng.integers(a, b + 1)) for a, b in zip(lo, hi)]
    nwg = 0 if rng.random() < 0.4 else int(rng.integers(1, 1201))
    return Hkv * G, Hkv, D, B, dtype, lens, nwg


@pytest.mark.parametrize("seed", range(16))
def test_random_shape_matches_oracle(seed):
    Hq, Hkv, D, B, dtype, lens, nwg = random_shape(seed)
    lens = np.asarray(lens, np.int32)
    spec = workloads.Spec(0, f"random {seed}: Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} S={len(lens)} "
                             f"workgroups={nwg}", len(lens), Hq, Hkv, D,
                          "bf16" if dtype == torch.bfloat16 else "fp16", 1, seed=seed,
                          block_size=B)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 5, seed=seed)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    poison_dead_slots_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
    max_ctx = max(int(lens.max()), 1)
    say("random shape", spec.name, "max len", max_ctx)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv, max_ctx,
                     nwg, block_size=B)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks, block_size=B)
    assert_close(out, ref, spec.name)
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[s]).item() == 0


def _spec(tag, seed, Hq, Hkv, D, B, dtype, lens, nwg):
    return workloads.Spec(0, f"{tag} {seed}: Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} S={len(lens)} "
                             f"workgroups={nwg}", len(lens), Hq, Hkv, D,
                          "bf16" if dtype == torch.bfloat16 else "fp16", 1, seed=seed,
                          block_size=B)


@pytest.mark.parametrize("seed", range(100, 108))
def test_random_shape_fp8_matches_oracle(seed):
    Hq, Hkv, D, B, dtype, lens, nwg = random_shape(seed)
    lens = np.asarray(lens, np.int32)
    rng = np.random.default_rng(seed)
    # |V| <= 3.75 * v_scale: v_scale <= 1 keeps |out| below 4, where one bf16 rounding step of
    # the output (2^-6 on [4, 8)) would already exceed the max-abs bar.
    k_scale, v_scale = float(2.0 ** rng.integers(-3, 2)), float(rng.uniform(0.05, 1.0))
    spec = _spec("random fp8", seed, Hq, Hkv, D, B, dtype, lens, nwg)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 5, seed=seed)
    b = workloads.make_batch_fp8(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    poison_dead_slots8_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
    max_ctx = max(int(lens.max()), 1)
    say("random shape fp8", spec.name, "scales", k_scale, v_scale)
    out = gpu_decode8(b.q, k, v, b.block_tables, b.context_lens, spec.scale, k_scale, v_scale,
                      Hq, Hkv, max_ctx, nwg, block_size=B)
    torch.cuda.synchronize()
    ref = oracle_decode8(b.q, k, v, t.block_tables, t.context_lens, spec.scale, k_scale, v_scale,
                         Hq, Hkv, t.num_blocks, block_size=B)
    assert_close(out, ref, spec.name)


def _poison_new_slots_(k, v, t, Hkv, D, B):
    """NaN into the slot each sequence's new token goes to (the fused step must write it first)."""
    idx = []
    for s, n in enumerate(t.context_lens):
        n = int(n)
        if n == 0:
            continue
        blk = int(t.block_tables[s][(n - 1) // B])
        for h in range(Hkv):
            for d in range(D):
                idx.append((oracle.pool_index(False, blk, h, (n - 1) % B, d, Hkv, B, D),
                            oracle.pool_index(True, blk, h, (n - 1) % B, d, Hkv, B, D)))
    if idx:
        ia = torch.tensor(idx, dtype=torch.long, device=k.device)
        set_plane_(k, ia[:, 0], float("nan"))
        set_plane_(v, ia[:, 1], float("nan"))


@pytest.mark.parametrize("seed", range(200, 208))
def test_random_shape_fused_append_matches_oracle(seed):
    Hq, Hkv, D, B, dtype, lens, nwg = random_shape(seed)
    lens = np.asarray(lens, np.int32)
    spec = _spec("random fused", seed, Hq, Hkv, D, B, dtype, lens, nwg)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 5, seed=seed)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    poison_dead_slots_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
    _poison_new_slots_(k, v, t, Hkv, D, B)
    kw, vw = words(k), words(v)
    oracle.reshape_and_cache(kw, vw, b.new_key.cpu(), b.new_value.cpu(), t.slot_mapping, Hkv, D,
                             B, t.num_blocks)
    ref = oracle_decode(b.q, None, None, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks, k_words=kw, v_words=vw, block_size=B)
    max_ctx = max(int(lens.max()), 1)
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(len(lens), Hq, Hkv, D, B, max_ctx,
                                                               nwg), DEV)
    out = torch.empty_like(b.q)
    say("random shape fused append", spec.name)
    pkv.paged_attention_decode_append(out, b.q, b.new_key, b.new_value, k, v, b.block_tables,
                                      b.context_lens, spec.scale, Hq, Hkv, D, B, max_ctx, nwg, ws)
    torch.cuda.synchronize()
    assert_close(out, ref, spec.name)
    assert np.array_equal(words(k), kw), "K pool differs from the oracle's scatter"
    assert np.array_equal(words(v), vw), "V pool differs from the oracle's scatter"


def _scatter_case(seed):
    """A pool and a multi-token scatter: whole blocks written token by token (as a prompt fills
    them), scattered single slots, skipped (-1) entries, all in a shuffled order."""
    rng = np.random.default_rng(5000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    NB = int(rng.integers(8, 64))
    blocks = rng.permutation(NB)
    full = blocks[: int(rng.integers(1, max(2, NB // 4)))]
    slots = [int(b) * B + t for b in full for t in range(B)]
    rest = np.setdiff1d(np.arange(NB * B), np.array(slots))
    slots += [int(x) for x in rng.choice(rest, size=int(rng.integers(1, 60)), replace=False)]
    slots += [-1] * int(rng.integers(0, 4))
    slots = np.array(slots, np.int64)[rng.permutation(len(slots))]
    return Hkv, D, B, dtype, NB, slots


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("fp8", [False, True])
def test_random_multi_token_scatter_bit_exact(seed, fp8):
    Hkv, D, B, dtype, NB, slots = _scatter_case(seed)
    T = len(slots)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    key = workloads.randn((T, Hkv, D), dtype, gen, DEV)
    value = workloads.randn((T, Hkv, D), dtype, gen, DEV)
    sm = torch.from_numpy(slots).to(DEV)
    say("random scatter", seed, "fp8" if fp8 else str(dtype), f"Hkv={Hkv} D={D} B={B} NB={NB} T={T}")
    if fp8:
        pool = workloads.new_pool(1, NB, Hkv, B, D, torch.uint8, DEV)
        pool.copy_(torch.randint(0, 256, pool.shape, generator=gen, device=DEV, dtype=torch.uint8))
        k, v = (p[0] for p in workloads.planes(pool))
        kb, vb = codes(k), codes(v)
        ks, vs = 0.25, 0.5
        oracle.reshape_and_cache8(kb, vb, key.cpu(), value.cpu(), oracle.BF16 if dtype ==
                                  torch.bfloat16 else oracle.FP16, ks, vs, slots, Hkv, D, B, NB)
        pkv.reshape_and_cache_fp8(key, value, k, v, sm, NB, ks, vs, B)
        torch.cuda.synchronize()
        assert np.array_equal(codes(k), kb), "K pool differs"
        assert np.array_equal(codes(v), vb), "V pool differs"
    else:
        pool = workloads.new_pool(1, NB, Hkv, B, D, dtype, DEV)
        pool.copy_(workloads.randn(pool.shape, dtype, gen, DEV))
        k, v = (p[0] for p in workloads.planes(pool))
        kw, vw = words(k), words(v)
        oracle.reshape_and_cache(kw, vw, key.cpu(), value.cpu(), slots, Hkv, D, B, NB)
        pkv.reshape_and_cache(key, value, k, v, sm, NB, B)
        torch.cuda.synchronize()
        assert np.array_equal(words(k), kw), "K pool differs"
        assert np.array_equal(words(v), vw), "V pool differs"


def _prompt_case(seed):
    """A scatter in prompt order: several sequences' prompts, each a run of consecutive slots
    through its blocks starting at a random offset (mid-group too); two of them interleaved token
    by token (so their 4-slot groups are not whole in call order); a skipped and a past-the-pool
    entry dropped into one run."""
    rng = np.random.default_rng(6000 + seed)
    Hkv = int(rng.choice([1, 2, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    NB = int(rng.integers(24, 80))
    order = iter(rng.permutation(NB).tolist())
    runs = []
    for _ in range(int(rng.integers(3, 6))):
        start = int(rng.integers(0, B))           # the prompt continues a partly filled block
        n = int(rng.integers(1, 3 * B))
        blocks = [next(order) for _ in range(-(-(start + n) // B))]
        runs.append([blocks[(start + p) // B] * B + (start + p) % B for p in range(n)])
    a, b = runs.pop(), runs.pop()
    mixed = [x for pair in zip(a, b) for x in pair] + a[len(b):] + b[len(a):]
    runs.append(mixed)
    where = int(rng.integers(0, len(runs[0]) + 1))
    runs[0][where:where] = [-1, NB * B + 2]
    slots = np.array([x for r in runs for x in r], np.int64)
    return Hkv, D, B, dtype, NB, slots


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("fp8", [False, True])
def test_prompt_order_scatter_bit_exact(seed, fp8):
    """reshape_and_cache of prompts in order, where consecutive tokens fill whole 4-slot groups
    of the V tile and are written a group at a time: the whole pool equals the oracle's token by
    token scatter."""
    Hkv, D, B, dtype, NB, slots = _prompt_case(seed)
    T = len(slots)
    skipped = np.where(slots >= NB * B, -1, slots)  # the oracle takes a skipped slot as -1
    gen = torch.Generator(device=DEV).manual_seed(seed + 100)
    key = workloads.randn((T, Hkv, D), dtype, gen, DEV)
    value = workloads.randn((T, Hkv, D), dtype, gen, DEV)
    sm = torch.from_numpy(slots).to(DEV)
    say("prompt-order scatter", seed, "fp8" if fp8 else str(dtype), f"Hkv={Hkv} D={D} B={B} T={T}")
    if fp8:
        pool = workloads.new_pool(1, NB, Hkv, B, D, torch.uint8, DEV)
        pool.copy_(torch.randint(0, 256, pool.shape, generator=gen, device=DEV, dtype=torch.uint8))
        k, v = (p[0] for p in workloads.planes(pool))
        kb, vb = codes(k), codes(v)
        oracle.reshape_and_cache8(kb, vb, key.cpu(), value.cpu(), oracle.BF16 if dtype ==
                                  torch.bfloat16 else oracle.FP16, 0.25, 0.5, skipped, Hkv, D, B,
                                  NB)
        pkv.reshape_and_cache_fp8(key, value, k, v, sm, NB, 0.25, 0.5, B)
        torch.cuda.synchronize()
        assert np.array_equal(codes(k), kb), "K pool differs"
        assert np.array_equal(codes(v), vb), "V pool differs"
    else:
        pool = workloads.new_pool(1, NB, Hkv, B, D, dtype, DEV)
        pool.copy_(workloads.randn(pool.shape, dtype, gen, DEV))
        k, v = (p[0] for p in workloads.planes(pool))
        kw, vw = words(k), words(v)
        oracle.reshape_and_cache(kw, vw, key.cpu(), value.cpu(), skipped, Hkv, D, B, NB)
        pkv.reshape_and_cache(key, value, k, v, sm, NB, B)
        torch.cuda.synchronize()
        assert np.array_equal(words(k), kw), "K pool differs"
        assert np.array_equal(words(v), vw), "V pool differs"
