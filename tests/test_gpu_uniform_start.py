"""GPU parity on uniform batches, where every sequence has (or nearly has) as many 16-token units
as max_context_len tokens make, and the library's range plan cuts the flattened positions on
stream boundaries: full and partly filled last blocks, the library's half grid, several streams per
range, two tile-id windows per wave, block size 32 and fp8 pools. Two cases pass a
max_context_len that the lengths do not fill (every sequence a unit short of it, or one sequence a
unit shorter than the rest), so their plans differ from the aligned one max_context_len alone
would suggest. Block tables are as wide as max_context_len needs; every entry past a sequence's
blocks names a spare block whose tiles are all NaN, and so do the dead slots, so a read of any
entry past a sequence's blocks could not go unnoticed. Each case is checked against the fp64
oracle to the usual bar (max-abs 1e-2, relative L2 2e-3)."""
import numpy as np
import pytest
import torch

import workloads
from helpers import (assert_close, gpu_decode, gpu_decode8, oracle_decode, oracle_decode8,
                     poison_dead_slots_, poison_dead_slots8_, say)

pytestmark = pytest.mark.gpu

DEV = "cuda"
E4M3_NAN = 0x7F


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


# name: (S, Hq, Hkv, D, B, lens rule, max_context_len, workgroups)
CASES = {
    # 512 streams of 64 units on the default 512 workgroups: one whole stream per range.
    "full blocks": (64, 64, 8, 128, 16, "full", 1024, 0),
    # Same units, fewer tokens: the last block of each sequence is partly dead.
    "partly filled last blocks": (64, 64, 8, 128, 16, "last block ragged", 1024, 0),
    # 256 streams of 128 units: the library picks all 512 workgroups, and its half grid gives
    # one whole stream per range.
    "half grid": (32, 32, 8, 128, 16, "full", 2048, 0),
    # 128 workgroups over 512 streams of 16 units: four whole streams per range.
    "four streams per range": (64, 8, 8, 64, 16, "full", 256, 128),
    # 8 streams of 512 units on 8 workgroups: 128 positions per wave, two windows of tile ids.
    "two windows per wave": (8, 8, 1, 128, 16, "full", 8192, 8),
    # 64 streams of 128 units (64 blocks of 32 tokens) on 64 workgroups.
    "block size 32": (16, 32, 4, 64, 32, "full", 2048, 64),
    # Every sequence a unit short of max_context_len.
    "max_context_len above every length": (64, 64, 8, 128, 16, "all a unit short", 1040, 0),
    "one sequence a unit shorter": (64, 64, 8, 128, 16, "one short", 1024, 0),
}


def _lens(rule, S, max_ctx, rng):
    if rule == "full":
        lens = np.full(S, max_ctx, np.int32)
    elif rule == "last block ragged":
        lens = (max_ctx - rng.integers(0, 16, size=S)).astype(np.int32)
    elif rule == "all a unit short":
        lens = np.full(S, max_ctx - 16, np.int32)
    elif rule == "one short":
        lens = np.full(S, max_ctx, np.int32)
        lens[S // 3] = max_ctx - 16
    else:
        raise ValueError(rule)
    return lens


def _case(name, fp8):
    S, Hq, Hkv, D, B, rule, max_ctx, nwg = CASES[name]
    rng = np.random.default_rng(sum(map(ord, name)))
    lens = _lens(rule, S, max_ctx, rng)
    spec = workloads.Spec(0, f"uniform start, {name}: S={S} Hq={Hq} Hkv={Hkv} D={D} B={B} "
                             f"max_ctx={max_ctx} workgroups={nwg}", S, Hq, Hkv, D, "bf16", 1,
                          seed=7, block_size=B)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 1, seed=7)
    spare = int(np.flatnonzero(~t.used_blocks)[0])  # the one block no sequence uses
    # Tables as wide as max_context_len needs; every entry past a sequence's blocks -> spare.
    width = -(-max_ctx // B)
    tables = np.full((S, width), spare, np.int32)
    for s, n in enumerate(lens):
        nb = -(-int(n) // B)
        tables[s, :nb] = t.block_tables[s, :nb]
    make = workloads.make_batch_fp8 if fp8 else workloads.make_batch
    b = make(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    if fp8:
        poison_dead_slots8_(k, v, tables, t.context_lens, Hkv, D, B)
        k[spare].fill_(E4M3_NAN)
        v[spare].fill_(E4M3_NAN)
    else:
        poison_dead_slots_(k, v, tables, t.context_lens, Hkv, D, B)
        k[spare].fill_(float("nan"))
        v[spare].fill_(float("nan"))
    bt = torch.from_numpy(tables).to(DEV)
    return spec, t, b, k, v, tables, bt, max_ctx, nwg


@pytest.mark.parametrize("name", list(CASES))
def test_uniform_start_matches_oracle(name):
    spec, t, b, k, v, tables, bt, max_ctx, nwg = _case(name, fp8=False)
    say(spec.name)
    out = gpu_decode(b.q, k, v, bt, b.context_lens, spec.scale, spec.num_q_heads,
                     spec.num_kv_heads, max_ctx, nwg, block_size=spec.block_size)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, tables, t.context_lens, spec.scale, spec.num_q_heads,
                        spec.num_kv_heads, t.num_blocks, block_size=spec.block_size)
    assert_close(out, ref, spec.name)


@pytest.mark.parametrize("name", ["full blocks", "partly filled last blocks",
                                  "one sequence a unit shorter"])
def test_uniform_start_fp8_matches_oracle(name):
    spec, t, b, k, v, tables, bt, max_ctx, nwg = _case(name, fp8=True)
    k_scale, v_scale = 0.5, 0.25
    say(spec.name, "fp8")
    out = gpu_decode8(b.q, k, v, bt, b.context_lens, spec.scale, k_scale, v_scale,
                      spec.num_q_heads, spec.num_kv_heads, max_ctx, nwg,
                      block_size=spec.block_size)
    torch.cuda.synchronize()
    ref = oracle_decode8(b.q, k, v, tables, t.context_lens, spec.scale, k_scale, v_scale,
                         spec.num_q_heads, spec.num_kv_heads, t.num_blocks,
                         block_size=spec.block_size)
    assert_close(out, ref, spec.name + " fp8")
