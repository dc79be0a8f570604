"""GPU parity on a wider seeded spread of batch shapes than the random-shape tests: batch sizes
around the 256 lengths one thread of the plan reads at once (255, 256, 257, 300, 513), contexts up
to 20,000 tokens on small batches, uniform batches, GQA groups of 5, 12 and 17 (a second head tile
holding one head), up to 128 query heads, and grids of 1 to 3,000 workgroups. Every unused block
and dead slot holds NaN (the fp8 NaN code for fp8 pools), and every case is checked against the
fp64 oracle to the usual bar (max-abs 1e-2, relative L2 2e-3); empty sequences must give zeros."""
import numpy as np
import pytest
import torch

import workloads
from helpers import (assert_close, gpu_decode, gpu_decode8, oracle_decode, oracle_decode8,
                     poison_dead_slots_, poison_dead_slots8_, say)

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_COST = 4e9  # tokens x query heads x head dim of a case: keeps each oracle run to seconds


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.synchronize()


def wide_shape(seed: int):
    """One case's shape and lengths from its seed (no arithmetic of the method here)."""
    rng = np.random.default_rng(70000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8, 16]))
    G = int(rng.choice([1, 2, 4, 5, 8, 12, 16, 17, 32]))
    while Hkv * G > 128:
        Hkv //= 2
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    S = int(rng.choice([1, 2, 3, 7, 64, 255, 256, 257, 300, 513]))
    kind = rng.choice(5, size=S, p=[0.1, 0.3, 0.3, 0.2, 0.1])
    lo = np.array([0, 1, 41, 601, 4000])[kind]
    hi = np.array([0, 40, 600, 3000, 20000 if S <= 8 else 6000])[kind]
    lens = np.array([int(rng.integers(a, b + 1)) for a, b in zip(lo, hi)], np.int32)
    if rng.random() < 0.2:  # uniform batch
        lens[:] = int(rng.integers(1, 4000))
    nwg = 0 if rng.random() < 0.4 else int(rng.integers(1, 3001))
    return Hkv * G, Hkv, D, B, dtype, lens, nwg


def _small_enough(seed: int) -> bool:
    Hq, _, D, _, _, lens, _ = wide_shape(seed)
    return int(lens.sum()) * Hq * D <= MAX_COST


# The first 32 seeds whose batch the oracle finishes in seconds; fp8 pools on every fourth.
_SEEDS = [seed for seed in range(40) if _small_enough(seed)][:32]
CASES = [(seed, fp8) for seed in _SEEDS for fp8 in ((False, True) if seed % 4 == 0 else (False,))]


@pytest.mark.parametrize("seed,fp8", CASES)
def test_wide_shape_matches_oracle(seed, fp8):
    Hq, Hkv, D, B, dtype, lens, nwg = wide_shape(seed)
    S = len(lens)
    spec = workloads.Spec(0, f"wide {seed}: S={S} Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} "
                             f"workgroups={nwg} fp8={fp8}", S, Hq, Hkv, D,
                          "bf16" if dtype == torch.bfloat16 else "fp16", 1, seed=seed,
                          block_size=B)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 3, seed=seed)
    max_ctx = max(int(lens.max()), 1)
    say(spec.name, "max len", max_ctx)
    if fp8:
        b = workloads.make_batch_fp8(spec, device=DEV, tables=t)
        k, v = b.k_pool[0], b.v_pool[0]
        poison_dead_slots8_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
        k_scale, v_scale = 0.5, 0.25
        out = gpu_decode8(b.q, k, v, b.block_tables, b.context_lens, spec.scale, k_scale, v_scale,
                          Hq, Hkv, max_ctx, nwg, block_size=B)
        torch.cuda.synchronize()
        ref = oracle_decode8(b.q, k, v, t.block_tables, t.context_lens, spec.scale, k_scale,
                             v_scale, Hq, Hkv, t.num_blocks, block_size=B)
    else:
        b = workloads.make_batch(spec, device=DEV, tables=t)
        k, v = b.k_pool[0], b.v_pool[0]
        poison_dead_slots_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
        out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv, max_ctx,
                         nwg, block_size=B)
        torch.cuda.synchronize()
        ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                            t.num_blocks, block_size=B)
    assert_close(out, ref, spec.name)
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[s]).item() == 0, f"{spec.name}: sequence {s} not zero"


# Seeds of the same generator whose batches (255 sequences, 128 and 68 query heads) produce
# attention outputs above 4 in magnitude. There the bf16 output format's spacing is 2^-5, so the
# rounding of the output alone can exceed the 1e-2 max-abs bar. Those outputs must lie within one
# spacing of the exact value; every other output meets 1e-2, and relative L2 meets 2e-3 over all.
@pytest.mark.parametrize("seed", [439, 754])
def test_wide_shape_outputs_above_4_within_one_bf16_spacing(seed):
    Hq, Hkv, D, B, dtype, lens, nwg = wide_shape(seed)
    assert dtype == torch.bfloat16
    S = len(lens)
    spec = workloads.Spec(0, f"wide {seed}: S={S} Hq={Hq} Hkv={Hkv} D={D} B={B} workgroups={nwg}",
                          S, Hq, Hkv, D, "bf16", 1, seed=seed, block_size=B)
    need = sum(-(-int(n) // B) for n in lens)
    t = workloads.make_tables(spec, lens=lens, num_blocks=need + 3, seed=seed)
    max_ctx = max(int(lens.max()), 1)
    say(spec.name, "max len", max_ctx)
    b = workloads.make_batch(spec, device=DEV, tables=t)
    k, v = b.k_pool[0], b.v_pool[0]
    poison_dead_slots_(k, v, t.block_tables, t.context_lens, Hkv, D, B)
    out = gpu_decode(b.q, k, v, b.block_tables, b.context_lens, spec.scale, Hq, Hkv, max_ctx, nwg,
                     block_size=B)
    torch.cuda.synchronize()
    ref = oracle_decode(b.q, k, v, t.block_tables, t.context_lens, spec.scale, Hq, Hkv,
                        t.num_blocks, block_size=B)
    got = out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    big = np.abs(ref) >= 4.0
    assert big.any(), "the case no longer produces outputs above 4"
    assert err[~big].max() <= 1e-2, f"max-abs {err[~big].max():.3e} on outputs below 4"
    spacing = 2.0 ** (np.floor(np.log2(np.abs(ref[big]))) - 7)  # bf16: 8 significant bits
    assert np.all(err[big] <= spacing), "an output above 4 is off by more than one bf16 spacing"
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 2e-3, f"relative L2 {rel:.3e}"
