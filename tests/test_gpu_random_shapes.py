"""GPU parity on seeded random shapes: sequence counts, GQA groups (including several head tiles
per kv head), head dims, block sizes, element types, context-length mixes with empty, short and
long sequences, and workgroup counts from 1 to many more than the chip holds. Each case is
checked against the fp64 oracle to the same bar as the fixed cases (max-abs 1e-2, relative L2
2e-3), with NaN in every unused block and dead slot."""
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
