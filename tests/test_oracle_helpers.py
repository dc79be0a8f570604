"""Pins of the oracle's index helpers the GPU tests use to plant NaN (CPU only): the vectorised
lists equal the element-by-element enumeration through pool_index / pool_index8."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("fp8", [False, True])
def test_dead_slot_indices_equal_the_per_element_enumeration(fp8):
    """The oracle's vectorised dead-slot list (used to NaN-poison unused slots) is exactly the
    slots t >= n mod B of each partly filled last block, located by pool_index / pool_index8."""
    Hkv, Bs, Dd = 3, 32, 64
    lens = np.array([0, 1, 31, 32, 33, 70], np.int32)
    rng = np.random.default_rng(3)
    bt = rng.permutation(40)[:6 * 3].reshape(6, 3).astype(np.int32)
    index = oracle.pool_index8 if fp8 else oracle.pool_index
    for is_v in (False, True):
        want = [index(is_v, int(bt[s][n // Bs]), h, t, d, Hkv, Bs, Dd)
                for s, n in enumerate(lens) if n % Bs
                for t in range(n % Bs, Bs) for h in range(Hkv) for d in range(Dd)]
        got = oracle.dead_slot_indices(is_v, fp8, bt, lens, Hkv, Bs, Dd)
        assert got.tolist() == want


@pytest.mark.parametrize("fp8", [False, True])
def test_slot_indices_equal_the_per_element_enumeration(fp8):
    """The oracle's token-row index list is exactly (slot / B, h, slot % B, d) for every
    non-negative slot, kv head and dim, through pool_index / pool_index8."""
    Hkv, Bs, Dd = 2, 16, 128
    slots = np.array([5, -1, 16 * 9 + 15, 0, 16 * 30 + 7], np.int64)
    index = oracle.pool_index8 if fp8 else oracle.pool_index
    for is_v in (False, True):
        want = [index(is_v, int(sl) // Bs, h, int(sl) % Bs, d, Hkv, Bs, Dd)
                for sl in slots if sl >= 0 for h in range(Hkv) for d in range(Dd)]
        got = oracle.slot_indices(is_v, fp8, slots, Hkv, Bs, Dd)
        assert got.tolist() == want
