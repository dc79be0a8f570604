"""The benchmark's accounting (no GPU): algorithmic bytes per launch and the code hash that keys
the committed counter traffic."""
import numpy as np

import bench


def test_algorithmic_bytes_70b_decode():
    lens = np.full(64, 4096)
    # K and V rows: 64 x 4096 tokens x 8 kv heads x 128 dims x 2 B x 2; q and out: 64 x 64 x 128 x
    # 2 B x 2; one table entry per block (4 B) and one length per sequence (4 B).
    want = 64 * 4096 * 8 * 128 * 2 * 2 + 64 * 64 * 128 * 2 * 2 + 64 * 256 * 4 + 64 * 4
    assert bench.algorithmic_bytes(lens, 64, 8, 128) == want == 1075904768


def test_algorithmic_bytes_fp8_and_fused():
    lens = np.array([0, 1, 17, 4096])
    base16 = bench.algorithmic_bytes(lens, 32, 8, 128)
    fp8 = bench.algorithmic_bytes(lens, 32, 8, 128, kv_elem=1)
    kv16 = int(lens.sum()) * 8 * 128 * 2 * 2
    assert base16 - fp8 == kv16 // 2                     # pool bytes halve, q/out stay 16-bit
    # fused: the new token's rows come from the step's input (16-bit) instead of the pool and are
    # written into the pool: + one 16-bit K and V row per non-empty sequence and kv head
    new_rows = 3 * 8 * 128 * 2
    assert bench.algorithmic_bytes(lens, 32, 8, 128, fused=True) - base16 == new_rows * 2
    assert bench.algorithmic_bytes(lens, 32, 8, 128, kv_elem=1, fused=True) - fp8 == new_rows * 2


def test_code_hash_ignores_comments_only():
    a = "int f(int x) {  // doubles\n  return 2 * x;\n}\n"
    b = "// header\nint f(int x) {\n\n  return 2 * x;   // same code\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench.code_hash(a) == bench.code_hash(b)
    assert bench.code_hash(a) != bench.code_hash(c)


def test_unique_kv_bytes_counts_shared_blocks_once():
    # Two sequences share physical blocks 5 and 9 (a 32-token prefix); sequence 0 then has 3
    # tokens in block 2, sequence 1 has 20 tokens in blocks 7 (full) and 4 (4 tokens).
    tables = np.array([[5, 9, 2, -1], [5, 9, 7, 4]], np.int32)
    lens = np.array([35, 52])
    row = 2 * 64 * 2 * 2     # one token: 2 kv heads x 64 dims x 2 B, K and V
    assert bench.unique_kv_bytes(tables, lens, 2, 64) == (16 + 16 + 3 + 16 + 4) * row
    # no sharing: the same as the logical K/V bytes
    private = np.array([[0, 1, -1, -1], [2, 3, 4, 5]], np.int32)
    assert bench.unique_kv_bytes(private, lens, 2, 64) == int(lens.sum()) * row
    # fp8 pools hold one byte per element
    assert bench.unique_kv_bytes(tables, lens, 2, 64, kv_elem=1) * 2 == \
        bench.unique_kv_bytes(tables, lens, 2, 64)


def test_percentiles_nearest_rank():
    assert bench.percentiles([5, 1, 4, 2, 3]) == {"p10": 1, "p50": 3, "p90": 5}
    assert bench.percentiles(list(range(1, 11))) == {"p10": 1, "p50": 5, "p90": 9}
    assert bench.percentiles([7.0]) == {"p10": 7.0, "p50": 7.0, "p90": 7.0}
