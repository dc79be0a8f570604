"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each test ties the oracle to something other than itself: numbers printed on the pages, a library
routine (torch SDPA in fp64, numpy/torch float conversions), a brute-force loop, closed forms, or
the worked offsets of the documented pool layout.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sizing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- sizing facts

def test_sizing_examples_from_pages():
    g = _load("sizing_examples.json")
    e = g["kv_per_token_13b"]
    # hidden 5120 = kv heads x head dim for this MHA model (40 x 128)
    per_tok = sizing.kv_bytes(e["num_layers"], 40, 128, 1, e["dtype_bytes"])
    assert per_tok == e["bytes"] == 819200
    assert round(per_tok / 1000) == 819                       # "about 819 KB"
    c = g["conversation_2000_tokens_13b"]
    one = sizing.kv_bytes(40, 40, 128, c["tokens"], 2)
    assert round(one / 1e9, 1) == c["printed_gb_one"]          # ~1.6 GB
    assert round(one * c["count"] / 1e9) == c["printed_gb_sixteen"]  # 26 GB
    cp = g["capacity_13b_on_80gb"]
    budget, tokens_max, conc_a = sizing.capacity_plan(cp["gpu_mem_gb"] * 1e9, cp["weights_gb"] * 1e9,
                                                      0.0, per_tok, cp["avg_tokens_a"])
    assert budget == cp["kv_budget_gb"] * 1e9
    assert round(tokens_max, -3) == cp["printed_tokens_max"]    # "roughly 66,000"
    assert round(conc_a) == cp["printed_concurrency_a"]         # "about 33"
    _, _, conc_b = sizing.capacity_plan(80e9, 26e9, 0.0, per_tok, cp["avg_tokens_b"])
    assert round(conc_b) == cp["printed_concurrency_b"]         # "~8"
    l70 = g["kv_per_token_llama3_70b"]
    b70 = sizing.kv_bytes(l70["num_layers"], l70["num_kv_heads"], l70["head_dim"], 1,
                          l70["dtype_bytes"])
    assert b70 == l70["bytes"] and b70 / 1024 == l70["printed_kb"]
    bt = g["batch_64x4096_llama3_70b"]
    total = sizing.kv_bytes(80, 8, 128, bt["tokens"], 2, bt["requests"])
    assert total == bt["bytes"]
    assert sizing.truncate(total / 1024 / 1e6, 2) == bt["printed_gb"]
    # a block spans all layers: 16384 blocks of 16 tokens hold the same 64 x 4096 tokens
    assert sizing.block_bytes(16, 80, 8, 128, 2) * (64 * 4096 // 16) == total
    o = g["over_reservation"]
    assert sizing.truncate(100 * sizing.reservation_idle_fraction(o["used"], o["reserved"]), 1) \
        == o["printed_percent"]
    f = g["contiguous_flowchart"]
    assert [sizing.reserved_but_unused(u, f["reserved"]) for u in f["used"]] == f["printed_wasted"]
    a = g["on_demand_allocation"]
    assert sizing.blocks_needed(a["tokens"], a["block_size"]) == a["printed_blocks"]
    w = g["waste_bound"]
    assert max(sizing.wasted_slots(n, w["block_size"]) for n in range(1, 4000)) \
        == w["printed_max_waste"]
    assert min(sizing.wasted_slots(n, w["block_size"]) for n in range(1, 4000)) == 0


# ----------------------------------------------------------------------------- layout

def test_pool_layout_worked_offsets():
    g = _load("tile_layout.json")
    D, B = g["head_dim"], g["block_size"]
    for t, d, off in g["k"]:
        assert oracle.pool_index(False, 0, 0, t, d, 1, B, D) == off, ("K", t, d)
    for t, d, off in g["v"]:
        assert oracle.pool_index(True, 0, 0, t, d, 1, B, D) == off, ("V", t, d)
    # tile base: (block, kv head) -> (block * Hkv + head) * B * D
    assert oracle.pool_index(False, 3, 2, 0, 0, 8, B, D) == (3 * 8 + 2) * B * D
    assert oracle.pool_index(True, 3, 2, 15, 127, 8, B, D) == (3 * 8 + 2) * B * D + 2047


@pytest.mark.parametrize("D,B", [(64, 16), (128, 16), (128, 32)])
def test_pool_layout_is_a_bijection_per_tile(D, B):
    for is_v in (False, True):
        idx = sorted(oracle.pool_index(is_v, 0, 0, t, d, 1, B, D)
                     for t in range(B) for d in range(D))
        assert idx == list(range(B * D))


# ----------------------------------------------------------------------------- helpers

def _round(x, dtype):
    return torch.as_tensor(x, dtype=torch.float64).to(dtype)


def _words(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _build_paged(Kc_list, Vc_list, num_kv_heads, D, B, num_blocks, rng, dtype):
    """Scatter contiguous per-sequence K/V ([n][Hkv][D] each) into fresh pools through the
    oracle's own scatter, with blocks drawn at random. Returns pools, tables, lens."""
    S = len(Kc_list)
    lens = np.array([k.shape[0] for k in Kc_list], np.int32)
    need = [-(-int(n) // B) for n in lens]
    max_blocks = max(max(need), 1)
    perm = rng.permutation(num_blocks)
    tables = np.full((S, max_blocks), -1, np.int32)
    pos = 0
    for s in range(S):
        tables[s, :need[s]] = perm[pos:pos + need[s]]
        pos += need[s]
    kp = np.full(num_blocks * num_kv_heads * B * D, 0x7FC0, np.uint16)  # NaN everywhere
    vp = kp.copy()
    for s in range(S):
        n = int(lens[s])
        slots = np.array([tables[s, t // B] * B + t % B for t in range(n)], np.int64)
        oracle.reshape_and_cache(kp, vp, _words(Kc_list[s].to(dtype)), _words(Vc_list[s].to(dtype)),
                                 slots, num_kv_heads, D, B, num_blocks)
    return kp, vp, tables, lens


# ----------------------------------------------------------------------------- gather

@pytest.mark.parametrize("case", ["page1_diagram", "page2_diagram"])
def test_gather_follows_page_block_tables(case):
    g = _load("block_tables.json")[case]
    B, table, n = g["block_size"], g["table"], g["num_tokens"]
    D, Hkv, NB = 64, 2, 32
    # mark each token with its slot number (exact in fp16: < 2048)
    kp = np.zeros(NB * Hkv * B * D, np.uint16)
    vp = np.zeros_like(kp)
    slots = np.array([table[t // B] * B + t % B for t in range(n)], np.int64)
    key = torch.tensor(slots, dtype=torch.float16)[:, None, None].expand(n, Hkv, D)
    val = -key
    oracle.reshape_and_cache(kp, vp, key, val, slots, Hkv, D, B, NB)
    for head in range(Hkv):
        K, V = oracle.gather(kp, vp, oracle.FP16, np.array(table, np.int32), n, head, Hkv, D, B, NB)
        expect = np.array([table[t // B] * B + t % B for t in range(n)], np.float64)
        assert np.array_equal(K[:, 0], expect) and np.array_equal(V[:, 5], -expect)
        assert np.all(K == K[:, :1])
    # tokens in the last logical block
    assert n - (len(table) - 1) * B == g["last_block_used"]
    assert sizing.blocks_needed(n, B) == len(table)


def test_element_decoding_exhaustive():
    """Every 16-bit pattern decodes to the value numpy (fp16) and torch (bf16) give it."""
    D, B, Hkv = 64, 16, 1
    NB = 65536 // (B * D)
    words = np.arange(65536, dtype=np.uint16)
    table = np.arange(NB, dtype=np.int32)
    n = NB * B
    for dtype, ref in ((oracle.FP16, words.view(np.float16).astype(np.float64)),
                       (oracle.BF16, torch.from_numpy(words.view(np.int16)).view(torch.bfloat16)
                        .to(torch.float64).numpy())):
        K, V = oracle.gather(words, words, dtype, table, n, 0, Hkv, D, B, NB)
        for is_v, M in ((False, K), (True, V)):
            got = np.empty(65536)
            for t in range(n):
                for d in range(D):
                    got[oracle.pool_index(is_v, t // B, 0, t % B, d, Hkv, B, D)] = M[t, d]
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(got), nan)
            assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------------------------------- attention

@pytest.mark.parametrize("Hq,Hkv,D,dtype,lens", [
    (4, 4, 64, torch.bfloat16, [1, 15, 16, 41]),
    (8, 2, 128, torch.bfloat16, [33, 7, 100]),
    (8, 4, 64, torch.float16, [48, 17, 1, 64]),
    (6, 1, 128, torch.bfloat16, [129, 31]),
])
def test_oracle_matches_torch_sdpa(Hq, Hkv, D, dtype, lens):
    rng = np.random.default_rng(sum(lens) + Hq)
    gen = torch.Generator().manual_seed(int(sum(lens)) * 31 + D)
    B = 16
    Kc = [torch.randn(n, Hkv, D, generator=gen).to(dtype) for n in lens]
    Vc = [torch.randn(n, Hkv, D, generator=gen).to(dtype) for n in lens]
    q = torch.randn(len(lens), Hq, D, generator=gen).to(dtype)
    NB = sum(-(-n // B) for n in lens) + 5
    kp, vp, tables, lns = _build_paged(Kc, Vc, Hkv, D, B, NB, rng, dtype)
    scale = 1.0 / math.sqrt(D)
    dt = oracle.FP16 if dtype == torch.float16 else oracle.BF16
    out = oracle.paged_decode(_words(q), kp, vp, tables, lns, scale, Hq, Hkv, D, B, NB, dt)
    sc = float(np.float32(scale))
    for s, n in enumerate(lens):
        qs = q[s].to(torch.float64)[None, :, None, :]                 # [1, Hq, 1, D]
        ks = Kc[s].to(torch.float64).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, n, D]
        vs = Vc[s].to(torch.float64).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=sc,
                                                               enable_gqa=True)
        np.testing.assert_allclose(out[s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_oracle_matches_bruteforce_loop():
    """The tiny 4-sequence shape checked by a direct triple loop in Python floats."""
    Hq = Hkv = 4
    D, B = 64, 16
    lens = [1, 15, 16, 41]
    rng = np.random.default_rng(7)
    gen = torch.Generator().manual_seed(7)
    Kc = [torch.randn(n, Hkv, D, generator=gen).to(torch.bfloat16) for n in lens]
    Vc = [torch.randn(n, Hkv, D, generator=gen).to(torch.bfloat16) for n in lens]
    q = torch.randn(4, Hq, D, generator=gen).to(torch.bfloat16)
    kp, vp, tables, lns = _build_paged(Kc, Vc, Hkv, D, B, 64, rng, torch.bfloat16)
    scale = 0.125
    out = oracle.paged_decode(_words(q), kp, vp, tables, lns, scale, Hq, Hkv, D, B, 64, oracle.BF16)
    for s, n in enumerate(lens):
        K = Kc[s].float().tolist()
        V = Vc[s].float().tolist()
        for h in range(Hq):
            qv = q[s, h].float().tolist()
            x = [scale * sum(qv[d] * K[t][h][d] for d in range(D)) for t in range(n)]
            m = max(x)
            w = [math.exp(xi - m) for xi in x]
            z = sum(w)
            ref = [sum(w[t] * V[t][h][d] for t in range(n)) / z for d in range(D)]
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-12)


def _single(q, Kc, Vc, dtype=torch.bfloat16, Hq=1, Hkv=1, D=None, B=16, scale=None, NB=None):
    D = D or q.shape[-1]
    n = Kc.shape[0]
    NB = NB or (-(-n // B) + 3)
    rng = np.random.default_rng(n)
    kp, vp, tables, lns = _build_paged([Kc], [Vc], Hkv, D, B, NB, rng, dtype)
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    dt = oracle.FP16 if dtype == torch.float16 else oracle.BF16
    return oracle.paged_decode(_words(q.to(dtype)), kp, vp, tables, lns, scale, Hq, Hkv, D, B, NB,
                               dt)


def test_closed_form_single_token_returns_its_value():
    gen = torch.Generator().manual_seed(1)
    q = torch.randn(1, 2, 64, generator=gen)
    K = torch.randn(1, 1, 64, generator=gen).to(torch.bfloat16)
    V = torch.randn(1, 1, 64, generator=gen).to(torch.bfloat16)
    out = _single(q, K, V, Hq=2, Hkv=1)
    for h in range(2):
        assert np.array_equal(out[0, h], V[0, 0].double().numpy())


def test_closed_form_zero_query_is_mean_of_values():
    gen = torch.Generator().manual_seed(2)
    n = 37
    q = torch.zeros(1, 1, 128)
    K = torch.randn(n, 1, 128, generator=gen).to(torch.bfloat16)
    V = torch.randn(n, 1, 128, generator=gen).to(torch.bfloat16)
    out = _single(q, K, V)
    np.testing.assert_allclose(out[0, 0], V[:, 0].double().mean(0).numpy(), rtol=0, atol=1e-14)


def test_closed_form_constant_values():
    gen = torch.Generator().manual_seed(3)
    n = 50
    q = torch.randn(1, 1, 64, generator=gen)
    K = torch.randn(n, 1, 64, generator=gen).to(torch.bfloat16)
    c = torch.randn(64, generator=gen).to(torch.bfloat16)
    V = c[None, None].expand(n, 1, 64).contiguous()
    out = _single(q, K, V)
    np.testing.assert_allclose(out[0, 0], c.double().numpy(), rtol=1e-14, atol=0)


def test_closed_form_key_shift_invariance():
    """Adding one vector to every key multiplies every weight by the same factor."""
    gen = torch.Generator().manual_seed(4)
    n, D = 45, 64
    q = torch.randn(1, 1, D, generator=gen).to(torch.bfloat16)
    # small integers keep K and K + u exact in bf16
    K = torch.randint(-8, 8, (n, 1, D), generator=gen).to(torch.bfloat16)
    u = torch.randint(-8, 8, (D,), generator=gen).to(torch.bfloat16)
    V = torch.randn(n, 1, D, generator=gen).to(torch.bfloat16)
    a = _single(q, K, V, scale=0.01)
    b = _single(q, (K + u).to(torch.bfloat16), V, scale=0.01)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # and the shift must matter for a different query direction if the keys differ (sanity)
    assert not np.allclose(a, _single(q, K * 2, V, scale=0.01))


def test_closed_form_dominant_key_selects_its_value():
    gen = torch.Generator().manual_seed(5)
    n, D, j = 40, 64, 23
    q = torch.ones(1, 1, D).to(torch.bfloat16)
    K = torch.zeros(n, 1, D).to(torch.bfloat16)
    K[j] = 4.0
    V = torch.randn(n, 1, D, generator=gen).to(torch.bfloat16)
    out = _single(q, K, V, scale=1.0)  # score gap 256 -> other weights ~e^-256
    np.testing.assert_allclose(out[0, 0], V[j, 0].double().numpy(), rtol=0, atol=1e-100)


def test_empty_sequence_gives_zero_and_padding_is_never_read():
    D, B, Hkv, NB = 64, 16, 1, 8
    kp = np.full(NB * Hkv * B * D, 0x7FC0, np.uint16)  # all NaN
    vp = kp.copy()
    tables = np.full((2, 4), -1, np.int32)              # padding -1 must never be read
    q = np.zeros((2, 1, D), np.uint16)
    out = oracle.paged_decode(q, kp, vp, tables, np.array([0, 0], np.int32), 0.125, 1, 1, D, B,
                              NB, oracle.BF16)
    assert np.array_equal(out, np.zeros((2, 1, D)))


def test_dead_slots_do_not_leak():
    """NaN in the unwritten slots of the last block must not reach the output."""
    gen = torch.Generator().manual_seed(6)
    n = 41
    q = torch.randn(1, 1, 64, generator=gen)
    K = torch.randn(n, 1, 64, generator=gen)
    V = torch.randn(n, 1, 64, generator=gen)
    out = _single(q, K, V)  # pools start all-NaN in _build_paged
    assert np.all(np.isfinite(out))


def test_gqa_head_mapping_is_contiguous_groups():
    """Query head h reads kv head h // G: giving kv heads distinct constant values shows it."""
    Hq, Hkv, D, n = 8, 2, 64, 20
    gen = torch.Generator().manual_seed(8)
    q = torch.randn(1, Hq, D, generator=gen)
    K = torch.randn(n, Hkv, D, generator=gen)
    V = torch.zeros(n, Hkv, D)
    V[:, 1] = 1.0
    out = _single(q, K, V, Hq=Hq, Hkv=Hkv)
    assert np.array_equal(out[0, :, 0], np.array([0, 0, 0, 0, 1, 1, 1, 1], np.float64))


def test_paired_and_full_outputs_agree():
    gen = torch.Generator().manual_seed(9)
    Hq, Hkv, D = 4, 2, 64
    lens = [20, 35]
    rng = np.random.default_rng(9)
    Kc = [torch.randn(n, Hkv, D, generator=gen).to(torch.bfloat16) for n in lens]
    Vc = [torch.randn(n, Hkv, D, generator=gen).to(torch.bfloat16) for n in lens]
    q = torch.randn(2, Hq, D, generator=gen).to(torch.bfloat16)
    kp, vp, tables, lns = _build_paged(Kc, Vc, Hkv, D, 16, 10, rng, torch.bfloat16)
    full = oracle.paged_decode(_words(q), kp, vp, tables, lns, 0.125, Hq, Hkv, D, 16, 10,
                               oracle.BF16)
    pairs = [(1, 3), (0, 0), (1, 0)]
    part = oracle.paged_decode(_words(q), kp, vp, tables, lns, 0.125, Hq, Hkv, D, 16, 10,
                               oracle.BF16, pairs=pairs)
    for i, (s, h) in enumerate(pairs):
        assert np.array_equal(part[i], full[s, h])


def test_reshape_skips_negative_slots_and_rejects_out_of_range():
    D, B, Hkv, NB = 64, 16, 2, 4
    kp = np.zeros(NB * Hkv * B * D, np.uint16)
    vp = kp.copy()
    key = np.arange(2 * Hkv * D, dtype=np.uint16).reshape(2, Hkv, D)
    oracle.reshape_and_cache(kp, vp, key, key, np.array([-1, 5], np.int64), Hkv, D, B, NB)
    assert np.count_nonzero(kp) == np.count_nonzero(key[1])
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(kp, vp, key, key, np.array([NB * B, 0], np.int64), Hkv, D, B, NB)


# ---- fp8 (OCP E4M3) KV pools -------------------------------------------------------------

def test_e4m3_decoding_exhaustive_against_torch():
    """All 256 codes: the oracle's definition-based value equals torch's float8_e4m3fn."""
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6 and oracle.e4m3_value(0x38) == 1.0


def test_e4m3_encoding_matches_torch_in_range():
    """Round to nearest even against torch's float8_e4m3fn cast wherever the two readings agree
    (|y| < 464, below the first value torch sends to NaN): every bf16 bit pattern in range, plus
    random fp32 values."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ys = bits.to(torch.float32)
    rng = np.random.default_rng(5)
    extra = torch.from_numpy(np.concatenate([
        rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)]).astype(np.float32))
    ys = torch.cat([ys, extra])
    ys = ys[torch.isfinite(ys) & (ys.abs() < 464.0)]
    want = ys.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(y)) for y in ys.numpy()], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encoding_saturates_and_keeps_nan_and_sign():
    """The reading for values the pages leave open: beyond the largest finite value the code
    saturates to +-448; NaN stays NaN with its sign; -0 keeps its sign."""
    for y, c in [(464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E), (float("inf"), 0x7E),
                 (-500.0, 0xFE), (float("nan"), 0x7F), (-0.0, 0x80), (-1e-9, 0x80)]:
        assert oracle.e4m3_encode(y) == c, (y, c)


def test_e4m3_round_trip_error_bound():
    """Every finite code round-trips exactly, and quantization error is at most half a step."""
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c
    rng = np.random.default_rng(6)
    for y in rng.standard_normal(2000).astype(np.float32) * 10:
        v = oracle.e4m3_value(oracle.e4m3_encode(float(y)))
        e = max(math.floor(math.log2(abs(y))), -6) if y != 0 else -6
        assert abs(v - float(y)) <= 2.0 ** (e - 3) / 2 + 1e-30


def test_fp8_pool_layout_worked_offsets_and_bijection():
    g = _load("tile_layout_fp8.json")
    D, B = g["head_dim"], g["block_size"]
    for t, d, off in g["k"]:
        assert oracle.pool_index8(False, 0, 0, t, d, 1, B, D) == off
    for t, d, off in g["v"]:
        assert oracle.pool_index8(True, 0, 0, t, d, 1, B, D) == off
    for D, B in [(64, 16), (128, 16), (128, 32), (64, 32)]:
        for is_v in (False, True):
            seen = sorted(oracle.pool_index8(is_v, 2, 1, t, d, 3, B, D)
                          for t in range(B) for d in range(D))
            base = (2 * 3 + 1) * B * D
            assert seen == list(range(base, base + B * D))


def test_fp8_decode_equals_16bit_decode_on_exactly_representable_values():
    """With power-of-two scales every dequantized value is exactly a bf16 value: decode over fp8
    pools must equal decode over 16-bit pools holding those values (an independent path)."""
    rng = np.random.default_rng(8)
    Hq, Hkv, D, B, NB = 8, 2, 64, 16, 16
    lens = np.array([1, 17, 40, 100], np.int32)   # 13 blocks
    tables = np.full((4, 8), -1, np.int32)
    perm = rng.permutation(NB)
    p = 0
    for s, n in enumerate(lens):
        k = -(-int(n) // B)
        tables[s, :k] = perm[p:p + k]
        p += k
    kb = rng.integers(0, 256, size=NB * Hkv * B * D).astype(np.uint8)
    vb = rng.integers(0, 256, size=NB * Hkv * B * D).astype(np.uint8)
    kb[(kb & 0x7F) == 0x7F] = 0x10   # no NaN codes
    vb[(vb & 0x7F) == 0x7F] = 0x11
    ks, vs = 0.25, 4.0
    kw = np.zeros(NB * Hkv * B * D, np.uint16)
    vw = np.zeros(NB * Hkv * B * D, np.uint16)
    for b in range(NB):
        for h in range(Hkv):
            for t in range(B):
                for d in range(D):
                    i8k = oracle.pool_index8(False, b, h, t, d, Hkv, B, D)
                    i8v = oracle.pool_index8(True, b, h, t, d, Hkv, B, D)
                    kval = torch.tensor(oracle.e4m3_value(kb[i8k]) * ks, dtype=torch.float64)
                    vval = torch.tensor(oracle.e4m3_value(vb[i8v]) * vs, dtype=torch.float64)
                    kw[oracle.pool_index(False, b, h, t, d, Hkv, B, D)] = kval.to(
                        torch.bfloat16).view(torch.int16).item() & 0xFFFF
                    vw[oracle.pool_index(True, b, h, t, d, Hkv, B, D)] = vval.to(
                        torch.bfloat16).view(torch.int16).item() & 0xFFFF
    q = torch.randn(4, Hq, D, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    got = oracle.paged_decode8(q, kb, vb, ks, vs, tables, lens, 0.125, Hq, Hkv, D, B, NB,
                               oracle.BF16)
    want = oracle.paged_decode(q, kw, vw, tables, lens, 0.125, Hq, Hkv, D, B, NB, oracle.BF16)
    assert np.array_equal(got, want)


def test_fp8_scatter_quantizes_each_element():
    """reshape_and_cache8 stores e4m3(fl32(x * fl32(1/scale))) at pool_index8 and nothing else."""
    rng = np.random.default_rng(9)
    Hkv, D, B, NB = 2, 64, 16, 4
    T = 3
    key = torch.randn(T, Hkv, D, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    val = torch.randn(T, Hkv, D, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    kp = np.full(NB * Hkv * B * D, 0xAA, np.uint8)
    vp = np.full(NB * Hkv * B * D, 0xAA, np.uint8)
    slots = np.array([5, -1, 3 * 16 + 15], np.int64)
    ks, vs = 0.3, 0.07
    oracle.reshape_and_cache8(kp, vp, key, val, oracle.BF16, ks, vs, slots, Hkv, D, B, NB)
    kinv = np.float32(1.0) / np.float32(ks)
    vinv = np.float32(1.0) / np.float32(vs)
    touched = set()
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, t = divmod(int(slot), B)
        for h in range(Hkv):
            for d in range(D):
                kx = np.float32(key[i, h, d].float().item()) * kinv
                vx = np.float32(val[i, h, d].float().item()) * vinv
                ik = oracle.pool_index8(False, b, h, t, d, Hkv, B, D)
                iv = oracle.pool_index8(True, b, h, t, d, Hkv, B, D)
                assert kp[ik] == oracle.e4m3_encode(float(kx))
                assert vp[iv] == oracle.e4m3_encode(float(vx))
                touched.add(ik)
    untouched = np.ones(kp.shape[0], bool)
    untouched[list(touched)] = False
    assert np.all(kp[untouched] == 0xAA)
