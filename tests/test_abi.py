"""The C ABI: exports, host-side argument checks and geometry (no GPU work is launched)."""
import ctypes
import math
import os
import re

import pytest

import paged_kv_cache_452_amd as pkv
from oracle import sizing

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP, NO_BLOCKS = 0, -1, -2, -3, -4, -5, -6
FAKE = 1 << 40  # a 4 KiB-aligned address that is never dereferenced on these paths


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


def test_library_exports_every_declared_function():
    lib = pkv.load_library()
    names = _declared_functions()
    assert set(names) == set(pkv.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in [(OK, "PKV_OK"), (INVALID, "PKV_ERR_INVALID_ARG"),
                       (UNSUPPORTED, "PKV_ERR_UNSUPPORTED"), (ALIGN, "PKV_ERR_ALIGNMENT"),
                       (WORKSPACE, "PKV_ERR_WORKSPACE"), (HIP, "PKV_ERR_HIP"),
                       (NO_BLOCKS, "PKV_ERR_NO_BLOCKS")]:
        assert pkv.pkv_status_string(code) == name


def test_kv_pool_bytes_matches_sizing_formula():
    # 70B-shaped: 80 layers x 16384 blocks x 8 kv heads x 16 x 128, bf16; K and V together
    total = pkv.kv_pool_bytes(80, 16384, 8, 128, 16, pkv.PKV_BF16)
    assert total == sizing.kv_bytes(80, 8, 128, 64 * 4096, 2) == 85899345920
    assert total == 16384 * sizing.block_bytes(16, 80, 8, 128, 2)
    assert pkv.kv_pool_bytes(1, 64, 4, 64, 16, pkv.PKV_BF16) == 2 * 64 * 4 * 16 * 64 * 2
    # unsupported shapes and bad sizes give 0
    assert pkv.kv_pool_bytes(1, 64, 4, 96, 16, pkv.PKV_BF16) == 0
    assert pkv.kv_pool_bytes(1, 64, 4, 128, 8, pkv.PKV_BF16) == 0
    assert pkv.kv_pool_bytes(1, 64, 4, 128, 32, pkv.PKV_BF16) == 2 * 64 * 4 * 32 * 128 * 2
    assert pkv.kv_pool_bytes(0, 64, 4, 128, 16, pkv.PKV_BF16) == 0
    assert pkv.kv_pool_bytes(1, 64, 4, 128, 16, 7) == 0
    # overflow is detected
    assert pkv.kv_pool_bytes(2**31 - 1, 2**31 - 1, 2**31 - 1, 128, 16, pkv.PKV_BF16) == 0


def test_kv_pool_create_and_layers():
    lib = pkv.load_library()
    total = pkv.kv_pool_bytes(80, 16384, 8, 128, 16, pkv.PKV_BF16)
    pool = pkv.kv_pool_create(FAKE, total, 80, 16384, 8, 128, 16, pkv.PKV_BF16)
    k0, v0 = pool.layer(0)
    k5, v5 = pool.layer(5)
    tile = 16 * 128 * 2  # the V plane starts one tile after the K plane
    assert (k0, v0) == (FAKE, FAKE + tile)
    assert k5 - k0 == 5 * total // 80 and v5 - k5 == tile
    with pytest.raises(pkv.PagedKVError):
        pool.layer(80)
    with pytest.raises(pkv.PagedKVError):
        pool.layer(-1)
    pool.destroy()
    h = ctypes.c_void_p()
    assert lib.kv_pool_create(ctypes.byref(h), FAKE + 16, total, 80, 16384, 8, 128, 16, 0) == ALIGN
    assert h.value is None
    assert lib.kv_pool_create(ctypes.byref(h), FAKE, total - 1, 80, 16384, 8, 128, 16, 0) == INVALID
    assert lib.kv_pool_create(ctypes.byref(h), None, total, 80, 16384, 8, 128, 16, 0) == INVALID
    assert lib.kv_pool_create(ctypes.byref(h), FAKE, total, 80, 16384, 8, 96, 16, 0) == UNSUPPORTED
    assert lib.kv_pool_create(None, FAKE, total, 80, 16384, 8, 128, 16, 0) == INVALID
    lib.kv_pool_destroy(None)


def _decode(lib, **kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, scale=0.1, hq=32, hkv=8,
                d=128, b=16, s=4, mb=8, maxc=128, nwg=1, dt=0, ws=None, wsb=0)
    args.update(kw)
    return lib.paged_attention_decode(args["out"], args["q"], args["k"], args["v"], args["bt"],
                                      args["cl"], args["scale"], args["hq"], args["hkv"],
                                      args["d"], args["b"], args["s"], args["mb"], args["maxc"],
                                      args["nwg"], args["dt"], args["ws"], args["wsb"], None)


def _ws(G, D=128):
    """G ranges x 2 partials x 16 heads x (D + 2) floats, then G counters (256-rounded)."""
    return G * 2 * 16 * (D + 2) * 4 + -(-4 * G // 256) * 256


def test_decode_argument_errors_return_before_launch():
    lib = pkv.load_library()
    assert _decode(lib, hq=30, hkv=8) == INVALID            # head ratio
    assert _decode(lib, hkv=0) == INVALID
    assert _decode(lib, d=96) == UNSUPPORTED
    assert _decode(lib, b=48) == UNSUPPORTED
    assert _decode(lib, b=8) == UNSUPPORTED
    assert _decode(lib, dt=5) == UNSUPPORTED
    assert _decode(lib, q=None, ws=FAKE, wsb=1 << 30) == INVALID
    assert _decode(lib, out=FAKE + 2) == ALIGN
    assert _decode(lib, k=FAKE + 8) == ALIGN
    assert _decode(lib, bt=FAKE + 2) == ALIGN
    assert _decode(lib, maxc=129, mb=8) == INVALID          # more than the table can hold
    assert _decode(lib, nwg=-1) == INVALID                  # negative workgroup count
    assert _decode(lib, nwg=(1 << 20) + 1) == INVALID
    assert _decode(lib, scale=float("nan")) == INVALID
    assert _decode(lib, s=-1) == INVALID
    assert _decode(lib, s=0) == OK                          # nothing to do, nothing launched
    assert _decode(lib, s=2049) == UNSUPPORTED              # beyond the per-launch plan size
    assert _decode(lib, s=4, mb=(1 << 28)) == UNSUPPORTED   # positions beyond 32 bits
    # every launch needs a workspace (counters + partials of its workgroup ranges)
    assert _decode(lib, nwg=32, ws=None, wsb=0) == WORKSPACE
    need = pkv.paged_attention_workspace_bytes(4, 32, 8, 128, 16, 128, 32)
    assert need == _ws(32)
    assert _decode(lib, nwg=32, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _decode(lib, nwg=32, ws=FAKE + 16, wsb=need) == ALIGN


def test_workspace_and_workgroup_choice():
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_attention_workspace_bytes(4, 30, 8, 128, 16, 100, 0)
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_attention_workspace_bytes(4, 32, 8, 128, 16, 100, -3)
    for G in (1, 2, 100, 512, 1000, 1 << 20):
        assert pkv.paged_attention_workspace_bytes(64, 64, 8, 128, 16, 4096, G) == _ws(G)
        assert pkv.paged_attention_workspace_bytes(64, 64, 8, 64, 16, 4096, G) == _ws(G, 64)
    for S, Hq, Hkv, maxc in [(64, 64, 8, 4096), (64, 32, 8, 8192), (32, 40, 40, 2048),
                             (66, 32, 8, 32768), (4, 4, 4, 41), (1, 8, 1, 1 << 20)]:
        g = pkv.paged_attention_num_workgroups(S, Hq, Hkv, maxc, 16)
        heads_tiles = -(-(Hq // Hkv) // 16)
        streams = S * Hkv * heads_tiles
        positions = streams * -(-maxc // 16)
        assert 1 <= g <= max(1, -(-positions // 64), streams)
        assert g >= min(streams, 2 * 256)   # at least one per stream (up to the resident limit)
        assert g <= 2 * 304   # two resident workgroups per compute unit
        assert pkv.paged_attention_workspace_bytes(S, Hq, Hkv, 128, 16, maxc, 0) == _ws(g)
    # tiny batch: 4 sequences x 4 kv heads = 16 streams of <= 3 blocks -> one workgroup each
    assert pkv.paged_attention_num_workgroups(4, 4, 4, 41, 16) == 16
    assert pkv.paged_attention_num_workgroups(4, 30, 8, 41, 16) == 0


def test_reshape_argument_errors():
    lib = pkv.load_library()
    f = lib.reshape_and_cache
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 10, 0, None) == OK     # no tokens
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, 0, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 80, 16, 10, 0, None) == UNSUPPORTED
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, None) == INVALID
    assert f(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 4, 8, 128, 16, 10, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 4, 4, 8, 128, 16, 10, 0, None) == ALIGN


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pkv.paged_attention_decode(q, q, q, q, torch.zeros(1, 1, dtype=torch.int32),
                                   torch.zeros(1, dtype=torch.int32), 0.125, 4, 4, 64, 16, 0)


@pytest.mark.parametrize("dtype,elem", [(pkv.PKV_BF16, 2), (pkv.PKV_FP8_E4M3, 1)])
@pytest.mark.parametrize("B", [16, 32])
def test_pool_views_match_kv_pool_layer(dtype, elem, B):
    """The K and V plane views the tests and the benchmark pass (workloads.new_pool / planes) sit
    at exactly the addresses kv_pool_layer gives for the same allocation (host memory; nothing is
    dereferenced), and each plane has the two-tile stride per (block, kv head)."""
    import torch
    import workloads
    L, NB, Hkv, D = 3, 5, 2, 64
    kv = workloads.new_pool(L, NB, Hkv, B, D, torch.uint8 if elem == 1 else torch.bfloat16, "cpu")
    nbytes = kv.numel() * kv.element_size()
    assert nbytes == pkv.kv_pool_bytes(L, NB, Hkv, D, B, dtype)
    base = kv.data_ptr()
    k, v = workloads.planes(kv)
    shift = -base % 256   # kv_pool_create wants a 256-byte aligned base: compare offsets from it
    pool = pkv.kv_pool_create(base + shift, nbytes, L, NB, Hkv, D, B, dtype)
    for layer in range(L):
        kl, vl = pool.layer(layer)
        assert kl - shift == k[layer].data_ptr() and vl - shift == v[layer].data_ptr()
        assert vl - kl == B * D * elem                         # V tile right after the K tile
    assert k.stride(2) == 2 * B * D and k.stride(1) == Hkv * 2 * B * D   # elements
    pool.destroy()


def test_copy_blocks_argument_errors():
    lib = pkv.load_library()
    total = pkv.kv_pool_bytes(2, 16, 4, 128, 16, pkv.PKV_BF16)
    pool = pkv.kv_pool_create(FAKE, total, 2, 16, 4, 128, 16, pkv.PKV_BF16)
    f = lib.copy_blocks
    assert f(pool._h, None, None, 0, None) == OK            # nothing to copy, nothing launched
    assert f(None, FAKE, FAKE, 1, None) == INVALID
    assert f(pool._h, FAKE, FAKE, -1, None) == INVALID
    assert f(pool._h, FAKE, FAKE, 65536, None) == INVALID
    assert f(pool._h, None, FAKE, 1, None) == INVALID
    assert f(pool._h, FAKE + 2, FAKE, 1, None) == ALIGN
    pool.destroy()


def test_fp8_pool_sizing_and_argument_errors():
    lib = pkv.load_library()
    FP8 = pkv.PKV_FP8_E4M3
    total = pkv.kv_pool_bytes(80, 16384, 8, 128, 16, FP8)
    assert total == sizing.kv_bytes(80, 8, 128, 64 * 4096, 1)
    assert total == pkv.kv_pool_bytes(80, 16384, 8, 128, 16, pkv.PKV_BF16) // 2
    pool = pkv.kv_pool_create(FAKE, total, 80, 16384, 8, 128, 16, FP8)
    k1, v1 = pool.layer(1)
    assert k1 - FAKE == 2 * 16384 * 8 * 16 * 128 and v1 - k1 == 16 * 128
    pool.destroy()

    r = lib.reshape_and_cache_fp8
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, pkv.PKV_BF16, 0.5, 0.5, None]

    def call(**kw):
        a = list(args)
        for i, x in kw.items():
            a[int(i[1:])] = x
        return r(*a)

    assert call(a5=0) == OK                                  # no tokens
    assert call(a11=0.0) == INVALID                          # scales must be finite and > 0
    assert call(a12=-1.0) == INVALID
    assert call(a11=float("inf")) == INVALID
    assert call(a12=float("nan")) == INVALID
    assert call(a10=FP8) == UNSUPPORTED                      # key/value are 16-bit
    assert call(a7=96) == UNSUPPORTED
    assert call(a9=0) == INVALID                             # empty pool
    assert call(a2=FAKE + 8) == ALIGN

    d = lib.paged_attention_decode_fp8

    def dec(**kw):
        a = dict(scale=0.1, ks=1.0, vs=1.0, dt=0, nwg=1, ws=None, wsb=0, s=4, d=128)
        a.update(kw)
        return d(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["scale"], a["ks"], a["vs"], 32, 8,
                 a["d"], 16, a["s"], 8, 128, a["nwg"], a["dt"], a["ws"], a["wsb"], None)

    assert dec(ks=0.0) == INVALID
    assert dec(vs=float("inf")) == INVALID
    assert dec(ks=-2.0) == INVALID
    assert dec(dt=FP8) == UNSUPPORTED                        # q and out are 16-bit
    assert dec(d=96) == UNSUPPORTED
    assert dec(s=0) == OK
    assert dec(nwg=32) == WORKSPACE
    assert dec(nwg=32, ws=FAKE, wsb=_ws(32) - 1) == WORKSPACE


def test_swap_blocks_argument_errors():
    lib = pkv.load_library()
    total = pkv.kv_pool_bytes(2, 16, 4, 128, 16, pkv.PKV_BF16)
    dev = pkv.kv_pool_create(FAKE, total, 2, 16, 4, 128, 16, pkv.PKV_BF16)
    total_h = pkv.kv_pool_bytes(2, 8, 4, 128, 16, pkv.PKV_BF16)
    host = pkv.kv_pool_create(FAKE * 3, total_h, 2, 8, 4, 128, 16, pkv.PKV_BF16)
    other = pkv.kv_pool_create(FAKE * 3, total_h, 2, 8, 4, 64, 16, pkv.PKV_BF16)
    fp8 = pkv.kv_pool_create(FAKE * 3, total_h, 2, 8, 4, 128, 16, pkv.PKV_FP8_E4M3)
    f = lib.swap_blocks
    assert f(dev._h, host._h, None, None, 0, 0, None) == OK      # nothing to copy
    assert f(dev._h, host._h, None, None, 0, 1, None) == OK
    assert f(None, host._h, FAKE, FAKE, 1, 0, None) == INVALID
    assert f(dev._h, None, FAKE, FAKE, 1, 0, None) == INVALID
    assert f(dev._h, host._h, FAKE, FAKE, 1, 2, None) == INVALID   # no such direction
    assert f(dev._h, host._h, FAKE, FAKE, -1, 0, None) == INVALID
    assert f(dev._h, host._h, FAKE, FAKE, 65536, 0, None) == INVALID
    assert f(dev._h, other._h, FAKE, FAKE, 1, 0, None) == INVALID  # head_dim differs
    assert f(dev._h, fp8._h, FAKE, FAKE, 1, 1, None) == INVALID    # element type differs
    assert f(dev._h, host._h, None, FAKE, 1, 0, None) == INVALID
    assert f(dev._h, host._h, FAKE + 2, FAKE, 1, 0, None) == ALIGN
    for p in (dev, host, other, fp8):
        p.destroy()


def test_fused_append_argument_errors():
    lib = pkv.load_library()
    f = lib.paged_attention_decode_append
    f8 = lib.paged_attention_decode_append_fp8

    def call(key=FAKE, value=FAKE, s=4, d=128, nwg=1, ws=None, wsb=0, kv=FAKE):
        return f(FAKE, FAKE, key, value, kv, FAKE, FAKE, FAKE, 0.1, 32, 8, d, 16, s, 8, 128, nwg,
                 0, ws, wsb, None)

    assert call(key=None) == INVALID                        # the new rows are required
    assert call(value=None) == INVALID
    assert call(key=FAKE + 4) == ALIGN
    assert call(d=96) == UNSUPPORTED
    assert call(s=0, key=None, value=None) == OK              # nothing to do
    assert call(nwg=32) == WORKSPACE
    assert call(kv=FAKE + 8) == ALIGN
    assert f8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 0.0, 1.0, 32, 8, 128, 16, 4, 8,
              128, 1, 0, None, 0, None) == INVALID            # k_scale must be > 0
    assert f8(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1.0, 1.0, 32, 8, 128, 16, 4, 8,
              128, 1, 0, None, 0, None) == INVALID
