"""Decode benchmark: one step = reshape_and_cache + paged_attention_decode for every layer.

Default workload: the Llama-3-70B-shaped batch (64 sequences x 4096 tokens, 64 query / 8 kv
heads, head dim 128, bf16, 80 layers in one 80 GiB K+V pool, 16384 blocks per layer scattered by
a seeded permutation). The default run also measures the Llama-3-8B-shaped ragged batch (8 layers)
as "secondary", and the CPU oracle as "cpu_baseline". Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--layers L] [--no-cpu-baseline]
                  [--no-secondary]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth, GB/s
METRIC = "decode KV-read GB/s (% of MI355X HBM peak) + tokens/s per layer-step"
# Workloads --config selects (the batches of workloads.SPECS).
SPEC_NAMES = {1: "tiny 4-sequence MHA batch", 2: "13B-shaped MHA batch (fp16)",
              3: "Llama-3-8B-shaped ragged GQA batch", 4: "Llama-3-70B-shaped GQA batch, 80 layers",
              5: "shared-prefix + skew GQA batch"}
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_452_amd", "csrc", f)
               for f in ("decode.hip", "pkv_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def algorithmic_bytes(lens, num_q_heads, num_kv_heads, head_dim, elem=2, block=16, kv_elem=None,
                      fused=False):
    """Bytes one decode launch must move: every cached K and V row of every sequence once per kv
    head, q in, out back, the used block-table entries and the context lengths. elem: bytes of a
    q/out element; kv_elem: bytes of a pool element (default elem; 1 for fp8 pools). fused: the
    launch also appends each sequence's newest token (its K/V rows read from the step's input
    instead of the pool, and written into the pool)."""
    kv_elem = elem if kv_elem is None else kv_elem
    kv = sum(int(n) for n in lens) * num_kv_heads * head_dim * kv_elem * 2
    if fused:
        new = sum(1 for n in lens if int(n) > 0) * num_kv_heads * head_dim * 2
        kv += new * (elem - kv_elem) + new * kv_elem   # input rows instead of pool rows, + write
    qo = len(lens) * num_q_heads * head_dim * elem * 2
    tables = sum(-(-int(n) // block) for n in lens) * 4
    return kv + qo + tables + 4 * len(lens)


def unique_kv_bytes(block_tables, lens, num_kv_heads, head_dim, kv_elem=2, block=16):
    """K and V bytes of one launch counting each physical block once: for every block some table
    references, the slots any sequence uses in it (a shared prefix block is read by every
    sequence that shares it, but holds its bytes once)."""
    used = {}
    for s, n in enumerate(lens):
        n = int(n)
        for j in range(-(-n // block)):
            b = int(block_tables[s][j])
            used[b] = max(used.get(b, 0), min(block, n - j * block))
    return sum(used.values()) * num_kv_heads * head_dim * kv_elem * 2


def percentiles(xs, qs=(10, 50, 90)):
    """Nearest-rank percentiles of a small list."""
    xs = sorted(xs)
    return {f"p{q}": xs[min(len(xs) - 1, max(0, -(-q * len(xs) // 100) - 1))] for q in qs}


def code_hash(text: str) -> str:
    """Hash of a C++ source with its // comments, trailing spaces and blank lines removed, so that
    a comment edit does not invalidate counters taken on the same code."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def source_hash() -> str:
    """Code hash of the decode kernel's sources (the kernel file and the internal header)."""
    text = ""
    for path in DECODE_SRCS:
        with open(path, encoding="utf-8") as f:
            text += f.read() + "\n"
    return code_hash(text)


def measured_traffic(workload: str):
    """L2-to-fabric bytes per decode launch (reads and writes) from the committed rocprofv3
    counter summary, if it was taken on the current kernel code (comments aside) and this
    workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f).get("records", [])
    except (OSError, ValueError, AttributeError):
        return None
    for rec in recs:
        if rec.get("decode_code_sha256_16") == source_hash() and rec.get("workload") == workload:
            return rec.get("bytes_per_launch")
    return None


def cpu_baseline(batch, spec, layers, budget_s=15.0, kv_scales=None):
    """The fp64 oracle on the host cores over whole layers of the same batch (bounded).
    kv_scales: (k_scale, v_scale) when the pools hold fp8 codes."""
    import numpy as np
    import torch
    import oracle

    threads = len(os.sched_getaffinity(0))
    t = batch.tables
    qdt = oracle.BF16 if spec.dtype == "bf16" else oracle.FP16
    per_layer = algorithmic_bytes(t.context_lens, spec.num_q_heads, spec.num_kv_heads,
                                  spec.head_dim, block=spec.block_size,
                                  kv_elem=1 if kv_scales else 2)
    done_bytes, cpu_s, d2h_s, n_layers = 0, 0.0, 0.0, 0
    q = batch.q.cpu()
    for L in layers:
        t0 = time.perf_counter()
        if kv_scales:
            kw = batch.k_pool[L].cpu().numpy()
            vw = batch.v_pool[L].cpu().numpy()
        else:
            kw = batch.k_pool[L].view(torch.int16).cpu().numpy().view(np.uint16)
            vw = batch.v_pool[L].view(torch.int16).cpu().numpy().view(np.uint16)
        d2h_s += time.perf_counter() - t0
        t0 = time.perf_counter()
        if kv_scales:
            oracle.paged_decode8(q, kw, vw, kv_scales[0], kv_scales[1], t.block_tables,
                                 t.context_lens, spec.scale, spec.num_q_heads, spec.num_kv_heads,
                                 spec.head_dim, spec.block_size, t.num_blocks, qdt,
                                 threads=threads)
        else:
            oracle.paged_decode(q, kw, vw, t.block_tables, t.context_lens, spec.scale,
                                spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                                spec.block_size, t.num_blocks, qdt, threads=threads)
        cpu_s += time.perf_counter() - t0
        done_bytes += per_layer
        n_layers += 1
        if cpu_s >= budget_s:
            break
    # The same oracle on one thread, over every head of the first sequences of the last layer
    # (about 100 MB of K/V), for the per-core rate.
    lens = np.asarray(t.context_lens)
    n_seq = 1
    while n_seq < len(lens) and algorithmic_bytes(lens[:n_seq], spec.num_q_heads,
                                                  spec.num_kv_heads, spec.head_dim,
                                                  block=spec.block_size,
                                                  kv_elem=1 if kv_scales else 2) < 100e6:
        n_seq += 1
    pairs = [(s, h) for s in range(n_seq) for h in range(spec.num_q_heads)]
    one_bytes = algorithmic_bytes(lens[:n_seq], spec.num_q_heads, spec.num_kv_heads,
                                  spec.head_dim, block=spec.block_size,
                                  kv_elem=1 if kv_scales else 2)
    t0 = time.perf_counter()
    if kv_scales:
        oracle.paged_decode8(q, kw, vw, kv_scales[0], kv_scales[1], t.block_tables,
                             t.context_lens, spec.scale, spec.num_q_heads, spec.num_kv_heads,
                             spec.head_dim, spec.block_size, t.num_blocks, qdt, pairs=pairs,
                             threads=1)
    else:
        oracle.paged_decode(q, kw, vw, t.block_tables, t.context_lens, spec.scale,
                            spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size,
                            t.num_blocks, qdt, pairs=pairs, threads=1)
    one_s = time.perf_counter() - t0
    return {"value": round(done_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n_layers} whole layer(s) of the same batch ({spec.num_seqs} seqs x "
                      f"{spec.num_q_heads} heads each), fp64, timed from host-resident pools; "
                      f"device-to-host copy {d2h_s:.2f} s not included",
            "seconds": round(cpu_s, 3),
            "single_thread": {"value": round(one_bytes / one_s / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "sample": f"every head of the first {n_seq} "
                              f"sequence(s) of one layer", "seconds": round(one_s, 3)}}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_rates(min_bytes: float = 100e6):
    """The oracle on one host thread over the tiny, 13B-shaped and 8B-shaped batches (one layer
    each, built on the GPU and copied to the host): the whole tiny batch (repeated for at least
    0.2 s), and every head of the first sequences of the others until about 100 MB of K/V."""
    import numpy as np
    import torch
    import oracle
    import workloads

    rates = {}
    for idx in (1, 2, 3):
        spec = workloads.SPECS[idx]
        t = workloads.make_tables(spec)
        b = workloads.make_batch(spec, device="cuda", tables=t)
        h = b.kv_pool[0].view(torch.int16).cpu().numpy().view(np.uint16)
        kw, vw = np.ascontiguousarray(h[:, :, 0, :]), np.ascontiguousarray(h[:, :, 1, :])
        q = b.q.cpu()
        del b
        lens = np.asarray(t.context_lens)
        qdt = oracle.BF16 if spec.dtype == "bf16" else oracle.FP16
        n_seq = 1
        while n_seq < len(lens) and algorithmic_bytes(
                lens[:n_seq], spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                block=spec.block_size) < min_bytes:
            n_seq += 1
        pairs = [(s, hh) for s in range(n_seq) for hh in range(spec.num_q_heads)]
        nbytes = algorithmic_bytes(lens[:n_seq], spec.num_q_heads, spec.num_kv_heads,
                                   spec.head_dim, block=spec.block_size)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_decode(q, kw, vw, t.block_tables, t.context_lens, spec.scale,
                                spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                                spec.block_size, t.num_blocks, qdt, pairs=pairs, threads=1)
            reps += 1
            if time.perf_counter() - t0 >= 0.2:
                break
        sec = (time.perf_counter() - t0) / reps
        rates[SPEC_NAMES[idx]] = {
            "value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": (f"every head of the first {n_seq} of {len(lens)} sequences of one layer "
                       f"({nbytes / 1e6:.1f} MB of algorithmic bytes)"),
            "seconds_per_sample": round(sec, 4)}
        torch.cuda.empty_cache()
    return rates


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 3) -> int:
    """A plain device copy of known size, to scale the HBM byte counters of a profiler run."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "reps": reps}), flush=True)
    return 0


def bench_copy_blocks(args) -> int:
    """Copy-on-write block copies on the 70B-shaped pool: 64 pairs (one per sequence of the
    batch), every layer, K and V. Bytes = 2 (read + write) x pairs x layers x 2 x block bytes."""
    import numpy as np
    import torch
    import paged_kv_cache_452_amd as pkv
    import workloads

    spec = workloads.SPECS[4]
    L, NB, Hkv, D = spec.num_layers, 16384, spec.num_kv_heads, spec.head_dim
    kv = workloads.new_pool(L, NB, Hkv, 16, D, torch.bfloat16, "cuda")
    kv.view(torch.int16).random_(-32768, 32767)
    pool = pkv.kv_pool_create(kv, kv.numel() * 2, L, NB, Hkv, D, 16, pkv.PKV_BF16)
    rng = np.random.default_rng(7)
    perm = rng.permutation(NB).astype(np.int32)
    npairs = 64
    src = torch.from_numpy(perm[:npairs].copy()).cuda()
    dst = torch.from_numpy(perm[npairs:2 * npairs].copy()).cuda()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pkv.copy_blocks(pool, src, dst, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        pkv.copy_blocks(pool, src, dst, stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    block_bytes = Hkv * 16 * D * 2
    moved = 2 * npairs * L * 2 * block_bytes
    gbs = moved / (us * 1e-6) / 1e9
    # CPU oracle beside it: the same copies as numpy block assignments on host copies of 8 layers.
    kvh = kv[:8].view(torch.int16).cpu().numpy()
    s_np, d_np = perm[:npairs], perm[npairs:2 * npairs]
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 2.0:
        kvh[:, d_np] = kvh[:, s_np]
        reps += 1
    cpu_s = (time.perf_counter() - t0) / reps
    cpu_gbs = 2 * npairs * 8 * 2 * block_bytes / cpu_s / 1e9
    print(json.dumps({
        "metric": "copy_blocks GB/s (read + write, % of MI355X HBM peak)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "us_per_call": round(us, 2), "higher_is_better": True, "data": "synthetic",
        "dtype": "bf16",
        "config": {"workload": "copy-on-write burst on the 70B-shaped pool: 64 block copies x "
                               "80 layers, K and V (64 KiB per block region)",
                   "bytes_per_call": moved},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": "numpy block copies of the same 64 pairs on host copies of 8 "
                                   "layers, single thread"}}), flush=True)
    return 0


PCIE_PEAK_GBS = 64.0    # PCIe 5.0 x16, per direction: the MI355X host link


def bench_swap(args) -> int:
    """Preemption by swapping on the 70B-shaped pool: the blocks of 2 of the batch's 64 sequences
    (512 blocks) go to a pinned host pool and come back, every layer, K and V. Bytes per call =
    pairs x layers x 2 x block bytes, each crossing the host link once."""
    import numpy as np
    import torch
    import paged_kv_cache_452_amd as pkv
    import workloads

    spec = workloads.SPECS[4]
    t = workloads.make_tables(spec)
    L, NB, Hkv, D, B = spec.num_layers, t.num_blocks, spec.num_kv_heads, spec.head_dim, 16
    kv = workloads.new_pool(L, NB, Hkv, B, D, torch.bfloat16, "cuda").zero_()
    victims = np.concatenate([t.block_tables[0], t.block_tables[1]]).astype(np.int32)
    n = victims.shape[0]
    hkv = workloads.new_pool(L, n, Hkv, B, D, torch.bfloat16, "cpu", pin_memory=True)
    dpool = pkv.kv_pool_create(kv, kv.numel() * 2, L, NB, Hkv, D, B, pkv.PKV_BF16)
    hpool = pkv.kv_pool_create(hkv, hkv.numel() * 2, L, n, Hkv, D, B, pkv.PKV_BF16)
    dev_ids = torch.from_numpy(victims).cuda()
    host_ids = torch.arange(n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    moved = n * L * 2 * Hkv * B * D * 2

    def timed(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    swap_out = lambda: pkv.swap_blocks(dpool, hpool, dev_ids, host_ids, pkv.PKV_SWAP_OUT, stream)
    swap_in = lambda: pkv.swap_blocks(dpool, hpool, host_ids, dev_ids, pkv.PKV_SWAP_IN, stream)
    for _ in range(max(1, args.warmup)):
        swap_out()
        swap_in()
    reps = max(1, args.steps)
    ms_out = timed(swap_out, reps)
    ms_in = timed(swap_in, reps)
    # The link's own ceiling on this machine: one contiguous pinned copy of the same size each way
    # (the runtime's DMA path).
    flat_d = torch.empty(moved // 2, dtype=torch.bfloat16, device="cuda")
    flat_h = torch.empty(moved // 2, dtype=torch.bfloat16, pin_memory=True)
    flat_h.copy_(flat_d, non_blocking=True)
    flat_d.copy_(flat_h, non_blocking=True)
    ms_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), reps)
    ms_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), reps)
    # The copy-engine path (swap_blocks_dma): ids on the host, one strided copy per block.
    dev_h = np.ascontiguousarray(victims)
    host_h = np.arange(n, dtype=np.int32)
    dma_out = lambda st: pkv.swap_blocks_dma(dpool, hpool, dev_h, host_h, pkv.PKV_SWAP_OUT, st)
    dma_in = lambda st: pkv.swap_blocks_dma(dpool, hpool, host_h, dev_h, pkv.PKV_SWAP_IN, st)
    dma_out(stream)
    dma_in(stream)
    ms_dma_out = timed(lambda: dma_out(stream), reps)
    ms_dma_in = timed(lambda: dma_in(stream), reps)
    # A decode sweep over all layers of the 64-sequence batch on one stream, alone and while each
    # kind of swap out runs on another (the swap outlasts the sweep).
    Hq = spec.num_q_heads
    S = spec.num_seqs
    gq = torch.Generator(device="cuda").manual_seed(11)
    q = workloads.randn((S, Hq, D), torch.bfloat16, gq, "cuda")
    k_planes, v_planes = workloads.planes(kv)
    bt = torch.from_numpy(t.block_tables).cuda()
    cl = torch.from_numpy(t.context_lens).cuda()
    max_ctx = int(t.context_lens.max())
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(S, Hq, Hkv, D, B, max_ctx, 0),
                           "cuda")
    dec_out = torch.empty_like(q)
    s_dec, s_swap = torch.cuda.Stream(), torch.cuda.Stream()  # default priority

    def sweep(st):
        for layer in range(L):
            pkv.paged_attention_decode(dec_out, q, k_planes[layer], v_planes[layer], bt, cl,
                                       spec.scale, Hq, Hkv, D, B, max_ctx, 0, ws, st)

    def decode_ms(swap_fn):
        times = []
        for _ in range(3):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            if swap_fn is not None:
                swap_fn(s_swap)
            a.record(s_dec)
            sweep(s_dec)
            e.record(s_dec)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(e))
        return sorted(times)[1]

    sweep(s_dec)
    kernel_out = lambda st: pkv.swap_blocks(dpool, hpool, dev_ids, host_ids, pkv.PKV_SWAP_OUT, st)
    beside = {"decode_alone_ms": decode_ms(None),
              "beside_swap_blocks_ms": decode_ms(kernel_out),
              "beside_swap_blocks_dma_ms": decode_ms(dma_out)}
    gbs = lambda ms: moved / (ms * 1e-3) / 1e9
    out_gbs, in_gbs = gbs(ms_out), gbs(ms_in)
    rt = 2 * moved / ((ms_out + ms_in) * 1e-3) / 1e9
    # CPU oracle beside it: the same block gather as numpy on host copies of 2 layers.
    rng = np.random.default_rng(3)
    kh = rng.integers(0, 65535, size=(2, NB, 2 * Hkv * B * D), dtype=np.uint16)
    dst = np.zeros((2, n, 2 * Hkv * B * D), np.uint16)
    t0 = time.perf_counter()
    creps = 0
    while time.perf_counter() - t0 < 2.0:
        dst[:] = kh[:, victims]
        creps += 1
    cpu_gbs = 2 * n * 2 * Hkv * B * D * 2 / ((time.perf_counter() - t0) / creps) / 1e9
    print(json.dumps({
        "metric": "swap_blocks GB/s over the host link (swap out + swap in)", "value": round(rt, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "higher_is_better": True, "data": "synthetic", "dtype": "bf16",
        "config": {"workload": "preempt 2 of 64 sequences of the 70B-shaped batch: 512 blocks x 80 "
                               "layers, K and V (64 KiB per block region), to a pinned host "
                               "pool and back", "bytes_per_call": moved},
        "swap_out_ms": round(ms_out, 3), "swap_out_gbs": round(out_gbs, 2),
        "swap_in_ms": round(ms_in, 3), "swap_in_gbs": round(in_gbs, 2),
        "swap_blocks_dma": {"out_ms": round(ms_dma_out, 3), "out_gbs": round(gbs(ms_dma_out), 2),
                            "in_ms": round(ms_dma_in, 3), "in_gbs": round(gbs(ms_dma_in), 2),
                            "what": "the same swaps on the copy engines (one strided copy per "
                                    "block, ids read on the host)"},
        "decode_beside_swap_out": dict({k: round(v, 3) for k, v in beside.items()},
                                       what=f"decode of all {L} layers of the 64-sequence batch "
                                            "on one stream, alone and while a swap out runs on "
                                            "another"),
        "dma_copy_same_bytes": {"d2h_gbs": round(gbs(ms_d2h), 2), "h2d_gbs": round(gbs(ms_h2d), 2),
                                "what": "one contiguous pinned hipMemcpyAsync each way"},
        "roofline": {"bound": "host link", "achieved": round(rt, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(rt / PCIE_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": "numpy gather of the same 512 blocks (K and V) from host "
                                   "copies of 2 layers of one pool"},
    }), flush=True)
    for p in (dpool, hpool):
        p.destroy()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, choices=sorted(SPEC_NAMES),
                    help="workload: " + "; ".join(f"{k} = {v}" for k, v in SPEC_NAMES.items()))
    ap.add_argument("--workgroups", type=int, default=0,
                    help="decode workgroups (0: the library's choice)")
    ap.add_argument("--block-size", type=int, default=16, choices=[16, 32])
    ap.add_argument("--layers", type=int, default=0,
                    help="layers in the pool (default: the workload's own; more layers of fresh "
                         "data keep a small single-layer workload from being served out of the "
                         "256 MB last-level cache between launches)")
    ap.add_argument("--kv-dtype", choices=["model", "fp8"], default="model",
                    help="pool element type: the model's 16-bit type (default) or E4M3 codes "
                         "with one scale per pool")
    ap.add_argument("--fused", action="store_true",
                    help="run each layer's step as one paged_attention_decode_append launch "
                         "instead of reshape_and_cache followed by paged_attention_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 8B-shaped batch measured after the default 70B-shaped one")
    ap.add_argument("--kernel", choices=["decode", "copy_blocks", "swap"], default="decode",
                    help="decode (the hot path, default), copy_blocks (copy-on-write copies) or "
                         "swap (preemption to and from pinned host memory)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this decode path is built and measured on a single "
              f"MI355X; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_452_amd as pkv
    import workloads

    if args.calibrate_copy:
        return calibrate_copy()
    if args.kernel == "copy_blocks":
        return bench_copy_blocks(args)
    if args.kernel == "swap":
        return bench_swap(args)
    pkv.load_library()
    spec = workloads.SPECS[args.config]
    if args.layers > 0:
        spec = dataclasses.replace(spec, num_layers=args.layers)
    if args.block_size != spec.block_size:
        spec = dataclasses.replace(spec, block_size=args.block_size)
    fp8 = args.kv_dtype == "fp8"
    m = measure_decode(spec, args.steps, args.warmup, args.workgroups, fp8, args.fused,
                       named_layers=args.layers > 0)
    t, L, S = m["tables"], spec.num_layers, spec.num_seqs
    Hq, Hkv, D, B = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    rec = {
        "metric": METRIC,
        "value": round(m["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": m["workload"], "num_seqs": S, "context_lens": "all 4096" if
                   args.config == 4 else "seeded", "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": B, "num_layers": L,
                   "num_blocks_per_layer": t.num_blocks, "decode_workgroups": m["grid"],
                   "kv_dtype": "fp8 e4m3, one scale per pool" if fp8 else spec.dtype,
                   "step": ("per layer: reshape_and_cache of the step's new tokens, then "
                            "paged_attention_decode" if not args.fused else
                            "per layer: one paged_attention_decode_append launch (the step's new "
                            "tokens appended to the pool and attended to with the cached "
                            "context)")},
        "pct_of_hbm_peak": round(100.0 * m["value"] / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer_step": round(S * L / (m["ms_step"] * 1e-3), 1),
        "decode_launch_us": round(m["decode_us"], 2),
        "decode_launch_us_spread": m["spread"],
        "timing": "roofline.achieved: back-to-back step launches of the decode kernel over all "
                  "layers between two HIP events on the launch stream (mean launch duration), "
                  "timed first; value: K whole steps between two HIP events",
        "roofline": m["roofline"],
    }
    if "unique_kv" in m:
        rec["unique_kv"] = m["unique_kv"]
    import torch
    props = torch.cuda.get_device_properties(0)
    rec["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count, "hip": torch.version.hip,
                     "torch": torch.__version__}
    # The second workload the decode is held to: the Llama-3-8B-shaped ragged batch, measured in
    # the same run right after the first (8 layers of fresh data, so that no layer is read from
    # the last-level cache; warmed up for at least 0.25 s so that the GPU clocks are settled).
    if args.config == 4 and args.layers <= 0 and not args.no_secondary:
        spec3 = dataclasses.replace(workloads.SPECS[3], num_layers=8,
                                    block_size=args.block_size)
        m3 = measure_decode(spec3, 40, 10, args.workgroups, fp8, args.fused, named_layers=True,
                            min_warmup_s=0.25)
        rec["secondary"] = {
            "workload": m3["workload"],
            "decode_launch_us": round(m3["decode_us"], 2),
            "decode_launch_us_spread": m3["spread"],
            "ms_per_step": round(m3["ms_step"], 4),
            "value": round(m3["value"], 2), "unit": "GB/s",
            "tokens_per_s_per_layer_step": round(spec3.num_seqs * 8 / (m3["ms_step"] * 1e-3), 1),
            "decode_workgroups": m3["grid"],
            "roofline": m3["roofline"]}
        del m3
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(m["batch"], spec, range(L),
                                           kv_scales=FP8_SCALES if fp8 else None)
    del m
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"]["single_thread_by_workload"] = single_thread_rates()
    print(json.dumps(rec), flush=True)
    return 0


FP8_SCALES = (0.05, 0.05)   # per-pool scales of the fp8 path (values do not change its cost)


def measure_decode(spec, steps, warmup, nwg, fp8, fused, named_layers=False, min_warmup_s=0.0):
    """Build a seeded batch of `spec` on the GPU and time it: back-to-back decode launches over
    all layers (mean launch duration, and the spread of per-sweep means), then whole steps (per
    layer: reshape_and_cache, then decode; or the fused launch). The warm-up runs `warmup` steps,
    and more until min_warmup_s seconds have passed. Returns the timings, the roofline record and
    the batch."""
    import torch
    import paged_kv_cache_452_amd as pkv
    import workloads

    dev = "cuda"
    B = spec.block_size
    t = workloads.make_tables(spec)
    ks, vs = FP8_SCALES
    if fp8:
        batch = workloads.make_batch_fp8(spec, device=dev, tables=t)
    else:
        batch = workloads.make_batch(spec, device=dev, tables=t)
    S, Hq, Hkv, D, L = (spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                        spec.num_layers)
    max_ctx = int(t.context_lens.max())
    ws = pkv.new_workspace(pkv.paged_attention_workspace_bytes(S, Hq, Hkv, D, B, max_ctx, nwg),
                           dev)
    outs = torch.empty((L, S, Hq, D), dtype=batch.q.dtype, device=dev)
    layers = [(batch.k_pool[i], batch.v_pool[i]) for i in range(L)]
    stream = torch.cuda.current_stream()

    def cache(k, v):
        if fp8:
            pkv.reshape_and_cache_fp8(batch.new_key, batch.new_value, k, v, batch.slot_mapping,
                                      t.num_blocks, ks, vs, B, stream)
        else:
            pkv.reshape_and_cache(batch.new_key, batch.new_value, k, v, batch.slot_mapping,
                                  t.num_blocks, B, stream)

    def decode(i, k, v):
        if fused:
            pkv.paged_attention_decode_append(outs[i], batch.q, batch.new_key, batch.new_value,
                                              k, v, batch.block_tables, batch.context_lens,
                                              spec.scale, Hq, Hkv, D, B, max_ctx, nwg, ws, stream,
                                              kv_scales=(ks, vs) if fp8 else None)
        elif fp8:
            pkv.paged_attention_decode_fp8(outs[i], batch.q, k, v, batch.block_tables,
                                           batch.context_lens, spec.scale, ks, vs, Hq, Hkv, D, B,
                                           max_ctx, nwg, ws, stream)
        else:
            pkv.paged_attention_decode(outs[i], batch.q, k, v, batch.block_tables,
                                       batch.context_lens, spec.scale, Hq, Hkv, D, B, max_ctx,
                                       nwg, ws, stream)

    def step():
        for i, (k, v) in enumerate(layers):
            if not fused:
                cache(k, v)
            decode(i, k, v)

    def sweep_decode():
        for i, (k, v) in enumerate(layers):
            decode(i, k, v)

    t_warm = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_warm < min_warmup_s:
        step()
        done += 1
        if done >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # Timed region B: the decode kernel alone, launched back to back over the layers; the mean
    # launch duration is the region's time over the launch count. An event after every sweep
    # (between launches, not inside any) also gives the spread of the per-sweep means.
    reps_b = max(1, steps // 2)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps_b + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for r in range(reps_b):
        sweep_decode()
        marks[r + 1].record(stream)
    torch.cuda.synchronize()
    avg_decode_ms = marks[0].elapsed_time(marks[-1]) / (reps_b * L)
    sweep_us = [marks[r].elapsed_time(marks[r + 1]) * 1e3 / L for r in range(reps_b)]
    # Timed region A: whole steps, no markers inside.
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps

    kv_elem = 1 if fp8 else 2
    per_launch = algorithmic_bytes(t.context_lens, Hq, Hkv, D, block=B, kv_elem=kv_elem,
                                   fused=fused)
    achieved = per_launch / (avg_decode_ms * 1e-3) / 1e9
    workload = ((spec.name if not named_layers else f"{spec.name}, {L} layers") +
                ("" if B == 16 else f", block size {B}") + (", fp8 E4M3 KV" if fp8 else "") +
                (", fused step" if fused else ""))
    traffic = measured_traffic(workload)
    res = {
        "tables": t, "batch": batch, "workload": workload,
        "grid": nwg or pkv.paged_attention_num_workgroups(S, Hq, Hkv, max_ctx, B),
        "decode_us": avg_decode_ms * 1e3, "ms_step": ms_step,
        "value": per_launch * L / (ms_step * 1e-3) / 1e9,
        "spread": dict({k: round(v, 2) for k, v in percentiles(sweep_us).items()},
                       sweeps=reps_b, launches_per_sweep=L),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_source": (f"{os.path.relpath(TRAFFIC_FILE, ROOT)}: L2-to-fabric "
                                        "bytes per launch (rocprofv3 TCC_EA0 read requests of "
                                        "32, 64 and 128 bytes and write requests of 32 and 64 "
                                        "bytes, times their sizes) of this workload, taken on "
                                        "the same decode code (hash of the kernel sources "
                                        "without comments); gfx950 has no MALL counter, so MALL "
                                        "hits are included") if traffic else None,
                     "algorithmic_bytes_per_launch": per_launch,
                     "kernel": ("paged_attention_decode" if not fused else
                                "paged_attention_decode_append") +
                               " (one persistent decode kernel; split streams merged in it)"},
    }
    uniq = unique_kv_bytes(t.block_tables, t.context_lens, Hkv, D, kv_elem=kv_elem, block=B)
    logical = algorithmic_bytes(t.context_lens, Hq, Hkv, D, block=B, kv_elem=kv_elem) - \
        algorithmic_bytes(t.context_lens, Hq, Hkv, D, block=B, kv_elem=0)
    if uniq < logical:   # blocks shared between sequences (a common prefix)
        res["unique_kv"] = {"bytes_per_launch": uniq, "logical_kv_bytes_per_launch": logical,
                            "gbps_at_decode_time": round(uniq / (avg_decode_ms * 1e-3) / 1e9, 2),
                            "what": "K/V bytes counting each physical block once (a shared "
                                    "prefix is read by every sharer but stored once)"}
    return res

if __name__ == "__main__":
    sys.exit(main())
