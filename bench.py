#!/usr/bin/env python3
"""Bench: one step of the paged, quantized KV-cache hot path on one MI355X.

A step is the whole path over one batch of synthetic input: the step's cache write of the
new K/V rows, the paged decode and, when the context is split into partitions, the
log-sum-exp merge (pa_merge). Where one new token per sequence goes to its last position
in a 16-bit or FP8 pool, the write and the decode run as one pa_append_decode launch;
otherwise (FP4 pools, or --separate-write) as pa_cache_write + pa_decode. The default workload is the
Llama-3.1-70B tensor-parallel one-GPU share: 256 sequences of 8192 tokens, 8 query heads
over 1 kv head, head_dim 128, FP8 E4M3 KV cache (xonoai.com field report on vLLM v0.7.2,
"Comparative Inference Engine Performance": 256 concurrent 8k-token streams of the 70B
model on 8 GPUs). Inputs are resident in HBM before the timed region; the pool is kept in
several copies, rotated step by step, so that no step finds its KV in the 256 MB
Infinity Cache left warm by the step before.

Prints one JSON line: value = algorithmic bytes of the step / step time (GB/s), plus the
dominant kernel's roofline (its algorithmic bytes / its average launch time from HIP events
on the launch stream) and the oracle's rate on the host cores (cpu_baseline).

    python bench.py [--steps K (300)] [--warmup W (50)] [--config c4] [--partition-size PS]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "paged decode attention: achieved KV-read GB/s (% HBM peak) + seq-tokens/s"
# the sources that decide the decode kernel's code and launch (the wave count is chosen in
# pa_api.cpp): committed counter traffic is used only while their hash is unchanged
KERNEL_SOURCES = ["paged_quantized_kv_reshape_amd/csrc/pa_decode.hip",
                  "paged_quantized_kv_reshape_amd/csrc/pa_tile.h",
                  "paged_quantized_kv_reshape_amd/csrc/pa_encode.h",
                  "paged_quantized_kv_reshape_amd/csrc/pa_fp4.h",
                  "paged_quantized_kv_reshape_amd/csrc/pa_device.h",
                  "paged_quantized_kv_reshape_amd/csrc/pa_api.cpp",
                  "paged_quantized_kv_reshape_amd/csrc/pa_launch.h"]
# the sources that decide the multi-token kernel's code and launch
PREFILL_SOURCES = ["paged_quantized_kv_reshape_amd/csrc/pa_prefill.hip",
                   "paged_quantized_kv_reshape_amd/csrc/pa_tile.h",
                   "paged_quantized_kv_reshape_amd/csrc/pa_device.h",
                   "paged_quantized_kv_reshape_amd/csrc/pa_launch.h",
                   "paged_quantized_kv_reshape_amd/csrc/pa_api.cpp"]
# decode output tolerance against the oracle: max |gpu - oracle| and relative L2 error
ATOL, RTOL_L2 = 2e-3, 1e-2


class HipTimer:
    """HIP timing events created with hipEventReleaseToDevice, recorded on a given stream.
    A default event performs a system-scope release when it is recorded (cache write-back
    and invalidation), which adds microseconds between the kernels it brackets; a
    device-scope release is enough for timing. The events come from the HIP runtime
    already loaded in this process (the one torch and libpa share)."""

    FLAGS = 0x40000000  # hipEventReleaseToDevice

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def event(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.events.append(e)
        return e

    def record(self, e, stream: int):
        if self.hip.hipEventRecord(e, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        t = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def kernel_source_hash(sources=None) -> str:
    """First 16 hex digits of the sha256 over the given sources (default: the decode's)."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_name(kv: str, fused: bool = False) -> str:
    """The decode kernel that runs for a pool format (FP4 has its own entry point); with
    the step fused into one launch (pa_append_decode) its append variant."""
    return "k_decode_fp4" if kv == "fp4" else "k_decode_append" if fused else "k_decode"


def counter_traffic(kernel: str, cfg: str, ps: int):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary of this
    workload, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{cfg}_ps{ps}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not tb or src.group(1) != kernel_source_hash():
        return None
    return float(tb.group(1))


def host_cores() -> dict:
    """What the host offers this process: logical CPUs, the ones it may run on, and the
    thread count of each BLAS / OpenMP pool NumPy would use."""
    from threadpoolctl import threadpool_info
    info = threadpool_info()
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": max([i.get("num_threads", 1) for i in info] or [1]),
            "pools": sorted({f"{i.get('internal_api')}:{i.get('num_threads')}" for i in info})}


def cpu_baseline(w, budget_s: float, decode_b_per_token: float):
    """The oracle (fp64 NumPy, unmodified) on a bounded sample of the same workload: the
    cache-write replay of a few whole sequences (every write call of setup and step,
    restricted to their blocks) and their exact decode. Timed twice in this process, first
    with every BLAS thread the host gives, then with one. Returns the record and the
    oracle's outputs {seq: out [Hq, D]} of the sample, for the parity check."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    from oracle import cache as C

    ks = vs = None
    if w.kv in ("fp8", "bf8"):  # inputs of the method (per-head scales), not timed
        fmt = C.FP8_KINDS[w.kv][0]
        ks = C.fp8_head_scale(w.k_rows, w.act, fmt)
        vs = C.fp8_head_scale(w.v_rows, w.act, fmt)
    calls = list(w.setup_calls) + [w.step_call]
    blk_of_call = [c.slots // 16 for c in calls]

    def run(seqs):
        pool = C.Pool.filled(w.kv, w.num_blocks, w.num_kv_heads, w.head_dim)
        t0 = time.perf_counter()
        blocks = set()
        for s in seqs:
            n = -(-int(w.context_lens[s]) // 16)
            blocks.update(int(b) for b in w.block_tables[s, :n])
        keep = np.asarray(sorted(blocks))
        for c, blk in zip(calls, blk_of_call):
            sel = np.isin(blk, keep)
            if sel.any():
                C.cache_write(pool, w.k_rows[c.rows[sel]], w.v_rows[c.rows[sel]], w.act,
                              c.slots[sel], ks, vs)
        res = A.paged_decode(w.q, w.act, pool, w.block_tables, w.context_lens, w.sm_scale, ks,
                             vs, partition_size=w.partition_size, seqs=seqs)
        return time.perf_counter() - t0, res

    cores = host_cores()
    order = list(range(w.num_seqs))
    t1, _ = run(order[:1])
    n = max(1, min(w.num_seqs - 1, int(budget_s / max(t1, 1e-3))))
    sample = order[1:1 + n]
    dt_all, res = run(sample)
    with threadpool_limits(limits=1):
        dt_one, _ = run(sample)
    tokens = int(sum(int(w.context_lens[s]) for s in sample))
    outs = {}
    for s in sample:
        o, lse = res[s]
        outs[s] = A.merge(o, lse)[0] if w.partition_size else o
    gbs = lambda dt: round(tokens * decode_b_per_token / dt / 1e9, 6)
    rec = {"value": gbs(dt_all), "unit": "GB/s", "cores": cores["blas_threads"],
           "kind": "oracle", "seconds": round(dt_all, 2),
           "seq_tokens_per_s": round(tokens / dt_all, 1),
           "host": cores,
           "single_thread": {"value": gbs(dt_one), "unit": "GB/s", "cores": 1,
                             "seconds": round(dt_one, 2),
                             "seq_tokens_per_s": round(tokens / dt_one, 1)},
           "sample": (f"{len(sample)} of {w.num_seqs} sequences ({tokens} KV tokens): replay of "
                      f"every cache-write call into their blocks, then exact fp64 decode "
                      f"(+ partitions and merge) of the sequences; bytes counted as for the "
                      f"GPU step; timed with all BLAS threads, then with one")}
    return rec, outs


def oracle_outputs(w, seqs) -> dict:
    """The oracle's decode of the listed sequences (replay of their blocks, then exact
    decode, merged when split), untimed."""
    import numpy as np

    from oracle import attention as A
    from oracle import cache as C
    ks = vs = None
    if w.kv in ("fp8", "bf8"):
        fmt = C.FP8_KINDS[w.kv][0]
        ks = C.fp8_head_scale(w.k_rows, w.act, fmt)
        vs = C.fp8_head_scale(w.v_rows, w.act, fmt)
    pool = C.Pool.filled(w.kv, w.num_blocks, w.num_kv_heads, w.head_dim)
    blocks = set()
    for s in seqs:
        blocks.update(int(b) for b in w.block_tables[s, :-(-int(w.context_lens[s]) // 16)])
    keep = np.asarray(sorted(blocks))
    for c in list(w.setup_calls) + [w.step_call]:
        sel = np.isin(c.slots // 16, keep)
        if sel.any():
            C.cache_write(pool, w.k_rows[c.rows[sel]], w.v_rows[c.rows[sel]], w.act,
                          c.slots[sel], ks, vs)
    res = A.paged_decode(w.q, w.act, pool, w.block_tables, w.context_lens, w.sm_scale, ks, vs,
                         partition_size=w.partition_size, seqs=seqs)
    return {s: (A.merge(*res[s])[0] if w.partition_size else res[s][0]) for s in seqs}


def parity_check(got, outs) -> dict:
    """The bench's own output against the oracle's on the sampled sequences: elementwise
    max |gpu - oracle| and relative L2 error, both within the decode tolerance."""
    import numpy as np
    g = np.stack([got[s] for s in outs]).astype(np.float64)
    o = np.stack([outs[s] for s in outs])
    max_abs = float(np.abs(g - o).max()) if g.size else 0.0
    rel = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))
    ok = bool(np.isfinite(g).all() and max_abs <= ATOL and rel <= RTOL_L2)
    return {"seqs": len(outs), "max_abs": max_abs, "rel_l2": rel, "atol": ATOL,
            "rtol_l2": RTOL_L2, "ok": ok}


def workload_of(args, config):
    """The named workload, with its KV-cache format replaced when --kv is given (fp4 needs
    head_dim 128; 16-bit pools store the activation dtype, so --kv f16 also makes the
    activations fp16)."""
    if args.kv is None:
        return config(args.config)
    over = dict(kv=args.kv)
    if args.kv in ("f16", "bf16"):
        over["act"] = args.kv
    return config(args.config, **over)


def profile_label(args) -> str:
    """Workload label of the committed profiles: the config name, plus the KV format when
    it was overridden and the FP4 calibration when it is per sequence."""
    label = args.config if args.kv is None else f"{args.config}_{args.kv}"
    return label + ("_seqcal" if getattr(args, "fp4_calibration", "block") == "sequence" else "")


def copy_probe(mib: int):
    """One plain elementwise kernel over mib MiB (n bytes read, n written): the known
    traffic that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: {n} bytes read + {n} written", file=sys.stderr, flush=True)
    del src, dst


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16 host link, per direction, published


def blocks_main(args, config, DESCRIPTIONS):
    """Whole-block copies on the workload's pool geometry: N block copies inside the pool
    (HBM-bound: each block's bytes are read and written once), N blocks swapped out to a
    pool in pinned host memory and back (bound by the host link), and torch's DMA copies of
    one contiguous buffer of the same size as the attainable link rate."""
    import numpy as np
    import torch

    from paged_quantized_kv_reshape_amd import KVPool, pa_copy_blocks, pa_pool_layout

    w = workload_of(args, config)
    nb, hkv, d, kv = w.num_blocks, w.num_kv_heads, w.head_dim, w.kv
    N = args.blocks
    if 2 * N > nb:
        raise SystemExit(f"--blocks {N}: the pool has {nb} blocks, at most {nb // 2} copies")
    per_block = sum(pa_pool_layout(kv, 1, hkv, d))
    ones = torch.ones(hkv, dtype=torch.float32, device="cuda")
    pool = KVPool(kv, nb, hkv, d, fill=0x5A, k_scale=ones, v_scale=ones)
    host = KVPool(kv, N, hkv, d, device="cpu", fill=0)
    rng = np.random.default_rng(0)
    perm = rng.permutation(nb).astype(np.int32)
    cow = torch.from_numpy(np.stack([perm[:N], perm[N:2 * N]], 1).copy()).cuda()
    out_p = torch.from_numpy(np.stack([perm[:N], np.arange(N, dtype=np.int32)], 1).copy()).cuda()
    in_p = torch.from_numpy(np.stack([np.arange(N, dtype=np.int32), perm[N:2 * N]], 1).copy()).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev_buf = torch.empty(N * per_block, dtype=torch.uint8, device="cuda")
    host_buf = torch.empty(N * per_block, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream().cuda_stream
    timer = HipTimer()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = timer.event(), timer.event()
        timer.record(a, stream)
        for _ in range(args.steps):
            fn()
        timer.record(b, stream)
        torch.cuda.synchronize()
        return timer.ms(a, b) * 1e-3 / args.steps

    print(f"[bench] {kv} pool of {nb} blocks ({per_block} B each), {N} blocks per call",
          file=sys.stderr, flush=True)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    t_cow = timed(lambda: pa_copy_blocks(pool, pool, cow, err))
    t_out = timed(lambda: pa_copy_blocks(pool, host, out_p, err))
    t_in = timed(lambda: pa_copy_blocks(host, pool, in_p, err))
    t_d2h = timed(lambda: host_buf.copy_(dev_buf, non_blocking=True))
    t_h2d = timed(lambda: dev_buf.copy_(host_buf, non_blocking=True))
    dev_buf2 = torch.empty_like(dev_buf)
    t_d2d = timed(lambda: dev_buf2.copy_(dev_buf))
    one = cow[:1].contiguous()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(200):
        pa_copy_blocks(pool, pool, one, err)
    host_us = (time.perf_counter() - t0) / 200 * 1e6
    torch.cuda.synchronize()
    timer.close()
    if int(err.item()):
        raise SystemExit(f"device error {int(err.item())}")
    moved = N * per_block
    cow_gbs = 2 * moved / t_cow / 1e9
    res = {
        "metric": "whole-block copy (copy on write) and swap: achieved GB/s",
        "value": round(cow_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_cow * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}"
                               + (f" (KV cache as {kv})" if args.kv else ""),
                   "kv_cache_dtype": kv, "pool_blocks": nb, "bytes_per_block": per_block,
                   "blocks_per_call": N},
        "roofline": {"kernel": "k_copy_blocks", "bound": "hbm", "achieved": round(cow_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(cow_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": 2 * moved, "traffic": None},
        "contiguous_d2d_copy_GBs": round(2 * moved / t_d2d / 1e9, 2),
        "swap": {"out_GBs": round(moved / t_out / 1e9, 2), "in_GBs": round(moved / t_in / 1e9, 2),
                 "out_ms": round(t_out * 1e3, 4), "in_ms": round(t_in * 1e3, 4),
                 "dma_contiguous_d2h_GBs": round(moved / t_d2h / 1e9, 2),
                 "dma_contiguous_h2d_GBs": round(moved / t_h2d / 1e9, 2),
                 "link_peak_GBs": PCIE_PEAK_GBS,
                 "out_frac_of_link": round(moved / t_out / 1e9 / PCIE_PEAK_GBS, 4),
                 "in_frac_of_link": round(moved / t_in / 1e9 / PCIE_PEAK_GBS, 4)},
        "host_us_per_call": round(host_us, 2),
    }
    if not args.no_cpu_baseline:
        from oracle import blocks as OB
        from oracle import cache as C
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        opool = C.Pool.filled(kv, nb, hkv, d)
        pairs = cow.cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0) or reps == 0:
            OB.copy_blocks(opool, opool, pairs)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(2 * moved / dt / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle", "seconds": round(dt * reps, 2),
                               "sample": f"{reps} x the same {N} in-pool copies (NumPy fancy "
                                         f"indexing), bytes counted as for the GPU"}
    print(json.dumps(res), flush=True)


def prefill_flops(w, qs) -> int:
    """Algorithmic flops of multi-token attention: query i of sequence s (position
    L - n + i) does 2 D flops per key for QK and 2 D for PV over L - n + i + 1 keys."""
    tot = 0
    for s in range(w.num_seqs):
        L, n = int(w.context_lens[s]), int(qs[s + 1] - qs[s])
        keys = n * (L - n) + n * (n + 1) // 2
        tot += 4 * w.head_dim * w.num_q_heads * keys
    return tot


def prefill_main(args, config, DESCRIPTIONS):
    """Chunked-prefill attention (pa_prefill) on the chosen workload: every sequence's last
    CHUNK positions are queries over its whole paged context."""
    import numpy as np
    import torch

    from oracle import attention as A
    from oracle import cache as C
    from paged_quantized_kv_reshape_amd import harness as H
    from paged_quantized_kv_reshape_amd import pa_prefill
    from workload import prefill_queries

    print(f"[bench] generating {args.config} (prefill chunk {args.prefill})", file=sys.stderr,
          flush=True)
    w = workload_of(args, config)
    run = H.DeviceRun(w, device="cuda", partition_size=0, pool_copies=1)
    run.prepare()
    torch.cuda.synchronize()
    q_bits, qs = prefill_queries(w, args.prefill)
    tdt = torch.bfloat16 if w.act == "bf16" else torch.float16
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    qs_t = torch.from_numpy(qs).cuda()
    out = torch.empty((q.shape[0], w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    nmax = int(np.diff(qs).max())
    flops = prefill_flops(w, qs)

    def launch():
        pa_prefill(q, qs_t, nmax, run.pool, run.block_tables, run.context_lens, w.sm_scale,
                   out, run.dev_err)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    if run.device_error():
        raise SystemExit(f"device error: {run.device_error()}")
    stream = torch.cuda.current_stream().cuda_stream
    timer = HipTimer()
    a, b = timer.event(), timer.event()
    t0 = time.perf_counter()
    timer.record(a, stream)
    for _ in range(args.steps):
        launch()
    timer.record(b, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    t = timer.ms(a, b) * 1e-3 / args.steps
    timer.close()
    tflops = flops / t / 1e12
    res = {
        "metric": "paged multi-token (chunked prefill) attention: achieved TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.act, "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}"
                               + (f" (KV cache as {w.kv})" if args.kv else ""),
                   "prefill_chunk": args.prefill, "queries": int(qs[-1]),
                   "kv_cache_dtype": w.kv, "num_seqs": w.num_seqs,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim},
        "algorithmic_flops": flops,
        "wall_ms_per_step": round(wall * 1e3, 4),
        "roofline": {"kernel": "k_prefill_mt", "bound": "mfma",
                     "achieved": round(tflops, 2),
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "traffic": None},
        "kernel_source_sha256": kernel_source_hash(PREFILL_SOURCES),
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        with threadpool_limits(limits=1):
            ks = vs = None
            if w.kv in ("fp8", "bf8"):
                fmt = C.FP8_KINDS[w.kv][0]
                ks = C.fp8_head_scale(w.k_rows, w.act, fmt)
                vs = C.fp8_head_scale(w.v_rows, w.act, fmt)
            pool = C.Pool.filled(w.kv, w.num_blocks, w.num_kv_heads, w.head_dim)
            s0 = 0
            n0 = -(-int(w.context_lens[s0]) // 16)
            keep = np.asarray(sorted(int(b) for b in w.block_tables[s0, :n0]))
            for c in list(w.setup_calls) + [w.step_call]:
                sel = np.isin(c.slots // 16, keep)
                if sel.any():
                    C.cache_write(pool, w.k_rows[c.rows[sel]], w.v_rows[c.rows[sel]], w.act,
                                  c.slots[sel], ks, vs)
            # a bounded sample: the first queries of sequence 0's chunk, about 10 s
            n_s = int(qs[1] - qs[0])
            t0 = time.perf_counter()
            done = 0
            while done < n_s and time.perf_counter() - t0 < args.cpu_seconds * 0.7:
                sub = np.array([0, 1], dtype=np.int32)  # one query at position L_sub - 1
                L_sub = np.array([int(w.context_lens[s0]) - n_s + done + 1], dtype=np.int32)
                A.paged_prefill(q_bits[done:done + 1], w.act, pool, w.block_tables[:1], L_sub,
                                sub, w.sm_scale, ks, vs)
                done += 1
            dt = time.perf_counter() - t0
        L0 = int(w.context_lens[s0])
        keys = sum(L0 - n_s + i + 1 for i in range(done))
        f = 4 * w.head_dim * w.num_q_heads * keys
        res["cpu_baseline"] = {"value": round(f / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                               "kind": "oracle", "seconds": round(dt, 2),
                               "sample": f"{done} queries of sequence 0's chunk (all heads), "
                                         f"exact fp64, flops counted as for the GPU"}
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c4", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's split (0 = one pass per sequence)")
    ap.add_argument("--copies", type=int, default=3, help="pool copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle work per timed run (it runs twice: all threads, then one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--kv", default=None,
                    choices=["f16", "bf16", "fp8", "bf8", "fp8t", "bf8t", "fp4"],
                    help="override the workload's KV-cache format (same shapes and inputs)")
    ap.add_argument("--separate-write", action="store_true",
                    help="run the step as pa_cache_write + pa_decode even where one "
                         "pa_append_decode launch can do both")
    ap.add_argument("--fp4-calibration", default="block", choices=["block", "sequence"],
                    help="FP4 pools: outlier sets per block (first write) or per sequence "
                         "(first 512-token prefill chunk)")
    ap.add_argument("--blocks", type=int, default=0, metavar="N",
                    help="time pa_copy_blocks instead: N copies inside the workload's pool "
                         "(copy on write), N blocks out to a pinned host pool and back "
                         "(swap), beside plain DMA copies of the same bytes")
    ap.add_argument("--prefill", type=int, default=0, metavar="CHUNK",
                    help="time pa_prefill instead: the last CHUNK positions of every sequence "
                         "as queries (chunked prefill), reported in TFLOP/s")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path needs no collective and this build "
              "runs on a single MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_quantized_kv_reshape_amd import harness as H
    from workload import DESCRIPTIONS, config

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.prefill > 0:
        prefill_main(args, config, DESCRIPTIONS)
        return
    if args.blocks > 0:
        blocks_main(args, config, DESCRIPTIONS)
        return

    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    w = workload_of(args, config)
    ps = w.partition_size if args.partition_size is None else args.partition_size
    w.partition_size = ps
    run = H.DeviceRun(w, device="cuda", partition_size=ps, pool_copies=args.copies,
                      fp4_calibration=args.fp4_calibration)
    run.prepare()
    torch.cuda.synchronize()
    if run.device_error():
        raise SystemExit(f"device error after setup: {run.device_error()}")
    counts = H.outlier_counts(run) if w.kv == "fp4" else None
    dec = H.decode_bytes(w, counts)
    step_tokens = len(w.step_call.rows)
    wr = H.write_bytes(w, step_tokens)
    step_bytes = dec["total"] + wr
    print(f"[bench] {w.num_seqs} seqs, {dec['tokens']} tokens, ps={ps}, decode bytes "
          f"{dec['total']}, write bytes {wr}", file=sys.stderr, flush=True)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)

    # The step: one pa_append_decode launch (+ merge) where the pool format and the step's
    # write allow it (one new token per sequence, at its last position), else
    # pa_cache_write + pa_decode (+ merge).
    fused = run.can_append and not args.separate_write
    step = run.step_fused if fused else run.step
    # every libpa call goes on torch's current stream; the events are recorded on it too
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        step(run.pools[i % args.copies])
    torch.cuda.synchronize()

    K = args.steps
    timer = HipTimer()

    def pool_of(i):
        return run.pools[(args.warmup + i) % args.copies]

    # (1) the timed region: K whole steps back to back, one event pair around all of them
    # (a marker between steps would sit between the kernels and add its own latency)
    bounds = [timer.event(), timer.event()]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.record(bounds[0], stream)
    for i in range(K):
        step(pool_of(i))
    timer.record(bounds[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step_ev = timer.ms(bounds[0], bounds[1]) * 1e-3 / K
    err = run.device_error()
    out = run.out.cpu().numpy()
    if err or not np.isfinite(out).all():
        raise SystemExit(f"bench run failed: device error {err}, finite {np.isfinite(out).all()}")

    # (2) per-kernel attribution: the same K steps with an event around every kernel (each
    # bracket also holds the runtime's dispatch latency, a few microseconds)
    # (fused: no write kernel, the first bracket is empty)
    ev = [[timer.event() for _ in range(4)] for _ in range(K)]
    for i in range(K):
        e = ev[i]
        timer.record(e[0], stream)
        if not fused:
            run.step_write(pool_of(i))
        timer.record(e[1], stream)
        if fused:
            run.append_decode(pool_of(i), merge=False)
        else:
            run.decode(pool_of(i), merge=False)
        timer.record(e[2], stream)
        run.merge()
        timer.record(e[3], stream)
    # (3) the dominant kernel's launch duration: K launches back to back (same pools, same
    # stream) between one pair of events, so no marker sits between them (fused: each
    # launch writes the same rows again, then decodes)
    burst = [timer.event(), timer.event()]
    timer.record(burst[0], stream)
    for i in range(K):
        if fused:
            run.append_decode(pool_of(i), merge=False)
        else:
            run.decode(pool_of(i), merge=False)
    timer.record(burst[1], stream)
    torch.cuda.synchronize()
    # per-step spread, from the attribution pass (its markers add their own latency, so
    # these run a few microseconds above the timed region's mean)
    step_ms = np.array([timer.ms(e[0], e[3]) for e in ev])
    dec_ms = np.array([timer.ms(e[1], e[2]) for e in ev])
    t_write = float(np.mean([timer.ms(e[0], e[1]) for e in ev])) * 1e-3
    t_dec_br = float(np.mean([timer.ms(e[1], e[2]) for e in ev])) * 1e-3
    t_merge = float(np.mean([timer.ms(e[2], e[3]) for e in ev])) * 1e-3
    t_dec = timer.ms(burst[0], burst[1]) * 1e-3 / K
    # (4) the gather-only ceiling: the decode's launch and tile reads with no arithmetic,
    # K launches back to back like (3)
    probe = [timer.event(), timer.event()]
    timer.record(probe[0], stream)
    for i in range(K):
        run.gather_probe(pool_of(i))
    timer.record(probe[1], stream)
    torch.cuda.synchronize()
    t_probe = timer.ms(probe[0], probe[1]) * 1e-3 / K
    timer.close()
    if run.device_error():
        raise SystemExit(f"device error during timing: {run.device_error()}")

    t_step = wall / K
    kernel_bytes = step_bytes if fused else dec["total"]  # the fused kernel also writes
    dec_gbs = kernel_bytes / t_dec / 1e9
    value = step_bytes / t_step / 1e9
    traffic = counter_traffic(decode_kernel_name(w.kv, fused), profile_label(args), ps)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}"
                               + (f" (KV cache as {w.kv})" if args.kv else ""),
                   "kv_cache_dtype": w.kv, "num_seqs": w.num_seqs,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": 16, "kv_tokens": dec["tokens"],
                   "partition_size": ps, "step_write_tokens": step_tokens,
                   "step": ((f"pa_append_decode_n ({run.step_rows_per_seq} rows per sequence; "
                             "write + decode, one launch)" if run.step_rows_per_seq > 1
                             else "pa_append_decode (write + decode, one launch)") if fused
                            else "pa_cache_write + pa_decode") + (" + pa_merge" if ps else ""),
                   "pool_copies": args.copies}
                  | ({"fp4_calibration": args.fp4_calibration} if w.kv == "fp4" else {}),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(dec["tokens"] / t_step, 1),
        "decode_tokens_per_s": round(w.num_seqs / t_step, 1),
        "step_bytes": step_bytes,
        "kernel_ms": {"decode": round(t_dec * 1e3, 4),
                      "bracketed": {"cache_write": round(t_write * 1e3, 4) if not fused else 0.0,
                                    "decode": round(t_dec_br * 1e3, 4),
                                    "merge": round(t_merge * 1e3, 4)},
                      "step_events": round(t_step_ev * 1e3, 4),
                      "bracketed_step_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4)
                                                     for q in (10, 50, 90)],
                      "bracketed_decode_p10_p50_p90": [round(float(np.percentile(dec_ms, q)), 4)
                                                       for q in (10, 50, 90)]},
        "roofline": {"kernel": decode_kernel_name(w.kv, fused), "bound": "hbm",
                     "achieved": round(dec_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": kernel_bytes,
                     "traffic": traffic},
        "ceiling": {"kernel": f"pa_gather_probe ({decode_kernel_name(w.kv)} with its "
                              "arithmetic compiled out)", "ms": round(t_probe * 1e3, 4),
                    "gbs": round(kernel_bytes / t_probe / 1e9, 2),
                    "pct_hbm_peak": round(100.0 * kernel_bytes / t_probe / 1e9 / HBM_PEAK_GBS, 2),
                    "decode_frac_of_ceiling": round(t_probe / t_dec, 4),
                    "what": "the decode's launch reading every attended K/V run through the "
                            "block tables with its streaming 16-byte loads, no arithmetic; "
                            "gbs counts the decode's algorithmic bytes"},
        "kernel_source_sha256": kernel_source_hash(),
    }
    print("[bench] checking the timed output against the oracle", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"], outs = cpu_baseline(w, args.cpu_seconds,
                                                 dec["total"] / max(dec["tokens"], 1))
    else:  # no timing: the parity check still runs, on one sequence
        outs = oracle_outputs(w, [w.num_seqs - 1])
    res["parity"] = parity_check(out, outs)
    print(json.dumps(res), flush=True)
    if not res["parity"]["ok"]:
        print(f"bench: the timed output differs from the oracle: {res['parity']}",
              file=sys.stderr, flush=True)
        sys.exit(3)


if __name__ == "__main__":
    main()
