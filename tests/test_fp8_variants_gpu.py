"""GPU parity of the FP8 pool variants: E5M2 codes with per-head scales ("bf8"), and E4M3 /
E5M2 codes with a dynamic per-token scale stored beside each token's codes ("fp8t",
"bf8t").

Writes bit-exact against the oracle (codes, per-token scales, untouched sentinel bytes),
including every 16-bit activation pattern; decode (fused and split-KV) and multi-token
attention within max-abs 2e-3 and relative L2 1e-2 of exact attention on the identical
dequantized cache."""

import numpy as np
import pytest

from oracle import attention as A
from oracle_side import (assert_close, assert_pool_equal, oracle_decode, replay, seq_blocks)
from workload import config, prefill_queries

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import FP8_SWEEP_SCALES, _say  # noqa: E402

KINDS = ["bf8", "fp8t", "bf8t"]
# Reduced shapes on the 8B-shaped and 70B-share layouts: several blocks per sequence,
# ragged tails, a sequence shorter than one block.
SHAPES = {
    "c3": dict(num_seqs=4, lens_range=(200, 900)),
    "c4": dict(num_seqs=4, lens=[2000, 2048, 1999, 13]),
}

_cache = {}


def _setup(kv, cfg):
    key = (kv, cfg)
    if key not in _cache:
        from paged_quantized_kv_reshape_amd.harness import DeviceRun
        w = config(cfg, kv=kv, **SHAPES[cfg])
        _say(f"[setup] {kv}/{cfg}: S={w.num_seqs} lens={w.context_lens.tolist()}")
        run = DeviceRun(w, partition_size=0)
        run.prepare()
        torch.cuda.synchronize()
        pool, ks, vs, near = replay(w)
        _cache[key] = (w, run, pool, ks, vs)
    return _cache[key]


@pytest.mark.parametrize("cfg", list(SHAPES))
@pytest.mark.parametrize("kv", KINDS)
def test_write_bit_exact(kv, cfg):
    w, run, pool, ks, vs = _setup(kv, cfg)
    if ks is not None:
        assert np.array_equal(run.k_scale.cpu().numpy().view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(run.v_scale.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    else:
        assert run.k_scale is None
    assert_pool_equal(run.pool.numpy(), pool)
    assert run.device_error() == 0


@pytest.mark.parametrize("waves", [1, 4])
@pytest.mark.parametrize("ps", [0, 512])
@pytest.mark.parametrize("cfg", list(SHAPES))
@pytest.mark.parametrize("kv", KINDS)
def test_decode_matches_oracle(kv, cfg, ps, waves):
    from paged_quantized_kv_reshape_amd import max_partitions
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w, run, pool, ks, vs = _setup(kv, cfg)
    _say(f"[decode] {kv}/{cfg} ps={ps} waves={waves}")
    r = DeviceRun.__new__(DeviceRun)
    r.__dict__.update(run.__dict__)
    if ps:
        S, Hq, D = w.q.shape
        P = max_partitions(w.max_blocks_per_seq, ps)
        r.part_out = torch.empty((S, Hq, P, D), dtype=torch.float32, device="cuda")
        r.part_lse = torch.empty((S, Hq, P), dtype=torch.float32, device="cuda")
    r.ps = ps
    r.waves = waves
    r.out = torch.full_like(run.out, float("nan"))
    r.lse = torch.full_like(run.lse, float("nan"))
    r.decode()
    torch.cuda.synchronize()
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(r.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"{kv}/{cfg} ps={ps} W={waves}")
    if ps:
        want_lse = np.stack([ref[s][1] for s in range(w.num_seqs)])
        assert np.abs(r.lse.cpu().numpy() - want_lse).max() < 1e-3
    assert r.device_error() == 0


@pytest.mark.parametrize("n", [1, 16, 37])
@pytest.mark.parametrize("kv", KINDS)
def test_prefill_matches_oracle(kv, n):
    from paged_quantized_kv_reshape_amd import pa_prefill
    w, run, pool, ks, vs = _setup(kv, "c4")
    q_bits, qs = prefill_queries(w, n)
    _say(f"[prefill] {kv} n={n}")
    tdt = torch.bfloat16 if w.act == "bf16" else torch.float16
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    out = torch.full((q.shape[0], w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    run.dev_err.zero_()
    pa_prefill(q, torch.from_numpy(qs).cuda(), int(np.diff(qs).max()), run.pool,
               run.block_tables, run.context_lens, w.sm_scale, out, run.dev_err)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    ref = A.paged_prefill(q_bits, w.act, pool, w.block_tables, w.context_lens, qs, w.sm_scale,
                          ks, vs)
    assert_close(out.cpu().numpy(), np.concatenate([ref[s] for s in range(w.num_seqs)]),
                 f"{kv} prefill n={n}")


@pytest.mark.parametrize("kv,act,d,hq", [("bf8", "f16", 64, 8), ("fp8t", "f16", 128, 16),
                                         ("bf8t", "bf16", 64, 2), ("fp8t", "bf16", 64, 1)])
def test_dtypes_head_dims_groups(kv, act, d, hq):
    """fp16 and bf16 activations, head_dim 64 and 128, query groups 1..16: write, decode
    (fused and split) and multi-token attention."""
    from paged_quantized_kv_reshape_amd import pa_prefill
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", num_seqs=3, lens=[300, 77, 16], num_q_heads=hq * 2, num_kv_heads=2,
               head_dim=d, kv=kv, act=act)
    _say(f"[variants] kv={kv} act={act} D={d} Hq={hq * 2}")
    pool, ks, vs, _ = replay(w)
    for ps in (0, 128):
        run = DeviceRun(w, partition_size=ps)
        run.prepare()
        run.decode()
        torch.cuda.synchronize()
        assert run.device_error() == 0
        assert_pool_equal(run.pool.numpy(), pool)
        ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
        assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                     f"kv={kv} act={act} D={d} ps={ps}")
    q_bits, qs = prefill_queries(w, 24)
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    out = torch.empty((q.shape[0], w.num_q_heads, d), dtype=torch.float32, device="cuda")
    pa_prefill(q, torch.from_numpy(qs).cuda(), int(np.diff(qs).max()), run.pool,
               run.block_tables, run.context_lens, w.sm_scale, out, run.dev_err)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    ref = A.paged_prefill(q_bits, act, pool, w.block_tables, w.context_lens, qs, w.sm_scale,
                          ks, vs)
    assert_close(out.cpu().numpy(), np.concatenate([ref[s] for s in range(w.num_seqs)]),
                 f"kv={kv} prefill")


@pytest.mark.parametrize("kv", ["fp8t", "bf8t"])
def test_full_size_sampled(kv):
    """The 70B one-GPU share (256 sequences of 8192 tokens, 8 q / 1 kv heads) in a
    per-token pool, in the bench's launch configuration, sampled against the oracle."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", kv=kv)
    _say(f"[full] {kv}: S={w.num_seqs} tokens={w.tokens}")
    run = DeviceRun(w)
    run.prepare()
    run.decode()
    torch.cuda.synchronize()
    assert run.device_error() == 0
    out = run.out.cpu().numpy()
    assert np.isfinite(out).all()
    seqs = [0, w.num_seqs // 2, w.num_seqs - 1]
    blocks = seq_blocks(w, seqs)
    pool, ks, vs, _ = replay(w, only_blocks=blocks)
    assert_pool_equal(run.pool.numpy(), pool, blocks=blocks)
    ref = oracle_decode(w, pool, ks, vs, seqs)
    for s in seqs:
        assert_close(out[s], ref[s][0], f"{kv} seq {s}")


def _sweep_rows(act, d, window):
    """Every non-NaN 16-bit pattern once, as [T, 1, d] rows. Patterns are sorted by
    magnitude and cut into windows of `window` consecutive patterns; each window is shuffled
    into whole rows, so a row's absmax (its per-token scale) sits at the top of a range of
    about log2(window / patterns-per-binade) binades and its other values fall on every
    code of the format, subnormals and flush-to-zero included."""
    pats = np.arange(65536, dtype=np.uint32)
    inf_bits = 0x7F80 if act == "bf16" else 0x7C00
    pats = np.where((pats & 0x7FFF) >= inf_bits, 0, pats).astype(np.uint16)  # no Inf/NaN
    mag = pats & 0x7FFF
    order = np.argsort(mag, kind="stable")
    rng = np.random.default_rng(5)
    s = pats[order].reshape(-1, window)
    s = np.stack([rng.permutation(r) for r in s])
    return s.reshape(-1, 1, d)


@pytest.mark.parametrize("fmt_kind", ["bf8", "fp8t", "bf8t"])
@pytest.mark.parametrize("act,d", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
def test_write_every_input(fmt_kind, act, d):
    """Every finite 16-bit activation pattern through the E5M2 head-scaled write (under the
    sweep scales: exact and inexact reciprocals, zero and negative scales, both ends of the
    fast quotient's range) and through the per-token writes (scales from the rows' own
    absmax): codes and stored scales bit for bit."""
    from oracle import cache as C
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write
    rng = np.random.default_rng(9)
    if fmt_kind == "bf8":
        pats = np.arange(65536, dtype=np.uint32)
        inf_bits = 0x7F80 if act == "bf16" else 0x7C00
        pats = np.where((pats & 0x7FFF) > inf_bits, 0, pats).astype(np.uint16)
        hkv, T = len(FP8_SWEEP_SCALES), 65536 // d
        k_rows = np.stack([rng.permutation(pats) for _ in range(hkv)], 1).reshape(T, d, hkv)
        k_rows = np.ascontiguousarray(k_rows.transpose(0, 2, 1))
        scales = np.asarray(FP8_SWEEP_SCALES, dtype=np.float32)
        ks_np, vs_np = scales, scales[::-1].copy()
    else:
        # f16 has 31 binades of 1024 magnitudes, bf16 255 of 128: windows of about 16
        # binades for E4M3 and 32 for E5M2 (a little more than each format's range)
        e5 = fmt_kind == "bf8t"
        window = {"f16": 65536 if e5 else 32768, "bf16": 8192 if e5 else 4096}[act]
        k_rows = _sweep_rows(act, d, window)
        hkv, T = 1, k_rows.shape[0]
        ks_np = vs_np = None
    v_rows = np.ascontiguousarray(k_rows[::-1])
    nb = T // 16 + 3
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    opool = C.Pool.filled(fmt_kind, nb, hkv, d)
    C.cache_write(opool, k_rows, v_rows, act, slots, k_scale=ks_np, v_scale=vs_np)
    ks = vs = None
    if ks_np is not None:
        ks, vs = torch.from_numpy(ks_np).cuda(), torch.from_numpy(vs_np).cuda()
    pool = KVPool(fmt_kind, nb, hkv, d, fill=0xA5, k_scale=ks, v_scale=vs)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    kt = torch.from_numpy(k_rows.view(np.int16)).cuda().view(tdt)
    vt = torch.from_numpy(v_rows.view(np.int16)).cuda().view(tdt)
    _say(f"[sweep] kv={fmt_kind} act={act} d={d} T={T} hkv={hkv}")
    pa_cache_write(pool, kt, vt, torch.from_numpy(slots).cuda(), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    if fmt_kind != "bf8":
        # the sweep reaches subnormal codes and flushes to zero within a row
        codes = C.fp8t_codes(opool, "k")
        mant_only = ((codes & 0x7F) != 0) & ((codes & (0x78 if fmt_kind == "fp8t" else 0x7C)) == 0)
        assert mant_only.sum() > 100
    assert_pool_equal(pool.numpy(), opool)


@pytest.mark.parametrize("fmt_kind", ["fp8", "bf8", "fp8t", "bf8t"])
@pytest.mark.parametrize("d", [64, 128])
def test_write_slot_patterns(fmt_kind, d):
    """The FP8 write stores four rows that land in an aligned four of slots (4 q .. 4 q + 3
    of one block, in order) together and every other row alone. Runs that start at any row
    and any offset, runs broken by a skipped (-1) or out-of-range slot, a four that ends at
    the call's last row and scattered single rows must all match the oracle bit for bit;
    the out-of-range slots are flagged and write nothing."""
    from oracle import cache as C
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write
    rng = np.random.default_rng(11 + d)
    nb, hkv = 24, 2
    nslots = nb * 16
    blocks = [int(b) for b in rng.permutation(nb)]
    slots = []

    def run(b, off, n):
        slots.extend(blocks[b] * 16 + off + j for j in range(n))

    def at_row(r):  # skipped rows until the next row is r mod 4
        while len(slots) % 4 != r:
            slots.append(-1)

    at_row(1)
    run(0, 0, 16)                            # a whole block: four aligned fours
    run(1, 2, 5)                             # offsets 2 .. 6: the four 4 .. 7 cut short
    at_row(0)
    run(2, 4, 8)                             # two aligned fours
    slots.append(nslots + 5)                 # out of range
    run(3, 0, 3)
    slots.append(-1)                         # a four broken by a skipped row
    at_row(2)
    run(3, 4, 4)                             # an aligned four
    run(4, 1, 4)                             # offsets 1 .. 4: no aligned four
    run(5, 0, 2)
    slots.append(nslots + 40)                # a four broken by an out-of-range slot
    run(5, 3, 1)
    singles = [blocks[b] * 16 + int(o) for b in range(10, 20) for o in rng.permutation(16)[:3]]
    slots.extend(int(x) for x in rng.permutation(singles))
    at_row(3)
    run(6, 8, 4)                             # the last four rows: an aligned four
    T = len(slots)
    assert T % 4 != 0
    slots = np.asarray(slots, dtype=np.int64)
    live = slots[(slots >= 0) & (slots < nslots)]
    assert len(np.unique(live)) == len(live)

    x = (rng.standard_normal((2, T, hkv, d)) * 3.0).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # bf16, nearest even
    k_rows, v_rows = bits[0], bits[1]
    ks_np = vs_np = None
    ks = vs = None
    if fmt_kind in ("fp8", "bf8"):
        ks_np = np.asarray([0.011, 0.023], dtype=np.float32)
        vs_np = np.asarray([0.017, 0.009], dtype=np.float32)
        ks, vs = torch.from_numpy(ks_np).cuda(), torch.from_numpy(vs_np).cuda()
    opool = C.Pool.filled(fmt_kind, nb, hkv, d)
    C.cache_write(opool, k_rows, v_rows, "bf16", np.where(slots < nslots, slots, -1),
                  k_scale=ks_np, v_scale=vs_np)
    pool = KVPool(fmt_kind, nb, hkv, d, fill=0xA5, k_scale=ks, v_scale=vs)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kt = torch.from_numpy(k_rows.view(np.int16)).cuda().view(torch.bfloat16)
    vt = torch.from_numpy(v_rows.view(np.int16)).cuda().view(torch.bfloat16)
    _say(f"[slot patterns] kv={fmt_kind} d={d} T={T}")
    pa_cache_write(pool, kt, vt, torch.from_numpy(slots).cuda(), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 2  # PA_DEVERR_BAD_SLOT
    assert_pool_equal(pool.numpy(), opool)


@pytest.mark.parametrize("fmt_kind", ["fp8", "fp8t"])
@pytest.mark.parametrize("T,first", [(1, 0), (2, 14), (3, 4), (4, 4), (5, 8), (5, 3)])
def test_write_short_calls(fmt_kind, T, first):
    """Calls of a few rows (less than a window of four, one four, one past it) into
    consecutive slots from `first` of one block: bit for bit against the oracle."""
    from oracle import cache as C
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write
    rng = np.random.default_rng(100 * T + first)
    nb, hkv, d = 3, 2, 128
    slots = (16 + first + np.arange(T)).astype(np.int64)  # block 1; may run into block 2
    x = (rng.standard_normal((2, T, hkv, d)) * 2.0).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    ks_np = vs_np = ks = vs = None
    if fmt_kind == "fp8":
        ks_np = np.asarray([0.01, 0.02], dtype=np.float32)
        vs_np = np.asarray([0.03, 0.015], dtype=np.float32)
        ks, vs = torch.from_numpy(ks_np).cuda(), torch.from_numpy(vs_np).cuda()
    opool = C.Pool.filled(fmt_kind, nb, hkv, d)
    C.cache_write(opool, bits[0], bits[1], "bf16", slots, k_scale=ks_np, v_scale=vs_np)
    pool = KVPool(fmt_kind, nb, hkv, d, fill=0xA5, k_scale=ks, v_scale=vs)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kt = torch.from_numpy(bits[0].view(np.int16)).cuda().view(torch.bfloat16)
    vt = torch.from_numpy(bits[1].view(np.int16)).cuda().view(torch.bfloat16)
    _say(f"[short write] kv={fmt_kind} T={T} first={first}")
    pa_cache_write(pool, kt, vt, torch.from_numpy(slots).cuda(), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert_pool_equal(pool.numpy(), opool)
