"""GPU parity: libpa's HIP path against the oracle on the same seeded inputs.

Cache writes (codes, scales, outlier records and values, untouched sentinel bytes) must be
bit-exact; decode outputs within max-abs 2e-3 and relative L2 1e-2 of exact attention on
the identical dequantized cache. Small cases check every output; the full-size workloads
run in the launch configuration the bench times and are checked on sampled sequences."""
import sys

import numpy as np
import pytest

from oracle_side import (assert_close, assert_pool_equal, oracle_decode, replay, seq_blocks)
from workload import config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Reduced shapes: several blocks per sequence, ragged tails, every format.
SMALL = {
    "c1": {},
    "c2": dict(num_seqs=4, lens_range=(200, 900)),
    "c3": dict(num_seqs=4, lens_range=(200, 900)),
    "c4": dict(num_seqs=4, lens=[2000, 2048, 1999, 33]),
    "c5": dict(num_seqs=3, lens_range=(1500, 4000)),
}

_cache = {}


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def _setup(cfg):
    """Workload, prepared device run, and the oracle's replay (cached per config)."""
    if cfg not in _cache:
        from paged_quantized_kv_reshape_amd.harness import DeviceRun
        w = config(cfg, **SMALL[cfg])
        _say(f"[setup] {cfg}: S={w.num_seqs} lens={w.context_lens.tolist()} kv={w.kv}")
        run = DeviceRun(w, partition_size=0)
        run.prepare()
        torch.cuda.synchronize()
        pool, ks, vs, near = replay(w)
        _cache[cfg] = (w, run, pool, ks, vs, near)
    return _cache[cfg]


@pytest.mark.parametrize("cfg", list(SMALL))
def test_cache_write_bit_exact(cfg):
    w, run, pool, ks, vs, near = _setup(cfg)
    _say(f"[write] {cfg}: near-ties excluded: {len(near)}")
    if ks is not None:
        assert np.array_equal(run.k_scale.cpu().numpy().view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(run.v_scale.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    assert_pool_equal(run.pool.numpy(), pool, near=near)
    assert len(near) == 0
    assert run.device_error() == 0


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("ps", [0, 64, 512])
@pytest.mark.parametrize("cfg", list(SMALL))
def test_decode_matches_oracle(cfg, ps, waves):
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w, run, pool, ks, vs, _ = _setup(cfg)
    _say(f"[decode] {cfg} ps={ps} waves={waves}")
    r = DeviceRun.__new__(DeviceRun)
    r.__dict__.update(run.__dict__)
    if ps:
        from paged_quantized_kv_reshape_amd import max_partitions
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
    got = r.out.cpu().numpy()
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    want = np.stack([ref[s][0] for s in range(w.num_seqs)])
    assert_close(got, want, f"{cfg} ps={ps} W={waves} out")
    if ps:
        lse = r.lse.cpu().numpy()
        want_lse = np.stack([ref[s][1] for s in range(w.num_seqs)])
        assert np.abs(lse - want_lse).max() < 1e-3
        parts = oracle_decode(w, pool, ks, vs, range(w.num_seqs), partition_size=ps)
        po, pl = r.part_out.cpu().numpy(), r.part_lse.cpu().numpy()
        for s in range(w.num_seqs):
            o, l = parts[s]
            n = o.shape[1]
            assert_close(po[s, :, :n], o, f"{cfg} ps={ps} partials of seq {s}")
            assert np.abs(pl[s, :, :n] - l).max() < 1e-3
    assert r.device_error() == 0


@pytest.mark.parametrize("cfg", ["c3", "c5"])
def test_decode_is_deterministic_and_relabelling_invariant(cfg):
    """Two runs give identical bits; moving every physical block to a new id (pool bytes
    and block tables together) gives identical bits too."""
    w, run, pool, ks, vs, _ = _setup(cfg)
    run.decode()
    a = run.out.clone()
    run.decode()
    assert torch.equal(a, run.out)
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(w.num_blocks, generator=g)  # old block i -> new id perm[i]
    inv = torch.argsort(perm)
    saved = {n: t.clone() for n, t in run.pool.bytes.items()}
    for n, t in run.pool.bytes.items():
        t.copy_(saved[n].view(w.num_blocks, -1)[inv.to(t.device)].reshape(-1))
    bt = run.block_tables.clone()
    live = run.block_tables >= 0
    run.block_tables[live] = perm.to(bt.device)[bt[live].long()].int()
    run.decode()
    b = run.out.clone()
    run.block_tables.copy_(bt)
    for n, t in run.pool.bytes.items():
        t.copy_(saved[n])
    assert torch.equal(a, b)


def test_device_side_checks_flag_and_skip():
    from paged_quantized_kv_reshape_amd import describe_device_error
    w, run, pool, ks, vs, _ = _setup("c4")
    # a block id outside the pool: flagged, output stays finite
    bt = run.block_tables.clone()
    run.block_tables[0, 3] = w.num_blocks + 5
    run.dev_err.zero_()
    run.decode()
    e = run.device_error()
    run.block_tables.copy_(bt)
    assert e & 1, describe_device_error(e)
    assert torch.isfinite(run.out).all()
    # a context length of 0 and one past the table: flagged, zero output for that sequence
    cl = run.context_lens.clone()
    run.context_lens[1] = 0
    run.context_lens[2] = w.max_blocks_per_seq * 16 + 1
    run.dev_err.zero_()
    run.decode()
    e = run.device_error()
    run.context_lens.copy_(cl)
    assert e & 4, describe_device_error(e)
    assert torch.count_nonzero(run.out[1]) == 0 and torch.count_nonzero(run.out[2]) == 0
    # a slot outside the pool: flagged, nothing written
    before = {n: t.clone() for n, t in run.pool.bytes.items()}
    from paged_quantized_kv_reshape_amd import pa_cache_write
    bad = torch.tensor([w.num_blocks * 16 + 3], dtype=torch.int64, device="cuda")
    run.dev_err.zero_()
    pa_cache_write(run.pool, run.step_k[:1], run.step_v[:1], bad, run.dev_err)
    e = run.device_error()
    assert e & 2, describe_device_error(e)
    for n, t in run.pool.bytes.items():
        assert torch.equal(t, before[n])


def test_fp4_reset_blocks_and_uncalibrated_read():
    from paged_quantized_kv_reshape_amd import pa_reset_blocks
    w, run, pool, ks, vs, _ = _setup("c5")
    saved = {n: t.clone() for n, t in run.pool.bytes.items()}
    n0 = -(-int(w.context_lens[0]) // 16)
    ids = run.block_tables[0, :n0].contiguous()
    pa_reset_blocks(run.pool, ids)
    rec = run.pool.fp4_records("k")
    assert bool((rec[ids.long()] == 0xFF).all())
    run.dev_err.zero_()
    run.decode()
    assert run.device_error() & 8
    # rewriting sequence 0 recalibrates its blocks to the same records
    from paged_quantized_kv_reshape_amd import pa_cache_write
    for call in list(w.setup_calls) + [w.step_call]:
        sel = np.isin(call.slots // 16, ids.cpu().numpy())
        if sel.any():
            idx = torch.from_numpy(call.rows[sel]).cuda()
            pa_cache_write(run.pool, run.k_rows.index_select(0, idx),
                           run.v_rows.index_select(0, idx),
                           torch.from_numpy(call.slots[sel]).cuda(), run.dev_err)
    torch.cuda.synchronize()
    for n, t in run.pool.bytes.items():
        assert torch.equal(t, saved[n]), n


def test_edge_lengths_and_empty_batch():
    """Contexts of 1, 15, 16, 17 and 33 tokens (single token, ragged tails, exact block
    ends) in one batch, and a zero-sequence call."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", num_seqs=5, lens=[1, 15, 16, 17, 33])
    run = DeviceRun(w, partition_size=16)
    run.prepare()
    run.decode()
    torch.cuda.synchronize()
    pool, ks, vs, _ = replay(w)
    ref = oracle_decode(w, pool, ks, vs, range(5))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(5)]), "edge lengths")
    from paged_quantized_kv_reshape_amd import pa_decode
    pa_decode(run.q[:0], run.pool, run.block_tables[:0], run.context_lens[:0], w.sm_scale,
              out=run.out[:0])
    assert run.device_error() == 0


@pytest.mark.parametrize("ps", [0, 128])
@pytest.mark.parametrize("hq", [1, 2, 16])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4"])
def test_gqa_group_sizes(kv, hq, ps):
    """Query-head groups of 1, 2 and 16 per kv head (the FP4 kernel keeps 8 or 16 head
    columns in LDS depending on the group), single pass and split, against the oracle."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base = "c5" if kv == "fp4" else "c4"
    over = dict(num_seqs=3, lens=[300, 77, 16], num_q_heads=hq)
    if kv == "bf16":
        over.update(kv="bf16", planted=False)
    w = config(base, **over)
    _say(f"[gqa] {kv} Hq={hq} ps={ps}")
    run = DeviceRun(w, partition_size=ps)
    run.prepare()
    run.decode()
    torch.cuda.synchronize()
    assert run.device_error() == 0
    pool, ks, vs, near = replay(w)
    assert_pool_equal(run.pool.numpy(), pool, near=near)
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"{kv} Hq={hq} ps={ps}")


@pytest.mark.parametrize("ps", [0, 128])
@pytest.mark.parametrize("hq,hkv", [(6, 2), (5, 1), (24, 2)])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8t", "fp4"])
def test_gqa_groups_not_powers_of_two(kv, hq, hkv, ps):
    """Query-head groups of 3, 5 and 12: the MFMA column tile holds G real heads and
    16 - G padding columns (the FP4 kernel's 8-column LDS layout for G <= 8, 16 above)."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base = "c5" if kv == "fp4" else "c4"
    over = dict(num_seqs=3, lens=[300, 77, 16], num_q_heads=hq, num_kv_heads=hkv)
    if kv == "bf16":
        over.update(kv="bf16", planted=False)
    elif kv == "fp8t":
        over.update(kv="fp8t")
    w = config(base, **over)
    _say(f"[gqa odd] {kv} Hq={hq} Hkv={hkv} ps={ps}")
    run = DeviceRun(w, partition_size=ps)
    run.prepare()
    run.decode()
    torch.cuda.synchronize()
    assert run.device_error() == 0
    pool, ks, vs, near = replay(w)
    assert_pool_equal(run.pool.numpy(), pool, near=near)
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"{kv} Hq={hq} Hkv={hkv} ps={ps}")


@pytest.mark.parametrize("ps", [0, 128])
@pytest.mark.parametrize("kv,act,d", [("fp8", "f16", 128), ("fp4", "f16", 128),
                                      ("fp8", "bf16", 64), ("fp8", "f16", 64),
                                      ("f16", "f16", 128), ("bf16", "bf16", 64),
                                      ("fp4", "bf16", 64), ("fp4", "f16", 64)])
def test_activation_dtypes_and_head_dims(kv, act, d, ps):
    """fp16 activations with the quantized pools (their fp16 MFMA variants), head_dim 64
    with FP8, FP4 and 16-bit pools, two kv heads: pools bit-exact, outputs within
    tolerance."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base = "c5" if kv == "fp4" else "c4"
    w = config(base, num_seqs=3, lens=[300, 77, 16], num_q_heads=8, num_kv_heads=2,
               head_dim=d, kv=kv, act=act, planted=kv in ("fp8", "fp4"))
    _say(f"[dtypes] kv={kv} act={act} D={d} ps={ps}")
    run = DeviceRun(w, partition_size=ps)
    run.prepare()
    run.decode()
    torch.cuda.synchronize()
    assert run.device_error() == 0
    pool, ks, vs, near = replay(w)
    assert_pool_equal(run.pool.numpy(), pool, near=near)
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"kv={kv} act={act} D={d} ps={ps}")


# ---------------------------------------------------------------------------------
# Full-size workloads, in the bench's launch configuration, sampled against the oracle.
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c5"])
def test_full_size_sampled(cfg):
    """Each full-size workload, sampled. Pool 0 gets the setup and step writes, then the
    separate decode (pa_decode + pa_merge). Where the bench runs the step as one
    pa_append_decode[_n] launch (the new tokens of every sequence at its last positions:
    one in c2, c4, c5, eight in c3), that launch is checked too, in the bench's own configuration (the workload's partition
    size, the library's wave count, then pa_merge): on pool 1, which holds the setup writes
    only, so the launch itself writes (and for FP4 calibrates) the step's rows; and again
    on pool 0, whose rows are already written, as every timed bench step after the first
    finds them."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config(cfg)
    _say(f"[full] {cfg}: S={w.num_seqs} tokens={w.tokens} blocks={w.num_blocks} ps={w.partition_size}")
    run = DeviceRun(w, pool_copies=2)
    fused = run.can_append
    run.setup_writes(run.pools[0])
    run.step_write(run.pools[0])
    run.decode(run.pools[0])
    torch.cuda.synchronize()
    assert run.device_error() == 0
    out = run.out.cpu().numpy()
    assert np.isfinite(out).all()
    seqs = [0, w.num_seqs - 1] if cfg == "c5" else [0, w.num_seqs // 2, w.num_seqs - 1]
    blocks = seq_blocks(w, seqs)
    pool, ks, vs, near = replay(w, only_blocks=blocks)
    _say(f"[full] {cfg}: sampled seqs {seqs}, {len(blocks)} blocks, near-ties {len(near)}")
    if ks is not None:
        assert np.array_equal(run.k_scale.cpu().numpy().view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(run.v_scale.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    assert_pool_equal(run.pools[0].numpy(), pool, blocks=blocks, near=near)
    ref = oracle_decode(w, pool, ks, vs, seqs)
    for s in seqs:
        assert_close(out[s], ref[s][0], f"{cfg} seq {s}")
    if w.kv == "fp4":
        # every full 16-token block calibrated by a prefill chunk flags exactly the
        # planted x20 channel (known a priori from the generator)
        rec = run.pools[0].fp4_records("k").cpu().numpy()
        s = seqs[0]
        full = w.block_tables[s, :(int(w.context_lens[s]) - 1) // 16]
        pk = int(w.planted_k[0]) % w.head_dim
        assert np.all(rec[full, 0, 0] == 1) and np.all(rec[full, 0, 1] == pk)
    if not fused:
        return
    for label, pool_i, setup in (("fresh rows", 1, True), ("rows already written", 0, False)):
        if setup:
            run.setup_writes(run.pools[pool_i])
        run.out.fill_(float("nan"))
        run.append_decode(run.pools[pool_i])  # + pa_merge when split, as the bench step
        torch.cuda.synchronize()
        _say(f"[full fused] {cfg}: {label}")
        assert run.device_error() == 0
        got = run.out.cpu().numpy()
        assert_pool_equal(run.pools[pool_i].numpy(), pool, blocks=blocks, near=near)
        for s in seqs:
            assert_close(got[s], ref[s][0], f"{cfg} fused ({label}) seq {s}")
        # the fused launch reads what the separate write stored, with the same arithmetic
        assert np.array_equal(got.view(np.uint32), out.view(np.uint32)), label


def test_all_blocks_bad_gives_zero_output_and_a_flag():
    """Sequences whose every block id is out of range, at 8 waves and ps > 0 (a merge
    follows) and at ps = 0: flagged, and the output of those sequences is zero (every wave
    of their workgroups has nothing to fold in), not NaN; the other sequences are unharmed.
    The same for a context length past the block table in split mode."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", num_seqs=4, lens=[16, 300, 1000, 77])
    for ps in (0, 64):
        run = DeviceRun(w, partition_size=ps, waves=8)
        run.prepare()
        run.decode()
        torch.cuda.synchronize()
        good = run.out.cpu().numpy().copy()
        run.block_tables[0, 0] = w.num_blocks + 7       # one-block sequence, its only block
        run.block_tables[1, :] = -5                      # every block of sequence 1
        run.dev_err.zero_()
        run.decode()
        torch.cuda.synchronize()
        assert run.device_error() & 1
        got = run.out.cpu().numpy()
        assert np.isfinite(got).all(), f"ps={ps}"
        assert np.all(got[:2] == 0.0), f"ps={ps}"
        assert np.array_equal(got[2:], good[2:]), f"ps={ps}"
        if ps:
            lse = run.lse.cpu().numpy()
            assert np.all(np.isneginf(lse[:2])) and np.isfinite(lse[2:]).all()
            # a context past the table (split): flagged, zero output, lse -inf
            run.context_lens[3] = w.max_blocks_per_seq * 16 + 1
            run.dev_err.zero_()
            run.decode()
            torch.cuda.synchronize()
            assert run.device_error() & 4
            assert np.all(run.out[3].cpu().numpy() == 0.0)
            assert np.isneginf(run.lse[3].cpu().numpy()).all()


# Scales of the FP8 sweep: reciprocals that are exact and inexact, a negative scale, a zero
# scale (zero codes); absmax / 448 scales as the head-scale call makes them (quotients
# 448 x / absmax of two 16-bit values land on and beside E4M3 midpoints); scales at both
# ends of the range the fast quotient accepts and just outside it (2^-81, 2^101, 1e-39,
# 2^126), a large scale that drives quotients of small inputs below fp32's normal range;
# and 3 moved by k = +-1..8 fp32 ulps, which puts the quotients of x = 3 m (m an E4M3
# midpoint) within a few ulps on either side of m.
FP8_SWEEP_SCALES = (
    [3.0, 1.0 / 3.0, 0.0123, -0.37, 1.0, 0.0]
    + [float(np.float32(b) / np.float32(448.0)) for b in (108.0, 96.0, 6.5, 0.8125, 21.25)]
    + [2.0 ** -80, 2.0 ** -81, 2.0 ** 100, 2.0 ** 101, 1e-39, 2.0 ** 126, 2.0 ** 17, -(2.0 ** 40)]
    + [float(np.float32(3.0) + np.float32(k) * np.spacing(np.float32(3.0)))
       for k in range(-8, 9) if k != 0])


@pytest.mark.parametrize("act,d", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
def test_fp8_write_every_input(act, d):
    """Every non-NaN 16-bit activation pattern through the FP8 write, under scales that put
    exact quotients on E4M3 rounding midpoints (x = 3 m for a midpoint m and s = 3), must
    give the oracle's codes bit for bit."""
    from oracle import cache as C
    from oracle.formats import act_decode, e4m3_magnitudes, f32_quotient
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write
    pats = np.arange(65536, dtype=np.uint32)
    inf_bits = 0x7F80 if act == "bf16" else 0x7C00
    pats = np.where((pats & 0x7FFF) > inf_bits, 0, pats).astype(np.uint16)
    hkv, T = len(FP8_SWEEP_SCALES), 65536 // d
    rng = np.random.default_rng(7)
    k_rows = np.stack([rng.permutation(pats) for _ in range(hkv)], 1).reshape(T, d, hkv)
    k_rows = np.ascontiguousarray(k_rows.transpose(0, 2, 1))
    v_rows = np.ascontiguousarray(k_rows[::-1])
    nb = T // 16 + 3
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    scales = np.asarray(FP8_SWEEP_SCALES, dtype=np.float32)

    # the sweep holds quotients that sit exactly on an E4M3 midpoint
    mags = e4m3_magnitudes()
    mids = (mags[1:] + mags[:-1]) / 2
    x = act_decode(k_rows, act)
    q = np.abs(f32_quotient(x[:, 0, :], np.float64(scales[0])))
    assert np.isin(q, mids).sum() > 0
    # ... and quotients a few ulps beside one (up to 8 ulps on each side)
    q = np.abs(f32_quotient(x[:, -16:, :], scales[None, -16:, None].astype(np.float64)))
    j = np.clip(np.searchsorted(mids, q), 1, len(mids) - 1)
    gap = np.minimum(np.abs(q - mids[j]), np.abs(q - mids[j - 1]))
    ulps = gap / np.spacing(q.astype(np.float32)).astype(np.float64)
    assert ((ulps > 0) & (ulps <= 8)).sum() > 100

    opool = C.Pool.filled("fp8", nb, hkv, d)
    C.cache_write(opool, k_rows, v_rows, act, slots, k_scale=scales, v_scale=scales[::-1].copy())
    ks = torch.from_numpy(scales).cuda()
    vs = torch.from_numpy(scales[::-1].copy()).cuda()
    pool = KVPool("fp8", nb, hkv, d, fill=0xA5, k_scale=ks, v_scale=vs)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    kt = torch.from_numpy(k_rows.view(np.int16)).cuda().view(tdt)
    vt = torch.from_numpy(v_rows.view(np.int16)).cuda().view(tdt)
    _say(f"[fp8 sweep] act={act} d={d} T={T} hkv={hkv}")
    pa_cache_write(pool, kt, vt, torch.from_numpy(slots).cuda(), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    tok = np.full(nb * 16, -1)
    tok[slots] = np.arange(T)
    got = pool.numpy()
    for name, rows, sc in (("k", k_rows, scales), ("v", v_rows, scales[::-1])):
        g = got[name].reshape(nb, hkv, 16, d)
        o = opool.arrays[name]
        bad = np.argwhere(g != o)
        msg = [f"{name}: x=0x{int(rows[tok[b * 16 + r], h, c]):04x} s={sc[h]!r} "
               f"gpu=0x{int(g[b, h, r, c]):02x} oracle=0x{int(o[b, h, r, c]):02x}"
               for b, h, r, c in bad[:8]]
        assert len(bad) == 0, f"{len(bad)} codes differ:\n" + "\n".join(msg)
    assert_pool_equal(got, opool)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_fp4_write_scattered_slots(act):
    """FP4 writes whose rows arrive in scrambled slot order, in calls that cover parts of
    4-token groups (V codes of four tokens share each word), mixed with whole aligned
    groups, over several calls: the pool must match the oracle byte for byte."""
    from oracle import cache as C
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write
    rng = np.random.default_rng(11)
    d, hkv, nb = 128, 2, 24
    x = rng.standard_normal((nb * 16, hkv, d)).astype(np.float32)
    x[:, :, 5] *= 20.0  # one planted outlier channel
    bits = (x.astype(np.float16).view(np.uint16) if act == "f16" else
            ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16))
    order = rng.permutation(nb * 16)
    # call 1: whole aligned fours of blocks 0..7, rows shuffled within the call
    quads = [np.arange(4 * q, 4 * q + 4) for q in range(32)]
    call1 = np.concatenate([quads[q] for q in rng.permutation(32)])
    rest = np.setdiff1d(order, call1, assume_unique=False)
    rest = rest[rng.permutation(len(rest))]
    calls = [call1] + list(np.array_split(rest, 5))  # scattered slots, partial fours
    opool = C.Pool.filled("fp4", nb, hkv, d)
    pool = KVPool("fp4", nb, hkv, d, fill=0xA5)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tdt = torch.bfloat16 if act == "bf16" else torch.float16
    for ci, slots in enumerate(calls):
        slots = np.asarray(slots, dtype=np.int64)
        rows = np.ascontiguousarray(bits[slots])
        C.cache_write(opool, rows, rows[::-1].copy(), act, slots)
        rt = torch.from_numpy(rows.view(np.int16)).cuda().view(tdt)
        rv = torch.from_numpy(rows[::-1].copy().view(np.int16)).cuda().view(tdt)
        _say(f"[fp4 scattered] act={act} call {ci}: {len(slots)} rows")
        pa_cache_write(pool, rt, rv, torch.from_numpy(slots).cuda(), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert_pool_equal(pool.numpy(), opool)
