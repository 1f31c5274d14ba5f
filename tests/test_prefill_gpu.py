"""GPU parity of multi-token paged attention (pa_prefill, chunked prefill and draft
verification over the same pool) against the oracle's causal definition.

Outputs within max-abs 2e-3 and relative L2 1e-2 of exact attention over the identical
dequantized cache, for every pool format, query groups 1..16, head_dim 64 and 128, query
counts from 1 to a whole sequence, ragged per sequence; the last query of a chunk agrees
with pa_decode; invalid query counts are flagged and their rows zeroed."""
import numpy as np
import pytest

from oracle import attention as A
from oracle_side import assert_close, replay
from workload import config, prefill_queries

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import SMALL, _say, _setup  # noqa: E402  (shared prepared workloads)


def _run_prefill(w, run, q_bits, qs):
    from paged_quantized_kv_reshape_amd import pa_prefill
    tdt = torch.bfloat16 if w.act == "bf16" else torch.float16
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    qs_t = torch.from_numpy(qs).cuda()
    out = torch.full((q.shape[0], w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    run.dev_err.zero_()
    nmax = int(np.diff(qs).max()) if len(qs) > 1 else 0
    pa_prefill(q, qs_t, nmax, run.pool, run.block_tables, run.context_lens, w.sm_scale, out,
               run.dev_err)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(w, run, pool, ks, vs, q_bits, qs, what):
    got = _run_prefill(w, run, q_bits, qs)
    assert run.device_error() == 0
    ref = A.paged_prefill(q_bits, w.act, pool, w.block_tables, w.context_lens, qs, w.sm_scale,
                          ks, vs)
    want = np.concatenate([ref[s] for s in range(w.num_seqs)])
    return assert_close(got, want, what), got


@pytest.mark.parametrize("n", [1, 7, 16, 33])
@pytest.mark.parametrize("cfg", list(SMALL))
def test_prefill_matches_oracle(cfg, n):
    w, run, pool, ks, vs, near = _setup(cfg)
    q, qs = prefill_queries(w, n)
    _say(f"[prefill] {cfg} n={n} lens={w.context_lens.tolist()}")
    _check(w, run, pool, ks, vs, q, qs, f"{cfg} n={n}")


@pytest.mark.parametrize("cfg", ["c2", "c4", "c5"])
def test_prefill_ragged_whole_sequence_and_last_query(cfg):
    """Query counts differ per sequence (one of them the whole sequence, so its first
    query sees one key); the last query of every chunk equals pa_decode's output."""
    w, run, pool, ks, vs, near = _setup(cfg)
    L = w.context_lens.astype(np.int64)
    ns = np.array([min(int(L[0]), 3), int(L[1]), 1] + [5] * (w.num_seqs - 3))[:w.num_seqs]
    ns = np.minimum(ns, L)
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((int(qs[-1]), w.num_q_heads, w.head_dim))
         .astype(np.float16).view(np.uint16))
    if w.act == "bf16":
        x = rng.standard_normal((int(qs[-1]), w.num_q_heads, w.head_dim)).astype(np.float32)
        q = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 bits will do
    _say(f"[prefill ragged] {cfg} ns={ns.tolist()}")
    _, got = _check(w, run, pool, ks, vs, q, qs, f"{cfg} ragged")
    # last query of each chunk against pa_decode with that query
    last = q[qs[1:] - 1]
    tdt = torch.bfloat16 if w.act == "bf16" else torch.float16
    from paged_quantized_kv_reshape_amd import pa_decode
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    pa_decode(torch.from_numpy(last.view(np.int16)).cuda().view(tdt), run.pool,
              run.block_tables, run.context_lens, w.sm_scale, 0, out, dev_err=run.dev_err)
    torch.cuda.synchronize()
    assert_close(got[qs[1:] - 1], out.cpu().numpy(), f"{cfg} last query vs decode")


@pytest.mark.parametrize("hq", [1, 2, 16])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4"])
def test_prefill_group_sizes(kv, hq):
    """Query groups of 1, 2 and 16 (16, 8 and 1 queries per wave)."""
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base = "c5" if kv == "fp4" else "c4"
    over = dict(num_seqs=3, lens=[300, 77, 16], num_q_heads=hq)
    if kv == "bf16":
        over.update(kv="bf16", planted=False)
    w = config(base, **over)
    run = DeviceRun(w, partition_size=0)
    run.prepare()
    torch.cuda.synchronize()
    pool, ks, vs, near = replay(w)
    q, qs = prefill_queries(w, 20)
    _say(f"[prefill gqa] {kv} Hq={hq}")
    _check(w, run, pool, ks, vs, q, qs, f"{kv} Hq={hq}")


@pytest.mark.parametrize("kv,act,d", [("fp8", "f16", 128), ("fp4", "f16", 128),
                                      ("fp8", "bf16", 64), ("f16", "f16", 64),
                                      ("fp4", "bf16", 64), ("fp4", "f16", 64)])
def test_prefill_dtypes_and_head_dims(kv, act, d):
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base = "c5" if kv == "fp4" else "c4"
    w = config(base, num_seqs=3, lens=[300, 77, 16], num_q_heads=8, num_kv_heads=2,
               head_dim=d, kv=kv, act=act, planted=kv in ("fp8", "fp4"))
    run = DeviceRun(w, partition_size=0)
    run.prepare()
    torch.cuda.synchronize()
    pool, ks, vs, near = replay(w)
    q, qs = prefill_queries(w, 24)
    _say(f"[prefill dtypes] kv={kv} act={act} D={d}")
    _check(w, run, pool, ks, vs, q, qs, f"kv={kv} act={act} D={d}")


def test_prefill_bad_query_count_is_flagged_and_zeroed():
    w, run, pool, ks, vs, near = _setup("c4")
    L = w.context_lens.astype(np.int64)
    ns = np.array([2, int(L[1]) + 1, 2, 2])[:w.num_seqs]  # sequence 1 asks for L + 1 queries
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q, _ = prefill_queries(w, int(ns.max()))
    q = q[:int(qs[-1])]
    try:
        got = _run_prefill(w, run, q, qs)
        assert run.device_error() & 4
        assert np.all(got[qs[1]:qs[2]] == 0.0)
        assert np.all(np.isfinite(got))
    finally:
        run.dev_err.zero_()  # the prepared run is shared with other test modules


@pytest.mark.parametrize("cfg", ["c2", "c4", "c5"])
def test_prefill_bad_block_is_flagged_and_skipped(cfg):
    """A block id outside the pool among a sequence's early blocks (read by every query,
    in the unmasked pairs) is flagged and skipped, as the decode skips it: that sequence's
    outputs equal exact attention over its other keys, the other sequences' are unchanged."""
    from oracle.attention import decode_dense, gather_sequence
    from oracle.formats import act_decode
    w, run, pool, ks, vs, near = _setup(cfg)
    n, bad = 16, 1  # block 1 (tokens 16 .. 31) of sequence 0
    q, qs = prefill_queries(w, n)
    L0 = int(w.context_lens[0])
    assert L0 - n >= 2 * 16 * 2  # the block lies in pairs before every query's position
    clean = _run_prefill(w, run, q, qs)
    assert run.device_error() == 0
    bt = run.block_tables.clone()
    try:
        run.block_tables[0, bad] = w.num_blocks + 7
        got = _run_prefill(w, run, q, qs)
        e = run.device_error()
    finally:
        run.block_tables.copy_(bt)
    assert e & 1
    assert np.array_equal(got[n:], clean[n:])
    k_seq, v_seq = gather_sequence(pool, w.block_tables[0], L0, ks, vs)
    qv = act_decode(q, w.act)
    want = np.zeros((n, w.num_q_heads, w.head_dim))
    for i in range(n):
        keep = np.arange(L0 - n + i + 1)
        keep = keep[(keep // 16) != bad]
        want[i], _ = decode_dense(qv[i], k_seq[keep], v_seq[keep], float(w.sm_scale))
    assert_close(got[:n], want, f"{cfg} bad block")
