"""GPU parity of FP4 per-sequence calibration: pa_fp4_sequence_outliers (one outlier set
per sequence, kv head and K|V from the sequence's first prefill chunk) and
pa_cache_write_seq_outliers (blocks a call opens adopt their sequence's set), against the
oracle's fp4_sequence_records and cache_write(seq_records=...).

Records bit-exact (a set whose closest channel lies within 1e-4, relative, of the
threshold is a near-tie that fp32 and fp64 statistics may decide differently: counted,
excluded, and 0 on these inputs); pools bit-exact after every write call of the workload;
decode within max-abs 2e-3 and relative L2 1e-2 of exact attention on the identical
dequantized cache; the full-size 70B long-context share checked on sampled sequences."""
import numpy as np
import pytest

from oracle import cache as C
from oracle_side import assert_close, assert_pool_equal, oracle_decode, seq_blocks
from workload import config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import _say  # noqa: E402

NEAR = 1e-4
CHUNK = 512


def _token_seq(w, rows):
    return (np.searchsorted(w.seq_start, rows, side="right") - 1).astype(np.int32)


def _first_chunk_rows(w):
    """Rows of each sequence's first prefill chunk (positions 0 .. min(512, L - 1) - 1)."""
    n = np.minimum(CHUNK, np.maximum(w.context_lens.astype(np.int64) - 1, 0))
    rows = np.concatenate([w.seq_start[s] + np.arange(n[s]) for s in range(w.num_seqs)])
    starts = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return rows.astype(np.int64), starts


def _dev(a, act):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if act == "bf16" else torch.float16)


def _records(w):
    from paged_quantized_kv_reshape_amd import pa_fp4_sequence_outliers
    rows, starts = _first_chunk_rows(w)
    kr, vr = w.k_rows[rows], w.v_rows[rows]
    recs = torch.full((w.num_seqs, 2, w.num_kv_heads, 16), 0xA5, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa_fp4_sequence_outliers(_dev(kr, w.act), _dev(vr, w.act), torch.from_numpy(starts).cuda(),
                             recs, err)
    orecs, margins = C.fp4_sequence_records(kr, vr, w.act, starts)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = recs.cpu().numpy()
    near = margins <= NEAR
    _say(f"[seq records] S={w.num_seqs} near-ties {int(near.sum())}")
    assert int(near.sum()) == 0
    assert np.array_equal(got, orecs)
    return recs, orecs


def _write_all(w, pool, opool, recs, orecs, only_blocks=None):
    from paged_quantized_kv_reshape_amd import pa_cache_write_seq_outliers
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for call in list(w.setup_calls) + [w.step_call]:
        ts = _token_seq(w, call.rows)
        pa_cache_write_seq_outliers(pool, _dev(w.k_rows[call.rows], w.act),
                                    _dev(w.v_rows[call.rows], w.act),
                                    torch.from_numpy(call.slots).cuda(),
                                    torch.from_numpy(ts).cuda(), recs, err)
        C.cache_write(opool, w.k_rows[call.rows], w.v_rows[call.rows], w.act, call.slots,
                      only_blocks=only_blocks, seq_records=orecs, token_seq=ts)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_seq_mode_write_and_decode(act):
    from paged_quantized_kv_reshape_amd import KVPool
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c5", num_seqs=3, lens=[1500, 977, 40], act=act)
    _say(f"[seq mode] {act}: lens {w.context_lens.tolist()}")
    recs, orecs = _records(w)
    run = DeviceRun(w, partition_size=512)
    pool = KVPool("fp4", w.num_blocks, w.num_kv_heads, w.head_dim, fill=0xA5)
    opool = C.Pool.filled("fp4", w.num_blocks, w.num_kv_heads, w.head_dim)
    _write_all(w, pool, opool, recs, orecs)
    assert_pool_equal(pool.numpy(), opool)
    # every block of a sequence carries that sequence's set
    for s in range(w.num_seqs):
        for b in w.block_tables[s, :-(-int(w.context_lens[s]) // 16)]:
            for side, name in enumerate("kv"):
                assert np.array_equal(C.fp4_records(opool, name)[b], orecs[s, side])
    run.decode(pool)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    ref = oracle_decode(w, opool, None, None, range(w.num_seqs))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"seq mode {act}")


def test_bad_ranges_and_sequence_ids_are_flagged():
    from paged_quantized_kv_reshape_amd import (KVPool, pa_cache_write_seq_outliers,
                                                pa_fp4_sequence_outliers)
    rng = np.random.default_rng(4)
    hkv, d = 2, 128
    x = torch.from_numpy(rng.standard_normal((20, hkv, d)).astype(np.float32)).cuda()
    xb = x.to(torch.bfloat16)
    starts = torch.tensor([0, 12, 8, 30], dtype=torch.int32, device="cuda")  # 2nd: 12 > 8; 3rd: 30 > 20
    recs = torch.full((3, 2, hkv, 16), 0xA5, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa_fp4_sequence_outliers(xb, xb, starts, recs, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 4  # PA_DEVERR_BAD_CONTEXT
    r = recs.cpu().numpy()
    assert (r[1:, :, :, 0] == 0).all() and (r[1:, :, :, 1:] == 0xFF).all()
    # a row naming a sequence outside [0, 3) opens its block with no outliers
    pool = KVPool("fp4", 4, hkv, d)
    err.zero_()
    slots = torch.tensor([16, 17, 32], dtype=torch.int64, device="cuda")
    pa_cache_write_seq_outliers(pool, xb[:3], xb[:3], slots,
                                torch.tensor([5, 5, 0], dtype=torch.int32, device="cuda"), recs, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 4
    rec = pool.fp4_records("k").cpu().numpy()
    assert (rec[1, :, 0] == 0).all()
    assert np.array_equal(rec[2], r[0, 0])


def test_full_size_seq_mode_sampled():
    """The 70B long-context share (32 sequences of 64k-120k tokens, 512-token prefill
    chunks) written in per-sequence mode and decoded with 512-token partitions; records
    compared in full, pools and outputs on sampled sequences."""
    from paged_quantized_kv_reshape_amd import KVPool, pa_cache_write_seq_outliers
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c5")
    _say(f"[full seq mode] S={w.num_seqs} tokens={w.tokens}")
    recs, orecs = _records(w)
    run = DeviceRun(w)
    pool = KVPool("fp4", w.num_blocks, w.num_kv_heads, w.head_dim, fill=0xA5)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for call in list(w.setup_calls) + [w.step_call]:
        idx = torch.from_numpy(call.rows).cuda()
        pa_cache_write_seq_outliers(pool, run.k_rows.index_select(0, idx),
                                    run.v_rows.index_select(0, idx),
                                    torch.from_numpy(call.slots).cuda(),
                                    torch.from_numpy(_token_seq(w, call.rows)).cuda(), recs, err)
    run.decode(pool)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and run.device_error() == 0
    seqs = [0, w.num_seqs - 1]
    blocks = seq_blocks(w, seqs)
    opool = C.Pool.filled("fp4", w.num_blocks, w.num_kv_heads, w.head_dim)
    for call in list(w.setup_calls) + [w.step_call]:
        C.cache_write(opool, w.k_rows[call.rows], w.v_rows[call.rows], w.act, call.slots,
                      only_blocks=blocks, seq_records=orecs, token_seq=_token_seq(w, call.rows))
    assert_pool_equal(pool.numpy(), opool, blocks=blocks)
    ref = oracle_decode(w, opool, None, None, seqs)
    out = run.out.cpu().numpy()
    for s in seqs:
        assert_close(out[s], ref[s][0], f"full seq mode, seq {s}")
