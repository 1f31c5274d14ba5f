"""GPU parity of pa_append_decode (each sequence's new row written at its last position by
the decode launch itself) against the oracle's cache write followed by its exact decode.

Pools bit-exact after the step in every format (fp16, bf16, FP8 E4M3 / E5M2 with per-head
or per-token scales, FP4 with outliers, including blocks the new row opens and calibrates);
outputs within max-abs 2e-3 and relative L2 1e-2, single pass and split (with pa_merge),
1 and 4 waves per workgroup; and bit for bit the output of pa_cache_write followed by
pa_decode on the same inputs."""

import numpy as np
import pytest

from oracle_side import assert_close, assert_pool_equal, oracle_decode, replay
from workload import config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import _say  # noqa: E402

CASES = {
    "f16": ("c1", {}),
    "bf16": ("c2", dict(num_seqs=4, lens=[300, 77, 16, 1])),
    "fp8": ("c3", dict(num_seqs=4, lens_range=(200, 900), step_tokens=1)),
    "fp8-c4": ("c4", dict(num_seqs=4, lens=[2000, 2048, 1999, 33])),
    "bf8": ("c4", dict(num_seqs=3, lens=[300, 77, 16], kv="bf8")),
    "fp8t": ("c4", dict(num_seqs=3, lens=[300, 77, 17], kv="fp8t")),
    "bf8t": ("c4", dict(num_seqs=3, lens=[300, 64, 16], kv="bf8t", head_dim=64,
                        num_kv_heads=2)),
    # FP4: last positions 299 (inside a calibrated block), 976, 32 and 16 (each the first
    # row of a fresh block, calibrated on that row alone, as the separate write does)
    "fp4": ("c5", dict(num_seqs=4, lens=[300, 977, 33, 17])),
    "fp4-2kv": ("c5", dict(num_seqs=3, lens=[129, 50, 1], num_kv_heads=2, num_q_heads=16,
                           act="f16")),
    "fp4-d64": ("c5", dict(num_seqs=4, lens=[300, 977, 33, 17], head_dim=64, num_kv_heads=2,
                           num_q_heads=8)),
}


@pytest.mark.parametrize("waves", [1, 4])
@pytest.mark.parametrize("ps", [0, 64, 512])
@pytest.mark.parametrize("case", list(CASES))
def test_append_decode_matches_oracle_and_separate_calls(case, ps, waves):
    from paged_quantized_kv_reshape_amd import max_partitions, pa_append_decode, pa_merge
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base, over = CASES[case]
    w = config(base, **over)
    sc = w.step_call
    assert len(sc.rows) == w.num_seqs  # one new token per sequence, at its last position
    last = w.seq_start + w.context_lens.astype(np.int64) - 1
    assert np.array_equal(sc.rows, last)
    _say(f"[append] {case} ({w.kv}) ps={ps} W={waves} lens={w.context_lens.tolist()}")
    run = DeviceRun(w, partition_size=ps, pool_copies=2, waves=waves)
    for p in run.pools:
        run.setup_writes(p)
    # (1) the fused step on pool 0
    S, Hq, D = w.q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    po = pl = None
    if ps:
        P = max_partitions(w.max_blocks_per_seq, ps)
        po = torch.empty((S, Hq, P, D), dtype=torch.float32, device="cuda")
        pl = torch.empty((S, Hq, P), dtype=torch.float32, device="cuda")
    pa_append_decode(run.q, run.pools[0], run.step_k, run.step_v, run.block_tables,
                     run.context_lens, w.sm_scale, ps, out=None if ps else out, part_out=po,
                     part_lse=pl, dev_err=run.dev_err, waves=waves)
    if ps:
        pa_merge(po, pl, run.context_lens, ps, out)
    # (2) the separate calls on pool 1
    run.step_write(run.pools[1])
    run.decode(run.pools[1])
    torch.cuda.synchronize()
    assert run.device_error() == 0
    pool, ks, vs, near = replay(w)
    assert_pool_equal(run.pools[0].numpy(), pool, near=near)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), run.out.cpu().numpy().view(np.uint32))
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(got, np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"append {case} ps={ps} W={waves}")


def test_append_decode_flags_a_bad_last_block():
    """A block table whose entry at a sequence's last position is out of range: flagged,
    nothing written, the other sequences unaffected."""
    from paged_quantized_kv_reshape_amd import pa_append_decode
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", num_seqs=3, lens=[300, 77, 16])
    run = DeviceRun(w, partition_size=0)
    run.setup_writes()
    before = {n: t.clone() for n, t in run.pool.bytes.items()}
    bt = run.block_tables.clone()
    bt[1, (77 - 1) // 16] = w.num_blocks + 5
    out = torch.empty_like(run.out)
    pa_append_decode(run.q, run.pool, run.step_k, run.step_v, bt, run.context_lens, w.sm_scale,
                     0, out=out, dev_err=run.dev_err)
    torch.cuda.synchronize()
    assert run.device_error() == 1  # PA_DEVERR_BAD_BLOCK
    pool, ks, vs, _ = replay(w)
    # sequences 0 and 2 got their new rows; sequence 1's last block was never touched
    got = run.pool.numpy()
    b1 = int(w.block_tables[1, (77 - 1) // 16])
    for name, t in before.items():
        g = got[name].reshape(w.num_blocks, -1)
        o = pool.arrays[name].view(np.uint8).reshape(w.num_blocks, -1)
        for s in (0, 2):
            b = int(w.block_tables[s, (int(w.context_lens[s]) - 1) // 16])
            assert np.array_equal(g[b], o[b])
        assert np.array_equal(g[b1], t.cpu().numpy().reshape(w.num_blocks, -1)[b1])
    ref = oracle_decode(w, pool, ks, vs, [0, 2])
    o = out.cpu().numpy()
    for s in (0, 2):
        assert_close(o[s], ref[s][0], f"bad block, seq {s}")


# several new rows per sequence (pa_append_decode_n): the last n positions of every
# sequence, written by the waves that read them; n = 8 is the 64-sequence FP8 workload's
# 512-row step, 20 and 33 span two and three blocks (rows of one sequence then go to
# different waves, and with ps = 64 to different partitions)
NCASES = {
    "fp8-n8": ("c3", dict(num_seqs=4, lens_range=(200, 900)), 8),
    "fp8-n20": ("c3", dict(num_seqs=3, lens=[300, 77, 20]), 20),
    "bf16-n33": ("c2", dict(num_seqs=3, lens=[300, 77, 33]), 33),
    "fp8t-n5": ("c4", dict(num_seqs=3, lens=[300, 77, 17], kv="fp8t"), 5),
    "bf8-d64-n16": ("c4", dict(num_seqs=3, lens=[300, 64, 16], kv="bf8", head_dim=64,
                               num_kv_heads=2), 16),
    "f16-n2": ("c1", {}, 2),
}


@pytest.mark.parametrize("waves", [1, 4])
@pytest.mark.parametrize("ps", [0, 64])
@pytest.mark.parametrize("case", list(NCASES))
def test_append_decode_n_matches_oracle_and_separate_calls(case, ps, waves):
    from paged_quantized_kv_reshape_amd import max_partitions, pa_append_decode_n, pa_merge
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base, over, n = NCASES[case]
    w = config(base, step_tokens=n, **over)
    run = DeviceRun(w, partition_size=ps, pool_copies=2, waves=waves)
    assert run.step_rows_per_seq == n  # the step writes the last n positions of each sequence
    _say(f"[append n] {case} ({w.kv}) n={n} ps={ps} W={waves} lens={w.context_lens.tolist()}")
    for p in run.pools:
        run.setup_writes(p)
    S, Hq, D = w.q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    po = pl = None
    if ps:
        P = max_partitions(w.max_blocks_per_seq, ps)
        po = torch.empty((S, Hq, P, D), dtype=torch.float32, device="cuda")
        pl = torch.empty((S, Hq, P), dtype=torch.float32, device="cuda")
    kn = run.step_k.view(S, n, *run.step_k.shape[1:])
    vn = run.step_v.view(S, n, *run.step_v.shape[1:])
    pa_append_decode_n(run.q, run.pools[0], kn, vn, run.block_tables, run.context_lens,
                       w.sm_scale, ps, out=None if ps else out, part_out=po, part_lse=pl,
                       dev_err=run.dev_err, waves=waves)
    if ps:
        pa_merge(po, pl, run.context_lens, ps, out)
    run.step_write(run.pools[1])
    run.decode(run.pools[1])
    torch.cuda.synchronize()
    assert run.device_error() == 0
    pool, ks, vs, near = replay(w)
    assert_pool_equal(run.pools[0].numpy(), pool, near=near)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), run.out.cpu().numpy().view(np.uint32))
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(got, np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"append n {case} ps={ps} W={waves}")


def test_append_decode_n_flags_a_context_shorter_than_its_new_rows():
    """A sequence with fewer tokens than new rows: flagged as a bad context, nothing of it
    written, a zero output; the other sequences as the separate calls give them."""
    from paged_quantized_kv_reshape_amd import pa_append_decode_n
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    n = 8
    w = config("c3", num_seqs=3, lens=[300, 77, 40], step_tokens=n)
    run = DeviceRun(w, partition_size=0)
    run.setup_writes()
    before = {k: t.clone() for k, t in run.pool.bytes.items()}
    cl = run.context_lens.clone()
    cl[1] = n - 1  # sequence 1 now claims 7 tokens but gets 8 new rows
    S = w.num_seqs
    out = torch.full_like(run.out, float("nan"))
    pa_append_decode_n(run.q, run.pool, run.step_k.view(S, n, *run.step_k.shape[1:]),
                       run.step_v.view(S, n, *run.step_v.shape[1:]), run.block_tables, cl,
                       w.sm_scale, 0, out=out, dev_err=run.dev_err)
    torch.cuda.synchronize()
    assert run.device_error() == 4  # PA_DEVERR_BAD_CONTEXT
    o = out.cpu().numpy()
    assert np.all(o[1] == 0.0)
    # sequence 1's blocks are untouched; 0 and 2 got their rows and decode as the oracle
    got = run.pool.numpy()
    for name, t in before.items():
        g = got[name].reshape(w.num_blocks, -1)
        b0 = t.cpu().numpy().reshape(w.num_blocks, -1)
        for b in w.block_tables[1, :-(-77 // 16)]:
            assert np.array_equal(g[int(b)], b0[int(b)])
    pool, ks, vs, _ = replay(w)
    ref = oracle_decode(w, pool, ks, vs, [0, 2])
    for s in (0, 2):
        assert_close(o[s], ref[s][0], f"short context, seq {s}")
