"""GPU checks of what the bench times beyond the decode step: multi-token queries at the
bench's size (every sequence of the 70B one-GPU share, FP8, 256 x 8192, with its last 512
positions as queries over the whole context, in the library's launch configuration),
sampled against the oracle; and the gather-only probe the bench reports as the ceiling of
the decode's access pattern (it reads, flags bad ids like the decode, and stays in
bounds)."""
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle_side import assert_close, replay, seq_blocks
from workload import config, prefill_queries

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


def test_prefill_chunk_full_size_sampled():
    """pa_prefill over 256 sequences x 8192 tokens with 512 queries each (chunked prefill,
    dailyaiworld.com engine diagram: 512-token chunks); queries at both ends and the middle
    of the chunks of three sequences, against exact causal attention over the oracle's
    replay of their blocks."""
    from paged_quantized_kv_reshape_amd import pa_prefill
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4")
    run = DeviceRun(w, partition_size=0)
    run.prepare()
    q_bits, qs = prefill_queries(w, 512)
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    qs_t = torch.from_numpy(qs).cuda()
    out = torch.full((q.shape[0], w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                     device="cuda")
    _say(f"[prefill full] c4: {q.shape[0]} queries")
    pa_prefill(q, qs_t, int(np.diff(qs).max()), run.pool, run.block_tables, run.context_lens,
               w.sm_scale, out, run.dev_err)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    seqs = [0, 128, 255]
    pool, ks, vs, _ = replay(w, only_blocks=seq_blocks(w, seqs))
    for s in seqs:
        n = int(qs[s + 1] - qs[s])
        L = int(w.context_lens[s])
        for i in (0, 1, 255, n - 2, n - 1):
            row = int(qs[s]) + i
            sub = np.array([0, 1], dtype=np.int32)  # one query, at position L - n + i
            L_sub = np.array([L - n + i + 1], dtype=np.int32)
            want = A.paged_prefill(q_bits[row:row + 1], w.act, pool, w.block_tables[s:s + 1],
                                   L_sub, sub, w.sm_scale, ks, vs)[0][0]
            assert_close(got[row], want, f"prefill seq {s} query {i}")


@pytest.mark.parametrize("cfg,ps", [("c4", 0), ("c5", 512), ("c2", 1024)])
def test_gather_probe_runs_and_flags(cfg, ps):
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    small = {"c4": dict(num_seqs=4, lens=[2000, 2048, 1999, 33]),
             "c5": dict(num_seqs=3, lens_range=(1500, 4000)),
             "c2": dict(num_seqs=4, lens_range=(200, 900))}[cfg]
    w = config(cfg, **small)
    run = DeviceRun(w, partition_size=ps)
    run.prepare()
    for waves in (None, 1, 8):
        run.waves = waves
        run.gather_probe()
        torch.cuda.synchronize()
        assert run.device_error() == 0, f"waves={waves}"
    run.block_tables[1, 2] = w.num_blocks + 3
    run.gather_probe()
    torch.cuda.synchronize()
    assert run.device_error() & 1
