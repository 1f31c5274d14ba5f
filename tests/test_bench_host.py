"""The bench's host-side legs, on the CPU: the oracle timing record (all threads, then one,
with the host's core counts) and the parity check the bench applies to its own timed
output (a correct output passes; one off by more than the tolerance fails)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from workload import config  # noqa: E402


def test_cpu_baseline_record_and_parity_check():
    w = config("c4", num_seqs=3, lens=[40, 77, 16])
    rec, outs = bench.cpu_baseline(w, 0.05, 256.0)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["single_thread"]["value"] > 0
    assert rec["host"]["cpu_count"] >= 1 and rec["host"]["affinity"] >= 1
    assert rec["cores"] == rec["host"]["blas_threads"] >= 1
    assert rec["single_thread"]["cores"] == 1
    assert set(outs) and all(outs[s].shape == (w.num_q_heads, w.head_dim) for s in outs)
    # the untimed path gives the same outputs
    again = bench.oracle_outputs(w, sorted(outs))
    for s in outs:
        assert np.array_equal(outs[s], again[s])
    got = np.zeros((w.num_seqs, w.num_q_heads, w.head_dim), dtype=np.float32)
    for s in outs:
        got[s] = outs[s]
    assert bench.parity_check(got, outs)["ok"]
    s0 = sorted(outs)[0]
    got[s0, 0, 0] += 3e-3
    p = bench.parity_check(got, outs)
    assert not p["ok"] and p["max_abs"] > 2e-3


def test_split_workload_outputs_are_merged():
    w = config("c5", num_seqs=2, lens=[1100, 700])
    outs = bench.oracle_outputs(w, [0, 1])
    assert all(outs[s].shape == (w.num_q_heads, w.head_dim) for s in outs)
    assert all(np.isfinite(outs[s]).all() for s in outs)
