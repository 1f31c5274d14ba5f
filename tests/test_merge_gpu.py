"""GPU parity of pa_merge alone: the log-sum-exp merge of split-KV partials against the
oracle's merge (fp64) on seeded partials.

The partials are drawn directly (normalized outputs ~ N(0, 1), lse values over a wide
range, some partitions empty with lse = -inf), so the cases reach what decode partials of a
real workload rarely do: hundreds of partitions per (sequence, head), so that every wave
takes several batches; maxima that rise batch after batch (each batch rescales the state),
fall, or sit in one partition; a sequence whose only partition is empty; and ragged counts
ceil(L / ps) against the allocated max_partitions. Outputs within max-abs 2e-3 and relative
L2 1e-2 (the decode's bar; the merge itself is good to about 1e-6), merged lse within 1e-4.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle_side import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _partials(rng, S, Hq, P, D, order):
    o = rng.standard_normal((S, Hq, P, D)).astype(np.float32)
    if order == "rising":  # every batch raises the running maximum
        lse = np.linspace(-40.0, 40.0, P)[None, None, :] + rng.standard_normal((S, Hq, P))
    elif order == "falling":
        lse = np.linspace(40.0, -40.0, P)[None, None, :] + rng.standard_normal((S, Hq, P))
    elif order == "spike":  # one partition dominates, the rest are far below it
        lse = rng.standard_normal((S, Hq, P)) - 30.0
        lse[..., P // 2] = 10.0
    else:
        lse = rng.standard_normal((S, Hq, P)) * 8.0
    lse = lse.astype(np.float32)
    lse[..., 5::13] = -np.inf  # empty partitions (every block id of the partition was bad)
    return o, lse


@pytest.mark.parametrize("order", ["random", "rising", "falling", "spike"])
@pytest.mark.parametrize("D,P,ps", [(128, 1, 512), (128, 17, 64), (128, 240, 512),
                                    (64, 300, 16), (128, 700, 16)])
def test_merge_matches_oracle(D, P, ps, order):
    from paged_quantized_kv_reshape_amd import pa_merge
    rng = np.random.default_rng(1000 + P + D)
    S, Hq = 6, 3
    o, lse = _partials(rng, S, Hq, P, D, order)
    # context lengths: a single token, a full last partition, everything, ragged counts;
    # with P = 1, sequence 5's only partition is empty
    lens = np.array([1, ps, P * ps, max(1, P * ps - ps + 3), max(1, (P * ps) // 3),
                     max(1, (P * ps * 2) // 3 + 1)], dtype=np.int32)
    if P == 1:
        lse[5, :, 0] = -np.inf
    dev = dict(device="cuda")
    po = torch.from_numpy(o).to(**dev)
    pl = torch.from_numpy(lse).to(**dev)
    cl = torch.from_numpy(lens).to(**dev)
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, **dev)
    lse_out = torch.full((S, Hq), float("nan"), dtype=torch.float32, **dev)
    pa_merge(po, pl, cl, ps, out, lse_out)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse_out.cpu().numpy()
    for s in range(S):
        n = min(-(-int(lens[s]) // ps), P)
        for h in range(Hq):
            what = f"merge D={D} P={P} ps={ps} {order} seq {s} head {h}"
            if np.all(np.isneginf(lse[s, h, :n])):  # nothing to merge: zeros, lse -inf
                assert np.all(got[s, h] == 0.0) and np.isneginf(got_lse[s, h]), what
                continue
            want, want_lse = A.merge(o[s, h, :n].astype(np.float64),
                                     lse[s, h, :n].astype(np.float64))
            assert_close(got[s, h], want, what)
            assert np.abs(got[s, h] - want).max() < 1e-4, what
            assert abs(got_lse[s, h] - want_lse) < 1e-4 * max(1.0, abs(want_lse)), what


def test_merge_ignores_nonfinite_partials_and_overlong_contexts():
    """A partition whose lse is not finite (NaN, +inf or -inf) weighs 0 and its row, which
    may hold anything (NaN here), is not read into the sum; a context that the partitions
    cannot hold (L > P * ps) or an empty one gives a zero output and lse -inf."""
    from paged_quantized_kv_reshape_amd import pa_merge
    rng = np.random.default_rng(5)
    S, Hq, P, D, ps = 4, 2, 40, 128, 64
    o = rng.standard_normal((S, Hq, P, D)).astype(np.float32)
    lse = (rng.standard_normal((S, Hq, P)) * 4.0).astype(np.float32)
    lse[:, :, 3] = -np.inf
    lse[:, :, 7] = np.nan
    lse[:, :, 11] = np.inf
    o[:, :, [3, 7, 11]] = np.nan
    lens = np.array([P * ps, 17 * ps + 5, P * ps + 1, 0], dtype=np.int32)
    dev = dict(device="cuda")
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, **dev)
    lse_out = torch.full((S, Hq), float("nan"), dtype=torch.float32, **dev)
    pa_merge(torch.from_numpy(o).to(**dev), torch.from_numpy(lse).to(**dev),
             torch.from_numpy(lens).to(**dev), ps, out, lse_out)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse_out.cpu().numpy()
    assert np.isfinite(got).all()
    for s in range(2):
        n = -(-int(lens[s]) // ps)
        for h in range(Hq):
            keep = np.isfinite(lse[s, h, :n])
            want, want_lse = A.merge(o[s, h, :n][keep].astype(np.float64),
                                     lse[s, h, :n][keep].astype(np.float64))
            assert_close(got[s, h], want, f"seq {s} head {h}")
            assert abs(got_lse[s, h] - want_lse) < 1e-4 * max(1.0, abs(want_lse))
    for s in (2, 3):
        assert np.all(got[s] == 0.0) and np.all(np.isneginf(got_lse[s]))
