"""GPU test of pa_decode_split_static, the split decode + merge that allocates nothing (its
partials live in the library's static device scratch): its output must equal, bit for bit,
pa_decode with caller-provided partials followed by pa_merge, on two calls in a row, the
second with a smaller input (fewer sequences, shorter contexts, a smaller table) so that the
scratch still holds the first call's partials; the first call is also checked against the
oracle. A call needing more than the scratch is refused before anything is queued."""
import numpy as np
import pytest

from oracle_side import assert_close, oracle_decode, replay
from workload import config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _reference(run, q, bt, cl, ps):
    """pa_decode (caller partials) + pa_merge on the given rows of the batch."""
    from paged_quantized_kv_reshape_amd import max_partitions, pa_decode, pa_merge
    S, Hq, D = q.shape
    P = max_partitions(bt.shape[1], ps)
    po = torch.full((S, Hq, P, D), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((S, Hq, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    pa_decode(q, run.pool, bt, cl, run.w.sm_scale, ps, part_out=po, part_lse=pl,
              dev_err=run.dev_err)
    pa_merge(po, pl, cl, ps, out, lse)
    return out, lse


def _static(run, q, bt, cl, ps):
    from paged_quantized_kv_reshape_amd import pa_decode_split_static
    S, Hq, D = q.shape
    out = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    pa_decode_split_static(q, run.pool, bt, cl, run.w.sm_scale, ps, out, lse, run.dev_err)
    return out, lse


@pytest.mark.parametrize("cfg,over,ps", [
    ("c5", dict(num_seqs=3, lens_range=(1500, 4000)), 512),
    ("c4", dict(num_seqs=4, lens=[2000, 2048, 1999, 33]), 64),
    ("c2", dict(num_seqs=3, lens=[700, 16, 300]), 128),
])
def test_static_scratch_matches_decode_and_merge(cfg, over, ps):
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config(cfg, **over)
    run = DeviceRun(w, partition_size=ps)
    run.prepare()
    # call 1: the whole batch
    got, got_lse = _static(run, run.q, run.block_tables, run.context_lens, ps)
    want, want_lse = _reference(run, run.q, run.block_tables, run.context_lens, ps)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    assert torch.equal(got, want) and torch.equal(got_lse, want_lse)
    pool, ks, vs, _ = replay(w)
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(got.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]),
                 f"static scratch {cfg}")
    # call 2, smaller: the last sequences only, their contexts cut short, a narrower table
    n = w.num_seqs - 1
    cl2 = torch.clamp(run.context_lens[1:] // 2, min=1).contiguous()
    mb2 = int((cl2.max().item() + 15) // 16)
    bt2 = run.block_tables[1:, :mb2].contiguous()
    q2 = run.q[1:].contiguous()
    got2, lse2 = _static(run, q2, bt2, cl2, ps)
    want2, wlse2 = _reference(run, q2, bt2, cl2, ps)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    assert got2.shape[0] == n
    assert torch.equal(got2, want2) and torch.equal(lse2, wlse2)


def test_static_scratch_refuses_oversize_calls():
    from paged_quantized_kv_reshape_amd import PAError, pa_decode_split_static
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    w = config("c4", num_seqs=2, lens=[40, 70])
    run = DeviceRun(w, partition_size=16)
    run.prepare()
    # 64 sequences x 8 heads x 4096 partitions x 129 floats: about 1 GB of partials
    bt = torch.zeros((64, 4096), dtype=torch.int32, device="cuda")
    cl = torch.ones(64, dtype=torch.int32, device="cuda")
    q = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((64, 8, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(PAError) as e:
        pa_decode_split_static(q, run.pool, bt, cl, w.sm_scale, 16, out)
    assert e.value.status == -12
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was queued
