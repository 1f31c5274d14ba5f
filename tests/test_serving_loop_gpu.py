"""A serving loop on the GPU, step for step against the oracle doing the same operations.

Block ids come from the library's reference-counted allocator. Prompts are written in
32-token chunks (pa_cache_write); then every step appends one token per running sequence
and decodes it in one launch (pa_append_decode), opening a new block whenever a sequence
crosses a 16-token boundary. Along the way a sequence forks (beam search: all its blocks
shared, the shared partial block copied on the next write, pa_copy_blocks), a sequence
finishes (its blocks freed, FP4 records re-armed with pa_reset_blocks before reuse), and a
sequence is preempted (its blocks swapped out to a pinned host pool and freed) and later
resumed (new blocks, swapped back in). After every step each running sequence's output is
within max-abs 2e-3 and relative L2 1e-2 of the oracle's exact decode over the oracle's
own pool, and at the end every block in use is bit-exact."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import blocks as OB
from oracle import cache as C
from oracle_side import assert_close, assert_pool_equal

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import _say  # noqa: E402

HKV, HQ, D, NB, CHUNK = 2, 8, 128, 48, 32


def _bf16(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


class Loop:
    def __init__(self, kind, seed):
        from paged_quantized_kv_reshape_amd import BlockAllocator, KVPool
        self.kind = kind
        self.rng = np.random.default_rng(seed)
        self.ks = self.vs = None
        dks = dvs = None
        if kind in ("fp8", "bf8"):  # per-head scales, fixed for the run
            self.ks = np.array([0.02, 0.03], dtype=np.float32)
            self.vs = np.array([0.025, 0.015], dtype=np.float32)
            dks, dvs = torch.from_numpy(self.ks).cuda(), torch.from_numpy(self.vs).cuda()
        self.dev = KVPool(kind, NB, HKV, D, fill=0xA5, k_scale=dks, v_scale=dvs)
        self.ora = C.Pool.filled(kind, NB, HKV, D)
        self.alloc = BlockAllocator(NB)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.tables = {}  # sequence id -> list of block ids
        self.lens = {}

    def rows(self, n):
        x = self.rng.standard_normal((2, n, HKV, D)).astype(np.float32)
        x[:, :, :, 7] *= 20.0  # an outlier channel (FP4 keeps it in fp16)
        return _bf16(x[0]), _bf16(x[1])

    def new_blocks(self, n):
        return self.alloc.alloc(n)

    def write(self, sid, kb, vb, positions):
        from paged_quantized_kv_reshape_amd import pa_cache_write
        t = self.tables[sid]
        slots = np.array([t[p // 16] * 16 + p % 16 for p in positions], dtype=np.int64)
        C.cache_write(self.ora, kb, vb, "bf16", slots, self.ks, self.vs)
        kt = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
        vt = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
        pa_cache_write(self.dev, kt, vt, torch.from_numpy(slots).cuda(), self.err)

    def prefill(self, sid, L):
        self.tables[sid] = self.new_blocks(-(-L // 16))
        self.lens[sid] = L
        kb, vb = self.rows(L)
        for lo in range(0, L, CHUNK):
            hi = min(lo + CHUNK, L)
            self.write(sid, kb[lo:hi], vb[lo:hi], range(lo, hi))

    def copy(self, src_pool, dst_pool, osrc, odst, pairs):
        from paged_quantized_kv_reshape_amd import pa_copy_blocks
        p = torch.from_numpy(np.asarray(pairs, dtype=np.int32).reshape(-1, 2)).cuda()
        pa_copy_blocks(src_pool, dst_pool, p, self.err)
        OB.copy_blocks(osrc, odst, pairs)

    def free(self, ids):
        from paged_quantized_kv_reshape_amd import pa_reset_blocks
        freed = self.alloc.release(ids)
        if self.kind == "fp4" and freed:
            pa_reset_blocks(self.dev, torch.tensor(freed, dtype=torch.int32, device="cuda"))
            for side in ("k", "v"):
                C.fp4_records(self.ora, side)[freed] = C.UNCALIBRATED
        return freed

    def step(self, sids):
        """Append one token to each sequence and decode them all in one launch."""
        from paged_quantized_kv_reshape_amd import pa_append_decode
        for sid in sids:
            L = self.lens[sid]
            t = self.tables[sid]
            if L % 16 == 0:  # the new token opens a block
                t.append(self.new_blocks(1)[0])
            else:  # it goes into the last block: copy it first if it is shared
                new, must_copy = self.alloc.writable(t[-1])
                if must_copy:
                    self.copy(self.dev, self.dev, self.ora, self.ora, [[t[-1], new]])
                    t[-1] = new
            self.lens[sid] = L + 1
        kb, vb = self.rows(len(sids))
        for i, sid in enumerate(sids):  # the oracle's write of the same rows
            L = self.lens[sid] - 1
            slot = self.tables[sid][L // 16] * 16 + L % 16
            C.cache_write(self.ora, kb[i:i + 1], vb[i:i + 1], "bf16", np.array([slot]),
                          self.ks, self.vs)
        mb = max(len(self.tables[s]) for s in sids)
        bt = np.full((len(sids), mb), -1, dtype=np.int32)
        for i, sid in enumerate(sids):
            bt[i, :len(self.tables[sid])] = self.tables[sid]
        cl = np.array([self.lens[s] for s in sids], dtype=np.int32)
        q = _bf16(self.rng.standard_normal((len(sids), HQ, D)))
        dq = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
        kt = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
        vt = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
        out = torch.empty((len(sids), HQ, D), dtype=torch.float32, device="cuda")
        pa_append_decode(dq, self.dev, kt, vt, torch.from_numpy(bt).cuda(),
                         torch.from_numpy(cl).cuda(), 1.0 / np.sqrt(D), 0, out=out,
                         dev_err=self.err)
        torch.cuda.synchronize()
        assert int(self.err.item()) == 0
        ref = A.paged_decode(q, "bf16", self.ora, bt, cl, 1.0 / np.sqrt(D), self.ks, self.vs)
        got = out.cpu().numpy()
        for i, sid in enumerate(sids):
            assert_close(got[i], ref[i][0], f"{self.kind} seq {sid} at length {cl[i]}")

    def check_pools(self):
        used = {b for t in self.tables.values() for b in t}
        assert_pool_equal(self.dev.numpy(), self.ora, blocks=used)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp8t", "fp4"])
def test_serving_loop(kind):
    from paged_quantized_kv_reshape_amd import KVPool
    lp = Loop(kind, seed={"bf16": 1, "fp8": 2, "fp8t": 3, "fp4": 4}[kind])
    for sid, L in ((0, 40), (1, 17), (2, 64)):
        lp.prefill(sid, L)
    running = [0, 1, 2]
    host = KVPool(kind, 8, HKV, D, device="cpu", fill=0)
    ohost = C.Pool.filled(kind, 8, HKV, D, sentinel=0)
    swapped = None
    for step in range(24):
        if step == 4:  # beam search: sequence 3 forks from sequence 0
            lp.alloc.share(lp.tables[0])
            lp.tables[3] = list(lp.tables[0])
            lp.lens[3] = lp.lens[0]
            running.append(3)
        if step == 9:  # sequence 1 finishes
            running.remove(1)
            lp.free(lp.tables.pop(1))
            lp.lens.pop(1)
        if step == 12:  # sequence 2 is preempted: swapped out, its blocks freed
            t = lp.tables.pop(2)
            lp.copy(lp.dev, host, lp.ora, ohost, [[b, i] for i, b in enumerate(t)])
            lp.free(t)
            swapped = (len(t), lp.lens.pop(2))
            running.remove(2)
        if step == 17:  # ... and resumed in new blocks
            n, L = swapped
            t = lp.alloc.alloc(n)
            lp.copy(host, lp.dev, ohost, lp.ora, [[i, b] for i, b in enumerate(t)])
            lp.tables[2], lp.lens[2] = t, L
            running.append(2)
        _say(f"[serving {kind}] step {step}: running {running} "
             f"lens {[lp.lens[s] for s in running]} free {lp.alloc.num_free}")
        lp.step(running)
    lp.check_pools()
    assert lp.alloc.refcount(lp.tables[0][0]) == 2  # still shared by the two beams
    lp.alloc.close()
