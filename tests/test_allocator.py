"""Host logic of libpa's reference-counted block allocator (pa_allocator_*), no GPU.

A plain Python model (a reference count per id and a stack of free ids) is driven through
the same long random sequence of alloc / share / release / writable calls as the library,
including calls that must fail; after every call both agree on the result, every
reference count and the free count, and the library's invariants hold: a live block is
never handed out, free + live = all blocks, and failed calls change nothing."""
import numpy as np
import pytest

B = pytest.importorskip("paged_quantized_kv_reshape_amd.binding")

SHAPE, EXHAUSTED, STATE = -2, -10, -11


class Model:
    def __init__(self, n):
        self.refs = [0] * n
        self.stack = list(range(n - 1, -1, -1))

    def alloc(self, k):
        if k > len(self.stack):
            return EXHAUSTED
        out = []
        for _ in range(k):
            i = self.stack.pop()
            self.refs[i] = 1
            out.append(i)
        return out

    def _bad(self, ids, need):
        for i in ids:
            if not 0 <= i < len(self.refs):
                return SHAPE
            if self.refs[i] == 0:
                return STATE
        if need:
            u, c = np.unique(ids, return_counts=True)
            if any(c[j] > self.refs[u[j]] for j in range(len(u))):
                return STATE
        return 0

    def share(self, ids):
        st = self._bad(ids, False)
        if st:
            return st
        for i in ids:
            self.refs[i] += 1
        return 0

    def release(self, ids):
        st = self._bad(ids, True)
        if st:
            return st
        freed = []
        for i in ids:
            self.refs[i] -= 1
            if self.refs[i] == 0:
                self.stack.append(i)
                freed.append(i)
        return freed

    def writable(self, i):
        if not 0 <= i < len(self.refs):
            return SHAPE
        if self.refs[i] == 0:
            return STATE
        if self.refs[i] == 1:
            return (i, False)
        if not self.stack:
            return EXHAUSTED
        j = self.stack.pop()
        self.refs[j] = 1
        self.refs[i] -= 1
        return (j, True)


def _call(fn, *a):
    try:
        return fn(*a)
    except B.PAError as e:
        return e.status


@pytest.mark.parametrize("seed", range(4))
def test_random_sequences_match_the_model(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    lib_a, m = B.BlockAllocator(n), Model(n)
    for step in range(3000):
        live = [i for i in range(n) if m.refs[i] > 0]
        op = rng.integers(0, 4)
        if op == 0:
            k = int(rng.integers(0, 6))
            want, got = m.alloc(k), _call(lib_a.alloc, k)
        elif op == 1:
            pick = list(rng.choice(live, size=min(len(live), 3))) if live else []
            if rng.random() < 0.1:
                pick.append(int(rng.integers(-2, n + 2)))  # sometimes free or out of range
            want, got = m.share(pick), _call(lib_a.share, pick)
            want = None if want == 0 else want
        elif op == 2:
            pick = list(rng.choice(live, size=min(len(live), int(rng.integers(1, 5))))) if live else []
            if rng.random() < 0.1:
                pick.append(int(rng.integers(-2, n + 2)))
            want, got = m.release(pick), _call(lib_a.release, pick)
        else:
            i = int(rng.choice(live)) if live and rng.random() < 0.9 else int(rng.integers(-1, n + 1))
            want, got = m.writable(i), _call(lib_a.writable, i)
        assert got == want, (step, op, got, want)
        assert lib_a.num_free == len(m.stack)
        assert [lib_a.refcount(i) for i in range(n)] == m.refs
        assert sum(r > 0 for r in m.refs) + len(m.stack) == n
    lib_a.close()


def test_order_and_edge_cases():
    a = B.BlockAllocator(4)
    assert a.alloc(2) == [0, 1]           # ascending at first
    assert a.release([1]) == [1]
    assert a.alloc(1) == [1]              # most recently freed first
    assert _call(a.alloc, 3) == EXHAUSTED and a.num_free == 2   # all or nothing
    assert a.alloc(0) == []
    a.share([0, 0])                       # repeats allowed
    assert a.refcount(0) == 3
    assert a.writable(0) == (2, True) and a.refcount(0) == 2 and a.refcount(2) == 1
    assert a.writable(2) == (2, False)
    assert _call(a.release, [0, 0, 0]) == STATE and a.refcount(0) == 2   # would go below 0
    assert a.release([0, 0]) == [0]
    assert _call(a.share, [0]) == STATE   # free block
    assert _call(a.refcount, 4) == SHAPE and _call(a.refcount, -1) == SHAPE
    assert a.refcount(0) == 0
    a.alloc(a.num_free)
    a.share([1])
    assert _call(a.writable, 1) == EXHAUSTED and a.refcount(1) == 2
    a.close()
    with pytest.raises(B.PAError):
        B.BlockAllocator(0)


def test_null_and_shape_rejects():
    import ctypes
    lib = B.lib()
    assert lib.pa_allocator_create(4, None) == -1
    assert lib.pa_allocator_destroy(None) == -1
    assert lib.pa_allocator_alloc(None, 1, None) == -1
    assert lib.pa_allocator_num_free(None) == -1
    a = B.BlockAllocator(3)
    assert lib.pa_allocator_alloc(a._h, -1, None) == SHAPE
    assert lib.pa_allocator_alloc(a._h, 1, None) == -1
    assert lib.pa_allocator_release(a._h, None, 1, None, None) == -1
    assert lib.pa_allocator_writable(a._h, 0, None) == -1
    # release with no outputs asked for
    ids = (ctypes.c_int32 * 1)(*a.alloc(1))
    assert lib.pa_allocator_release(a._h, ids, 1, None, None) == 0 and a.num_free == 3
    a.close()
