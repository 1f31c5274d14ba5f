"""C-ABI checks that need no GPU: libpa.so loads, exports every entry point include/pa.h
declares, and rejects each invalid argument with its status before any HIP call.

Only rejected calls (and the no-op num_tokens = 0 / num_seqs = 0 forms) are made here:
fake device addresses never reach a kernel launch."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

B = pytest.importorskip("paged_quantized_kv_reshape_amd.binding")

PA_OK, NULL, SHAPE, DTYPE, BLOCK, CONTEXT, PART, LAUNCH, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7, -8
MEMORY, EXHAUSTED, STATE, SCRATCH, SCALE = -9, -10, -11, -12, -13
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _declared():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(pa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_entry_point():
    lib = B.lib()
    names = _declared()
    assert {"pa_cache_write", "pa_decode", "pa_merge", "pa_pool_layout"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = B.lib()
    for code in (PA_OK, NULL, SHAPE, DTYPE, BLOCK, CONTEXT, PART, LAUNCH, ALIGN, MEMORY,
                 EXHAUSTED, STATE, SCRATCH, SCALE):
        s = lib.pa_status_string(code).decode()
        assert s.startswith("PA_"), s
    assert "unknown" in lib.pa_status_string(-99).decode()


@pytest.mark.parametrize("kv,d,expect", [
    ("f16", 128, [2 * 10 * 3 * 16 * 128] * 2 + [0] * 2),
    ("bf16", 64, [2 * 10 * 3 * 16 * 64] * 2 + [0] * 2),
    ("fp8", 128, [10 * 3 * 16 * 128] * 2 + [0] * 2),
    # FP4: per (block, head) 1024 code bytes + 64 scale bytes + 16 record bytes + 32 bytes of
    # the first outlier, padded to 1152; then 10 more outlier slots of 16 fp16 values
    ("fp4", 128, [10 * 3 * 1152] * 2 + [10 * 3 * 10 * 16 * 2] * 2),
    # head_dim 64: 512 + 64 + 16 + 32 bytes padded to 640; 4 more outlier slots (capacity 5)
    ("fp4", 64, [10 * 3 * 640] * 2 + [10 * 3 * 4 * 16 * 2] * 2),
    ("bf8", 128, [10 * 3 * 16 * 128] * 2 + [0] * 2),
    # per-token FP8: 16 x D code bytes + 16 fp32 scales per (block, head), padded to 128
    # per-token FP8: the K run holds the codes and the token scales of K and V (2048 + 128
    # bytes at D = 128), the V run the codes only
    ("fp8t", 128, [10 * 3 * 2176, 10 * 3 * 2048] + [0] * 2),
    ("bf8t", 64, [10 * 3 * 1152, 10 * 3 * 1024] + [0] * 2),
])
def test_pool_layout_sizes(kv, d, expect):
    assert B.pa_pool_layout(kv, 10, 3, d) == expect


def test_pool_layout_rejects():
    lib = B.lib()
    out = (ctypes.c_size_t * 4)()
    assert lib.pa_pool_layout(9, 10, 1, 128, out) == DTYPE
    assert lib.pa_pool_layout(7, 10, 1, 128, out) == DTYPE
    assert lib.pa_pool_layout(0, 0, 1, 128, out) == SHAPE
    assert lib.pa_pool_layout(0, 10, 1, 96, out) == SHAPE
    assert lib.pa_pool_layout(3, 10, 1, 96, out) == SHAPE
    assert lib.pa_pool_layout(0, 10, 1, 128, None) == NULL
    assert lib.pa_outlier_capacity(128) == 11 and lib.pa_outlier_capacity(64) == 5
    assert lib.pa_outlier_capacity(80) == SHAPE


def _pool(dtype=2, nb=8, hkv=1, d=128, bs=16, scales=True, fp4=True, base=FAKE):
    s = B.pa_kv_pool()
    s.dtype, s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim = dtype, nb, bs, hkv, d
    s.k = s.v = base
    if scales:
        s.k_scale = s.v_scale = FAKE
    if fp4:
        s.k_out_val = s.v_out_val = FAKE
    return s


def _write(pool, act=1, T=4, k=FAKE, v=FAKE, slots=FAKE, err=None):
    p = None if pool is None else ctypes.byref(pool)
    return B.lib().pa_cache_write(p, k, v, act, T, slots, err, None)


def test_cache_write_rejects():
    assert _write(None) == NULL
    assert _write(_pool(bs=8)) == BLOCK
    assert _write(_pool(dtype=7)) == DTYPE
    assert _write(_pool(d=96)) == SHAPE
    assert _write(_pool(nb=0)) == SHAPE
    assert _write(_pool(dtype=3, d=96)) == SHAPE
    assert _write(_pool(dtype=0), act=1) == DTYPE      # fp16 pool, bf16 rows
    assert _write(_pool(dtype=1), act=0) == DTYPE      # bf16 pool, fp16 rows
    assert _write(_pool(), act=4) == DTYPE
    assert _write(_pool(), T=-1) == SHAPE
    assert _write(_pool(), k=None) == NULL
    assert _write(_pool(), slots=None) == NULL
    assert _write(_pool(scales=False)) == NULL         # fp8 without scales
    assert _write(_pool(dtype=3, fp4=False)) == NULL   # fp4 without its arrays
    assert _write(_pool(), k=FAKE + 8) == ALIGN
    assert _write(_pool(), slots=FAKE + 4) == ALIGN
    s = _pool()
    s.k = FAKE + 2
    assert _write(s) == ALIGN
    assert _write(_pool(), T=0) == PA_OK  # no rows: nothing to launch


def _decode(pool=None, q=FAKE, qd=1, S=2, Hq=8, bt=FAKE, MB=4, cl=FAKE, ps=0, out=FAKE,
            po=FAKE, pl=FAKE):
    pool = pool if pool is not None else _pool()
    return B.lib().pa_decode(q, qd, S, Hq, ctypes.byref(pool), bt, MB, cl, 0.1, ps, out, po, pl,
                             None, None)


def test_decode_rejects():
    assert _decode(pool=_pool(bs=32)) == BLOCK
    assert _decode(qd=3) == DTYPE
    assert _decode(pool=_pool(dtype=0), qd=1) == DTYPE
    assert _decode(pool=_pool(hkv=3), Hq=8) == SHAPE        # Hq % Hkv != 0
    assert _decode(pool=_pool(hkv=1), Hq=32) == SHAPE       # group of 32 > 16
    assert _decode(S=-1) == SHAPE
    assert _decode(Hq=0) == SHAPE
    assert _decode(MB=0) == CONTEXT
    assert _decode(MB=2 ** 28) == CONTEXT
    assert _decode(ps=24) == PART
    assert _decode(ps=-16) == PART
    assert _decode(q=None) == NULL
    assert _decode(bt=None) == NULL
    assert _decode(cl=None) == NULL
    assert _decode(out=None) == NULL
    assert _decode(ps=512, po=None) == NULL
    assert _decode(ps=512, pl=None) == NULL
    assert _decode(q=FAKE + 4) == ALIGN
    assert _decode(out=FAKE + 4) == ALIGN
    assert _decode(S=0) == PA_OK  # empty batch: nothing to launch


def test_append_decode_rejects():
    lib = B.lib()
    f = lambda pool=None, kn=FAKE, vn=FAKE, **k: lib.pa_append_decode(
        FAKE, 1, k.get("S", 2), 8, ctypes.byref(pool if pool is not None else _pool()), kn, vn,
        FAKE, 4, FAKE, 0.1, k.get("ps", 0), FAKE, FAKE, FAKE, None, None)
    assert f(pool=_pool(dtype=3, fp4=False)) == NULL  # FP4 without its outlier arrays
    assert f(kn=None) == NULL and f(vn=None) == NULL
    assert f(kn=FAKE + 8) == ALIGN
    assert f(ps=24) == PART
    assert f(pool=_pool(bs=8)) == BLOCK
    assert f(S=0) == PA_OK


def test_append_decode_n_rejects():
    lib = B.lib()
    f = lambda n, pool=None, S=2, MB=4: lib.pa_append_decode_n(
        FAKE, 1, S, 8, ctypes.byref(pool if pool is not None else _pool()), FAKE, FAKE, n,
        FAKE, MB, FAKE, 0.1, 0, FAKE, FAKE, FAKE, None, None, None)
    assert f(0) == SHAPE and f(-3) == SHAPE
    assert f(4 * 16 + 1) == SHAPE  # more new rows than the block table can hold
    assert f(2, pool=_pool(dtype=3)) == DTYPE  # FP4 pools take one new row per sequence
    assert f(8, S=0) == PA_OK


def _prefill(pool=None, q=FAKE, qd=1, S=2, Hq=8, T=10, qs=FAKE, mq=5, bt=FAKE, MB=4,
             cl=FAKE, out=FAKE, sc=0.1):
    pool = pool if pool is not None else _pool()
    return B.lib().pa_prefill(q, qd, S, Hq, T, qs, mq, ctypes.byref(pool), bt, MB, cl, sc, out,
                              None, None)


def test_prefill_rejects():
    assert _prefill(pool=_pool(bs=32)) == BLOCK
    assert _prefill(qd=3) == DTYPE
    assert _prefill(pool=_pool(dtype=0), qd=1) == DTYPE
    assert _prefill(pool=_pool(hkv=1), Hq=3) == SHAPE      # group 3 does not divide 16
    assert _prefill(pool=_pool(hkv=1), Hq=32) == SHAPE     # group 32 > 16
    assert _prefill(pool=_pool(hkv=3), Hq=8) == SHAPE      # Hq % Hkv != 0
    assert _prefill(S=-1) == SHAPE and _prefill(T=-1) == SHAPE and _prefill(mq=-1) == SHAPE
    assert _prefill(MB=0) == CONTEXT
    assert _prefill(q=None) == NULL and _prefill(qs=None) == NULL and _prefill(out=None) == NULL
    assert _prefill(bt=None) == NULL and _prefill(cl=None) == NULL
    assert _prefill(q=FAKE + 4) == ALIGN and _prefill(out=FAKE + 4) == ALIGN
    assert _prefill(S=0) == PA_OK  # nothing to launch


@pytest.mark.parametrize("sc", [0.0, -0.0, -0.125, float("nan"), float("inf"), float("-inf")])
def test_softmax_scale_must_be_positive_and_finite(sc):
    lib = B.lib()
    assert _prefill(sc=sc) == SCALE and _prefill(sc=sc, S=0) == SCALE
    dec = lambda S: lib.pa_decode(FAKE, 1, S, 8, ctypes.byref(_pool()), FAKE, 4, FAKE, sc, 0,
                                  FAKE, None, None, None, None)
    assert dec(2) == SCALE and dec(0) == SCALE
    assert lib.pa_append_decode_n(FAKE, 1, 2, 8, ctypes.byref(_pool()), FAKE, FAKE, 2, FAKE, 4,
                                  FAKE, sc, 0, FAKE, FAKE, FAKE, None, None, None) == SCALE
    # tiny and huge scales pass the check (and S = -1 then fails the next one)
    assert _prefill(sc=1e-30, S=-1) == SHAPE and _prefill(sc=3e38, S=-1) == SHAPE


def test_merge_and_scale_and_reset_reject():
    lib = B.lib()
    m = lambda **k: lib.pa_merge(k.get("po", FAKE), k.get("pl", FAKE), k.get("cl", FAKE),
                                 k.get("S", 2), k.get("Hq", 8), k.get("D", 128), k.get("P", 4),
                                 k.get("ps", 512), k.get("out", FAKE), None, None)
    assert m(ps=0) == PART and m(ps=100) == PART
    assert m(D=96) == SHAPE and m(P=0) == SHAPE and m(Hq=0) == SHAPE
    assert m(out=None) == NULL and m(po=None) == NULL
    assert m(po=FAKE + 4) == ALIGN
    assert m(S=0) == PA_OK
    f = lambda **k: lib.pa_fp8_head_scales(k.get("x", FAKE), k.get("act", 1), k.get("kv", 2),
                                           k.get("rows", 5), k.get("hkv", 1), k.get("d", 128),
                                           k.get("out", FAKE), None)
    assert f(act=2) == DTYPE and f(hkv=0) == SHAPE and f(d=32) == SHAPE and f(rows=-1) == SHAPE
    assert f(kv=1) == DTYPE and f(kv=3) == DTYPE and f(kv=5) == DTYPE
    assert f(out=None) == NULL and f(x=None) == NULL and f(x=FAKE + 2) == ALIGN
    p = _pool(dtype=3)
    assert lib.pa_reset_blocks(ctypes.byref(p), None, 3, None) == NULL
    assert lib.pa_reset_blocks(ctypes.byref(p), FAKE, -1, None) == SHAPE
    assert lib.pa_reset_blocks(ctypes.byref(_pool(dtype=2)), FAKE, 3, None) == PA_OK  # no records
    assert lib.pa_read_device_error(None, None, None) == NULL


def test_copy_blocks_rejects():
    """Every check of pa_copy_blocks runs before a launch. With no GPU here, no pointer is
    memory a GPU can access, so well-formed calls between two pools (their arrays at
    different addresses) stop at the memory check. A well-formed call within one pool
    would launch, so none is made here."""
    lib = B.lib()
    c = lambda a, b, pairs=FAKE, n=3, err=None: lib.pa_copy_blocks(
        None if a is None else ctypes.byref(a), None if b is None else ctypes.byref(b),
        pairs, n, err, None)
    a = _pool(nb=8)
    assert c(None, a) == NULL and c(a, None) == NULL
    assert c(a, _pool(dtype=4)) == DTYPE                 # E4M3 -> E5M2
    assert c(a, _pool(hkv=2)) == SHAPE and c(a, _pool(d=64)) == SHAPE
    assert c(a, _pool(bs=32)) == BLOCK
    assert c(a, a, n=-1) == SHAPE
    assert c(a, a, n=0) == PA_OK                         # nothing to copy
    assert c(a, a, pairs=None) == NULL
    assert c(a, a, pairs=FAKE + 4) == ALIGN and c(a, a, err=FAKE + 2) == ALIGN
    s = _pool(dtype=3)
    s.k_out_val = FAKE + 8                               # outlier slots need 16 bytes here
    assert c(s, _pool(dtype=3)) == ALIGN
    assert c(_pool(dtype=3, fp4=False), _pool(dtype=3)) == NULL
    other = FAKE + (1 << 30)
    assert c(_pool(scales=False), _pool(nb=4, scales=False, base=other)) == MEMORY  # no scales
    for kv in range(7):
        assert c(_pool(dtype=kv), _pool(dtype=kv, nb=3, base=other)) == MEMORY


def test_fp4_sequence_calls_reject():
    lib = B.lib()
    f = lambda **k: lib.pa_fp4_sequence_outliers(
        k.get("k", FAKE), k.get("v", FAKE), k.get("act", 1), k.get("rows", 10), k.get("hkv", 1),
        k.get("d", 128), k.get("rs", FAKE), k.get("S", 2), k.get("out", FAKE), k.get("err"), None)
    assert f(act=3) == DTYPE
    assert f(d=96) == SHAPE and f(rows=-1) == SHAPE and f(S=-1) == SHAPE and f(hkv=0) == SHAPE
    assert f(S=0) == PA_OK
    assert f(rs=None) == NULL and f(out=None) == NULL and f(k=None) == NULL
    assert f(out=FAKE + 4) == ALIGN and f(k=FAKE + 2) == ALIGN and f(err=FAKE + 1) == ALIGN
    w = lambda pool=None, **k: lib.pa_cache_write_seq_outliers(
        ctypes.byref(pool if pool is not None else _pool(dtype=3)), FAKE, FAKE, k.get("act", 1),
        k.get("T", 4), k.get("slots", FAKE), k.get("ts", FAKE), k.get("recs", FAKE),
        k.get("S", 2), None, None)
    assert w(pool=_pool(dtype=2)) == DTYPE  # FP4 pools only
    assert w(act=2) == DTYPE and w(T=-1) == SHAPE and w(S=-1) == SHAPE
    assert w(T=0) == PA_OK
    assert w(ts=None) == NULL and w(recs=None) == NULL and w(slots=None) == NULL
    assert w(recs=FAKE + 4) == ALIGN and w(ts=FAKE + 2) == ALIGN
    assert w(pool=_pool(dtype=3, fp4=False)) == NULL


def _opts(waves=0, tiles=0, reserved=0):
    o = B.pa_launch_options()
    o.decode_waves, o.prefill_col_tiles = waves, tiles
    o.reserved[5] = reserved
    return ctypes.byref(o)


@pytest.mark.parametrize("opts,expect", [
    (dict(waves=3), SHAPE), (dict(waves=16), SHAPE), (dict(waves=-1), SHAPE),
    (dict(tiles=1), SHAPE), (dict(tiles=4), SHAPE), (dict(reserved=1), SHAPE),
])
def test_launch_options_reject(opts, expect):
    """The _ex entry points check their launch options before anything else is launched;
    valid options on an empty batch launch nothing."""
    lib = B.lib()
    pool = ctypes.byref(_pool())
    d = lambda o, S=2: lib.pa_decode_ex(FAKE, 1, S, 8, pool, FAKE, 4, FAKE, 0.1, 0, FAKE, FAKE,
                                        FAKE, None, o, None)
    a = lambda o, S=2: lib.pa_append_decode_ex(FAKE, 1, S, 8, pool, FAKE, FAKE, FAKE, 4, FAKE,
                                               0.1, 0, FAKE, FAKE, FAKE, None, o, None)
    p = lambda o, S=2: lib.pa_prefill_ex(FAKE, 1, S, 8, 10, FAKE, 5, pool, FAKE, 4, FAKE, 0.1,
                                         FAKE, None, o, None)
    g = lambda o, S=2: lib.pa_gather_probe(S, 8, pool, FAKE, 4, FAKE, 0, FAKE, None, o, None)
    for fn in (d, a, p, g):
        assert fn(_opts(**opts)) == expect
        assert fn(_opts(waves=8, tiles=2), S=0) == PA_OK
        assert fn(None, S=0) == PA_OK


def test_gather_probe_rejects():
    lib = B.lib()
    f = lambda pool=None, **k: lib.pa_gather_probe(
        k.get("S", 2), k.get("Hq", 8), ctypes.byref(pool if pool is not None else _pool()),
        k.get("bt", FAKE), k.get("MB", 4), k.get("cl", FAKE), k.get("ps", 0),
        k.get("sink", FAKE), k.get("err"), None, None)
    assert f(pool=_pool(bs=8)) == BLOCK and f(pool=_pool(dtype=9)) == DTYPE
    assert f(pool=_pool(hkv=3)) == SHAPE and f(S=-1) == SHAPE and f(Hq=0) == SHAPE
    assert f(MB=0) == CONTEXT and f(ps=24) == PART
    assert f(bt=None) == NULL and f(cl=None) == NULL and f(sink=None) == NULL
    assert f(sink=FAKE + 2) == ALIGN and f(err=FAKE + 1) == ALIGN
    assert f(S=0) == PA_OK


def test_static_scratch_decode_rejects():
    """pa_decode_split_static checks its sizes against the static scratch, and the merge's
    output, before anything is queued."""
    lib = B.lib()
    f = lambda pool=None, **k: lib.pa_decode_split_static(
        FAKE, 1, k.get("S", 2), k.get("Hq", 8),
        None if pool == "null" else ctypes.byref(pool if pool is not None else _pool()),
        FAKE, k.get("MB", 4), FAKE, 0.1, k.get("ps", 512), k.get("out", FAKE), k.get("lse"),
        None, None)
    assert f(pool="null") == NULL
    assert f(ps=0) == PART and f(ps=24) == PART
    assert f(MB=0) == CONTEXT and f(S=-1) == SHAPE and f(Hq=0) == SHAPE
    assert f(pool=_pool(d=96)) == SHAPE
    # 64 x 8 x 4096 partitions x 129 floats is about 1 GB, past the 32 MiB scratch
    assert f(S=64, MB=4096, ps=16) == SCRATCH
    assert f(S=0) == PA_OK
    assert f(out=None) == NULL and f(out=FAKE + 4) == ALIGN and f(lse=FAKE + 2) == ALIGN


def test_library_reads_no_environment_knob():
    """Launch geometry comes only from arguments: the library's text names no environment
    variable it would read."""
    data = open(B._LIB_PATH, "rb").read()
    assert b"getenv" not in data
    assert b"PA_DECODE_WAVES" not in data and b"PA_PREFILL_NCT" not in data


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libpa.so not found"):
        B.lib()
