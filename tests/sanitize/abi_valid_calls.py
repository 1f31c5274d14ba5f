"""Well-formed calls through every host check of the C ABI, for the sanitizer build whose
launchers are stand-ins returning PA_ERR_LAUNCH: each call must get that far (status -7)
with AddressSanitizer / UndefinedBehaviorSanitizer watching the validation code. Run only
against that build (tests/test_sanitizers.py); the real library would launch kernels on
these fake addresses."""
import ctypes

import pytest

B = pytest.importorskip("paged_quantized_kv_reshape_amd.binding")
LAUNCH = -7
FAKE = 0x7F0000000000


def _pool(dtype=2, nb=64, hkv=2, d=128):
    s = B.pa_kv_pool()
    s.dtype, s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim = dtype, nb, 16, hkv, d
    s.k = s.v = s.k_out_val = s.v_out_val = s.k_scale = s.v_scale = FAKE
    return ctypes.byref(s)


@pytest.mark.parametrize("dtype", range(7))
@pytest.mark.parametrize("d", [64, 128])
def test_valid_calls_reach_the_launchers(dtype, d):
    lib = B.lib()
    act = 0 if dtype == 0 else 1
    p = _pool(dtype, d=d)
    assert lib.pa_cache_write(p, FAKE, FAKE, act, 40, FAKE, FAKE, None) == LAUNCH
    for ps in (0, 64, 512):
        assert lib.pa_decode(FAKE, act, 3, 16, p, FAKE, 9, FAKE, 0.1, ps, FAKE, FAKE, FAKE,
                             FAKE, None) == LAUNCH
        assert lib.pa_append_decode(FAKE, act, 3, 16, p, FAKE, FAKE, FAKE, 9, FAKE, 0.1, ps,
                                    FAKE, FAKE, FAKE, FAKE, None) == LAUNCH
        assert lib.pa_gather_probe(3, 16, p, FAKE, 9, FAKE, ps, FAKE, FAKE, None,
                                   None) == LAUNCH
    for w in (1, 2, 4, 8):
        o = B.pa_launch_options()
        o.decode_waves = w
        assert lib.pa_decode_ex(FAKE, act, 3, 16, p, FAKE, 9, FAKE, 0.1, 0, FAKE, FAKE, FAKE,
                                FAKE, ctypes.byref(o), None) == LAUNCH
    assert lib.pa_prefill(FAKE, act, 3, 16, 30, FAKE, 10, p, FAKE, 9, FAKE, 0.1, FAKE, FAKE,
                          None) == LAUNCH
    assert lib.pa_merge(FAKE, FAKE, FAKE, 3, 16, d, 5, 64, FAKE, FAKE, None) == LAUNCH
    if dtype == 3:
        assert lib.pa_reset_blocks(p, FAKE, 5, None) == LAUNCH
        assert lib.pa_fp4_sequence_outliers(FAKE, FAKE, act, 100, 2, d, FAKE, 3, FAKE, FAKE,
                                            None) == LAUNCH
        assert lib.pa_cache_write_seq_outliers(p, FAKE, FAKE, act, 40, FAKE, FAKE, FAKE, 3,
                                               FAKE, None) == LAUNCH
    if dtype in (2, 4):
        assert lib.pa_fp8_head_scales(FAKE, act, dtype, 100, 2, d, FAKE, None) == LAUNCH
    # copy within one pool: no pointer lookup, straight to the launcher
    assert lib.pa_copy_blocks(p, p, FAKE, 4, FAKE, None) == LAUNCH
