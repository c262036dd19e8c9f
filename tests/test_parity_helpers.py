"""CPU checks of the parity helpers the GPU tests rely on: the requantisation
comparison excuses a differing code only at a certified near-tie, only by one
grid step, and never a differing scale byte outside a near-tie block."""

import numpy as np
import pytest

from oracle import quantize as Q
from parity import assert_requant_matches, assert_close


def _h():
    # gs_h = 64; block 0 of row 0: amax 6/64 -> a_s 6, t 1, sd 1, r 64
    h = (np.random.default_rng(3).standard_normal((4, 2048)) * 0.03).astype(np.float32)
    h[0, 0:16] = 0
    h[0, 0] = 6.0 / 64
    h[0, 5] = 2.5 / 64          # v = 2.5 exactly: the tie of 2 and 3 (goes to 2)
    h[0, 6] = 1.0 / 64          # v = 1: far from any midpoint
    return h


def _gpu_like(h):
    codes, sf = Q.quantize_blocks(h, np.float32(64.0))
    return codes, sf


def test_identical_requant_passes_and_marks_no_row():
    h = _h()
    codes, sf = _gpu_like(h)
    rows = assert_requant_matches(Q.pack_codes(codes), sf, h, 64.0, "identical")
    assert not rows.any()


def test_one_step_at_a_certified_tie_is_excused_and_reported():
    h = _h()
    codes, sf = _gpu_like(h)
    assert codes[0, 5] == 4
    codes[0, 5] = 5
    rows = assert_requant_matches(Q.pack_codes(codes), sf, h, 64.0, "tie")
    assert rows.tolist() == [True, False, False, False]


@pytest.mark.parametrize("where,new", [((0, 6), 3), ((0, 5), 6), ((0, 5), 0xC)])
def test_difference_outside_a_tie_or_beyond_one_step_fails(where, new):
    h = _h()
    codes, sf = _gpu_like(h)
    codes[where] = new          # far element / two steps / sign flip
    with pytest.raises(AssertionError):
        assert_requant_matches(Q.pack_codes(codes), sf, h, 64.0, "bad")


def test_scale_byte_outside_a_tie_block_fails():
    h = _h()
    codes, sf = _gpu_like(h)
    sf[2, 1] ^= 1
    with pytest.raises(AssertionError):
        assert_requant_matches(Q.pack_codes(codes), sf, h, 64.0, "bad scale")


def test_floating_point_bar():
    ref = np.random.default_rng(4).standard_normal(1000)
    assert_close(ref * (1 + 1e-6), ref, "near")
    bad = ref.copy()
    bad[7] += 0.05 * np.sqrt(np.mean(ref ** 2))      # one element beyond 2e-2 * RMS
    with pytest.raises(AssertionError):
        assert_close(bad, ref, "one outlier")


def test_bf16_step_allowance():
    from parity import bf16_step
    assert bf16_step(np.array([1.0, 1.5, 4.0, 7.9, 0.3]) ).tolist() == \
        [2.0 ** -7, 2.0 ** -7, 2.0 ** -5, 2.0 ** -5, 2.0 ** -9]
    ref = np.random.default_rng(5).standard_normal(4000)
    ref[10] = 6.0                                     # above 5 * RMS: one step is 2^-5
    gpu = ref.copy()
    gpu[10] += 2.0 ** -5                              # one BF16 step apart
    with pytest.raises(AssertionError):
        assert_close(gpu, ref, "strict")
    assert_close(gpu, ref, "one step", bf16=True)
    gpu[10] += 2.0 ** -5                              # two steps: not excused
    with pytest.raises(AssertionError):
        assert_close(gpu, ref, "two steps", bf16=True)
    many = np.random.default_rng(6).standard_normal(4000)
    many[:20] = 6.0
    shifted = many.copy()
    shifted[:20] += 2.0 ** -5                         # 20 of 4000 one step apart (0.5%)
    with pytest.raises(AssertionError, match="elements above the bound"):
        assert_close(shifted, many, "many", bf16=True)
    shifted[2:20] = many[2:20]                        # 2 of 4000 (0.05%): excused
    assert_close(shifted, many, "few", bf16=True)
