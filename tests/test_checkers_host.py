"""The GPU parity checks' comparison helpers catch planted output mistakes
(host only: the mistakes are planted in copies of oracle outputs, never in a
kernel): a swapped head block, a payload row off by more than the bar, an
LSE off by more than its bound or with a changed -inf pattern, a nonzero
gradient where the oracle is exactly zero."""

import numpy as np
import pytest

import synth
from helpers import (OUT_ROW_RTOL, assert_bits_equal, assert_grad_lse_close, assert_lse_close, assert_rows_close,
                     grad_lse_scale)


def test_bits_check_catches_swapped_head_block(orc):
    P, B, S, H, D = 2, 1, 8, 4, 8
    x = synth.iota32(P * B * (S // P) * H * D).reshape(P, B, S // P, H, D)
    want = orc.seq_to_head(x, P, B, S, H, D)
    assert_bits_equal(want.copy(), want, "identical")
    bad = want.copy()
    bad[0, 0, 3], bad[1, 0, 3] = want[1, 0, 3], want[0, 0, 3]   # one token's head blocks of ranks 0 and 1 swapped
    with pytest.raises(AssertionError):
        assert_bits_equal(bad, want, "swapped head block")


def test_row_check_bar_and_zero_rows():
    rng = np.random.default_rng(1)
    want = rng.normal(size=(16, 64))
    want[5] = 0.0
    got = want.copy()
    assert_rows_close(got, want, "identical")
    got[3, 7] += 0.5 * OUT_ROW_RTOL * np.max(np.abs(want[3]))       # inside the bar
    assert_rows_close(got, want, "inside the bar")
    got[3, 7] += 2.0 * OUT_ROW_RTOL * np.max(np.abs(want[3]))       # beyond it
    with pytest.raises(AssertionError):
        assert_rows_close(got, want, "beyond the bar")
    got = want.copy()
    got[5, 0] = 1e-30                                                # a row that must be exactly zero
    with pytest.raises(AssertionError):
        assert_rows_close(got, want, "nonzero zero row")
    got = want.copy()
    got[2, 2] = np.nan
    with pytest.raises(AssertionError):
        assert_rows_close(got, want, "NaN")


def test_lse_check_bound_and_neg_inf_pattern():
    want = np.array([0.5, -np.inf, 3.25, -1.0], dtype=np.float32)
    assert_lse_close(want + np.float32(5e-6) * (want > -np.inf), want, "inside 1e-5")
    with pytest.raises(AssertionError):
        assert_lse_close(want + np.float32(2e-5) * (want > -np.inf), want, "beyond 1e-5")
    bad = want.copy()
    bad[1] = -80.0                                                   # -inf turned finite
    with pytest.raises(AssertionError):
        assert_lse_close(bad, want, "-inf pattern")
    bad = want.copy()
    bad[0] = -np.inf                                                 # finite turned -inf
    with pytest.raises(AssertionError):
        assert_lse_close(bad, want, "-inf pattern")


def test_grad_lse_check_zeros_and_scale():
    rng = np.random.default_rng(2)
    P, R, D = 3, 5, 8
    po, go = rng.normal(size=(P, R, D)), rng.normal(size=(R, D))
    scale = grad_lse_scale(po, go, None)
    want = rng.normal(size=(P, R)).astype(np.float32)
    want[1, 2] = 0.0                                                 # an invalid partial: exactly zero
    assert_grad_lse_close(want.copy(), want, scale, "identical")
    bad = want.copy()
    bad[1, 2] = np.float32(1e-30)
    with pytest.raises(AssertionError):
        assert_grad_lse_close(bad, want, scale, "nonzero where zero")
    bad = want.copy()
    bad[0, 0] += np.float32(1e-3 * scale[0])
    with pytest.raises(AssertionError):
        assert_grad_lse_close(bad, want, scale, "beyond the bound")
