"""Host-side mu auto-scaling policy (tensor_scaled_fp8_amd.mu.MuScaler).

The pages say only that mu is changed dynamically [FP8-LM reading note, O1,
Eq. 3]; the policy (lower mu by one power of two when the clipped fraction
exceeds a threshold, raise it after a window of clean steps, clamp to
[lo, hi]) is a reading, so its parity is unpinned; these tests fix its
behaviour."""
import pytest

from tensor_scaled_fp8_amd.mu import MuScaler


def test_lowers_on_saturation_and_resets_the_window():
    m = MuScaler(mu_log2=3, threshold=1e-3, window=4)
    assert m.update(0, 1000) == 3
    assert m.update(0, 1000) == 3
    assert m.update(2, 1000) == 2          # 2e-3 > 1e-3: lower, window restarts
    for _ in range(3):
        assert m.update(1, 1000) == 2      # 1e-3 is not above the threshold
    assert m.update(0, 1000) == 3          # fourth clean step in a row: raise


def test_clamps_and_empty_steps():
    m = MuScaler(mu_log2=0, threshold=0.0, window=1, lo=-2, hi=1)
    assert m.update(0, 10) == 1
    assert m.update(0, 10) == 1            # at hi
    assert m.update(1, 10) == 0
    assert m.update(5, 10) == -1
    assert m.update(5, 10) == -2
    assert m.update(5, 10) == -2           # at lo
    assert m.update(0, 0) == -1            # an empty step is clean


def test_rejects_bad_settings():
    with pytest.raises(ValueError):
        MuScaler(mu_log2=20)
    with pytest.raises(ValueError):
        MuScaler(window=0)
