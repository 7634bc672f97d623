"""The host-side parity checks themselves (CPU): the top-k tie allowance."""

import numpy as np
import pytest

from tests import parity


def _row():
    o = np.linspace(-1.0, 1.0, 200)
    o[150] = 0.2000
    o[151] = 0.2003          # 0.15 % above: outside the 1e-3 tie window
    return o


def test_topk_swap_outside_tie_window_fails_without_magnitude():
    o = _row()
    k = int(np.sum(o >= 0.2003))                 # 0.2003 is the k-th value
    ref = np.sort(np.argsort(o)[-k:])
    swapped = np.sort(np.concatenate([ref[ref != 151], [150]]))
    with pytest.raises(AssertionError):
        parity.check_topk_row(swapped, o, k, "swap")


def test_topk_swap_within_logits_tolerance_passes_with_magnitude():
    o = _row()
    k = int(np.sum(o >= 0.2003))
    ref = np.sort(np.argsort(o)[-k:])
    swapped = np.sort(np.concatenate([ref[ref != 151], [150]]))
    m = np.zeros_like(o)                          # relative term only
    assert parity.check_topk_row(swapped, o, k, "swap", m) == 1
    # a gap wider than both tolerances together still fails
    o2 = o.copy()
    o2[150] = 0.1980
    with pytest.raises(AssertionError):
        parity.check_topk_row(swapped, o2, k, "far", m)
