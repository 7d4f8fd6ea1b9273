"""The parity checker's selection rule, on the CPU (no GPU): inside the 1e-4 margin a GPU selection may
differ from the oracle's only among experts whose oracle key is within the margin of the k-th key."""
import numpy as np
import pytest

from gpu_util import MARGIN, check_near_tie_selection


def _sel(keys, k):
    key = np.asarray(keys, dtype=np.float64)[None, :]
    order = sorted(range(key.shape[1]), key=lambda e: (-key[0, e], e))
    return dict(key=key, ids=np.array([order[:k]], dtype=np.int32))


def test_swap_inside_the_margin_is_accepted():
    # experts 2 and 3 tie within the margin at the k-th place: either may be chosen
    sel = _sel([0.9, 0.8, 0.5, 0.5 - MARGIN / 2, 0.1], k=3)
    check_near_tie_selection(sel, np.array([[0, 1, 2]]), 0, "t", 0)
    check_near_tie_selection(sel, np.array([[1, 3, 0]]), 0, "t", 0)


@pytest.mark.parametrize("gpu_ids", [
    [0, 1, 4],        # an expert far below the k-th key swapped in
    [0, 2, 3],        # a clear top expert (key 0.8) swapped out
    [0, 1, 1],        # a repeated id
    [0, 1, 5],        # an id out of range
])
def test_wrong_selection_for_a_near_tie_token_is_rejected(gpu_ids):
    sel = _sel([0.9, 0.8, 0.5, 0.5 - MARGIN / 2, 0.1], k=3)
    with pytest.raises(AssertionError):
        check_near_tie_selection(sel, np.array([gpu_ids]), 0, "t", 0)
