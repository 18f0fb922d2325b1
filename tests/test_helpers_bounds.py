"""The carried multi-step bound of tests/helpers.py (StepBounds), on the CPU:
it grows with every step that touches a row, leaves other rows at 0, accepts
the oracle's own values and rejects a difference just past the bound."""
import numpy as np
import pytest

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import ABS, REL, StepBounds, abs_grad_sums


def _run(steps=3):
    rows = np.array([40, 7, 300], np.int64)
    D, B = 8, 50
    o = orc.Oracle(rows, D, seed=3)
    bounds = StepBounds(int(rows.sum()), D)
    touched = set()
    for s in range(steps):
        off, ids, grad = synth.random_small(10 + s, rows.size, D, B, rows, max_len=4)
        uniq, sums = abs_grad_sums(off, ids, B, rows, grad, False, D)
        assert bounds.step(o, uniq, sums, 0.05, 1e-6,
                           lambda: o.backward_adagrad(off, ids, B, False, grad, 0.05, 1e-6)) == 0
        touched |= set(uniq.tolist())
    return o, bounds, rows, np.array(sorted(touched))


def test_bounds_grow_and_untouched_rows_stay_zero():
    o, bounds, rows, touched = _run()
    eW, eG = bounds.bounds_of(touched)
    assert (eW >= ABS).all() and (eG >= ABS).all()
    untouched = np.setdiff1d(np.arange(int(rows.sum())), touched)
    eWu, eGu = bounds.bounds_of(untouched)
    assert not eWu.any() and not eGu.any()
    # a row touched by every step carries at least one step's floor per step
    assert eG.max() >= 3 * ABS


def test_check_accepts_oracle_values_and_rejects_past_the_bound():
    o, bounds, rows, touched = _run()
    W, G = o.read_rows(touched)
    bounds.check(W, G, W, G, touched, "identical")
    eW, eG = bounds.bounds_of(touched)
    bad = W.astype(np.float64).copy()
    bad[0, 0] += 1.5 * eW[0, 0]
    with pytest.raises(AssertionError):
        bounds.check(bad, G, W, G, touched, "perturbed")
    inside = W.astype(np.float64).copy()
    inside[0, 0] += 0.5 * eW[0, 0]
    bounds.check(inside, G, W, G, touched, "inside")


def test_assigned_rows_restart_at_the_new_row_bound():
    o, bounds, rows, touched = _run()
    r = touched[:3]
    bounds.assigned(o, r)
    eW, eG = bounds.bounds_of(r)
    W, _ = o.read_rows(r)
    np.testing.assert_allclose(eW, REL * np.abs(W.astype(np.float64)) + ABS)
    assert not eG.any()
