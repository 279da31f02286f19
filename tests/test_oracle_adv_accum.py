"""Pins of the oracle's group advantage (closed forms, library std) and of the
step accumulator (roll-up, deferred divisor, poisoned-window countdown)."""

import math

import numpy as np
import pytest

import oracle
from oracle import ACC_NONFINITE, ACC_OK, ACC_SKIPPED


# ---------------------------------------------------------------- advantage

def test_advantage_closed_form():
    # rewards [1,0,0,0]: mean 0.25, unbiased std sqrt(0.75/3) = 0.5
    A = oracle.group_advantage([1, 0, 0, 0], 4)
    want = np.array([0.75, -0.25, -0.25, -0.25]) / (0.5 + 1e-6)
    assert np.allclose(A, want, rtol=1e-15, atol=0)


def test_advantage_degenerate_groups():
    assert not oracle.group_advantage([1, 1, 1, 1, 0, 0, 0, 0], 4).any()   # all-equal groups
    assert not oracle.group_advantage([0.3, 0.9, 0.1], 1).any()            # groups of one
    A = oracle.group_advantage([1, 0, 0, 0], 4, norm_by_std=False)
    assert np.allclose(A, [0.75, -0.25, -0.25, -0.25], rtol=0, atol=1e-16)


def test_advantage_matches_library_std_and_sums_to_zero():
    rng = np.random.default_rng(2)
    r = rng.normal(size=48)
    for G in (2, 4, 8, 16):
        A = oracle.group_advantage(r, G)
        g = r.reshape(-1, G)
        want = (g - g.mean(axis=1, keepdims=True)) / (g.std(axis=1, ddof=1, keepdims=True) + 1e-6)
        assert np.allclose(A, want.reshape(-1), rtol=1e-12, atol=1e-14)
        assert np.allclose(A.reshape(-1, G).sum(axis=1), 0.0, atol=1e-12)


def test_advantage_rejects_partial_group():
    with pytest.raises(ValueError):
        oracle.group_advantage([1, 0, 1], 2)


def test_rows_advantage_copies_and_zeroes_pads():
    # [P4] compaction example: 6 rollouts, 16 rows, 3 pads.
    p = oracle.plan_compaction([1, 3, 2, 5, 1, 1], 3, 2, 4, 6)
    A = np.array([1.0, -1.0, 0.5, -0.5, 2.0, -2.0])
    rows = oracle.rows_advantage(A, p["row_rollout"])
    for i, (r, pad) in enumerate(zip(p["row_rollout"], p["is_pad"])):
        assert rows[i] == (0.0 if pad else A[r])


# ---------------------------------------------------------------- accumulator

def _st(loss_sum, n_valid, nonfinite=0, ent=0.0, clipped=0, rows=1):
    return {"loss_sum": loss_sum, "entropy_sum": ent, "n_valid": n_valid,
            "n_clipped": clipped, "n_nonfinite": nonfinite, "n_valid_rows": rows}


def test_window_rollup_and_grad_scale():
    acc = oracle.Accumulator(2)
    assert acc.add(_st(6.0, 30, ent=3.0, clipped=2, rows=3)) == ACC_OK
    assert acc.finalize() is None                      # window not complete
    assert acc.add(_st(-1.5, 3, ent=0.3, clipped=1, rows=1)) == ACC_OK
    f = acc.finalize()
    assert f["loss"] == pytest.approx(4.5 / 33)
    assert f["n_valid"] == 33 and f["n_clipped"] == 3 and f["n_valid_rows"] == 4
    assert f["grad_scale"] == pytest.approx(1 / 33)
    assert f["entropy"] == pytest.approx(3.3 / 33)
    assert acc.finalize() is None


def test_empty_step_guard():
    acc = oracle.Accumulator(3)
    for _ in range(3):
        assert acc.add(_st(0.0, 0, rows=0)) == ACC_OK
    f = acc.finalize()
    assert f["loss"] == 0.0 and f["grad_scale"] == 1.0 and math.isfinite(f["loss"])


@pytest.mark.parametrize("n_micro,j", [(4, 0), (4, 1), (4, 3), (1, 0), (2, 1)])
def test_poisoned_window_countdown(n_micro, j):
    # [P1] a non-finite chunk at position j discards the window and swallows
    # exactly n_micro - 1 - j calls; the next window starts clean.
    acc = oracle.Accumulator(n_micro)
    for _ in range(j):
        assert acc.add(_st(100.0, 10)) == ACC_OK
    assert acc.add(_st(float("nan"), 10)) == ACC_NONFINITE
    for _ in range(n_micro - 1 - j):
        assert acc.add(_st(5.0, 10)) == ACC_SKIPPED
    assert acc.finalize() is None
    for k in range(n_micro):
        assert acc.add(_st(1.0 + k, 2)) == ACC_OK
    f = acc.finalize()
    assert f["n_valid"] == 2 * n_micro                       # divisor was reset
    assert f["loss"] == pytest.approx(sum(1.0 + k for k in range(n_micro)) / (2 * n_micro))


def test_nonfinite_by_count_flag():
    acc = oracle.Accumulator(2)
    assert acc.add(_st(1.0, 4, nonfinite=1)) == ACC_NONFINITE
    assert acc.add(_st(1.0, 4)) == ACC_SKIPPED
    assert acc.add(_st(1.0, 4)) == ACC_OK


def test_add_after_complete_window_needs_finalize():
    acc = oracle.Accumulator(1)
    assert acc.add(_st(1.0, 1)) == ACC_OK
    assert acc.add(_st(1.0, 1)) == "STATE"
    assert acc.finalize() is not None
    assert acc.add(_st(1.0, 1)) == ACC_OK
