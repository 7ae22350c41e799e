"""Pins of the parity metrics (``oracle/metrics.py``), on which every gate rests.

Definitions ([Parity "Results -- image models"]): the per-token cosine between matching
rows of two token maps (rows = tokens, the last axis = features), summarised by its mean,
median and minimum; rel_max = max|a - b| / max|b| with b the reference; max_abs =
max|a - b|.  Each case below has a closed-form answer, and each would catch a plausible
slip: the cosine taken over the wrong axis, a missing normalisation, a sign lost in the
difference, or the reference's magnitude taken from the wrong operand.
"""
import math

import numpy as np

from oracle import metrics


def test_cosine_closed_forms():
    # orthogonal rows -> 0; a row against a positive multiple -> 1, a negative one -> -1
    a = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0], [3.0, -1.0, 2.0], [3.0, -1.0, 2.0]])
    b = np.array([[0.0, 5.0, 0.0], [0.0, 0.5, 0.0], [6.0, -2.0, 4.0], [-0.3, 0.1, -0.2]])
    c = metrics.per_token_cosine(a, b)
    assert np.allclose(c, [0.0, 1.0, 1.0, -1.0], atol=1e-15)
    # a known angle in a plane of a 5-dim space
    for th in (0.1, 0.7, 2.0, 3.0):
        u = np.array([[math.cos(th), math.sin(th), 0.0, 0.0, 0.0]]) * 3.0
        v = np.array([[1.0, 0.0, 0.0, 0.0, 0.0]]) * 0.25
        assert abs(metrics.per_token_cosine(u, v)[0] - math.cos(th)) < 1e-14


def test_cosine_is_per_row_over_the_last_axis():
    # rows: identical, orthogonal, opposite; the column-wise cosines are different numbers
    a = np.array([[1.0, 2.0], [1.0, 0.0], [0.0, 1.0]])
    b = np.array([[1.0, 2.0], [0.0, 1.0], [0.0, -1.0]])
    c = metrics.per_token_cosine(a, b)
    assert c.shape == (3,)
    assert np.allclose(c, [1.0, 0.0, -1.0], atol=1e-15)
    # leading axes are flattened into rows: [B, N, D] -> B*N cosines in row-major order
    A = np.random.default_rng(0).standard_normal((2, 3, 4))
    B = A.copy()
    B[1, 2] = -B[1, 2]
    B[0, 1] = 7.0 * B[0, 1]
    c = metrics.per_token_cosine(A, B)
    assert c.shape == (6,)
    assert np.allclose(c, [1, 1, 1, 1, 1, -1], atol=1e-14)


def test_cosine_summary():
    a = np.array([[1.0, 0.0], [1.0, 1.0], [1.0, 0.0], [0.0, 1.0]])
    b = np.array([[1.0, 0.0], [1.0, 0.0], [1.0, 1.0], [1.0, 0.0]])
    s = metrics.summary(a, b)
    r = 1.0 / math.sqrt(2.0)
    assert abs(s["cos_mean"] - (1.0 + r + r + 0.0) / 4) < 1e-15
    assert abs(s["cos_median"] - r) < 1e-15
    assert s["cos_min"] == 0.0 and s["worst_row"] == 3


def test_rel_max_and_max_abs_closed_forms():
    b = np.array([[1.0, -4.0, 2.0]])
    a = np.array([[1.0, -4.4, 2.1]])           # the largest difference is negative
    assert abs(metrics.max_abs(a, b) - 0.4) < 1e-15
    assert abs(metrics.rel_max(a, b) - 0.1) < 1e-15
    # the reference's magnitude comes from b, not a
    a2 = np.array([[1.0, -40.0, 2.0]])
    assert abs(metrics.rel_max(a2, b) - 36.0 / 4.0) < 1e-15
    assert abs(metrics.rel_max(b, a2) - 36.0 / 40.0) < 1e-15
    # sign-flipped differences of equal size count the same
    c = np.array([[1.0, -3.6, 2.0]])
    assert abs(metrics.rel_max(a, b) - metrics.rel_max(c, b)) < 1e-15
    assert metrics.rel_max(b, b) == 0.0 and metrics.max_abs(b, b) == 0.0
    s = metrics.summary(a, b)
    assert s["rel_max"] == metrics.rel_max(a, b) and s["max_abs"] == metrics.max_abs(a, b)
