"""Pins of the oracle's token positions and 3-D RoPE (CPU only).

What fixes each piece, besides the oracle itself:
  * printed values of [Notes §1]/[Notes §4]/[Notes §4.3] stored in
    tests/golden/pages_printed_values.json (split sizes, the tiled and interleaved pair ->
    frequency maps, interpolation factors, token counts);
  * closed forms: the frequencies in the page's other spelling, identity at position 0,
    the tiled pair matrix and its determinant cos(a - b);
  * textbook rotation invariants for the interleaved layout (norm per pair, relative
    position, composition);
  * the permutation that maps the interleaved angle table onto the tiled one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_split_sizes_match_pages():
    for c in GOLD["rope_split"]["cases"]:
        d = oracle.rope_axis_dim(c["head_dim"])
        assert d == c["d"]
        assert 3 * d == c["rotated"]
        assert c["head_dim"] - 3 * d == c["pass_through"]


@pytest.mark.parametrize("d", [20, 10, 4])
def test_frequencies_other_spelling(d):
    # [Notes §4]: theta ** (-(2k)/d), written with Python's float power per k
    th = GOLD["frequency_table_spellings"]["theta"]
    om = oracle.rope_omegas(d, th)
    want = [th ** (-(2 * k) / d) for k in range(d // 2)]
    np.testing.assert_allclose(om, want, rtol=1e-15)
    assert om[0] == 1.0
    if d == 20:
        # omega_5 = 10000**(-1/2) = 1/100 exactly in real arithmetic
        assert abs(om[5] - 0.01) < 1e-17
    # omega_k * omega_{m-k} = 1/theta for the geometric table
    m = d // 2
    for k in range(1, m):
        assert abs(om[k] * (th ** (-(2 * (m - k)) / d)) - 1.0 / th) < 1e-18


def _pair_freqs(layout, d, pos=1.0):
    """Read back, from the oracle's rotation, which frequency drives each element of
    every pair: rotating e_{2k} (resp. e_{2k+1}) at position pos puts cos(angle) in
    place and +/- sin(angle) in the partner."""
    hd = 3 * d
    om = oracle.rope_omegas(d)
    P = np.array([[pos, 0.0, 0.0]])
    out = []
    for k in range(d // 2):
        e0 = np.zeros((1, hd)); e0[0, 2 * k] = 1.0
        e1 = np.zeros((1, hd)); e1[0, 2 * k + 1] = 1.0
        r0 = oracle.rope_rotate(e0, P, layout)[0]
        r1 = oracle.rope_rotate(e1, P, layout)[0]
        # even element: out[2k] = x[2k] cos a - x[2k+1] sin a  -> from e1: -sin a at 2k
        a_even = math.atan2(-r1[2 * k], r0[2 * k])
        # odd element: out[2k+1] = x[2k+1] cos b + x[2k] sin b -> from e0: sin b at 2k+1
        a_odd = math.atan2(r0[2 * k + 1], r1[2 * k + 1])
        fe = int(np.argmin(np.abs(om * pos - a_even)))
        fo = int(np.argmin(np.abs(om * pos - a_odd)))
        assert abs(om[fe] * pos - a_even) < 1e-12 and abs(om[fo] * pos - a_odd) < 1e-12
        out.append([fe, fo])
    return out


def test_tiled_pair_map_matches_worked_example():
    assert _pair_freqs("tiled", 20) == GOLD["tiled_d20_pair_frequencies"]["pairs"]


def test_interleaved_pair_map_matches_page():
    assert _pair_freqs("interleaved", 20) == GOLD["interleaved_d20_pair_frequencies"]["pairs"]


@pytest.mark.parametrize("hd", [64, 32])
@pytest.mark.parametrize("layout", ["tiled", "interleaved"])
def test_position_zero_identity_and_pass_through(hd, layout):
    rng = np.random.default_rng(1)
    u = rng.standard_normal((5, 7, hd))
    pos = np.zeros((7, 3))
    np.testing.assert_array_equal(oracle.rope_rotate(u, pos, layout), u)
    pos = rng.uniform(0, 31, size=(7, 3))
    y = oracle.rope_rotate(u, pos, layout)
    r = 3 * oracle.rope_axis_dim(hd)
    np.testing.assert_array_equal(y[..., r:], u[..., r:])  # bit-identical pass-through
    assert not np.allclose(y[..., :r], u[..., :r])


def test_axis_segments_use_their_own_coordinate():
    # dims [0,d) follow t, [d,2d) follow h, [2d,3d) follow w ([Notes §4])
    hd, d = 64, 20
    u = np.random.default_rng(2).standard_normal((1, hd))
    for a in range(3):
        pos = np.zeros((1, 3)); pos[0, a] = 3.0
        y = oracle.rope_rotate(u, pos, "tiled")
        changed = np.nonzero(np.abs(y - u)[0] > 0)[0]
        assert changed.min() >= a * d and changed.max() < (a + 1) * d


def test_interleaved_is_a_rotation():
    rng = np.random.default_rng(3)
    hd = 64
    u = rng.standard_normal((50, hd))
    pos = rng.uniform(0, 31, size=(50, 3))
    y = oracle.rope_rotate(u, pos, "interleaved")
    # each pair keeps its norm
    np.testing.assert_allclose(y[:, 0::2] ** 2 + y[:, 1::2] ** 2,
                               u[:, 0::2] ** 2 + u[:, 1::2] ** 2, rtol=1e-12)
    # relative position: <R(p) q, R(p') k> depends only on p - p'
    q = rng.standard_normal((1, hd)); k = rng.standard_normal((1, hd))
    p1, p2 = np.array([[3.0, 5.0, 7.0]]), np.array([[1.0, 2.0, 11.0]])
    for shift in ([0, 0, 0], [4, -2, 9], [0.5, 1.25, -3.0]):
        s = np.array([shift], dtype=float)
        a = oracle.rope_rotate(q, p1 + s, "interleaved") @ oracle.rope_rotate(k, p2 + s, "interleaved").T
        b = oracle.rope_rotate(q, p1, "interleaved") @ oracle.rope_rotate(k, p2, "interleaved").T
        assert abs(a[0, 0] - b[0, 0]) < 1e-12
    # composition R(p) R(p') = R(p + p')
    a = oracle.rope_rotate(oracle.rope_rotate(q, p1, "interleaved"), p2, "interleaved")
    b = oracle.rope_rotate(q, p1 + p2, "interleaved")
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_tiled_pair_matrix_and_determinant():
    # [Notes §4.1]: out[2k] = x[2k] cos a - x[2k+1] sin a, out[2k+1] = x[2k+1] cos b + x[2k] sin b
    # so the pair matrix is [[cos a, -sin a], [sin b, cos b]] with det = cos(a - b):
    # not orthogonal once a != b.
    d, hd = 20, 64
    om = oracle.rope_omegas(d)
    p = 2.5
    pos = np.array([[p, 0.0, 0.0]])
    for k, (fe, fo) in enumerate(GOLD["tiled_d20_pair_frequencies"]["pairs"]):
        a, b = p * om[fe], p * om[fo]
        e0 = np.zeros((1, hd)); e0[0, 2 * k] = 1
        e1 = np.zeros((1, hd)); e1[0, 2 * k + 1] = 1
        c0 = oracle.rope_rotate(e0, pos, "tiled")[0, 2 * k:2 * k + 2]
        c1 = oracle.rope_rotate(e1, pos, "tiled")[0, 2 * k:2 * k + 2]
        M = np.stack([c0, c1], axis=1)
        np.testing.assert_allclose(M, [[math.cos(a), -math.sin(a)], [math.sin(b), math.cos(b)]], atol=1e-15)
        assert abs(np.linalg.det(M) - math.cos(a - b)) < 1e-14
    # the pair norm is not preserved at p != 0 (negative check)
    u = np.random.default_rng(4).standard_normal((1, hd))
    y = oracle.rope_rotate(u, np.array([[3.0, 2.0, 1.0]]), "tiled")
    assert not np.allclose(y[:, 0:60:2] ** 2 + y[:, 1:60:2] ** 2, u[:, 0:60:2] ** 2 + u[:, 1:60:2] ** 2)


@pytest.mark.parametrize("hd", [64, 32])
def test_layouts_agree_up_to_angle_permutation(hd):
    # tiled angle of dim j equals the interleaved angle of dim pi(j) = 2*(j mod m) + j // m
    d = oracle.rope_axis_dim(hd)
    m = d // 2
    pi = np.array([2 * (j % m) + j // m for j in range(d)])
    assert sorted(pi.tolist()) == list(range(d))  # a bijection
    rng = np.random.default_rng(5)
    pos = rng.uniform(0, 31, size=(9, 3))
    ang_i = oracle.rope_angles(pos, hd, "interleaved")
    perm = np.concatenate([a * d + pi for a in range(3)])
    u = rng.standard_normal((2, 9, hd))
    a = oracle.rope_rotate(u, pos, "tiled")
    b = oracle.rope_rotate_with_angles(u, ang_i[:, perm])
    np.testing.assert_array_equal(a, b)


def test_interpolation_values():
    g = GOLD["interpolation"]
    R = g["ref_grid"]
    for c in g["cases"]:
        n = c["grid_side"]
        ids = np.arange(2 * n * n)  # two temporal slots on an n x n grid
        pos = oracle.rope_positions(ids, n, n, R)
        t, h, w = oracle.id_to_thw(ids, n, n)
        np.testing.assert_array_equal(pos[:, 0], t)  # time not rescaled
        np.testing.assert_allclose(pos[:, 1], h * c["num"] / c["den"], rtol=1e-15)
        np.testing.assert_allclose(pos[:, 2], w * c["num"] / c["den"], rtol=1e-15)
        assert pos[:, 1].max() == g["last_lands_on"] and pos[:, 2].max() == g["last_lands_on"]
    with pytest.raises(ValueError):
        oracle.rope_positions(np.arange(4), 1, 4, R)


def test_id_decode_roundtrip_and_counts():
    for c in GOLD["token_counts"]["cases"]:
        gt, gh, gw = c["frames"] // 2, c["size"] // 16, c["size"] // 16
        assert [gt, gh, gw] == c["grid"] and gt * gh * gw == c["N"]
    gt, gh, gw = 8, 16, 16
    ids = np.arange(gt * gh * gw)
    t, h, w = oracle.id_to_thw(ids, gh, gw)
    assert (t * gh * gw + h * gw + w == ids).all()
    assert t.max() == gt - 1 and h.max() == gh - 1 and w.max() == gw - 1
    # a few by hand: T-major, then H, then W
    assert tuple(int(a[300]) for a in (t, h, w)) == (1, 2, 12)
    assert tuple(int(a[255]) for a in (t, h, w)) == (0, 15, 15)
    # non-square grid (actual grid, [Notes §4]: non-square works)
    t, h, w = oracle.id_to_thw(np.array([37]), 16, 20)
    assert (int(t[0]), int(h[0]), int(w[0])) == (0, 1, 17)
