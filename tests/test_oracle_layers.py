"""Pins of the oracle's pixel path, LayerNorm, GELU and attention (CPU only).

  * normalisation: closed-form end points and the page's fused form;
  * patchify: a single lit pixel lands in exactly one token and one feature, the
    position the C,T,H,W flattening and T-major order put it;
  * LayerNorm: zero mean and mean square var/(var+eps) with the identity affine; affine
    terms applied after;
  * GELU: odd-part identity, GELU(0) = 0, agreement with math.erf element by element;
  * attention: rows of softmax sum to one, one key returns v, equal keys average V,
    brute-force enumeration on tiny grids.
"""
import json
import math
import os

import numpy as np
import pytest

import bruteforce
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_normalisation_end_points_and_fused_form():
    mean = GOLD["imagenet_stats"]["mean"]
    std = GOLD["imagenet_stats"]["std"]
    px = np.arange(256, dtype=np.uint8)
    u8 = np.stack([px, px, px], axis=-1).reshape(1, 16, 16, 3)
    X = oracle.normalize_frames(u8)  # [3, 1, 16, 16]
    for c in range(3):
        v = X[c].reshape(-1)
        assert abs(v[0] - (-mean[c] / std[c])) < 1e-15
        assert abs(v[255] - (1 - mean[c]) / std[c]) < 1e-15
        fused = (np.arange(256) - 255.0 * mean[c]) / (255.0 * std[c])
        np.testing.assert_allclose(v, fused, rtol=0, atol=1e-15)  # a few ulp
    assert abs(X[0].reshape(-1)[0] - (-2.1179039301310043)) < 1e-14  # -0.485/0.229


def test_patchify_single_pixel():
    T, H, W = 4, 48, 32
    gh, gw = H // 16, W // 16
    for (c, t, y, x) in [(0, 0, 0, 0), (2, 3, 47, 31), (1, 2, 17, 5), (0, 1, 31, 16)]:
        X = np.zeros((3, T, H, W))
        X[c, t, y, x] = 7.0
        p = oracle.patchify(X)
        assert p.shape == ((T // 2) * gh * gw, 1536)
        n = (t // 2) * gh * gw + (y // 16) * gw + x // 16
        f = c * 512 + (t % 2) * 256 + (y % 16) * 16 + x % 16
        nz = np.argwhere(p != 0)
        assert nz.tolist() == [[n, f]]


def test_patch_embed_single_pixel_through_linear():
    rng = np.random.default_rng(0)
    D = 8
    Wpe = rng.standard_normal((D, 1536))
    b = rng.standard_normal(D)
    X = np.zeros((3, 2, 32, 32)); X[1, 1, 20, 3] = 2.0
    x = oracle.linear(oracle.patchify(X), Wpe, b)
    n = 0 * 4 + 1 * 2 + 0
    for i in range(4):
        want = b + (2.0 * Wpe[:, 512 + 256 + 4 * 16 + 3] if i == n else 0)
        np.testing.assert_allclose(x[i], want, rtol=1e-15)


@pytest.mark.parametrize("D", [384, 768, 1024, 7])
def test_layer_norm_closed_form(D):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((20, D)) * 3 + 5
    eps = 1e-6
    y = oracle.layer_norm(x, np.ones(D), np.zeros(D), eps)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    var = x.var(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-13)
    g = rng.standard_normal(D); b = rng.standard_normal(D)
    np.testing.assert_allclose(oracle.layer_norm(x, g, b, eps), y * g + b, rtol=1e-13, atol=1e-13)
    # constant rows: variance 0 -> output = bias
    np.testing.assert_allclose(oracle.layer_norm(np.full((2, D), 3.0), g, b, eps), np.tile(b, (2, 1)))


def test_gelu_identities():
    z = np.linspace(-8, 8, 1001)
    g = oracle.gelu_erf(z)
    np.testing.assert_allclose(g - oracle.gelu_erf(-z), z, atol=1e-14)
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
    want = [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in z]
    np.testing.assert_allclose(g, want, rtol=1e-14, atol=1e-15)
    # tanh approximation differs: guards against the wrong GELU
    tanh = 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert np.max(np.abs(tanh - g)) > 1e-4


def _qkv(rng, N, D):
    return rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal((N, D))


def test_attention_invariants():
    rng = np.random.default_rng(7)
    N, D, H = 12, 128, 2
    q, k, v = _qkv(rng, N, D)
    pos = oracle.rope_positions(np.arange(N), 2, 3)
    o = oracle.attention(q, k, v, H, pos, pos, "tiled")
    # one key: output = v (for every query)
    o1 = oracle.attention(q, k[:1], v[:1], H, pos, pos[:1], "tiled")
    np.testing.assert_allclose(o1, np.tile(v[:1], (N, 1)), rtol=1e-14)
    # identical keys at identical positions: output = mean of V
    kk = np.tile(k[:1], (N, 1))
    pz = np.zeros((N, 3))
    o2 = oracle.attention(q, kk, v, H, pz, pz, "interleaved")
    np.testing.assert_allclose(o2, np.tile(v.mean(axis=0), (N, 1)), rtol=1e-12)
    # output rows are convex combinations of V rows (softmax rows sum to 1):
    # attention on v = constant vector c returns c
    c = np.tile(rng.standard_normal(D), (N, 1))
    np.testing.assert_allclose(oracle.attention(q, k, c, H, pos, pos, "tiled"), c, rtol=1e-13)
    # selected rows equal the full evaluation
    r = np.array([0, 5, 11])
    np.testing.assert_allclose(oracle.attention(q, k, v, H, pos, pos, "tiled", rows=r), o[r], rtol=1e-15)
    np.testing.assert_allclose(oracle.attention(q, k, v, H, pos, pos, "tiled", slab=5), o, rtol=1e-15)


@pytest.mark.parametrize("layout", ["tiled", "interleaved"])
@pytest.mark.parametrize("grid,heads,hd", [((1, 2, 2), 1, 64), ((2, 2, 2), 2, 32), ((2, 2, 3), 2, 16)])
def test_attention_brute_force(layout, grid, heads, hd):
    rng = np.random.default_rng(11)
    gt, gh, gw = grid
    N, D = gt * gh * gw, heads * hd
    q, k, v = _qkv(rng, N, D)
    pos = oracle.rope_positions(np.arange(N), gh, gw)
    o = oracle.attention(q, k, v, heads, pos, pos, layout)
    bpos = [bruteforce.positions(i, gh, gw, 0) for i in range(N)]
    ob = bruteforce.attention(q.tolist(), k.tolist(), v.tolist(), heads, bpos, layout, 10000.0)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
