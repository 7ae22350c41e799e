"""Pins of the oracle's block-causal attention with a CLS row ([Parity] "LeVJEPA ViT-L/16 —
CLS, block-causal attention, tubelet 1") (CPU only).

  * printed values: 1 + 16*14*14 = 3137 rows and a visible fraction of 53.1 % of the grid
    (tests/golden/pages_printed_values.json, "block_causal_levjepa");
  * structure: the CLS row is all open, the CLS column open only to CLS rows, rows of
    one slot share their visibility, a patch row sees exactly the patch keys of its slot
    and the earlier ones;
  * brute force: the element-by-element attention with the same visibility, to ~1e-12;
  * causality: the outputs of slot-0 queries do not move when later tokens change, and
    no patch output moves when the CLS key/value changes; the CLS row does move;
  * one slot holding every token and no CLS row gives plain attention.
"""
import json
import os

import numpy as np

import bruteforce
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_levjepa_rows_and_density():
    g = GOLD["block_causal_levjepa"]
    N = 1 + g["frames"] * g["side_patches"] ** 2
    assert N == g["rows"]
    vis = oracle.block_causal_mask(N, 1, g["side_patches"] ** 2)
    assert round(100.0 * vis.mean(), 1) == g["visible_pct"]


def test_mask_structure():
    slot = 4
    vis = oracle.block_causal_mask(1 + 3 * slot, 1, slot)
    assert vis[0].all()
    assert vis[:, 0].sum() == 1 and vis[0, 0]
    for r in range(1, 13):
        t = (r - 1) // slot
        expect = np.zeros(13, bool)
        expect[1:1 + (t + 1) * slot] = True
        np.testing.assert_array_equal(vis[r], expect)


def _qkv(N, D, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((N, D)), g.standard_normal((N, D)), g.standard_normal((N, D))


def test_masked_attention_brute_force():
    N, slot = 1 + 2 * 3, 3
    q, k, v = _qkv(N, 32, 1)
    pos = oracle.rope_positions(np.r_[0, np.arange(N - 1)], 2, 3)
    vis = oracle.block_causal_mask(N, 1, slot)
    a = oracle.attention(q, k, v, 2, pos, pos, "interleaved", visible=vis)
    def sees(i, n):          # the pages' wording: CLS row open, CLS column closed, slots causal
        return i == 0 or (n >= 1 and (n - 1) // slot <= (i - 1) // slot)
    b = np.array(bruteforce.attention(q.tolist(), k.tolist(), v.tolist(), 2, [tuple(p) for p in pos],
                                      "interleaved", 10000.0, visible=sees))
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_causality():
    N, slot = 1 + 3 * 4, 4
    q, k, v = _qkv(N, 32, 2)
    pos = np.zeros((N, 3))
    vis = oracle.block_causal_mask(N, 1, slot)
    base = oracle.attention(q, k, v, 2, pos, pos, "tiled", visible=vis)
    k2, v2 = k.copy(), v.copy()
    k2[1 + slot:] += 1.0; v2[1 + slot:] -= 2.0                 # slots 1 and 2 change
    moved = oracle.attention(q, k2, v2, 2, pos, pos, "tiled", visible=vis)
    np.testing.assert_array_equal(moved[1:1 + slot], base[1:1 + slot])
    assert np.abs(moved[1 + slot:] - base[1 + slot:]).max() > 1e-3
    k3, v3 = k.copy(), v.copy()
    k3[0] += 3.0; v3[0] += 3.0                                  # the CLS key/value changes
    c = oracle.attention(q, k3, v3, 2, pos, pos, "tiled", visible=vis)
    np.testing.assert_array_equal(c[1:], base[1:])
    assert np.abs(c[0] - base[0]).max() > 1e-3


def test_one_slot_no_cls_is_plain_attention():
    N = 10
    q, k, v = _qkv(N, 32, 3)
    pos = oracle.rope_positions(np.arange(N), 2, 5)
    a = oracle.attention(q, k, v, 2, pos, pos, "tiled", visible=oracle.block_causal_mask(N, 0, N))
    np.testing.assert_array_equal(a, oracle.attention(q, k, v, 2, pos, pos, "tiled"))
