"""Pins of the oracle's pooled outputs (CPU only): the mean pool ([Card] "Run it",
``--pool mean``) and the attentive-pool classifier head ([Notes §2] "Attentive-pool head —
exact forward").

  * mean pool: a token map of identical rows pools to that row; the mean of the rows
    equals the closed form (sum / N) on integers;
  * head: the brute-force element-by-element head (tests/bruteforce.py) to ~1e-12, with
    and without pool blocks;
  * invariants: the logits do not change when the tokens are permuted (pool blocks
    without RoPE are permutation-equivariant, the single-query cross-attention pools
    over all tokens), and with one token the cross-attention returns that token's value
    row, so the head reduces to a plain MLP on q0 + v;
  * negative controls: giving the pool blocks RoPE positions, or adding an output
    projection to the cross-attention, moves the logits.
"""
import numpy as np

import bruteforce
import oracle
import synth
from oracle import metrics


def weights(n_layer=1, seed=0):
    s = synth.HeadShape(32, n_layer, 2, 48, 5)
    W = synth.head_weights(s, seed=seed, dtype="f32", ln="random")
    return {k: (v * 10 if k.endswith(("attn_qkv.weight", "xattn.k.weight", "xattn.q.weight")) else v)
            for k, v in W.items()}


def test_mean_pool_closed_forms():
    row = np.arange(7, dtype=np.float64)
    np.testing.assert_array_equal(oracle.mean_pool(np.tile(row, (5, 1))), row)
    x = np.arange(12, dtype=np.float64).reshape(4, 3)
    np.testing.assert_array_equal(oracle.mean_pool(x), np.array([4.5, 5.5, 6.5]))


def test_head_brute_force():
    x = np.random.default_rng(1).standard_normal((6, 32))
    for n_layer in (0, 2):
        W = weights(n_layer, seed=n_layer)
        a = oracle.attentive_pool_head(x, W, n_layer, 2)
        b = np.array(bruteforce.head(x, W, n_layer, 2))
        assert a.shape == (5,)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_head_token_permutation_invariance():
    x = np.random.default_rng(2).standard_normal((9, 32))
    W = weights(2, seed=3)
    a = oracle.attentive_pool_head(x, W, 2, 2)
    b = oracle.attentive_pool_head(x[np.random.default_rng(3).permutation(9)], W, 2, 2)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_head_single_token_is_an_mlp_on_q0_plus_v():
    x = np.random.default_rng(4).standard_normal((1, 32))
    W = {k: np.asarray(v, np.float64) for k, v in weights(0, seed=5).items()}
    got = oracle.attentive_pool_head(x, W, 0, 2)
    kv = oracle.layer_norm(x, W["head.xattn.ln_kv.weight"], W["head.xattn.ln_kv.bias"], 1e-6)
    y = W["head.query"] + oracle.linear(kv, W["head.xattn.v.weight"], W["head.xattn.v.bias"])
    h = oracle.layer_norm(y, W["head.xattn.ln2.weight"], W["head.xattn.ln2.bias"], 1e-6)
    y = y + oracle.linear(oracle.gelu_erf(oracle.linear(h, W["head.xattn.ffn_up.weight"], W["head.xattn.ffn_up.bias"])),
                          W["head.xattn.ffn_down.weight"], W["head.xattn.ffn_down.bias"])
    np.testing.assert_allclose(got, oracle.linear(y, W["head.cls.weight"], W["head.cls.bias"])[0],
                               rtol=1e-12, atol=1e-12)


def test_head_negative_controls():
    x = np.random.default_rng(6).standard_normal((8, 32))
    W = weights(1, seed=7)
    base = oracle.attentive_pool_head(x, W, 1, 2)
    # RoPE positions in the pool block (a plausible mistake) change the logits
    Wd = {k: np.asarray(v, np.float64) for k, v in W.items()}
    pos = oracle.rope_positions(np.arange(8), 2, 4)
    xr = oracle.block(np.asarray(x, np.float64), Wd, "head.blk.0", 2, pos, "tiled")
    with_rope = oracle.attentive_pool_head(xr, W, 0, 2)
    assert metrics.rel_max(with_rope, base) > 1e-3
    # a rescaled value path (what a stray output projection would do) changes them too
    W2 = dict(W)
    W2["head.xattn.v.weight"] = W["head.xattn.v.weight"] * 2
    W2["head.xattn.v.bias"] = W["head.xattn.v.bias"] * 2
    assert metrics.rel_max(oracle.attentive_pool_head(x, W2, 1, 2), base) > 1e-3
