"""Pins of the oracle's masked-encoder forward (CPU only).

[HFport "Usage"] passes the context ids to the encoder so that the other tokens are
dropped before the first block, attention sees only the context and RoPE takes each kept
token's own grid position; [HFport "Validation"] adds the control that this differs from
gathering rows of the full forward's output.  ``oracle.masked_encoder_forward`` is pinned
by:

  * brute force: the pure-Python element-by-element encoder (tests/bruteforce.py) with
    the same context ids, to ~1e-12, both layouts, with interpolation and the modality
    vector;
  * the pages' control: the masked forward moves far away from the gathered rows of the
    full forward;
  * all ids in grid order give the full forward exactly;
  * permutation equivariance: permuting the context ids permutes the output rows (so
    positions follow the ids, not the row order);
  * temporal-shift invariance of the interleaved layout: the same tubelets one slice
    later in the clip, with ids shifted by one slice, give the same output (so q and k
    take their positions from the same ids).
"""
import numpy as np
import pytest

import bruteforce
import oracle
import synth
from oracle import metrics


def spec(layout, ref_grid=0, mod=False, n_layer=2):
    return oracle.EncoderSpec(32, n_layer, 2, 48, has_mod_embed=mod, layout=layout, ref_grid=ref_grid)


def weights(mod=False, seed=0, n_layer=2):
    s = synth.EncoderShape(32, n_layer, 2, 48, has_mod_embed=mod)
    W = synth.encoder_weights(s, seed=seed, dtype="f32", ln="random")
    return {k: (v * 10 if k.endswith("attn_qkv.weight") else v) for k, v in W.items()}


@pytest.mark.parametrize("layout,ref_grid,mod", [("tiled", 0, False), ("interleaved", 16, True)])
def test_masked_brute_force(layout, ref_grid, mod):
    clip = synth.clip_u8(3, 1, 4, 32, 48)[0]          # grid 2 x 2 x 3 = 12 tokens
    ids = np.array([7, 0, 10, 3, 4])                  # any order, gaps on every axis
    W = weights(mod)
    a = oracle.masked_encoder_forward(clip, W, spec(layout, ref_grid, mod), ids)
    b = np.array(bruteforce.encoder(clip, W, 2, 2, layout, ref_grid, mod, ctx_ids=ids))
    assert a.shape == (5, 32)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    assert metrics.rel_max(a, b) < 1e-12


def test_masked_is_not_gathered_output():
    clip = synth.clip_u8(5, 1, 4, 48, 48)[0]          # 2 x 3 x 3 = 18 tokens
    ids = np.array([1, 2, 5, 9, 11, 16])
    W = weights()
    s = spec("tiled")
    masked = oracle.masked_encoder_forward(clip, W, s, ids)
    gathered = oracle.encoder_forward(clip, W, s)[ids]
    assert metrics.rel_max(masked, gathered) > 1e-2


def test_all_ids_give_the_full_forward():
    clip = synth.clip_u8(6, 1, 4, 32, 48)[0]
    W = weights(mod=True)
    s = spec("interleaved", 16, True)
    full = oracle.encoder_forward(clip, W, s)
    np.testing.assert_array_equal(oracle.masked_encoder_forward(clip, W, s, np.arange(12)), full)


def test_masked_permutation_equivariance():
    clip = synth.clip_u8(7, 1, 6, 48, 48)[0]          # 3 x 3 x 3 = 27 tokens
    ids = np.array([0, 4, 8, 13, 17, 21, 26, 3])
    perm = np.random.default_rng(2).permutation(len(ids))
    W = weights()
    s = spec("tiled")
    a = oracle.masked_encoder_forward(clip, W, s, ids)
    b = oracle.masked_encoder_forward(clip, W, s, ids[perm])
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_masked_temporal_shift_interleaved():
    # clip B holds clip A's frames 0..3 at frames 2..5: the tubelets of A's slices 0, 1
    # are B's slices 1, 2.  Interleaved RoPE depends on position differences only.
    a_clip = synth.clip_u8(8, 1, 6, 32, 48)[0]        # 3 x 2 x 3 grid, 6 tokens per slice
    b_clip = np.concatenate([synth.clip_u8(9, 1, 2, 32, 48)[0], a_clip[:4]])
    ids = np.array([0, 2, 4, 5, 7, 9, 10])            # slices 0 and 1 of A
    W = weights()
    s = spec("interleaved")
    a = oracle.masked_encoder_forward(a_clip, W, s, ids)
    b = oracle.masked_encoder_forward(b_clip, W, s, ids + 6)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    # the tiled layout is not relative: the same shift moves the output
    st = spec("tiled")
    assert metrics.rel_max(oracle.masked_encoder_forward(b_clip, W, st, ids + 6),
                           oracle.masked_encoder_forward(a_clip, W, st, ids)) > 1e-3
