"""Pins of the oracle's V-JEPA 2.1 additions (CPU only): the native image path of the
encoder and the 2.1 predictor's modality vector and context projection ([Notes §3] "2.1
encoder forward" and "2.1 predictor forward", [Notes §2] key map).

  * image path = video path on a two-frame clip of the same image, with the tubelet-2
    kernel built from the tubelet-1 one (each half carries half the weight) and the
    image modality vector in the video slot: a closed form that fixes the tubelet-1
    feature order, the image tensors and the one-slot grid;
  * image path against the brute-force encoder fed one frame with tubelet 1;
  * 2.1 predictor (modality vector on every row, context projection) against the
    brute-force predictor, both layouts;
  * the modality vector matters (image against video vector, the pages' wrong-vector
    case) and the context outputs follow the context rows when they are permuted, while
    the predictions stay put.
"""
import numpy as np
import pytest

import bruteforce
import oracle
import synth
from oracle import metrics


def enc_spec(layout="interleaved", ref_grid=16):
    return oracle.EncoderSpec(32, 2, 2, 48, has_mod_embed=True, layout=layout, ref_grid=ref_grid)


def enc_weights(seed=0):
    s = synth.EncoderShape(32, 2, 2, 48, has_mod_embed=True, has_image_embed=True)
    W = synth.encoder_weights(s, seed=seed, dtype="f32", ln="random")
    return {k: (v * 10 if k.endswith("attn_qkv.weight") else v) for k, v in W.items()}


def test_image_path_equals_video_path_on_a_doubled_frame():
    img = synth.clip_u8(21, 1, 1, 48, 32)[0, 0]            # 3 x 2 grid
    W = enc_weights()
    Wv = dict(W)
    wi = W["enc.patch_embed_img.weight"].astype(np.float64).reshape(32, 3, 1, 256)
    Wv["enc.patch_embed.weight"] = np.concatenate([wi / 2, wi / 2], axis=2).reshape(32, 1536)
    Wv["enc.patch_embed.bias"] = W["enc.patch_embed_img.bias"]
    Wv["enc.mod_embed_video"] = W["enc.mod_embed_img"]
    s = enc_spec()
    a = oracle.encoder_forward_image(img, W, s)
    b = oracle.encoder_forward(np.stack([img, img]), Wv, s)
    assert a.shape == (6, 32)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_image_path_brute_force():
    img = synth.clip_u8(22, 1, 1, 32, 48)[0, 0]            # 2 x 3 grid
    W = enc_weights(1)
    Wb = dict(W)
    Wb["enc.patch_embed.weight"] = W["enc.patch_embed_img.weight"]
    Wb["enc.patch_embed.bias"] = W["enc.patch_embed_img.bias"]
    Wb["enc.mod_embed_video"] = W["enc.mod_embed_img"]
    a = oracle.encoder_forward_image(img, W, enc_spec())
    b = np.array(bruteforce.encoder(img[None], Wb, 2, 2, "interleaved", 16, True, tubelet=1))
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    assert metrics.rel_max(a, b) < 1e-12


def pred_setup(layout, seed=3):
    rng = np.random.default_rng(seed)
    grid = (2, 3, 3)
    z = rng.standard_normal((18, 32))
    ps = synth.PredictorShape(32, 16, 2, 1, 24, 3, 20, has_mod_embed=True, has_proj_context=True)
    W = synth.predictor_weights(ps, seed=seed, dtype="f32", ln="random")
    spec = oracle.PredictorSpec(32, 16, 2, 1, 24, 3, 20, layout=layout, has_mod_embed=True,
                                has_proj_context=True)
    return z, W, spec, grid


@pytest.mark.parametrize("layout,modality", [("interleaved", "video"), ("tiled", "img")])
def test_v21_predictor_brute_force(layout, modality):
    z, W, spec, grid = pred_setup(layout)
    ids_ctx = np.array([0, 4, 5, 9, 13]); ids_tgt = np.array([1, 2, 17, 8])
    pa, ca = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, 1, grid, modality=modality,
                                      return_context=True)
    pb, cb = bruteforce.predictor(z, W, ids_ctx, ids_tgt, 1, grid, 2, 1, 3, layout,
                                  mod=f"pred.mod_embed_{modality}", context=True)
    assert pa.shape == (4, 20) and ca.shape == (5, 20)
    np.testing.assert_allclose(pa, np.array(pb), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(ca, np.array(cb), rtol=1e-10, atol=1e-11)


def test_v21_predictor_modality_and_context_order():
    z, W, spec, grid = pred_setup("interleaved", seed=4)
    ids_ctx = np.array([3, 4, 10, 12, 16]); ids_tgt = np.array([0, 7, 8])
    pv, cv = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, 1, grid, return_context=True)
    pi, _ = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, 1, grid, modality="img",
                                     return_context=True)
    assert metrics.rel_max(pi, pv) > 1e-2
    perm = np.array([4, 2, 0, 3, 1])
    pp, cp = oracle.predictor_forward(z, W, spec, ids_ctx[perm], ids_tgt, 1, grid, return_context=True)
    np.testing.assert_allclose(pp, pv, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(cp, cv[perm], rtol=1e-11, atol=1e-12)
