"""Parity of the V-JEPA 2.1 additions against the oracle, through the C ABI: the native
image path (jepa_encode_image) and the 2.1 predictor (jepa_predict_mod: modality vector
on every row, context projection; [Notes §3] "2.1 encoder forward" / "2.1 predictor
forward").

  * tiny fp32 encoder (interleaved, interpolated, modality vectors) on a 64x64 image:
    fp32 gate;
  * 2.1 ViT-B/16 on a 384x384 image (576 tokens, 12 layers, bf16): bf16 gate; 16 such
    images give each image's tokens bit for bit as it alone does (other GEMM tiles);
  * 2.1 ViT-B predictor, full 12 blocks, on the 24x24 image grid (64 context, 512 targets,
    image vector): predictions and projected context rows within the bf16 gate, while
    the oracle's video-vector output fails it (the pages' wrong-vector case); AUTO picks
    the image vector there (bit for bit);
  * the same predictor with 2 blocks on the 8x24x24 video grid (512 context, 4096
    targets): bf16 gate; jepa_predict equals jepa_predict_mod with the video vector;
  * argument errors: the image path on an encoder without it, a context output without
    pred.proj_context, a bad modality.
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, assert_f32_gate, banner, f32, host, i32, u8
from oracle import metrics

pytestmark = pytest.mark.gpu


def test_tiny_fp32_image_path():
    banner("tiny fp32 image path 64x64")
    s = synth.EncoderShape(768, 2, 12, 3072, has_mod_embed=True, has_image_embed=True)
    W = synth.encoder_weights(s, seed=5, dtype="f32", ln="random")
    img = synth.clip_u8(31, 1, 1, 64, 64)[:, 0]
    enc = J.Encoder(768, 2, 12, 3072, layout="interleaved", ref_grid=16, has_mod_embed=True,
                    dtype="f32", max_rows=32, has_image_embed=True)
    enc.set_weights(W)
    got = host(enc.encode_image(u8(img)))[0]
    spec = oracle.EncoderSpec(768, 2, 12, 3072, has_mod_embed=True, layout="interleaved", ref_grid=16)
    ref = oracle.encoder_forward_image(img[0], W, spec)
    assert got.shape == (16, 768)
    assert_f32_gate(got, ref, "tiny image path")


def test_vitb16_image_384():
    w = synth.workload("vitb16_img384")
    banner("2.1 ViT-B image 384x384, 576 tokens, 12 layers")
    e = w["enc"]
    W = synth.encoder_weights(e, seed=0, dtype="bf16")
    img = synth.clip_u8(32, 1, 1, 384, 384)[:, 0]
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, layout="interleaved", ref_grid=16,
                    has_mod_embed=True, dtype="bf16", max_rows=576, has_image_embed=True)
    enc.set_weights(W)
    got = host(enc.encode_image(u8(img)))[0]
    spec = oracle.EncoderSpec(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, has_mod_embed=True,
                              layout="interleaved", ref_grid=16)
    ref = oracle.encoder_forward_image(img[0], W, spec)
    assert_bf16_gate(got, ref, "vitb image 384")



def test_vitb16_image_384_batch_of_16_equals_single():
    # 16 images (9216 rows) take one round of 256 x 128 tiles in the N = 768 projections and
    # 256-row tiles in QKV, a single image (576 rows) 128 x 128 tiles; every output element
    # sums over K in the same order with any tile, so each image's tokens are the same bits
    # alone and in the batch
    w = synth.workload("vitb16_img384")
    banner("2.1 ViT-B image 384x384: 16 images against images 0 and 15 alone")
    e = w["enc"]
    W = synth.encoder_weights(e, seed=0, dtype="bf16")
    imgs = synth.clip_u8(33, 16, 1, 384, 384)[:, 0]
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, layout="interleaved", ref_grid=16,
                    has_mod_embed=True, dtype="bf16", max_rows=16 * 576, has_image_embed=True)
    enc.set_weights(W)
    batch = host(enc.encode_image(u8(imgs)))
    assert batch.shape == (16, 576, e.embed_dim) and np.all(np.isfinite(batch))
    for i in (0, 15):
        one = host(enc.encode_image(u8(imgs[i:i + 1])))[0]
        assert np.array_equal(one, batch[i]), (i, float(np.max(np.abs(one - batch[i]))))

def _pred(w, n_layer=None):
    p = w["pred"]
    L = p.n_layer if n_layer is None else n_layer
    ps = synth.PredictorShape(p.enc_dim, p.embed_dim, L, p.n_head, p.ffn_dim, p.n_mask_tokens, p.out_dim,
                              has_mod_embed=True, has_proj_context=True)
    W = synth.predictor_weights(ps, seed=1, dtype="bf16")
    pred = J.Predictor(p.enc_dim, p.embed_dim, L, p.n_head, p.ffn_dim, p.n_mask_tokens, p.out_dim,
                       layout="interleaved", dtype="bf16", max_rows=4608, has_mod_embed=True,
                       has_proj_context=True)
    pred.set_weights(W)
    spec = oracle.PredictorSpec(p.enc_dim, p.embed_dim, L, p.n_head, p.ffn_dim, p.n_mask_tokens,
                                p.out_dim, layout="interleaved", has_mod_embed=True, has_proj_context=True)
    return pred, W, spec


def test_v21_predictor_image_grid():
    w = synth.workload("vitb16_pred21")
    grid = w["grid_image"]
    banner("2.1 predictor, image grid 24x24, 64 ctx + 512 targets, 12 blocks")
    pred, W, spec = _pred(w)
    ids_ctx, ids_tgt = synth.tube_mask(3, *grid)
    z = synth.tokens_normal(6, 1, 576, 768)[0]
    out, ctx = pred.predict_mod(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid,
                                modality="image", context=True)
    out, ctx = host(out), host(ctx)
    ref, ref_ctx = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, w["mask_index"], grid,
                                            modality="img", return_context=True)
    assert out.shape == (512, 1664) and ctx.shape == (64, 1664)
    assert_bf16_gate(out, ref, "2.1 predictor image targets")
    assert_bf16_gate(ctx, ref_ctx, "2.1 predictor image context")
    wrong, _ = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, w["mask_index"], grid,
                                        modality="video", return_context=True)
    assert metrics.rel_max(out, wrong) > 2e-2
    auto = host(pred.predict_mod(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid, modality="auto"))
    assert np.array_equal(auto, out)


def test_v21_predictor_video_grid():
    w = synth.workload("vitb16_pred21")
    grid = w["grid_video"]
    banner("2.1 predictor, video grid 8x24x24, 512 ctx + 4096 targets, 2 blocks")
    pred, W, spec = _pred(w, n_layer=2)
    ids_ctx, ids_tgt = synth.tube_mask(4, *grid)
    z = synth.tokens_normal(7, 1, 4608, 768)[0]
    out, ctx = pred.predict_mod(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid,
                                modality="video", context=True)
    out, ctx = host(out), host(ctx)
    ref, ref_ctx = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, w["mask_index"], grid,
                                            modality="video", return_context=True)
    assert_bf16_gate(out, ref, "2.1 predictor video targets")
    assert_bf16_gate(ctx, ref_ctx, "2.1 predictor video context")
    plain = host(pred.predict(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid))
    assert np.array_equal(plain, out)
    auto = host(pred.predict_mod(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid, modality="auto"))
    assert np.array_equal(auto, out)


def test_v21_argument_errors():
    import torch
    banner("2.1 argument errors")
    enc = J.Encoder(768, 0, 12, 3072, dtype="f32", max_rows=16)
    img = u8(synth.clip_u8(33, 1, 1, 64, 64)[:, 0])
    out = torch.full((1, 16, 768), 7.0, device="cuda")
    with pytest.raises(J.JepaError):
        J.jepa_encode_image(enc.handle, img, out)
    pred = J.Predictor(64, 64, 0, 2, 128, 2, 128, dtype="f32", max_rows=8)
    z = f32(np.zeros((4, 64)))
    ic, it = i32(np.array([0, 1])), i32(np.array([2, 3]))
    o = torch.full((2, 128), 7.0, device="cuda")
    c = torch.full((2, 128), 7.0, device="cuda")
    with pytest.raises(J.JepaError):   # no pred.proj_context
        J.jepa_predict_mod(pred.handle, z, ic, it, 1, "video", (1, 2, 2), o, c)
    with pytest.raises(ValueError):
        J.jepa_predict_mod(pred.handle, z, ic, it, 1, "sideways", (1, 2, 2), o)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((o == 7.0).all()) and bool((c == 7.0).all())
