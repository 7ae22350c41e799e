"""Pins of the oracle's composed encoder and predictor (CPU only).

  * brute force: a pure-Python, element-by-element forward (tests/bruteforce.py) of a
    tiny encoder (D = 32, two heads of 16, so d = 4 per axis and 4 pass-through dims)
    and of a tiny predictor agrees with the numpy oracle to ~1e-12, for both layouts,
    with interpolation, the modality vector and non-trivial LayerNorm affines;
  * invariants: permutation equivariance of the blocks (rows moved with their ids),
    temporal-shift invariance of the interleaved layout (and its failure for tiled),
    batch independence, predictor context-order invariance;
  * negative controls: swapping the RoPE layout and a +1 % change of one weight matrix
    both move the output far outside the fp32 gate (rel_max 1e-3);
  * shapes: the ViT-L encoder + predictor tensor list has the pages' 443 tensors and
    326 M parameters.
"""
import json
import os

import numpy as np
import pytest

import bruteforce
import oracle
import synth
from oracle import metrics

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))

TINY = synth.EncoderShape(32, 2, 2, 48)


def tiny_spec(layout, ref_grid=0, mod=False, final_norm=True, n_layer=2):
    return oracle.EncoderSpec(32, n_layer, 2, 48, has_mod_embed=mod, final_norm=final_norm,
                              layout=layout, ref_grid=ref_grid)


def tiny_weights(mod=False, seed=0, n_layer=2, final_norm=True):
    s = synth.EncoderShape(32, n_layer, 2, 48, has_mod_embed=mod, final_norm=final_norm)
    W = synth.encoder_weights(s, seed=seed, dtype="f32", ln="random")
    # larger weights than the workload recipe so every term matters at 1e-12
    return {k: (v * 10 if k.endswith("attn_qkv.weight") else v) for k, v in W.items()}


@pytest.mark.parametrize("layout,ref_grid,mod", [("tiled", 0, False), ("interleaved", 16, True),
                                                 ("interleaved", 0, False), ("tiled", 16, True)])
def test_tiny_encoder_brute_force(layout, ref_grid, mod):
    clip = synth.clip_u8(3, 1, 4, 32, 48)[0]  # grid 2 x 2 x 3 = 12 tokens
    W = tiny_weights(mod)
    a = oracle.encoder_forward(clip, W, tiny_spec(layout, ref_grid, mod))
    b = np.array(bruteforce.encoder(clip, W, 2, 2, layout, ref_grid, mod))
    assert a.shape == (12, 32)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    assert metrics.rel_max(a, b) < 1e-12


def test_tiny_predictor_brute_force():
    rng = np.random.default_rng(5)
    grid = (2, 3, 3)
    z = rng.standard_normal((18, 32))
    ps = synth.PredictorShape(32, 16, 2, 1, 24, 3, 20)  # head dim 16
    W = synth.predictor_weights(ps, seed=1, dtype="f32", ln="random")
    W = {k: (v * 10 if k.endswith("attn_qkv.weight") or k == "pred.mask_tokens" else v) for k, v in W.items()}
    spec = oracle.PredictorSpec(32, 16, 2, 1, 24, 3, 20)
    ids_ctx = np.array([0, 4, 5, 9, 13])
    ids_tgt = np.array([1, 2, 17, 8, 4])  # target id 4 also in context: same position
    a = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, 4, grid)
    b = np.array(bruteforce.predictor(z, W, ids_ctx, ids_tgt, 4, grid, 2, 1, 3))
    assert a.shape == (5, 20)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def _tokens(N, D, seed=0):
    return np.random.default_rng(seed).standard_normal((N, D)) * 2


def test_block_permutation_equivariance():
    # moving token rows together with their ids permutes the output the same way
    spec = tiny_spec("tiled", final_norm=True)
    W = tiny_weights()
    grid = (2, 3, 4)
    N = 24
    x = _tokens(N, 32)
    ids = np.arange(N)
    perm = np.random.default_rng(1).permutation(N)
    a = oracle.encode_tokens(x, W, spec, ids, grid)
    b = oracle.encode_tokens(x[perm], W, spec, ids[perm], grid)
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


def test_temporal_shift_invariance_interleaved_only():
    W = tiny_weights()
    grid = (2, 3, 3)
    x = _tokens(18, 32, 3)
    ids = np.arange(18)
    shifted = ids + 3 * 9  # t -> t + 3 on a grid with 5 temporal slots
    for layout, same in (("interleaved", True), ("tiled", False)):
        spec = tiny_spec(layout)
        a = oracle.encode_tokens(x, W, spec, ids, grid)
        b = oracle.encode_tokens(x, W, spec, shifted, (5, 3, 3))
        if same:
            np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
        else:
            assert metrics.rel_max(b, a) > 1e-3


def test_batch_independence():
    spec = tiny_spec("tiled")
    W = tiny_weights()
    clips = synth.clip_u8(4, 3, 4, 32, 32)
    out = oracle.encoder_forward_batch(clips, W, spec)
    np.testing.assert_array_equal(out[1], oracle.encoder_forward(clips[1], W, spec))
    clips2 = clips.copy(); clips2[0] = 255 - clips2[0]
    out2 = oracle.encoder_forward_batch(clips2, W, spec)
    np.testing.assert_array_equal(out2[1:], out[1:])


def test_predictor_context_order_invariance():
    # Meta sorts the tokens by id and unsorts; attention is permutation-equivariant so
    # the order of the context rows does not change the target predictions ([Notes §3])
    rng = np.random.default_rng(9)
    grid = (2, 3, 3)
    z = rng.standard_normal((18, 32))
    ps = synth.PredictorShape(32, 16, 1, 1, 24, 3, 20)
    W = synth.predictor_weights(ps, seed=2, dtype="f32", ln="random")
    spec = oracle.PredictorSpec(32, 16, 1, 1, 24, 3, 20)
    ids_ctx = np.array([0, 4, 5, 9, 13]); ids_tgt = np.array([1, 2, 17, 8])
    a = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt, 1, grid)
    b = oracle.predictor_forward(z, W, spec, ids_ctx[::-1], ids_tgt, 1, grid)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    pt = np.array([2, 0, 3, 1])
    c = oracle.predictor_forward(z, W, spec, ids_ctx, ids_tgt[pt], 1, grid)
    np.testing.assert_allclose(c, a[pt], rtol=1e-12, atol=1e-13)


def test_negative_controls_fail_the_fp32_gate():
    # [Notes §6]: a wrong RoPE layout collapses parity; [Parity "Thresholds"]: +1 % on
    # one weight tensor fails rel_max.  Same here at tiny scale with D = 768 heads.
    spec = oracle.EncoderSpec(768, 1, 12, 3072, layout="tiled")
    s = synth.EncoderShape(768, 1, 12, 3072)
    W = synth.encoder_weights(s, seed=0, dtype="f32")
    clip = synth.clip_u8(0, 1, 4, 64, 64)[0]
    ref = oracle.encoder_forward(clip, W, spec)
    swapped = oracle.encoder_forward(clip, W, oracle.EncoderSpec(768, 1, 12, 3072, layout="interleaved"))
    assert metrics.rel_max(swapped, ref) > 1e-3
    # with these random weights the attention branch is small next to the residual, so
    # the perturbed tensors are the FFN matrices and the patch embedding
    for name in ("enc.blk.0.ffn_down.weight", "enc.blk.0.ffn_up.weight", "enc.patch_embed.weight"):
        W2 = dict(W); W2[name] = W[name] * 1.01
        pert = oracle.encoder_forward(clip, W2, spec)
        assert metrics.rel_max(pert, ref) > 2e-3, name


def test_vitl_tensor_and_parameter_counts():
    enc = synth.encoder_tensor_list(synth.EncoderShape(1024, 24, 16, 4096))
    pred = synth.predictor_tensor_list(synth.PredictorShape(1024, 384, 12, 12, 1536, 10, 1024))
    g = GOLD["vitl_fpc64_counts"]
    assert len(enc) + len(pred) == g["tensors"]
    params = sum(int(np.prod(s)) for _, s, _ in enc + pred)
    assert round(params / 1e6) == g["params_millions_rounded"]
    assert params == 325_971_328


def test_vitb21_tensor_and_parameter_counts():
    # the 2.1 ViT-B encoder (video and image embeddings, modality vectors) and the 2.1
    # predictor (modality vectors, context projection) as built here; the checkpoint also
    # holds three more hierarchical LayerNorms of the encoder (the final norm is the fourth;
    # the hierarchical taps are not built) and stores each of the 8 mask tokens as its own
    # tensor (one [8, 384] tensor here)
    enc = synth.encoder_tensor_list(synth.WORKLOADS["vitb16_img384"]["enc"])
    pred = synth.predictor_tensor_list(synth.WORKLOADS["vitb16_pred21"]["pred"])
    g = GOLD["vitb21_counts"]
    assert len(enc) + 3 * 2 == g["encoder_tensors"]
    assert len(pred) + (8 - 1) == g["predictor_tensors"]
    params = sum(int(np.prod(s)) for _, s, _ in enc + pred)
    assert round(params / 1e6, 1) == g["params_millions_1dp"]
    assert round((params + 3 * 2 * 768) / 1e6, 1) == g["params_millions_1dp"]


@pytest.mark.parametrize("layout,ref_grid", [("tiled", 0), ("interleaved", 16)])
def test_last_rows_restriction_equals_full_rows(layout, ref_grid):
    # the sampled-row evaluation used by the full-size parity tests returns exactly the
    # selected rows of the full forward (brute force anchors the full forward above)
    clip = synth.clip_u8(4, 1, 4, 32, 48)[0]
    W = tiny_weights(ref_grid > 0)
    spec = tiny_spec(layout, ref_grid, ref_grid > 0)
    full = oracle.encoder_forward(clip, W, spec)
    rows = np.array([11, 0, 5, 7])
    part = oracle.encoder_forward(clip, W, spec, last_rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-13)

    rng = np.random.default_rng(6)
    z = rng.standard_normal((18, 32))
    ps = oracle.PredictorSpec(32, 16, 2, 1, 24, 3, 20)
    Wp = synth.predictor_weights(synth.PredictorShape(32, 16, 2, 1, 24, 3, 20), seed=2,
                                 dtype="f32", ln="random")
    ids_ctx, ids_tgt = np.array([0, 4, 5, 9]), np.array([1, 2, 17, 8, 3])
    fullp = oracle.predictor_forward(z, Wp, ps, ids_ctx, ids_tgt, 1, (2, 3, 3))
    r = np.array([4, 1])
    partp = oracle.predictor_forward(z, Wp, ps, ids_ctx, ids_tgt, 1, (2, 3, 3), last_rows=r)
    np.testing.assert_allclose(partp, fullp[r], rtol=1e-13, atol=1e-13)
