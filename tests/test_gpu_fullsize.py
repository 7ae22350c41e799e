"""Parity at the full depth and size of the two largest workloads, against oracle values
stored by ``tests/golden/make_fullsize.py`` (the float64 oracle needs tens of minutes for
them; that script calls only ``oracle`` and ``synth``):

  * the V-JEPA 2.1 ViT-B/16 encoder, all 12 layers on one 64 x 384 x 384 clip (the full
    32 x 24 x 24 grid, 18,432 tokens, interleaved RoPE interpolated to 16, video modality
    vector; [HFport "Usage"], [Notes §4.3]), checked on 195 sampled rows of the output;
  * the 64-frame chain: the V-JEPA 2 ViT-L/16 encoder (24 layers) on one 64 x 256 x 256
    clip (8192 tokens), its output fed to the masked predictor (12 layers, head dim 32,
    2048 tube-mask context rows, 6144 targets; [Notes §3], [Notes §4.4]), the encoder
    checked on 192 sampled rows and the predictor on 128 sampled targets.

Both run in the launch configuration of the benchmark legs; bf16 gate on each.
"""
import json
import os
import sys

import numpy as np
import pytest

import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, banner, host, i32, u8

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_fullsize as mf  # noqa: E402

pytestmark = pytest.mark.gpu


def _load(path):
    with np.load(path, allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def test_vitb21_384_full_depth_sampled_rows():
    banner("vitb 2.1 384 64f, 12 layers, full grid, 195 sampled rows vs stored oracle")
    g = _load(mf.VITB_FILE)
    w, W, clip, rows = mf.vitb21_case()
    assert np.array_equal(rows, g["rows"])
    e = w["enc"]
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, layout=w["layout"],
                    ref_grid=w["ref_grid"], has_mod_embed=e.has_mod_embed, dtype="bf16",
                    max_rows=18432)
    enc.set_weights(W)
    out = host(enc.encode(u8(clip)))[0]
    assert out.shape == (18432, 768) and np.all(np.isfinite(out))
    assert_bf16_gate(out[rows], g["out"], "vitb 384 12 layers")
    enc.close()


def test_vitl16_64f_encoder_predictor_chain():
    banner("vitl16 64f 8192 tokens, 24 layers -> predictor 12 layers, vs stored oracle chain")
    g = _load(mf.CHAIN_FILE)
    w, W, Wp, clip, ids_ctx, ids_tgt, enc_rows, tgt_rows = mf.chain_case()
    e, p = w["enc"], w["pred"]
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, dtype="bf16", max_rows=8192)
    enc.set_weights(W)
    z = enc.encode(u8(clip))                       # [1, 8192, 1024] on the device
    zh = host(z)[0]
    assert_bf16_gate(zh[enc_rows], g["enc_out"], "64f encoder")
    pred = J.Predictor(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim, p.n_mask_tokens,
                       p.out_dim, dtype="bf16", max_rows=8192)
    pred.set_weights(Wp)
    out = host(pred.predict(z[0], i32(ids_ctx), i32(ids_tgt), w["mask_index"], w["grid"]))
    assert out.shape == (6144, 1024) and np.all(np.isfinite(out))
    assert_bf16_gate(out[tgt_rows], g["pred_out"], "chain predictor")
    enc.close()
    pred.close()
