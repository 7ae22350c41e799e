"""Parity of jepa_encode_masked (the masked-encoder forward, [HFport "Usage"]) against the
oracle's masked_encoder_forward, through the C ABI.

  * tiny fp32 encoder, 2 clips with different context ids (20 of 32 tokens, random order):
    each clip within the fp32 gate (rel_max <= 1e-3); the gathered rows of the full
    forward fail that gate ([HFport "Validation"] control);
  * all ids in grid order reproduce jepa_encode bit for bit (fp32 and bf16);
  * ViT-L/16 (24 layers, bf16), 4 clips x 16 frames x 256x256 with the tube-mask context
    (an 8x8 block of patches in every temporal slot, 512 of 2048 tokens): clip 0 against
    the full oracle (bf16 gate); each clip equals its own single-clip run bit for bit;
  * ragged and degenerate context sizes on the ViT-L path: 300 tokens (not a multiple of
    16) and a single token, against the oracle;
  * shape errors leave the output untouched.
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, assert_f32_gate, banner, host, i32, u8
from oracle import metrics

pytestmark = pytest.mark.gpu


def _spec(w):
    e = w["enc"]
    return oracle.EncoderSpec(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, has_mod_embed=e.has_mod_embed,
                              final_norm=e.final_norm, layout=w["layout"], ref_grid=w["ref_grid"])


def _encoder(w, W, max_rows):
    e = w["enc"]
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, layout=w["layout"],
                    ref_grid=w["ref_grid"], has_mod_embed=e.has_mod_embed, final_norm=e.final_norm,
                    dtype=w["dtype"], max_rows=max_rows)
    enc.set_weights(W)
    return enc


def test_tiny_fp32_masked_two_clips():
    w = synth.workload("tiny_fp32")
    banner("tiny fp32 masked, 2 clips x 20 of 32 tokens")
    W = synth.encoder_weights(w["enc"], seed=2, dtype="f32", ln="random")
    clips = synth.clip_u8(11, 2, w["frames"], w["size"], w["size"])
    ids = synth.context_ids(1, 2, 32, 20)
    assert not np.array_equal(ids[0], ids[1])
    enc = _encoder(w, W, 64)
    got = host(enc.encode_masked(u8(clips), i32(ids)))
    assert got.shape == (2, 20, 768)
    for b in range(2):
        ref = oracle.masked_encoder_forward(clips[b], W, _spec(w), ids[b])
        assert_f32_gate(got[b], ref, f"masked clip {b}")
        gathered = oracle.encoder_forward(clips[b], W, _spec(w))[ids[b]]
        assert metrics.rel_max(got[b], gathered) > 1e-3


def test_tiny_fp32_masked_all_ids_equals_encode():
    w = synth.workload("tiny_fp32")
    banner("tiny fp32 masked, all ids")
    W = synth.encoder_weights(w["enc"], seed=3, dtype="f32", ln="random")
    clips = synth.clip_u8(12, 2, w["frames"], w["size"], w["size"])
    enc = _encoder(w, W, 64)
    full = host(enc.encode(u8(clips)))
    ids = np.tile(np.arange(32, dtype=np.int32), (2, 1))
    masked = host(enc.encode_masked(u8(clips), i32(ids)))
    assert np.array_equal(masked, full)


@pytest.fixture(scope="module")
def vitl():
    w = synth.workload("vitl16_16f256")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    clips = synth.clip_u8(0, w["B"], w["frames"], w["size"], w["size"])
    enc = _encoder(w, W, w["B"] * 2048)
    return w, W, clips, enc


def _tube_ids(B, seed=0):
    return np.stack([synth.tube_mask(seed + b, 8, 16, 16)[0] for b in range(B)]).astype(np.int32)


def test_vitl16_masked_tube_context(vitl):
    w, W, clips, enc = vitl
    ids = _tube_ids(4)
    assert ids.shape == (4, 512)
    banner("vitl16 masked, 4 clips x 512 tube-mask context tokens, clip 0 vs oracle")
    out = host(enc.encode_masked(u8(clips), i32(ids)))
    ref = oracle.masked_encoder_forward(clips[0], W, _spec(w), ids[0])
    assert_bf16_gate(out[0], ref, "vitl16 masked clip 0")
    banner("vitl16 masked, batch independence")
    for b in range(4):
        one = host(enc.encode_masked(u8(clips[b:b + 1]), i32(ids[b:b + 1])))[0]
        assert np.array_equal(one, out[b]), b


def test_vitl16_masked_all_ids_equals_encode(vitl):
    w, W, clips, enc = vitl
    banner("vitl16 masked, all ids of 2 clips vs jepa_encode")
    full = host(enc.encode(u8(clips[:2])))
    ids = np.tile(np.arange(2048, dtype=np.int32), (2, 1))
    masked = host(enc.encode_masked(u8(clips[:2]), i32(ids)))
    assert np.array_equal(masked, full)


@pytest.mark.parametrize("K", [300, 1])
def test_vitl16_masked_ragged_and_single(vitl, K):
    w, W, clips, enc = vitl
    ids = synth.context_ids(5, 2, 2048, K)
    banner(f"vitl16 masked, 2 clips x {K} random context tokens, clip 1 vs oracle")
    out = host(enc.encode_masked(u8(clips[:2]), i32(ids)))
    assert out.shape == (2, K, 1024)
    ref = oracle.masked_encoder_forward(clips[1], W, _spec(w), ids[1])
    assert_bf16_gate(out[1], ref, f"vitl16 masked K={K}")


def test_masked_shape_errors():
    import torch
    w = synth.workload("tiny_fp32")
    banner("masked shape errors")
    W = synth.encoder_weights(w["enc"], seed=4, dtype="f32")
    enc = _encoder(w, W, 40)
    clips = u8(synth.clip_u8(13, 2, w["frames"], w["size"], w["size"]))
    for K in (0, 33, 21):   # K < 1, K > N, B*K > max_rows
        ids = i32(np.zeros((2, K), dtype=np.int32)) if K else torch.zeros((2, 0), dtype=torch.int32, device="cuda")
        out = torch.full((2, max(K, 1), 768), 7.0, device="cuda")
        if K == 0:
            out = torch.full((2, 0, 768), 7.0, device="cuda")
        with pytest.raises(J.JepaError):
            J.jepa_encode_masked(enc.handle, clips, ids, out)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
