"""End-to-end parity of jepa_encode / jepa_encode_tokens / jepa_predict against the oracle
on the five workloads, through the C ABI.

  * tiny fp32 encoder (4 frames x 64x64, 32 tokens): full forward, rel_max <= 1e-3, with
    the page recipe (LN 1/0) and with random LN affines; swapping the RoPE layout or
    nudging one weight matrix by +1 % must fail the same gate;
  * one ViT-L block on [1, 2048, 1024] N(0,1) tokens, bf16: full, bf16 gate;
  * the ViT-L/16 encoder on 4 clips x 16 frames x 256x256 in the launch configuration
    the benchmark times: clip 0 against the full 24-layer oracle (bf16 gate); every clip
    equals its own single-clip run bit for bit (batch independence);
  * the V-JEPA 2.1 ViT-B/16 encoder at 64 x 384x384 (18,432 tokens, interleaved,
    interpolated, modality vector): two layers on the full grid, the oracle evaluating the
    last layer on sampled rows (all 12 layers: tests/test_gpu_fullsize.py);
  * the masked predictor on the 32x16x16 grid (2048 context + 6144 targets, 12 layers,
    head dim 32): full depth, the oracle's last layer on sampled target rows.
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, assert_f32_gate, banner, f32, host, i32, u8
from oracle import metrics

pytestmark = pytest.mark.gpu


def _spec(w, n_layer=None):
    e = w["enc"]
    return oracle.EncoderSpec(e.embed_dim, e.n_layer if n_layer is None else n_layer, e.n_head,
                              e.ffn_dim, has_mod_embed=e.has_mod_embed, final_norm=e.final_norm,
                              layout=w["layout"], ref_grid=w["ref_grid"])


def _gpu_encoder(w, W, max_rows, n_layer=None):
    e = w["enc"]
    enc = J.Encoder(e.embed_dim, e.n_layer if n_layer is None else n_layer, e.n_head, e.ffn_dim,
                    layout=w["layout"], ref_grid=w["ref_grid"], has_mod_embed=e.has_mod_embed,
                    final_norm=e.final_norm, dtype=w["dtype"], max_rows=max_rows)
    enc.set_weights(W)
    return enc


# ------------------------------------------------------------------ tiny fp32


@pytest.mark.parametrize("ln", ["identity", "random"])
def test_tiny_fp32_encoder(ln):
    w = synth.workload("tiny_fp32")
    banner("tiny fp32 encoder", ln)
    W = synth.encoder_weights(w["enc"], seed=0, dtype="f32", ln=ln)
    clip = synth.clip_u8(0, 1, w["frames"], w["size"], w["size"])
    enc = _gpu_encoder(w, W, 32)
    got = host(enc.encode(u8(clip)))[0]
    ref = oracle.encoder_forward(clip[0], W, _spec(w))
    assert got.shape == (32, 768)
    assert_f32_gate(got, ref, "tiny fp32")
    # negative controls: wrong layout, +1 % on one weight matrix
    wrong = oracle.encoder_forward(clip[0], W, oracle.EncoderSpec(768, 2, 12, 3072,
                                                                  layout="interleaved"))
    assert metrics.rel_max(got, wrong) > 1e-3
    W2 = dict(W)
    W2["enc.blk.1.ffn_up.weight"] = W["enc.blk.1.ffn_up.weight"] * 1.01
    nudged = oracle.encoder_forward(clip[0], W2, _spec(w))
    assert metrics.rel_max(got, nudged) > 1e-3


def test_tiny_fp32_encode_tokens_with_ids_matches_oracle():
    # jepa_encode_tokens with shuffled ids: positions follow the ids
    w = synth.workload("tiny_fp32")
    banner("tiny fp32 encode_tokens ids")
    W = synth.encoder_weights(w["enc"], seed=1, dtype="f32", ln="random")
    rng = np.random.default_rng(4)
    ids = rng.permutation(32).astype(np.int32)
    x = synth.normal(3, (2, 32, 768), k=30)
    enc = _gpu_encoder(w, W, 64)
    got = host(enc.encode_tokens(f32(x), (2, 4, 4), ids=i32(ids)))
    for b in range(2):
        ref = oracle.encode_tokens(x[b], W, _spec(w), ids, (2, 4, 4))
        assert_f32_gate(got[b], ref, f"encode_tokens clip {b}")


# ------------------------------------------------------------------ one ViT-L block


def test_vitl_block_bf16():
    w = synth.workload("vitl_block")
    banner("vitl block bf16 [1, 2048, 1024]")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    x = synth.tokens_normal(0, 1, 2048, 1024)
    enc = _gpu_encoder(w, W, 2048)
    got = host(enc.encode_tokens(f32(x), w["grid"]))[0]
    ref = oracle.encode_tokens(x[0], W, _spec(w), np.arange(2048), w["grid"])
    assert_bf16_gate(got, ref, "vitl block")


# ------------------------------------------------------------------ ViT-L/16, 4 clips


@pytest.fixture(scope="module")
def vitl16():
    w = synth.workload("vitl16_16f256")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    clips = synth.clip_u8(0, w["B"], w["frames"], w["size"], w["size"])
    enc = _gpu_encoder(w, W, w["B"] * 2048)
    out = host(enc.encode(u8(clips)))
    return w, W, clips, enc, out


def test_vitl16_clip0_full_oracle(vitl16):
    w, W, clips, enc, out = vitl16
    banner("vitl16 4 clips, clip 0 vs 24-layer oracle")
    ref = oracle.encoder_forward(clips[0], W, _spec(w))
    assert out.shape == (4, 2048, 1024)
    assert_bf16_gate(out[0], ref, "vitl16 clip 0")


def test_vitl16_batch_independence(vitl16):
    w, W, clips, enc, out = vitl16
    banner("vitl16 batch independence")
    for b in range(4):
        one = host(enc.encode(u8(clips[b:b + 1])))[0]
        assert np.array_equal(one, out[b]), b


# ------------------------------------------------------------------ ViT-B 2.1 at 384


def test_vitb21_384_two_layers_sampled_rows():
    w = synth.scaled(synth.workload("vitb16_64f384"), n_layer=2)
    banner("vitb 2.1 384 64f, 2 layers, sampled rows")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    clip = synth.clip_u8(0, 1, 64, 384, 384)
    enc = _gpu_encoder(w, W, 18432)
    out = host(enc.encode(u8(clip)))[0]
    assert out.shape == (18432, 768)
    rows = np.sort(np.random.default_rng(7).choice(18432, 192, replace=False))
    rows = np.concatenate([[0, 575, 18431], rows])
    ref = oracle.encoder_forward(clip[0], W, _spec(w), last_rows=rows)
    assert_bf16_gate(out[rows], ref, "vitb 384 2 layers")


# ------------------------------------------------------------------ predictor


def test_predictor_full_grid_full_depth_sampled_rows():
    w = synth.workload("vitl16_64f256_pred")
    p = w["pred"]
    banner("predictor 8192 rows, 12 layers, sampled targets")
    Wp = synth.predictor_weights(p, seed=0, dtype="bf16")
    grid = w["grid"]
    ids_ctx, ids_tgt = synth.tube_mask(0, *grid)
    assert len(ids_ctx) == 2048 and len(ids_tgt) == 6144
    # the encoder's token map stands in as N(0,1) rows (an LN output is ~N(0,1))
    z = synth.tokens_normal(5, 1, 8192, 1024)[0]
    pred = J.Predictor(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim, p.n_mask_tokens,
                       p.out_dim, dtype="bf16", max_rows=8192)
    pred.set_weights(Wp)
    got = host(pred.predict(f32(z), i32(ids_ctx), i32(ids_tgt), w["mask_index"], grid))
    assert got.shape == (6144, 1024)
    rows = np.sort(np.random.default_rng(8).choice(6144, 128, replace=False))
    spec = oracle.PredictorSpec(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim,
                                p.n_mask_tokens, p.out_dim)
    ref = oracle.predictor_forward(z, Wp, spec, ids_ctx, ids_tgt, w["mask_index"], grid,
                                   last_rows=rows)
    assert_bf16_gate(got[rows], ref, "predictor")


def test_predictor_small_grid_full_rows():
    # every target row, on a small grid with a context id repeated among the targets
    w = synth.workload("vitl16_64f256_pred")
    p = w["pred"]
    banner("predictor small grid, all rows")
    Wp = synth.predictor_weights(p, seed=1, dtype="bf16", ln="random")
    grid = (4, 6, 6)
    rng = np.random.default_rng(12)
    perm = rng.permutation(144).astype(np.int32)
    ids_ctx, ids_tgt = perm[:40], np.concatenate([perm[40:], perm[:3]])
    z = synth.tokens_normal(6, 1, 144, 1024)[0]
    pred = J.Predictor(p.enc_dim, p.embed_dim, 3, p.n_head, p.ffn_dim, p.n_mask_tokens,
                       p.out_dim, dtype="bf16", max_rows=256)
    Wp3 = {k: v for k, v in Wp.items() if not k.startswith("pred.blk.") or int(k.split(".")[2]) < 3}
    pred.set_weights(Wp3)
    got = host(pred.predict(f32(z), i32(ids_ctx), i32(ids_tgt), 7, grid))
    spec = oracle.PredictorSpec(p.enc_dim, p.embed_dim, 3, p.n_head, p.ffn_dim, p.n_mask_tokens,
                                p.out_dim)
    ref = oracle.predictor_forward(z, Wp3, spec, ids_ctx, ids_tgt, 7, grid)
    assert_bf16_gate(got, ref, "predictor small")


# ------------------------------------------------------------------ errors


def test_encode_errors_leave_output_untouched():
    import torch
    w = synth.workload("tiny_fp32")
    banner("encode error paths")
    enc = J.Encoder(768, 2, 12, 3072, dtype="f32", max_rows=32)
    out = torch.full((1, 32, 768), 7.0, device="cuda:0")
    clip = u8(synth.clip_u8(0, 1, 4, 64, 64))
    with pytest.raises(J.JepaError) as e:       # weights never set
        enc.encode(clip, out=out)
    assert e.value.status == -3
    enc.set_weights(synth.encoder_weights(w["enc"], seed=0, dtype="f32"))
    lib = J.load()
    stream = torch.cuda.current_stream().cuda_stream

    def raw(clip_np, T=None):
        c = u8(clip_np)
        B, T0, H, W_, _ = clip_np.shape
        return lib.jepa_encode(enc.handle, c.data_ptr(), B, T0 if T is None else T, H, W_,
                               out.data_ptr(), stream)

    assert raw(synth.clip_u8(0, 1, 3, 64, 64)) == -2      # odd T
    assert raw(synth.clip_u8(0, 1, 4, 72, 64)) == -2      # H not a multiple of 16
    assert raw(synth.clip_u8(0, 2, 4, 64, 64)) == -2      # B*N above max_rows
    assert raw(synth.clip_u8(0, 1, 4, 64, 64), T=0) == -2  # no frames
    assert lib.jepa_encode(enc.handle, None, 1, 4, 64, 64, out.data_ptr(), stream) == -1
    with pytest.raises(J.JepaError) as e:       # unknown tensor name
        J.jepa_encoder_set_tensor(enc.handle, "enc.blk.9.ln1.weight", np.ones(768, np.float32))
    assert e.value.status == -4
    with pytest.raises(J.JepaError) as e:       # wrong shape
        J.jepa_encoder_set_tensor(enc.handle, "enc.norm.weight", np.ones(767, np.float32))
    assert e.value.status == -4
    assert bool(torch.all(out == 7.0))


def test_kernel_timing_counts_every_launch():
    import torch
    w = synth.workload("tiny_fp32")
    banner("kernel timing counts, tiny fp32 encoder x 2 forwards")
    enc = J.Encoder(768, 2, 12, 3072, dtype="f32", max_rows=32)
    enc.set_weights(synth.encoder_weights(w["enc"], seed=0, dtype="f32"))
    clip = u8(synth.clip_u8(0, 1, 4, 64, 64))
    ref = host(enc.encode(clip))
    J.jepa_timing_begin(8)
    try:
        got = [host(enc.encode(clip)) for _ in range(2)]
    finally:
        rec = J.jepa_timing_end()
    # timing changes no result
    for g in got:
        assert np.array_equal(g, ref)
    per_fwd = {"patchify": 1, "gemm_embed": 1, "layernorm": 2 * 2 + 1, "gemm_qkv": 2,
               "attention": 2, "gemm_out": 2, "gemm_up": 2, "gemm_down": 2, "other": 0}
    for k, n in per_fwd.items():
        ms, cnt = rec[k]
        assert cnt == min(2 * n, 8), (k, cnt)
        assert (ms > 0) == (cnt > 0), (k, ms)
    with pytest.raises(J.JepaError):
        J.jepa_timing_end()
    enc.close()
