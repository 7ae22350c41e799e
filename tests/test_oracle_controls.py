"""The negative controls of the bf16 gate, on the CPU.

  * With nothing planted, each control forward of ``tests/controls.py`` equals the
    oracle's bit for bit, so a control that fails the gate fails it for its planted
    mistake alone.
  * On the sharp-attention draws (q/k/v weights with std 0.02 s, see ``synth``) every
    planted mistake of the RoPE and transposed-V code fails the bf16 gate against the
    oracle: the frequency layout swapped ([Notes §4.1] vs §4.2), no rotation (all
    positions 0), no interpolation ([Notes §4.3]), row index used as position, and value
    rows permuted against the keys.  Mirrors, at sizes the oracle finishes in seconds,
    the controls the GPU tests assert on the full workloads.
  * The temporal-shift invariance of the interleaved layout ([Notes §4.2]: a rotation, so
    scores depend on position differences only) holds on the sharp draws too, and the
    tiled layout ([Notes §4.1]: not a rotation) fails the bf16 gate under the same shift.
"""
import numpy as np
import pytest

import controls
import oracle
import synth


def _vitl(n_layer=1, qkv_scale=3.0, layout="tiled", ref_grid=0, final_norm=False):
    shape = synth.EncoderShape(1024, n_layer, 16, 4096, final_norm=final_norm)
    W = synth.encoder_weights(shape, seed=3, dtype="bf16", qkv_scale=qkv_scale)
    spec = oracle.EncoderSpec(1024, n_layer, 16, 4096, final_norm=final_norm, layout=layout,
                              ref_grid=ref_grid)
    return W, spec


def test_vt_bitswap_is_the_bit_2_3_exchange():
    p = controls.vt_bitswap(16)
    assert list(p) == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]
    q = controls.vt_bitswap(70)
    assert sorted(q) == list(range(70))
    assert np.array_equal(q[q], np.arange(70))     # an involution
    # 68 and 69 would swap to 72 and 73, past the end: they stay
    assert list(q[64:70]) == [64, 65, 66, 67, 68, 69]


def test_controls_without_a_planted_mistake_equal_the_oracle():
    W, spec = _vitl(n_layer=2, final_norm=True, layout="interleaved", ref_grid=16)
    grid = (2, 4, 6)
    ids = np.random.default_rng(0).permutation(48)
    x = synth.tokens_normal(1, 1, 48, 1024)[0]
    pos = oracle.rope_positions(ids, grid[1], grid[2], 16)
    rows = np.array([0, 5, 47])
    assert np.array_equal(controls.encode_tokens(x, W, spec, pos),
                          oracle.encode_tokens(x, W, spec, ids, grid))
    assert np.array_equal(controls.encode_tokens(x, W, spec, pos, last_rows=rows),
                          oracle.encode_tokens(x, W, spec, ids, grid, last_rows=rows))
    # embedding + blocks = the pixel forward
    clip = synth.clip_u8(2, 1, 4, 64, 96)[0]
    e = controls.embed(clip, W, spec)
    pos = oracle.rope_positions(np.arange(48), 4, 6, 16)
    assert np.array_equal(controls.encode_tokens(e, W, spec, pos), oracle.encoder_forward(clip, W, spec))
    # predictor
    p = synth.PredictorShape(1024, 384, 2, 12, 1536, 10, 1024)
    Wp = synth.predictor_weights(p, seed=4, dtype="bf16", qkv_scale=3.0)
    ps = oracle.PredictorSpec(1024, 384, 2, 12, 1536, 10, 1024)
    z = synth.tokens_normal(5, 1, 64, 1024)[0]
    ids_ctx, ids_tgt = synth.tube_mask(1, 1, 8, 8, bh=4, bw=4)
    pos = oracle.rope_positions(np.concatenate([ids_ctx, ids_tgt]), 8, 8, 0)
    last = np.array([1, 7, 40])
    for lr in (None, last):
        assert np.array_equal(controls.predictor(z, Wp, ps, ids_ctx, ids_tgt, 1, pos, last_rows=lr),
                              oracle.predictor_forward(z, Wp, ps, ids_ctx, ids_tgt, 1, (1, 8, 8), last_rows=lr))


def test_sharp_block_controls_fail_the_bf16_gate():
    # one ViT-L block on a 2 x 8 x 8 grid (128 tokens), tiled
    W, spec = _vitl()
    grid = (2, 8, 8)
    ids = np.arange(128)
    x = synth.tokens_normal(0, 1, 128, 1024)[0]
    ref = oracle.encode_tokens(x, W, spec, ids, grid)
    pos = oracle.rope_positions(ids, 8, 8, 0)
    planted = {
        "layout swapped": controls.encode_tokens(x, W, spec, pos, layout="interleaved"),
        "no rotation": controls.encode_tokens(x, W, spec, np.zeros_like(pos)),
        "V^T bit swap": controls.encode_tokens(x, W, spec, pos, v_perm=controls.vt_bitswap(128)),
    }
    for what, got in planted.items():
        assert controls.fails_bf16_gate(got, ref), what
    # the unsharpened draws are what the old gates ran on: there the swap passes
    W1, _ = _vitl(qkv_scale=1.0)
    ref1 = oracle.encode_tokens(x, W1, spec, ids, grid)
    assert not controls.fails_bf16_gate(controls.encode_tokens(x, W1, spec, pos, layout="interleaved"), ref1)


def test_sharp_interpolated_controls_fail_the_bf16_gate():
    # 2.1 ViT-B width, interleaved, positions interpolated onto a 16 grid on 2 x 24 x 24
    shape = synth.EncoderShape(768, 1, 12, 3072, has_mod_embed=True)
    W = synth.encoder_weights(shape, seed=3, dtype="bf16", qkv_scale=3.0)
    spec = oracle.EncoderSpec(768, 1, 12, 3072, has_mod_embed=True, layout="interleaved", ref_grid=16)
    grid = (2, 24, 24)
    ids = np.arange(1152)
    x = synth.tokens_normal(0, 1, 1152, 768)[0]
    rows = np.arange(0, 1152, 7)
    ref = oracle.encode_tokens(x, W, spec, ids, grid, last_rows=rows)
    pos = oracle.rope_positions(ids, 24, 24, 16)
    planted = {
        "layout swapped": controls.encode_tokens(x, W, spec, pos, layout="tiled", last_rows=rows),
        "no interpolation": controls.encode_tokens(x, W, spec, oracle.rope_positions(ids, 24, 24, 0),
                                                   last_rows=rows),
        "no rotation": controls.encode_tokens(x, W, spec, np.zeros_like(pos), last_rows=rows),
        "V^T bit swap": controls.encode_tokens(x, W, spec, pos, last_rows=rows,
                                               v_perm=controls.vt_bitswap(1152)),
    }
    for what, got in planted.items():
        assert controls.fails_bf16_gate(got, ref), what


def test_sharp_predictor_controls_fail_the_bf16_gate():
    # head dim 32 (10 rotated dims per axis, 2 pass-through), tiled, ids from a tube mask
    p = synth.PredictorShape(1024, 384, 1, 12, 1536, 10, 1024)
    Wp = synth.predictor_weights(p, seed=3, dtype="bf16", qkv_scale=3.0)
    ps = oracle.PredictorSpec(1024, 384, 1, 12, 1536, 10, 1024)
    grid = (4, 8, 8)
    ids_ctx, ids_tgt = synth.tube_mask(2, *grid, bh=4, bw=4)
    z = synth.tokens_normal(6, 1, 256, 1024)[0]
    ref = oracle.predictor_forward(z, Wp, ps, ids_ctx, ids_tgt, 1, grid)
    pos = oracle.rope_positions(np.concatenate([ids_ctx, ids_tgt]), 8, 8, 0)
    n = len(pos)
    planted = {
        "layout swapped": controls.predictor(z, Wp, ps, ids_ctx, ids_tgt, 1, pos, layout="interleaved"),
        "no rotation": controls.predictor(z, Wp, ps, ids_ctx, ids_tgt, 1, np.zeros_like(pos)),
        "row index as position": controls.predictor(
            z, Wp, ps, ids_ctx, ids_tgt, 1, oracle.rope_positions(np.arange(n), 8, 8, 0)),
        "V^T bit swap": controls.predictor(z, Wp, ps, ids_ctx, ids_tgt, 1, pos,
                                           v_perm=controls.vt_bitswap(n)),
    }
    for what, got in planted.items():
        assert controls.fails_bf16_gate(got, ref), what


@pytest.mark.parametrize("layout", ["interleaved", "tiled"])
def test_sharp_temporal_shift(layout):
    W, spec = _vitl(layout=layout)
    x = synth.tokens_normal(0, 1, 128, 1024)[0]
    ids = np.arange(128)
    ref = oracle.encode_tokens(x, W, spec, ids, (2, 8, 8))
    shifted = oracle.encode_tokens(x, W, spec, ids + 3 * 64, (5, 8, 8))
    if layout == "interleaved":
        assert oracle.metrics.rel_max(shifted, ref) < 1e-9
    else:
        assert controls.fails_bf16_gate(shifted, ref)
