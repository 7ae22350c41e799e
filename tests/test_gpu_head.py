"""Parity of the pooled outputs against the oracle, through the C ABI: jepa_pool_mean
([Card] "Run it", --pool mean) and the attentive-pool classifier head (jepa_head_forward,
[Notes §2] "Attentive-pool head — exact forward").

  * mean pool of 3 clips x 1000 tokens x 768 (and x 100 columns): within fp32 rounding of
    the fp64 mean;
  * tiny fp32 head (D 128, 2 heads of 64, 2 pool blocks, 10 classes) on 2 clips of 37
    tokens: fp32 gate (rel_max <= 1e-3) per clip;
  * the V-JEPA 2 SSv2 head shape (D 1024, 3 pool blocks, 16 heads, FFN 4096, 174
    classes) in bf16 on 2 clips of 2048 LayerNorm-like tokens: bf16 gate over the clips'
    logit rows; each clip's logits equal its single-clip run bit for bit;
  * shape and state errors.
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, assert_f32_gate, banner, f32, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [768, 100])
def test_mean_pool(D):
    import torch
    banner(f"mean pool 3 x 1000 x {D}")
    x = synth.normal(41, (3, 1000, D), k=9) + 0.5
    out = torch.empty((3, D), dtype=torch.float32, device="cuda")
    J.jepa_pool_mean(f32(x), out)
    got = host(out)
    for b in range(3):
        np.testing.assert_allclose(got[b], oracle.mean_pool(x[b]), rtol=2e-7, atol=1e-7)


def test_tiny_fp32_head():
    banner("tiny fp32 head, 2 clips x 37 tokens")
    s = synth.HeadShape(128, 2, 2, 256, 10)
    W = synth.head_weights(s, seed=1, dtype="f32", ln="random")
    x = synth.normal(42, (2, 37, 128), k=9)
    head = J.Head(128, 2, 2, 256, 10, dtype="f32", max_rows=80)
    head.set_weights(W)
    got = host(head.forward(f32(x)))
    for b in range(2):
        assert_f32_gate(got[b][None], oracle.attentive_pool_head(x[b], W, 2, 2)[None], f"tiny head {b}")


def test_ssv2_head_bf16():
    banner("SSv2-shaped head bf16, 2 clips x 2048 tokens")
    s = synth.HeadShape(1024, 3, 16, 4096, 174)
    W = synth.head_weights(s, seed=2, dtype="bf16")
    x = synth.tokens_normal(43, 2, 2048, 1024)
    head = J.Head(1024, 3, 16, 4096, 174, dtype="bf16", max_rows=4096)
    head.set_weights(W)
    got = host(head.forward(f32(x)))
    assert got.shape == (2, 174)
    ref = np.stack([oracle.attentive_pool_head(x[b], W, 3, 16) for b in range(2)])
    assert_bf16_gate(got, ref, "ssv2 head logits")
    for b in range(2):
        one = host(head.forward(f32(x[b:b + 1])))[0]
        assert np.array_equal(one, got[b]), b


def test_head_errors():
    import torch
    banner("head errors")
    head = J.Head(128, 1, 2, 256, 10, dtype="f32", max_rows=64)
    x = f32(np.zeros((1, 8, 128)))
    out = torch.full((1, 10), 7.0, device="cuda")
    with pytest.raises(J.JepaError):        # tensors never set
        head.forward(x, out=out)
    s = synth.HeadShape(128, 1, 2, 256, 10)
    head.set_weights(synth.head_weights(s, seed=3, dtype="f32"))
    with pytest.raises(J.JepaError):        # B*N > max_rows
        head.forward(f32(np.zeros((1, 65, 128))), out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
