"""GPU parity of jepa_attention_block_causal against the oracle, through the C ABI.

[Parity] "LeVJEPA ViT-L/16 — CLS, block-causal attention, tubelet 1": the CLS rows first
(no position: identity RoPE), then the patch tokens T-major; a patch query sees the patch
keys of its own and earlier temporal slots, a CLS query sees every key.  The oracle is
``oracle.attention`` with ``oracle.block_causal_mask`` (pinned in test_oracle_mask.py)
and position (0, 0, 0) for the CLS rows.

  * small cases on both paths (bf16 gate, fp32 rel_max <= 1e-5): 0, 1 and 3 CLS rows,
    slots smaller than a key tile, ragged tails, interpolation, both layouts; the
    unmasked oracle is far away (the mask acts);
  * the LeVJEPA shape: 2 clips of 1 + 16 x 14 x 14 = 3137 rows, ViT-L heads (16 x 64), on
    sampled rows (the CLS, both sides of every slot boundary, the last row, random rows);
  * one slot and no CLS row: bit-identical to jepa_attention (the mask keeps every key);
  * causality, bit for bit: changing the keys and values of later slots leaves the patch
    rows of the first slot unchanged (the CLS row moves), changing the CLS key and value
    leaves every patch row unchanged;
  * growing key norms, so that the lazy rescale runs on tiles that straddle a slot limit;
  * argument errors.
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import assert_bf16_gate, assert_f32_gate, banner, bf16, f32, host
from oracle import metrics

pytestmark = pytest.mark.gpu


def _positions(n_cls, grid, ref_grid):
    _, gh, gw = grid
    ntot = grid[0] * gh * gw
    pos = oracle.rope_positions(np.arange(ntot), gh, gw, ref_grid)
    return np.concatenate([np.zeros((n_cls, 3)), pos])


def _ref(qkv, n_cls, grid, H, hd, layout, ref_grid, rows=None, masked=True):
    B, N, _ = qkv.shape
    D = H * hd
    pos = _positions(n_cls, grid, ref_grid)
    vis = oracle.block_causal_mask(N, n_cls, grid[1] * grid[2]) if masked else None
    out = []
    for b in range(B):
        q, k, v = qkv[b, :, :D], qkv[b, :, D:2 * D], qkv[b, :, 2 * D:]
        out.append(oracle.attention(q, k, v, H, pos, pos, layout, rows=rows, visible=vis))
    return np.stack(out)


def _run(qkv, n_cls, grid, H, hd, layout, ref_grid, dt):
    import torch
    B, N, _ = qkv.shape
    D = H * hd
    if dt == "bf16":
        qd = bf16(qkv.reshape(B * N, 3 * D))
        od = torch.empty((B * N, D), dtype=torch.bfloat16, device="cuda:0")
    else:
        qd = f32(qkv.reshape(B * N, 3 * D))
        od = torch.empty((B * N, D), dtype=torch.float32, device="cuda:0")
    J.jepa_attention_block_causal(qd, od, B, n_cls, H, hd, grid, layout, ref_grid=ref_grid)
    return host(od).reshape(B, N, D)


def _inputs(B, N, D, seed, dt):
    qkv = np.random.default_rng(seed).standard_normal((B, N, 3 * D)).astype(np.float32)
    return synth.round_to_bf16(qkv) if dt == "bf16" else qkv


CASES = [
    # name, B, n_cls, grid, n_head, hd, layout, ref_grid, dtype
    ("hd64 bf16 cls ragged", 2, 1, (3, 5, 7), 2, 64, "tiled", 0, "bf16"),
    ("hd32 bf16 interleaved interp", 1, 1, (4, 9, 11), 3, 32, "interleaved", 16, "bf16"),
    ("hd64 bf16 no cls tile-sized slots", 1, 0, (5, 8, 8), 2, 64, "tiled", 0, "bf16"),
    ("hd64 bf16 three cls", 1, 3, (6, 10, 10), 2, 64, "interleaved", 0, "bf16"),
    ("hd64 bf16 slots of 4", 1, 1, (40, 2, 2), 2, 64, "tiled", 0, "bf16"),
    ("hd64 bf16 1537 rows", 1, 1, (6, 16, 16), 2, 64, "tiled", 0, "bf16"),
    ("hd64 f32 cls", 2, 1, (3, 4, 5), 2, 64, "tiled", 0, "f32"),
    ("hd32 f32 two cls interp", 1, 2, (2, 6, 6), 3, 32, "interleaved", 16, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_causal(case):
    name, B, n_cls, grid, H, hd, layout, ref_grid, dt = case
    banner("block-causal attention", name, B, n_cls, grid, H, hd, layout, ref_grid, dt)
    N = n_cls + grid[0] * grid[1] * grid[2]
    qkv = _inputs(B, N, H * hd, N + H, dt)
    got = _run(qkv, n_cls, grid, H, hd, layout, ref_grid, dt)
    ref = _ref(qkv.astype(np.float64), n_cls, grid, H, hd, layout, ref_grid)
    if dt == "bf16":
        assert_bf16_gate(got, ref, name)
    else:
        assert_f32_gate(got, ref, name, bound=1e-5)
    unmasked = _ref(qkv.astype(np.float64), n_cls, grid, H, hd, layout, ref_grid, masked=False)
    assert metrics.rel_max(got, unmasked) > 5e-2


def test_block_causal_levjepa_shape():
    # 16 frames of 224 px at tubelet 1: 16 slots of 14 x 14 patch tokens after one CLS row
    B, n_cls, grid, H, hd = 2, 1, (16, 14, 14), 16, 64
    banner("block-causal attention LeVJEPA shape", B, grid, H, hd)
    slot = grid[1] * grid[2]
    N = n_cls + grid[0] * slot
    assert N == 3137
    qkv = _inputs(B, N, H * hd, 3137, "bf16")
    got = _run(qkv, n_cls, grid, H, hd, "tiled", 0, "bf16")
    edges = [n_cls + t * slot + d for t in range(1, grid[0]) for d in (-1, 0)]
    rows = np.unique(np.r_[0, 1, 2, edges, N - 1,
                           np.random.default_rng(5).choice(N, 24, replace=False)])
    ref = _ref(qkv.astype(np.float64), n_cls, grid, H, hd, "tiled", 0, rows=rows)
    assert_bf16_gate(got[:, rows], ref, "LeVJEPA 3137 rows (sampled)")
    assert np.isfinite(got).all()


def test_block_causal_growing_scores():
    # key norms grow along the clip: later key tiles raise a query's running maximum past
    # the kernel's lazy-rescale threshold, so tiles that straddle a slot limit get their
    # scores formed a second time and masked again
    B, n_cls, grid, H, hd = 1, 1, (6, 10, 10), 2, 64
    banner("block-causal attention growing scores", B, n_cls, grid, H, hd)
    N, D = n_cls + grid[0] * grid[1] * grid[2], H * hd
    rng = np.random.default_rng(33)
    qkv = rng.standard_normal((B, N, 3 * D))
    qkv[..., :D] *= 2.0
    qkv[..., D:2 * D] *= (4.0 * np.arange(N) / N)[:, None]
    qkv = synth.round_to_bf16(qkv.astype(np.float32))
    got = _run(qkv, n_cls, grid, H, hd, "tiled", 0, "bf16")
    ref = _ref(qkv.astype(np.float64), n_cls, grid, H, hd, "tiled", 0)
    assert_bf16_gate(got, ref, "block-causal growing scores")
    unmasked = _ref(qkv.astype(np.float64), n_cls, grid, H, hd, "tiled", 0, masked=False)
    assert metrics.rel_max(got, unmasked) > 5e-2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_one_slot_equals_unmasked(dt):
    import torch
    B, grid, H, hd = 2, (1, 20, 24), 2, 64
    banner("block-causal one slot == unmasked", dt)
    N, D = 480, 128
    qkv = _inputs(B, N, D, 11, dt)
    got = _run(qkv, 0, grid, H, hd, "tiled", 0, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    qd = (bf16 if dt == "bf16" else f32)(qkv.reshape(B * N, 3 * D))
    od = torch.empty((B * N, D), dtype=tdt, device="cuda:0")
    J.jepa_attention(qd, od, B, N, H, hd, None, grid, "tiled")
    np.testing.assert_array_equal(got, host(od).reshape(B, N, D))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_causality_bitwise(dt):
    B, n_cls, grid, H, hd = 1, 1, (5, 12, 12), 2, 64
    banner("block-causal causality", dt)
    slot = grid[1] * grid[2]
    N, D = n_cls + grid[0] * slot, H * hd
    qkv = _inputs(B, N, D, 13, dt)
    base = _run(qkv, n_cls, grid, H, hd, "tiled", 0, dt)
    later = qkv.copy()
    later[:, n_cls + slot:, D:] = _inputs(B, N - n_cls - slot, D, 14, dt)[:, :, D:] * 3
    moved = _run(later, n_cls, grid, H, hd, "tiled", 0, dt)
    np.testing.assert_array_equal(moved[:, n_cls:n_cls + slot], base[:, n_cls:n_cls + slot])
    assert np.abs(moved[:, n_cls + slot:] - base[:, n_cls + slot:]).max() > 1e-2
    cls = qkv.copy()
    cls[:, :n_cls, D:] = _inputs(B, n_cls, D, 15, dt)[:, :, D:] * 3
    c = _run(cls, n_cls, grid, H, hd, "tiled", 0, dt)
    np.testing.assert_array_equal(c[:, n_cls:], base[:, n_cls:])
    assert np.abs(c[:, :n_cls] - base[:, :n_cls]).max() > 1e-2


def test_block_causal_errors():
    import torch
    banner("block-causal errors")
    qkv = torch.zeros((65 + 8, 3 * 128), dtype=torch.bfloat16, device="cuda:0")
    out = torch.zeros((65 + 8, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(J.JepaError):      # at most 63 CLS rows
        J.jepa_attention_block_causal(qkv, out, 1, 65, 2, 64, (2, 2, 2), "tiled")
    q48 = torch.zeros((9, 3 * 96), dtype=torch.bfloat16, device="cuda:0")
    o48 = torch.zeros((9, 96), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(J.JepaError):      # head dim 48
        J.jepa_attention_block_causal(q48, o48, 1, 1, 2, 48, (2, 2, 2), "tiled")
    with pytest.raises(J.JepaError):      # interpolation needs sides of at least 2
        J.jepa_attention_block_causal(qkv[:9], out[:9], 1, 1, 2, 64, (8, 1, 1), "tiled", ref_grid=16)
