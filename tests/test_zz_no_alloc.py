"""jepa_attention_noalloc (no device allocation; the library's per-GPU scratch array)
against jepa_attention with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must agree bit for bit.
Two calls in a row, the second on a smaller input, show that what the first call left in
the shared array does not leak into the second; a third, longer clip takes its keys in
pieces, whose partial results live in the same array.  A size beyond the
array is refused with JEPA_ERR_SHAPE and leaves the output untouched.
"""
import numpy as np
import pytest

import synth
import video_vit_encoder_amd as J
from gpu_helpers import banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu


def _qkv(seed, B, N, D, dtype):
    x = synth.normal(seed, (B * N, 3 * D), k=40)
    return bf16(x) if dtype == "bf16" else f32(x)


CASES = [
    # B, grid, n_head, head_dim, layout, ref_grid, ids
    (2, (8, 16, 16), 16, 64, "tiled", 0, False),          # 2 clips x 2048 tokens, 24 MiB
    (1, (3, 10, 10), 4, 32, "interleaved", 16, True),      # ragged 300 tokens, shuffled ids
    (1, (5, 29, 29), 2, 64, "tiled", 0, False),            # 4205 tokens, keys in 8 pieces
]


def test_noalloc_matches_workspace_entry_point_twice_smaller_second():
    import torch
    for i, (B, grid, H, hd, layout, rg, with_ids) in enumerate(CASES):
        N = grid[0] * grid[1] * grid[2]
        banner("attention noalloc call", i, "B", B, "grid", grid, "heads", H, "hd", hd, layout)
        qkv = _qkv(50 + i, B, N, H * hd, "bf16")
        ids = i32(np.random.default_rng(i).permutation(N)) if with_ids else None
        ref = torch.empty((B * N, H * hd), dtype=torch.bfloat16, device="cuda:0")
        got = torch.full_like(ref, 3.0)
        J.jepa_attention(qkv, ref, B, N, H, hd, ids, grid, layout, ref_grid=rg)
        J.jepa_attention_noalloc(qkv, got, B, N, H, hd, ids, grid, layout, ref_grid=rg)
        r, g = host(ref), host(got)
        assert np.all(np.isfinite(g))
        assert np.array_equal(g, r), (i, float(np.max(np.abs(g - r))))


def test_noalloc_fp32_matches_workspace_entry_point():
    import torch
    banner("attention noalloc fp32, 1 clip x 2 x 6 x 6, 3 heads of 32")
    B, grid, H, hd = 1, (2, 6, 6), 3, 32
    N = 72
    qkv = _qkv(60, B, N, H * hd, "f32")
    ref = torch.empty((B * N, H * hd), dtype=torch.float32, device="cuda:0")
    got = torch.full_like(ref, 3.0)
    J.jepa_attention(qkv, ref, B, N, H, hd, None, grid, "tiled")
    J.jepa_attention_noalloc(qkv, got, B, N, H, hd, None, grid, "tiled")
    assert np.array_equal(host(got), host(ref))


def test_noalloc_refuses_sizes_beyond_the_scratch_array():
    import torch
    banner("attention noalloc beyond the scratch array")
    B, grid, H, hd = 4, (16, 16, 16), 16, 64       # 4 x 4096 x 1024 x 6 B = 96 MiB > 64 MiB
    N = 4096
    qkv = torch.zeros((B * N, 3 * H * hd), dtype=torch.bfloat16, device="cuda:0")
    out = torch.full((B * N, H * hd), 7.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(J.JepaError) as e:
        J.jepa_attention_noalloc(qkv, out, B, N, H, hd, None, grid, "tiled")
    assert e.value.status == J._lib.JEPA_ERR_SHAPE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
