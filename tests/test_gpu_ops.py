"""Parity of the stand-alone entry points (jepa_rope3d, jepa_layernorm, jepa_linear,
jepa_attention) against the oracle, through the C ABI, on seeded inputs.

Sizes span several tiles and a ragged tail (GEMM rows not a multiple of 256, token
counts not a multiple of the 128-query / 64-key attention tiles), plus every
workload's real token grid for the RoPE.  Gates: RoPE fp32 max |diff| <= 1e-5; bf16
outputs within one bf16 rounding (2^-8 relative) of the oracle evaluated on the same
bf16-valued inputs; attention on the bf16 path at the bf16 gate (mean cosine >= 0.9999,
rel_max <= 2e-2).
"""
import numpy as np
import pytest

import oracle
import synth
import video_vit_encoder_amd as J
from gpu_helpers import (ROPE_F32_MAX_ABS, assert_bf16_gate, assert_f32_gate, banner, bf16, f32,
                         host, i32)
from oracle import metrics

pytestmark = pytest.mark.gpu

BF16_ULP = 2.0 ** -8


def _rope_ref(x, B, N, H, hd, ids, grid, layout, ref_grid):
    """oracle RoPE of x [B, N, H*hd] (float64)."""
    _, gh, gw = grid
    pos = oracle.rope_positions(ids, gh, gw, ref_grid)
    u = x.reshape(B, N, H, hd).transpose(0, 2, 1, 3)          # [B, H, N, hd]
    r = oracle.rope_rotate(u, pos, layout)
    return r.transpose(0, 2, 1, 3).reshape(B, N, H * hd)


ROPE_CASES = [
    # (name, grid, n_head, head_dim, layout, ref_grid, B, use_ids)
    ("tiny_fp32 grid", (2, 4, 4), 12, 64, "tiled", 0, 1, False),
    ("vitl 16f grid", (8, 16, 16), 16, 64, "tiled", 0, 2, False),
    ("vitb 2.1 384 grid", (32, 24, 24), 12, 64, "interleaved", 16, 1, False),
    ("predictor grid", (32, 16, 16), 12, 32, "tiled", 0, 1, True),
    ("interleaved hd32", (3, 5, 7), 3, 32, "interleaved", 0, 2, True),
    ("tiled + interp", (5, 6, 4), 2, 64, "tiled", 16, 1, False),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope3d_f32(case):
    name, grid, H, hd, layout, ref_grid, B, use_ids = case
    banner("rope3d f32", name, grid, H, hd, layout, ref_grid)
    ntot = grid[0] * grid[1] * grid[2]
    rng = np.random.default_rng(11)
    if use_ids:
        ids = rng.permutation(ntot)[: ntot - 5].astype(np.int32)   # ragged, shuffled ids
    else:
        ids = np.arange(ntot, dtype=np.int32)
    N = len(ids)
    x = synth.normal(1, (B, N, H * hd), k=20)
    xd = f32(x)
    yd = f32(np.zeros_like(x))
    J.jepa_rope3d(xd, yd, B, N, H, hd, H * hd, i32(ids) if use_ids else None, grid, layout,
                  ref_grid=ref_grid)
    got = host(yd)
    ref = _rope_ref(x.astype(np.float64), B, N, H, hd, ids, grid, layout, ref_grid)
    err = metrics.max_abs(got, ref)
    print(f"  max_abs={err:.3e}")
    assert err <= ROPE_F32_MAX_ABS
    # pass-through dims are copied bit for bit
    d = oracle.rope_axis_dim(hd)
    g4 = got.reshape(B, N, H, hd)[..., 3 * d:]
    x4 = x.reshape(B, N, H, hd)[..., 3 * d:]
    assert np.array_equal(g4.astype(np.float32), x4)


def test_rope3d_in_place_strided_and_layout_swap_fails():
    banner("rope3d in-place strided qkv rows")
    grid, H, hd, B = (4, 6, 6), 4, 64, 2
    N = 144
    D = H * hd
    rng = np.random.default_rng(3)
    x = rng.standard_normal((B, N, 3 * D)).astype(np.float32)   # q | k | v rows
    xd = f32(x)
    # rotate the k third in place, rows of stride 3D
    kview = xd.view(-1)[D:]
    J.jepa_rope3d(kview, kview, B, N, H, hd, 3 * D, None, grid, "tiled")
    got = host(xd)
    ids = np.arange(N)
    ref_k = _rope_ref(x[..., D:2 * D].astype(np.float64), B, N, H, hd, ids, grid, "tiled", 0)
    assert metrics.max_abs(got[..., D:2 * D], ref_k) <= ROPE_F32_MAX_ABS
    assert np.array_equal(got[..., :D].astype(np.float32), x[..., :D])       # q untouched
    assert np.array_equal(got[..., 2 * D:].astype(np.float32), x[..., 2 * D:])  # v untouched
    # negative control: the other layout's oracle is far outside the gate
    wrong = _rope_ref(x[..., D:2 * D].astype(np.float64), B, N, H, hd, ids, grid, "interleaved", 0)
    assert metrics.max_abs(got[..., D:2 * D], wrong) > 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope3d_pair_path_unaligned_rows_and_head_dim_6(dtype):
    # rows starting 2 elements past an aligned address, and a head dim (6: 2 rotated dims
    # per axis, no pass-through) that is not a multiple of 4, take the pair-at-a-time path
    import torch
    banner("rope3d pair path", dtype)
    for hd, off in ((64, 2), (6, 0)):
        grid, H, B = (3, 5, 6), 3, 2
        N = 90
        D = H * hd
        x = synth.normal(4, (B * N * D + 2,), k=22)
        if dtype == "bf16":
            x = synth.round_to_bf16(x)
        xd = (bf16 if dtype == "bf16" else f32)(x)
        yd = torch.zeros_like(xd)
        J.jepa_rope3d(xd[off:], yd[off:], B, N, H, hd, D, None, grid, "interleaved", ref_grid=16)
        got = host(yd)[off:off + B * N * D].reshape(B, N, D)
        ref = _rope_ref(x[off:off + B * N * D].astype(np.float64).reshape(B, N, D), B, N, H, hd,
                        np.arange(N), grid, "interleaved", 16)
        if dtype == "bf16":
            assert np.all(np.abs(got - ref) <= BF16_ULP * np.abs(ref) + 1e-6), hd
        else:
            assert metrics.max_abs(got, ref) <= ROPE_F32_MAX_ABS, hd


def test_rope3d_bf16():
    banner("rope3d bf16")
    grid, H, hd, B = (8, 16, 16), 16, 64, 1
    N = 2048
    x = synth.round_to_bf16(synth.normal(2, (B, N, H * hd), k=21))
    xd = bf16(x)
    yd = bf16(np.zeros_like(x))
    J.jepa_rope3d(xd, yd, B, N, H, hd, H * hd, None, grid, "tiled")
    got = host(yd)
    ref = _rope_ref(x.astype(np.float64), B, N, H, hd, np.arange(N), grid, "tiled", 0)
    assert np.all(np.abs(got - ref) <= BF16_ULP * np.abs(ref) + 1e-6)


def test_rope3d_empty_and_errors():
    banner("rope3d empty + errors")
    xd = f32(np.zeros((1, 4, 64)))
    J.jepa_rope3d(xd, xd, 0, 4, 1, 64, 64, None, (1, 2, 2), "tiled")   # B = 0: no-op
    J.jepa_rope3d(xd, xd, 1, 0, 1, 64, 64, None, (1, 2, 2), "tiled")   # N = 0: no-op
    with pytest.raises(J.JepaError):   # interpolation on a grid side of 1
        J.jepa_rope3d(xd, xd, 1, 4, 1, 64, 64, None, (4, 1, 1), "tiled", ref_grid=16)
    with pytest.raises(J.JepaError):   # more tokens than the grid holds, no ids
        J.jepa_rope3d(xd, xd, 1, 4, 1, 64, 64, None, (1, 1, 2), "tiled")


@pytest.mark.parametrize("D,M,out", [(1024, 2048 + 37, "f32"), (768, 301, "bf16"),
                                     (384, 130, "bf16"), (1024, 5, "bf16"), (768, 64, "f32"),
                                     # two rows per wavefront (half-wave rows, 16-byte chunks),
                                     # an odd row count leaving the last half wave idle
                                     (384, 8192 + 3, "f32"), (640, 77, "bf16"), (128, 9, "f32"),
                                     (1408, 33, "bf16")])
def test_layernorm(D, M, out):
    import torch
    banner("layernorm", D, M, out)
    rng = np.random.default_rng(D + M)
    x = (rng.standard_normal((M, D)) * 3 + rng.standard_normal((M, 1)) * 2).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32)
    od = torch.empty((M, D), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                     device="cuda:0")
    J.jepa_layernorm(f32(x), f32(w), f32(b), 1e-6, od)
    got = host(od)
    ref = oracle.layer_norm(x.astype(np.float64), w, b, 1e-6)
    if out == "f32":
        assert metrics.rel_max(got, ref) <= 2e-6
    else:
        assert np.all(np.abs(got - ref) <= BF16_ULP * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("D", [1024, 384])   # a row per wavefront; two per wavefront
def test_layernorm_in_place(D):
    banner("layernorm in place", D)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((77, D)).astype(np.float32)
    xd = f32(x)
    ones, zeros = f32(np.ones(D)), f32(np.zeros(D))
    J.jepa_layernorm(xd, ones, zeros, 1e-6, xd)
    ref = oracle.layer_norm(x.astype(np.float64), np.ones(D), np.zeros(D), 1e-6)
    assert metrics.rel_max(host(xd), ref) <= 2e-6


LINEAR_CASES = [
    # M, N, K, epilogue, out
    (300, 384, 1024, J.JEPA_EPI_STORE, "bf16"),
    (2048 + 77, 3072, 1024, J.JEPA_EPI_STORE, "bf16"),
    (513, 4096, 1024, J.JEPA_EPI_GELU, "bf16"),
    (700, 1024, 4096, J.JEPA_EPI_RESIDUAL, "f32"),
    (33, 768, 1536, J.JEPA_EPI_STORE, "f32"),
    (1, 128, 64, J.JEPA_EPI_GELU, "f32"),
    # full-height shapes of the 4-clip ViT-L forward with a ragged last row tile: they take
    # the 256x256 (N = 4096) and 256x192 (N = 3072) tiles
    (8192 - 5, 4096, 1024, J.JEPA_EPI_GELU, "bf16"),
    (8192 - 77, 3072, 1024, J.JEPA_EPI_STORE, "bf16"),
    (8192 - 130, 1024, 4096, J.JEPA_EPI_RESIDUAL, "f32"),
    # fewer 256 x 128 tiles than CUs (216), yet one round of them beats 1.7 rounds of
    # 128 x 128 tiles: the 2.1 image path's down-projection shape, ragged
    (9216 - 19, 768, 3072, J.JEPA_EPI_RESIDUAL, "f32"),
    # 2048 rows (the masked forward) at N = 1024: one round of 256 tiles of 128 x 64, ragged
    (2048 - 3, 1024, 4096, J.JEPA_EPI_RESIDUAL, "f32"),
    (2048 - 3, 1024, 1024, J.JEPA_EPI_STORE, "bf16"),
    # shallow K with many tiles per workgroup: K = 64 (one slab per tile) on 256x256 tiles
    # (4 tiles per CU) and K = 128 on 256x128 tiles (3-slab ring, 2-3 tiles per CU); every
    # tile's bias must be its own although the slab ring runs several tiles ahead
    (65536 - 3, 1024, 64, J.JEPA_EPI_STORE, "f32"),
    (140000, 128, 128, J.JEPA_EPI_GELU, "bf16"),
]


@pytest.mark.parametrize("M,N,K,epi,out", LINEAR_CASES)
def test_linear_bf16(M, N, K, epi, out):
    import torch
    banner("linear bf16", M, N, K, epi, out)
    rng = np.random.default_rng(M * 7 + N)
    A = synth.round_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    W = synth.round_to_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = (rng.standard_normal(N) * 0.01).astype(np.float32)
    ref = oracle.linear(A.astype(np.float64), W, bias)
    if epi == J.JEPA_EPI_GELU:
        ref = oracle.gelu_erf(ref)
    if epi == J.JEPA_EPI_RESIDUAL:
        C0 = rng.standard_normal((M, N)).astype(np.float32)
        Cd = f32(C0)
        ref = ref + C0
    else:
        Cd = torch.empty((M, N), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                         device="cuda:0")
    J.jepa_linear(bf16(A), bf16(W), f32(bias), Cd, epi)
    got = host(Cd)
    if out == "bf16":
        assert np.all(np.abs(got - ref) <= BF16_ULP * np.abs(ref) + 1e-4 * np.abs(ref).max())
    else:
        assert metrics.rel_max(got, ref) <= 1e-5


@pytest.mark.parametrize("M,N,K,epi", [(37, 768, 1536, J.JEPA_EPI_STORE),
                                       (32, 3072, 768, J.JEPA_EPI_GELU),
                                       (100, 768, 3072, J.JEPA_EPI_RESIDUAL)])
def test_linear_f32(M, N, K, epi):
    banner("linear f32", M, N, K, epi)
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.01).astype(np.float32)
    ref = oracle.linear(A.astype(np.float64), W, bias)
    if epi == J.JEPA_EPI_GELU:
        ref = oracle.gelu_erf(ref)
    C0 = rng.standard_normal((M, N)).astype(np.float32) if epi == J.JEPA_EPI_RESIDUAL else np.zeros((M, N), np.float32)
    if epi == J.JEPA_EPI_RESIDUAL:
        ref = ref + C0
    Cd = f32(C0)
    J.jepa_linear(f32(A), f32(W), f32(bias), Cd, epi)
    assert metrics.rel_max(host(Cd), ref) <= 1e-5


ATTN_CASES = [
    # name, B, grid, n_head, hd, layout, ref_grid, ids mode, dtype
    ("hd64 tiled ragged", 2, (2, 10, 10), 3, 64, "tiled", 0, None, "bf16"),
    ("hd64 interleaved interp", 1, (3, 9, 11), 2, 64, "interleaved", 16, None, "bf16"),
    ("hd32 tiled shuffled ids", 1, (4, 8, 8), 4, 32, "tiled", 0, "perm", "bf16"),
    ("hd64 one tile", 1, (1, 2, 3), 2, 64, "tiled", 0, None, "bf16"),
    ("hd64 two 2048-token clips", 2, (8, 16, 16), 2, 64, "tiled", 0, None, "bf16"),
    ("hd32 interleaved 1000 tokens", 1, (10, 10, 10), 3, 32, "interleaved", 16, None, "bf16"),
    # the longest clip of 256-query workgroups, and the shortest of 512-query ones (ragged)
    ("hd64 1024 tokens", 1, (4, 16, 16), 2, 64, "tiled", 0, None, "bf16"),
    ("hd32 1058 tokens", 1, (2, 23, 23), 2, 32, "tiled", 0, None, "bf16"),
    # long clips with few heads: the keys of each query block go in 8 pieces (the last
    # piece short, its last tile ragged at 4205 tokens), merged at the end
    ("hd64 4205 tokens in key pieces", 1, (5, 29, 29), 2, 64, "tiled", 0, None, "bf16"),
    ("hd32 2 x 4608 tokens in key pieces", 2, (8, 24, 24), 2, 32, "interleaved", 16, None, "bf16"),
    # a ViT-L clip of 32 frames: 16 heads of 64 over 4096 tokens, keys in 2 pieces
    ("hd64 4096 tokens, 16 heads, keys in 2 pieces", 1, (16, 16, 16), 16, 64, "tiled", 0, None,
     "bf16"),
    # 4225 tokens: 8 pieces of 9 tiles but the last, of 4 tiles whose last holds one key
    ("hd32 4225 tokens, one key in the last piece's last tile", 1, (25, 13, 13), 2, 32, "tiled", 0,
     None, "bf16"),
    ("hd64 f32 tiny grid", 1, (2, 4, 4), 12, 64, "tiled", 0, None, "f32"),
    ("hd64 f32 ragged", 2, (3, 7, 5), 2, 64, "interleaved", 16, None, "f32"),
    ("hd32 f32 ids", 1, (2, 6, 6), 3, 32, "tiled", 0, "perm", "f32"),
]


def _attn_ref(qkv, B, N, H, hd, ids, grid, layout, ref_grid):
    D = H * hd
    _, gh, gw = grid
    pos = oracle.rope_positions(ids, gh, gw, ref_grid)
    out = np.zeros((B, N, D))
    for b in range(B):
        q, k, v = qkv[b, :, :D], qkv[b, :, D:2 * D], qkv[b, :, 2 * D:]
        out[b] = oracle.attention(q, k, v, H, pos, pos, layout)
    return out


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention(case):
    import torch
    name, B, grid, H, hd, layout, ref_grid, ids_mode, dt = case
    banner("attention", name, B, grid, H, hd, layout, ref_grid, dt)
    ntot = grid[0] * grid[1] * grid[2]
    rng = np.random.default_rng(ntot + H)
    ids = rng.permutation(ntot).astype(np.int32) if ids_mode == "perm" else np.arange(ntot, dtype=np.int32)
    N = ntot
    D = H * hd
    qkv = rng.standard_normal((B, N, 3 * D)).astype(np.float32)
    if dt == "bf16":
        qkv = synth.round_to_bf16(qkv)
        qd = bf16(qkv)
        od = torch.empty((B * N, D), dtype=torch.bfloat16, device="cuda:0")
    else:
        qd = f32(qkv)
        od = torch.empty((B * N, D), dtype=torch.float32, device="cuda:0")
    J.jepa_attention(qd, od, B, N, H, hd, i32(ids) if ids_mode else None, grid, layout,
                     ref_grid=ref_grid)
    got = host(od).reshape(B, N, D)
    ref = _attn_ref(qkv.astype(np.float64), B, N, H, hd, ids, grid, layout, ref_grid)
    if dt == "bf16":
        assert_bf16_gate(got, ref, name)
    else:
        assert_f32_gate(got, ref, name, bound=1e-5)
    # negative control: the other RoPE layout is far outside the gate
    other = "interleaved" if layout == "tiled" else "tiled"
    wrong = _attn_ref(qkv.astype(np.float64), B, N, H, hd, ids, grid, other, ref_grid)
    assert metrics.rel_max(got, wrong) > 5e-2


def test_attention_softmax_properties_identical_keys():
    # every key identical -> each head's output is that value row, whatever the query
    banner("attention identical keys")
    B, grid, H, hd = 1, (2, 8, 12), 2, 64
    N, D = 192, 128
    rng = np.random.default_rng(9)
    qkv = synth.round_to_bf16(rng.standard_normal((N, 3 * D)).astype(np.float32))
    qkv[:, D:2 * D] = 0.0      # zero keys: RoPE keeps them zero, every score is 0
    vrow = qkv[0, 2 * D:].copy()
    qkv[:, 2 * D:] = vrow
    import torch
    od = torch.empty((N, D), dtype=torch.bfloat16, device="cuda:0")
    J.jepa_attention(bf16(qkv), od, B, N, H, hd, None, grid, "tiled")
    got = host(od)
    assert np.array_equal(got, np.broadcast_to(vrow.astype(np.float64), (N, D)))


@pytest.mark.parametrize("grid", [(4, 12, 16), (4, 12, 15), (4, 32, 36), (5, 29, 29)],
                         ids=["768 rows", "720 rows ragged", "4608 rows in key pieces",
                              "4205 rows ragged in key pieces"])
def test_attention_growing_scores_rescale(grid):
    # key norms grow along the clip, so later key tiles keep raising each query's running
    # maximum by more than 2^8 (the kernel's lazy-rescale threshold, in log2 units) and
    # the rescale path runs many times; the first tile's scores are small.  With 720 rows
    # the last key tile is ragged, so its scores are masked again after they are formed
    # a second time.  From 4096 rows on (two heads) the keys go in 8 pieces whose maxima
    # differ by 2^8.6 to 2^31 (median 2^15; 4608 rows, head 0), so the merge weights of
    # the early pieces are tiny.  There q is not doubled: the bf16 rounding of the rotated
    # q and k (the kernel's inputs) moves each score by an amount that grows with its
    # size, and over these longer clips the largest scores would put that error alone at
    # 2.3-2.7 % of the output's scale (exact softmax on the rounded inputs), beyond the
    # gate.
    banner("attention growing scores", grid)
    B, H, hd = 1, 2, 64
    N, D = grid[0] * grid[1] * grid[2], 128
    rng = np.random.default_rng(21)
    qkv = rng.standard_normal((N, 3 * D))
    qkv[:, :D] *= 2.0 if N < 4096 else 1.0
    qkv[:, D:2 * D] *= (4.0 * np.arange(N) / N)[:, None]
    qkv = synth.round_to_bf16(qkv.astype(np.float32))
    import torch
    od = torch.empty((N, D), dtype=torch.bfloat16, device="cuda:0")
    J.jepa_attention(bf16(qkv), od, B, N, H, hd, None, grid, "tiled")
    got = host(od).reshape(B, N, D)
    ref = _attn_ref(qkv.astype(np.float64).reshape(B, N, 3 * D), B, N, H, hd,
                    np.arange(N, dtype=np.int32), grid, "tiled", 0)
    assert_bf16_gate(got, ref, "growing scores")


def test_attention_key_pieces_batch_invariant():
    # 4608 tokens, two heads of 32: the keys of each query block go in pieces, chosen from
    # the clip length and head count only, so a clip's output is the same bits alone and
    # as the middle clip of three
    import torch
    banner("attention key pieces, batch invariance, 1 and 3 clips of 8 x 24 x 24")
    grid, H, hd = (8, 24, 24), 2, 32
    N, D = grid[0] * grid[1] * grid[2], 2 * 32
    rng = np.random.default_rng(33)
    qkv = synth.round_to_bf16(rng.standard_normal((3, N, 3 * D)).astype(np.float32))
    one = torch.empty((N, D), dtype=torch.bfloat16, device="cuda:0")
    three = torch.empty((3 * N, D), dtype=torch.bfloat16, device="cuda:0")
    J.jepa_attention(bf16(qkv[1]), one, 1, N, H, hd, None, grid, "interleaved", ref_grid=16)
    J.jepa_attention(bf16(qkv.reshape(3 * N, 3 * D)), three, 3, N, H, hd, None, grid,
                     "interleaved", ref_grid=16)
    a, b = host(one), host(three).reshape(3, N, D)[1]
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b), float(np.max(np.abs(a - b)))
