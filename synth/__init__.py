"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path's tests/bench.

This module draws numbers and nothing else: it holds none of the encoder's arithmetic
(no normalisation, patchify, RoPE, LayerNorm, attention or GELU).  Both sides receive
the arrays it returns; neither side imports the other.

Recipe (one numpy PCG64 stream per tensor, ``default_rng([seed, k])`` with ``k`` the
tensor's index in a fixed name order):
  * pixels: uint8 uniform over [0, 255], laid out [B, T, H, W, 3] (frames, THWC);
  * token activations: N(0, 1) float32;
  * linear weights N(0, 0.02), linear biases N(0, 0.01), modality/mask tokens N(0, 0.02);
  * LayerNorm weight 1 and bias 0 (``ln="identity"``), or, for parity tests that must
    see the affine terms, weight 1 + N(0, 0.1) and bias N(0, 0.1) (``ln="random"``);
  * for the bf16 workloads every drawn tensor is rounded once to bf16
    (round-to-nearest-even) and handed to both sides as the same float32 values;
  * "sharp attention" variants (``qkv_scale`` s > 1) draw the fused q/k/v projection
    weights with std 0.02 s (the same stream times s, before the bf16 rounding).  With
    std 0.02 on width-1024 rows the attention scores have a std of about 0.4, the softmax
    is almost flat and the attention branch is small next to the residual, so a wrong or
    missing rotation barely moves the output; at s = 2 to 3 the scores spread over several
    units and such mistakes show.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------- helpers


def rng(seed: int, k: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(k)])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


# --------------------------------------------------------------------------- shapes


@dataclasses.dataclass(frozen=True)
class EncoderShape:
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    patch: int = 16
    tubelet: int = 2
    in_chans: int = 3
    has_mod_embed: bool = False
    final_norm: bool = True
    has_image_embed: bool = False   # V-JEPA 2.1 image path: patch_embed_img (+ mod_embed_img)


@dataclasses.dataclass(frozen=True)
class PredictorShape:
    enc_dim: int
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    n_mask_tokens: int
    out_dim: int
    has_mod_embed: bool = False      # V-JEPA 2.1: pred.mod_embed_video / _img
    has_proj_context: bool = False   # V-JEPA 2.1: pred.proj_context


@dataclasses.dataclass(frozen=True)
class HeadShape:
    """Attentive-pool classifier head: width, pool blocks, heads, FFN width, classes."""
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    n_classes: int


def _block_tensors(prefix: str, d: int, f: int) -> List[Tuple[str, Tuple[int, ...], str]]:
    return [
        (f"{prefix}.ln1.weight", (d,), "lnw"),
        (f"{prefix}.ln1.bias", (d,), "lnb"),
        (f"{prefix}.attn_qkv.weight", (3 * d, d), "w"),
        (f"{prefix}.attn_qkv.bias", (3 * d,), "b"),
        (f"{prefix}.attn_out.weight", (d, d), "w"),
        (f"{prefix}.attn_out.bias", (d,), "b"),
        (f"{prefix}.ln2.weight", (d,), "lnw"),
        (f"{prefix}.ln2.bias", (d,), "lnb"),
        (f"{prefix}.ffn_up.weight", (f, d), "w"),
        (f"{prefix}.ffn_up.bias", (f,), "b"),
        (f"{prefix}.ffn_down.weight", (d, f), "w"),
        (f"{prefix}.ffn_down.bias", (d,), "b"),
    ]


def encoder_tensor_list(s: EncoderShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) in generation order; names follow the GGUF tensor map."""
    feat = s.in_chans * s.tubelet * s.patch * s.patch
    out = [("enc.patch_embed.weight", (s.embed_dim, feat), "w"),
           ("enc.patch_embed.bias", (s.embed_dim,), "b")]
    if s.has_mod_embed:
        out.append(("enc.mod_embed_video", (s.embed_dim,), "tok"))
    for i in range(s.n_layer):
        out += _block_tensors(f"enc.blk.{i}", s.embed_dim, s.ffn_dim)
    if s.final_norm:
        out += [("enc.norm.weight", (s.embed_dim,), "lnw"), ("enc.norm.bias", (s.embed_dim,), "lnb")]
    # appended last, so the tensors above keep their streams
    if s.has_image_embed:
        out += [("enc.patch_embed_img.weight", (s.embed_dim, s.in_chans * s.patch * s.patch), "w"),
                ("enc.patch_embed_img.bias", (s.embed_dim,), "b")]
        if s.has_mod_embed:
            out.append(("enc.mod_embed_img", (s.embed_dim,), "tok"))
    return out


def predictor_tensor_list(s: PredictorShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    out = [("pred.embed.weight", (s.embed_dim, s.enc_dim), "w"),
           ("pred.embed.bias", (s.embed_dim,), "b"),
           ("pred.mask_tokens", (s.n_mask_tokens, s.embed_dim), "tok")]
    for i in range(s.n_layer):
        out += _block_tensors(f"pred.blk.{i}", s.embed_dim, s.ffn_dim)
    out += [("pred.norm.weight", (s.embed_dim,), "lnw"), ("pred.norm.bias", (s.embed_dim,), "lnb"),
            ("pred.proj.weight", (s.out_dim, s.embed_dim), "w"),
            ("pred.proj.bias", (s.out_dim,), "b")]
    # appended last, so the tensors above keep their streams
    if s.has_mod_embed:
        out += [("pred.mod_embed_video", (s.embed_dim,), "tok"), ("pred.mod_embed_img", (s.embed_dim,), "tok")]
    if s.has_proj_context:
        out += [("pred.proj_context.weight", (s.out_dim, s.embed_dim), "w"),
                ("pred.proj_context.bias", (s.out_dim,), "b")]
    return out


def head_tensor_list(s: HeadShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    d, f = s.embed_dim, s.ffn_dim
    out = [("head.query", (1, d), "tok")]
    for i in range(s.n_layer):
        out += _block_tensors(f"head.blk.{i}", d, f)
    out += [("head.xattn.ln_kv.weight", (d,), "lnw"), ("head.xattn.ln_kv.bias", (d,), "lnb")]
    for p in ("q", "k", "v"):
        out += [(f"head.xattn.{p}.weight", (d, d), "w"), (f"head.xattn.{p}.bias", (d,), "b")]
    out += [("head.xattn.ln2.weight", (d,), "lnw"), ("head.xattn.ln2.bias", (d,), "lnb"),
            ("head.xattn.ffn_up.weight", (f, d), "w"), ("head.xattn.ffn_up.bias", (f,), "b"),
            ("head.xattn.ffn_down.weight", (d, f), "w"), ("head.xattn.ffn_down.bias", (d,), "b"),
            ("head.cls.weight", (s.n_classes, d), "w"), ("head.cls.bias", (s.n_classes,), "b")]
    return out


def _draw(kind: str, shape, g: np.random.Generator, ln: str) -> np.ndarray:
    if kind == "w":
        a = g.standard_normal(shape) * 0.02
    elif kind == "b":
        a = g.standard_normal(shape) * 0.01
    elif kind == "tok":
        a = g.standard_normal(shape) * 0.02
    elif kind == "lnw":
        a = np.ones(shape) if ln == "identity" else 1.0 + 0.1 * g.standard_normal(shape)
    elif kind == "lnb":
        a = np.zeros(shape) if ln == "identity" else 0.1 * g.standard_normal(shape)
    else:
        raise ValueError(kind)
    return a.astype(np.float32)


def make_weights(tensors, seed: int, dtype: str = "bf16", ln: str = "identity",
                 base_index: int = 1000, qkv_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Draw every tensor of ``tensors`` (from *_tensor_list).  float32 arrays; bf16-valued
    when ``dtype == 'bf16'``.  ``qkv_scale`` multiplies the draws of every
    ``*.attn_qkv.weight`` before the rounding (sharp-attention variants)."""
    out = {}
    for k, (name, shape, kind) in enumerate(tensors):
        a = _draw(kind, shape, rng(seed, base_index + k), ln)
        if qkv_scale != 1.0 and name.endswith(".attn_qkv.weight"):
            a = (a * np.float32(qkv_scale)).astype(np.float32)
        if dtype == "bf16":
            a = round_to_bf16(a)
        out[name] = a
    return out


def encoder_weights(s: EncoderShape, seed: int = 0, dtype: str = "bf16", ln: str = "identity",
                    qkv_scale: float = 1.0):
    return make_weights(encoder_tensor_list(s), seed, dtype, ln, base_index=1000, qkv_scale=qkv_scale)


def head_weights(s: HeadShape, seed: int = 0, dtype: str = "bf16", ln: str = "identity"):
    return make_weights(head_tensor_list(s), seed, dtype, ln, base_index=9000)


def predictor_weights(s: PredictorShape, seed: int = 0, dtype: str = "bf16", ln: str = "identity",
                      qkv_scale: float = 1.0):
    return make_weights(predictor_tensor_list(s), seed, dtype, ln, base_index=5000, qkv_scale=qkv_scale)


# --------------------------------------------------------------------------- activations


def clip_u8(seed: int, B: int, T: int, H: int, W: int, C: int = 3, k: int = 1) -> np.ndarray:
    """Uniform uint8 frames, [B, T, H, W, C]."""
    return rng(seed, k).integers(0, 256, size=(B, T, H, W, C), dtype=np.uint8)


def tokens_normal(seed: int, B: int, N: int, D: int, k: int = 2) -> np.ndarray:
    return rng(seed, k).standard_normal((B, N, D)).astype(np.float32)


def normal(seed: int, shape, k: int, scale: float = 1.0) -> np.ndarray:
    return (rng(seed, k).standard_normal(shape) * scale).astype(np.float32)


def tube_mask(seed: int, gt: int, gh: int, gw: int, bh: int = 8, bw: int = 8,
              k: int = 3) -> Tuple[np.ndarray, np.ndarray]:
    """Seeded spatiotemporal block ("tube") mask on a T-major grid.

    One spatial block of bh x bw patches, its corner drawn uniformly, is kept in every
    temporal slot: those ids are the context (ascending), the rest are targets
    (ascending).  Returns int32 (ids_ctx, ids_tgt)."""
    g = rng(seed, k)
    h0 = int(g.integers(0, gh - bh + 1))
    w0 = int(g.integers(0, gw - bw + 1))
    keep = np.zeros((gt, gh, gw), dtype=bool)
    keep[:, h0:h0 + bh, w0:w0 + bw] = True
    flat = keep.reshape(-1)
    ids = np.arange(flat.size, dtype=np.int32)
    return ids[flat], ids[~flat]


def context_ids(seed: int, B: int, N: int, K: int, k: int = 4) -> np.ndarray:
    """Seeded context ids of the masked-encoder forward: for each of B clips, K distinct
    grid ids in [0, N) in random order.  int32 [B, K]."""
    g = rng(seed, k)
    return np.stack([g.permutation(N)[:K] for _ in range(B)]).astype(np.int32)


# --------------------------------------------------------------------------- workloads

# The five workloads of the build, by what they are.  ``grid`` is (t, h, w) in
# tokens; ``frames``/``size`` give the uint8 clip when the workload starts from pixels.
WORKLOADS = {
    "tiny_fp32": dict(
        desc="tiny V-JEPA-2-style encoder, fp32, 1 clip x 4 frames x 64x64",
        enc=EncoderShape(768, 2, 12, 3072), layout="tiled", ref_grid=0, dtype="f32",
        B=1, frames=4, size=64, grid=(2, 4, 4)),
    "vitl_block": dict(
        desc="one V-JEPA 2 ViT-L block on [1, 2048, 1024] N(0,1) tokens, bf16",
        enc=EncoderShape(1024, 1, 16, 4096, final_norm=False), layout="tiled", ref_grid=0,
        dtype="bf16", B=1, frames=None, size=None, grid=(8, 16, 16)),
    "vitl16_16f256": dict(
        desc="V-JEPA 2 ViT-L/16 encoder, 4 clips x 16 frames x 256x256, bf16",
        enc=EncoderShape(1024, 24, 16, 4096), layout="tiled", ref_grid=0, dtype="bf16",
        B=4, frames=16, size=256, grid=(8, 16, 16)),
    "vitb16_64f384": dict(
        desc="V-JEPA 2.1 ViT-B/16 encoder, 1 clip x 64 frames x 384x384, bf16",
        enc=EncoderShape(768, 12, 12, 3072, has_mod_embed=True), layout="interleaved",
        ref_grid=16, dtype="bf16", B=1, frames=64, size=384, grid=(32, 24, 24)),
    "vitl16_64f256_pred": dict(
        desc="V-JEPA 2 ViT-L/16 encoder, 1 clip x 64 frames x 256x256, + masked predictor, bf16",
        enc=EncoderShape(1024, 24, 16, 4096), layout="tiled", ref_grid=0, dtype="bf16",
        B=1, frames=64, size=256, grid=(32, 16, 16),
        pred=PredictorShape(1024, 384, 12, 12, 1536, 10, 1024), mask_index=1),
    "vitb16_img384": dict(
        desc="V-JEPA 2.1 ViT-B/16 native image path, 1 image 384x384 (576 tokens), bf16",
        enc=EncoderShape(768, 12, 12, 3072, has_mod_embed=True, has_image_embed=True),
        layout="interleaved", ref_grid=16, dtype="bf16", B=1, frames=1, size=384, grid=(1, 24, 24)),
    "vitb16_pred21": dict(
        desc="V-JEPA 2.1 ViT-B predictor (384 / 12 / 12 / 1536, 8 mask tokens, out 1664, "
             "modality vectors, context projection) on the grid of 384 px (24 x 24 per slot), bf16",
        pred=PredictorShape(768, 384, 12, 12, 1536, 8, 1664, has_mod_embed=True, has_proj_context=True),
        layout="interleaved", dtype="bf16", mask_index=1, grid_video=(8, 24, 24), grid_image=(1, 24, 24)),
}


def workload(name: str) -> dict:
    return dict(WORKLOADS[name])


def scaled(w: dict, n_layer: Optional[int] = None) -> dict:
    """The same workload with a different encoder depth (same per-layer shapes)."""
    w = dict(w)
    if n_layer is not None:
        w["enc"] = dataclasses.replace(w["enc"], n_layer=n_layer)
    return w
