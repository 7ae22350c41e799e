"""video_vit_encoder_amd: the V-JEPA 2 / 2.1 video ViT encoder forward (and the V-JEPA 2
masked predictor) as hand-written gfx950 HIP kernels behind the C ABI of include/jepa.h.

The functions named ``jepa_*`` are the C entry points (see ``_lib``).  ``Encoder`` and
``Predictor`` are small owners of a C handle: they upload a dict of host weights by name
and call ``jepa_encode`` / ``jepa_encode_masked`` / ``jepa_encode_tokens`` /
``jepa_predict``.  Nothing here computes any part of the forward.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from ._lib import (  # noqa: F401
    DTYPES, JEPA_BF16, JEPA_EPI_GELU, JEPA_EPI_RESIDUAL, JEPA_EPI_STORE, JEPA_F32, LAYOUTS,
    KERNEL_CLASSES, JepaError, header_functions, jepa_attention, jepa_attention_block_causal,
    jepa_attention_noalloc, jepa_attention_workspace_size,
    jepa_encode, jepa_encode_image, jepa_encode_masked, jepa_encode_tokens, jepa_predict_mod,
    jepa_head_config, jepa_head_create, jepa_head_forward, jepa_head_free, jepa_head_set_tensor,
    jepa_pool_mean,
    jepa_encoder_config, jepa_encoder_create, jepa_encoder_free, jepa_encoder_set_tensor,
    jepa_layernorm, jepa_linear, jepa_predict, jepa_predictor_config, jepa_predictor_create,
    jepa_predictor_free, jepa_predictor_set_tensor, jepa_rope3d, jepa_status_str,
    jepa_timing_begin, jepa_timing_end, jepa_version, load,
)


class Encoder:
    """Owner of a jepa_encoder handle."""

    def __init__(self, embed_dim: int, n_layer: int, n_head: int, ffn_dim: int, *,
                 layout: str = "tiled", ref_grid: int = 0, has_mod_embed: bool = False,
                 final_norm: bool = True, dtype: str = "bf16", max_rows: int = 2048,
                 ln_eps: float = 1e-6, theta: float = 10000.0, has_image_embed: bool = False):
        cfg = jepa_encoder_config(
            embed_dim=embed_dim, n_layer=n_layer, n_head=n_head, ffn_dim=ffn_dim, patch=16,
            tubelet=2, in_chans=3, rope_layout=LAYOUTS[layout], rope_ref_grid=ref_grid,
            has_mod_embed=int(has_mod_embed), final_norm=int(final_norm),
            compute=DTYPES[dtype], max_rows=max_rows, ln_eps=ln_eps, rope_theta=theta,
            has_image_embed=int(has_image_embed))
        self.cfg = cfg
        self.embed_dim = embed_dim
        self.handle = jepa_encoder_create(cfg)

    def set_weights(self, weights: Dict[str, np.ndarray]) -> None:
        for name, arr in weights.items():
            jepa_encoder_set_tensor(self.handle, name, arr)

    def encode(self, clip, out=None, stream=None):
        """clip: uint8 device tensor [B, T, H, W, 3] -> fp32 [B, N, D]."""
        import torch
        B, T, H, W, _ = clip.shape
        N = (T // 2) * (H // 16) * (W // 16)
        if out is None:
            out = torch.empty((B, N, self.embed_dim), dtype=torch.float32, device=clip.device)
        jepa_encode(self.handle, clip, out, stream)
        return out

    def encode_image(self, img, out=None, stream=None):
        """img: uint8 device tensor [B, H, W, 3] -> fp32 [B, N, D] (2.1 image path)."""
        import torch
        B, H, W, _ = img.shape
        if out is None:
            out = torch.empty((B, (H // 16) * (W // 16), self.embed_dim), dtype=torch.float32,
                              device=img.device)
        jepa_encode_image(self.handle, img, out, stream)
        return out

    def encode_masked(self, clip, ids, out=None, stream=None):
        """clip: uint8 device tensor [B, T, H, W, 3], ids: int32 device tensor [B, K] ->
        fp32 [B, K, D], the blocks run on each clip's K context tokens only."""
        import torch
        if out is None:
            out = torch.empty((clip.shape[0], ids.shape[1], self.embed_dim), dtype=torch.float32,
                              device=clip.device)
        jepa_encode_masked(self.handle, clip, ids, out, stream)
        return out

    def encode_tokens(self, x, grid: Sequence[int], ids=None, out=None, stream=None):
        """x: fp32 device tensor [B, N, D] -> fp32 [B, N, D]."""
        import torch
        if out is None:
            out = torch.empty_like(x)
        jepa_encode_tokens(self.handle, x, ids, grid, out, stream)
        return out

    def close(self) -> None:
        if getattr(self, "handle", None):
            jepa_encoder_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Head:
    """Owner of a jepa_head handle (attentive-pool classifier head)."""

    def __init__(self, embed_dim: int, n_layer: int, n_head: int, ffn_dim: int, n_classes: int, *,
                 dtype: str = "bf16", max_rows: int = 8192, ln_eps: float = 1e-6):
        cfg = jepa_head_config(embed_dim=embed_dim, n_layer=n_layer, n_head=n_head, ffn_dim=ffn_dim,
                               n_classes=n_classes, compute=DTYPES[dtype], max_rows=max_rows,
                               ln_eps=ln_eps)
        self.cfg = cfg
        self.n_classes = n_classes
        self.handle = jepa_head_create(cfg)

    def set_weights(self, weights: Dict[str, np.ndarray]) -> None:
        for name, arr in weights.items():
            jepa_head_set_tensor(self.handle, name, arr)

    def forward(self, x, out=None, stream=None):
        """x: fp32 device tensor [B, N, D] -> fp32 logits [B, n_classes]."""
        import torch
        if out is None:
            out = torch.empty((x.shape[0], self.n_classes), dtype=torch.float32, device=x.device)
        jepa_head_forward(self.handle, x, out, stream)
        return out

    def close(self) -> None:
        if getattr(self, "handle", None):
            jepa_head_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass


class Predictor:
    """Owner of a jepa_predictor handle."""

    def __init__(self, enc_dim: int, embed_dim: int, n_layer: int, n_head: int, ffn_dim: int,
                 n_mask_tokens: int, out_dim: int, *, layout: str = "tiled", dtype: str = "bf16",
                 max_rows: int = 8192, ln_eps: float = 1e-6, theta: float = 10000.0,
                 has_mod_embed: bool = False, has_proj_context: bool = False):
        cfg = jepa_predictor_config(
            enc_dim=enc_dim, embed_dim=embed_dim, n_layer=n_layer, n_head=n_head,
            ffn_dim=ffn_dim, n_mask_tokens=n_mask_tokens, out_dim=out_dim,
            rope_layout=LAYOUTS[layout], compute=DTYPES[dtype], max_rows=max_rows,
            ln_eps=ln_eps, rope_theta=theta, has_mod_embed=int(has_mod_embed),
            has_proj_context=int(has_proj_context))
        self.cfg = cfg
        self.out_dim = out_dim
        self.handle = jepa_predictor_create(cfg)

    def set_weights(self, weights: Dict[str, np.ndarray]) -> None:
        for name, arr in weights.items():
            jepa_predictor_set_tensor(self.handle, name, arr)

    def predict(self, z, ids_ctx, ids_tgt, mask_index: int, grid: Sequence[int], out=None,
                stream=None):
        import torch
        if out is None:
            out = torch.empty((ids_tgt.numel(), self.out_dim), dtype=torch.float32,
                              device=z.device)
        jepa_predict(self.handle, z, ids_ctx, ids_tgt, mask_index, grid, out, stream)
        return out

    def predict_mod(self, z, ids_ctx, ids_tgt, mask_index: int, grid: Sequence[int],
                    modality: str = "video", context: bool = False, stream=None):
        """The 2.1 predictor: returns the target predictions, and with context=True also
        the projected context rows."""
        import torch
        out = torch.empty((ids_tgt.numel(), self.out_dim), dtype=torch.float32, device=z.device)
        ctx = (torch.empty((ids_ctx.numel(), self.out_dim), dtype=torch.float32, device=z.device)
               if context else None)
        jepa_predict_mod(self.handle, z, ids_ctx, ids_tgt, mask_index, modality, grid, out, ctx, stream)
        return (out, ctx) if context else out

    def close(self) -> None:
        if getattr(self, "handle", None):
            jepa_predictor_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
