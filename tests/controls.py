"""Negative controls: the oracle's forwards with one planted mistake (CPU, test-only).

A parity gate is only worth something if the plausible mistakes of the path it guards
fail it.  These forwards repeat the oracle's steps with the oracle's own primitives
(``oracle.layer_norm``, ``oracle.linear``, ``oracle.attention``, ``oracle.gelu_erf``,
``oracle.rope_positions``) in the same order, and let a test plant one mistake:

  * ``pos``: RoPE positions passed in directly, so a test can hand over all-zero positions
    (no rotation), positions without the interpolation of [Notes §4.3], or the row index
    instead of the token's grid id;
  * ``layout``: the other frequency layout of [Notes §4.1] / §4.2;
  * ``v_perm``: the value rows permuted against the key rows (a transposed-V write that
    puts key n's values at another key's column).

With nothing planted each forward equals the oracle's bit for bit
(``tests/test_oracle_controls.py``).  Nothing here is imported by the HIP path.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import oracle


def vt_bitswap(n: int) -> np.ndarray:
    """Permutation of n keys that swaps bits 2 and 3 of the key index (the key order of a
    transposed-V layout read back as if it were plain): index i -> i with bits 2 and 3
    exchanged, for indices whose swapped value stays below n (the others stay put)."""
    i = np.arange(n)
    j = (i & ~0b1100) | ((i & 0b0100) << 1) | ((i & 0b1000) >> 1)
    return np.where(j < n, j, i)


def block(x: np.ndarray, W: Dict[str, np.ndarray], prefix: str, n_head: int, pos: np.ndarray,
          layout: str, rows: Optional[np.ndarray] = None,
          v_perm: Optional[np.ndarray] = None, theta: float = 10000.0, eps: float = 1e-6) -> np.ndarray:
    """``oracle.block`` with the value rows optionally permuted against the keys."""
    D = x.shape[1]
    h = oracle.layer_norm(x, W[f"{prefix}.ln1.weight"], W[f"{prefix}.ln1.bias"], eps)
    qkv = oracle.linear(h, W[f"{prefix}.attn_qkv.weight"], W[f"{prefix}.attn_qkv.bias"])
    q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
    if v_perm is not None:
        v = v[v_perm]
    o = oracle.attention(q, k, v, n_head, pos, pos, layout, theta, rows=rows)
    xr = x if rows is None else x[rows]
    xr = xr + oracle.linear(o, W[f"{prefix}.attn_out.weight"], W[f"{prefix}.attn_out.bias"])
    h2 = oracle.layer_norm(xr, W[f"{prefix}.ln2.weight"], W[f"{prefix}.ln2.bias"], eps)
    g = oracle.gelu_erf(oracle.linear(h2, W[f"{prefix}.ffn_up.weight"], W[f"{prefix}.ffn_up.bias"]))
    return xr + oracle.linear(g, W[f"{prefix}.ffn_down.weight"], W[f"{prefix}.ffn_down.bias"])


def _f64(W):
    return {k: np.asarray(v, dtype=np.float64) for k, v in W.items()}


def encode_tokens(x: np.ndarray, W: Dict[str, np.ndarray], spec: "oracle.EncoderSpec",
                  pos: np.ndarray, layout: Optional[str] = None,
                  last_rows: Optional[np.ndarray] = None,
                  v_perm: Optional[np.ndarray] = None) -> np.ndarray:
    """``oracle.encode_tokens`` with the positions given directly, the layout overridable
    and ``v_perm`` planted in every block."""
    W = _f64(W)
    layout = spec.layout if layout is None else layout
    x = np.asarray(x, dtype=np.float64)
    L = spec.n_layer
    for i in range(L):
        rows = last_rows if i == L - 1 else None
        x = block(x, W, f"enc.blk.{i}", spec.n_head, pos, layout, rows=rows, v_perm=v_perm,
                  theta=spec.theta, eps=spec.ln_eps)
    if L == 0 and last_rows is not None:
        x = x[last_rows]
    if spec.final_norm:
        x = oracle.layer_norm(x, W["enc.norm.weight"], W["enc.norm.bias"], spec.ln_eps)
    return x


def embed(clip: np.ndarray, W: Dict[str, np.ndarray], spec: "oracle.EncoderSpec") -> np.ndarray:
    """The patch embedding of ``oracle.encoder_forward`` (normalise, patchify, Wpe, bias,
    modality vector) on one uint8 clip [T, H, W, 3]."""
    W = _f64(W)
    p = oracle.patchify(oracle.normalize_frames(clip), spec.tubelet, spec.patch)
    x = oracle.linear(p, W["enc.patch_embed.weight"], W["enc.patch_embed.bias"])
    if spec.has_mod_embed:
        x = x + W["enc.mod_embed_video"]
    return x


def predictor(z: np.ndarray, W: Dict[str, np.ndarray], spec: "oracle.PredictorSpec",
              ids_ctx: np.ndarray, ids_tgt: np.ndarray, mask_index: int, pos: np.ndarray,
              layout: Optional[str] = None, last_rows: Optional[np.ndarray] = None,
              v_perm: Optional[np.ndarray] = None) -> np.ndarray:
    """``oracle.predictor_forward`` (V-JEPA 2 form: no modality vector, no context
    projection) with the positions of the concatenated rows given directly, the layout
    overridable and ``v_perm`` planted in every block."""
    W = _f64(W)
    layout = spec.layout if layout is None else layout
    ids_ctx = np.asarray(ids_ctx, dtype=np.int64)
    ctx = oracle.linear(np.asarray(z, dtype=np.float64)[ids_ctx], W["pred.embed.weight"],
                        W["pred.embed.bias"])
    tok = W["pred.mask_tokens"][mask_index % spec.n_mask_tokens]
    x = np.concatenate([ctx, np.broadcast_to(tok, (len(ids_tgt), spec.embed_dim))], axis=0)
    n_ctx = len(ids_ctx)
    tgt_rows = n_ctx + (np.arange(len(ids_tgt)) if last_rows is None else np.asarray(last_rows))
    L = spec.n_layer
    for i in range(L):
        rows = tgt_rows if (i == L - 1 and last_rows is not None) else None
        x = block(x, W, f"pred.blk.{i}", spec.n_head, pos, layout, rows=rows, v_perm=v_perm,
                  theta=spec.theta, eps=spec.ln_eps)
    if not (L > 0 and last_rows is not None):
        x = x[tgt_rows]
    x = oracle.layer_norm(x, W["pred.norm.weight"], W["pred.norm.bias"], spec.ln_eps)
    return oracle.linear(x, W["pred.proj.weight"], W["pred.proj.bias"])


def fails_bf16_gate(a: np.ndarray, b: np.ndarray, cos_mean: float = 0.9999,
                    rel_max: float = 2e-2) -> bool:
    """True when a and b differ by more than the bf16 gate allows (either measure)."""
    s = oracle.metrics.summary(a, b)
    return s["cos_mean"] < cos_mean or s["rel_max"] > rel_max
