"""float64 oracle of the V-JEPA 2 / 2.1 encoder forward and the V-JEPA 2 masked predictor.

Test infrastructure (see the package docstring): plain numpy, float64, no blocking,
fusion or reordering beyond what each cited definition states.  The only liberty taken
is that attention is evaluated a slab of query rows at a time, which changes nothing:
each output row is a function of its own query row and all keys/values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "IMAGENET_MEAN", "IMAGENET_STD", "EncoderSpec", "PredictorSpec",
    "normalize_frames", "patchify", "id_to_thw", "rope_positions", "rope_axis_dim",
    "rope_omegas", "rope_angle_index", "rope_angles", "rope_rotate", "rope_rotate_with_angles",
    "layer_norm", "gelu_erf", "linear", "attention", "block_causal_mask", "block", "encoder_forward",
    "encode_tokens", "encoder_forward_batch", "encoder_forward_image", "masked_encoder_forward",
    "predictor_forward", "mean_pool", "attentive_pool_head",
]

# [Notes §1 "pre.mean / std / rescale": ImageNet, 1/255]; values as given on [HFport
# "Preprocessing"] and [Notes §5].
IMAGENET_MEAN = (0.485, 0.456, 0.406)
IMAGENET_STD = (0.229, 0.224, 0.225)


@dataclasses.dataclass(frozen=True)
class EncoderSpec:
    """Hyper-parameters of one encoder ([Notes §1 table])."""
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    patch: int = 16
    tubelet: int = 2
    in_chans: int = 3
    has_mod_embed: bool = False
    final_norm: bool = True
    layout: str = "tiled"          # "tiled" (V-JEPA 2) or "interleaved" (V-JEPA 2.1)
    ref_grid: int = 0              # 0: no interpolation; else R ([Notes §4.3], R = 16)
    ln_eps: float = 1e-6
    theta: float = 10000.0

    @property
    def head_dim(self) -> int:
        return self.embed_dim // self.n_head


@dataclasses.dataclass(frozen=True)
class PredictorSpec:
    """V-JEPA 2 masked predictor ([Notes §1]: 384 / 12 / 12 / 1536, 10 mask tokens,
    out_dim 1024, tiled, not interpolated)."""
    enc_dim: int
    embed_dim: int
    n_layer: int
    n_head: int
    ffn_dim: int
    n_mask_tokens: int
    out_dim: int
    layout: str = "tiled"
    ln_eps: float = 1e-6
    theta: float = 10000.0
    has_mod_embed: bool = False      # V-JEPA 2.1: a modality vector on every row
    has_proj_context: bool = False   # V-JEPA 2.1: projection of the context rows

    @property
    def head_dim(self) -> int:
        return self.embed_dim // self.n_head


# --------------------------------------------------------------------------- pixels


def normalize_frames(u8: np.ndarray) -> np.ndarray:
    """uint8 frames [T, H, W, 3] -> model input X [3, T, H, W] float64.

    Rescale by 1/255 then subtract the ImageNet mean and divide by the std, per channel
    ([Notes §5], [HFport "Preprocessing"]); the model layout is channels first, then
    time, height, width ([Notes §5]: the HF processor's [B, T, C, H, W] is permuted to
    [B, C, T, H, W] before the Conv3d).
    """
    x = u8.astype(np.float64) / 255.0
    x = (x - np.asarray(IMAGENET_MEAN)) / np.asarray(IMAGENET_STD)
    return np.transpose(x, (3, 0, 1, 2))


def patchify(X: np.ndarray, tubelet: int = 2, patch: int = 16) -> np.ndarray:
    """Tubelet patchify [C, T, H, W] -> [N, C*tubelet*patch*patch].

    Token order is T-major, then H, then W ([Notes §4]: t = i // (gh*gw), ...).  Feature
    order is C, T, H, W: the Conv3d kernel [D, 3, 2, 16, 16] flattened row-major to
    [D, 1536] ([Notes §2], first row of the key-map table), so feature
    f = ((c*tubelet + dt)*patch + dy)*patch + dx reads X[c, tubelet*t' + dt,
    patch*h' + dy, patch*w' + dx].
    """
    C, T, H, W = X.shape
    if T % tubelet or H % patch or W % patch:
        raise ValueError("clip not divisible into tubelets")
    gt, gh, gw = T // tubelet, H // patch, W // patch
    p = X.reshape(C, gt, tubelet, gh, patch, gw, patch)      # c t' dt h' dy w' dx
    p = np.transpose(p, (1, 3, 5, 0, 2, 4, 6))                # t' h' w' | c dt dy dx
    return p.reshape(gt * gh * gw, C * tubelet * patch * patch)


# --------------------------------------------------------------------------- positions


def id_to_thw(ids: np.ndarray, gh: int, gw: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Token id -> integer grid coordinates, T-major ([Notes §4]):
    t = i // (gh*gw), h = (i mod gh*gw) // gw, w = i mod gw."""
    ids = np.asarray(ids, dtype=np.int64)
    t = ids // (gh * gw)
    h = (ids % (gh * gw)) // gw
    w = ids % gw
    return t, h, w


def rope_positions(ids: np.ndarray, gh: int, gw: int, ref_grid: int = 0) -> np.ndarray:
    """float64 positions [N, 3] = (p_t, p_h, p_w) of the token ids.

    Without interpolation the positions are the integer coordinates cast to float
    ([Notes §4.2]: positions cast to float).  With interpolation (V-JEPA 2.1 encoder,
    [Notes §4.3]): h' = h*(R-1)/(gh-1), w' = w*(R-1)/(gw-1), t unchanged; a grid side of
    1 is rejected (division by zero).
    """
    t, h, w = id_to_thw(ids, gh, gw)
    pt, ph, pw = t.astype(np.float64), h.astype(np.float64), w.astype(np.float64)
    if ref_grid:
        if gh <= 1 or gw <= 1:
            raise ValueError("position interpolation needs gh > 1 and gw > 1")
        ph = ph * (ref_grid - 1) / (gh - 1)
        pw = pw * (ref_grid - 1) / (gw - 1)
    return np.stack([pt, ph, pw], axis=1)


# --------------------------------------------------------------------------- RoPE


def rope_axis_dim(head_dim: int) -> int:
    """Rotated dims per axis, d = 2*((head_dim // 3) // 2) ([Notes §1], [Notes §4])."""
    return 2 * ((head_dim // 3) // 2)


def rope_omegas(d: int, theta: float = 10000.0) -> np.ndarray:
    """omega_k = 1 / theta**(k / (d/2)), k = 0 .. d/2-1 ([Notes §4], frequencies)."""
    k = np.arange(d // 2, dtype=np.float64)
    return 1.0 / theta ** (k / (d / 2.0))


def rope_angle_index(d: int, layout: str) -> np.ndarray:
    """Which of the d/2 frequencies each of the d rotated dims of an axis uses.

    tiled ([Notes §4.1]): the length-d/2 table is repeated whole, dim j uses j mod d/2.
    interleaved ([Notes §4.2]): each entry is repeated twice in place, dim j uses j // 2.
    """
    j = np.arange(d)
    if layout == "tiled":
        return j % (d // 2)
    if layout == "interleaved":
        return j // 2
    raise ValueError(f"unknown RoPE layout {layout!r}")


def rope_angles(pos: np.ndarray, head_dim: int, layout: str, theta: float = 10000.0) -> np.ndarray:
    """Per-dim angles [N, 3d]: axis a in (t, h, w) owns dims [a*d, (a+1)*d) and dim
    a*d + j gets angle pos[:, a] * omega[idx(j)] ([Notes §4])."""
    d = rope_axis_dim(head_dim)
    om = rope_omegas(d, theta)[rope_angle_index(d, layout)]
    return np.concatenate([pos[:, a:a + 1] * om[None, :] for a in range(3)], axis=1)


def rope_rotate_with_angles(u: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """u * COS + rot90(u) * SIN over the first ang.shape[-1] dims, rest unchanged.

    rot90 acts on adjacent pairs: rot90(u)[2k] = -u[2k+1], rot90(u)[2k+1] = u[2k]
    ([Notes §4]).  u: [..., N, hd]; ang: [N, r] with r even and r <= hd.
    """
    r = ang.shape[-1]
    out = np.array(u, dtype=np.float64, copy=True)
    seg = out[..., :r].copy()
    rot = np.empty_like(seg)
    rot[..., 0::2] = -seg[..., 1::2]
    rot[..., 1::2] = seg[..., 0::2]
    out[..., :r] = seg * np.cos(ang) + rot * np.sin(ang)
    return out


def rope_rotate(u: np.ndarray, pos: np.ndarray, layout: str, theta: float = 10000.0) -> np.ndarray:
    """3-D RoPE of head vectors u [..., N, hd] at positions pos [N, 3] ([Notes §4]);
    the last hd - 3d dims pass through unchanged."""
    return rope_rotate_with_angles(u, rope_angles(pos, u.shape[-1], layout, theta))


# --------------------------------------------------------------------------- layers


def layer_norm(x: np.ndarray, weight: np.ndarray, bias: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm over the last axis: centred (two-pass) biased variance, eps inside the
    square root, then the affine weight and bias.  eps = 1e-6 ([Notes §1]); the centred
    variance is the CPU backend's ([Parity "Parity on a GPU", backend table])."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * weight + bias


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """Exact GELU, z/2 * (1 + erf(z / sqrt 2)) ([Notes §1]: gelu = exact erf GELU)."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b with W stored [out, in] ([Notes §2] key map)."""
    y = x @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + b
    return y


def block_causal_mask(N: int, n_cls: int, slot: int) -> np.ndarray:
    """Visibility [N, N] (query row, key column) of the block-causal attention of
    [Parity] "LeVJEPA ViT-L/16 — CLS, block-causal attention, tubelet 1": rows [0, n_cls)
    are CLS rows, open to every key; the patch tokens that follow sit in temporal slots of
    ``slot`` tokens, and a patch query sees every patch key of its own and earlier slots
    (bidirectional inside a slot, causal across slots) and no CLS key."""
    idx = np.arange(N)
    slot_of = np.where(idx >= n_cls, (idx - n_cls) // slot, -1)
    vis = (slot_of[None, :] <= slot_of[:, None]) & (idx[None, :] >= n_cls)
    vis[:n_cls, :] = True
    return vis


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_head: int,
              pos_q: np.ndarray, pos_k: np.ndarray, layout: str, theta: float = 10000.0,
              rows: Optional[np.ndarray] = None, slab: int = 1024,
              visible: Optional[np.ndarray] = None) -> np.ndarray:
    """Multi-head softmax attention with 3-D RoPE on q and k.

    q [Nq, D], k, v [Nk, D]; head e owns columns [e*hd, (e+1)*hd) (contiguous split of
    the fused projection).  RoPE is applied to q and k, not v, after the projection and
    before the 1/sqrt(hd) scaling ([Notes §4]); softmax runs over every key, no mask
    ([Notes §2] attentive-pool head uses the same softmax(q k^T / sqrt(hd)) v form).
    ``rows`` selects query rows (default all); each output row depends only on its own
    query row, so the result is evaluated a slab of rows at a time.  ``visible`` [Nq, Nk]
    (default all true) hides keys from queries: their scores are -inf before the softmax.
    """
    Nq, D = q.shape
    hd = D // n_head
    if rows is None:
        rows = np.arange(Nq)
    out = np.zeros((len(rows), D))
    for e in range(n_head):
        cs = slice(e * hd, (e + 1) * hd)
        kh = rope_rotate(k[:, cs], pos_k, layout, theta)
        vh = v[:, cs]
        for s0 in range(0, len(rows), slab):
            r = rows[s0:s0 + slab]
            qh = rope_rotate(q[r, cs], pos_q[r], layout, theta)
            s = qh @ kh.T / math.sqrt(hd)
            if visible is not None:
                s = np.where(visible[r], s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[s0:s0 + len(r), cs] = p @ vh
    return out


def block(x: np.ndarray, W: Dict[str, np.ndarray], prefix: str, n_head: int, pos: np.ndarray,
          layout: str, theta: float = 10000.0, eps: float = 1e-6,
          rows: Optional[np.ndarray] = None) -> np.ndarray:
    """One pre-norm transformer block ([Notes §2]: norm1 / fused q,k,v / proj / norm2 /
    fc1 / fc2; the residual form x += attn(ln1(x)); x += mlp(ln2(x)) is written out for
    the attentive-pool blocks; [Notes §1]: no layer-scale, no CLS, no registers).

    ``rows`` (default: all) selects the output rows.  Keys and values always come from
    every row; everything after the attention is row-wise, so the selected rows equal
    the same rows of the full result."""
    D = x.shape[1]
    h = layer_norm(x, W[f"{prefix}.ln1.weight"], W[f"{prefix}.ln1.bias"], eps)
    qkv = linear(h, W[f"{prefix}.attn_qkv.weight"], W[f"{prefix}.attn_qkv.bias"])
    # fused rows are [q; k; v] ([Notes §2], attn_qkv)
    q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
    o = attention(q, k, v, n_head, pos, pos, layout, theta, rows=rows)
    xr = x if rows is None else x[rows]
    xr = xr + linear(o, W[f"{prefix}.attn_out.weight"], W[f"{prefix}.attn_out.bias"])
    h2 = layer_norm(xr, W[f"{prefix}.ln2.weight"], W[f"{prefix}.ln2.bias"], eps)
    g = gelu_erf(linear(h2, W[f"{prefix}.ffn_up.weight"], W[f"{prefix}.ffn_up.bias"]))
    return xr + linear(g, W[f"{prefix}.ffn_down.weight"], W[f"{prefix}.ffn_down.bias"])


def _f64(W: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in W.items()}


def encode_tokens(x: np.ndarray, W: Dict[str, np.ndarray], spec: EncoderSpec,
                  ids: np.ndarray, grid: Tuple[int, int, int],
                  n_layer: Optional[int] = None,
                  last_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """The encoder's blocks (and final norm when ``spec.final_norm``) on token
    activations x [N, D] whose grid ids are ``ids`` on ``grid`` = (gt, gh, gw).
    Positions come from the ids ([Notes §4], [Notes §4.4]).  ``last_rows`` restricts
    the last block (and the norm) to those output rows; earlier blocks run in full."""
    W = _f64(W)
    _, gh, gw = grid
    pos = rope_positions(ids, gh, gw, spec.ref_grid)
    x = np.asarray(x, dtype=np.float64)
    L = spec.n_layer if n_layer is None else n_layer
    for i in range(L):
        rows = last_rows if i == L - 1 else None
        x = block(x, W, f"enc.blk.{i}", spec.n_head, pos, spec.layout, spec.theta, spec.ln_eps,
                  rows=rows)
    if L == 0 and last_rows is not None:
        x = x[last_rows]
    if spec.final_norm:
        x = layer_norm(x, W["enc.norm.weight"], W["enc.norm.bias"], spec.ln_eps)
    return x


def encoder_forward(clip: np.ndarray, W: Dict[str, np.ndarray], spec: EncoderSpec,
                    last_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """One clip, uint8 [T, H, W, 3] -> token map [N, D] float64.

    tokens = patchify(x) Wpe^T + bpe (+ mod_embed_video for V-JEPA 2.1) ([Notes §3
    "2.1 encoder forward"], [Notes §2] patch_embed), then the blocks with 3-D RoPE on the
    clip's own grid, then the final norm ([Notes §3]: out = enc.norm(x)).  ``last_rows``
    as in ``encode_tokens``.
    """
    X = normalize_frames(clip)
    p = patchify(X, spec.tubelet, spec.patch)
    Wd = _f64(W)
    x = linear(p, Wd["enc.patch_embed.weight"], Wd["enc.patch_embed.bias"])
    if spec.has_mod_embed:
        x = x + Wd["enc.mod_embed_video"]
    T, H, Wd_ = clip.shape[0], clip.shape[1], clip.shape[2]
    grid = (T // spec.tubelet, H // spec.patch, Wd_ // spec.patch)
    ids = np.arange(grid[0] * grid[1] * grid[2])
    return encode_tokens(x, W, spec, ids, grid, last_rows=last_rows)


def masked_encoder_forward(clip: np.ndarray, W: Dict[str, np.ndarray], spec: EncoderSpec,
                           ctx_ids: np.ndarray) -> np.ndarray:
    """Pre-training forward on the context tokens of one clip, uint8 [T, H, W, 3] ->
    [K, D] float64 for the K grid ids ``ctx_ids`` ([HFport "Usage"]: masks passed to the
    encoder; [HFport "Validation"], masked-encoder row).

    The tokens outside ``ctx_ids`` are dropped before the first block: the patch rows are
    embedded as in ``encoder_forward``, the rows of the kept ids are taken in the given
    order, and the blocks and the final norm run on those K rows with the RoPE positions
    of their own grid ids.  Attention therefore sees only the context, which is not the
    same as taking rows of the full forward's output.
    """
    X = normalize_frames(clip)
    p = patchify(X, spec.tubelet, spec.patch)
    Wd = _f64(W)
    x = linear(p, Wd["enc.patch_embed.weight"], Wd["enc.patch_embed.bias"])
    if spec.has_mod_embed:
        x = x + Wd["enc.mod_embed_video"]
    T, H, Wd_ = clip.shape[0], clip.shape[1], clip.shape[2]
    grid = (T // spec.tubelet, H // spec.patch, Wd_ // spec.patch)
    ids = np.asarray(ctx_ids, dtype=np.int64)
    return encode_tokens(x[ids], W, spec, ids, grid)


def encoder_forward_image(img: np.ndarray, W: Dict[str, np.ndarray], spec: EncoderSpec) -> np.ndarray:
    """V-JEPA 2.1 native image path, one uint8 image [H, W, 3] -> [N, D] float64
    ([Notes §3] "2.1 encoder forward", image line; [Notes §2] patch_embed_img with
    tubelet 1; [Notes §5]: fed as one frame).

    tokens = patchify(x, 1, 16) Wpe_img^T + bpe_img (+ mod_embed_img), features in C, T, H, W
    order with T = 1; then the blocks with 3-D RoPE on the grid (1, H/16, W/16) and the
    final norm, as for a clip.
    """
    X = normalize_frames(img[None])
    p = patchify(X, 1, spec.patch)
    Wd = _f64(W)
    x = linear(p, Wd["enc.patch_embed_img.weight"], Wd["enc.patch_embed_img.bias"])
    if spec.has_mod_embed:
        x = x + Wd["enc.mod_embed_img"]
    grid = (1, img.shape[0] // spec.patch, img.shape[1] // spec.patch)
    return encode_tokens(x, W, spec, np.arange(grid[1] * grid[2]), grid)


def mean_pool(x: np.ndarray) -> np.ndarray:
    """Mean of a token map [N, D] over its tokens -> [D] ([Card] "Run it": ``--pool mean``
    turns the token map into one pooled feature)."""
    return np.asarray(x, dtype=np.float64).mean(axis=0)


def attentive_pool_head(x: np.ndarray, W: Dict[str, np.ndarray], n_layer: int, n_head: int,
                        eps: float = 1e-6) -> np.ndarray:
    """Attentive-pool classifier head on one token map x [N, D] (the encoder output after
    its final norm) -> logits [n_classes] ([Notes §2] "Attentive-pool head — exact
    forward" and the head.* rows of its key map).

    ``n_layer`` self-attention blocks head.blk.{i} as the encoder's but without RoPE (every
    position 0, i.e. no rotation); then one cross-attention: the raw learned query
    head.query takes q from it, the normed tokens (head.xattn.ln_kv) give k and v through
    their own projections, softmax(q k^T / sqrt(hd)) v per head with the heads
    concatenated and no output projection; the raw query is the residual; a GELU MLP
    after head.xattn.ln2 with its own residual; the linear classifier head.cls, no final
    norm.
    """
    W = _f64(W)
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    pos0 = np.zeros((N, 3))
    for i in range(n_layer):
        x = block(x, W, f"head.blk.{i}", n_head, pos0, "tiled", eps=eps)
    q0 = W["head.query"]                                                  # [1, D]
    kv = layer_norm(x, W["head.xattn.ln_kv.weight"], W["head.xattn.ln_kv.bias"], eps)
    q = linear(q0, W["head.xattn.q.weight"], W["head.xattn.q.bias"])
    k = linear(kv, W["head.xattn.k.weight"], W["head.xattn.k.bias"])
    v = linear(kv, W["head.xattn.v.weight"], W["head.xattn.v.bias"])
    o = attention(q, k, v, n_head, np.zeros((1, 3)), pos0, "tiled")
    y = q0 + o
    h = layer_norm(y, W["head.xattn.ln2.weight"], W["head.xattn.ln2.bias"], eps)
    g = gelu_erf(linear(h, W["head.xattn.ffn_up.weight"], W["head.xattn.ffn_up.bias"]))
    y = y + linear(g, W["head.xattn.ffn_down.weight"], W["head.xattn.ffn_down.bias"])
    return linear(y, W["head.cls.weight"], W["head.cls.bias"])[0]


def encoder_forward_batch(clips: np.ndarray, W, spec: EncoderSpec) -> np.ndarray:
    """[B, T, H, W, 3] -> [B, N, D]; each clip is encoded on its own."""
    return np.stack([encoder_forward(c, W, spec) for c in clips])


def predictor_forward(z: np.ndarray, W: Dict[str, np.ndarray], spec: PredictorSpec,
                      ids_ctx: np.ndarray, ids_tgt: np.ndarray, mask_index: int,
                      grid: Tuple[int, int, int],
                      last_rows: Optional[np.ndarray] = None, modality: str = "video",
                      return_context: bool = False):
    """Masked predictor: encoder token map z [N, D_enc] -> predictions [len(ids_tgt), out].

    ctx = z[ids_ctx] Wemb^T + b; every target row is mask_tokens[mask_index mod n];
    x = concat(ctx, tgt) with positions decoded from concat(ids_ctx, ids_tgt) on the
    encoder grid; blocks with 3-D RoPE (tiled, not interpolated); final norm; the output
    projection on the target rows ([Notes §3 "2.1 predictor forward"] for the order of
    operations, [Notes §2] for the V-JEPA 2 tensors, [Notes §4.4] for the ids).  Tokens
    are not sorted by id: attention is permutation-equivariant ([Notes §3]).
    ``last_rows`` (indices into the targets) restricts the last block, the norm and the
    projection to those target rows.

    V-JEPA 2.1 ([Notes §3] "2.1 predictor forward"): with ``spec.has_mod_embed`` every row
    (context and mask tokens) takes ``pred.mod_embed_{modality}`` after the concatenation;
    with ``return_context`` the normed context rows are projected by ``pred.proj_context``
    and (predictions, context output) is returned.
    """
    W = _f64(W)
    ids_ctx = np.asarray(ids_ctx, dtype=np.int64)
    ids_tgt = np.asarray(ids_tgt, dtype=np.int64)
    ctx = linear(np.asarray(z, dtype=np.float64)[ids_ctx], W["pred.embed.weight"], W["pred.embed.bias"])
    tok = W["pred.mask_tokens"][mask_index % spec.n_mask_tokens]
    tgt = np.broadcast_to(tok, (len(ids_tgt), spec.embed_dim))
    x = np.concatenate([ctx, tgt], axis=0)
    if spec.has_mod_embed:
        x = x + W[f"pred.mod_embed_{modality}"]
    if return_context:
        assert spec.has_proj_context and last_rows is None
    _, gh, gw = grid
    pos = rope_positions(np.concatenate([ids_ctx, ids_tgt]), gh, gw, 0)
    n_ctx = len(ids_ctx)
    tgt_rows = n_ctx + (np.arange(len(ids_tgt)) if last_rows is None else np.asarray(last_rows))
    L = spec.n_layer
    for i in range(L):
        rows = tgt_rows if (i == L - 1 and last_rows is not None) else None
        x = block(x, W, f"pred.blk.{i}", spec.n_head, pos, spec.layout, spec.theta, spec.ln_eps,
                  rows=rows)
    if return_context:
        x = layer_norm(x, W["pred.norm.weight"], W["pred.norm.bias"], spec.ln_eps)
        return (linear(x[n_ctx:], W["pred.proj.weight"], W["pred.proj.bias"]),
                linear(x[:n_ctx], W["pred.proj_context.weight"], W["pred.proj_context.bias"]))
    if not (L > 0 and last_rows is not None):
        x = x[tgt_rows]
    x = layer_norm(x, W["pred.norm.weight"], W["pred.norm.bias"], spec.ln_eps)
    return linear(x, W["pred.proj.weight"], W["pred.proj.bias"])
