"""Pure-Python brute force of the encoder and predictor on tiny inputs.

Written element by element from the pages' formulas, with Python floats, lists and the
``math`` module only (no numpy), so it shares no code path with the numpy oracle:
  * pixel normalisation in the fused form (px - 255*mean)/(255*std)
    ([Parity "Preprocessing parity"]);
  * patch features by explicit index: feature (c, dt, dy, dx) of token (t', h', w')
    ([Notes §2] C,T,H,W flattening; [Notes §4] T-major token order);
  * frequencies spelled omega_k = theta ** (-(2k)/d) ([Notes §4]);
  * RoPE written pair by pair as the elementwise formulas of [Notes §4.1] (tiled: the
    even element of pair k uses omega_{(2k) mod d/2}, the odd one omega_{(2k+1) mod d/2})
    and [Notes §4.2] (interleaved: both use omega_k);
  * attention as explicit sums of exp over every key.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

MEAN = (0.485, 0.456, 0.406)
STD = (0.229, 0.224, 0.225)


def to_list(a):
    return a.tolist() if hasattr(a, "tolist") else a


def matvec_rows(x: List[List[float]], w: List[List[float]], b: Sequence[float]) -> List[List[float]]:
    """y[n][o] = sum_i x[n][i] * w[o][i] + b[o]."""
    out = []
    for row in x:
        out.append([sum(row[i] * wo[i] for i in range(len(row))) + b[o] for o, wo in enumerate(w)])
    return out


def layer_norm_rows(x, g, b, eps):
    out = []
    for row in x:
        n = len(row)
        mu = sum(row) / n
        var = sum((v - mu) ** 2 for v in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(row[i] - mu) * inv * g[i] + b[i] for i in range(n)])
    return out


def gelu(z):
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def positions(i, gh, gw, ref_grid):
    t = i // (gh * gw)
    h = (i % (gh * gw)) // gw
    w = i % gw
    pt, ph, pw = float(t), float(h), float(w)
    if ref_grid:
        ph = h * (ref_grid - 1) / (gh - 1)
        pw = w * (ref_grid - 1) / (gw - 1)
    return (pt, ph, pw)


def rope_vec(u: List[float], pos, layout: str, theta: float) -> List[float]:
    hd = len(u)
    d = 2 * ((hd // 3) // 2)
    m = d // 2
    out = list(u)
    for a in range(3):
        s = a * d
        p = pos[a]
        for k in range(m):  # pair k of this axis segment: elements s+2k, s+2k+1
            x0, x1 = u[s + 2 * k], u[s + 2 * k + 1]
            if layout == "tiled":
                fe, fo = (2 * k) % m, (2 * k + 1) % m
            else:
                fe, fo = k, k
            ae = p * theta ** (-(2 * fe) / d)
            ao = p * theta ** (-(2 * fo) / d)
            out[s + 2 * k] = x0 * math.cos(ae) - x1 * math.sin(ae)
            out[s + 2 * k + 1] = x1 * math.cos(ao) + x0 * math.sin(ao)
    return out


def attention(q, k, v, n_head, pos, layout, theta, visible=None):
    """visible(i, n) -> bool hides key n from query i (default: every key visible)."""
    N = len(q)
    D = len(q[0])
    hd = D // n_head
    out = [[0.0] * D for _ in range(N)]
    for e in range(n_head):
        c0 = e * hd
        qs = [rope_vec(q[n][c0:c0 + hd], pos[n], layout, theta) for n in range(N)]
        ks = [rope_vec(k[n][c0:c0 + hd], pos[n], layout, theta) for n in range(N)]
        for i in range(N):
            s = [sum(qs[i][j] * ks[n][j] for j in range(hd)) / math.sqrt(hd) for n in range(N)]
            keep = [visible is None or visible(i, n) for n in range(N)]
            mx = max(s[n] for n in range(N) if keep[n])
            ex = [math.exp(s[n] - mx) if keep[n] else 0.0 for n in range(N)]
            tot = sum(ex)
            for j in range(hd):
                out[i][c0 + j] = sum(ex[n] * v[n][c0 + j] for n in range(N)) / tot
    return out


def block(x, W, prefix, n_head, pos, layout, theta, eps):
    D = len(x[0])
    h = layer_norm_rows(x, W[prefix + ".ln1.weight"], W[prefix + ".ln1.bias"], eps)
    qkv = matvec_rows(h, W[prefix + ".attn_qkv.weight"], W[prefix + ".attn_qkv.bias"])
    q = [r[:D] for r in qkv]
    k = [r[D:2 * D] for r in qkv]
    v = [r[2 * D:] for r in qkv]
    o = attention(q, k, v, n_head, pos, layout, theta)
    a = matvec_rows(o, W[prefix + ".attn_out.weight"], W[prefix + ".attn_out.bias"])
    x = [[x[n][i] + a[n][i] for i in range(D)] for n in range(len(x))]
    h2 = layer_norm_rows(x, W[prefix + ".ln2.weight"], W[prefix + ".ln2.bias"], eps)
    g = [[gelu(z) for z in r] for r in matvec_rows(h2, W[prefix + ".ffn_up.weight"], W[prefix + ".ffn_up.bias"])]
    f = matvec_rows(g, W[prefix + ".ffn_down.weight"], W[prefix + ".ffn_down.bias"])
    return [[x[n][i] + f[n][i] for i in range(D)] for n in range(len(x))]


def encoder(clip, Wnp: Dict, n_layer, n_head, layout, ref_grid=0, mod_embed=False,
            final_norm=True, theta=10000.0, eps=1e-6, tubelet=2, patch=16, ctx_ids=None):
    """clip: uint8 [T, H, W, 3] (numpy or nested lists).  ctx_ids: keep only these tokens
    (in this order) before the first block, each at its own grid position."""
    W = {k: to_list(v) for k, v in Wnp.items()}
    c = to_list(clip)
    T, H, Wd = len(c), len(c[0]), len(c[0][0])
    gt, gh, gw = T // tubelet, H // patch, Wd // patch
    N = gt * gh * gw
    feats = []
    for n in range(N):
        tp, hp, wp = n // (gh * gw), (n % (gh * gw)) // gw, n % gw
        row = []
        for ch in range(3):
            for dt in range(tubelet):
                for dy in range(patch):
                    for dx in range(patch):
                        px = c[tubelet * tp + dt][patch * hp + dy][patch * wp + dx][ch]
                        row.append((px - 255.0 * MEAN[ch]) / (255.0 * STD[ch]))
        feats.append(row)
    x = matvec_rows(feats, W["enc.patch_embed.weight"], W["enc.patch_embed.bias"])
    if mod_embed:
        x = [[r[i] + W["enc.mod_embed_video"][i] for i in range(len(r))] for r in x]
    pos = [positions(n, gh, gw, ref_grid) for n in range(N)]
    if ctx_ids is not None:
        keep = [int(i) for i in ctx_ids]
        x = [x[i] for i in keep]
        pos = [pos[i] for i in keep]
    for li in range(n_layer):
        x = block(x, W, f"enc.blk.{li}", n_head, pos, layout, theta, eps)
    if final_norm:
        x = layer_norm_rows(x, W["enc.norm.weight"], W["enc.norm.bias"], eps)
    return x


def predictor(z, Wnp: Dict, ids_ctx, ids_tgt, mask_index, grid, n_layer, n_head, n_mask,
              layout="tiled", theta=10000.0, eps=1e-6, mod=None, context=False):
    """mod: name of a modality vector added to every row after the concatenation;
    context: also return the context rows projected by pred.proj_context."""
    W = {k: to_list(v) for k, v in Wnp.items()}
    z = to_list(z)
    ids_ctx = [int(i) for i in ids_ctx]
    ids_tgt = [int(i) for i in ids_tgt]
    ctx = matvec_rows([z[i] for i in ids_ctx], W["pred.embed.weight"], W["pred.embed.bias"])
    tok = W["pred.mask_tokens"][mask_index % n_mask]
    x = ctx + [list(tok) for _ in ids_tgt]
    if mod is not None:
        x = [[r[i] + W[mod][i] for i in range(len(r))] for r in x]
    _, gh, gw = grid
    pos = [positions(i, gh, gw, 0) for i in ids_ctx + ids_tgt]
    for li in range(n_layer):
        x = block(x, W, f"pred.blk.{li}", n_head, pos, layout, theta, eps)
    x = layer_norm_rows(x, W["pred.norm.weight"], W["pred.norm.bias"], eps)
    pred = matvec_rows(x[len(ids_ctx):], W["pred.proj.weight"], W["pred.proj.bias"])
    if not context:
        return pred
    return pred, matvec_rows(x[:len(ids_ctx)], W["pred.proj_context.weight"], W["pred.proj_context.bias"])


def head(x, Wnp: Dict, n_layer, n_head, eps=1e-6):
    """Attentive-pool head on one token map x [N][D] -> logits, element by element."""
    W = {k: to_list(v) for k, v in Wnp.items()}
    x = to_list(x)
    N, D = len(x), len(x[0])
    hd = D // n_head
    pos = [(0.0, 0.0, 0.0)] * N
    for li in range(n_layer):
        x = block(x, W, f"head.blk.{li}", n_head, pos, "tiled", 10000.0, eps)
    q0 = W["head.query"][0]
    kv = layer_norm_rows(x, W["head.xattn.ln_kv.weight"], W["head.xattn.ln_kv.bias"], eps)
    q = matvec_rows([q0], W["head.xattn.q.weight"], W["head.xattn.q.bias"])[0]
    k = matvec_rows(kv, W["head.xattn.k.weight"], W["head.xattn.k.bias"])
    v = matvec_rows(kv, W["head.xattn.v.weight"], W["head.xattn.v.bias"])
    y = list(q0)
    for e in range(n_head):
        c0 = e * hd
        s = [sum(q[c0 + j] * k[n][c0 + j] for j in range(hd)) / math.sqrt(hd) for n in range(N)]
        mx = max(s)
        ex = [math.exp(t - mx) for t in s]
        tot = sum(ex)
        for j in range(hd):
            y[c0 + j] += sum(ex[n] * v[n][c0 + j] for n in range(N)) / tot
    h = layer_norm_rows([y], W["head.xattn.ln2.weight"], W["head.xattn.ln2.bias"], eps)
    g = [[gelu(z) for z in r] for r in matvec_rows(h, W["head.xattn.ffn_up.weight"], W["head.xattn.ffn_up.bias"])]
    f = matvec_rows(g, W["head.xattn.ffn_down.weight"], W["head.xattn.ffn_down.bias"])[0]
    y = [y[i] + f[i] for i in range(D)]
    return matvec_rows([y], W["head.cls.weight"], W["head.cls.bias"])[0]
