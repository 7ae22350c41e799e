"""Throughput of the V-JEPA 2 ViT-L/16 encoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--masked | --image | --head | --block-causal | --predictor [--v21] |
                     --chain | --vitb384 | --rope3d]

One step is one jepa_encode call on a batch of 4 synthetic clips of 16 frames x 256x256
uint8 (2048 tokens per clip, 8192 token rows), already resident in HBM: patch
embedding, 24 pre-norm blocks with 3-D RoPE attention and the final norm, in bf16 MFMA
with fp32 accumulation.  Weights are random N(0, 0.02) rounded to bf16, biases
N(0, 0.01), LayerNorm 1/0; the clips are uniform uint8 (no dataset, no checkpoint).

Prints one JSON line.  ``value`` is encoder tokens/s over the K timed steps (HIP events
on the stream the library launches on, bracketed by device synchronisation).  Beside it:
  * ``roofline``: the dominant kernel (the largest share of a step's time), its
    algorithmic TFLOP/s or GB/s per launch against the MI355X peak (bf16 dense MFMA
    2500 TFLOP/s, HBM 8000 GB/s).  Launch durations come from a second pass of K
    forwards in which the library records a HIP event pair around every launch on the
    stream it launches on (jepa_timing_begin / jepa_timing_end);
  * ``kernels``: the same figures for every kernel class of the step;
  * ``cpu_baseline``: the float64 oracle timed on the host on one clip, the whole 24-layer
    forward end to end (a reported baseline, not a target).

``--masked`` measures the masked-encoder forward instead (jepa_encode_masked, the
pre-training path): the same clips, each with the context of a seeded tube mask (an 8x8
block of patches in every temporal slot, 512 of the 2048 tokens); ``value`` is context
tokens/s and the oracle baseline runs oracle.masked_encoder_forward.

``--predictor`` measures the V-JEPA 2 masked predictor (jepa_predict) on its workload: an
8192-token ViT-L token map (N(0,1) rows standing in for the encoder output), the seeded tube
mask's 2048 context and 6144 target ids, 12 blocks at width 384 (head dim 32); ``value`` is
target tokens/s.  ``--predictor --v21`` runs the V-JEPA 2.1 ViT-B predictor instead (768 -> 384,
8 mask tokens, output 1664, interleaved RoPE, modality vector on every row, context rows
projected too) on the 8x24x24 grid of a 16-frame 384-px clip with the tube mask's 512
context and 4096 target ids.

``--chain`` measures the encoder + predictor chain as one step: the ViT-L/16 encoder on one
64-frame 256-px clip (8192 tokens, 24 layers), then the masked predictor on that output (the
tube mask's 2048 context and 6144 target ids); ``value`` is clip tokens/s through both.

``--head`` measures the attentive-pool classifier head of the V-JEPA 2 SSv2 classifier (3
pool blocks, 16 heads, 174 classes) on 4 token maps of 2048 x 1024 (N(0,1) rows standing in
for the encoder output); ``value`` is clips/s.

``--image`` measures the V-JEPA 2.1 ViT-B/16 native image path (jepa_encode_image) on 16
uniform uint8 images of 384x384 (576 tokens each, 12 layers); ``value`` is image tokens/s.

``--vitb384`` measures the V-JEPA 2.1 ViT-B/16 encoder (12 layers, interleaved RoPE
interpolated to 16, video modality vector) on one uniform uint8 clip of 64 frames x 384x384
(18,432 tokens), where attention is about 80 % of the work; the oracle baseline times the
clip's embedding and final norm and one block on its own, scaled to 12 blocks.

``--rope3d`` measures the stand-alone 3-D RoPE (jepa_rope3d, fp32, out of place) on the q
tensor of the ViT-L batch, [4, 2048, 16, 64] in the tiled layout: an HBM-bound kernel with
8*B*N*H*hd algorithmic bytes per call; ``value`` is GB/s.

``--block-causal`` measures the block-causal attention with a CLS row
(jepa_attention_block_causal) at the LeVJEPA ViT-L/16 shape: 8 clips of 1 + 16 x 14 x 14 =
3137 rows (16 frames of 224 px at tubelet 1), 16 heads of 64, N(0,1) bf16 q/k/v rows;
``value`` is rows/s of the whole call (RoPE table, q/k/v preparation, flash kernel), the
roofline counts the visible (query, key) pairs only, and the unmasked kernel on the same
rows is timed beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
WORKLOAD = "vitl16_16f256"


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def forward_flops(B, N, D, F, L, feat=1536):
    """Algorithmic FLOPs of one encoder forward (2 per multiply-add; attention counted
    as QK^T plus PV, 4*N^2*D per clip and layer; norms, softmax, GELU excluded)."""
    gemm = 2 * B * N * (3 * D * D + D * D + 2 * D * F)
    attn = 4 * B * N * N * D
    return 2 * B * N * feat * D + L * (gemm + attn)


def kernel_work(B, N, D, F, L, feat=1536):
    """Algorithmic work per step of each kernel class: (bound, FLOPs or bytes per step)."""
    M = B * N
    ln_bytes = 2 * L * (M * D * (4 + 2) + 2 * D * 4) + (M * D * (4 + 4) + 2 * D * 4)
    return {
        "patchify": ("hbm", M * feat * (1 + 2)),          # u8 pixels in, bf16 rows out
        "gemm_embed": ("mfma", 2 * M * feat * D),
        "layernorm": ("hbm", ln_bytes),                  # 2L of fp32 -> bf16, final fp32 -> fp32
        "gemm_qkv": ("mfma", L * 2 * M * D * 3 * D),
        "attention": ("mfma", L * 4 * B * N * N * D),
        "gemm_out": ("mfma", L * 2 * M * D * D),
        "gemm_up": ("mfma", L * 2 * M * D * F),
        "gemm_down": ("mfma", L * 2 * M * F * D),
    }


def kernel_timing(J, run_step, steps, work):
    """Per-class launch durations over `steps` forwards, from HIP event pairs the library
    records around each launch on the stream it launches on."""
    import torch
    torch.cuda.synchronize()
    J.jepa_timing_begin(64 * steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        run_step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    rec = J.jepa_timing_end()
    ks = {}
    for name, (bound, per_step) in work.items():
        ms, n = rec[name]
        if n == 0:
            continue
        per_launch = per_step * steps / n
        avg = ms / n
        k = {"bound": bound, "launches_per_step": n // steps, "avg_ms": round(avg, 5),
             "ms_per_step": round(ms / steps, 4)}
        if bound == "mfma":
            k["flops_per_launch"] = int(per_launch)
            k["tflops"] = round(per_launch / (avg * 1e-3) / 1e12, 2)
            k["frac"] = round(k["tflops"] / PEAK_BF16_TFLOPS, 4)
        else:
            k["bytes_per_launch"] = int(per_launch)
            k["gbs"] = round(per_launch / (avg * 1e-3) / 1e9, 1)
            k["frac"] = round(k["gbs"] / PEAK_HBM_GBS, 4)
        ks[name] = k
    return ks, wall * 1e3


def measured_traffic(kind):
    """HBM bytes per launch of kernel class `kind` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (profiles/hbm_traffic.json), or None when there is no entry or the
    kernel's sources changed since the counters were taken (source hash differs)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        tab = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = tab.get(kind)
    if not isinstance(ent, dict):
        return None
    h = hashlib.sha256()
    for fn in ent["sources"]:
        try:
            h.update(open(os.path.join(ROOT, "video_vit_encoder_amd", "csrc", fn), "rb").read())
        except OSError:
            return None
    if h.hexdigest() != ent["source_sha256"]:
        return None
    return ent["read_bytes"] + ent["write_bytes"]


def cpu_baseline(w, W, clips, budget_layers=None, ids0=None, direct=False):
    """The float64 oracle on clip 0.  By default the whole forward (embedding, every block,
    final norm) is run and timed end to end.  With ``budget_layers``: the patch embedding +
    final norm alone, then with that many blocks, the per-block time scaling the forward to
    all its blocks.  With ``ids0`` the masked forward on those context tokens.  ``direct``:
    the blocks are timed on their own (oracle.encode_tokens on N(0,1) rows of the clip's
    grid), for clips whose embedding takes longer than a block."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    e = w["enc"]

    def spec(n):
        return oracle.EncoderSpec(e.embed_dim, n, e.n_head, e.ffn_dim, layout=w["layout"],
                                  ref_grid=w["ref_grid"], has_mod_embed=e.has_mod_embed)

    def run(n):
        if ids0 is None:
            return oracle.encoder_forward(clips[0], W, spec(n))
        return oracle.masked_encoder_forward(clips[0], W, spec(n), ids0)

    N = w["grid"][0] * w["grid"][1] * w["grid"][2] if ids0 is None else len(ids0)
    what = "masked forward, " if ids0 is not None else ""
    if budget_layers is None and not direct:
        t0 = time.perf_counter()
        run(e.n_layer)
        t_clip = time.perf_counter() - t0
        return {"value": N / t_clip, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
                "sample": (f"float64 numpy oracle, {what}clip 0 only ({N} tokens): the whole "
                           f"forward (embedding, all {e.n_layer} blocks, final norm) run and timed "
                           f"end to end, {t_clip:.1f} s; host CPU {host_cpu()}, numpy BLAS on "
                           f"{cores} threads")}
    t0 = time.perf_counter()
    run(0)
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    if direct:
        n = w["grid"][0] * w["grid"][1] * w["grid"][2]
        x = np.random.default_rng(0).standard_normal((n, e.embed_dim))
        oracle.encode_tokens(x, W, spec(budget_layers), np.arange(n), w["grid"])
        t_run = t_fixed + time.perf_counter() - t0
    else:
        run(budget_layers)
        t_run = time.perf_counter() - t0
    t_layer = max(t_run - t_fixed, 1e-9) / budget_layers
    t_clip = t_fixed + e.n_layer * t_layer
    if direct:
        what = "blocks timed on N(0,1) rows, "
    return {"value": N / t_clip, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float64 numpy oracle, {what}clip 0 only ({N} tokens): embedding+norm "
                       f"{t_fixed:.2f} s, {budget_layers} of the {e.n_layer} blocks run and timed "
                       f"({t_run - t_fixed:.2f} s); the other {e.n_layer - budget_layers} blocks are "
                       f"not run but extrapolated at the measured per-block time, giving "
                       f"{t_clip:.1f} s/clip; host CPU {host_cpu()}, numpy BLAS on {cores} threads")}


def predictor_work(n_ctx, n_tgt, Denc, E, F, L, Dout):
    """Algorithmic work per predictor forward by kernel class (as kernel_work)."""
    M = n_ctx + n_tgt
    ln_bytes = 2 * L * (M * E * (4 + 2) + 2 * E * 4) + (n_tgt * E * (4 + 2) + 2 * E * 4)
    return {
        "gemm_embed": ("mfma", 2 * n_ctx * Denc * E + 2 * n_tgt * E * Dout),   # embed + output proj
        "layernorm": ("hbm", ln_bytes),
        "gemm_qkv": ("mfma", L * 2 * M * E * 3 * E),
        "attention": ("mfma", L * 4 * M * M * E),
        "gemm_out": ("mfma", L * 2 * M * E * E),
        "gemm_up": ("mfma", L * 2 * M * E * F),
        "gemm_down": ("mfma", L * 2 * M * F * E),
    }


def bench_predictor(args):
    import torch
    import synth
    import video_vit_encoder_amd as J

    v21 = args.v21
    w = synth.workload("vitb16_pred21" if v21 else "vitl16_64f256_pred")
    p = w["pred"]
    grid = w["grid_video"] if v21 else w["grid"]
    N = grid[0] * grid[1] * grid[2]
    log(f"predictor workload: {N} encoder tokens, width {p.embed_dim}, {p.n_layer} blocks; drawing weights")
    Wp = synth.predictor_weights(p, seed=args.seed, dtype="bf16")
    ids_ctx, ids_tgt = synth.tube_mask(args.seed, *grid)
    z = synth.tokens_normal(5, 1, N, p.enc_dim)[0]
    dev = torch.device("cuda:0")
    pred = J.Predictor(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim, p.n_mask_tokens,
                       p.out_dim, dtype="bf16", max_rows=len(ids_ctx) + len(ids_tgt),
                       layout=w.get("layout", "tiled"), has_mod_embed=p.has_mod_embed,
                       has_proj_context=p.has_proj_context)
    pred.set_weights(Wp)
    z_d = torch.from_numpy(z).to(dev)
    ic = torch.from_numpy(ids_ctx.astype(np.int32)).to(dev)
    it = torch.from_numpy(ids_tgt.astype(np.int32)).to(dev)
    out = torch.empty((len(ids_tgt), p.out_dim), dtype=torch.float32, device=dev)
    ctx = torch.empty((len(ids_ctx), p.out_dim), dtype=torch.float32, device=dev)

    def step():
        if v21:
            J.jepa_predict_mod(pred.handle, z_d, ic, it, w["mask_index"], "video", grid, out, ctx)
        else:
            pred.predict(z_d, ic, it, w["mask_index"], grid, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite predictor output")
    n_ctx, n_tgt = len(ids_ctx), len(ids_tgt)
    work = predictor_work(n_ctx, n_tgt, p.enc_dim, p.embed_dim, p.ffn_dim, p.n_layer, p.out_dim)
    if v21:   # the context rows are normed and projected as well
        b, f = work["gemm_embed"]
        work["gemm_embed"] = (b, f + 2 * n_ctx * p.embed_dim * p.out_dim)
    flops = sum(v for b, v in work.values() if b == "mfma")
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/forward, {n_tgt / (ms * 1e-3):,.0f} target tokens/s, {tflops:.1f} TFLOP/s")
    roof, kernels = None, None
    if not args.no_kernels:
        kernels, _ = kernel_timing(J, step, args.steps, work)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        roof = {"kernel": dom, "bound": k["bound"], "achieved": k.get("tflops", k.get("gbs")),
                "peak": PEAK_BF16_TFLOPS if k["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": "TFLOP/s" if k["bound"] == "mfma" else "GB/s", "frac": k["frac"],
                "traffic": None, "launch_ms": k["avg_ms"]}
        log(f"dominant kernel {dom}: {k['avg_ms'] * 1e3:.1f} us/launch, frac {k['frac']:.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle predictor, 0 and 1 blocks, scaled to 12)")

        def spec(n):
            return oracle.PredictorSpec(p.enc_dim, p.embed_dim, n, p.n_head, p.ffn_dim,
                                        p.n_mask_tokens, p.out_dim, layout=w.get("layout", "tiled"),
                                        has_mod_embed=p.has_mod_embed, has_proj_context=p.has_proj_context)

        def run(n):
            return oracle.predictor_forward(z, Wp, spec(n), ids_ctx, ids_tgt, w["mask_index"], grid,
                                            return_context=v21)
        t0 = time.perf_counter()
        run(0)
        t_fixed = time.perf_counter() - t0
        t0 = time.perf_counter()
        run(1)
        t_layer = max(time.perf_counter() - t0 - t_fixed, 1e-9)
        t_fwd = t_fixed + p.n_layer * t_layer
        try:
            from threadpoolctl import threadpool_info
            cores = max([q.get("num_threads", 1) for q in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": n_tgt / t_fwd, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": (f"float64 numpy oracle predictor, embedding+norm+projection {t_fixed:.2f} s, "
                          f"1 block {t_layer:.2f} s; scaled to {p.n_layer} blocks = {t_fwd:.1f} s")}
    metric = ("predictor target tokens/sec at 1 GPU (V-JEPA 2 ViT-L predictor, 2048 context + "
              "6144 targets); % bf16 MFMA peak")
    wl = ("V-JEPA 2 ViT-L masked predictor on a 32x16x16 grid (8192 tokens): 2048 context + 6144 "
          "target rows, width 384, 12 heads of 32, 12 blocks, bf16 MFMA")
    if v21:
        metric = ("predictor target tokens/sec at 1 GPU (V-JEPA 2.1 ViT-B predictor, 512 context + "
                  "4096 targets on 8x24x24); % bf16 MFMA peak")
        wl = ("V-JEPA 2.1 ViT-B predictor on the 8x24x24 grid of a 16-frame 384-px clip: 512 context + "
              "4096 target rows, width 384, 12 heads of 32, 12 blocks, interleaved RoPE, video modality "
              "vector, targets and context projected to 1664, bf16 MFMA")
    res = {
        "metric": metric,
        "value": round(n_tgt / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) encoder tokens, random N(0,0.02) bf16 weights, seeded tube mask)",
        "config": {"workload": wl,
                   "context_tokens": n_ctx, "target_tokens": n_tgt, "embed_dim": p.embed_dim,
                   "layers": p.n_layer, "heads": p.n_head, "ffn_dim": p.ffn_dim},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops, "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def bench_chain(args):
    """The encoder + predictor chain as one step: the V-JEPA 2 ViT-L/16 encoder on one 64-frame 256-px clip
    (32 x 16 x 16 = 8192 tokens, 24 layers), then the masked predictor on that output (the
    seeded tube mask's 2048 context and 6144 target ids, 12 blocks at width 384, head dim 32).
    ``value`` is clip tokens/s through both."""
    import torch
    import synth
    import video_vit_encoder_amd as J

    w = synth.workload("vitl16_64f256_pred")
    e, p = w["enc"], w["pred"]
    grid = w["grid"]
    N = grid[0] * grid[1] * grid[2]
    log(f"chain workload: 1 clip x {w['frames']} x {w['size']}^2 -> {N} tokens, encoder {e.n_layer} "
        f"blocks, predictor {p.n_layer} blocks; drawing weights")
    W = synth.encoder_weights(e, seed=args.seed, dtype="bf16")
    Wp = synth.predictor_weights(p, seed=args.seed, dtype="bf16")
    clips = synth.clip_u8(args.seed, 1, w["frames"], w["size"], w["size"])
    ids_ctx, ids_tgt = synth.tube_mask(args.seed, *grid)
    dev = torch.device("cuda:0")
    enc = J.Encoder(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim, dtype="bf16", max_rows=N)
    enc.set_weights(W)
    pred = J.Predictor(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim, p.n_mask_tokens,
                       p.out_dim, dtype="bf16", max_rows=len(ids_ctx) + len(ids_tgt))
    pred.set_weights(Wp)
    clip_d = torch.from_numpy(clips).to(dev)
    ic = torch.from_numpy(ids_ctx.astype(np.int32)).to(dev)
    it = torch.from_numpy(ids_tgt.astype(np.int32)).to(dev)
    z = torch.empty((1, N, e.embed_dim), dtype=torch.float32, device=dev)
    out = torch.empty((len(ids_tgt), p.out_dim), dtype=torch.float32, device=dev)

    def step():
        enc.encode(clip_d, out=z)
        pred.predict(z[0], ic, it, w["mask_index"], grid, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite chain output")
    n_ctx, n_tgt = len(ids_ctx), len(ids_tgt)
    work = kernel_work(1, N, e.embed_dim, e.ffn_dim, e.n_layer)
    for name, (bound, v) in predictor_work(n_ctx, n_tgt, p.enc_dim, p.embed_dim, p.ffn_dim,
                                           p.n_layer, p.out_dim).items():
        work[name] = (bound, work[name][1] + v)
    flops = sum(v for b, v in work.values() if b == "mfma")
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {N / (ms * 1e-3):,.0f} clip tokens/s, {tflops:.1f} TFLOP/s")
    roof, kernels = None, None
    if not args.no_kernels:
        kernels, _ = kernel_timing(J, step, args.steps, work)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        roof = {"kernel": dom, "bound": k["bound"], "achieved": k.get("tflops", k.get("gbs")),
                "peak": PEAK_BF16_TFLOPS if k["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": "TFLOP/s" if k["bound"] == "mfma" else "GB/s", "frac": k["frac"],
                "traffic": None, "launch_ms": k["avg_ms"]}
        log(f"dominant kernel {dom}: {k['avg_ms'] * 1e3:.1f} us/launch, frac {k['frac']:.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle: encoder embedding + 1 block, predictor 0 and 1 blocks, scaled)")
        spec = oracle.EncoderSpec(e.embed_dim, 1, e.n_head, e.ffn_dim)
        t0 = time.perf_counter()
        zo = oracle.encoder_forward(clips[0], W, spec)
        t_enc1 = time.perf_counter() - t0
        spec0 = oracle.EncoderSpec(e.embed_dim, 0, e.n_head, e.ffn_dim)
        t0 = time.perf_counter()
        oracle.encoder_forward(clips[0], W, spec0)
        t_enc0 = time.perf_counter() - t0
        t_enc = t_enc0 + e.n_layer * max(t_enc1 - t_enc0, 1e-9)

        def pspec(n):
            return oracle.PredictorSpec(p.enc_dim, p.embed_dim, n, p.n_head, p.ffn_dim,
                                        p.n_mask_tokens, p.out_dim)
        t0 = time.perf_counter()
        oracle.predictor_forward(zo, Wp, pspec(0), ids_ctx, ids_tgt, w["mask_index"], grid)
        t_p0 = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.predictor_forward(zo, Wp, pspec(1), ids_ctx, ids_tgt, w["mask_index"], grid)
        t_p1 = time.perf_counter() - t0
        t_pred = t_p0 + p.n_layer * max(t_p1 - t_p0, 1e-9)
        try:
            from threadpoolctl import threadpool_info
            cores = max([q.get("num_threads", 1) for q in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": N / (t_enc + t_pred), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": (f"float64 numpy oracle: encoder embedding+norm {t_enc0:.1f} s and one block "
                          f"{t_enc1 - t_enc0:.1f} s run, scaled to {e.n_layer} blocks = {t_enc:.0f} s; "
                          f"predictor without blocks {t_p0:.1f} s and one block {t_p1 - t_p0:.1f} s run, "
                          f"scaled to {p.n_layer} blocks = {t_pred:.0f} s; the other blocks are not run; "
                          f"host CPU {host_cpu()}, numpy BLAS on {cores} threads")}
    res = {
        "metric": ("encoder + predictor clip tokens/sec at 1 GPU (V-JEPA 2 ViT-L/16 on a 64-frame "
                   "256-px clip, then the masked predictor); % bf16 MFMA peak"),
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (uniform uint8 clip, random N(0,0.02) bf16 weights, seeded tube mask)",
        "config": {"workload": ("V-JEPA 2 ViT-L/16 encoder on 1 clip x 64 x 256x256 (8192 tokens, 24 "
                                "layers), then the masked predictor on its output: 2048 context + 6144 "
                                "target rows, width 384, 12 heads of 32, 12 blocks, bf16 MFMA"),
                   "clips": 1, "tokens": N, "context_tokens": n_ctx, "target_tokens": n_tgt},
        "clips_per_s": round(1.0 / (ms * 1e-3), 2),
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops, "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def bench_head(args, B=4, N=2048):
    import torch
    import synth
    import video_vit_encoder_amd as J

    s = synth.HeadShape(1024, 3, 16, 4096, 174)
    D, F, L, C = s.embed_dim, s.ffn_dim, s.n_layer, s.n_classes
    log(f"head workload: {B} token maps of {N} x {D}, {L} pool blocks, {C} classes")
    W = synth.head_weights(s, seed=args.seed, dtype="bf16")
    x = synth.tokens_normal(5, B, N, D)
    dev = torch.device("cuda:0")
    head = J.Head(D, L, s.n_head, F, C, dtype="bf16", max_rows=B * N)
    head.set_weights(W)
    x_d = torch.from_numpy(x).to(dev)
    out = torch.empty((B, C), dtype=torch.float32, device=dev)

    def step():
        head.forward(x_d, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite logits")
    M = B * N
    work = kernel_work(B, N, D, F, L, feat=0)
    work.pop("patchify"); work.pop("gemm_embed")
    b_, f_ = work["gemm_qkv"]; work["gemm_qkv"] = (b_, f_ + 2 * 2 * M * D * D)      # + k, v
    b_, f_ = work["attention"]; work["attention"] = (b_, f_ + 4 * B * N * D)         # + 1-query
    b_, f_ = work["gemm_up"]; work["gemm_up"] = (b_, f_ + 2 * B * D * F)
    b_, f_ = work["gemm_down"]; work["gemm_down"] = (b_, f_ + 2 * B * F * D)
    work["gemm_embed"] = ("mfma", 2 * D * D + 2 * B * D * C)                         # q, classifier
    work["layernorm"] = ("hbm", 2 * L * (M * D * 6 + 8 * D) + (M * D * 6 + 8 * D) + (B * D * 6 + 8 * D))
    flops = sum(v for b, v in work.values() if b == "mfma")
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {B / (ms * 1e-3):,.0f} clips/s, {tflops:.1f} TFLOP/s")
    roof, kernels = None, None
    if not args.no_kernels:
        kernels, _ = kernel_timing(J, step, args.steps, work)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        roof = {"kernel": dom, "bound": k["bound"], "achieved": k.get("tflops", k.get("gbs")),
                "peak": PEAK_BF16_TFLOPS if k["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": "TFLOP/s" if k["bound"] == "mfma" else "GB/s", "frac": k["frac"],
                "traffic": None, "launch_ms": k["avg_ms"]}
        log(f"dominant kernel {dom}: {k['avg_ms'] * 1e3:.1f} us/launch, frac {k['frac']:.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle head on one token map)")
        t0 = time.perf_counter()
        oracle.attentive_pool_head(x[0], W, L, s.n_head)
        t1 = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            cores = max([q.get("num_threads", 1) for q in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": 1.0 / t1, "unit": "clips/s", "cores": int(cores), "kind": "oracle",
               "sample": f"float64 numpy oracle head on token map 0 ({N} tokens): {t1:.2f} s"}
    res = {
        "metric": "attentive-pool head clips/sec at 1 GPU (V-JEPA 2 SSv2 head on ViT-L token maps); "
                  "% bf16 MFMA peak",
        "value": round(B / (ms * 1e-3), 2), "unit": "clips/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) token maps, random N(0,0.02) bf16 weights)",
        "config": {"workload": f"attentive-pool head: {B} token maps of {N} x {D}, {L} pool blocks "
                               "(no RoPE), 16 heads, FFN 4096, single-query cross-attention with fp32 "
                               f"k/v, {C} classes, bf16 MFMA",
                   "batch_clips": B, "tokens_per_clip": N, "embed_dim": D, "pool_layers": L,
                   "classes": C},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops, "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def bench_block_causal(args, B=8, n_cls=1, grid=(16, 14, 14), H=16, hd=64):
    import torch
    import video_vit_encoder_amd as J

    slot = grid[1] * grid[2]
    N = n_cls + grid[0] * slot
    D = H * hd
    log(f"block-causal workload: {B} clips of {N} rows ({n_cls} CLS + {grid}), {H} heads of {hd}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(args.seed)
    qkv = torch.randn((B * N, 3 * D), generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty((B * N, D), dtype=torch.bfloat16, device=dev)
    out_full = torch.empty_like(out)
    work = torch.empty(J.jepa_attention_workspace_size(J.JEPA_BF16, B, N, H, hd), dtype=torch.uint8,
                       device=dev)
    ids = torch.from_numpy(np.r_[np.zeros(n_cls), np.arange(N - n_cls)].astype(np.int32)).to(dev)

    def step():
        J.jepa_attention_block_causal(qkv, out, B, n_cls, H, hd, grid, "tiled", work=work)

    def step_full():
        J.jepa_attention(qkv, out_full, B, N, H, hd, ids, grid, "tiled", work=work)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    ms = timed(step)
    ms_full = timed(step_full)
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError("non-finite output")
    # visible (query, key) pairs: CLS rows see all N keys, a patch row of slot t sees (t+1)*slot
    pairs = n_cls * N + slot * slot * sum(t + 1 for t in range(grid[0]))
    flops = 4 * hd * pairs * H * B
    log(f"{ms:.3f} ms/step ({ms_full:.3f} unmasked), {B * N / (ms * 1e-3):,.0f} rows/s, "
        f"density {pairs / N / N:.4f}")
    roof, kernels = None, None
    if not args.no_kernels:
        wk = {"attention": ("mfma", flops),
              "other": ("hbm", B * N * 3 * D * 2 + B * N * 3 * D * 2)}
        kernels, _ = kernel_timing(J, step, args.steps, wk)
        full_k, _ = kernel_timing(J, step_full, args.steps, {"attention": ("mfma", 4 * hd * N * N * H * B)})
        k = kernels["attention"]
        roof = {"kernel": "attention", "bound": "mfma", "achieved": k["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": k["frac"], "traffic": None, "launch_ms": k["avg_ms"]}
        kernels["attention_unmasked_same_rows"] = full_k["attention"]
        log(f"flash kernel: {k['avg_ms'] * 1e3:.1f} us/launch masked, "
            f"{full_k['attention']['avg_ms'] * 1e3:.1f} us unmasked; frac {k['frac']:.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle block-causal attention, whole clips, all heads, >= 10 s)")
        pos = np.concatenate([np.zeros((n_cls, 3)),
                              oracle.rope_positions(np.arange(N - n_cls), grid[1], grid[2], 0)])
        vis = oracle.block_causal_mask(N, n_cls, slot)
        done, t1 = 0, 0.0
        while t1 < 10.0:
            x = qkv[(done % B) * N:(done % B + 1) * N].float().cpu().numpy().astype(np.float64)
            t0 = time.perf_counter()
            oracle.attention(x[:, :D], x[:, D:2 * D], x[:, 2 * D:], H, pos, pos, "tiled", visible=vis)
            t1 += time.perf_counter() - t0
            done += 1
        try:
            from threadpoolctl import threadpool_info
            cores = max([q.get("num_threads", 1) for q in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": round(done * N / t1, 1), "unit": "rows/s", "cores": int(cores), "kind": "oracle",
               "sample": f"float64 numpy oracle attention with the block-causal mask on {done} whole "
                         f"clips ({N} rows, {H} heads each): {t1:.2f} s"}
    res = {
        "metric": "block-causal attention rows/sec at 1 GPU (LeVJEPA ViT-L/16 shape, 16f/224px + CLS); "
                  "% bf16 MFMA peak",
        "value": round(B * N / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) q/k/v rows rounded to bf16)",
        "config": {"workload": f"block-causal attention: {B} clips of {N} rows (CLS + 16 x 14 x 14 patch "
                               f"tokens, slots of {slot}), {H} heads of {hd}, tiled 3-D RoPE, bf16 MFMA",
                   "batch_clips": B, "rows_per_clip": N, "n_cls": n_cls, "slot": slot, "heads": H,
                   "head_dim": hd, "mask_density": round(pairs / N / N, 4)},
        "ms_per_step_unmasked": round(ms_full, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "flops_per_step": flops,
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def bench_image(args, B=16):
    import torch
    import synth
    import video_vit_encoder_amd as J

    w = synth.workload("vitb16_img384")
    e = w["enc"]
    S = w["size"]
    N = w["grid"][1] * w["grid"][2]
    D, F, L, H = e.embed_dim, e.ffn_dim, e.n_layer, e.n_head
    log(f"image workload: {B} images {S}x{S}, N={N}, D={D}, L={L}; drawing weights")
    W = synth.encoder_weights(e, seed=args.seed, dtype="bf16")
    imgs = synth.clip_u8(args.seed, B, 1, S, S)[:, 0]
    dev = torch.device("cuda:0")
    enc = J.Encoder(D, L, H, F, layout=w["layout"], ref_grid=w["ref_grid"], has_mod_embed=True,
                    dtype="bf16", max_rows=B * N, has_image_embed=True)
    enc.set_weights(W)
    img_d = torch.from_numpy(imgs).to(dev)
    out = torch.empty((B, N, D), dtype=torch.float32, device=dev)

    def step():
        enc.encode_image(img_d, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite encoder output")
    feat = 768
    flops = forward_flops(B, N, D, F, L, feat=feat)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {B * N / (ms * 1e-3):,.0f} tokens/s, {tflops:.1f} TFLOP/s")
    roof, kernels = None, None
    if not args.no_kernels:
        work = kernel_work(B, N, D, F, L, feat=feat)
        kernels, _ = kernel_timing(J, step, args.steps, work)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        roof = {"kernel": dom, "bound": k["bound"], "achieved": k.get("tflops", k.get("gbs")),
                "peak": PEAK_BF16_TFLOPS if k["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": "TFLOP/s" if k["bound"] == "mfma" else "GB/s", "frac": k["frac"],
                "traffic": None, "launch_ms": k["avg_ms"]}
        log(f"dominant kernel {dom}: {k['avg_ms'] * 1e3:.1f} us/launch, frac {k['frac']:.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle image path, 0 and 2 blocks, scaled to 12)")

        def spec(n):
            return oracle.EncoderSpec(D, n, H, F, has_mod_embed=True, layout=w["layout"],
                                      ref_grid=w["ref_grid"])
        t0 = time.perf_counter()
        oracle.encoder_forward_image(imgs[0], W, spec(0))
        t_fixed = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.encoder_forward_image(imgs[0], W, spec(2))
        t_layer = max(time.perf_counter() - t0 - t_fixed, 1e-9) / 2
        t_img = t_fixed + L * t_layer
        try:
            from threadpoolctl import threadpool_info
            cores = max([q.get("num_threads", 1) for q in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": N / t_img, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": (f"float64 numpy oracle image path, image 0 ({N} tokens): embedding+norm "
                          f"{t_fixed:.2f} s, 2 blocks {2 * t_layer:.2f} s; scaled to {L} blocks = {t_img:.1f} s")}
    res = {
        "metric": "image tokens/sec at 1 GPU (V-JEPA 2.1 ViT-B/16 image path, 384px); % bf16 MFMA peak",
        "value": round(B * N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (uniform uint8 images, random N(0,0.02) bf16 weights)",
        "config": {"workload": f"V-JEPA 2.1 ViT-B/16 native image path, {B} images x 384x384 (576 tokens "
                               "each), tubelet-1 patches, image modality vector, interleaved RoPE "
                               "interpolated to 16, 12 layers, bf16 MFMA",
                   "batch_images": B, "tokens_per_image": N, "embed_dim": D, "layers": L, "heads": H,
                   "ffn_dim": F},
        "images_per_s": round(B / (ms * 1e-3), 2),
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops, "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


def host_cpu() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the baseline record."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_rope3d(args, B=4, N=2048, H=16, hd=64, grid=(8, 16, 16)):
    """The stand-alone 3-D RoPE (jepa_rope3d), fp32, out of place, on the q tensor of the
    ViT-L batch: [B, N, H, hd] rows, tiled layout on the clip's grid.  HBM-bound:
    8*B*N*H*hd algorithmic bytes per call (fp32 read and write)."""
    import torch
    import oracle
    import video_vit_encoder_amd as J

    log(f"rope3d workload: fp32 [{B}, {N}, {H}, {hd}], tiled, grid {grid}")
    dev = torch.device("cuda:0")
    x_h = np.random.default_rng(args.seed).standard_normal((B, N, H, hd)).astype(np.float32)
    x = torch.from_numpy(x_h).to(dev)
    y = torch.empty_like(x)

    def step():
        J.jepa_rope3d(x, y, B, N, H, hd, H * hd, None, grid, "tiled")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    nbytes = 8 * B * N * H * hd
    gbs = nbytes / (ms * 1e-3) / 1e9
    # one launch per call: the step is the kernel
    roof = {"kernel": "rope3d", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("rope3d"),
            "launch_ms": round(ms, 5), "bytes_per_launch": nbytes}
    log(f"{ms * 1e3:.1f} us/call, {gbs:,.0f} GB/s ({gbs / PEAK_HBM_GBS:.3f} of HBM)")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle rope_rotate on clip 0)")
        pos = oracle.rope_positions(np.arange(N), grid[1], grid[2], 0)
        u = np.transpose(x_h[0], (1, 0, 2))               # [H, N, hd]
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.rope_rotate(u, pos, "tiled")
            reps += 1
            if time.perf_counter() - t0 > 10.0:
                break
        t = (time.perf_counter() - t0) / reps
        cpu = {"value": round(8 * N * H * hd / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"float64 numpy oracle rope_rotate on clip 0 ([{H}, {N}, {hd}]), {reps} repetitions "
                         f"in {time.perf_counter() - t0:.1f} s, bytes counted as the fp32 call's; "
                         f"host CPU {host_cpu()}"}
    res = {
        "metric": "stand-alone 3-D RoPE HBM GB/s at 1 GPU (fp32 q of the ViT-L 4 x 2048-token batch); "
                  "% HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (N(0,1) fp32 head vectors)",
        "config": {"workload": f"jepa_rope3d fp32 out of place on [{B}, {N}, {H}, {hd}] (4 clips x 2048 "
                               "tokens x 16 heads x 64), tiled, grid 8x16x16, no interpolation",
                   "batch_clips": B, "tokens_per_clip": N, "heads": H, "head_dim": hd},
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": nbytes,
        "roofline": roof, "cpu_baseline": cpu, "kernels": None,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--predictor", action="store_true",
                    help="time the masked predictor (jepa_predict) on its 8192-token workload")
    ap.add_argument("--v21", action="store_true",
                    help="with --predictor: the V-JEPA 2.1 ViT-B predictor (jepa_predict_mod)")
    ap.add_argument("--chain", action="store_true",
                    help="time the ViT-L encoder on one 64-frame 256-px clip (8192 tokens), "
                         "then the masked predictor on its output, as one step")
    ap.add_argument("--head", action="store_true",
                    help="time the attentive-pool classifier head on 4 ViT-L token maps")
    ap.add_argument("--image", action="store_true",
                    help="time the V-JEPA 2.1 ViT-B/16 image path on 16 images of 384x384")
    ap.add_argument("--vitb384", action="store_true",
                    help="time the V-JEPA 2.1 ViT-B/16 encoder on one 64-frame 384x384 clip "
                         "(18,432 tokens) instead of the ViT-L batch")
    ap.add_argument("--block-causal", action="store_true",
                    help="time the block-causal attention with a CLS row at the LeVJEPA shape")
    ap.add_argument("--masked", action="store_true",
                    help="time the masked-encoder forward on tube-mask contexts (512 of 2048 "
                         "tokens per clip) instead of the full forward")
    ap.add_argument("--rope3d", action="store_true",
                    help="time the stand-alone 3-D RoPE (jepa_rope3d, fp32) on the ViT-L q tensor")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy 3 times, the "
                         "reference for scaling HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.chain:
        bench_chain(args)
        return
    if args.predictor:
        bench_predictor(args)
        return
    if args.image:
        bench_image(args)
        return
    if args.head:
        bench_head(args)
        return
    if args.block_causal:
        bench_block_causal(args)
        return
    if args.rope3d:
        bench_rope3d(args)
        return

    import torch
    import synth
    import video_vit_encoder_amd as J

    wl = "vitb16_64f384" if args.vitb384 else WORKLOAD
    w = synth.workload(wl)
    e = w["enc"]
    B, T, S = w["B"], w["frames"], w["size"]
    N = w["grid"][0] * w["grid"][1] * w["grid"][2]
    D, F, L, H = e.embed_dim, e.ffn_dim, e.n_layer, e.n_head
    log(f"workload {wl}: B={B} T={T} {S}x{S} N={N} D={D} L={L}; drawing weights")
    W = synth.encoder_weights(e, seed=args.seed, dtype="bf16")
    clips = synth.clip_u8(args.seed, B, T, S, S)
    dev = torch.device("cuda:0")
    enc = J.Encoder(D, L, H, F, layout=w["layout"], ref_grid=w["ref_grid"], dtype="bf16",
                    max_rows=B * N, has_mod_embed=e.has_mod_embed)
    enc.set_weights(W)
    clip_d = torch.from_numpy(clips).to(dev)
    ids = None
    if args.masked:
        ids = np.stack([synth.tube_mask(args.seed + b, *w["grid"])[0] for b in range(B)])
        ids_d = torch.from_numpy(ids.astype(np.int32)).to(dev)
        K = ids.shape[1]
        out = torch.empty((B, K, D), dtype=torch.float32, device=dev)

        def step():
            enc.encode_masked(clip_d, ids_d, out=out)
    else:
        K = N
        out = torch.empty((B, N, D), dtype=torch.float32, device=dev)

        def step():
            enc.encode(clip_d, out=out)
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite encoder output")
    tok_s = B * K / (ms * 1e-3)
    flops = forward_flops(B, K, D, F, L)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {tok_s:,.0f} tokens/s, {tflops:.1f} TFLOP/s "
        f"(wall {t_wall * 1e3 / args.steps:.3f} ms/step)")

    roof, kernels = None, None
    if not args.no_kernels:
        log(f"per-kernel launch timing over {args.steps} more steps (HIP events in the library)")
        kernels, prof_ms = kernel_timing(J, step, args.steps, kernel_work(B, K, D, F, L))
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        # the committed counter passes were taken on the full ViT-L forward's shapes
        traffic = None if args.masked or args.vitb384 else measured_traffic(dom)
        if k["bound"] == "mfma":
            roof = {"kernel": dom, "bound": "mfma", "achieved": k["tflops"],
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": k["frac"],
                    "traffic": traffic, "launch_ms": k["avg_ms"],
                    "flops_per_launch": k["flops_per_launch"]}
        else:
            roof = {"kernel": dom, "bound": "hbm", "achieved": k["gbs"],
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": k["frac"],
                    "traffic": traffic, "launch_ms": k["avg_ms"],
                    "bytes_per_launch": k["bytes_per_launch"]}
        log(f"dominant kernel {dom}: {k['avg_ms'] * 1e3:.1f} us/launch, frac {k['frac']:.3f}; "
            f"timed pass {prof_ms:.3f} ms/step (wall)")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        if args.vitb384:
            # bounded sample: the clip's embedding and final norm, and one of the 12 blocks
            # timed on its own, scaled to the 12 blocks
            cpu = cpu_baseline(w, W, clips, budget_layers=1, direct=True)
        else:
            cpu = cpu_baseline(w, W, clips, ids0=None if ids is None else ids[0])

    metric = "encoder tokens/sec at 1 GPU (ViT-L, 16f/256px); % bf16 MFMA peak"
    workload = ("V-JEPA 2 ViT-L/16 encoder forward, 4 clips x 16 frames x 256x256 (2048 tokens "
                "per clip), 24 layers, bf16 MFMA")
    if args.masked:
        metric = "masked-encoder context tokens/sec at 1 GPU (ViT-L, 16f/256px); % bf16 MFMA peak"
        workload = ("V-JEPA 2 ViT-L/16 masked-encoder forward, 4 clips x 16 frames x 256x256, "
                    f"context = tube mask of 8x8 patches in each of 8 temporal slots ({K} of "
                    f"{N} tokens per clip), 24 layers, bf16 MFMA")
    rope = "tiled 3-D"
    if args.vitb384:
        metric = ("encoder tokens/sec at 1 GPU (V-JEPA 2.1 ViT-B/16, 64f/384px, 18,432 tokens); "
                  "% bf16 MFMA peak")
        workload = ("V-JEPA 2.1 ViT-B/16 encoder forward, 1 clip x 64 frames x 384x384 (18,432 tokens), "
                    "12 layers, interleaved 3-D RoPE interpolated to 16, video modality vector, bf16 MFMA")
        rope = "interleaved 3-D, interpolation 16"
    res = {
        "metric": metric,
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (uniform uint8 clips, random N(0,0.02) bf16 weights)",
        "config": {"workload": workload,
                   "batch_clips": B, "tokens_per_clip": K, "embed_dim": D, "layers": L,
                   "heads": H, "ffn_dim": F, "rope": rope},
        "clips_per_s": round(B / (ms * 1e-3), 2),
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
