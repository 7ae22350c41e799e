"""Throughput of the V-JEPA 2 ViT-L/16 encoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one jepa_encode call on a batch of 4 synthetic clips of 16 frames x 256x256
uint8 (2048 tokens per clip, 8192 token rows), already resident in HBM: patch
embedding, 24 pre-norm blocks with 3-D RoPE attention and the final norm, in bf16 MFMA
with fp32 accumulation.  Weights are random N(0, 0.02) rounded to bf16, biases
N(0, 0.01), LayerNorm 1/0; the clips are uniform uint8 (no dataset, no checkpoint).

Prints one JSON line.  ``value`` is encoder tokens/s over the K timed steps (HIP events
on the stream the library launches on, bracketed by device synchronisation).  Beside it:
  * ``roofline``: the dominant kernel (the largest share of a step's time, its launch
    durations measured here with HIP events through the library's stand-alone entry
    points at the step's shapes), its algorithmic TFLOP/s or GB/s against the MI355X
    peak (bf16 dense MFMA 2500 TFLOP/s, HBM 8000 GB/s);
  * ``kernels``: the same figures for every kernel class of the step;
  * ``cpu_baseline``: the float64 oracle timed on the host on one clip through a few
    layers, scaled to the 24-layer forward (a reported baseline, not a target).
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


def time_launches(fn, reps, warm=3):
    """Average duration (ms) of fn() over reps launches, HIP events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def kernel_breakdown(w, B, N, D, F, H, hd, L):
    """Per-kernel launch durations at the step's shapes, through the C ABI."""
    import torch
    import video_vit_encoder_amd as J
    dev = torch.device("cuda:0")
    M = B * N
    g = torch.Generator(device=dev).manual_seed(0)

    def rn(*shape, scale=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shape, generator=g, device=dev) * scale).to(dtype)

    x = rn(M, D, dtype=torch.float32)
    h = rn(M, D)
    lw, lb = torch.ones(D, device=dev), torch.zeros(D, device=dev)
    Wqkv, bqkv = rn(3 * D, D, scale=0.02), rn(3 * D, scale=0.01, dtype=torch.float32)
    Wo, bo = rn(D, D, scale=0.02), rn(D, scale=0.01, dtype=torch.float32)
    Wu, bu = rn(F, D, scale=0.02), rn(F, scale=0.01, dtype=torch.float32)
    Wd, bd = rn(D, F, scale=0.02), rn(D, scale=0.01, dtype=torch.float32)
    qkv = torch.empty(M, 3 * D, device=dev, dtype=torch.bfloat16)
    o = rn(M, D)
    gg = torch.empty(M, F, device=dev, dtype=torch.bfloat16)
    grid = w["grid"]
    J.jepa_linear(h, Wqkv, bqkv, qkv, J.JEPA_EPI_STORE)
    J.jepa_linear(h, Wu, bu, gg, J.JEPA_EPI_GELU)
    reps = 20
    ks = {}
    ks["layernorm"] = dict(
        ms=time_launches(lambda: J.jepa_layernorm(x, lw, lb, 1e-6, h), reps), per_step=2 * L + 1,
        bound="hbm", bytes=M * D * (4 + 2) + 2 * D * 4)
    ks["gemm_qkv"] = dict(
        ms=time_launches(lambda: J.jepa_linear(h, Wqkv, bqkv, qkv, J.JEPA_EPI_STORE), reps),
        per_step=L, bound="mfma", flops=2 * M * D * 3 * D)
    ks["attention"] = dict(
        ms=time_launches(lambda: J.jepa_attention(qkv, o, B, N, H, hd, None, grid, "tiled"), reps),
        per_step=L, bound="mfma", flops=4 * B * N * N * D)
    ks["gemm_out_residual"] = dict(
        ms=time_launches(lambda: J.jepa_linear(o, Wo, bo, x, J.JEPA_EPI_RESIDUAL), reps),
        per_step=L, bound="mfma", flops=2 * M * D * D)
    ks["gemm_ffn_up_gelu"] = dict(
        ms=time_launches(lambda: J.jepa_linear(h, Wu, bu, gg, J.JEPA_EPI_GELU), reps),
        per_step=L, bound="mfma", flops=2 * M * D * F)
    ks["gemm_ffn_down_residual"] = dict(
        ms=time_launches(lambda: J.jepa_linear(gg, Wd, bd, x, J.JEPA_EPI_RESIDUAL), reps),
        per_step=L, bound="mfma", flops=2 * M * F * D)
    for k, v in ks.items():
        if v["bound"] == "mfma":
            v["tflops"] = v["flops"] / (v["ms"] * 1e-3) / 1e12
            v["frac"] = v["tflops"] / PEAK_BF16_TFLOPS
        else:
            v["gbs"] = v["bytes"] / (v["ms"] * 1e-3) / 1e9
            v["frac"] = v["gbs"] / PEAK_HBM_GBS
        v["ms_per_step"] = v["ms"] * v["per_step"]
    torch.cuda.synchronize()
    return ks


def cpu_baseline(w, W, clips, budget_layers=12):
    """The float64 oracle on clip 0: patch embedding + final norm alone, then with
    ``budget_layers`` blocks; the per-block time scales the forward to 24 blocks."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    e = w["enc"]

    def spec(n):
        return oracle.EncoderSpec(e.embed_dim, n, e.n_head, e.ffn_dim, layout=w["layout"])

    t0 = time.perf_counter()
    oracle.encoder_forward(clips[0], W, spec(0))
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.encoder_forward(clips[0], W, spec(budget_layers))
    t_run = time.perf_counter() - t0
    t_layer = max(t_run - t_fixed, 1e-9) / budget_layers
    t_clip = t_fixed + e.n_layer * t_layer
    N = w["grid"][0] * w["grid"][1] * w["grid"][2]
    return {"value": N / t_clip, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float64 numpy oracle, clip 0 only (2048 tokens): embedding+norm "
                       f"{t_fixed:.2f} s, {budget_layers} blocks {t_run - t_fixed:.2f} s; "
                       f"scaled to 24 blocks = {t_clip:.1f} s/clip")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import video_vit_encoder_amd as J

    w = synth.workload(WORKLOAD)
    e = w["enc"]
    B, T, S = w["B"], w["frames"], w["size"]
    N = w["grid"][0] * w["grid"][1] * w["grid"][2]
    D, F, L, H = e.embed_dim, e.ffn_dim, e.n_layer, e.n_head
    log(f"workload {WORKLOAD}: B={B} T={T} {S}x{S} N={N} D={D} L={L}; drawing weights")
    W = synth.encoder_weights(e, seed=args.seed, dtype="bf16")
    clips = synth.clip_u8(args.seed, B, T, S, S)
    dev = torch.device("cuda:0")
    enc = J.Encoder(D, L, H, F, layout=w["layout"], ref_grid=w["ref_grid"], dtype="bf16",
                    max_rows=B * N)
    enc.set_weights(W)
    clip_d = torch.from_numpy(clips).to(dev)
    out = torch.empty((B, N, D), dtype=torch.float32, device=dev)
    log("warmup")
    for _ in range(args.warmup):
        enc.encode(clip_d, out=out)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        enc.encode(clip_d, out=out)
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("non-finite encoder output")
    tok_s = B * N / (ms * 1e-3)
    flops = forward_flops(B, N, D, F, L)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {tok_s:,.0f} tokens/s, {tflops:.1f} TFLOP/s "
        f"(wall {t_wall * 1e3 / args.steps:.3f} ms/step)")

    roof, kernels = None, None
    if not args.no_kernels:
        log("per-kernel launch timing")
        kernels = kernel_breakdown(w, B, N, D, F, H, D // H, L)
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        k = kernels[dom]
        if k["bound"] == "mfma":
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(k["tflops"], 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(k["frac"], 4),
                    "traffic": None, "launch_ms": round(k["ms"], 4),
                    "flops_per_launch": k["flops"]}
        else:
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(k["gbs"], 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(k["frac"], 4),
                    "traffic": None, "launch_ms": round(k["ms"], 4),
                    "bytes_per_launch": k["bytes"]}
        kernels = {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for n, v in kernels.items()}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(w, W, clips)

    res = {
        "metric": "encoder tokens/sec at 1 GPU (ViT-L, 16f/256px); % bf16 MFMA peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (uniform uint8 clips, random N(0,0.02) bf16 weights)",
        "config": {"workload": "V-JEPA 2 ViT-L/16 encoder forward, 4 clips x 16 frames x "
                               "256x256 (2048 tokens per clip), 24 layers, bf16 MFMA",
                   "batch_clips": B, "tokens_per_clip": N, "embed_dim": D, "layers": L,
                   "heads": H, "ffn_dim": F, "rope": "tiled 3-D"},
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
