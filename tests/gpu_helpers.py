"""Helpers of the GPU parity tests: device transfers, the gates, case banners.

Gates (stated for this path): standalone fp32 RoPE max |diff| <= 1e-5; the fp32 encoder
rel_max <= 1e-3; the bf16 MFMA path mean per-token cosine >= 0.9999 and rel_max <= 2e-2,
with rel_max = max|gpu - oracle| / max|oracle| and cosines computed in float64 against
the oracle ([Parity "Results -- image models"] metric definitions).
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import metrics

ROPE_F32_MAX_ABS = 1e-5
F32_REL_MAX = 1e-3
BF16_COS_MEAN = 0.9999
BF16_REL_MAX = 2e-2


def banner(*parts) -> None:
    """Name the case on stdout (flushed) before its GPU work starts."""
    sys.stdout.write("[case] " + " ".join(str(p) for p in parts) + "\n")
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bf16(a):
    """bf16 device tensor holding float32 values (exact when they are bf16-valued)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev()).to(torch.bfloat16)


def i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_bf16_gate(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    s = metrics.summary(gpu, ref)
    print(f"  {what} cos_mean={s['cos_mean']:.7f} cos_min={s['cos_min']:.6f} "
          f"rel_max={s['rel_max']:.3e}")
    assert np.all(np.isfinite(gpu)), what
    assert s["cos_mean"] >= BF16_COS_MEAN, (what, s)
    assert s["rel_max"] <= BF16_REL_MAX, (what, s)
    return s


def assert_f32_gate(gpu: np.ndarray, ref: np.ndarray, what: str = "", bound: float = F32_REL_MAX) -> float:
    r = metrics.rel_max(gpu, ref)
    print(f"  {what} rel_max={r:.3e}")
    assert np.all(np.isfinite(gpu)), what
    assert r <= bound, (what, r)
    return r
