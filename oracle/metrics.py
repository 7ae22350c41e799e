"""Parity metrics, computed in float64 (test infrastructure).

Definitions from [Parity "Results -- image models"]: per-token cosine between rows of
the two token maps, summarised as mean / median / min, and
rel_max = max|a - b| / max|b| with b the reference (here: the oracle).
"""
from __future__ import annotations

import numpy as np


def per_token_cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, b.shape[-1])
    num = (a * b).sum(axis=1)
    den = np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1)
    return num / np.maximum(den, 1e-300)


def rel_max(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def summary(a: np.ndarray, b: np.ndarray) -> dict:
    c = per_token_cosine(a, b)
    return dict(cos_mean=float(c.mean()), cos_median=float(np.median(c)), cos_min=float(c.min()),
                worst_row=int(np.argmin(c)), rel_max=rel_max(a, b), max_abs=max_abs(a, b))
