"""Write the oracle's values for the two full-size parity cases whose float64 forward
takes too long to run inside a GPU test:

  * ``vitb21_384_full.npz``: the V-JEPA 2.1 ViT-B/16 encoder (12 layers, interleaved RoPE
    interpolated to 16, video modality vector) on one 64 x 384 x 384 clip, the full
    32 x 24 x 24 grid of 18,432 tokens ([HFport "Usage"]; [Notes §4.3]); every layer runs
    on all rows except the last, which the oracle evaluates on 195 sampled rows (rows 0,
    575 and 18431 and 192 drawn ones);
  * ``vitl16_64f_chain.npz``: the V-JEPA 2 ViT-L/16 encoder (24 layers, tiled) on one
    64 x 256 x 256 clip (32 x 16 x 16 = 8192 tokens, [Card] "Measured" / [Parity "Results
    -- video encoders"]), its last layer on the 2048 context rows of the tube mask plus 192
    drawn rows; then the masked predictor ([Notes §3] "2.1 predictor forward" order of
    operations, [Notes §4.4] ids) fed with that output, its last layer on 128 drawn target
    rows.

This script calls only ``oracle`` and ``synth``: no value here comes from the HIP path.
Values are stored as float32 (the parity gates are a cosine of 1e-4 and a relative error
of 2e-2).  Each file records the input recipe, the sampled rows, a SHA-256 of the drawn
inputs and of the oracle's source; ``tests/test_golden_fullsize.py`` checks that both
still match, so a change to either makes the stale file fail loudly.

    python tests/golden/make_fullsize.py [vitb21|chain|all]
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

VITB_FILE = os.path.join(HERE, "vitb21_384_full.npz")
CHAIN_FILE = os.path.join(HERE, "vitl16_64f_chain.npz")


def oracle_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("vjepa.py",):
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def inputs_sha(*arrays, weights=None) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    if weights is not None:
        for k in sorted(weights):
            h.update(k.encode())
            h.update(np.ascontiguousarray(weights[k]).tobytes())
    return h.hexdigest()


# ------------------------------------------------------------------ the two cases


def vitb21_case():
    """Inputs and sampled rows of the 12-layer 2.1 ViT-B case."""
    w = synth.workload("vitb16_64f384")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    clip = synth.clip_u8(0, 1, 64, 384, 384)
    rows = np.sort(np.random.default_rng(7).choice(18432, 192, replace=False))
    rows = np.concatenate([[0, 575, 18431], rows]).astype(np.int64)
    return w, W, clip, rows


def chain_case():
    """Inputs and sampled rows of the 64-frame ViT-L encoder + predictor chain."""
    w = synth.workload("vitl16_64f256_pred")
    W = synth.encoder_weights(w["enc"], seed=0, dtype="bf16")
    Wp = synth.predictor_weights(w["pred"], seed=0, dtype="bf16")
    clip = synth.clip_u8(0, 1, 64, 256, 256)
    ids_ctx, ids_tgt = synth.tube_mask(0, *w["grid"])
    enc_rows = np.sort(np.random.default_rng(9).choice(8192, 192, replace=False)).astype(np.int64)
    tgt_rows = np.sort(np.random.default_rng(10).choice(len(ids_tgt), 128, replace=False)).astype(np.int64)
    return w, W, Wp, clip, ids_ctx, ids_tgt, enc_rows, tgt_rows


def enc_spec(w):
    e = w["enc"]
    return oracle.EncoderSpec(e.embed_dim, e.n_layer, e.n_head, e.ffn_dim,
                              has_mod_embed=e.has_mod_embed, final_norm=e.final_norm,
                              layout=w["layout"], ref_grid=w["ref_grid"])


def pred_spec(p):
    return oracle.PredictorSpec(p.enc_dim, p.embed_dim, p.n_layer, p.n_head, p.ffn_dim,
                                p.n_mask_tokens, p.out_dim)


def _meta(recipe: str, sha: str) -> np.ndarray:
    return np.array(json.dumps({"recipe": recipe, "inputs_sha256": sha,
                                "oracle_sha256": oracle_source_sha(), "dtype": "float32"}))


def make_vitb21() -> None:
    t0 = time.time()
    w, W, clip, rows = vitb21_case()
    print(f"vitb21: 12 layers on 18432 tokens, last layer on {len(rows)} rows", flush=True)
    ref = oracle.encoder_forward(clip[0], W, enc_spec(w), last_rows=rows)
    recipe = ("V-JEPA 2.1 ViT-B/16, 12 layers, interleaved RoPE, ref grid 16, mod_embed_video; "
              "synth.encoder_weights(seed=0, bf16), synth.clip_u8(0, 1, 64, 384, 384); "
              "rows = [0, 575, 18431] + sorted(default_rng(7).choice(18432, 192))")
    np.savez(VITB_FILE, rows=rows, out=ref.astype(np.float32),
             meta=_meta(recipe, inputs_sha(clip, weights=W)))
    print(f"vitb21: wrote {VITB_FILE} in {time.time() - t0:.0f} s", flush=True)


def make_chain() -> None:
    t0 = time.time()
    w, W, Wp, clip, ids_ctx, ids_tgt, enc_rows, tgt_rows = chain_case()
    last = np.union1d(ids_ctx, enc_rows)
    print(f"chain: ViT-L 24 layers on 8192 tokens, last layer on {len(last)} rows", flush=True)
    z_rows = oracle.encoder_forward(clip[0], W, enc_spec(w), last_rows=last)
    z = np.zeros((8192, w["enc"].embed_dim))
    z[last] = z_rows
    print(f"chain: encoder done in {time.time() - t0:.0f} s; predictor 12 layers on "
          f"{len(ids_ctx) + len(ids_tgt)} rows", flush=True)
    pred = oracle.predictor_forward(z, Wp, pred_spec(w["pred"]), ids_ctx, ids_tgt, w["mask_index"],
                                    w["grid"], last_rows=tgt_rows)
    recipe = ("V-JEPA 2 ViT-L/16, 24 layers, tiled; synth.encoder_weights(seed=0, bf16), "
              "synth.clip_u8(0, 1, 64, 256, 256); predictor synth.predictor_weights(seed=0, bf16) "
              "384/12/12/1536, 10 mask tokens, mask_index 1, synth.tube_mask(0, 32, 16, 16); "
              "enc_rows = sorted(default_rng(9).choice(8192, 192)); "
              "tgt_rows = sorted(default_rng(10).choice(6144, 128))")
    np.savez(CHAIN_FILE, enc_rows=enc_rows, enc_out=z[enc_rows].astype(np.float32),
             tgt_rows=tgt_rows, pred_out=pred.astype(np.float32),
             meta=_meta(recipe, inputs_sha(clip, ids_ctx, ids_tgt, weights={**W, **Wp})))
    print(f"chain: wrote {CHAIN_FILE} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    what = sys.argv[1] if len(sys.argv) > 1 else "all"
    if what in ("vitb21", "all"):
        make_vitb21()
    if what in ("chain", "all"):
        make_chain()
