"""The stored oracle values of the full-size parity cases (``tests/golden/*.npz``, written
by ``tests/golden/make_fullsize.py`` from ``oracle`` and ``synth`` only) still belong to
the current inputs and the current oracle: the drawn inputs and the oracle's source hash
to the values recorded in each file.  A change to either makes this fail; rerun the
script (it takes tens of minutes of float64 work) to refresh the files."""
import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_fullsize as mf  # noqa: E402


def _meta(path):
    with np.load(path, allow_pickle=False) as z:
        return json.loads(str(z["meta"])), {k: z[k] for k in z.files if k != "meta"}


def test_oracle_source_matches_the_goldens():
    for path in (mf.VITB_FILE, mf.CHAIN_FILE):
        meta, _ = _meta(path)
        assert meta["oracle_sha256"] == mf.oracle_source_sha(), (
            f"{os.path.basename(path)} was written by another oracle; rerun make_fullsize.py")


def test_vitb21_golden_inputs_and_shapes():
    meta, d = _meta(mf.VITB_FILE)
    w, W, clip, rows = mf.vitb21_case()
    assert meta["inputs_sha256"] == mf.inputs_sha(clip, weights=W)
    assert np.array_equal(d["rows"], rows)
    assert d["out"].shape == (len(rows), 768) and np.all(np.isfinite(d["out"]))
    # final norm with weight 1 and bias 0: every row has mean 0 and mean square near 1
    assert np.max(np.abs(d["out"].mean(axis=1))) < 1e-5


def test_chain_golden_inputs_and_shapes():
    meta, d = _meta(mf.CHAIN_FILE)
    w, W, Wp, clip, ids_ctx, ids_tgt, enc_rows, tgt_rows = mf.chain_case()
    assert meta["inputs_sha256"] == mf.inputs_sha(clip, ids_ctx, ids_tgt, weights={**W, **Wp})
    assert np.array_equal(d["enc_rows"], enc_rows) and np.array_equal(d["tgt_rows"], tgt_rows)
    assert d["enc_out"].shape == (192, 1024) and d["pred_out"].shape == (128, 1024)
    assert np.all(np.isfinite(d["enc_out"])) and np.all(np.isfinite(d["pred_out"]))
