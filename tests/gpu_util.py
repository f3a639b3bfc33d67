"""Helpers shared by the GPU parity tests: comparison rows in the parity report's schema
("Proving it's the same model", ``logits_parity``: max and mean absolute error, argmax
agreement, tolerance, finiteness), and oracle runs of a batch."""

from __future__ import annotations

import json
import os

import numpy as np
import torch


def gpu_available() -> bool:
    return torch.cuda.is_available()


def compare(gpu: np.ndarray, ref: np.ndarray, tol: float | None = None, rel_range: float | None = None) -> dict:
    """Parity row of ``gpu`` (float32) against ``ref`` (float64), per P1's fields.

    tol: absolute gate on the max error; rel_range: per-row gate as a fraction of the
    row's oracle logit range (max - min).
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    delta = np.abs(gpu - ref)
    rng = ref.max(axis=-1) - ref.min(axis=-1)
    row_max = delta.max(axis=-1)
    agree = int(np.sum(np.argmax(gpu, axis=-1) == np.argmax(ref, axis=-1)))
    row = {
        "max_absolute_error": float(delta.max()),
        "mean_absolute_error": float(delta.mean()),
        "argmax_agreement": agree,
        "positions": int(ref.shape[0]),
        "finite": bool(np.isfinite(gpu).all()),
        "logit_range_median": float(np.median(rng)),
        "max_error_over_range": float(np.max(row_max / rng)),
    }
    if tol is not None:
        row["tolerance"] = tol
        row["pass"] = row["finite"] and row["max_absolute_error"] <= tol
    if rel_range is not None:
        row["tolerance_rel_range"] = rel_range
        row["pass"] = row["finite"] and bool(np.all(row_max <= rel_range * rng))
    return row


def report(row: dict) -> None:
    """Append a parity row to $DEC_REPORT_DIR/parity.jsonl when that directory is set."""
    d = os.environ.get("DEC_REPORT_DIR")
    print(json.dumps(row), flush=True)
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "parity.jsonl"), "a") as f:
            f.write(json.dumps(row) + "\n")
