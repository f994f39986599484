"""Comparison of the HIP path's outputs with the oracle's (test helper).

Tolerances are the ones the quantizer is held to: >= 99.9 % identical
integer codes, group scales/zero points within 1e-5 relative, layer loss
within 1e-3 relative. A code that flips near a rounding tie changes the
error fed to later columns of that row, so scales/zeros of later groups of
that row may legitimately differ; they are compared as a fraction too.
"""
from __future__ import annotations

import sys

import numpy as np

CODE_AGREE = 0.999
SCALE_RTOL = 1e-5
SCALE_AGREE = 0.999
LOSS_RTOL = 1e-3


def first_divergence(a, b):
    """Per row: index of the first differing column (cols if none)."""
    d = a != b
    cols = a.shape[1]
    return np.where(d.any(axis=1), d.argmax(axis=1), cols)


def compare_layer(gpu, ref, *, name="layer", strict=True, verbose=True):
    """gpu/ref: dicts of numpy arrays codes, scales, zeros, row_loss, g_idx."""
    codes_eq = np.mean(gpu["codes"] == ref["codes"]) if ref["codes"].size else 1.0
    rows_diff = np.mean(np.any(gpu["codes"] != ref["codes"], axis=1)) if ref["codes"].size else 0.0
    s_ok = np.abs(gpu["scales"] - ref["scales"]) <= SCALE_RTOL * np.abs(ref["scales"])
    z_ok = gpu["zeros"] == ref["zeros"]
    scale_eq = float(np.mean(s_ok)) if s_ok.size else 1.0
    zero_eq = float(np.mean(z_ok)) if z_ok.size else 1.0
    lg, lr = float(np.sum(gpu["row_loss"])), float(np.sum(ref["row_loss"]))
    loss_rel = abs(lg - lr) / max(abs(lr), 1e-300)
    report = dict(name=name, codes_agree=float(codes_eq), rows_with_diff=float(rows_diff),
                  scales_agree=scale_eq, zeros_agree=zero_eq, loss_gpu=lg, loss_ref=lr,
                  loss_rel=loss_rel)
    if verbose:
        print(f"[parity] {name}: codes {codes_eq:.6f} rows_diff {rows_diff:.4f} "
              f"scales {scale_eq:.6f} zeros {zero_eq:.6f} loss_rel {loss_rel:.2e}", flush=True)
        sys.stdout.flush()
    if strict:
        assert codes_eq >= CODE_AGREE, report
        assert scale_eq >= SCALE_AGREE and zero_eq >= SCALE_AGREE, report
        assert loss_rel <= LOSS_RTOL, report
        if "g_idx" in ref and "g_idx" in gpu:
            assert np.array_equal(gpu["g_idx"], ref["g_idx"]), "g_idx differs"
    return report


def to_numpy_layer(q):
    """QuantizedLayer (torch, device) -> dict of numpy arrays in oracle units."""
    return dict(codes=q.codes.cpu().numpy().astype(np.int64),
                scales=q.scales.cpu().numpy().astype(np.float64),
                zeros=q.zeros.cpu().numpy().astype(np.float64),
                g_idx=q.g_idx.cpu().numpy().astype(np.int64),
                row_loss=q.row_loss.cpu().numpy())
