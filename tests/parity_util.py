"""Comparison of the HIP path's outputs with the oracle's (test helper).

Tolerances are the ones the quantizer is held to: >= 99.9 % identical
integer codes (mismatches only at rounding ties), group scales/zero points
within 1e-5 relative, layer loss within 1e-3 relative.

Two kinds of ties start a legitimate divergence of a row: a code whose
value sits at a rounding tie, and a group scale whose unrounded value sits at
an fp16 rounding boundary (the two sides then store neighbouring fp16 values,
one unit in the last place apart, and the zero point moves by at most one).
Either changes the error fed to every later column of the row, so the row's
later groups are taken from other (equally valid) values and their grids may
differ. Scales and zero points are therefore held to the tolerance in every
group of a row before its first divergence (in sweep order: the smallest
group among the differing codes, or the first group whose grid differs),
which is all groups of a row without one; a divergence that starts at a
grid must be such a one-unit step; later groups of the row are counted in
the reported fraction only. The number of such rows is bounded by the code
agreement.
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


def first_flip_group(gpu_codes, ref_codes, g_idx):
    """Per row: the group (sweep order) of the first differing code, or the
    number of groups when the row agrees everywhere."""
    d = gpu_codes != ref_codes
    big = int(np.max(g_idx)) + 1 if len(g_idx) else 0
    return np.where(d, np.asarray(g_idx)[None, :], big).min(axis=1) if d.size else \
        np.full(d.shape[0], big)


def compare_layer(gpu, ref, *, name="layer", strict=True, verbose=True):
    """gpu/ref: dicts of numpy arrays codes, scales, zeros, row_loss and
    (in ref) g_idx, the group in sweep order of every original column."""
    codes_eq = np.mean(gpu["codes"] == ref["codes"]) if ref["codes"].size else 1.0
    rows_diff = np.mean(np.any(gpu["codes"] != ref["codes"], axis=1)) if ref["codes"].size else 0.0
    s_ok = np.abs(gpu["scales"] - ref["scales"]) <= SCALE_RTOL * np.abs(ref["scales"])
    z_ok = gpu["zeros"] == ref["zeros"]
    scale_eq = float(np.mean(s_ok)) if s_ok.size else 1.0
    zero_eq = float(np.mean(z_ok)) if z_ok.size else 1.0
    # groups up to each row's first flip must all agree
    g_idx = ref.get("g_idx")
    if g_idx is None:  # identity order: groups of equal width from the scales' shape
        ng = ref["scales"].shape[1] if ref["scales"].ndim == 2 else 0
        cols = ref["codes"].shape[1]
        width = gpu.get("group_size") or ref.get("group_size")
        if width is None:
            raise ValueError("compare_layer needs g_idx or group_size")
        g_idx = np.arange(cols) // int(width)
        assert ng == -(-cols // int(width))
    flip = first_flip_group(gpu["codes"], ref["codes"], g_idx)
    grids_before_flip = True
    if s_ok.size:
        ng = s_ok.shape[1]
        g_ok = s_ok & z_ok
        # first group whose grid differs (ng: none); every group before it
        # agrees by definition
        first_bad = np.where(g_ok.all(axis=1), ng, np.argmin(g_ok, axis=1))
        # a grid is taken before any code of its group, so a row whose first
        # differing grid is at or before its first differing code diverges
        # at that grid: it must be a one-unit fp16 step of the scale (and of
        # at most one in the zero point)
        rows_g = np.nonzero((first_bad < ng) & (first_bad <= flip))[0]
        if len(rows_g):
            fb = first_bad[rows_g]
            gs_ = gpu["scales"][rows_g, fb].astype(np.float16).view(np.int16).astype(np.int64)
            rs_ = ref["scales"][rows_g, fb].astype(np.float16).view(np.int16).astype(np.int64)
            dz = np.abs(gpu["zeros"][rows_g, fb] - ref["zeros"][rows_g, fb])
            grids_before_flip = bool(np.all(np.abs(gs_ - rs_) <= 1) and np.all(dz <= 1))
            if verbose:
                for k in range(min(len(rows_g), 4)):
                    print(f"[parity] {name}: row {int(rows_g[k])} diverges at the grid of group "
                          f"{int(fb[k])} (first differing code in group {int(flip[rows_g[k]])}): "
                          f"scale {float(gpu['scales'][rows_g[k], fb[k]])!r} vs "
                          f"{float(ref['scales'][rows_g[k], fb[k]])!r} "
                          f"({int(gs_[k] - rs_[k])} fp16 units), zero "
                          f"{float(gpu['zeros'][rows_g[k], fb[k]])} vs "
                          f"{float(ref['zeros'][rows_g[k], fb[k]])}", flush=True)
    lg, lr = float(np.sum(gpu["row_loss"])), float(np.sum(ref["row_loss"]))
    loss_rel = abs(lg - lr) / max(abs(lr), 1e-300)
    report = dict(name=name, codes_agree=float(codes_eq), rows_with_diff=float(rows_diff),
                  scales_agree=scale_eq, zeros_agree=zero_eq,
                  grids_agree_before_first_flip=grids_before_flip, loss_gpu=lg, loss_ref=lr,
                  loss_rel=loss_rel)
    if verbose:
        print(f"[parity] {name}: codes {codes_eq:.6f} rows_diff {rows_diff:.4f} "
              f"scales {scale_eq:.6f} zeros {zero_eq:.6f} (before each row's first tie: "
              f"{'all agree' if grids_before_flip else 'DIFFER'}) loss_rel {loss_rel:.2e}",
              flush=True)
        sys.stdout.flush()
    if strict:
        assert codes_eq >= CODE_AGREE, report
        assert grids_before_flip, report
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
