"""CPU checks of the parity comparison itself (tests/parity_util.py): grids
must agree in every group up to each row's first differing code, and only
later groups of a flipped row may differ."""
import numpy as np

from tests.parity_util import compare_layer, first_flip_group


def _case():
    rng = np.random.default_rng(0)
    rows, cols, gs = 4, 12, 3
    perm = rng.permutation(cols)
    g_idx = np.empty(cols, dtype=np.int64)
    g_idx[perm] = np.arange(cols) // gs
    ref = dict(codes=rng.integers(0, 16, (rows, cols)), scales=rng.uniform(0.1, 1, (rows, 4)),
               zeros=rng.integers(0, 16, (rows, 4)).astype(float), row_loss=np.ones(rows),
               g_idx=g_idx)
    return ref, perm


def test_first_flip_group_is_in_sweep_order():
    ref, perm = _case()
    codes = ref["codes"].copy()
    codes[1, perm[7]] += 1   # sweep position 7: group 2
    codes[1, perm[10]] += 1  # a later one in the same row
    codes[3, perm[0]] += 1   # group 0
    assert first_flip_group(codes, ref["codes"], ref["g_idx"]).tolist() == [4, 2, 4, 0]


def _ok(gpu, ref):
    return compare_layer(gpu, ref, strict=False, verbose=False)["grids_agree_before_first_flip"]


def test_grids_after_a_rows_first_tie_may_differ_only_there():
    ref, perm = _case()
    ref["scales"] = ref["scales"].astype(np.float16).astype(np.float64)
    gpu = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    gpu["codes"][1, perm[7]] += 1
    gpu["scales"][1, 3] *= 1.5   # after row 1's flip group: tolerated
    assert _ok(gpu, ref)
    gpu["scales"][1, 2] *= 1.5   # the flip's own group: its grid predates the flip
    assert not _ok(gpu, ref)
    gpu["scales"][1, 2] = ref["scales"][1, 2]
    gpu["zeros"][0, 3] += 2      # row 0 has no flip: a grid that differs by more
    assert not _ok(gpu, ref)     # than a rounding step is a failure
    gpu["zeros"][0, 3] -= 1      # a zero point one apart ...
    up = np.nextafter(np.float16(ref["scales"][0, 3]), np.float16(np.inf))
    gpu["scales"][0, 3] = float(up)  # ... with the scale one fp16 unit apart: a tie
    gpu["scales"][0, 3:] = gpu["scales"][0, 3:]
    assert _ok(gpu, ref)
    gpu["scales"][0, 1] = float(np.nextafter(np.float16(ref["scales"][0, 1]),
                                             np.float16(np.inf)))
    gpu["zeros"][0, 1] += 3      # an earlier group of that row off by more: failure
    assert not _ok(gpu, ref)
