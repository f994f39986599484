"""GPU: the digit-sliced int8 Hessian (GPTQ_FLAG_HESSIAN_SPLIT8).

Two independent checks per case, both through the C ABI:

* tight: against what the flag defines, X~^T X~ for the fixed-point X~ (each
  column rounded to the nearest multiple of 2^(e_f - 30), 2^e_f the smallest
  power of two above the column's largest magnitude) without its digit
  orders 5 and 6, summed here in exact integer arithmetic; only fp64
  additions separate the two;
* against the oracle's exact S = X^T X, within the bound that the rounding
  of X implies (|x~ - x| <= 2^(e_f - 31) per value, so
  |X~^T X~ - X^T X|_fg <= 2^-31 (s_f sum|x_g| + s_g sum|x_f|) + n 2^-62 s_f s_g)
  plus the bound of the orders left out.
"""
import sys

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402
from post_weight_quantization_hessian_amd import synth  # noqa: E402
from tests.parity_util import compare_layer, to_numpy_layer  # noqa: E402
from tests.split8_ref import split8_bound, split8_gram  # noqa: E402

DEV = torch.device("cuda:0")
U53 = 2.0 ** -53


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def skewed_inputs(n, dim, seed):
    """Columns on very different scales (log-normal, sigma 2), a shared
    component, one all-zero column and one lone large value."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, dim)) + 0.7 * rng.standard_normal((n, 1))
    X *= np.exp(2.0 * rng.standard_normal(dim))[None, :]
    if dim > 2:
        X[:, 1] = 0.0
        X[rng.integers(n), dim - 1] *= 1000.0
    return X.astype(np.float32)


def run_split8(S, X, overwrite, ws=None):
    Xd = torch.from_numpy(X).to(DEV)
    G.hessian_accumulate(S, Xd, workspace=ws, overwrite=overwrite, split8=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n,dim", [(15, 7), (300, 130), (2048, 576), (1000, 257), (37, 1),
                                   (4100, 384), (20000, 200)])
def test_split8_matches_fixed_point_and_oracle(n, dim):
    say(f"split8 n={n} dim={dim}")
    X = skewed_inputs(n, dim, 11 * n + dim)
    S = torch.full((dim, dim), 7.0, dtype=torch.float64, device=DEV)  # overwritten
    run_split8(S, X, overwrite=True)
    Sg = S.cpu().numpy()
    assert np.array_equal(Sg, Sg.T), "S is not exactly symmetric"
    St, mag = split8_gram(X)
    err = np.abs(Sg - St)
    assert np.all(err <= 32 * U53 * mag), float(np.max(err / np.maximum(mag, 1e-300)))
    Sx, _ = O.hessian_sum(X)
    assert np.all(np.abs(Sg - Sx) <= split8_bound(X) + 32 * U53 * mag)


def test_split8_strided_rows():
    """X as a column slice of a wider array (row stride > in_features)."""
    say("split8 strided X")
    n, dim, ld = 777, 300, 333
    big = skewed_inputs(n, ld, 9)
    X = big[:, :dim]
    Xd = torch.from_numpy(big).to(DEV)[:, :dim]
    assert Xd.stride(0) == ld
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, Xd, overwrite=True, split8=True)
    torch.cuda.synchronize()
    St, mag = split8_gram(np.ascontiguousarray(X))
    assert np.all(np.abs(S.cpu().numpy() - St) <= 32 * U53 * mag)


def test_split8_accumulates_calls_with_their_own_scales():
    say("split8 accumulate over three calls")
    dim = 300
    chunks = [skewed_inputs(n, dim, 70 + n) * f for n, f in ((700, 1.0), (64, 1e-3), (1500, 50.0))]
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    St = np.zeros((dim, dim))
    mag = np.zeros((dim, dim))
    for c in chunks:
        run_split8(S, c, overwrite=False)
        t, m = split8_gram(c)
        St += t
        mag += m
    Sg = S.cpu().numpy()
    assert np.all(np.abs(Sg - St) <= 48 * U53 * mag)
    Sx, _ = O.hessian_sum(chunks)
    bound = sum(split8_bound(c) for c in chunks) + 48 * U53 * mag
    assert np.all(np.abs(Sg - Sx) <= bound)


def test_split8_non_finite_column_gives_nan_row_and_column():
    say("split8 non-finite column")
    n, dim = 500, 260
    X = skewed_inputs(n, dim, 5)
    X[17, 200] = np.inf
    X[3, 40] = np.nan
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    run_split8(S, X, overwrite=True)
    Sg = S.cpu().numpy()
    bad = np.zeros(dim, dtype=bool)
    bad[[40, 200]] = True
    assert np.all(np.isnan(Sg[bad, :])) and np.all(np.isnan(Sg[:, bad]))
    good = ~bad
    Xg = X[:, good]
    St, mag = split8_gram(Xg)
    sub = Sg[np.ix_(good, good)]
    assert np.all(np.abs(sub - St) <= 32 * U53 * mag)


def test_split8_workspace_is_required():
    say("split8 workspace checks")
    X = torch.ones((256, 64), dtype=torch.float32, device=DEV)
    S = torch.zeros((64, 64), dtype=torch.float64, device=DEV)
    need = G.hessian_split8_workspace_bytes(64, 256)
    assert need >= 4 * 64 * 256
    small = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError):
        G.hessian_accumulate(S, X, workspace=small, split8=True)
    ok = torch.empty(need, dtype=torch.uint8, device=DEV)
    G.hessian_accumulate(S, X, workspace=ok, overwrite=True, split8=True)
    torch.cuda.synchronize()
    assert torch.all(S == 256.0)


def test_split8_layer_parity_with_oracle():
    """End to end: the split8 Hessian feeding prepare and quantize, against
    the oracle's layer from the exact Hessian (SiLU-gated activations)."""
    say("split8 end-to-end 384x1536, 2048 tokens")
    rows, dim, n = 384, 1536, 2048
    X = synth.activations(61, "split8_down", n, dim, kind="silu_gated")
    W = synth.weights(61, "split8_w", rows, dim)
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    run_split8(S, X, overwrite=True)
    perm, U = G.prepare_hinv(S, n, damp=0.01, act_order=True)
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), U, perm, bits=4, group_size=128)
    torch.cuda.synchronize()
    Sr, nr = O.hessian_sum(X)
    ref = O.gptq_layer(W, Sr, nr, bits=4, group_size=128, act_order=True)
    compare_layer(to_numpy_layer(q), ref, name="split8 384x1536")
