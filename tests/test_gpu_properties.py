"""GPU: parity with the oracle over random problems (hypothesis, derandomized):
ragged shapes, every group size and bit width, act-order on and off, the
exact and the int8 digit-slice Hessian, anisotropic activations (including
fewer tokens than features, SPD through the damping). Each case runs the
whole path through the C ABI and meets the parity bar against the oracle's
layer from the same seeded inputs."""
import sys

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402
from tests.parity_util import compare_layer, to_numpy_layer  # noqa: E402

DEV = torch.device("cuda:0")


@st.composite
def cases(draw):
    cols = draw(st.integers(1, 700))
    rows = draw(st.integers(1, 300))
    n = draw(st.integers(1, 2 * cols + 64))
    gs = draw(st.sampled_from([16, 32, 64, 128]))
    bits = draw(st.sampled_from([2, 3, 4, 8]))
    act = draw(st.booleans())
    split8 = draw(st.booleans())
    aniso = draw(st.floats(0.0, 1.5))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return rows, cols, n, gs, bits, act, split8, aniso, seed


@pytest.mark.timeout(900)
@settings(max_examples=25, deadline=None, derandomize=True)
@given(cases())
def test_random_layers_match_oracle(case):
    rows, cols, n, gs, bits, act, split8, aniso, seed = case
    print(f"[case] {case}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, cols)) * np.exp(aniso * rng.standard_normal(cols))[None, :]
         + 0.7 * rng.standard_normal((n, 1))).astype(np.float32)
    W = (0.02 * rng.standard_t(4, size=(rows, cols))).astype(np.float16)
    S = torch.empty((cols, cols), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True, split8=split8)
    perm, U = G.prepare_hinv(S, n, damp=0.01, act_order=act)
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), U, perm if act else None, bits=bits,
                         group_size=gs)
    torch.cuda.synchronize()
    Sr, nr = O.hessian_sum(X)
    H = O.damped_hessian(Sr, nr, 0.01)
    pg = perm.cpu().numpy().astype(np.int64) if act else np.arange(cols)
    if act:
        # the split8 Hessian rounds X per column: the order may differ only
        # between near-equal diagonals, and the reference then sweeps in the
        # library's (equally valid) order
        pr = O.act_order_perm(H)
        hd = np.diag(H)
        assert np.array_equal(np.sort(pg), np.arange(cols))
        for k in np.nonzero(pg != pr)[0]:
            assert abs(hd[pg[k]] - hd[pr[k]]) <= 1e-7 * hd[pr[k]], k
    res = O.gptq_sweep(W.astype(np.float64)[:, pg], O.hinv_upper(O.permute_sym(H, pg)), bits, gs)
    codes = np.empty_like(res["codes"])
    codes[:, pg] = res["codes"]
    g_idx = np.empty(cols, dtype=np.int64)
    g_idx[pg] = np.arange(cols) // gs
    ref = dict(codes=codes, scales=res["scales"], zeros=res["zeros"], row_loss=res["row_loss"],
               g_idx=g_idx)
    compare_layer(to_numpy_layer(q), ref, name=f"random {case}")
