"""GPU parity: the HIP path against the fp64 oracle on identical seeded inputs.

Every call goes through the C ABI (via the thin binding). Sizes span several
128-wide tiles and ragged tails; the workload tests use the full layer shapes
of the small and medium workloads.
"""
import sys

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_hessian_amd import synth
from post_weight_quantization_hessian_amd.pipeline import hessian_mode
from post_weight_quantization_hessian_amd.workloads import WORKLOADS
from tests.parity_util import compare_layer, to_numpy_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_hessian(Xs, dim, use_ws=True, split8=False):
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    n = 0
    for X in Xs:
        Xd = torch.from_numpy(X).to(DEV)
        ws = None if use_ws else torch.empty(1, dtype=torch.uint8, device=DEV)
        G.hessian_accumulate(S, Xd, workspace=ws, split8=split8)
        n += X.shape[0]
    return S, n


def gpu_layer(W, Xs, *, bits, gs, damp=0.01, act_order=False):
    dim = W.shape[1]
    S, n = gpu_hessian(Xs, dim)
    perm, U = G.prepare_hinv(S, n, damp=damp, act_order=act_order)
    Wd = torch.from_numpy(W).to(DEV)
    q = G.quantize_layer(Wd, U, perm if act_order else None, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    return S, perm, U, q


def rand_inputs(rows, cols, n, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, cols)) + 0.8 * rng.standard_normal((n, 1))).astype(np.float32)
    W = (0.02 * rng.standard_t(4, size=(rows, cols))).astype(np.float16)
    return W, X


# ---------------------------------------------------------------- step 1

@pytest.mark.parametrize("n,dim", [(15, 7), (300, 130), (2048, 576), (1000, 257), (37, 1),
                                   (4100, 384)])
@pytest.mark.parametrize("use_ws", [True, False])
def test_hessian_matches_oracle(n, dim, use_ws):
    say(f"hessian n={n} dim={dim} ws={use_ws}")
    rng = np.random.default_rng(n * 1000 + dim)
    X = rng.standard_normal((n, dim)).astype(np.float32)
    chunks = [X[: n // 3], X[n // 3:]]
    S, nt = gpu_hessian(chunks, dim, use_ws)
    Sr, nr = O.hessian_sum(chunks)
    Sg = S.cpu().numpy()
    assert nt == nr
    scale = np.sqrt(np.outer(np.diag(Sr), np.diag(Sr))) + 1e-300
    err = np.max(np.abs(Sg - Sr) / scale)
    assert err < 1e-13, err
    assert np.array_equal(Sg, Sg.T)


def test_hessian_overwrite_ignores_old_contents():
    say("hessian overwrite")
    rng = np.random.default_rng(8)
    for n, dim in [(700, 300), (64, 129)]:  # split and unsplit plans
        X = rng.standard_normal((n, dim)).astype(np.float32)
        S = torch.full((dim, dim), float("nan"), dtype=torch.float64, device=DEV)
        G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
        Sr, _ = O.hessian_sum(X)
        np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-12, atol=1e-9)
    S = torch.full((50, 50), 3.0, dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.zeros((0, 50), dtype=torch.float32, device=DEV), overwrite=True)
    assert torch.all(S == 0)


def test_hessian_unaligned_rows_and_exact_entries():
    say("hessian strided X")
    rng = np.random.default_rng(5)
    big = rng.standard_normal((513, 203)).astype(np.float32)
    Xt = torch.from_numpy(big).to(DEV)[:, 1:202]  # ldx = 203, offset 1 float
    S = torch.zeros((201, 201), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, Xt)
    Sg = S.cpu().numpy()
    X = big[:, 1:202]
    for f, g in [(0, 0), (3, 200), (100, 57), (200, 200)]:
        exact = O.hessian_entry(X, f, g)
        assert abs(Sg[f, g] - exact) <= 1e-13 * np.sqrt(Sg[f, f] * Sg[g, g])


# ---------------------------------------------------------------- steps 2-3

@pytest.mark.parametrize("dim,act", [(7, False), (130, True), (576, False), (576, True),
                                     (300, True), (896, True)])
def test_prepare_matches_oracle(dim, act):
    say(f"prepare dim={dim} act={act}")
    rng = np.random.default_rng(dim)
    X = (rng.standard_normal((2 * dim + 50, dim)) * rng.lognormal(0, 1, dim)).astype(np.float32)
    Sr, n = O.hessian_sum(X)
    S = torch.from_numpy(Sr).to(DEV)
    perm, U = G.prepare_hinv(S, n, damp=0.01, act_order=act)
    H = O.damped_hessian(Sr, n, 0.01)
    pr = O.act_order_perm(H) if act else np.arange(dim)
    assert np.array_equal(perm.cpu().numpy(), pr)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    Ug = U.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(Ug, -1) == 0)
    err = np.max(np.abs(Ug - Ur)) / np.max(np.abs(Ur))
    assert err < 2e-6, err


def test_prepare_rejects_non_spd():
    say("prepare non-SPD")
    S = torch.zeros((200, 200), dtype=torch.float64, device=DEV)
    with pytest.raises(G.GPTQError) as ei:
        G.prepare_hinv(S, 10, damp=0.0)
    assert ei.value.status == G.GPTQ_ENOTSPD
    S[5, 5] = float("nan")
    with pytest.raises(G.GPTQError) as ei:
        G.prepare_hinv(S, 10, damp=0.1)
    assert ei.value.status == G.GPTQ_ENOTSPD


# ---------------------------------------------------------------- steps 4-6

CASES = [  # rows, cols, n, bits, gs, act
    (5, 200, 400, 3, 32, False),
    (37, 333, 700, 2, 16, True),
    (64, 576, 2048, 4, 128, False),
    (130, 260, 600, 8, 64, True),
    (1, 129, 300, 4, 128, True),
    (200, 640, 1500, 4, 64, True),
    (16, 131, 300, 3, 32, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}_b{c[3]}_g{c[4]}_a{int(c[5])}"
                                             for c in CASES])
def test_end_to_end_small(case):
    rows, cols, n, bits, gs, act = case
    say(f"e2e {case}")
    W, X = rand_inputs(rows, cols, n, rows * 7 + cols)
    S, perm, U, q = gpu_layer(W, [X], bits=bits, gs=gs, act_order=act)
    Sr, nr = O.hessian_sum(X)
    ref = O.gptq_layer(W, Sr, nr, bits=bits, group_size=gs, damp=0.01, act_order=act)
    compare_layer(to_numpy_layer(q), ref, name=f"e2e{case}")


def test_quantize_with_oracle_factor():
    """Sweep alone: the oracle's factor (rounded to fp32) as input."""
    say("quantize with oracle U")
    W, X = rand_inputs(96, 448, 1000, 11)
    Sr, n = O.hessian_sum(X)
    ref = O.gptq_layer(W, Sr, n, bits=4, group_size=64, act_order=True)
    U = torch.from_numpy(ref["U"].astype(np.float32)).to(DEV)
    perm = torch.from_numpy(ref["perm"].astype(np.int32)).to(DEV)
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), U, perm, bits=4, group_size=64)
    compare_layer(to_numpy_layer(q), ref, name="oracle-U")


def test_determinism():
    say("determinism")
    W, X = rand_inputs(70, 300, 500, 3)
    outs = [gpu_layer(W, [X], bits=4, gs=32, act_order=True) for _ in range(2)]
    (S1, p1, U1, q1), (S2, p2, U2, q2) = outs
    assert torch.equal(S1, S2) and torch.equal(U1, U2) and torch.equal(p1, p2)
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.row_loss, q2.row_loss)


def test_empty_and_error_paths():
    say("empty/error paths")
    U = torch.eye(64, dtype=torch.float32, device=DEV)
    W0 = torch.zeros((0, 64), dtype=torch.float16, device=DEV)
    q = G.quantize_layer(W0, U, None, bits=4, group_size=64)
    assert q.codes.shape == (0, 64)
    W = torch.full((3, 64), 0.01, dtype=torch.float16, device=DEV)
    W[1, 7] = float("nan")
    with pytest.raises(G.GPTQError) as ei:
        G.quantize_layer(W, U, None, bits=4, group_size=64)
    assert ei.value.status == G.GPTQ_ENONFINITE
    W = torch.full((3, 64), 0.01, dtype=torch.float16, device=DEV)
    bad = torch.arange(64, dtype=torch.int32, device=DEV)
    bad[3] = 70
    with pytest.raises(G.GPTQError) as ei:
        G.quantize_layer(W, U, bad, bits=4, group_size=64)
    assert ei.value.status == G.GPTQ_EINVAL
    dup = torch.arange(64, dtype=torch.int32, device=DEV)
    dup[3] = 4
    with pytest.raises(G.GPTQError) as ei:
        G.quantize_layer(W, U, dup, bits=4, group_size=64)
    assert ei.value.status == G.GPTQ_EINVAL
    # all-zero rows: degenerate groups, scale 1, zero 0, codes 0, loss 0
    Wz = torch.zeros((4, 64), dtype=torch.float16, device=DEV)
    q = G.quantize_layer(Wz, U, None, bits=4, group_size=16)
    assert torch.all(q.codes == 0) and torch.all(q.scales == 1) and torch.all(q.zeros == 0)
    assert torch.all(q.row_loss == 0)


def test_identity_hessian_is_rtn():
    """Diagonal H: the GPU sweep must reproduce round-to-nearest exactly."""
    say("identity H = RTN")
    rng = np.random.default_rng(9)
    W = (0.02 * rng.standard_t(4, size=(50, 384))).astype(np.float16)
    U = torch.eye(384, dtype=torch.float32, device=DEV) * 0.5
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), U, None, bits=3, group_size=32)
    codes, scales, zeros = O.rtn_quantize(W.astype(np.float64), 3, 32)
    assert np.array_equal(q.codes.cpu().numpy(), codes)
    assert np.array_equal(q.scales.cpu().numpy().astype(np.float64), scales)
    assert np.array_equal(q.zeros.cpu().numpy().astype(np.float64), zeros)


# ---------------------------------------------------------------- workloads

def workload_inputs(wl, hname):
    h = wl.input(hname)
    X = synth.activations(wl.wid, hname, wl.n_tokens, h.dim, kind=h.kind,
                          lognormal_sigma=h.lognormal_sigma)
    Ws = [synth.weights(wl.wid, l.name, l.rows, h.dim, outlier_frac=l.outlier_frac)
          for l in wl.layers_of(hname)]
    return X, np.concatenate(Ws, axis=0)


def run_workload_input(wl, hname, block):
    """The Hessian mode is the benchmark's ("auto": the int8 digit-slice
    products from 256 features on); the oracle's S is exact either way."""
    X, W = workload_inputs(wl, hname)
    chunks = [X[s:s + wl.token_chunk] for s in range(0, X.shape[0], wl.token_chunk)]
    split8 = hessian_mode("auto", X.shape[1])
    S, n = gpu_hessian(chunks, X.shape[1], split8=split8)
    perm, U = G.prepare_hinv(S, n, damp=wl.damp, act_order=wl.act_order)
    Sr, nr = O.hessian_sum(chunks)
    H = O.damped_hessian(Sr, nr, wl.damp)
    pr = O.act_order_perm(H) if wl.act_order else np.arange(H.shape[0])
    pg = perm.cpu().numpy().astype(np.int64)
    if split8:
        # diag S rounds X per column (relative error far below 1e-7): the
        # order may differ only between near-equal diagonals, and the
        # reference then sweeps in the library's (equally valid) order
        hd = np.diag(H)
        assert np.array_equal(np.sort(pg), np.arange(len(pg)))
        for k in np.nonzero(pg != pr)[0]:
            assert abs(hd[pg[k]] - hd[pr[k]]) <= 1e-7 * hd[pr[k]], k
        pr = pg
    assert np.array_equal(pg, pr)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    Wd = torch.from_numpy(W).to(DEV)
    for bits in wl.bits:
        say(f"{wl.name}/{hname} rows={W.shape[0]} cols={W.shape[1]} bits={bits}")
        q = G.quantize_layer(Wd, U, perm if wl.act_order else None, bits=bits,
                             group_size=wl.group_size)
        res = O.gptq_sweep(W.astype(np.float64)[:, pr], Ur, bits, wl.group_size, block=block)
        codes = np.empty_like(res["codes"])
        codes[:, pr] = res["codes"]
        g_idx = np.empty(len(pr), dtype=np.int64)
        g_idx[pr] = np.arange(len(pr)) // wl.group_size
        ref = dict(codes=codes, scales=res["scales"], zeros=res["zeros"],
                   row_loss=res["row_loss"], g_idx=g_idx)
        compare_layer(to_numpy_layer(q), ref, name=f"{wl.name}/{hname}/b{bits}")


def test_workload_smollm_q576_strict_oracle():
    wl = WORKLOADS["smollm_q576"]
    run_workload_input(wl, "x", block=None)


@pytest.mark.parametrize("hname", ["mlp_in", "down_in"])
def test_workload_qwen05b_mlp(hname):
    wl = WORKLOADS["qwen05b_mlp"]
    run_workload_input(wl, hname, block=128)


@pytest.mark.parametrize("hname", ["attn_in", "o_in", "mlp_in", "down_in"])
def test_workload_tinyllama_block(hname):
    wl = WORKLOADS["tinyllama_block"]
    run_workload_input(wl, hname, block=128)
