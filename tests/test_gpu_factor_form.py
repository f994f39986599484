"""GPU: the sweep in the factor form against the fp64 oracle.

prepare_hinv(..., factor_form=True) returns, in sweep order, U's 128-wide
diagonal blocks and, beyond them, R[blk_a, blk_b] U[blk_b, blk_b] with R =
U^-1 the factor of H_p itself (H_p = R R^T, so R needs no inverse: it is the
order-reversed Cholesky factor; only the diagonal blocks are inverted). The
sweep then carries the residuals q - w of the original weights through that
matrix, which gives the same update sums as the errors through U (The
Geometry of LLM Quantization 2.2: the nearest-plane step works with a
triangular factor of the lattice's Gram matrix; E = (W - Q) U^-1), so codes,
scales, zero points and the loss are held to the oracle's sweep (CHMC
article, Methodik, Schritt 2) at the usual bar. Shapes: ragged columns (not a multiple of 128), every group
size, 2 to 8 bits, act-order on and off, the no-clipping sweep, and the full
small and medium workload layers in the benchmark's configuration.
"""
import sys

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_hessian_amd.pipeline import LayerGroup, hessian_mode
from post_weight_quantization_hessian_amd.workloads import WORKLOADS
from tests.parity_util import compare_layer, to_numpy_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402
from tests.test_gpu_parity import gpu_hessian, rand_inputs, workload_inputs  # noqa: E402

DEV = torch.device("cuda:0")
B = 128


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def expected_matrix(Ur):
    """U's diagonal blocks, R[blk_a, blk_b] U[blk_b, blk_b] beyond them (R =
    U^-1, from the oracle's U)."""
    R = np.linalg.inv(Ur)
    n = Ur.shape[0]
    M = np.zeros_like(Ur)
    for b0 in range(0, n, B):
        b1 = min(b0 + B, n)
        M[b0:b1, b0:b1] = Ur[b0:b1, b0:b1]
        M[:b0, b0:b1] = R[:b0, b0:b1] @ Ur[b0:b1, b0:b1]
    return M


@pytest.mark.parametrize("dim,act", [(7, False), (130, True), (333, False), (576, True),
                                     (896, True), (1000, False)])
def test_factor_form_matrix_matches_oracle(dim, act):
    say(f"factor-form prepare dim={dim} act={act}")
    rng = np.random.default_rng(dim + 17)
    X = (rng.standard_normal((2 * dim + 50, dim)) * rng.lognormal(0, 1, dim)
         + 0.5 * rng.standard_normal((2 * dim + 50, 1))).astype(np.float32)
    Sr, n = O.hessian_sum(X)
    S = torch.from_numpy(Sr).to(DEV)
    perm, M = G.prepare_hinv(S, n, damp=0.01, act_order=act, factor_form=True)
    H = O.damped_hessian(Sr, n, 0.01)
    pr = O.act_order_perm(H) if act else np.arange(dim)
    assert np.array_equal(perm.cpu().numpy(), pr)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    Me = expected_matrix(Ur)
    Mg = M.cpu().numpy().astype(np.float64)
    assert np.all(np.tril(Mg, -1) == 0)
    # per 128-block of rows and columns: fp32 storage of fp64 values (the
    # off-diagonal blocks relative to the block column of R U's scale)
    for b0 in range(0, dim, B):
        col = np.max(np.abs(Me[:b0 + B, b0:b0 + B])) if b0 else 0.0
        for a0 in range(0, b0 + 1, B):
            e = Me[a0:a0 + B, b0:b0 + B]
            g = Mg[a0:a0 + B, b0:b0 + B]
            scale = np.max(np.abs(e)) if a0 == b0 else col
            err = np.max(np.abs(g - e)) / max(scale, 1e-300)
            assert err < 2e-6, (a0, b0, err)


CASES = [  # rows, cols, n, bits, gs, act, clip
    (5, 200, 400, 3, 32, False, True),
    (37, 333, 700, 2, 16, True, True),
    (64, 576, 2048, 4, 128, False, True),
    (130, 260, 600, 8, 64, True, True),
    (1, 129, 300, 4, 128, True, True),
    (200, 640, 1500, 4, 64, True, True),
    (16, 131, 300, 3, 32, False, True),
    (96, 448, 1000, 3, 64, True, False),
    (700, 384, 900, 4, 128, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}_b{c[3]}_g{c[4]}_a{int(c[5])}"
                                             f"_c{int(c[6])}" for c in CASES])
def test_factor_form_end_to_end(case):
    rows, cols, n, bits, gs, act, clip = case
    say(f"factor-form e2e {case}")
    W, X = rand_inputs(rows, cols, n, rows * 7 + cols + 1)
    S, nt = gpu_hessian([X], cols)
    perm, M = G.prepare_hinv(S, nt, damp=0.01, act_order=act, factor_form=True)
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), M, perm if act else None, bits=bits,
                         group_size=gs, clip=clip, factor_form=True)
    torch.cuda.synchronize()
    Sr, nr = O.hessian_sum(X)
    if clip:
        ref = O.gptq_layer(W, Sr, nr, bits=bits, group_size=gs, damp=0.01, act_order=act)
    else:
        H = O.damped_hessian(Sr, nr, 0.01)
        pr = O.act_order_perm(H) if act else np.arange(cols)
        res = O.gptq_sweep(W.astype(np.float64)[:, pr], O.hinv_upper(O.permute_sym(H, pr)),
                           bits, gs, clip=False)
        codes = np.empty_like(res["codes"])
        codes[:, pr] = np.clip(res["codes"], 0, 255)
        g_idx = np.empty(cols, dtype=np.int64)
        g_idx[pr] = np.arange(cols) // gs
        ref = dict(codes=codes, scales=res["scales"], zeros=res["zeros"],
                   row_loss=res["row_loss"], g_idx=g_idx)
    compare_layer(to_numpy_layer(q), ref, name=f"factor-form {case}")


def test_factor_form_identity_hessian_is_rtn():
    """Diagonal H (the factor form of 0.5 I is U = 0.5 I on the diagonal
    blocks and 0 beyond): round-to-nearest exactly."""
    say("factor-form identity H = RTN")
    rng = np.random.default_rng(19)
    W = (0.02 * rng.standard_t(4, size=(50, 384))).astype(np.float16)
    M = torch.eye(384, dtype=torch.float32, device=DEV) * 0.5
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), M, None, bits=3, group_size=32,
                         factor_form=True)
    codes, scales, zeros = O.rtn_quantize(W.astype(np.float64), 3, 32)
    assert np.array_equal(q.codes.cpu().numpy(), codes)
    assert np.array_equal(q.scales.cpu().numpy().astype(np.float64), scales)
    assert np.array_equal(q.zeros.cpu().numpy().astype(np.float64), zeros)


@pytest.mark.parametrize("wname,hname", [("qwen05b_mlp", "mlp_in"), ("qwen05b_mlp", "down_in"),
                                         ("tinyllama_block", "attn_in"),
                                         ("tinyllama_block", "down_in"),
                                         ("smollm_q576", "x")])
def test_factor_form_workload_layers(wname, hname):
    """The benchmark's launch configuration (LayerGroup.enqueue: the Hessian
    mode of the benchmark, every bit width on one stream), here with the
    factor form forced on (the benchmark takes it from 768 features),
    against the oracle's sweep on the exact S."""
    wl = WORKLOADS[wname]
    X, W = workload_inputs(wl, hname)
    dim = X.shape[1]
    chunks = [torch.from_numpy(X[s:s + wl.token_chunk]).to(DEV)
              for s in range(0, X.shape[0], wl.token_chunk)]
    grp = LayerGroup(dim, W.shape[0], max_chunk_tokens=max(c.shape[0] for c in chunks),
                     bits=wl.bits, group_size=wl.group_size, act_order=wl.act_order,
                     damp=wl.damp, device=DEV, hessian="auto", factor_form=True)
    assert grp.factor_form and grp.split8 == hessian_mode("auto", dim)
    grp.enqueue(chunks, torch.from_numpy(W).to(DEV))
    grp.check()
    Sr, nr = O.hessian_sum([X[s:s + wl.token_chunk] for s in range(0, X.shape[0],
                                                                    wl.token_chunk)])
    H = O.damped_hessian(Sr, nr, wl.damp)
    pg = grp.perm.cpu().numpy().astype(np.int64)
    pr = O.act_order_perm(H) if wl.act_order else np.arange(dim)
    if wl.act_order:
        hd = np.diag(H)
        assert np.array_equal(np.sort(pg), np.arange(dim))
        for k in np.nonzero(pg != pr)[0]:  # near-equal diagonals only
            assert abs(hd[pg[k]] - hd[pr[k]]) <= 1e-7 * hd[pr[k]], k
        pr = pg
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    for bi, bits in enumerate(wl.bits):
        say(f"factor-form {wname}/{hname} rows={W.shape[0]} cols={dim} bits={bits}")
        res = O.gptq_sweep(W.astype(np.float64)[:, pr], Ur, bits, wl.group_size,
                           block=None if dim <= 576 else 128)
        codes = np.empty_like(res["codes"])
        codes[:, pr] = res["codes"]
        g_idx = np.empty(dim, dtype=np.int64)
        g_idx[pr] = np.arange(dim) // wl.group_size
        ref = dict(codes=codes, scales=res["scales"], zeros=res["zeros"],
                   row_loss=res["row_loss"], g_idx=g_idx)
        q = grp.outs[bi]
        gpu = to_numpy_layer(q)
        if not wl.act_order:
            gpu["g_idx"] = g_idx
        compare_layer(gpu, ref, name=f"factor-form {wname}/{hname}/b{bits}")


@pytest.mark.parametrize("dim,rows,gs", [(300, 40, 64), (700, 24, 128)])
def test_factor_form_with_min_pivot_order(dim, rows, gs):
    """The min-pivot order (The Geometry of LLM Quantization 2.3) in the
    factor form: the same order as with U, and the layer at the parity bar
    against the oracle swept in that order."""
    say(f"factor-form min-pivot dim={dim}")
    W, X = rand_inputs(rows, dim, 2 * dim, dim + 5)
    S, n = gpu_hessian([X], dim)
    p_u, _ = G.prepare_hinv(S, n, damp=0.01, min_pivot=True)
    perm, M = G.prepare_hinv(S, n, damp=0.01, min_pivot=True, factor_form=True)
    assert torch.equal(perm, p_u)
    q = G.quantize_layer(torch.from_numpy(W).to(DEV), M, perm, bits=4, group_size=gs,
                         factor_form=True)
    torch.cuda.synchronize()
    Sr, nr = O.hessian_sum(X)
    H = O.damped_hessian(Sr, nr, 0.01)
    pr = perm.cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(pr), np.arange(dim))  # (the order itself: test_gpu_minpivot)
    res = O.gptq_sweep(W.astype(np.float64)[:, pr], O.hinv_upper(O.permute_sym(H, pr)), 4, gs)
    codes = np.empty_like(res["codes"])
    codes[:, pr] = res["codes"]
    g_idx = np.empty(dim, dtype=np.int64)
    g_idx[pr] = np.arange(dim) // gs
    ref = dict(codes=codes, scales=res["scales"], zeros=res["zeros"], row_loss=res["row_loss"],
               g_idx=g_idx)
    compare_layer(to_numpy_layer(q), ref, name=f"factor-form min-pivot {dim}")


def test_workload_inputs_on_concurrent_streams_like_the_benchmark():
    """The benchmark's step for the Qwen MLP workload: both calibration inputs
    (896 and 4864 features, the stacked gate/up rows and the down rows) as
    LayerGroups enqueued asynchronously on two streams at once, largest
    Hessian first; each against the oracle (and the same results as one
    input at a time)."""
    wl = WORKLOADS["qwen05b_mlp"]
    order = sorted(wl.inputs, key=lambda h: -h.dim)
    groups, inputs = [], []
    for h in order:
        X, W = workload_inputs(wl, h.name)
        chunks = [torch.from_numpy(X[s:s + wl.token_chunk]).to(DEV)
                  for s in range(0, X.shape[0], wl.token_chunk)]
        grp = LayerGroup(h.dim, W.shape[0], max_chunk_tokens=max(c.shape[0] for c in chunks),
                         bits=wl.bits, group_size=wl.group_size, act_order=wl.act_order,
                         damp=wl.damp, device=DEV, hessian="auto")
        groups.append(grp)
        inputs.append((X, W, chunks, torch.from_numpy(W).to(DEV)))
    streams = [torch.cuda.Stream(device=DEV) for _ in order]
    torch.cuda.synchronize()
    for grp, (_, _, chunks, Wd), s in zip(groups, inputs, streams):
        with torch.cuda.stream(s):
            grp.enqueue(chunks, Wd)
    torch.cuda.synchronize()
    for grp, s in zip(groups, streams):
        with torch.cuda.stream(s):
            grp.check()
    conc = [[(q.codes.clone(), q.row_loss.clone()) for q in g.outs] for g in groups]
    for grp, (_, _, chunks, Wd) in zip(groups, inputs):  # one at a time
        grp.enqueue(chunks, Wd)
        grp.check()
    for grp, c in zip(groups, conc):
        for (codes, loss), q in zip(c, grp.outs):
            assert torch.equal(codes, q.codes) and torch.equal(loss, q.row_loss)
    for h, grp, (X, W, _, _) in zip(order, groups, inputs):
        dim = h.dim
        Sr, nr = O.hessian_sum([X[s:s + wl.token_chunk] for s in range(0, X.shape[0],
                                                                        wl.token_chunk)])
        H = O.damped_hessian(Sr, nr, wl.damp)
        pr = np.arange(dim)
        Ur = O.hinv_upper(O.permute_sym(H, pr))
        for bi, bits in enumerate(wl.bits):
            say(f"concurrent {wl.name}/{h.name} bits={bits} factor_form={grp.factor_form}")
            res = O.gptq_sweep(W.astype(np.float64), Ur, bits, wl.group_size, block=128)
            ref = dict(codes=res["codes"], scales=res["scales"], zeros=res["zeros"],
                       row_loss=res["row_loss"], g_idx=np.arange(dim) // wl.group_size)
            gpu = to_numpy_layer(grp.outs[bi])
            gpu["g_idx"] = ref["g_idx"]
            compare_layer(gpu, ref, name=f"concurrent {wl.name}/{h.name}/b{bits}")
