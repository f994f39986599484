"""GPU: the CHMC frontend (CHMC article, Methodik, Schritt 1-3) against the
oracle's chmc_layer.

Through the C ABI: the GPU Hessian and factor, then gptq_chmc_layer with a
seeded Gaussian sketch. The fp16 factors A and B must equal the oracle's up to
the sign of each component (an fp16 rounding tie may land one ulp apart);
codes, per-row-group scales and zero points and the loss of the residual
sweep meet the sweep's parity bar. Shapes: the page's worked size (576 x 576
at 4.2875 bits per weight, rank 2), ragged rows, columns and groups, no
low-rank part, the largest rank, and the Qwen2.5-0.5B down projection at
full size; error paths: a weight of too low rank and a bad permutation.
"""
import sys

import numpy as np
import pytest

import oracle as O
from tests.parity_util import CODE_AGREE, LOSS_RTOL, SCALE_AGREE, SCALE_RTOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402
from post_weight_quantization_hessian_amd import synth  # noqa: E402

DEV = torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def problem(rows, cols, n, seed, lowrank=0):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, cols)) * np.exp(0.5 * rng.standard_normal(cols))[None, :]
         + 0.8 * rng.standard_normal((n, 1))).astype(np.float32)
    W = 0.02 * rng.standard_t(4, size=(rows, cols))
    if lowrank:
        W += 0.05 * rng.standard_normal((rows, lowrank)) @ rng.standard_normal((lowrank, cols))
    return W.astype(np.float16), X


def gpu_inputs(X, act_order):
    dim = X.shape[1]
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
    perm, U = G.prepare_hinv(S, X.shape[0], damp=O.CHMC_DAMP, act_order=act_order)
    return S, (perm if act_order else None), U


def compare_factor(gpu, ref, name):
    g = gpu.cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return
    exact = float(np.mean(g == ref))
    ulp = np.abs(np.spacing(ref.astype(np.float16)).astype(np.float64))
    near = bool(np.all(np.abs(g - ref) <= ulp))
    say(f"{name}: exact {exact:.6f}, within one ulp {near}")
    assert exact >= 0.999 and near


def compare_chmc(res, ref, name):
    r = ref["rank"]
    assert res.rank == r
    if r > 0:
        Ag = res.A.cpu().numpy().astype(np.float64)
        sgn = np.sign(np.sum(Ag * ref["A"], axis=0))
        sgn[sgn == 0] = 1.0
        compare_factor(res.A * torch.from_numpy(sgn).to(DEV).half()[None, :], ref["A"],
                       f"{name} A")
        compare_factor(res.B * torch.from_numpy(sgn).to(DEV).half()[:, None], ref["B"],
                       f"{name} B")
    codes = res.codes.cpu().numpy().astype(np.int64)
    agree = float(np.mean(codes == ref["codes"]))
    sc = res.scales.cpu().numpy().astype(np.float64)
    s_ok = float(np.mean(np.abs(sc - ref["scales"]) <= SCALE_RTOL * np.abs(ref["scales"])))
    z_ok = float(np.mean(res.zeros.cpu().numpy().astype(np.float64) == ref["zeros"]))
    lg, lr = float(res.row_loss.sum().item()), float(ref["row_loss"].sum())
    say(f"{name}: rank {r} codes {agree:.6f} scales {s_ok:.6f} zeros {z_ok:.6f} "
        f"loss gpu {lg:.6e} oracle {lr:.6e}")
    assert agree >= CODE_AGREE and s_ok >= SCALE_AGREE and z_ok >= SCALE_AGREE
    assert abs(lg - lr) <= LOSS_RTOL * lr


def run_case(rows, cols, n, bits, gs, act, rank, seed, lowrank=0, bpw=4.2875):
    W, X = problem(rows, cols, n, seed, lowrank)
    S, perm, U = gpu_inputs(X, act)
    om = np.random.default_rng(seed + 1).standard_normal((cols, max(rank or 0, 64)))
    Sr, nr = O.hessian_sum(X)
    ref = O.chmc_layer(W, Sr, nr, om, bits=bits, group_size=gs, bpw_target=bpw, act_order=act,
                       rank=rank)
    if act:
        assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    res = G.chmc_layer(torch.from_numpy(W).to(DEV), S, n, U, perm, torch.from_numpy(om).to(DEV),
                       rank=rank, bits=bits, group_size=gs, bpw_target=bpw)
    return res, ref


def test_chmc_page_example_576():
    """576 x 576 at 4.2875 bits per weight: rank 2 from the budget."""
    say("chmc 576x576 b4 g128 act, rank from the budget")
    res, ref = run_case(576, 576, 1300, 4, 128, True, None, 11, lowrank=3)
    assert ref["rank"] == 2
    compare_chmc(res, ref, "chmc 576")


@pytest.mark.parametrize("rows,cols,n,bits,gs,act,rank", [
    (200, 333, 700, 3, 64, False, 5),
    (37, 129, 300, 2, 32, True, 0),
    (130, 260, 600, 4, 128, True, 64),
    (300, 128, 400, 4, 32, True, 3),
])
def test_chmc_ragged_matches_oracle(rows, cols, n, bits, gs, act, rank):
    say(f"chmc {rows}x{cols} b{bits} g{gs} act={act} rank={rank}")
    res, ref = run_case(rows, cols, n, bits, gs, act, rank, rows * 7 + cols, lowrank=2)
    compare_chmc(res, ref, f"chmc {rows}x{cols}")


def test_chmc_qwen_down_projection_full_shape():
    """896 x 4864 (the Qwen2.5-0.5B down projection), SiLU-gated activations,
    rank from the 4.2875-bit budget (6). The oracle's factors in full; its
    residual sweep for one sampled row group (row groups are independent:
    each has its own grids and rows), compared with that group of the GPU
    result."""
    say("chmc qwen down 896x4864")
    rows, dim, n, gs = 896, 4864, 2048, 128
    X = synth.activations(1, "down_in", n, dim, kind="silu_gated")
    W = synth.weights(1, "down_proj", rows, dim)
    S, perm, U = gpu_inputs(X, True)
    om = np.random.default_rng(5).standard_normal((dim, 64))
    res = G.chmc_layer(torch.from_numpy(W).to(DEV), S, n, U, perm, torch.from_numpy(om).to(DEV))
    Sr, nr = O.hessian_sum(X)
    r = O.chmc_rank(rows, dim, 4, gs, 4.2875)
    assert r == 6 and res.rank == r
    c = O.chmc_energies(np.diag(Sr), nr)
    A, B = O.chmc_lowrank(W.astype(np.float64), c, om[:, :r], 5)
    ref = {"rank": r, "A": A, "B": B}
    H = O.damped_hessian(Sr, nr, O.CHMC_DAMP)
    pr = O.act_order_perm(H)
    assert np.array_equal(perm.cpu().numpy(), pr)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    g = 3
    rs = slice(g * gs, (g + 1) * gs)
    R = W.astype(np.float64)[rs] - A[rs] @ B
    sw = O.gptq_sweep_outgroups(R[:, pr], Ur, 4, gs)
    for key in ("codes", "scales", "zeros"):
        a = np.empty_like(sw[key])
        a[:, pr] = sw[key]
        ref[key] = a
    ref["row_loss"] = sw["row_loss"]
    sub = G.CHMCLayer(res.A, res.B, res.codes[rs], res.scales[g:g + 1], res.zeros[g:g + 1],
                      res.row_loss[rs], r, 4, gs)
    compare_chmc(sub, ref, f"chmc qwen down, row group {g}")


def test_chmc_rank_matches_oracle():
    for shape in [(576, 576), (896, 4864), (4864, 896), (37, 129), (1, 1)]:
        for bits, gs, bpw in [(4, 128, 4.2875), (3, 64, 3.5), (2, 32, 8.0), (4, 128, 4.0)]:
            assert G.chmc_rank(*shape, bits, gs, bpw) == O.chmc_rank(*shape, bits, gs, bpw,
                                                                       max_rank=64)


def test_chmc_low_rank_weight_is_rejected():
    say("chmc zero weight, rank 2: the sketch loses rank")
    _, X = problem(64, 128, 300, 3)
    S, perm, U = gpu_inputs(X, True)
    W = torch.zeros((64, 128), dtype=torch.float16, device=DEV)
    om = torch.from_numpy(np.random.default_rng(1).standard_normal((128, 2))).to(DEV)
    with pytest.raises(G.GPTQError) as e:
        G.chmc_layer(W, S, 300, U, perm, om, rank=2)
    assert e.value.status == G.GPTQ_ENOTSPD


def test_chmc_bad_permutation_is_rejected():
    say("chmc duplicate entry in perm")
    W, X = problem(64, 128, 300, 4)
    S, perm, U = gpu_inputs(X, True)
    bad = perm.clone()
    bad[5] = bad[6]
    om = torch.from_numpy(np.random.default_rng(1).standard_normal((128, 2))).to(DEV)
    with pytest.raises(G.GPTQError) as e:
        G.chmc_layer(torch.from_numpy(W).to(DEV), S, 300, U, bad, om, rank=2)
    assert e.value.status == G.GPTQ_EINVAL


@pytest.mark.parametrize("rank", [0, 2])
def test_chmc_nonfinite_weight_is_reported(rank):
    say(f"chmc NaN weight, rank {rank}")
    W, X = problem(64, 128, 300, 6)
    S, perm, U = gpu_inputs(X, True)
    W[3, 17] = np.nan
    om = torch.from_numpy(np.random.default_rng(1).standard_normal((128, 2))).to(DEV)
    with pytest.raises(G.GPTQError) as e:
        G.chmc_layer(torch.from_numpy(W).to(DEV), S, 300, U, perm, om, rank=rank)
    assert e.value.status == G.GPTQ_ENONFINITE


def test_chmc_square_2048_g64_sampled():
    """2048 x 2048 (the TinyLlama attention output shape), 3 bits, groups of
    64 output rows, act-order, rank from a 3.5-bit budget: the oracle's
    factors in full and its residual sweep for one sampled row group."""
    rows = cols = 2048
    n, gs, bits, bpw = 2048, 64, 3, 3.5
    say("chmc 2048x2048 b3 g64, sampled row group")
    W, X = problem(rows, cols, n, 77, lowrank=4)
    S, perm, U = gpu_inputs(X, True)
    om = np.random.default_rng(78).standard_normal((cols, 64))
    res = G.chmc_layer(torch.from_numpy(W).to(DEV), S, n, U, perm, torch.from_numpy(om).to(DEV),
                       bits=bits, group_size=gs, bpw_target=bpw)
    Sr, nr = O.hessian_sum(X)
    r = O.chmc_rank(rows, cols, bits, gs, bpw, max_rank=64)
    assert r > 0 and res.rank == r
    c = O.chmc_energies(np.diag(Sr), nr)
    A, B = O.chmc_lowrank(W.astype(np.float64), c, om[:, :r], 5)
    ref = {"rank": r, "A": A, "B": B}
    H = O.damped_hessian(Sr, nr, O.CHMC_DAMP)
    pr = O.act_order_perm(H)
    assert np.array_equal(perm.cpu().numpy(), pr)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    g = 17
    rs = slice(g * gs, (g + 1) * gs)
    R = W.astype(np.float64)[rs] - A[rs] @ B
    sw = O.gptq_sweep_outgroups(R[:, pr], Ur, bits, gs)
    for key in ("codes", "scales", "zeros"):
        a = np.empty_like(sw[key])
        a[:, pr] = sw[key]
        ref[key] = a
    ref["row_loss"] = sw["row_loss"]
    sub = G.CHMCLayer(res.A, res.B, res.codes[rs], res.scales[g:g + 1], res.zeros[g:g + 1],
                      res.row_loss[rs], r, bits, gs)
    compare_chmc(sub, ref, f"chmc 2048, row group {g}")


def test_chmc_strided_weight_matches_contiguous():
    """W given as a column slice of a wider matrix (row stride > cols): the
    same results as the contiguous copy, bit for bit."""
    say("chmc strided W (ldw 300 > cols 256)")
    W, X = problem(96, 256, 600, 9, lowrank=2)
    S, perm, U = gpu_inputs(X, True)
    om = torch.from_numpy(np.random.default_rng(2).standard_normal((256, 4))).to(DEV)
    wide = torch.zeros((96, 300), dtype=torch.float16, device=DEV)
    wide[:, 17:17 + 256] = torch.from_numpy(W).to(DEV)
    Ws = wide[:, 17:17 + 256]
    assert Ws.stride(0) == 300
    a = G.chmc_layer(Ws, S, 600, U, perm, om, rank=4, group_size=32)
    b = G.chmc_layer(torch.from_numpy(W).to(DEV), S, 600, U, perm, om, rank=4, group_size=32)
    for x, y in ((a.A, b.A), (a.B, b.B), (a.codes, b.codes), (a.scales, b.scales),
                 (a.zeros, b.zeros), (a.row_loss, b.row_loss)):
        assert torch.equal(x, y)


def test_chmc_no_sync_reports_through_the_workspace():
    """With GPTQ_FLAG_NO_SYNC the call returns after enqueueing; the status
    is read from the workspace afterwards (a bad permutation here)."""
    say("chmc no-sync: status from the workspace")
    W, X = problem(64, 128, 300, 10)
    S, perm, U = gpu_inputs(X, True)
    om = torch.from_numpy(np.random.default_rng(3).standard_normal((128, 2))).to(DEV)
    ws = torch.empty(G.chmc_workspace_bytes(64, 128, 2), dtype=torch.uint8, device=DEV)
    good = G.chmc_layer(torch.from_numpy(W).to(DEV), S, 300, U, perm, om, rank=2, sync=False,
                        workspace=ws)
    G.workspace_status(ws)  # no error
    ref = G.chmc_layer(torch.from_numpy(W).to(DEV), S, 300, U, perm, om, rank=2)
    assert torch.equal(good.codes, ref.codes) and torch.equal(good.A, ref.A)
    bad = perm.clone()
    bad[1] = bad[0]  # a repeated entry
    G.chmc_layer(torch.from_numpy(W).to(DEV), S, 300, U, bad, om, rank=2, sync=False,
                 workspace=ws)
    with pytest.raises(G.GPTQError) as e:
        G.workspace_status(ws)
    assert e.value.status == G.GPTQ_EINVAL


def test_chmc_frontend_overlaps_the_factorization():
    """prepare_hinv enqueued on one stream, the CHMC call on another with
    u_stream = the first: the frontend runs at once, the sweep waits for U;
    the results equal those of the call made after U is ready, bit for bit."""
    say("chmc with u_stream: overlap with prepare")
    W, X = problem(256, 1024, 2100, 12, lowrank=3)
    dim, n = 1024, 2100
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
    om = torch.from_numpy(np.random.default_rng(4).standard_normal((dim, 8))).to(DEV)
    Wd = torch.from_numpy(W).to(DEV)
    perm0, U0 = G.prepare_hinv(S, n, damp=O.CHMC_DAMP, act_order=True)
    ref = G.chmc_layer(Wd, S, n, U0, perm0, om, rank=8, group_size=64)
    perm = torch.empty(dim, dtype=torch.int32, device=DEV)
    U = torch.empty((dim, dim), dtype=torch.float32, device=DEV)
    pws = torch.empty(G.prepare_workspace_bytes(dim), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        G.prepare_hinv(S, n, damp=O.CHMC_DAMP, act_order=True, workspace=pws, out=(perm, U),
                       sync=False)
    with torch.cuda.stream(s2):
        res = G.chmc_layer(Wd, S, n, U, perm, om, rank=8, group_size=64, u_stream=s1)
    torch.cuda.synchronize()
    G.workspace_status(pws)
    for x, y in ((res.A, ref.A), (res.B, ref.B), (res.codes, ref.codes),
                 (res.scales, ref.scales), (res.zeros, ref.zeros), (res.row_loss, ref.row_loss)):
        assert torch.equal(x, y)


def test_chmc_pipeline_two_streams_equals_serial_calls():
    """LayerGroup.chmc (the benchmark's configuration: Hessian, factor on the
    calling stream, the CHMC calls forked onto a side stream that overlaps the
    factorization, outputs in the group's buffers) against a serial run of the
    same library calls, bit for bit, twice in a row (the buffers are reused),
    with every status read through check()."""
    from post_weight_quantization_hessian_amd.pipeline import CHMC_DAMP, LayerGroup
    say("chmc pipeline fork/join against serial calls")
    dim, n, gs, bpw = 640, 1500, 64, 5.0  # ranks 6, 15, 1, 5
    layers = [("a", 192), ("b", 70)]
    rng = np.random.default_rng(31)
    X = (rng.standard_normal((n, dim)) * np.exp(0.5 * rng.standard_normal(dim))[None, :]
         + 0.8 * rng.standard_normal((n, 1))).astype(np.float32)
    W = np.concatenate([(0.02 * rng.standard_t(4, size=(r, dim))
                         + 0.05 * rng.standard_normal((r, 2)) @ rng.standard_normal((2, dim)))
                        .astype(np.float16) for _, r in layers], axis=0)
    Wd = torch.from_numpy(W).to(DEV)
    chunks = [torch.from_numpy(X[:700]).to(DEV), torch.from_numpy(X[700:]).to(DEV)]
    om = torch.from_numpy(rng.standard_normal((dim, 64))).to(DEV)
    grp = LayerGroup(dim, W.shape[0], max_chunk_tokens=800, bits=(4, 3), group_size=gs,
                     act_order=True, damp=0.01, device=DEV)
    # serial reference: the same calls, one after the other on one stream
    S = torch.empty((dim, dim), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, chunks[0], overwrite=True)
    G.hessian_accumulate(S, chunks[1])
    ff = grp.factor_form  # the group's form (U below 768 features)
    perm, U = G.prepare_hinv(S, n, damp=CHMC_DAMP, act_order=True, factor_form=ff)
    ref, r0 = {}, 0
    for name, rows in layers:
        for b in (4, 3):
            ref[(name, b)] = G.chmc_layer(Wd[r0:r0 + rows], S, n, U, perm, om, bits=b,
                                          group_size=gs, bpw_target=bpw, factor_form=ff)
        r0 += rows
    for rep in range(2):
        out = grp.chmc(chunks, Wd, layers, bpw, om)
        grp.check()
        torch.cuda.synchronize()
        assert torch.equal(grp.S, S) and torch.equal(grp.U, U) and torch.equal(grp.perm, perm)
        assert [(nm, b) for nm, b, _ in out] == list(ref)
        for name, b, q in out:
            e = ref[(name, b)]
            assert q.rank == e.rank > 0
            for x, y in ((q.A, e.A), (q.B, e.B), (q.codes, e.codes), (q.scales, e.scales),
                         (q.zeros, e.zeros), (q.row_loss, e.row_loss)):
                assert torch.equal(x, y), (rep, name, b)


@pytest.mark.parametrize("rows,cols,n,bits,gs,act,rank", [
    (200, 333, 700, 3, 64, False, 5),
    (300, 896, 1900, 4, 128, True, 6),
])
def test_chmc_factor_form_matches_oracle(rows, cols, n, bits, gs, act, rank):
    """The residual sweep in the factor form (U's diagonal blocks, R U beyond
    them; the residuals q - r through it give the errors' update sums)
    against the oracle's CHMC layer, at the same bar."""
    say(f"chmc factor form {rows}x{cols} b{bits} g{gs} act={act} rank={rank}")
    W, X = problem(rows, cols, n, rows * 11 + cols, lowrank=2)
    S = torch.zeros((cols, cols), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
    perm, M = G.prepare_hinv(S, n, damp=O.CHMC_DAMP, act_order=act, factor_form=True)
    om = np.random.default_rng(rows + 1).standard_normal((cols, 64))
    Sr, nr = O.hessian_sum(X)
    ref = O.chmc_layer(W, Sr, nr, om, bits=bits, group_size=gs, act_order=act, rank=rank)
    if act:
        assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    res = G.chmc_layer(torch.from_numpy(W).to(DEV), S, n, M, perm if act else None,
                       torch.from_numpy(om).to(DEV), rank=rank, bits=bits, group_size=gs,
                       factor_form=True)
    compare_chmc(res, ref, f"chmc factor form {rows}x{cols}")
