"""Full-size parity of the two largest layer workloads, in the launch
configuration the benchmark times (LayerGroup.enqueue: chunked accumulate
with overwrite on the first chunk, asynchronous prepare and quantize).

* 8B-shape down projection 4096 x 14336: 131072 calibration tokens in 8192-
  token chunks, 0.1 % outlier input columns, 3-bit groups of 128, act-order.
* 70B-shape down projection 8192 x 28672: 65536 tokens with log-normal channel
  scales, 2-bit and 4-bit groups of 64, act-order.

The oracle's own results for 64 seeded rows of every layer and bit width are
stored under tests/golden/ (written by tests/golden/make_fullsize_goldens.py,
which calls only the seeded generator and the oracle: the whole S over all
tokens, the damped H, act-order, U = chol(inv(H_p))^T and the strict sweep of
those rows). The GPU's act-order must equal the stored one, and its codes,
scales, zero points and row losses on those rows meet the parity bar against
the stored ones (CHMC article, Methodik, Schritt 2).

Beside that, the oracle computes what it can on the box one piece at a time:

* sampled entries of S, each the exactly rounded sum over all tokens;
* diag S of every feature, the damping term and the act-order permutation;
* the trailing 256 x 256 block of the factor-form matrix that the benchmark's
  sweep takes (U's 128-wide diagonal blocks, R = U^-1 beyond them): with
  U^T U = H_p^-1 and H_p = R R^T, that block depends only on the trailing
  block of H_p, which the oracle forms and factors;
* the first group of every row: nothing has been propagated into it yet, so
  its grid and its first column's codes are round-to-nearest of the weights.

When the layer group takes the int8 digit-slice Hessian (as the benchmark
does at these widths), S is X~^T X~ for the per-chunk fixed-point X~ that the
library documents; the oracle quantities above are then formed from X~ (exact
integer sums), and the sampled entries are also held to the exact X^T X
within the bound that the rounding of X implies.

and properties of the library's outputs hold at any size:

* R's last column is H_p's last column over its last diagonal entry's
  square root (sampled rows), and nothing is stored below the diagonal;
* sum_j e_j^2 = (w - q) H (w - q)^T (the loss identity, sampled rows);
* codes, zero points and g_idx are valid; a second run is bit-identical.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_hessian_amd import synth
from post_weight_quantization_hessian_amd.workloads import WORKLOADS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

from post_weight_quantization_hessian_amd.pipeline import LayerGroup  # noqa: E402
from tests import split8_ref as R8  # noqa: E402
from tests.parity_util import CODE_AGREE, compare_layer, first_divergence  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

DEV = torch.device("cuda:0")
F64 = np.float64

S_SAMPLES = 40
TRAIL = 256
# |(U H_p)[j, k>j]| <= U_TOL (|U| |H_p|)[j, k]: storing U in fp32 alone
# leaves about 3e-8 (2^-24 per entry).
U_TOL = 4e-7
# loss identity with the fp32-stored U: about 1e-7 at the medium shapes
LOSS_ID_TOL = 1e-4
HOST_CHUNK = 8192


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def host_chunks(X):
    return [X[s:s + HOST_CHUNK] for s in range(0, X.shape[0], HOST_CHUNK)]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("wname", ["llama8b_down", "llama70b_down"])
def test_fullsize_sampled(wname):
    wl = WORKLOADS[wname]
    (h,) = wl.inputs
    dim, n, gsz = h.dim, wl.n_tokens, wl.group_size
    t0 = time.time()
    say(f"{wname}: generating X {n} x {dim}")
    X = synth.activations(wl.wid, h.name, n, dim, kind=h.kind, lognormal_sigma=h.lognormal_sigma)
    W = np.concatenate([synth.weights(wl.wid, l.name, l.rows, dim, outlier_frac=l.outlier_frac)
                        for l in wl.layers_of(h.name)], axis=0)
    rows = W.shape[0]
    say(f"{wname}: inputs ready after {time.time() - t0:.0f} s; path run 1")
    chunks = [torch.from_numpy(X[s:s + wl.token_chunk]).to(DEV)
              for s in range(0, n, wl.token_chunk)]
    Wd = torch.from_numpy(W).to(DEV)
    grp = LayerGroup(dim, rows, max_chunk_tokens=max(c.shape[0] for c in chunks), bits=wl.bits,
                     group_size=gsz, act_order=wl.act_order, damp=wl.damp, device=DEV,
                     hessian="auto")
    split8 = grp.split8
    # the library's calls: one per token chunk (split8 scales are per call)
    calls = [X[s:s + wl.token_chunk] for s in range(0, n, wl.token_chunk)]
    grp.enqueue(chunks, Wd)
    grp.check()
    first = dict(S=grp.S.clone(), U=grp.U.clone(), perm=grp.perm.clone(),
                 outs=[(q.codes.clone(), q.scales.clone(), q.zeros.clone(), q.row_loss.clone())
                       for q in grp.outs])
    say(f"{wname}: path run 2 (determinism)")
    grp.enqueue(chunks, Wd)
    grp.check()
    assert torch.equal(first["S"], grp.S) and torch.equal(first["U"], grp.U)
    assert torch.equal(first["perm"], grp.perm)
    for (c, s, z, l), q in zip(first["outs"], grp.outs):
        assert torch.equal(c, q.codes) and torch.equal(s, q.scales)
        assert torch.equal(z, q.zeros) and torch.equal(l, q.row_loss)
    del first, chunks
    torch.cuda.empty_cache()

    S, U = grp.S, grp.U
    perm = grp.perm.cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(20240 + wl.wid)

    # ---- S: sampled entries against exactly rounded sums
    say(f"{wname}: sampled Hessian entries")
    fs = rng.integers(0, dim, S_SAMPLES)
    gs_ = rng.integers(0, dim, S_SAMPLES)
    pairs = list(zip(fs.tolist(), gs_.tolist())) + [(f, f) for f in fs[:8].tolist()]
    pairs += [(0, dim - 1), (dim - 1, dim - 1), (dim - 1, 0), (0, 0)]
    fi = torch.tensor([p[0] for p in pairs], device=DEV)
    gi = torch.tensor([p[1] for p in pairs], device=DEV)
    Sg = S[fi, gi].cpu().numpy()
    assert np.array_equal(Sg, S[gi, fi].cpu().numpy()), "S is not exactly symmetric"
    if split8:
        # per chunk: the call's column exponents, then the fixed-point sums
        # and rounding bounds on the sampled columns only
        ucols = np.unique(np.array(pairs).ravel())
        pos = {c: i for i, c in enumerate(ucols.tolist())}
        Tref = np.zeros((len(ucols), len(ucols)))
        Tmag = np.zeros_like(Tref)
        Tbnd = np.zeros_like(Tref)
        for c in calls:
            e = R8.col_exponent(c)[ucols]
            cu = c[:, ucols]
            t, mg = R8.split8_gram(cu, e=e)
            Tref += t
            Tmag += mg
            Tbnd += R8.split8_bound(cu, e=e)
    worst = 0.0
    for k, (f, g) in enumerate(pairs):
        exact = O.hessian_entry(X, f, g)
        mag = float(np.abs(X[:, f].astype(F64) * X[:, g].astype(F64)).sum())
        err = abs(Sg[k] - exact)
        if split8:
            # the split8 sum (X~^T X~ without the digit orders 5 and 6)
            # exactly per chunk; the library adds 5 digit orders, the chunk
            # to S, and rounds each
            i, j = pos[f], pos[g]
            ref, rmag, bnd = Tref[i, j], Tmag[i, j], Tbnd[i, j]
            assert abs(Sg[k] - ref) <= (24 + len(calls)) * 2.0 ** -53 * rmag, (f, g)
            assert err <= bnd + n * 2.0 ** -53 * mag, (f, g, Sg[k], exact, bnd)
            worst = max(worst, abs(Sg[k] - ref) / rmag)
        else:
            assert err <= n * 2.0 ** -53 * mag, (f, g, Sg[k], exact)
            worst = max(worst, err / mag)
    # a running fp64 sum over n terms: worst case n*u (asserted per entry
    # above), typically sqrt(n)*u, about 4e-14 at 131072 tokens (split8:
    # against the fixed-point sums, a few roundings per chunk)
    assert worst < 1e-12, worst

    # ---- diag, damping, act-order
    say(f"{wname}: diagonal and act-order")
    if split8:
        d = sum(R8.split8_diag(c) for c in calls)
        nn = sum(c.shape[0] for c in calls)
    else:
        d, nn = O.hessian_diag(host_chunks(X))
    assert nn == n
    dg = torch.diagonal(S).cpu().numpy()
    assert np.max(np.abs(dg - d) / d) < 1e-12  # running sums, as for the entries above
    hdiag, lam = O.damped_diagonal(d, n, wl.damp)
    pr = O.act_order_from_diag(hdiag)
    assert np.array_equal(np.sort(perm), np.arange(dim))
    for k in np.nonzero(perm != pr)[0]:  # only inside classes of near-equal diagonals
        assert abs(hdiag[perm[k]] - hdiag[pr[k]]) <= 1e-12 * hdiag[pr[k]], k

    # ---- trailing block of the factor-form matrix from the trailing block of
    # H_p alone: U's two diagonal 128-blocks, R U_bb above them (the trailing
    # block of R = U^-1 is the inverse of the trailing block of U)
    say(f"{wname}: trailing {TRAIL}x{TRAIL} block of the factor-form matrix")
    assert grp.factor_form and dim % 128 == 0
    assert np.array_equal(perm[-TRAIL:], pr[-TRAIL:])
    cols_b = pr[-TRAIL:]
    if split8:  # chunk scales come from the full columns, which cols_b keeps
        Sb = sum(R8.split8_gram(c[:, cols_b], e=R8.col_exponent(c)[cols_b])[0]
                 for c in calls)
    else:
        Sb, _ = O.hessian_sum([c[:, cols_b] for c in host_chunks(X)])
    Ub = O.hinv_upper(O.damped_hessian(Sb, n, wl.damp, lam=lam))
    Rb = np.linalg.inv(Ub)
    Mg = U[-TRAIL:, -TRAIL:].double().cpu().numpy()
    RU = Rb.copy()
    RU[:128, 128:] = Rb[:128, 128:] @ Ub[128:, 128:]
    for (a0, b0, ref) in ((0, 0, Ub), (128, 128, Ub), (0, 128, RU)):
        e = ref[a0:a0 + 128, b0:b0 + 128]
        g_ = Mg[a0:a0 + 128, b0:b0 + 128]
        rowmax = np.abs(e).max(axis=1, keepdims=True)
        bound = 2.0 ** -23 * np.abs(e) + 1e-7 * rowmax
        assert np.all(np.abs(g_ - e) <= bound), (a0, b0, float(np.max(np.abs(g_ - e) / rowmax)))
    assert np.all(Mg[128:, :128] == 0)

    # ---- sampled rows: zero below the diagonal, and the last block column:
    # (R U)[j, B] = H_p[j, B] H_p[B, B]^-1 for the last 128-block B (H_p =
    # R R^T with R upper: R[j, B] R[B, B]^T = H_p[j, B], and R[B, B]^-T
    # U[B, B] = U[B, B]^T U[B, B] = H_p[B, B]^-1)
    say(f"{wname}: the last block column of the factor-form matrix on sampled rows")
    Hd = S * (2.0 / n)
    Hd.diagonal().add_(lam)
    J = sorted(set([0, 1, dim // 3, dim // 2, dim - TRAIL - 1]
                   + rng.integers(0, dim - 128, 7).tolist()))
    jt = torch.tensor(J, device=DEV)
    cols = torch.arange(dim, device=DEV)
    Mrows = U[jt].double()
    assert torch.all(Mrows[cols[None, :] < jt[:, None]] == 0), "entries below the diagonal"
    pt = torch.from_numpy(perm).to(DEV)
    last = pt[dim - 128:]
    HjB = Hd[pt[jt]][:, last]
    HBB = Hd[last][:, last]
    ref = torch.linalg.solve(HBB, HjB.T).T  # H_p[j, B] H_p[B, B]^-1 (HBB symmetric)
    rel = ((Mrows[:, dim - 128:] - ref).abs().max() / ref.abs().max()).item()
    assert rel <= U_TOL, rel

    # ---- the oracle's stored sweep of 64 sampled rows (whole-Hessian oracle)
    gold = np.load(os.path.join(GOLDEN, f"fullsize_{wname}.npz"))
    assert int(gold["n_rows_total"]) == rows and int(gold["group_size"]) == gsz
    assert tuple(gold["bits"].tolist()) == tuple(wl.bits)
    assert np.array_equal(perm, gold["perm"].astype(np.int64)), "act-order differs from the oracle's"
    sel = gold["rows"].astype(np.int64)
    g_gold = np.empty(dim, dtype=np.int64)
    g_gold[gold["perm"].astype(np.int64)] = np.arange(dim) // gsz
    for bi, bits in enumerate(wl.bits):
        q = grp.outs[bi]
        gpu = dict(codes=q.codes[sel].cpu().numpy().astype(np.int64),
                   scales=q.scales[sel].cpu().numpy().astype(F64),
                   zeros=q.zeros[sel].cpu().numpy().astype(F64),
                   row_loss=q.row_loss[sel].cpu().numpy())
        ref = dict(codes=gold[f"codes_{bits}"].astype(np.int64),
                   scales=gold[f"scales_{bits}"].astype(F64),
                   zeros=gold[f"zeros_{bits}"].astype(F64),
                   row_loss=gold[f"row_loss_{bits}"], g_idx=g_gold)
        rep = compare_layer(gpu, ref, name=f"{wname} {bits}-bit, {len(sel)} oracle rows")
        fd = first_divergence(gpu["codes"][:, pr], ref["codes"][:, pr])
        say(f"{wname}/{bits}-bit: rows with a differing code {int((fd < dim).sum())}, "
            f"first divergence (sweep order) min {int(fd.min())}")
        assert rep["codes_agree"] >= CODE_AGREE

    # ---- sweep outputs, per bit width
    Wp = W.astype(F64)[:, pr]
    g_ref = np.empty(dim, dtype=np.int64)
    g_ref[pr] = np.arange(dim) // gsz
    for bi, bits in enumerate(wl.bits):
        say(f"{wname}: sweep outputs, {bits}-bit")
        q = grp.outs[bi]
        codes = q.codes.cpu().numpy().astype(np.int64)
        scales = q.scales.cpu().numpy().astype(F64)
        zeros = q.zeros.cpu().numpy().astype(F64)
        row_loss = q.row_loss.cpu().numpy()
        maxq = 2 ** bits - 1
        assert codes.min() >= 0 and codes.max() <= maxq
        assert np.all(zeros == np.rint(zeros)) and zeros.min() >= 0 and zeros.max() <= maxq
        assert np.all(np.isfinite(scales)) and np.all(scales > 0)
        assert np.array_equal(q.g_idx.cpu().numpy().astype(np.int64), g_ref)
        # first group: round-to-nearest of the untouched weights
        c_rtn, s_rtn, z_rtn = O.rtn_quantize(Wp[:, :gsz], bits, gsz)
        assert np.array_equal(scales[:, 0], s_rtn[:, 0])
        assert np.array_equal(zeros[:, 0], z_rtn[:, 0])
        assert np.array_equal(codes[:, pr[0]], c_rtn[:, 0])
        # loss identity on sampled rows
        R = np.sort(rng.choice(rows, 16, replace=False))
        deq = O.dequantize_sweep(codes[R][:, pr], scales[R], zeros[R], gsz)
        D = np.empty((len(R), dim))
        D[:, pr] = Wp[R] - deq
        Dt = torch.from_numpy(D).to(DEV)
        lq = ((Dt @ Hd) * Dt).sum(dim=1).cpu().numpy()
        rel = np.abs(lq / row_loss[R] - 1.0)
        say(f"{wname}/{bits}-bit: loss identity max rel {rel.max():.2e}; "
            f"mean row loss {row_loss.mean():.4e}")
        assert rel.max() <= LOSS_ID_TOL, rel
    say(f"{wname}: done after {time.time() - t0:.0f} s")
