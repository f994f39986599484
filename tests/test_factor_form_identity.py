"""CPU: the factor form of the blocked sweep reproduces the oracle's sweep.

The library's benchmark path sweeps with M = R[blk_a, blk_b] U[blk_b, blk_b]
beyond U's 128-wide diagonal blocks, R = U^-1 the order-reversed Cholesky
factor of H_p (H_p = R R^T): with the scaled errors E = (W - Q) R (from
W - Q = E U, since each column's total change is the sum of its errors
through U), the current values of a block are
    W~[:, blk] = W[:, blk] - E[:, :j0] U[:j0, blk]
               = W[:, blk] - (Q - W)[:, :j0] M[:j0, blk]
(R[:j0, :j0] U[:j0, blk] = -R[:j0, blk] U[blk, blk], U being upper). This
test restates that sweep in plain numpy, written from the derivation above
(not from the library), and holds it to the oracle's strict sweep (CHMC
article, Methodik, Schritt 2) exactly in fp64 on small problems: every code,
grid and the loss.
"""
import numpy as np
import pytest

import oracle as O
from oracle import gptq_oracle as OO

B = 128


def factor_form_sweep(Wp, Hp, bits, gs):
    n = Hp.shape[0]
    R = np.linalg.cholesky(Hp[::-1, ::-1])[::-1, ::-1]  # upper, Hp = R R^T
    U = np.linalg.inv(R)
    M = np.zeros_like(R)  # R U over the block columns, beyond the diagonal blocks
    for b0 in range(0, n, B):
        b1 = min(b0 + B, n)
        M[:b0, b0:b1] = R[:b0, b0:b1] @ U[b0:b1, b0:b1]
    maxq = (1 << bits) - 1
    rows = Wp.shape[0]
    codes = np.zeros((rows, n), np.int64)
    resid = np.zeros((rows, n))
    loss = np.zeros(rows)
    scales = np.zeros((rows, -(-n // gs)))
    zeros = np.zeros_like(scales)
    for j0 in range(0, n, B):
        j1 = min(j0 + B, n)
        Ub = U[j0:j1, j0:j1]
        V = Wp[:, j0:j1] - resid[:, :j0] @ M[:j0, j0:j1]
        for jj in range(j1 - j0):
            j = j0 + jj
            g = j // gs
            if j % gs == 0:
                scales[:, g], zeros[:, g] = O.group_grid(V[:, jj:jj + gs], bits)
            q, dq = OO._quantize(V[:, jj], scales[:, g], zeros[:, g], maxq, True)
            codes[:, j] = q
            e = (V[:, jj] - dq) / Ub[jj, jj]
            loss += e * e
            V[:, jj + 1:] -= np.outer(e, Ub[jj, jj + 1:])
            resid[:, j] = dq - Wp[:, j]
    return codes, scales, zeros, loss


@pytest.mark.parametrize("rows,cols,bits,gs,seed", [
    (8, 300, 4, 128, 1), (12, 260, 3, 64, 2), (5, 129, 2, 32, 3), (16, 400, 4, 16, 4),
])
def test_factor_form_equals_oracle_sweep(rows, cols, bits, gs, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((3 * cols, cols)) * np.exp(0.5 * rng.standard_normal(cols))
         + 0.8 * rng.standard_normal((3 * cols, 1))).astype(np.float32)
    W = (0.02 * rng.standard_t(4, size=(rows, cols))).astype(np.float16).astype(np.float64)
    S, n = O.hessian_sum(X)
    H = O.damped_hessian(S, n, 0.01)
    p = O.act_order_perm(H)
    Hp = O.permute_sym(H, p)
    ref = O.gptq_sweep(W[:, p], O.hinv_upper(Hp), bits, gs)
    codes, scales, zeros, loss = factor_form_sweep(W[:, p], Hp, bits, gs)
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(scales, ref["scales"]) and np.array_equal(zeros, ref["zeros"])
    assert abs(loss.sum() - ref["row_loss"].sum()) <= 1e-9 * ref["row_loss"].sum()


def test_factor_form_with_a_wrong_block_fails():
    """The same check fails when the block's own diagonal block of U is left
    out of the conversion (a plausible slip: R used as if it were U)."""
    rng = np.random.default_rng(7)
    cols = 300
    X = (rng.standard_normal((900, cols)) + 0.8 * rng.standard_normal((900, 1))).astype(np.float32)
    W = (0.02 * rng.standard_t(4, size=(8, cols))).astype(np.float16).astype(np.float64)
    S, n = O.hessian_sum(X)
    Hp = O.damped_hessian(S, n, 0.01)
    ref = O.gptq_sweep(W, O.hinv_upper(Hp), 4, 128)
    R = np.linalg.cholesky(Hp[::-1, ::-1])[::-1, ::-1]
    U = np.linalg.inv(R)
    # block 1's current values without the diagonal-block factor
    V_wrong = W[:, 128:256] + (W[:, :128] - ref["deq"][:, :128]) @ R[:128, 128:256]
    V_right = W[:, 128:256] + (W[:, :128] - ref["deq"][:, :128]) @ R[:128, 128:256] @ U[128:256, 128:256]
    V_ref = W[:, 128:256] - ref["E"][:, :128] @ hinv_block(Hp)[:128, 128:256]
    assert np.allclose(V_right, V_ref, rtol=0, atol=1e-12)
    assert not np.allclose(V_wrong, V_ref, rtol=0, atol=1e-6)


def hinv_block(Hp):
    return O.hinv_upper(Hp)
