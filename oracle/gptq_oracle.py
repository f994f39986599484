"""Plain fp64 CPU oracle of the GPTQ layer quantizer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s cpu_baseline leg, never by the HIP product path. It shares
no code with the HIP library; the only thing both sides share is the seeded
input generator, which holds none of the method's arithmetic.

Sources (web pages, cited by title and section):

* [CHMC] "Warum Geometrie Gewichte nicht komprimiert" (nonndazone.ru), section
  "Methodik. Was ist CHMC", Schritt 2 (GPTQ residual step: Hessian from the
  calibration activations, damping lambda*mean(diag H)*I, inverse via Cholesky,
  act-order, per-column rounding and error propagation with the row of the
  inverse factor), Schritt 3 (bits-per-weight formula, groups along input
  channels for GPTQ), Tabelle 1 (GPTQ stores integer indices + group scales).
* [BABAI] "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
  Algorithm" (gist.science), section 2.1 (CVP with basis X*diag(s); Satz 1: any
  factorisation of the Hessian gives an equivalent instance), 2.2 (error
  propagation = projection on the nearest hyperplane; Satz 4: GPTQ run from
  the back equals Babai without LLL), 2.3 (Satz 5: no-clipping bound with the
  LDL diagonal of the permuted Hessian; min-pivot vs act-order).
* [HIGHRATE] "Quantisierte Matrixmultiplikation mit hoher Rate I"
  (gist.science), "Methodik und Theoretischer Rahmen" (rounding error modelled
  as independent uniform noise).

Readings of what the pages leave open (each listed in the design doc):

* H = (2/n) * X^T X. The CHMC page writes X^T X / n; the positive factor does
  not change codes (the update uses U[j,k]/U[j,j]) and only scales the loss.
* Damping: H += damp * mean(diag H) * I, mean over the undamped diagonal.
* The "row of H^-1" in the propagation step is the row of the upper Cholesky
  factor U of H^-1 (U^T U = H^-1), the page's "inverse via Cholesky".
* Groups: gs consecutive columns in sweep (permuted) order, along input
  channels, one fp16 scale and one integer zero point per (row, group).
* Grid (asymmetric min-max): when the sweep reaches a group's first column the
  grid is taken from the *current* (error-updated) values of the group's
  columns: xmin = min(0, min v), xmax = max(0, max v);
  scale = (xmax - xmin)/maxq rounded to the nearest-even fp16 value,
  zero = clamp(rint(-xmin/scale), 0, maxq). A group with xmax == xmin, or
  whose scale rounds to fp16 zero, gets scale 1 and zero 0. A scale that
  overflows fp16 is an error.
* Rounding is round-half-to-even (rint); codes are clamped to [0, maxq]
  unless ``clip=False`` (the no-clipping regime of [BABAI] 2.3).
* Act-order: stable argsort of -diag(H) (ties keep the lower index first).
* Min-pivot order: greedy LDL of the damped H with the smallest Schur
  diagonal as the next pivot (ties: the higher index first); the sweep runs
  in the reverse elimination order (so for a diagonal H it equals act-order,
  ties included).
* Per-row loss: sum_j e_j^2 with e_j = (w~_j - q_j)/U[j,j]; this equals
  (w-q) H (w-q)^T for the damped, permuted H.
* SSQR ([BABAI] 3, "Skalengerechte SpQR"; the page names the scheme and its
  binary search, and prints no rule): a weight whose level would fall
  outside [0, maxq] is an outlier and is kept as its current value rounded to
  fp16 (only that rounding error propagates); one factor alpha per layer
  multiplies every group's min-max scale, scale = fp16(alpha * (xmax -
  xmin)/maxq), with the zero point of the unscaled grid, so the grid shrinks
  about 0; the search bisects alpha for the smallest value whose outlier
  fraction is at most the target.
* HPTQ ([BABAI] 3, Huffman-coded PTQ; named, no rule printed): inliers and
  outliers share one unbounded integer grid, the group step alpha * (xmax -
  xmin)/maxq (fp16) with levels k = rint(v/step) relative to 0 (no zero
  point, no clipping); the layer's levels are Huffman-coded with one
  codebook; bits per weight = (the Huffman-coded length of all levels + 16 per
  group step) / weights (a single distinct level costs 1 bit per weight); the
  search bisects alpha for the smallest value meeting a bits-per-weight
  budget.
* SSQR's and HPTQ's exact grid rules (the alpha factor on the fp16-rounded
  min-max step) are readings of pages that print no rule: their tests pin
  what the readings claim (alpha = 1 is the plain grid, the all-outlier
  limit, nested outliers with a zero point fixed in alpha, one unbounded
  grid); the rules beyond that are parity unpinned.
* CHMC frontend ([CHMC] Schritt 1-3): c_j = (1/n) sum_t x_tj^2 plus 0.05 *
  mean(c); W~ = W diag(sqrt c); a rank-r approximation of W~ by randomized
  subspace iteration (Halko, Martinsson, Tropp 2011, Algorithm 4.4) with q = r
  sketch columns, niter = 5 power iterations and a Gaussian sketch passed in
  (any orthonormal basis of each iterate's span: the result depends on the
  spans only), then the SVD of the small projected matrix; stored factors
  A = fp16(U S) and B = fp16(V^T diag(1/sqrt c)); the residual R = W - A B
  is swept like GPTQ (act-order, H damped with 0.05 as in Anhang A) with one
  grid per group of gs consecutive output channels (rows) and column; r from
  the page's bit budget formula with the residual grid's zero point counted
  at b bits per output group and column (the page counts only the scales).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

__all__ = [
    "NotSPD", "NonFinite", "hessian_sum", "hessian_entry", "hessian_diag",
    "damping_lambda", "damped_diagonal", "damped_hessian", "act_order_from_diag", "act_order_perm", "min_pivot_order", "permute_sym", "hinv_upper", "fp16_round", "group_grid",
    "gptq_sweep", "gptq_layer", "rtn_quantize", "dequantize_sweep",
    "babai_nearest_plane", "brute_force_cvp", "ldl_diag", "noclip_bound",
    "loss_quadratic", "bpw_gptq", "bpw_page", "num_groups", "group_grid_ssqr", "ssqr_search",
    "ssqr_csr", "bpw_ssqr",
    "group_step_hptq", "huffman_lengths", "hptq_bits_per_weight", "hptq_search",
    "huffman_canonical", "huffman_encode", "huffman_decode",
    "CHMC_DAMP", "chmc_energies", "chmc_bits", "chmc_rank", "randomized_lowrank", "chmc_lowrank", "gptq_sweep_outgroups",
    "chmc_layer",
]

F64 = np.float64


class NotSPD(ValueError):
    """The damped Hessian is not symmetric positive definite."""


class NonFinite(ValueError):
    """A non-finite input, or a group scale that overflows fp16."""


# --------------------------------------------------------------------------
# Hessian statistics  ([CHMC] Schritt 2: H = X^T X / n from the calibration
# activations of the layer; accumulation is a plain sum over tokens)
# --------------------------------------------------------------------------

def hessian_sum(chunks):
    """S = sum over token chunks of X_c^T X_c in fp64, and the token count.

    ``chunks`` is one fp32 array [n_tokens x in_features] or an iterable of
    them. fp32 x fp32 products are exact in fp64; only the summation rounds.
    """
    if isinstance(chunks, np.ndarray):
        chunks = [chunks]
    S = None
    n = 0
    for X in chunks:
        Xd = np.asarray(X, dtype=np.float32).astype(F64)
        if not np.all(np.isfinite(Xd)):
            raise NonFinite("calibration activations contain NaN/Inf")
        part = Xd.T @ Xd
        S = part if S is None else S + part
        n += Xd.shape[0]
    return S, n


def hessian_entry(X, f, g):
    """One entry S[f, g] = sum_t X[t,f] X[t,g], summed with math.fsum.

    The products are exact in fp64 and fsum returns the correctly rounded
    sum, so this is the exact value rounded once; used for sampled checks of
    Hessians too large to form on the CPU.
    """
    a = np.asarray(X[:, f], dtype=np.float32).astype(F64)
    b = np.asarray(X[:, g], dtype=np.float32).astype(F64)
    return math.fsum((a * b).tolist())


def hessian_diag(chunks):
    """diag(S) = sum_t X[t,f]^2 for every feature f in fp64, without forming
    S (the diagonal of ``hessian_sum``; for Hessians too large for the CPU)."""
    if isinstance(chunks, np.ndarray):
        chunks = [chunks]
    d = None
    n = 0
    for X in chunks:
        Xd = np.asarray(X, dtype=np.float32).astype(F64)
        part = np.einsum("tf,tf->f", Xd, Xd)
        d = part if d is None else d + part
        n += Xd.shape[0]
    return d, n


def damping_lambda(diag_S, n_tokens, damp):
    """lambda = damp * mean(diag((2/n) S))   ([CHMC] Schritt 2)."""
    if n_tokens <= 0:
        raise ValueError("n_tokens must be positive")
    return damp * float(np.mean((2.0 / n_tokens) * np.asarray(diag_S, dtype=F64)))


def damped_diagonal(diag_S, n_tokens, damp):
    """diag of the damped Hessian, (2/n) diag(S) + lambda, and lambda, from
    diag(S) alone ([CHMC] Schritt 2)."""
    lam = damping_lambda(diag_S, n_tokens, damp)
    return (2.0 / n_tokens) * np.asarray(diag_S, dtype=F64) + lam, lam


def damped_hessian(S, n_tokens, damp, lam=None):
    """H = (2/n) S + damp * mean(diag((2/n) S)) * I   ([CHMC] Schritt 2).

    ``lam`` overrides the damping term when S is a principal block of a
    larger Hessian, whose mean diagonal the block alone does not give."""
    if n_tokens <= 0:
        raise ValueError("n_tokens must be positive")
    H = (2.0 / n_tokens) * np.asarray(S, dtype=F64)
    if lam is None:
        lam = damping_lambda(np.diag(S), n_tokens, damp)
    H = H + lam * np.eye(H.shape[0])
    return H


def act_order_from_diag(hdiag):
    """Columns in descending importance = descending diagonal of the damped
    Hessian, ties kept in index order ([CHMC] Schritt 2 "act-order";
    [BABAI] 2.3)."""
    return np.argsort(-np.asarray(hdiag, dtype=F64), kind="stable").astype(np.int64)


def act_order_perm(H):
    """act-order permutation of a full damped Hessian."""
    return act_order_from_diag(np.diag(H))


def min_pivot_order(H):
    """Min-pivot order ([BABAI] 2.3): the LDL factorisation of H taking, at
    every step, the pivot with the smallest diagonal among the columns not yet
    eliminated, i.e. the smallest diagonal of the current Schur complement
    (ties: the higher index first). The pivots D_j of the no-clipping bound
    are those of the LDL taken from the back of the sweep order, so the sweep
    takes the columns in the reverse elimination order. Returns the sweep
    permutation (as act_order_perm does) and the pivots in elimination order.
    """
    M = np.array(H, dtype=F64, copy=True)
    n = M.shape[0]
    alive = np.ones(n, dtype=bool)
    elim = np.empty(n, dtype=np.int64)
    piv = np.empty(n, dtype=F64)
    for step in range(n):
        d = np.where(alive, np.diag(M), np.inf)
        m = d.min()
        if not (m > 0.0) or not np.isfinite(m):
            raise NotSPD("non-positive pivot in the min-pivot LDL")
        p = int(np.nonzero(d == m)[0][-1])
        elim[step], piv[step] = p, m
        alive[p] = False
        col = M[:, p].copy()
        M -= np.outer(col, col) / m  # Schur complement on the columns still alive
    return elim[::-1].copy(), piv


def permute_sym(H, perm):
    return H[np.ix_(perm, perm)]


def hinv_upper(Hp):
    """U upper triangular with U^T U = Hp^-1: inverse of the Hessian, then
    its Cholesky factor, written as the upper factor ([CHMC] Schritt 2
    "H^-1 via the Cholesky decomposition")."""
    try:
        np.linalg.cholesky(Hp)  # SPD check on H itself
        Hinv = np.linalg.inv(Hp)
        L = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from exc
    return L.T.copy()


# --------------------------------------------------------------------------
# Grid and rounding  ([CHMC] Schritt 2: q_j = round(col_j/scale_g)*scale_g;
# asymmetric min-max grid per group, fp16 scale, integer zero point)
# --------------------------------------------------------------------------

def fp16_round(x):
    """Nearest-even fp16 value of fp64 ``x`` (returned as fp64)."""
    return np.asarray(x, dtype=F64).astype(np.float16).astype(F64)


def group_grid(V, bits):
    """Per-row (scale, zero) from the current values V [rows x g] of a group."""
    maxq = (1 << bits) - 1
    V = np.asarray(V, dtype=F64)
    xmin = np.minimum(V.min(axis=1), 0.0)
    xmax = np.maximum(V.max(axis=1), 0.0)
    with np.errstate(over="ignore"):
        scale = fp16_round((xmax - xmin) / maxq)
    if not np.all(np.isfinite(scale)):
        raise NonFinite("group scale overflows fp16")
    degenerate = (xmax == xmin) | (scale == 0.0)
    scale = np.where(degenerate, 1.0, scale)
    zero = np.clip(np.rint(-xmin / scale), 0, maxq)
    zero = np.where(degenerate, 0.0, zero)
    return scale, zero


def group_grid_ssqr(V, bits, alpha):
    """SSQR grid: the min-max step times ``alpha`` (fp16-rounded), the zero
    point of the unscaled grid. Degenerate (scale 1, zero 0) when
    xmax == xmin or either step rounds to fp16 zero."""
    maxq = (1 << bits) - 1
    V = np.asarray(V, dtype=F64)
    xmin = np.minimum(V.min(axis=1), 0.0)
    xmax = np.maximum(V.max(axis=1), 0.0)
    step = (xmax - xmin) / maxq
    with np.errstate(over="ignore"):
        s1 = fp16_round(step)
        scale = fp16_round(alpha * step)
    if not (np.all(np.isfinite(s1)) and np.all(np.isfinite(scale))):
        raise NonFinite("group scale overflows fp16")
    degenerate = (xmax == xmin) | (s1 == 0.0) | (scale == 0.0)
    zero = np.clip(np.rint(-xmin / np.where(degenerate, 1.0, s1)), 0, maxq)
    return np.where(degenerate, 1.0, scale), np.where(degenerate, 0.0, zero)


def group_step_hptq(V, bits, alpha):
    """HPTQ step of a group: fp16(alpha * (xmax - xmin)/maxq), 1 when
    degenerate (xmax == xmin or the step rounds to fp16 zero)."""
    maxq = (1 << bits) - 1
    V = np.asarray(V, dtype=F64)
    xmin = np.minimum(V.min(axis=1), 0.0)
    xmax = np.maximum(V.max(axis=1), 0.0)
    with np.errstate(over="ignore"):
        step = fp16_round(alpha * (xmax - xmin) / maxq)
    if not np.all(np.isfinite(step)):
        raise NonFinite("group scale overflows fp16")
    return np.where((xmax == xmin) | (step == 0.0), 1.0, step)


def huffman_lengths(counts):
    """Code length of every symbol of a Huffman code for ``counts`` (dict
    symbol -> count > 0), by repeatedly merging the two lightest subtrees. A
    single symbol gets length 1. Every Huffman code has the same total
    length sum(count * length), the optimum over prefix codes."""
    import heapq
    syms = sorted(counts)
    if len(syms) == 1:
        return {syms[0]: 1}
    length = {s_: 0 for s_ in syms}
    heap = [(counts[s_], i, [s_]) for i, s_ in enumerate(syms)]
    heapq.heapify(heap)
    nxt = len(syms)
    while len(heap) > 1:
        c1, _, a = heapq.heappop(heap)
        c2, _, b = heapq.heappop(heap)
        for s_ in a + b:
            length[s_] += 1
        heapq.heappush(heap, (c1 + c2, nxt, a + b))
        nxt += 1
    return length


def huffman_canonical(lengths):
    """Canonical prefix code for code lengths ``lengths`` (dict symbol ->
    length >= 1): symbols in order of (length, symbol value); the first gets
    code 0, each next one the previous code plus one, shifted left by the
    growth in length. Returns dict symbol -> (code, length)."""
    order = sorted(lengths, key=lambda s_: (lengths[s_], s_))
    codes = {}
    code, prev = 0, lengths[order[0]]
    for i, s_ in enumerate(order):
        ln = lengths[s_]
        if i > 0:
            code = (code + 1) << (ln - prev)
        codes[s_] = (code, ln)
        prev = ln
    return codes


def huffman_encode(levels, lengths):
    """[BABAI] 3 (HPTQ stores the integer levels Huffman-coded): the levels
    [rows x cols] in row-major order as one bit stream of their canonical
    codes, most significant code bit first; bit b of the stream is bit
    31 - b % 32 of 32-bit word b // 32. Returns (words uint32, row_bit int64
    [rows + 1] with the stream position of each row's first code, total
    bits)."""
    lv = np.asarray(levels)
    codes = huffman_canonical(lengths)
    bits = []
    row_bit = [0]
    for r in range(lv.shape[0]):
        for v in lv[r].tolist():
            code, ln = codes[int(v)]
            bits.extend((code >> (ln - 1 - i)) & 1 for i in range(ln))
        row_bit.append(len(bits))
    nw = (len(bits) + 31) // 32
    words = np.zeros(nw, dtype=np.uint64)
    for b, bit in enumerate(bits):
        if bit:
            words[b // 32] |= np.uint64(1) << np.uint64(31 - b % 32)
    return words.astype(np.uint32), np.array(row_bit, dtype=np.int64), len(bits)


def huffman_decode(words, row_bit, rows, cols, lengths):
    """Inverse of huffman_encode: read each row's bits from row_bit[r] and
    match codes bit by bit against the canonical code."""
    codes = huffman_canonical(lengths)
    inv = {(c, ln): s_ for s_, (c, ln) in codes.items()}
    w = np.asarray(words, dtype=np.uint64)
    out = np.zeros((rows, cols), dtype=np.int64)
    for r in range(rows):
        b = int(row_bit[r])
        for j in range(cols):
            code, ln = 0, 0
            while (code, ln) not in inv:
                bit = int((w[b // 32] >> np.uint64(31 - b % 32)) & np.uint64(1))
                code, ln, b = (code << 1) | bit, ln + 1, b + 1
                if ln > 64:
                    raise ValueError("not a code of this prefix code")
            out[r, j] = inv[(code, ln)]
    return out


def hptq_bits_per_weight(levels, n_groups_total):
    """(Huffman-coded bits of all levels + 16 per group step) / weights."""
    levels = np.asarray(levels).ravel()
    vals, cnt = np.unique(levels, return_counts=True)
    ln = huffman_lengths({int(v): int(c) for v, c in zip(vals, cnt)})
    total = sum(int(c) * ln[int(v)] for v, c in zip(vals, cnt))
    return (total + 16.0 * n_groups_total) / levels.size


def _quantize_ssqr(v, scale, zero, maxq):
    """(stored code, dequantized value, outlier mask): the level outside
    [0, maxq] makes an outlier, kept as fp16(v); its stored code is the
    clamped one."""
    code = np.rint(v / scale) + zero
    out = (code < 0) | (code > maxq)
    dq = np.where(out, fp16_round(v), scale * (code - zero))
    return np.clip(code, 0, maxq), dq, out


def _quantize(v, scale, zero, maxq, clip):
    q = np.rint(v / scale) + zero
    if clip:
        q = np.clip(q, 0, maxq)
    return q, scale * (q - zero)


def num_groups(cols, group_size):
    return -(-cols // group_size)


# --------------------------------------------------------------------------
# The column sweep  ([CHMC] Schritt 2 "strict_sequential": one column at a
# time with the full row of the factor; [BABAI] 2.2: the propagation is the
# projection onto the nearest hyperplane)
# --------------------------------------------------------------------------

def gptq_sweep(Wp, U, bits, group_size, *, clip=True, static_grid=None,
               block=None, ssqr_alpha=None, hptq_alpha=None):
    """Sweep the columns of Wp (already in sweep order) with the factor U.

    Strict form (``block=None``): after column j is rounded, its scaled error
    e_j = (w~_j - q_j)/U[j,j] is subtracted from every later column through
    row j of U. Lazy form (``block=B``): within a block of B columns the
    update reaches only the block; the remaining columns receive
    E[:, block] @ U[block, rest] when the block ends — the same sums in
    another order. ``static_grid=(scales, zeros)`` [rows x groups] fixes the
    grid instead of taking it at each group start. ``ssqr_alpha`` runs the
    SSQR rule (grid step times alpha, out-of-grid levels kept as fp16
    outliers) and adds ``outlier`` (bool) and ``outlier_vals`` [rows x cols].
    ``hptq_alpha`` runs the HPTQ grid (step times alpha, unbounded levels
    relative to 0); ``codes`` are then those levels and ``zeros`` are 0.

    Returns dict with codes (sweep order, int64), scales, zeros
    [rows x groups], E [rows x cols], row_loss [rows], deq (dequantized).
    """
    W = np.array(Wp, dtype=F64, copy=True)
    if not np.all(np.isfinite(W)):
        raise NonFinite("weights contain NaN/Inf")
    rows, cols = W.shape
    U = np.asarray(U, dtype=F64)
    assert U.shape == (cols, cols)
    maxq = (1 << bits) - 1
    gs = group_size
    ng = num_groups(cols, gs)
    if block is not None and not (block % gs == 0 or gs % block == 0):
        raise ValueError("lazy blocks need group_size | block or block | group_size")
    codes = np.zeros((rows, cols), dtype=np.int64)
    deq = np.zeros((rows, cols), dtype=F64)
    E = np.zeros((rows, cols), dtype=F64)
    scales = np.zeros((rows, ng), dtype=F64)
    zeros = np.zeros((rows, ng), dtype=F64)
    loss = np.zeros(rows, dtype=F64)
    ssqr = ssqr_alpha is not None
    outl = np.zeros((rows, cols), dtype=bool)
    step = cols if block is None else block
    for j0 in range(0, cols, step):
        j1 = min(j0 + step, cols)
        for j in range(j0, j1):
            g = j // gs
            if j % gs == 0:
                if hptq_alpha is not None:
                    s = group_step_hptq(W[:, j:min(j + gs, cols)], bits, hptq_alpha)
                    z = np.zeros(rows)
                elif ssqr:
                    s, z = group_grid_ssqr(W[:, j:min(j + gs, cols)], bits, ssqr_alpha)
                elif static_grid is None:
                    s, z = group_grid(W[:, j:min(j + gs, cols)], bits)
                else:
                    s = np.asarray(static_grid[0], dtype=F64)[:, g]
                    z = np.asarray(static_grid[1], dtype=F64)[:, g]
                scales[:, g] = s
                zeros[:, g] = z
            if ssqr:
                q, dq, outl[:, j] = _quantize_ssqr(W[:, j], scales[:, g], zeros[:, g], maxq)
            elif hptq_alpha is not None:
                q, dq = _quantize(W[:, j], scales[:, g], zeros[:, g], maxq, False)
            else:
                q, dq = _quantize(W[:, j], scales[:, g], zeros[:, g], maxq, clip)
            codes[:, j] = q.astype(np.int64)
            deq[:, j] = dq
            e = (W[:, j] - dq) / U[j, j]
            E[:, j] = e
            loss += e * e
            W[:, j + 1:j1] -= np.outer(e, U[j, j + 1:j1])
        if j1 < cols:
            W[:, j1:] -= E[:, j0:j1] @ U[j0:j1, j1:]
    res = {"codes": codes, "scales": scales, "zeros": zeros, "E": E,
           "row_loss": loss, "deq": deq}
    if ssqr:
        res["outlier"] = outl
        res["outlier_vals"] = np.where(outl, deq, 0.0)
    return res


def gptq_layer(W_fp16, S, n_tokens, *, bits, group_size, damp=0.01,
               act_order=False, clip=True, block=None, min_pivot=False,
               ssqr_alpha=None, hptq_alpha=None):
    """The whole layer: damping, optional act-order (or min-pivot order), U,
    sweep, un-permute.

    Outputs follow the library's layout: codes [rows x cols] in the original
    column order, scales/zeros [rows x groups] with groups in sweep order,
    g_idx[perm[k]] = k // group_size, perm, U, H (damped, permuted), loss.
    """
    W = np.asarray(W_fp16)
    if W.dtype != np.float16:
        raise TypeError("W must be fp16")
    Wd = W.astype(F64)
    H = damped_hessian(S, n_tokens, damp)
    if not np.all(np.isfinite(H)):
        raise NonFinite("Hessian is not finite")
    cols = H.shape[0]
    if min_pivot:
        perm = min_pivot_order(H)[0]
    elif act_order:
        perm = act_order_perm(H)
    else:
        perm = np.arange(cols, dtype=np.int64)
    Hp = permute_sym(H, perm)
    U = hinv_upper(Hp)
    res = gptq_sweep(Wd[:, perm], U, bits, group_size, clip=clip, block=block,
                     ssqr_alpha=ssqr_alpha, hptq_alpha=hptq_alpha)
    codes = np.empty_like(res["codes"])
    codes[:, perm] = res["codes"]
    if ssqr_alpha is not None:  # outliers back to the original column order
        for key in ("outlier", "outlier_vals"):
            a = np.empty_like(res[key])
            a[:, perm] = res[key]
            res[key] = a
    g_idx = np.empty(cols, dtype=np.int64)
    g_idx[perm] = np.arange(cols) // group_size
    res.update({"codes_sweep": res["codes"], "codes": codes, "g_idx": g_idx,
                "perm": perm, "U": U, "Hp": Hp})
    return res


def ssqr_search(Wp, U, bits, group_size, target, *, iters=12, lo=1.0 / 64, hi=1.0,
                block=None):
    """[BABAI] 3 (SSQR): bisection on the layer's scale factor alpha for the
    smallest alpha whose outlier fraction is at most ``target``. The upper
    end is tried first; if even it exceeds the target it is returned. Each
    probe is a full sweep (outliers depend on the propagated values).
    Returns (alpha, the sweep at alpha, the probes [(alpha, fraction)])."""
    Wp = np.asarray(Wp, dtype=F64)
    n = Wp.size

    def probe(a):
        r = gptq_sweep(Wp, U, bits, group_size, block=block, ssqr_alpha=a)
        return r, float(r["outlier"].sum()) / n

    best, f = probe(hi)
    probes = [(hi, f)]
    if f > target:
        return hi, best, probes
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r, f = probe(mid)
        probes.append((mid, f))
        if f <= target:
            hi, best = mid, r
        else:
            lo = mid
    return hi, best, probes


def ssqr_csr(outlier, outlier_vals):
    """[BABAI] 3 (SSQR keeps its outliers sparse, in floating point): the
    outliers of a sweep as compressed sparse rows, row by row in increasing
    column order. Returns row offsets [rows + 1] (row r's entries are
    row_ptr[r]:row_ptr[r+1]), their columns and their values."""
    m = np.asarray(outlier) != 0
    v = np.asarray(outlier_vals)
    row_ptr = [0]
    cols, vals = [], []
    for r in range(m.shape[0]):
        for c in range(m.shape[1]):
            if m[r, c]:
                cols.append(c)
                vals.append(v[r, c])
        row_ptr.append(len(cols))
    return (np.array(row_ptr, dtype=np.int64), np.array(cols, dtype=np.int64),
            np.array(vals, dtype=v.dtype))


def bpw_ssqr(o, i, bits, group_size, n_outliers):
    """Bits per weight of an SSQR layer stored as b-bit codes, an fp16 scale
    and zero point per (row, group), and its outliers in compressed sparse
    rows (32-bit column and fp16 value per outlier, 64-bit row offsets)."""
    return (bits * o * i + 32 * o * num_groups(i, group_size) + 48 * n_outliers
            + 64 * (o + 1)) / (o * i)


def hptq_search(Wp, U, bits, group_size, budget, *, iters=12, lo=1.0 / 64, hi=1.0,
                block=None):
    """[BABAI] 3 (HPTQ): bisection on the layer's scale factor alpha for the
    smallest alpha whose Huffman-coded bits per weight are at most
    ``budget`` (the same probe order as ssqr_search). Returns (alpha, the
    sweep at alpha with its "bpw", the probes [(alpha, bpw)])."""
    Wp = np.asarray(Wp, dtype=F64)
    rows, cols = Wp.shape
    ngt = rows * num_groups(cols, group_size)

    def probe(a):
        r = gptq_sweep(Wp, U, bits, group_size, block=block, hptq_alpha=a)
        r["bpw"] = hptq_bits_per_weight(r["codes"], ngt)
        return r, r["bpw"]

    best, f = probe(hi)
    probes = [(hi, f)]
    if f > budget:
        return hi, best, probes
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r, f = probe(mid)
        probes.append((mid, f))
        if f <= budget:
            hi, best = mid, r
        else:
            lo = mid
    return hi, best, probes


# --------------------------------------------------------------------------
# CHMC frontend ([CHMC] "Methodik", Schritt 1-3)
# --------------------------------------------------------------------------

# Anhang A of the CHMC article: the CHMC v6 quantization runs with dampening
# 0.05, both for the activation energies (Schritt 1) and for the Hessian of the
# residual's GPTQ step (Schritt 2).
CHMC_DAMP = 0.05


def chmc_energies(S_diag, n_tokens, lam=CHMC_DAMP):
    """Schritt 1: damped activation energies c_j = (1/n) sum_t x_tj^2 +
    lam * mean(c)."""
    c = np.asarray(S_diag, dtype=F64) / n_tokens
    return c + lam * c.mean()


def chmc_bits(o, i, r, bits, group_size):
    """Schritt 3's count of the stored bits of a CHMC layer: fp16 factors
    16 r (o + i), b-bit residual codes, one 16-bit scale per output group and
    column, plus that group's zero point of the asymmetric grid (an integer in
    [0, maxq]: b bits), which the page's formula has no term for."""
    ng = num_groups(o, group_size)
    return 16 * r * (o + i) + bits * o * i + (16 + bits) * ng * i


def chmc_rank(o, i, bits, group_size, bpw_target, max_rank=None):
    """Schritt 3: the largest rank whose layer (chmc_bits) fits the budget,
    floor((BPW o i - b o i - (16 + b) ceil(o/gs) i) / (16 (o + i))), within
    [0, min(o, i)] and at most ``max_rank`` when given (a smaller rank stays
    under the budget, which the page only asks not to exceed)."""
    ng = num_groups(o, group_size)
    r = (bpw_target * o * i - bits * o * i - (16 + bits) * ng * i) // (16 * (o + i))
    r = int(max(0, min(r, min(o, i))))
    return r if max_rank is None else min(r, int(max_rank))


def _orth(Y):
    return np.linalg.qr(Y, mode="reduced")[0]


def randomized_lowrank(A, Omega, niter):
    """Randomized subspace iteration (Halko, Martinsson, Tropp 2011,
    Algorithm 4.4): Q = orth(A Omega), then niter times Q = orth(A orth(A^T
    Q)); B = Q^T A = Ub S Vt (SVD), U = Q Ub. Returns (U, S, Vt)."""
    A = np.asarray(A, dtype=F64)
    Q = _orth(A @ Omega)
    for _ in range(niter):
        Q = _orth(A @ _orth(A.T @ Q))
    Ub, S, Vt = np.linalg.svd(Q.T @ A, full_matrices=False)
    return Q @ Ub, S, Vt


def chmc_lowrank(W, c, Omega, niter=5):
    """Schritt 1: the low-rank part of W in the norm weighted by sqrt(c), as
    fp16 factors A = U S [o x r] and B = V^T diag(1/sqrt c) [r x i]."""
    sc = np.sqrt(np.asarray(c, dtype=F64))
    U, S, Vt = randomized_lowrank(np.asarray(W, dtype=F64) * sc[None, :], Omega, niter)
    return fp16_round(U * S[None, :]), fp16_round(Vt / sc[None, :])


def gptq_sweep_outgroups(Rp, U, bits, row_group):
    """Schritt 2 with the page's grouping: the strict GPTQ sweep of Rp (sweep
    order) where each column gets one grid per group of ``row_group``
    consecutive rows, from the group's current values of that column.
    Returns codes [rows x cols], scales/zeros [groups x cols] (sweep order),
    E, row_loss and deq."""
    R = np.array(Rp, dtype=F64, copy=True)
    rows, cols = R.shape
    U = np.asarray(U, dtype=F64)
    maxq = (1 << bits) - 1
    ng = num_groups(rows, row_group)
    codes = np.zeros((rows, cols), dtype=np.int64)
    deq = np.zeros((rows, cols))
    E = np.zeros((rows, cols))
    scales = np.zeros((ng, cols))
    zeros = np.zeros((ng, cols))
    loss = np.zeros(rows)
    for j in range(cols):
        s_col = np.empty(rows)
        z_col = np.empty(rows)
        for g in range(ng):
            r0, r1 = g * row_group, min((g + 1) * row_group, rows)
            s, z = group_grid(R[r0:r1, j][None, :], bits)
            scales[g, j], zeros[g, j] = s[0], z[0]
            s_col[r0:r1], z_col[r0:r1] = s[0], z[0]
        q, dq = _quantize(R[:, j], s_col, z_col, maxq, True)
        codes[:, j] = q.astype(np.int64)
        deq[:, j] = dq
        e = (R[:, j] - dq) / U[j, j]
        E[:, j] = e
        loss += e * e
        R[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    return {"codes": codes, "scales": scales, "zeros": zeros, "E": E, "row_loss": loss,
            "deq": deq}


def chmc_layer(W_fp16, S, n_tokens, Omega, *, bits=4, group_size=128, bpw_target=4.2875,
               damp=CHMC_DAMP, act_order=True, niter=5, rank=None, max_rank=None):
    """The CHMC layer: energies, rank from the budget (or ``rank``), the
    low-rank fp16 factors from the first r columns of the sketch Omega
    [i x >= r], the residual swept with output-channel groups. Codes and
    scales/zeros come back in the original column order; row_loss is the
    residual sweep's (its H-weighted error)."""
    W = np.asarray(W_fp16)
    if W.dtype != np.float16:
        raise TypeError("W must be fp16")
    Wd = W.astype(F64)
    o, i = Wd.shape
    c = chmc_energies(np.diag(S), n_tokens)
    r = (chmc_rank(o, i, bits, group_size, bpw_target, max_rank) if rank is None
         else int(rank))
    if r > 0:
        A, B = chmc_lowrank(Wd, c, np.asarray(Omega, dtype=F64)[:, :r], niter)
    else:
        A, B = np.zeros((o, 0)), np.zeros((0, i))
    R = Wd - A @ B
    H = damped_hessian(S, n_tokens, damp)
    perm = act_order_perm(H) if act_order else np.arange(i)
    U = hinv_upper(permute_sym(H, perm))
    res = gptq_sweep_outgroups(R[:, perm], U, bits, group_size)
    out = {"A": A, "B": B, "rank": r, "c": c, "R": R, "perm": perm, "U": U,
           "row_loss": res["row_loss"]}
    for key in ("codes", "scales", "zeros", "deq"):
        a = np.empty_like(res[key])
        a[:, perm] = res[key]
        out[key] = a
    return out


def dequantize_sweep(codes_sweep, scales, zeros, group_size):
    """Q[:, j] = scale[:, g] * (code[:, j] - zero[:, g]) with g = j // gs."""
    cols = codes_sweep.shape[1]
    g = np.arange(cols) // group_size
    return scales[:, g] * (codes_sweep.astype(F64) - zeros[:, g])


def loss_quadratic(D, H):
    """Per-row (w-q) H (w-q)^T for residual rows D."""
    return np.einsum("ij,jk,ik->i", D, H, D)


# --------------------------------------------------------------------------
# Special cases and independent algorithms used as pins
# --------------------------------------------------------------------------

def rtn_quantize(W, bits, group_size):
    """Round-to-nearest on the grid of each group of the untouched weights:
    what the sweep must reduce to when H is diagonal (no propagation)."""
    W = np.asarray(W, dtype=F64)
    rows, cols = W.shape
    maxq = (1 << bits) - 1
    ng = num_groups(cols, group_size)
    codes = np.zeros((rows, cols), dtype=np.int64)
    scales = np.zeros((rows, ng))
    zeros = np.zeros((rows, ng))
    for g in range(ng):
        sl = slice(g * group_size, min((g + 1) * group_size, cols))
        s, z = group_grid(W[:, sl], bits)
        scales[:, g], zeros[:, g] = s, z
        q = np.clip(np.rint(W[:, sl] / s[:, None]) + z[:, None], 0, maxq)
        codes[:, sl] = q.astype(np.int64)
    return codes, scales, zeros


def babai_nearest_plane(A, w, s, z, maxq, clip=True):
    """Babai's nearest-plane algorithm ([BABAI] 2.1-2.2) for one row.

    Lattice basis: columns of A @ diag(s) (A any factor with A^T A = H,
    Satz 1), shifted by the zero points z; target A @ w. The basis is taken
    in reverse sweep order and processed from its last vector to its first
    (textbook Babai on the QR factor), which is GPTQ's front-to-back order
    (Satz 4). Returns integer codes in sweep order.
    """
    A = np.asarray(A, dtype=F64)
    c = A.shape[1]
    B = (A * s[None, :])[:, ::-1]
    y = A @ (w + s * z)
    Q, R = np.linalg.qr(B)
    yt = Q.T @ y
    cr = np.zeros(c)
    for k in range(c - 1, -1, -1):
        t = (yt[k] - R[k, k + 1:] @ cr[k + 1:]) / R[k, k]
        v = np.rint(t)
        if clip:
            v = min(max(v, 0.0), float(maxq))
        cr[k] = v
    return cr[::-1].astype(np.int64)


def brute_force_cvp(H, w, s, z, maxq):
    """Exact minimiser of (w-q) H (w-q)^T over all codes in [0,maxq]^d
    (the closest-vector problem of [BABAI] 2.1), by enumeration; d small."""
    d = len(w)
    grid = np.array(list(itertools.product(range(maxq + 1), repeat=d)), dtype=F64)
    Dm = w[None, :] - s[None, :] * (grid - z[None, :])
    losses = np.einsum("ij,jk,ik->i", Dm, H, Dm)
    k = int(np.argmin(losses))
    return grid[k].astype(np.int64), float(losses[k])


def ldl_diag(M):
    """Diagonal D of the LDL^T factorisation M = L D L^T (L unit lower),
    plain Doolittle recursion without pivoting."""
    M = np.asarray(M, dtype=F64)
    n = M.shape[0]
    L = np.eye(n)
    D = np.zeros(n)
    for j in range(n):
        D[j] = M[j, j] - np.sum(L[j, :j] ** 2 * D[:j])
        if D[j] <= 0:
            raise NotSPD("non-positive pivot in LDL")
        for i in range(j + 1, n):
            L[i, j] = (M[i, j] - np.sum(L[i, :j] * L[j, :j] * D[:j])) / D[j]
    return D


def noclip_bound(s_cols, U):
    """Satz 5 ([BABAI] 2.3): without clipping |w~_j - q_j| <= s_j/2, so a
    row's loss is at most (1/4) sum_j s_j^2 D_j, where D_j = 1/U[j,j]^2 is
    the LDL pivot of the Hessian taken in reverse sweep order."""
    d = np.diag(np.asarray(U, dtype=F64))
    return 0.25 * np.sum(np.asarray(s_cols, dtype=F64) ** 2 / d ** 2, axis=-1)


# --------------------------------------------------------------------------
# Bit accounting  ([CHMC] Schritt 3)
# --------------------------------------------------------------------------

def bpw_page(o, i, bits, group_size):
    """The page's GPTQ formula: [b*o*i + 16*o*ceil(i/gs)] / (o*i)."""
    return (bits * o * i + 16 * o * num_groups(i, group_size)) / (o * i)


def bpw_gptq(o, i, bits, group_size):
    """Bits per weight of this library's output: b-bit codes plus an fp16
    scale and an fp16 zero point per (row, group)."""
    return (bits * o * i + 32 * o * num_groups(i, group_size)) / (o * i)
