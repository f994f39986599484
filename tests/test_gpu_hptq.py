"""GPU: HPTQ (The Geometry of LLM Quantization, section 3) against the oracle.

Through the C ABI: the full path (Hessian, prepare, the no-clipping sweep on
the HPTQ grid) at fixed scale factors, with and without act-order; the
unbounded levels element by element; the bits per weight against the
oracle's Huffman code of the same levels; the bisection search against the
oracle's; the Qwen down projection's full shape at the alpha the search
picks.
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


def problem(rows, cols, n, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, cols)) + 0.8 * rng.standard_normal((n, 1))).astype(np.float32)
    W = (0.02 * rng.standard_t(4, size=(rows, cols))).astype(np.float16)
    return W, X


def gpu_factor(X, act_order):
    dim = X.shape[1]
    S = torch.zeros((dim, dim), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
    perm, U = G.prepare_hinv(S, X.shape[0], damp=0.01, act_order=act_order)
    return perm if act_order else None, U


def compare_hptq(res, ref, gs, name):
    lv = res.levels.cpu().numpy().astype(np.int64)
    rows, cols = lv.shape
    agree = float(np.mean(lv == ref["codes"]))
    sc = res.scales.cpu().numpy().astype(np.float64)
    s_ok = float(np.mean(np.abs(sc - ref["scales"]) <= SCALE_RTOL * np.abs(ref["scales"])))
    lg, lr = float(res.row_loss.sum().item()), float(ref["row_loss"].sum())
    ngt = rows * O.num_groups(cols, gs)
    own = O.hptq_bits_per_weight(lv, ngt)
    refb = O.hptq_bits_per_weight(ref["codes"], ngt)
    say(f"{name}: levels {agree:.6f} scales {s_ok:.6f} loss_rel {abs(lg - lr) / lr:.2e} "
        f"bpw gpu {res.bpw:.6f} oracle {refb:.6f} range [{lv.min()}, {lv.max()}]")
    assert agree >= CODE_AGREE and s_ok >= SCALE_AGREE
    assert abs(lg - lr) <= LOSS_RTOL * lr
    assert res.bpw == own  # the device histogram and host Huffman total
    assert abs(res.bpw - refb) <= 1e-3 * refb
    assert np.array_equal(res.g_idx.cpu().numpy().astype(np.int64), ref["g_idx"])


@pytest.mark.parametrize("rows,cols,bits,gs,act,alpha", [
    (64, 576, 4, 128, False, 0.8),
    (37, 333, 3, 32, True, 1.5),
    (130, 260, 2, 64, True, 0.4),
    (1, 129, 4, 128, True, 2.0),
])
def test_hptq_fixed_alpha_matches_oracle(rows, cols, bits, gs, act, alpha):
    say(f"hptq {rows}x{cols} b{bits} g{gs} act={act} alpha={alpha}")
    W, X = problem(rows, cols, 2 * cols + 11, rows * 17 + cols)
    perm, U = gpu_factor(X, act)
    res = G.quantize_layer_hptq(torch.from_numpy(W).to(DEV), U, perm, bits=bits, group_size=gs,
                                alpha=alpha)
    Sr, n = O.hessian_sum(X)
    ref = O.gptq_layer(W, Sr, n, bits=bits, group_size=gs, act_order=act, block=128,
                       hptq_alpha=alpha)
    if act:
        assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    compare_hptq(res, ref, gs, f"hptq {rows}x{cols}")


def test_hptq_search_matches_oracle():
    say("hptq search 96x384, budget 3.25 bits")
    W, X = problem(96, 384, 900, 23)
    perm, U = gpu_factor(X, True)
    res = G.hptq_search(torch.from_numpy(W).to(DEV), U, perm, bits=4, group_size=64,
                        budget=3.25, iters=10, alpha_lo=0.25, alpha_hi=4.0)
    Sr, n = O.hessian_sum(X)
    H = O.damped_hessian(Sr, n, 0.01)
    pr = O.act_order_perm(H)
    Ur = O.hinv_upper(O.permute_sym(H, pr))
    alpha, best, probes = O.hptq_search(W.astype(np.float64)[:, pr], Ur, 4, 64, 3.25,
                                        iters=10, lo=0.25, hi=4.0, block=128)
    say(f"gpu alpha {res.alpha} bpw {res.bpw}, oracle alpha {alpha} bpw {best['bpw']}; "
        f"probes {probes}")
    assert res.bpw <= 3.25
    assert res.alpha == alpha
    ref = O.gptq_layer(W, Sr, n, bits=4, group_size=64, act_order=True, block=128,
                       hptq_alpha=res.alpha)
    compare_hptq(res, ref, 64, "hptq search result")


def test_hptq_qwen_down_projection_full_shape():
    """896 x 4864 (the Qwen2.5-0.5B down projection): the GPU search for 3.125
    bits per weight, then the oracle's lazy sweep at that alpha."""
    say("hptq qwen down 896x4864, budget 3.125")
    rows, dim, n = 896, 4864, 2048
    X = synth.activations(1, "down_in", n, dim, kind="silu_gated")
    W = synth.weights(1, "down_proj", rows, dim)
    perm, U = gpu_factor(X, False)
    res = G.hptq_search(torch.from_numpy(W).to(DEV), U, None, bits=4, group_size=128,
                        budget=3.125, iters=8)
    say(f"alpha {res.alpha}, bpw {res.bpw}")
    assert res.bpw <= 3.125
    Sr, nr = O.hessian_sum(X)
    ref = O.gptq_layer(W, Sr, nr, bits=4, group_size=128, block=128, hptq_alpha=res.alpha)
    compare_hptq(res, ref, 128, "hptq qwen down")


def _check_stream(lv_dev, name, bit_exact=True):
    """gptq_hptq_encode / gptq_hptq_decode on a level matrix: the code
    lengths are a Huffman code of its histogram (the oracle's, same tie
    rule), the stream equals the oracle's canonical encoding bit for bit,
    and decoding gives the levels back."""
    lv = lv_dev.cpu().numpy().astype(np.int64)
    s = G.hptq_encode(lv_dev)
    vals, cnt = np.unique(lv, return_counts=True)
    ref_len = O.huffman_lengths({int(v): int(c) for v, c in zip(vals, cnt)})
    lib_len = {int(v): int(s.code_len[int(v) + 32768]) for v in vals}
    assert int(np.count_nonzero(s.code_len)) == len(vals)
    assert lib_len == ref_len
    total = sum(int(c) * ref_len[int(v)] for v, c in zip(vals, cnt))
    say(f"{name}: {len(vals)} distinct levels, {total} bits ({total / lv.size:.4f} per level)")
    assert s.total_bits == total
    if bit_exact:
        words, row_bit, tb = O.huffman_encode(lv, lib_len)
        assert tb == total
        assert np.array_equal(s.row_bit.cpu().numpy(), row_bit)
        assert np.array_equal(s.words.cpu().numpy().view(np.uint32), words)
    back = G.hptq_decode(s)
    assert torch.equal(back, lv_dev)


def test_hptq_code_stream_matches_oracle_and_round_trips():
    say("hptq code stream 150x333")
    W, X = problem(150, 333, 800, 91)
    perm, U = gpu_factor(X, True)
    res = G.quantize_layer_hptq(torch.from_numpy(W).to(DEV), U, perm, bits=3, group_size=32,
                                alpha=0.8)
    _check_stream(res.levels, "hptq 150x333")


@pytest.mark.parametrize("shape,spread", [((1, 1), 0), ((3, 70), 0), ((40, 129), 3),
                                          ((1500, 64), 40), ((7, 100), 3000)])
def test_hptq_code_stream_edge_cases(shape, spread):
    """One level only (1 bit each), a single row, ragged widths, more than
    1024 rows (several scan rounds), levels beyond the LDS histogram range."""
    say(f"hptq code stream {shape} spread {spread}")
    rng = np.random.default_rng(shape[0] * 31 + spread)
    lv = np.rint(rng.standard_normal(shape) * spread).astype(np.int16)
    _check_stream(torch.from_numpy(lv).to(DEV), f"stream {shape}")


def test_hptq_code_stream_full_shape_round_trip():
    """The 896 x 4864 down projection at the search's alpha: the stream size
    is the Huffman part of the bits per weight, and it decodes to the levels."""
    say("hptq code stream 896x4864")
    rows, dim, n = 896, 4864, 2048
    X = synth.activations(1, "down_in", n, dim, kind="silu_gated")
    W = synth.weights(1, "down_proj", rows, dim)
    perm, U = gpu_factor(X, False)
    res = G.hptq_search(torch.from_numpy(W).to(DEV), U, None, bits=4, group_size=128,
                        budget=3.125, iters=6)
    _check_stream(res.levels, "hptq 896x4864", bit_exact=False)
    s = G.hptq_encode(res.levels)
    ngt = rows * O.num_groups(dim, 128)
    assert abs((s.total_bits + 16.0 * ngt) / (rows * dim) - res.bpw) <= 1e-12
