"""GPU: gptq_quantize_layer_noalloc (scratch from the library's fixed device
array, no workspace argument) against gptq_quantize_layer with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
layer, each bit for bit equal to the existing entry point's results; a layer
too large for the array is rejected before anything is enqueued."""
import ctypes as C
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP device", allow_module_level=True)

import post_weight_quantization_hessian_amd.gptq as G  # noqa: E402

DEV = torch.device("cuda:0")
P = C.c_void_p


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def noalloc(W, U, perm, bits, gs, out, flags=0):
    f = G.lib.gptq_quantize_layer_noalloc
    rows, cols = W.shape
    return f(G._ptr(W), rows, cols, W.stride(0), G._ptr(U), G._ptr(perm), bits, gs, flags,
             G._ptr(out.codes), G._ptr(out.scales), G._ptr(out.zeros), G._ptr(out.g_idx),
             G._ptr(out.row_loss), G._stream())


def outputs(rows, cols, gs, bits):
    ng = -(-cols // gs)
    return G.QuantizedLayer(torch.full((rows, cols), 255, dtype=torch.uint8, device=DEV),
                            torch.zeros((rows, ng), dtype=torch.float16, device=DEV),
                            torch.zeros((rows, ng), dtype=torch.float16, device=DEV),
                            torch.full((cols,), -1, dtype=torch.int32, device=DEV),
                            torch.zeros(rows, dtype=torch.float64, device=DEV), bits, gs)


def factor(cols, n, seed, act):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, cols)) * np.exp(0.4 * rng.standard_normal(cols))[None, :]
         + 0.7 * rng.standard_normal((n, 1))).astype(np.float32)
    S = torch.zeros((cols, cols), dtype=torch.float64, device=DEV)
    G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
    perm, U = G.prepare_hinv(S, n, damp=0.01, act_order=act)
    return (perm if act else None), U


def weights(rows, cols, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((0.02 * rng.standard_t(4, size=(rows, cols))).astype(np.float16)).to(DEV)


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(512, 1536, 4, 128, True, 11), (200, 576, 3, 64, False, 12)]
    for rows, cols, bits, gs, act, seed in cases:  # the second is smaller
        say(f"noalloc {rows}x{cols} b{bits} g{gs} act={act}")
        assert G.quantize_workspace_bytes(rows, cols, gs) <= 64 << 20
        perm, U = factor(cols, 2 * cols + 5, seed, act)
        W = weights(rows, cols, seed + 100)
        ref = G.quantize_layer(W, U, perm, bits=bits, group_size=gs)
        out = outputs(rows, cols, gs, bits)
        st = noalloc(W, U, perm, bits, gs, out)
        assert st == G.GPTQ_OK, G.lib.gptq_status_string(st)
        torch.cuda.synchronize()
        for x, y in ((out.codes, ref.codes), (out.scales, ref.scales), (out.zeros, ref.zeros),
                     (out.g_idx, ref.g_idx), (out.row_loss, ref.row_loss)):
            assert torch.equal(x, y)
    # asynchronous: the status is the one of the array's status word
    rows, cols, bits, gs = 96, 384, 2, 32
    perm, U = factor(cols, 900, 13, True)
    W = weights(rows, cols, 113)
    ref = G.quantize_layer(W, U, perm, bits=bits, group_size=gs)
    out = outputs(rows, cols, gs, bits)
    assert noalloc(W, U, perm, bits, gs, out, flags=G.GPTQ_FLAG_NO_SYNC) == G.GPTQ_OK
    torch.cuda.synchronize()
    assert torch.equal(out.codes, ref.codes) and torch.equal(out.row_loss, ref.row_loss)


def test_noalloc_rejects_a_layer_beyond_its_array():
    say("noalloc: a layer too large for the 64 MiB array")
    f = G.lib.gptq_quantize_layer_noalloc
    rows, cols = 9728, 896
    assert G.quantize_workspace_bytes(rows, cols, 128) > 64 << 20
    fake = P(0x10000)  # never dereferenced: rejected before any launch
    st = f(fake, rows, cols, cols, fake, None, 4, 128, 0, fake, fake, fake, fake, fake,
           G._stream())
    assert st == G.GPTQ_EWORKSPACE


def test_noalloc_factor_form_matches_workspace_entry_point():
    """The flags pass through: the factor form (the matrix of prepare_hinv
    with that flag) gives the workspace entry point's results bit for bit,
    on two calls in a row, the second smaller."""
    for rows, cols, bits, gs, seed in [(256, 1024, 4, 128, 21), (64, 300, 3, 32, 22)]:
        say(f"noalloc factor form {rows}x{cols} b{bits} g{gs}")
        rng = np.random.default_rng(seed)
        n = 2 * cols + 7
        X = (rng.standard_normal((n, cols)) + 0.7 * rng.standard_normal((n, 1))).astype(np.float32)
        S = torch.zeros((cols, cols), dtype=torch.float64, device=DEV)
        G.hessian_accumulate(S, torch.from_numpy(X).to(DEV), overwrite=True)
        perm, M = G.prepare_hinv(S, n, damp=0.01, act_order=True, factor_form=True)
        W = weights(rows, cols, seed + 100)
        ref = G.quantize_layer(W, M, perm, bits=bits, group_size=gs, factor_form=True)
        out = outputs(rows, cols, gs, bits)
        st = noalloc(W, M, perm, bits, gs, out, flags=G.GPTQ_FLAG_FACTOR_FORM)
        assert st == G.GPTQ_OK, G.lib.gptq_status_string(st)
        torch.cuda.synchronize()
        for x, y in ((out.codes, ref.codes), (out.scales, ref.scales), (out.zeros, ref.zeros),
                     (out.g_idx, ref.g_idx), (out.row_loss, ref.row_loss)):
            assert torch.equal(x, y)
