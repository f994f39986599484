"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/gptq.h, validates arguments before
touching the device, and its fp16 rounding routine is the nearest-even one."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")

g = pytest.importorskip("post_weight_quantization_hessian_amd.gptq")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(g.lib, n), n
        assert n in g.EXPORTS, n


def test_status_strings_and_version():
    assert g.lib.gptq_version() == 1
    for s in range(6):
        assert g.lib.gptq_status_string(s)
    assert g.lib.gptq_status_string(99) == b"unknown status"


def test_fp16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        # exact ties between neighbouring fp16 values (binary64 midpoints)
        (np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (1024 + np.arange(0, 1023) + 0.5) * 2.0 ** -10,
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2 ** -25, 2 ** -24, 6e-8],
    ])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(g.fp16_round_host(v), want)


def test_workspace_sizes():
    assert g.quantize_workspace_bytes(0, 10, 128) == 0
    assert g.quantize_workspace_bytes(10, 10, 100) == 0  # bad group size
    q = g.quantize_workspace_bytes(896, 4864, 128)
    assert q >= 896 * 4864 * (2 + 1 + 4)
    p = g.prepare_workspace_bytes(576)
    assert p >= 2 * 640 * 640 * 8
    assert g.hessian_workspace_bytes(576, 2048) > 0
    assert g.hessian_workspace_bytes(28672, 65536) == 0  # enough tiles, no split
    # split8: column maxima and exponents, four int8 digit planes padded to
    # 128 features x 64 tokens, and partial tiles only when split
    assert g.hessian_split8_workspace_bytes(0, 2048) == 0
    assert g.hessian_split8_workspace_bytes(64, 0) == 0
    s = g.hessian_split8_workspace_bytes(4864, 2048)  # 741 tiles: no token split
    assert 4 * 4864 * 2048 <= s <= 4 * 4864 * 2048 + 2 * 256 + 8 * 4992 + 4 * 4992 * 2048
    assert s == g.hessian_split8_workspace_bytes(4864, 2048)
    # more than 16384 tokens per call always splits, so partial tiles appear
    big = g.hessian_split8_workspace_bytes(1024, 40000)
    assert big > 4 * 1024 * 40000 + 3 * 36 * 128 * 128 * 8 - 1


FAKE = C.c_void_p(0x10000)  # never dereferenced: validation fails first
NULL = C.c_void_p(0)


def test_invalid_arguments_rejected_on_host():
    L = g.lib
    # quantize: bits / group size / null outputs / ld / workspace
    args = lambda **kw: dict(dict(W=FAKE, rows=4, cols=8, ldw=8, U=FAKE, perm=NULL, bits=4, gs=16,
                                  codes=FAKE, scales=FAKE, zeros=FAKE, g_idx=NULL, loss=FAKE,
                                  ws=FAKE, wsb=1 << 40), **kw)

    def q(**kw):
        a = args(**kw)
        return L.gptq_quantize_layer(a["W"], a["rows"], a["cols"], a["ldw"], a["U"], a["perm"],
                                     a["bits"], a["gs"], a.get("flags", 0), a["codes"], a["scales"],
                                     a["zeros"], a["g_idx"], a["loss"], a["ws"], a["wsb"], NULL)
    assert q(bits=1) == g.GPTQ_EINVAL
    assert q(bits=9) == g.GPTQ_EINVAL
    assert q(gs=48) == g.GPTQ_EINVAL
    assert q(gs=0) == g.GPTQ_EINVAL
    assert q(codes=NULL) == g.GPTQ_EINVAL
    assert q(W=NULL) == g.GPTQ_EINVAL
    assert q(ldw=7) == g.GPTQ_EINVAL
    assert q(rows=-1) == g.GPTQ_EINVAL
    assert q(ws=NULL) == g.GPTQ_EWORKSPACE
    assert q(wsb=16) == g.GPTQ_EWORKSPACE
    assert q(flags=8) == g.GPTQ_EINVAL
    assert q(flags=128) == g.GPTQ_EINVAL
    # the factor form is a flag of the plain sweep (its size checks still apply)
    assert q(flags=g.GPTQ_FLAG_FACTOR_FORM, ws=NULL) == g.GPTQ_EWORKSPACE
    assert q(flags=g.GPTQ_FLAG_FACTOR_FORM, bits=1) == g.GPTQ_EINVAL
    assert q(rows=0) == g.GPTQ_OK and q(cols=0) == g.GPTQ_OK  # empty: no-op
    assert L.gptq_workspace_status(NULL, NULL) == g.GPTQ_EINVAL
    # prepare
    pw = L.gptq_prepare_hinv
    assert pw(NULL, 8, 10, 0.01, 0, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 0, 0.01, 0, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, -0.1, 0, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, float("nan"), 0, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, 0.01, 16, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    # act-order and min-pivot are exclusive
    assert pw(FAKE, 8, 10, 0.01, 9, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, 0.01, 2, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, 0.01, 0, FAKE, FAKE, FAKE, 64, NULL) == g.GPTQ_EWORKSPACE
    ff = g.GPTQ_FLAG_FACTOR_FORM
    assert pw(FAKE, 8, 10, 0.01, ff, FAKE, FAKE, FAKE, 64, NULL) == g.GPTQ_EWORKSPACE
    assert pw(FAKE, 8, 10, 0.01, ff | 128, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 8, 10, 0.01, ff | 9, FAKE, FAKE, FAKE, 1 << 40, NULL) == g.GPTQ_EINVAL
    assert pw(FAKE, 0, 10, 0.01, 0, NULL, NULL, NULL, 0, NULL) == g.GPTQ_OK
    # hessian
    ha = L.gptq_hessian_accumulate
    assert ha(NULL, 8, FAKE, 10, 8, 0, NULL, 0, NULL) == g.GPTQ_EINVAL
    assert ha(FAKE, 8, FAKE, 10, 7, 0, NULL, 0, NULL) == g.GPTQ_EINVAL
    assert ha(FAKE, 8, NULL, 0, 8, 0, NULL, 0, NULL) == g.GPTQ_OK  # no tokens: no-op
    assert ha(FAKE, -1, FAKE, 10, 8, 0, NULL, 0, NULL) == g.GPTQ_EINVAL
    assert ha(FAKE, 8, FAKE, 10, 8, 4, NULL, 0, NULL) == g.GPTQ_EINVAL  # unknown flag
    assert ha(NULL, 8, FAKE, 0, 8, 2, NULL, 0, NULL) == g.GPTQ_EINVAL  # overwrite needs S
    assert ha(FAKE, 8, FAKE, 10, 8, 64, NULL, 0, NULL) == g.GPTQ_EINVAL  # unknown flag
    # split8 needs its workspace (checked before any launch)
    assert ha(FAKE, 8, FAKE, 10, 8, 32, NULL, 0, NULL) == g.GPTQ_EWORKSPACE
    need = g.hessian_split8_workspace_bytes(8, 10)
    assert ha(FAKE, 8, FAKE, 10, 8, 32, FAKE, need - 1, NULL) == g.GPTQ_EWORKSPACE
    assert ha(FAKE, 8, FAKE, 10, 7, 32, FAKE, need, NULL) == g.GPTQ_EINVAL  # ldx < i


def test_ssqr_arguments_rejected_on_host():
    L = g.lib
    C_ = C
    n = C_.c_uint64(0)
    a = C_.c_double(0.0)
    q = L.gptq_quantize_layer_ssqr

    def qs(alpha=0.5, flags=0, mask=FAKE, cnt=None, ws=FAKE, wsb=1 << 40):
        return q(FAKE, 4, 8, 8, FAKE, NULL, 4, 16, flags, alpha, FAKE, FAKE, FAKE, NULL, FAKE,
                 mask, FAKE, C_.byref(n) if cnt is None else cnt, ws, wsb, NULL)
    assert qs(alpha=0.0) == g.GPTQ_EINVAL
    assert qs(alpha=17.0) == g.GPTQ_EINVAL
    assert qs(alpha=float("nan")) == g.GPTQ_EINVAL
    assert qs(flags=g.GPTQ_FLAG_NO_CLIP) == g.GPTQ_EINVAL  # its own rule replaces clipping
    assert qs(flags=g.GPTQ_FLAG_FACTOR_FORM) == g.GPTQ_EINVAL  # U itself only
    assert qs(flags=g.GPTQ_FLAG_NO_SYNC) == g.GPTQ_EINVAL  # a count needs a synchronize
    assert qs(mask=NULL) == g.GPTQ_EINVAL
    assert qs(ws=NULL, wsb=0) == g.GPTQ_EWORKSPACE
    s = L.gptq_ssqr_search

    def ss(target=0.01, iters=8, lo=0.1, hi=1.0, flags=0, aout=None):
        return s(FAKE, 4, 8, 8, FAKE, NULL, 4, 16, flags, target, iters, lo, hi,
                 C_.byref(a) if aout is None else aout, FAKE, FAKE, FAKE, NULL, FAKE, FAKE,
                 FAKE, C_.byref(n), FAKE, 1 << 40, NULL)
    assert ss(target=-0.1) == g.GPTQ_EINVAL
    assert ss(target=1.5) == g.GPTQ_EINVAL
    assert ss(iters=61) == g.GPTQ_EINVAL
    assert ss(lo=0.0) == g.GPTQ_EINVAL
    assert ss(lo=1.0, hi=0.5) == g.GPTQ_EINVAL
    assert ss(hi=17.0) == g.GPTQ_EINVAL
    assert ss(flags=g.GPTQ_FLAG_NO_SYNC) == g.GPTQ_EINVAL
    assert ss(aout=NULL) == g.GPTQ_EINVAL


def test_hptq_arguments_rejected_on_host():
    L = g.lib
    b = C.c_double(0.0)
    a = C.c_double(0.0)
    q = L.gptq_quantize_layer_hptq

    def qh(alpha=0.5, flags=0, lv=FAKE, bp=None, ws=FAKE, wsb=1 << 40):
        return q(FAKE, 4, 8, 8, FAKE, NULL, 4, 16, flags, alpha, lv, FAKE, FAKE, NULL, FAKE,
                 C.byref(b) if bp is None else bp, ws, wsb, NULL)
    assert qh(alpha=0.0) == g.GPTQ_EINVAL
    assert qh(alpha=16.5) == g.GPTQ_EINVAL
    assert qh(flags=g.GPTQ_FLAG_NO_CLIP) == g.GPTQ_EINVAL
    assert qh(flags=g.GPTQ_FLAG_NO_SYNC) == g.GPTQ_EINVAL  # bits per weight need a sync
    assert qh(lv=NULL) == g.GPTQ_EINVAL
    assert qh(ws=NULL, wsb=0) == g.GPTQ_EWORKSPACE
    s = L.gptq_hptq_search

    def hs(budget=3.0, iters=8, lo=0.1, hi=1.0, flags=0, aout=None):
        return s(FAKE, 4, 8, 8, FAKE, NULL, 4, 16, flags, budget, iters, lo, hi,
                 C.byref(a) if aout is None else aout, FAKE, FAKE, FAKE, NULL, FAKE,
                 C.byref(b), FAKE, 1 << 40, NULL)
    assert hs(budget=0.0) == g.GPTQ_EINVAL
    assert hs(iters=-1) == g.GPTQ_EINVAL
    assert hs(lo=0.5, hi=0.5) == g.GPTQ_EINVAL
    assert hs(flags=1) == g.GPTQ_EINVAL
    assert hs(aout=NULL) == g.GPTQ_EINVAL


def test_chmc_host_checks():
    """Rank formula against the oracle's, workspace sizes and the argument
    checks of gptq_chmc_layer (rejected before anything is enqueued)."""
    import oracle as O
    L = g.lib
    for shape in [(576, 576), (896, 4864), (4864, 896), (37, 129), (1, 1), (8192, 28672)]:
        for bits, gs, bpw in [(4, 128, 4.2875), (3, 64, 3.5), (2, 32, 8.0), (4, 128, 4.0)]:
            assert g.chmc_rank(*shape, bits, gs, bpw) == O.chmc_rank(*shape, bits, gs, bpw,
                                                                       max_rank=64)
    assert g.chmc_rank(576, 576, 4, 128, 4.2875) == 2
    # every layer shape and bit width of the workloads at the page's budget:
    # the rank fits the layer call's limit (64) and its workspace query
    from post_weight_quantization_hessian_amd.workloads import WORKLOADS
    for wl in WORKLOADS.values():
        for lay in wl.layers:
            cols = wl.input(lay.hessian).dim
            for bits in wl.bits:
                r = g.chmc_rank(lay.rows, cols, bits, wl.group_size, 4.2875)
                assert 0 <= r <= 64
                assert r == min(64, O.chmc_rank(lay.rows, cols, bits, wl.group_size, 4.2875))
                if r > 0:  # (at 4 bits and 64-row groups even rank 0 is over)
                    assert O.chmc_bits(lay.rows, cols, r, bits, wl.group_size) <= \
                        4.2875 * lay.rows * cols
                if lay.rows * cols <= 1 << 24:
                    assert g.chmc_workspace_bytes(lay.rows, cols, r) > 0
    assert g.chmc_workspace_bytes(576, 576, 2) >= 3 * 8 * 576 * 576
    assert g.chmc_workspace_bytes(576, 576, 65) == 0
    assert g.chmc_workspace_bytes(37, 129, 0) >= 3 * 8 * 37 * 129  # no low-rank part
    assert g.chmc_workspace_bytes(0, 576, 2) == 0
    f = L.gptq_chmc_layer

    def ch(rows=64, cols=128, ldw=128, n=100, perm=NULL, om=FAKE, rank=2, bits=4, gs=64,
           flags=0, A=FAKE, B=FAKE, ws=FAKE, wsb=1 << 40):
        return f(FAKE, rows, cols, ldw, FAKE, n, FAKE, perm, om, rank, bits, gs, flags, A, B,
                 FAKE, FAKE, FAKE, FAKE, ws, wsb, NULL, NULL)
    assert ch(rank=65) == g.GPTQ_EINVAL
    assert ch(rank=-1) == g.GPTQ_EINVAL
    assert ch(rows=1, rank=2) == g.GPTQ_EINVAL
    assert ch(bits=1) == g.GPTQ_EINVAL
    assert ch(gs=100) == g.GPTQ_EINVAL
    assert ch(n=0) == g.GPTQ_EINVAL
    assert ch(ldw=127) == g.GPTQ_EINVAL
    assert ch(flags=1) == g.GPTQ_EINVAL
    assert ch(flags=g.GPTQ_FLAG_FACTOR_FORM | 1) == g.GPTQ_EINVAL
    # the factor form passes the flag check (the workspace check comes next)
    assert ch(flags=g.GPTQ_FLAG_FACTOR_FORM, ws=NULL) == g.GPTQ_EWORKSPACE
    assert ch(om=NULL) == g.GPTQ_EINVAL
    assert ch(A=NULL) == g.GPTQ_EINVAL
    assert ch(ws=NULL, wsb=0) == g.GPTQ_EWORKSPACE
    assert ch(wsb=g.chmc_workspace_bytes(64, 128, 2) - 1) == g.GPTQ_EWORKSPACE


def test_profile_api_without_launches():
    g.profile_enable(True)
    r = g.profile_read()
    g.profile_enable(False)
    assert "quant_sweep" in r and "hessian_tile" in r
    assert all(v == (0.0, 0) for v in r.values())


def test_ssqr_csr_host_checks():
    """gptq_ssqr_outliers_csr rejects bad arguments before any launch."""
    f = g.lib.gptq_ssqr_outliers_csr
    n = C.c_int64(0)

    def call(mask=FAKE, vals=FAKE, rows=4, cols=8, rp=FAKE, ci=FAKE, cv=FAKE, cap=3, flags=0,
             nnz=None):
        return f(mask, vals, rows, cols, rp, ci, cv, cap, flags, nnz, NULL)
    assert call(rp=NULL) == g.GPTQ_EINVAL
    assert call(rows=-1) == g.GPTQ_EINVAL
    assert call(cols=-1) == g.GPTQ_EINVAL
    assert call(cap=-1) == g.GPTQ_EINVAL
    assert call(cols=1 << 31) == g.GPTQ_EINVAL
    assert call(mask=NULL) == g.GPTQ_EINVAL
    assert call(vals=NULL) == g.GPTQ_EINVAL
    assert call(ci=NULL) == g.GPTQ_EINVAL
    assert call(cv=NULL) == g.GPTQ_EINVAL
    assert call(flags=1) == g.GPTQ_EINVAL
    assert call(flags=g.GPTQ_FLAG_NO_SYNC, nnz=C.byref(n)) == g.GPTQ_EINVAL


def test_noalloc_host_checks():
    """gptq_quantize_layer_noalloc: the argument checks of gptq_quantize_layer,
    then a layer whose workspace exceeds the 64 MiB array is rejected, all
    before any HIP call."""
    f = g.lib.gptq_quantize_layer_noalloc

    def call(rows=4, cols=8, ldw=8, bits=4, gs=16, flags=0, W=FAKE, U=FAKE, codes=FAKE):
        return f(W, rows, cols, ldw, U, NULL, bits, gs, flags, codes, FAKE, FAKE, NULL, FAKE,
                 NULL)
    assert call(bits=1) == g.GPTQ_EINVAL
    assert call(gs=100) == g.GPTQ_EINVAL
    assert call(ldw=7) == g.GPTQ_EINVAL
    assert call(W=NULL) == g.GPTQ_EINVAL
    assert call(codes=NULL) == g.GPTQ_EINVAL
    assert call(flags=1) == g.GPTQ_EINVAL
    assert call(rows=0) == g.GPTQ_OK  # an empty layer: nothing to do
    assert g.quantize_workspace_bytes(9728, 896, 128) > 64 << 20
    assert call(rows=9728, cols=896, ldw=896, gs=128) == g.GPTQ_EWORKSPACE
    assert g.quantize_workspace_bytes(4096, 14336, 128) > 64 << 20
    assert call(rows=4096, cols=14336, ldw=14336, gs=128) == g.GPTQ_EWORKSPACE


def test_hptq_code_host_checks():
    """gptq_hptq_encode / gptq_hptq_decode reject bad calls before any launch."""
    enc, dec = g.lib.gptq_hptq_encode, g.lib.gptq_hptq_decode
    wsb = g.lib.gptq_hptq_code_workspace_bytes()
    assert 0 < wsb < 4 << 20
    n = C.c_int64(0)
    clen = (C.c_uint8 * 65536)()
    assert enc(FAKE, -1, 4, None, FAKE, 1, FAKE, C.byref(n), FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert enc(NULL, 4, 4, None, FAKE, 1, FAKE, C.byref(n), FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert enc(FAKE, 4, 4, None, FAKE, 1, NULL, C.byref(n), FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert enc(FAKE, 4, 4, None, FAKE, 1, FAKE, None, FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert enc(FAKE, 4, 4, None, NULL, 1, FAKE, C.byref(n), FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert enc(FAKE, 4, 4, None, FAKE, 1, FAKE, C.byref(n), FAKE, wsb - 1, NULL) == \
        g.GPTQ_EWORKSPACE
    assert dec(FAKE, 1, FAKE, 4, 4, None, FAKE, FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert dec(FAKE, -1, FAKE, 4, 4, clen, FAKE, FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert dec(NULL, 1, FAKE, 4, 4, clen, FAKE, FAKE, wsb, NULL) == g.GPTQ_EINVAL
    assert dec(FAKE, 1, FAKE, 4, 4, clen, FAKE, FAKE, 0, NULL) == g.GPTQ_EWORKSPACE
    clen[5] = 64  # longer than the 63 bits a code may have
    assert dec(FAKE, 1, FAKE, 4, 4, clen, FAKE, FAKE, wsb, NULL) == g.GPTQ_EINVAL
