"""Thin Python binding of libgptq (argument marshalling only).

Every step of the quantizer runs in the HIP library; this module only checks
tensor shapes/dtypes/devices, allocates outputs and workspaces with torch on
the current HIP device, and passes raw pointers plus torch's current stream.
If the library is missing the import fails: there is no fallback.

Names mirror the C ABI in include/gptq.h:
    hessian_accumulate(S, X)                    -> S (updated in place)
    prepare_hinv(S, n_tokens, damp, act_order)  -> (perm, U)
    quantize_layer(W, U, perm, bits, group_size)-> QuantizedLayer
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq.so")

GPTQ_OK, GPTQ_EINVAL, GPTQ_ENOTSPD, GPTQ_EHIP, GPTQ_EWORKSPACE, GPTQ_ENONFINITE = range(6)
GPTQ_FLAG_ACT_ORDER = 1
GPTQ_FLAG_HESSIAN_OVERWRITE = 2
GPTQ_FLAG_NO_SYNC = 4
GPTQ_FLAG_MIN_PIVOT = 8
GPTQ_FLAG_NO_CLIP = 16
GPTQ_FLAG_HESSIAN_SPLIT8 = 32
GPTQ_FLAG_FACTOR_FORM = 64

EXPORTS = {
    "gptq_hessian_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64]),
    "gptq_hessian_split8_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64]),
    "gptq_hessian_accumulate": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int64,
                                          C.c_uint32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "gptq_prepare_workspace_bytes": (C.c_size_t, [C.c_int64]),
    "gptq_prepare_hinv": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_double, C.c_uint32,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "gptq_quantize_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int]),
    "gptq_quantize_layer": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                                      C.c_void_p, C.c_int, C.c_int, C.c_uint32, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_size_t, C.c_void_p]),
    "gptq_quantize_layer_ssqr": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                           C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_uint32,
                                           C.c_double, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "gptq_ssqr_search": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                                   C.c_void_p, C.c_int, C.c_int, C.c_uint32, C.c_double, C.c_int,
                                   C.c_double, C.c_double, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "gptq_quantize_layer_noalloc": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                              C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                              C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                              C.c_void_p, C.c_void_p, C.c_void_p]),
    "gptq_ssqr_outliers_csr": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                         C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                         C.c_uint32, C.c_void_p, C.c_void_p]),
    "gptq_quantize_layer_hptq": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                           C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_uint32,
                                           C.c_double, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_size_t, C.c_void_p]),
    "gptq_hptq_search": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                                   C.c_void_p, C.c_int, C.c_int, C.c_uint32, C.c_double, C.c_int,
                                   C.c_double, C.c_double, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_size_t, C.c_void_p]),
    "gptq_hptq_code_workspace_bytes": (C.c_size_t, []),
    "gptq_hptq_encode": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                   C.c_void_p]),
    "gptq_hptq_decode": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int64,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "gptq_chmc_rank": (C.c_int, [C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_double]),
    "gptq_chmc_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int]),
    "gptq_chmc_layer": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                                  C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                  C.c_int, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                  C.c_void_p, C.c_void_p]),
    "gptq_workspace_status": (C.c_int, [C.c_void_p, C.c_void_p]),
    "gptq_status_string": (C.c_char_p, [C.c_int]),
    "gptq_fp16_round_host": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64]),
    "gptq_version": (C.c_int, []),
    "gptq_last_error_string": (C.c_char_p, []),
    "gptq_profile_enable": (C.c_int, [C.c_uint32]),
    "gptq_profile_kernel_count": (C.c_int, []),
    "gptq_profile_kernel_name": (C.c_char_p, [C.c_int]),
    "gptq_profile_read": (C.c_int, [C.c_void_p, C.c_void_p]),
}


def _load():
    # torch ships its own HIP runtime (same soname as /opt/rocm's). Import it
    # first so that libgptq binds to that one runtime: loading libgptq first
    # would map /opt/rocm's copy and torch would then load a second runtime
    # in the same process, whose device pointers the first cannot use.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libgptq.so is not built ({LIB_PATH}); run "
                          "`python -m post_weight_quantization_hessian_amd.build`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.gptq_status_string(status).decode()
        if status == GPTQ_EHIP:
            msg += f" [{lib.gptq_last_error_string().decode()}]"
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str):
    if status != GPTQ_OK:
        raise GPTQError(status, where)


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else C.c_void_p(0)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} tensor on a HIP device")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- step 1

def hessian_workspace_bytes(in_features: int, n_tokens: int) -> int:
    return int(lib.gptq_hessian_workspace_bytes(in_features, n_tokens))


def hessian_split8_workspace_bytes(in_features: int, n_tokens: int) -> int:
    return int(lib.gptq_hessian_split8_workspace_bytes(in_features, n_tokens))


def hessian_accumulate(S, X, workspace=None, overwrite=False, split8=False):
    """S += X^T X, or S = X^T X with ``overwrite`` (fp64 S [i x i], fp32 X
    [n x i] with unit stride along i). ``split8``: products from int8 digit
    slices on the int8 matrix cores (X rounded per column to 30 fractional
    bits of a power-of-two scale)."""
    torch = _torch()
    _need(S, torch.float64, "S", 2)
    _need(X, torch.float32, "X", 2)
    n, i = X.shape
    if S.shape != (i, i) or not S.is_contiguous():
        raise ValueError("S must be a contiguous [in_features x in_features] tensor")
    if X.stride(1) != 1:
        raise ValueError("X rows must be contiguous")
    if workspace is None:
        nb = hessian_split8_workspace_bytes(i, n) if split8 else hessian_workspace_bytes(i, n)
        workspace = _workspace(nb, X.device)
    flags = GPTQ_FLAG_HESSIAN_OVERWRITE if overwrite else 0
    if split8:
        flags |= GPTQ_FLAG_HESSIAN_SPLIT8
    st = lib.gptq_hessian_accumulate(_ptr(S), i, _ptr(X), n, X.stride(0) if n > 0 else i, flags,
                                     _ptr(workspace), workspace.numel(), _stream())
    _check(st, "gptq_hessian_accumulate")
    return S


# ---------------------------------------------------------------- steps 2-3

def prepare_workspace_bytes(in_features: int) -> int:
    return int(lib.gptq_prepare_workspace_bytes(in_features))


def prepare_hinv(S, n_tokens: int, damp: float = 0.01, act_order: bool = False,
                 workspace=None, out=None, sync: bool = True, min_pivot: bool = False,
                 factor_form: bool = False):
    """Damped, optionally act-ordered (or min-pivot-ordered) Hessian ->
    (perm int32 [i], U fp32 [i x i]). ``factor_form=True`` returns the mixed
    matrix of the factor form instead of U (U's 128-wide diagonal blocks, the
    factor U^-1 of H beyond them), for quantize_layer(..., factor_form=True).
    ``sync=False`` returns after enqueueing; check with workspace_status()."""
    torch = _torch()
    _need(S, torch.float64, "S", 2)
    i = S.shape[0]
    if S.shape != (i, i) or not S.is_contiguous():
        raise ValueError("S must be a contiguous square tensor")
    if out is None:
        perm = torch.empty(i, dtype=torch.int32, device=S.device)
        U = torch.empty((i, i), dtype=torch.float32, device=S.device)
    else:
        perm, U = out
    if workspace is None:
        workspace = _workspace(prepare_workspace_bytes(i), S.device)
    flags = ((GPTQ_FLAG_ACT_ORDER if act_order else 0) | (GPTQ_FLAG_MIN_PIVOT if min_pivot else 0)
             | (0 if sync else GPTQ_FLAG_NO_SYNC)
             | (GPTQ_FLAG_FACTOR_FORM if factor_form else 0))
    st = lib.gptq_prepare_hinv(_ptr(S), i, int(n_tokens), float(damp), flags, _ptr(perm), _ptr(U),
                               _ptr(workspace), workspace.numel(), _stream())
    _check(st, "gptq_prepare_hinv")
    return perm, U


# ---------------------------------------------------------------- steps 4-6

@dataclass
class QuantizedLayer:
    codes: object      # uint8 [rows x cols], original column order
    scales: object     # fp16  [rows x groups], groups in sweep order
    zeros: object      # fp16  [rows x groups]
    g_idx: object      # int32 [cols]
    row_loss: object   # fp64  [rows]
    bits: int
    group_size: int


def quantize_workspace_bytes(rows: int, cols: int, group_size: int) -> int:
    return int(lib.gptq_quantize_workspace_bytes(rows, cols, group_size))


def quantize_layer(W, U, perm=None, bits: int = 4, group_size: int = 128, workspace=None,
                   out=None, sync: bool = True, clip: bool = True, factor_form: bool = False):
    """Sweep the fp16 weights W [rows x cols] with the factor U (and perm).
    ``out`` may be a QuantizedLayer whose tensors are reused; ``sync=False``
    returns after enqueueing (check with workspace_status()); ``clip=False``
    is the no-clipping regime (stored codes saturate to [0, 255]);
    ``factor_form=True`` takes U from prepare_hinv(..., factor_form=True)."""
    torch = _torch()
    _need(W, torch.float16, "W", 2)
    _need(U, torch.float32, "U", 2)
    rows, cols = W.shape
    if U.shape != (cols, cols) or not U.is_contiguous():
        raise ValueError("U must be a contiguous [cols x cols] tensor")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    if perm is not None:
        _need(perm, torch.int32, "perm", 1)
        if perm.numel() != cols:
            raise ValueError("perm must have cols entries")
    ng = -(-cols // group_size) if group_size > 0 else 0
    dev = W.device
    if out is not None:
        codes, scales, zeros, g_idx, row_loss = out.codes, out.scales, out.zeros, out.g_idx, out.row_loss
        if codes.shape != (rows, cols) or scales.shape != (rows, ng) or row_loss.shape != (rows,):
            raise ValueError("out tensors have the wrong shape")
    else:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, ng), dtype=torch.float16, device=dev)
        zeros = torch.empty((rows, ng), dtype=torch.float16, device=dev)
        g_idx = torch.empty(cols, dtype=torch.int32, device=dev)
        row_loss = torch.empty(rows, dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = _workspace(quantize_workspace_bytes(rows, cols, group_size), dev)
    st = lib.gptq_quantize_layer(_ptr(W), rows, cols, W.stride(0) if rows > 0 else cols, _ptr(U),
                                 _ptr(perm), int(bits), int(group_size),
                                 (0 if sync else GPTQ_FLAG_NO_SYNC)
                                 | (0 if clip else GPTQ_FLAG_NO_CLIP)
                                 | (GPTQ_FLAG_FACTOR_FORM if factor_form else 0), _ptr(codes),
                                 _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(row_loss),
                                 _ptr(workspace), workspace.numel(), _stream())
    _check(st, "gptq_quantize_layer")
    return QuantizedLayer(codes, scales, zeros, g_idx, row_loss, bits, group_size)


@dataclass
class SSQRLayer:
    layer: QuantizedLayer
    outlier_mask: object  # uint8 [rows x cols], original column order, 1 = outlier
    outlier_vals: object  # fp16  [rows x cols], the outlier's value (0 elsewhere)
    n_outliers: int
    alpha: float
    # the stored form of the outliers: compressed sparse rows
    row_ptr: object = None   # int64 [rows + 1]
    col_idx: object = None   # int32 [n_outliers], increasing within a row
    csr_vals: object = None  # fp16  [n_outliers]

    @property
    def bits_per_weight(self) -> float:
        """Stored bits per weight: the b-bit codes, an fp16 scale and zero
        point per (row, group), and the outliers in CSR form (32-bit column
        index and fp16 value each, 64-bit row offsets)."""
        rows, cols = self.layer.codes.shape
        ng = -(-cols // self.layer.group_size)
        bits = (self.layer.bits * rows * cols + 32 * rows * ng + 48 * self.n_outliers
                + 64 * (rows + 1))
        return bits / (rows * cols)


def ssqr_outliers_csr(mask, vals, capacity=None, sync: bool = True):
    """Compressed sparse rows of a dense outlier mask and values (the device
    compaction of gptq_ssqr_outliers_csr). ``capacity`` defaults to the
    number of set mask entries counted on the device (one synchronize).
    Returns (row_ptr int64 [rows + 1], col_idx int32 [nnz], vals fp16 [nnz])."""
    torch = _torch()
    _need(mask, torch.uint8, "mask", 2)
    _need(vals, torch.float16, "vals", 2)
    if mask.shape != vals.shape or not (mask.is_contiguous() and vals.is_contiguous()):
        raise ValueError("mask and vals must be contiguous and of one shape")
    rows, cols = mask.shape
    dev = mask.device
    if capacity is None:
        capacity = int((mask != 0).sum().item())
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device=dev)
    col_idx = torch.empty(max(int(capacity), 1), dtype=torch.int32, device=dev)
    out = torch.empty(max(int(capacity), 1), dtype=torch.float16, device=dev)
    nnz = C.c_int64(0)
    st = lib.gptq_ssqr_outliers_csr(_ptr(mask), _ptr(vals), rows, cols, _ptr(row_ptr),
                                    _ptr(col_idx), _ptr(out), int(capacity),
                                    0 if sync else GPTQ_FLAG_NO_SYNC,
                                    C.byref(nnz) if sync else None, _stream())
    _check(st, "gptq_ssqr_outliers_csr")
    n = int(nnz.value) if sync else int(capacity)
    return row_ptr, col_idx[:n], out[:n]


def _with_csr(layer: SSQRLayer) -> SSQRLayer:
    layer.row_ptr, layer.col_idx, layer.csr_vals = ssqr_outliers_csr(
        layer.outlier_mask, layer.outlier_vals, capacity=layer.n_outliers)
    return layer


def _ssqr_args(W, U, perm, group_size):
    torch = _torch()
    _need(W, torch.float16, "W", 2)
    _need(U, torch.float32, "U", 2)
    rows, cols = W.shape
    if U.shape != (cols, cols) or not U.is_contiguous():
        raise ValueError("U must be a contiguous [cols x cols] tensor")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    if perm is not None:
        _need(perm, torch.int32, "perm", 1)
        if perm.numel() != cols:
            raise ValueError("perm must have cols entries")
    ng = -(-cols // group_size) if group_size > 0 else 0
    dev = W.device
    outs = dict(codes=torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                scales=torch.empty((rows, ng), dtype=torch.float16, device=dev),
                zeros=torch.empty((rows, ng), dtype=torch.float16, device=dev),
                g_idx=torch.empty(cols, dtype=torch.int32, device=dev),
                row_loss=torch.empty(rows, dtype=torch.float64, device=dev),
                mask=torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                vals=torch.empty((rows, cols), dtype=torch.float16, device=dev))
    ws = _workspace(quantize_workspace_bytes(rows, cols, group_size), dev)
    return rows, cols, outs, ws


def quantize_layer_ssqr(W, U, perm=None, bits: int = 4, group_size: int = 128,
                        alpha: float = 1.0) -> SSQRLayer:
    """The sweep under the SSQR rule at scale factor ``alpha`` (synchronous):
    out-of-grid levels kept as fp16 outliers, reported as a dense mask and
    values in the original column order and compacted on the device into
    compressed sparse rows (their stored form)."""
    rows, cols, o, ws = _ssqr_args(W, U, perm, group_size)
    n = C.c_uint64(0)
    st = lib.gptq_quantize_layer_ssqr(_ptr(W), rows, cols, W.stride(0) if rows > 0 else cols,
                                      _ptr(U), _ptr(perm), int(bits), int(group_size), 0,
                                      float(alpha), _ptr(o["codes"]), _ptr(o["scales"]),
                                      _ptr(o["zeros"]), _ptr(o["g_idx"]), _ptr(o["row_loss"]),
                                      _ptr(o["mask"]), _ptr(o["vals"]), C.byref(n), _ptr(ws),
                                      ws.numel(), _stream())
    _check(st, "gptq_quantize_layer_ssqr")
    q = QuantizedLayer(o["codes"], o["scales"], o["zeros"], o["g_idx"], o["row_loss"], bits,
                       group_size)
    return _with_csr(SSQRLayer(q, o["mask"], o["vals"], int(n.value), float(alpha)))


def ssqr_search(W, U, perm=None, bits: int = 4, group_size: int = 128, target: float = 0.01,
                iters: int = 12, alpha_lo: float = 1.0 / 64, alpha_hi: float = 1.0) -> SSQRLayer:
    """Bisection on the SSQR scale factor for the smallest alpha in
    [alpha_lo, alpha_hi] whose outlier fraction is at most ``target``; the
    result holds the sweep at that alpha."""
    rows, cols, o, ws = _ssqr_args(W, U, perm, group_size)
    n = C.c_uint64(0)
    a = C.c_double(0.0)
    st = lib.gptq_ssqr_search(_ptr(W), rows, cols, W.stride(0) if rows > 0 else cols, _ptr(U),
                              _ptr(perm), int(bits), int(group_size), 0, float(target),
                              int(iters), float(alpha_lo), float(alpha_hi), C.byref(a),
                              _ptr(o["codes"]), _ptr(o["scales"]), _ptr(o["zeros"]),
                              _ptr(o["g_idx"]), _ptr(o["row_loss"]), _ptr(o["mask"]),
                              _ptr(o["vals"]), C.byref(n), _ptr(ws), ws.numel(), _stream())
    _check(st, "gptq_ssqr_search")
    q = QuantizedLayer(o["codes"], o["scales"], o["zeros"], o["g_idx"], o["row_loss"], bits,
                       group_size)
    return _with_csr(SSQRLayer(q, o["mask"], o["vals"], int(n.value), float(a.value)))


@dataclass
class HPTQLayer:
    levels: object     # int16 [rows x cols], original column order
    scales: object     # fp16  [rows x groups], groups in sweep order (the steps)
    g_idx: object      # int32 [cols]
    row_loss: object   # fp64  [rows]
    bpw: float         # Huffman-coded bits per weight, with 16 per group step
    alpha: float


@dataclass
class HPTQStream:
    words: object      # uint32 [ceil(total_bits / 32)] on the device
    row_bit: object    # int64 [rows + 1] on the device
    code_len: object   # numpy uint8 [65536]: length of level v at v + 32768
    total_bits: int
    shape: tuple


def hptq_encode(levels) -> HPTQStream:
    """The Huffman code stream of an int16 level matrix (gptq_hptq_encode)."""
    torch = _torch()
    import numpy as np
    _need(levels, torch.int16, "levels", 2)
    if not levels.is_contiguous():
        raise ValueError("levels must be contiguous")
    rows, cols = levels.shape
    dev = levels.device
    ws = _workspace(int(lib.gptq_hptq_code_workspace_bytes()), dev)
    row_bit = torch.empty(rows + 1, dtype=torch.int64, device=dev)
    clen = np.zeros(65536, dtype=np.uint8)
    total = C.c_int64(0)

    def call(words, cap):
        return lib.gptq_hptq_encode(_ptr(levels), rows, cols, clen.ctypes.data_as(C.c_void_p),
                                    _ptr(words), cap, _ptr(row_bit), C.byref(total), _ptr(ws),
                                    ws.numel(), _stream())
    # first the size (a capacity of 0 returns the total with GPTQ_EINVAL),
    # then the stream
    st = call(None, 0)
    nw = -(-int(total.value) // 32)
    words = torch.zeros(max(nw, 1), dtype=torch.int32, device=dev)
    if nw > 0:
        if st != GPTQ_EINVAL:
            _check(st, "gptq_hptq_encode")
        st = call(words, nw)
    _check(st, "gptq_hptq_encode")
    return HPTQStream(words[:nw], row_bit, clen, int(total.value), (rows, cols))


def hptq_decode(s: HPTQStream):
    """The levels back from a code stream (gptq_hptq_decode)."""
    torch = _torch()
    rows, cols = s.shape
    dev = s.row_bit.device
    ws = _workspace(int(lib.gptq_hptq_code_workspace_bytes()), dev)
    out = torch.empty((rows, cols), dtype=torch.int16, device=dev)
    st = lib.gptq_hptq_decode(_ptr(s.words), s.words.numel(), _ptr(s.row_bit), rows, cols,
                              s.code_len.ctypes.data_as(C.c_void_p), _ptr(out), _ptr(ws),
                              ws.numel(), _stream())
    _check(st, "gptq_hptq_decode")
    return out


def _hptq_args(W, U, perm, group_size):
    rows, cols, o, ws = _ssqr_args(W, U, perm, group_size)
    torch = _torch()
    o["levels"] = torch.empty((rows, cols), dtype=torch.int16, device=W.device)
    return rows, cols, o, ws


def quantize_layer_hptq(W, U, perm=None, bits: int = 4, group_size: int = 128,
                        alpha: float = 1.0) -> HPTQLayer:
    """The no-clipping sweep on the HPTQ grid at scale factor ``alpha``
    (synchronous), with its Huffman-coded bits per weight."""
    rows, cols, o, ws = _hptq_args(W, U, perm, group_size)
    b = C.c_double(0.0)
    st = lib.gptq_quantize_layer_hptq(_ptr(W), rows, cols, W.stride(0) if rows > 0 else cols,
                                      _ptr(U), _ptr(perm), int(bits), int(group_size), 0,
                                      float(alpha), _ptr(o["levels"]), _ptr(o["scales"]),
                                      _ptr(o["zeros"]), _ptr(o["g_idx"]), _ptr(o["row_loss"]),
                                      C.byref(b), _ptr(ws), ws.numel(), _stream())
    _check(st, "gptq_quantize_layer_hptq")
    return HPTQLayer(o["levels"], o["scales"], o["g_idx"], o["row_loss"], float(b.value),
                     float(alpha))


def hptq_search(W, U, perm=None, bits: int = 4, group_size: int = 128, budget: float = 4.0,
                iters: int = 12, alpha_lo: float = 1.0 / 16, alpha_hi: float = 4.0) -> HPTQLayer:
    """Bisection on the HPTQ scale factor for the smallest alpha in
    [alpha_lo, alpha_hi] whose bits per weight are at most ``budget``."""
    rows, cols, o, ws = _hptq_args(W, U, perm, group_size)
    b = C.c_double(0.0)
    a = C.c_double(0.0)
    st = lib.gptq_hptq_search(_ptr(W), rows, cols, W.stride(0) if rows > 0 else cols, _ptr(U),
                              _ptr(perm), int(bits), int(group_size), 0, float(budget),
                              int(iters), float(alpha_lo), float(alpha_hi), C.byref(a),
                              _ptr(o["levels"]), _ptr(o["scales"]), _ptr(o["zeros"]),
                              _ptr(o["g_idx"]), _ptr(o["row_loss"]), C.byref(b), _ptr(ws),
                              ws.numel(), _stream())
    _check(st, "gptq_hptq_search")
    return HPTQLayer(o["levels"], o["scales"], o["g_idx"], o["row_loss"], float(b.value),
                     float(a.value))


@dataclass
class CHMCLayer:
    A: object          # fp16 [rows x rank]
    B: object          # fp16 [rank x cols]
    codes: object      # uint8 [rows x cols], original column order
    scales: object     # fp16 [row groups x cols], original column order
    zeros: object      # fp16 [row groups x cols]
    row_loss: object   # fp64 [rows]
    rank: int
    bits: int
    group_size: int


def chmc_outputs(rows: int, cols: int, rank: int, bits: int, group_size: int,
                 device) -> CHMCLayer:
    """Uninitialized output buffers of one CHMC layer call (for ``out=``)."""
    torch = _torch()
    ng = -(-rows // group_size)
    return CHMCLayer(torch.empty((rows, rank), dtype=torch.float16, device=device),
                     torch.empty((rank, cols), dtype=torch.float16, device=device),
                     torch.empty((rows, cols), dtype=torch.uint8, device=device),
                     torch.empty((ng, cols), dtype=torch.float16, device=device),
                     torch.empty((ng, cols), dtype=torch.float16, device=device),
                     torch.empty(rows, dtype=torch.float64, device=device),
                     int(rank), int(bits), int(group_size))


def chmc_rank(rows: int, cols: int, bits: int = 4, group_size: int = 128,
              bpw_target: float = 4.2875) -> int:
    return int(lib.gptq_chmc_rank(rows, cols, bits, group_size, bpw_target))


def chmc_workspace_bytes(rows: int, cols: int, rank: int) -> int:
    return int(lib.gptq_chmc_workspace_bytes(rows, cols, rank))


def chmc_layer(W, S, n_tokens, U, perm, omega, rank=None, bits: int = 4, group_size: int = 128,
               bpw_target: float = 4.2875, sync: bool = True, workspace=None,
               u_stream=None, out: CHMCLayer | None = None,
               factor_form: bool = False) -> CHMCLayer:
    """The CHMC layer on the device: energies from diag(S), the rank-``rank``
    fp16 factors of W from the sketch ``omega`` (fp64 [cols x >= rank]; its
    first ``rank`` columns are used), the residual swept with one grid per
    group of ``group_size`` output rows and column. ``rank`` defaults to the
    largest that fits ``bpw_target``. ``u_stream``: a torch stream on which U and
    perm are still being produced; the frontend then overlaps with that work
    and only the sweep waits for it. ``out``: buffers from chmc_outputs of the
    same shape, rank, bits and group size to write into. ``factor_form``: U
    is the matrix of prepare_hinv(..., factor_form=True)."""
    torch = _torch()
    _need(W, torch.float16, "W", 2)
    _need(S, torch.float64, "S", 2)
    _need(U, torch.float32, "U", 2)
    rows, cols = W.shape
    if W.stride(1) != 1:
        raise ValueError("W must have unit column stride")
    r = chmc_rank(rows, cols, bits, group_size, bpw_target) if rank is None else int(rank)
    om = None
    if r > 0:
        _need(omega, torch.float64, "omega", 2)
        if omega.shape[0] != cols or omega.shape[1] < r:
            raise ValueError("omega must be [cols x >= rank]")
        om = omega[:, :r].contiguous()
    if perm is not None:
        _need(perm, torch.int32, "perm", 1)
    if tuple(S.shape) != (cols, cols) or not S.is_contiguous():
        raise ValueError("S must be a contiguous [cols x cols] tensor")
    if tuple(U.shape) != (cols, cols) or not U.is_contiguous():
        raise ValueError("U must be a contiguous [cols x cols] tensor")
    dev = W.device
    if out is None:
        out = chmc_outputs(rows, cols, r, bits, group_size, dev)
    elif (out.rank, out.bits, out.group_size) != (r, int(bits), int(group_size)) or \
            tuple(out.codes.shape) != (rows, cols) or tuple(out.A.shape) != (rows, r):
        raise ValueError("out does not match this call's shape, rank, bits or group size")
    A, B, codes, scales, zeros, row_loss = (out.A, out.B, out.codes, out.scales, out.zeros,
                                            out.row_loss)
    nb = chmc_workspace_bytes(rows, cols, r)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _workspace(nb, dev)
    st = lib.gptq_chmc_layer(_ptr(W), rows, cols, W.stride(0), _ptr(S), int(n_tokens), _ptr(U),
                             _ptr(perm), _ptr(om), r, int(bits), int(group_size),
                             (0 if sync else GPTQ_FLAG_NO_SYNC)
                             | (GPTQ_FLAG_FACTOR_FORM if factor_form else 0), _ptr(A), _ptr(B),
                             _ptr(codes),
                             _ptr(scales), _ptr(zeros), _ptr(row_loss), _ptr(ws), ws.numel(),
                             _stream(),
                             C.c_void_p(u_stream.cuda_stream) if u_stream is not None
                             else C.c_void_p(0))
    _check(st, "gptq_chmc_layer")
    return out


def workspace_status(workspace):
    """Synchronize the current stream and return the status left in a
    workspace by an asynchronous prepare_hinv / quantize_layer (raises on error)."""
    _check(lib.gptq_workspace_status(_ptr(workspace), _stream()), "gptq_workspace_status")


# ---------------------------------------------------------------- utilities

def fp16_round_host(values):
    """Nearest-even fp16 bit patterns of fp64 values (host routine of the library)."""
    import numpy as np
    a = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(lib.gptq_fp16_round_host(a.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p),
                                    a.size), "gptq_fp16_round_host")
    return out


def kernel_names():
    return [lib.gptq_profile_kernel_name(k).decode() for k in range(lib.gptq_profile_kernel_count())]


def profile_enable(kernels=True):
    """True: time every kernel; False/None: off; or an iterable of kernel names."""
    if kernels is True:
        mask = 0xFFFFFFFF
    elif not kernels:
        mask = 0
    else:
        names = kernel_names()
        mask = 0
        for k in kernels:
            mask |= 1 << names.index(k)
    _check(lib.gptq_profile_enable(mask), "gptq_profile_enable")


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} since the last read."""
    n = lib.gptq_profile_kernel_count()
    tot = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    _check(lib.gptq_profile_read(C.cast(tot, C.c_void_p), C.cast(cnt, C.c_void_p)),
           "gptq_profile_read")
    return {lib.gptq_profile_kernel_name(k).decode(): (tot[k], cnt[k]) for k in range(n)}
