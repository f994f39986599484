#!/usr/bin/env python3
"""Benchmark of the GPTQ layer quantizer on one MI355X.

A step is one pass of the whole hot path over one workload: for every
calibration input, the Hessian (S = X^T X over its token chunks), the damped
and act-ordered factor U of the inverse, and the column sweep of every layer
that reads the input (rows stacked), at every bit width of the workload.
Inputs (activations and fp16 weights) are resident in HBM before timing.

Prints ONE JSON line: throughput in quantized weights per second, the
roofline of the dominant kernel (HIP-event durations measured inside the
timed steps on the launch stream), and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = ("quantized weights/sec per layer + XXᵀ/trailing-GEMM % MFMA peak, 1×MI355X")
DEFAULT_WORKLOAD = "llama70b_down"
CHOL_MERGE_TILES = 504  # the library's threshold for the merged factor + update launch
CHOL_FUSE_NT = 48  # the library's bound on panels for the inverse accumulated in the factorization
QEMB_KMAX = 512  # the library's longest early update-GEMM piece inside a sweep launch

# MI355X published peaks
PEAK = {"f64_mfma": 78.6, "f64_vec": 78.6, "f32_mfma": 157.3, "bf16_mfma": 2500.0, "i8_mfma": 5000.0,
        "hbm_gbs": 8000.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--order", choices=("workload", "min_pivot"), default="workload",
                    help="column order: the workload's (act-order or none), or the "
                         "min-pivot order for every input")
    ap.add_argument("--hessian", choices=("auto", "exact", "split8"), default="auto",
                    help="Hessian products: exact fp64, int8 digit slices, or split8 from "
                         "256 input features on (auto)")
    ap.add_argument("--factor-form", choices=("auto", "on", "off"), default="auto",
                    help="the plain sweep in the factor form (no triangular inverse beyond "
                         "the 128-wide diagonal blocks): from 768 features (auto), always "
                         "or never")
    ap.add_argument("--no-clip", action="store_true",
                    help="the no-clipping sweep: levels are not clamped to [0, maxq]")
    ap.add_argument("--ssqr", type=float, default=None, metavar="TARGET",
                    help="quantize with SSQR instead: bisection on the scale factor for at "
                         "most this outlier fraction (every probe is a full sweep)")
    ap.add_argument("--ssqr-iters", type=int, default=12)
    ap.add_argument("--hptq", type=float, default=None, metavar="BUDGET",
                    help="quantize with HPTQ instead: bisection on the scale factor for at "
                         "most this many Huffman-coded bits per weight")
    ap.add_argument("--chmc", type=float, default=None, metavar="BPW",
                    help="quantize with the CHMC frontend instead: per layer, the fp16 "
                         "low-rank factors of the largest rank that fits BPW bits per weight "
                         "and the residual swept with one grid per output-row group")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="rows per layer group for the oracle sample (0 = auto)")
    ap.add_argument("--counters-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                              "COPY_WRITE"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of this benchmark, then of --calibrate-copy) into "
                         "the HBM traffic summary under profiles/ and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the "
                         "reference transfer for hardware traffic counters) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work

def chmc_flops(plan, bits_n, in_block):
    """fp64 multiply-adds (2 flops each) of the CHMC residual sweep: the lazy
    update of block b (at j0) is rows x j0 x bw, the in-block propagation rows
    x bw (bw - 1) / 2; per bit width."""
    f = 0.0
    for h in plan:
        for j0 in range(0, h.dim, 128):
            bw = min(128, h.dim - j0)
            f += 2.0 * h.rows * (bw * (bw - 1) / 2.0 if in_block else j0 * bw)
    return f * bits_n


def chmc_bpw(o, i, r, bits, gs):
    """Stored bits per weight of a CHMC layer: fp16 factors 16 r (o + i), the
    b-bit residual codes, per output group and column an fp16 scale and a
    zero point in [0, 2^b - 1] (b bits)."""
    ng = -(-o // gs)
    return (16 * r * (o + i) + bits * o * i + (16 + bits) * ng * i) / (o * i)


def kernel_work(name, wl, plan, sweeps=1.0):
    """Algorithmic flops (or bytes) of all launches of one kernel class in a
    step, with the unit and the roofline it is priced against. ``sweeps``:
    full sweeps per layer and bit width in a step (the SSQR search runs
    several; measured from the sweep launches)."""
    if name in ("chmc_update", "chmc_sweep"):
        return chmc_flops(plan, len(wl.bits), name == "chmc_sweep"), "flop", "f64_vec"
    if name == "hessian_tile":
        f = sum(h.n * h.dim * (h.dim + 1) for h in plan if not h.split8)  # symmetric half
        return f, "flop", "f64_mfma"
    if name == "hessian_split8":
        # the 13 digit-pair products (orders a + b <= 4) of the symmetric
        # half, int8 multiply + add
        f = sum(13 * h.n * h.dim * (h.dim + 1) for h in plan if h.split8)
        return f, "op", "i8_mfma"
    if name == "hessian_digits":
        # column maxima (read X), digit planes (read X, write 4 int8 per value)
        b = sum(12 * h.n * h.dim for h in plan if h.split8)
        return b, "byte", "hbm"
    if name in ("chol_trsm", "chol_potrf_syrk", "chol_potrf", "chol_col"):
        # Mirrors the library's launch sequence. Per panel p with m trailing
        # tile rows: trsm m tiles (a triangular solve with 128 right-hand
        # sides, 128^3 per tile); the next tile column, m tiles (chol_col);
        # the rest of the trailing update, r = m(m-1)/2 tiles of 2 128^3,
        # beside the next diagonal block (chol_potrf_syrk, the block's
        # (2/3) 128^3 counted there) up to CHOL_MERGE_TILES (at least the m-1
        # tiles of the next column), the others beside the next panel's
        # column update. With the inverse accumulated in the factorization
        # (nt <= CHOL_FUSE_NT, never in the factor form, which needs no inverse
        # beyond the diagonal tiles), trsm also solves the p + 1 tiles of X's row
        # block p (and the last row block after the loop), and the m (p + 1)
        # inverse tile updates of the step (2 128^3 each, half at j = p, where
        # the operand X_pp is triangular) fill the rest of the merged launch,
        # the others beside the column update.
        f = 0.0
        for h in plan:
            nt = -(-h.dim // 128)
            fused = nt <= CHOL_FUSE_NT and not h.factor_form
            if name == "chol_potrf":
                f += 2 * 128 ** 3 / 3.0  # panel 0
            if name == "chol_trsm" and fused:
                f += 128 ** 3 * nt  # last row block of X
            sov = 0
            for p in range(nt - 1):
                m = nt - 1 - p
                r = m * (m - 1) // 2
                xt = m * (p + 1) if fused else 0
                ns = min(r, max(CHOL_MERGE_TILES, m - 1))
                xstep = min(xt, max(0, CHOL_MERGE_TILES - ns))
                xcol = xt - xstep

                def xflops(ids):
                    return sum(2 * 128 ** 3 if i % (p + 1) != p else 128 ** 3 for i in ids)
                if name == "chol_trsm":
                    f += 128 ** 3 * (m + ((p + 1) if fused else 0))
                elif name == "chol_col":
                    f += 2 * 128 ** 3 * (m + sov) + xflops(range(xcol))
                elif name == "chol_potrf_syrk":
                    f += 2 * 128 ** 3 * ns + 2 * 128 ** 3 / 3.0 + xflops(range(xcol, xt))
                sov = r - ns
        return f, "flop", "f64_mfma"
    if name in ("trtri_t", "trtri_x"):
        # X21 = -X22 (L21 X11) at each doubling level, triangular zeros skipped
        f = 0.0
        for h in plan:
            nt = -(-h.dim // 128)
            hh = nt if (h.factor_form or nt <= CHOL_FUSE_NT) else 1  # no doubling levels
            while hh < nt:
                for q0 in range(0, nt, 2 * hh):
                    h2 = min(hh, nt - q0 - hh)
                    for r in range(max(h2, 0)):
                        for c in range(hh):
                            f += 2 * 128 ** 3 * ((hh - c) if name == "trtri_t" else (r + 1))
                hh *= 2
        return f, "flop", "f64_mfma"
    if name == "minpivot_update":
        # after every full panel of the min-pivot search: A -= P P^T on all
        # nt(nt+1)/2 lower tiles, 2 128^3 each
        f = 0.0
        for h in plan:
            nt = -(-h.dim // 128)
            f += 2 * 128 ** 3 * nt * (nt + 1) // 2 * ((h.dim - 1) // 128)
        return f, "flop", "f64_mfma"
    if name == "quant_gemm":
        # the update GEMM flops that run in q_gemm launches (the rest run
        # inside the sweep launches, see quant_gemm_split)
        f = 0.0
        for h in plan:
            f += len(wl.bits) * quant_gemm_split(h.rows, h.dim)[0]
        return f * sweeps, "flop", "f32_mfma"
    if name == "quant_sweep":
        # bytes per weight: fp16 weight 2 + fp64 update 8 + code 1 + fp32 error 4;
        # plus 4 bytes (fp16 scale + zero) per group and the fp32 U slab per block
        # (the next block's early update GEMM, run by extra workgroups of the
        # same launches, is not counted here)
        b = 0.0
        for h in plan:
            for bits in wl.bits:
                b += h.rows * h.dim * 15 + h.rows * (-(-h.dim // wl.group_size)) * 4
                b += sum(4 * min(128, h.dim - j0) ** 2 for j0 in range(0, h.dim, 128))
        return b * sweeps, "byte", "hbm"
    return None, None, None


def quant_gemm_split(rows, cols):
    """(flops in q_gemm launches, flops inside sweep launches) of one layer's
    update GEMM, W~_b = W_b - E[:, :j0] U[:j0, b]. Mirrors the library: while
    the sweep leaves CUs idle (4 waves per workgroup, room for at least one
    GEMM workgroup per 64-row tile beside it), the sum over the errors of
    blocks before b-1 runs inside the sweep launch of block b-1 (pieces of at
    most QEMB_KMAX) and the sum over block b-1's errors inside the sweep of
    block b; otherwise (and for a block whose early pieces would be longer)
    the whole sum runs in a q_gemm launch before the sweep."""
    rt = -(-rows // 64)
    pmax = min(16, max(1, -(-512 // rt)))
    nw = 8 if -(-rows // 32) >= 256 else 4
    nsweep = -(-rows // (4 * nw))
    emb_max = min(pmax, (256 - nsweep) // rt) if nw == 4 else 0
    ep = 0 if emb_max > 0 else -1
    fg = fe = 0.0
    for j0 in range(0, cols, 128):
        bw = min(128, cols - j0)
        if j0 > 0:
            if ep >= 0:
                fe += 2.0 * rows * 128 * bw
            else:
                fg += 2.0 * rows * j0 * bw
        nxt = 0 if emb_max > 0 else -1
        if emb_max > 0 and j0 > 0 and j0 + 128 < cols:
            pe = min(emb_max, -(-j0 // QEMB_KMAX))
            ks = -(-(-(-j0 // pe)) // 32) * 32
            if ks <= QEMB_KMAX:
                nxt = -(-j0 // ks)
                fe += 2.0 * rows * j0 * min(128, cols - j0 - 128)
            else:
                nxt = -1
        ep = nxt
    return fg, fe


class HPlan:
    def __init__(self, name, dim, n, rows, split8=False, factor_form=False):
        self.name, self.dim, self.n, self.rows = name, dim, n, rows
        self.split8 = split8
        # the plain sweep's factor form: no inverse beyond the diagonal tiles
        self.factor_form = factor_form


# ---------------------------------------------------------------- HBM traffic

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "post_weight_quantization_hessian_amd", "csrc")
KERNEL_CLASS = {  # device function name -> timing class
    "hess_tile_kernel": "hessian_tile", "hess_reduce_kernel": "hessian_reduce",
    "chol_potrf_syrk_kernel": "chol_potrf_syrk", "chol_potrf_kernel": "chol_potrf",
    "chol_col_kernel": "chol_col",
    "chol_trsm_kernel": "chol_trsm",
    "trtri_t_kernel": "trtri_t", "trtri_x_kernel": "trtri_x", "trtri_sum_kernel": "trtri_sum",
    "trtri_diag_kernel": "trtri_diag", "q_gemm_kernel": "quant_gemm",
    "q_sweep_kernel": "quant_sweep",
    "prep_gather_kernel": "prepare_gather", "prep_uout_kernel": "prepare_uout",
    "prep_uout_z_kernel": "prepare_uout", "prep_mout_kernel": "prepare_uout",
    "prep_mfac_kernel": "prepare_uout",
    "mp_init_kernel": "minpivot_step",
    "mp_step_kernel": "minpivot_step", "mp_panel_kernel": "minpivot_step",
    "mp_update_kernel": "minpivot_update",
    "h8_tile_kernel": "hessian_split8", "h8_colmax_kernel": "hessian_digits",
    "h8_split_kernel": "hessian_digits", "q_hist_kernel": "quant_hist",
    "ch_update_kernel": "chmc_update", "ch_cur_kernel": "chmc_update",
    "ch_sweep_rows_kernel": "chmc_sweep", "ch_rowdot_kernel": "chmc_front",
    "hf_hist_kernel": "hptq_code", "hf_rowbits_kernel": "hptq_code",
    "hf_scan_kernel": "hptq_code", "hf_encode_kernel": "hptq_code",
    "hf_decode_kernel": "hptq_code", "hf_zero_kernel": "hptq_code",
    "sp_count_kernel": "ssqr_csr", "sp_scan_kernel": "ssqr_csr", "sp_fill_kernel": "ssqr_csr",
    "ch_gemm_nn": "chmc_front", "ch_gemm_tn": "chmc_front", "ch_sum_kernel": "chmc_front",
    "ch_chol_inv_kernel": "chmc_front", "ch_jacobi_kernel": "chmc_front",
    "ch_energy_kernel": "chmc_front", "ch_scale_kernel": "chmc_front",
    "ch_factor_kernel": "chmc_front", "ch_resid_kernel": "chmc_front",
    "ch_perm_count_kernel": "chmc_front", "ch_perm_check_kernel": "chmc_front",
    "ch_zero_kernel": "fill"}


def _code_only(text):
    """The source without its comments and blank-line differences (a comment
    edit does not change a kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_hash(csrc=None):
    """sha256 over the HIP sources' code: counters taken on other code are
    stale."""
    import hashlib
    csrc = csrc or CSRC
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()


def kernel_source_hash(kernel_class, csrc=None):
    """sha256 over the code of the sources that define the kernels of one
    timing class, and every header: a class's counters stay valid while
    that code is unchanged (None if no source defines the class)."""
    import hashlib
    import re
    csrc = csrc or CSRC
    names = [k for k, c in KERNEL_CLASS.items() if c == kernel_class]
    files = sorted(os.listdir(csrc))
    code = {f: _code_only(open(os.path.join(csrc, f), encoding="utf-8").read()) for f in files
            if f.endswith((".hip", ".h"))}
    own = [f for f in files if f.endswith(".hip")
           and any(re.search(rf"\b{n}\s*\(", code[f]) for n in names)]
    if not own:
        return None
    h = hashlib.sha256()
    for f in sorted(own) + [f for f in files if f.endswith(".h")]:
        h.update(f.encode())
        h.update(code[f].encode())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")


def _pmc_per_class(folder):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    tot = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            key = next((c for k, c in KERNEL_CLASS.items() if f"::{k}" in name), None)
            if key is None and "copyBuffer" in name:
                key = "copy"
            if key is None:
                continue
            v = tot.setdefault(key, [0.0, 0])
            v[0] += float(r["Counter_Value"])
            v[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in tot.items()}


def counters_summary(args):
    fetch, write, cfetch, cwrite = (_pmc_per_class(d) for d in args.counters_summary)
    copy_bytes = 1 << 30
    # KiB per dispatch that the same counter reads for a plain 1 GiB copy
    f_fac = copy_bytes / (cfetch["copy"][0] * 1024.0)
    w_fac = copy_bytes / (cwrite["copy"][0] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        fb = fetch[k][0] * 1024.0 * f_fac
        wb = write[k][0] * 1024.0 * w_fac
        kernels[k] = {"fetch_kib_per_dispatch": fetch[k][0], "write_kib_per_dispatch": write[k][0],
                      "dispatches": fetch[k][1], "bytes_per_launch": fb + wb,
                      "read_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                      "source_sha256": kernel_source_hash(k)}
    out = {"workload": args.workload, "source_sha256": source_hash(),
           "fetch_scale": f_fac, "write_scale": w_fac,
           "copy_reference": "bench.py --calibrate-copy 1024 (1 GiB device copy, 5 dispatches)",
           "commands": [f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 "
                        f"bench.py --workload {args.workload} --steps 2 --warmup 1 "
                        "--no-cpu-baseline" for c in ("FETCH_SIZE", "WRITE_SIZE")]
                       + [f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 "
                          "bench.py --calibrate-copy 1024" for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "kernels": kernels}
    with open(traffic_path(args.workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v["bytes_per_launch"] for k, v in kernels.items()}))


def measured_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary,
    or None when there is none or the code of that kernel's sources (or of a
    header) changed since it was taken."""
    try:
        d = json.load(open(traffic_path(workload)))
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") is None:
        return None
    if k["source_sha256"] != kernel_source_hash(kernel):
        return None
    return k["bytes_per_launch"]


# ---------------------------------------------------------------- CPU oracle

CPU_FLOP_BUDGET = 2.5e11   # accumulate sample: tokens x dim^2 x 2 flops
CPU_FACTOR_DIM = 6144      # larger Hessians are factored on a leading sub-block


def cpu_baseline(wl, host_inputs, sample_rows):
    """The fp64 oracle timed on a bounded sample of one step's work, scaled to
    the whole step by each phase's operation count: the accumulate on a token
    sample (x tokens), the damping/act-order/factor on the full Hessian or,
    above CPU_FACTOR_DIM features, on its leading sub-block (x dim^3), and the
    strict sweep on a row sample (x rows, x dim^2 when the factor was a
    sub-block)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    t_total = 0.0
    sampled = []
    for hname, (Xs, W) in host_inputs.items():
        dim = Xs.shape[1]
        n_s = int(min(wl.n_tokens, Xs.shape[0], max(256, CPU_FLOP_BUDGET // (2 * dim * dim))))
        t0 = time.perf_counter()
        S, n = O.hessian_sum([Xs[:n_s]])
        t_acc = (time.perf_counter() - t0) * wl.n_tokens / n_s
        d_s = min(dim, CPU_FACTOR_DIM)
        t0 = time.perf_counter()
        H = O.damped_hessian(S[:d_s, :d_s], n, wl.damp)
        perm = O.act_order_perm(H) if wl.act_order else np.arange(d_s)
        U = O.hinv_upper(O.permute_sym(H, perm))
        t_fac = (time.perf_counter() - t0) * (dim / d_s) ** 3
        rows = W.shape[0]
        rs = min(rows, sample_rows)
        Wp = W[:rs, :d_s].astype(np.float64)[:, perm]
        t_sw = 0.0
        for bits in wl.bits:
            t0 = time.perf_counter()
            O.gptq_sweep(Wp, U, bits, wl.group_size)
            t_sw += (time.perf_counter() - t0) * (rows / rs) * (dim / d_s) ** 2
        t_total += t_acc + t_fac + t_sw
        sampled.append(f"{hname}: accumulate {n_s}/{wl.n_tokens} tokens x {dim}, "
                       f"damp/act-order/factor {d_s}/{dim} features, strict sweep "
                       f"{rs}/{rows} rows x {d_s} columns x {len(wl.bits)} widths")
    weights = wl.weights_per_step()
    return {"value": weights / t_total, "unit": "weights/s", "cores": int(threads),
            "kind": "oracle", "sample": "; ".join(sampled) + " (each phase scaled to the "
            "full step by its operation count)",
            "seconds_per_step_extrapolated": t_total, "cpu_model": host_cpu_model(),
            "blas": numpy_blas()}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def numpy_blas():
    """The BLAS NumPy was built against (name and version), as NumPy reports it."""
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:  # older NumPy or an unexpected layout: not essential
        return None


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.counters_summary:
        counters_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the quantizer's hot path is measured "
              "on one MI355X (multi-GPU sharding is design-only).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": 5}), flush=True)
        return
    from post_weight_quantization_hessian_amd import synth
    from post_weight_quantization_hessian_amd.workloads import WORKLOADS
    import post_weight_quantization_hessian_amd.gptq as G
    from post_weight_quantization_hessian_amd.pipeline import CHMC_DAMP, LayerGroup

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident on the device (host copies kept only for the
    # oracle's token sample)
    host_inputs = {}
    dev_inputs = {}
    plan = []
    layer_rows = {}
    for h in wl.inputs:
        print(f"[bench] generating {h.name}: {wl.n_tokens} x {h.dim}", file=sys.stderr, flush=True)
        X = synth.activations(wl.wid, h.name, wl.n_tokens, h.dim, kind=h.kind,
                              lognormal_sigma=h.lognormal_sigma)
        Ws = [synth.weights(wl.wid, l.name, l.rows, h.dim, outlier_frac=l.outlier_frac)
              for l in wl.layers_of(h.name)]
        W = np.concatenate(Ws, axis=0)
        chunks = [torch.from_numpy(X[s:s + wl.token_chunk]).to(dev)
                  for s in range(0, wl.n_tokens, wl.token_chunk)]
        host_inputs[h.name] = (X[:min(wl.n_tokens, 16384)].copy(), W)
        del X
        grp = LayerGroup(h.dim, W.shape[0], max_chunk_tokens=max(c.shape[0] for c in chunks),
                         bits=wl.bits, group_size=wl.group_size, act_order=wl.act_order,
                         min_pivot=args.order == "min_pivot", hessian=args.hessian,
                         factor_form={"auto": "auto", "on": True, "off": False}[args.factor_form],
                         clip=not args.no_clip,
                         damp=wl.damp, device=dev)
        dev_inputs[h.name] = (chunks, torch.from_numpy(W).to(dev), grp)
        # the plain and CHMC sweeps may take the factor form; SSQR and HPTQ take U
        plain = args.ssqr is None and args.hptq is None
        plan.append(HPlan(h.name, h.dim, wl.n_tokens, W.shape[0], split8=grp.split8,
                          factor_form=grp.factor_form and plain))
        layer_rows[h.name] = [(l.name, l.rows) for l in wl.layers_of(h.name)]
    torch.cuda.synchronize()

    # Each calibration input (with the layers that read it) is an independent
    # pipeline; the pipelines are enqueued asynchronously on their own streams
    # and overlap on the device, the largest Hessian first (its chain of
    # dependent launches is the longest, so it should not wait for the host
    # to enqueue the others). Statuses are checked after the timed steps.
    order = sorted(wl.inputs, key=lambda h: -h.dim)
    streams = [torch.cuda.Stream(device=dev) for _ in order]

    ssqr_last = {}
    hptq_last = {}
    chmc_last = {}
    if sum(a is not None for a in (args.ssqr, args.hptq, args.chmc)) > 1:
        raise SystemExit("--ssqr, --hptq and --chmc are exclusive")
    omegas = {}
    if args.chmc is not None:  # the sketch the method draws: seeded Gaussian per input
        for h in order:
            rng = np.random.default_rng(1000 + h.dim)
            omegas[h.name] = torch.from_numpy(rng.standard_normal((h.dim, 64))).to(dev)

    def step():
        for h, s in zip(order, streams):
            chunks, Wd, grp = dev_inputs[h.name]
            with torch.cuda.stream(s):
                if args.ssqr is not None:
                    ssqr_last[h.name] = grp.ssqr(chunks, Wd, args.ssqr, args.ssqr_iters)
                elif args.hptq is not None:
                    hptq_last[h.name] = grp.hptq(chunks, Wd, args.hptq, args.ssqr_iters)
                elif args.chmc is not None:
                    chmc_last[h.name] = grp.chmc(chunks, Wd, layer_rows[h.name], args.chmc,
                                                 omegas[h.name])
                else:
                    grp.enqueue(chunks, Wd)

    def check_status():
        for h, s in zip(order, streams):
            with torch.cuda.stream(s):
                dev_inputs[h.name][2].check()

    # ---- warmup: all kernels timed to find the dominant class
    G.profile_enable(True)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    check_status()
    prof_warm = G.profile_read()
    G.profile_enable(False)
    # sweeps per layer and bit width in a step: one, or the SSQR search's
    # probes (sweep launches over the launches of one sweep of every layer)
    sweeps = 1.0
    if args.ssqr is not None or args.hptq is not None:
        per_sweep = sum(len(wl.bits) * -(-h.dim // 128) for h in plan)
        sweeps = prof_warm["quant_sweep"][1] / max(args.warmup, 1) / per_sweep
    # the dominant kernel: the most device time among the classes with a work
    # model (the status fills and init kernels have none; on launch-bound
    # shapes their event times also carry the host's submission gaps)
    modelled = [k for k in prof_warm
                if prof_warm[k][1] > 0 and kernel_work(k, wl, plan, sweeps)[0] is not None]
    dominant = max(modelled or list(prof_warm), key=lambda k: prof_warm[k][0])

    # ---- timed steps: the dominant kernel's launches of the last step are
    # bracketed by HIP events on their stream (an event pair per launch sits
    # on the dependent chain, so bracketing every step would slow the steps
    # it measures)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i == args.steps - 1:
            G.profile_enable([dominant])
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = G.profile_read()
    G.profile_enable(False)
    check_status()

    ms_per_step = 1000.0 * elapsed / args.steps
    # the spread: five more steps, each alone between two synchronizations
    # (after the timed steps, so the K-step figure above is untouched)
    reps = []
    for _ in range(5):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        reps.append(1000.0 * (time.perf_counter() - t1))
    check_status()
    reps.sort()
    step_repeats = {"n": len(reps), "median_ms": reps[len(reps) // 2], "min_ms": reps[0],
                    "max_ms": reps[-1],
                    "note": "single steps, each between two device synchronizations"}
    weights = wl.weights_per_step()
    value = weights * args.steps / elapsed

    dom_ms, dom_launches = prof[dominant]
    work, unit, peak_key = kernel_work(dominant, wl, plan, sweeps)
    roofline = None
    traffic = measured_traffic(wl.name, dominant)
    if work is not None and dom_ms > 0:
        per_step_s = dom_ms / 1000.0  # one bracketed step
        if unit in ("flop", "op"):
            achieved = work / per_step_s / 1e12
            peak = PEAK[peak_key]
            roofline = {"bound": "alu" if peak_key == "f64_vec" else "mfma",
                        "achieved": achieved, "peak": peak,
                        "unit": "TFLOP/s" if unit == "flop" else "TOP/s",
                        "frac": achieved / peak, "traffic": traffic,
                        "kernel": dominant, "precision": peak_key,
                        "launches_per_step": dom_launches,
                        "avg_launch_ms": dom_ms / max(dom_launches, 1)}
            if unit == "flop":
                roofline["frac_vs_bf16_dense"] = achieved / PEAK["bf16_mfma"]
                roofline["frac_vs_f32_mfma"] = achieved / PEAK["f32_mfma"]
        else:
            achieved = work / per_step_s / 1e9
            roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK["hbm_gbs"],
                        "unit": "GB/s", "frac": achieved / PEAK["hbm_gbs"], "traffic": traffic,
                        "kernel": dominant, "launches_per_step": dom_launches,
                        "avg_launch_ms": dom_ms / max(dom_launches, 1)}

    breakdown = {k: {"ms_per_step": v[0] / max(args.warmup, 1),
                     "launches_per_step": v[1] / max(args.warmup, 1)}
                 for k, v in prof_warm.items() if v[1] > 0}
    for k, v in breakdown.items():
        w, u, pk = kernel_work(k, wl, plan, sweeps)
        if w is not None and v["ms_per_step"] > 0:
            rate = w / (v["ms_per_step"] / 1000.0)
            v["achieved"] = rate / (1e9 if u == "byte" else 1e12)
            v["unit"] = {"flop": "TFLOP/s", "op": "TOP/s", "byte": "GB/s"}[u]
            v["peak"] = PEAK["hbm_gbs"] if u == "byte" else PEAK[pk]
            v["frac"] = v["achieved"] / v["peak"]
    # X^T X of the int8 digit-slice Hessian as the flops of the product it
    # stands for (n i (i+1), symmetric half): its rate against the fp64 MFMA
    # peak, the instruction the exact products use
    if "hessian_split8" in breakdown and breakdown["hessian_split8"]["ms_per_step"] > 0:
        xf = sum(h.n * h.dim * (h.dim + 1) for h in plan if h.split8)
        eq = xf / (breakdown["hessian_split8"]["ms_per_step"] / 1000.0) / 1e12
        breakdown["hessian_split8"]["xxt_tflops"] = eq
        breakdown["hessian_split8"]["xxt_frac_vs_f64_mfma"] = eq / PEAK["f64_mfma"]
        if roofline is not None and roofline.get("kernel") == "hessian_split8":
            xeq = xf / per_step_s / 1e12
            roofline["xxt_tflops"] = xeq
            roofline["xxt_frac_vs_f64_mfma"] = xeq / PEAK["f64_mfma"]
    # device time per phase (kernel classes summed; the inputs' streams
    # overlap, so these add up to more than the step) and weights per second
    # of the quantize phase alone, U given
    phase_of = {"hessian": "accumulate", "prepare": "prepare", "chol": "prepare",
                "trtri": "prepare", "minpivot": "prepare", "quant": "quantize",
                "chmc": "quantize"}
    phase_ms = {"accumulate": 0.0, "prepare": 0.0, "quantize": 0.0}
    for k, v in breakdown.items():
        ph = phase_of.get(k.split("_")[0])
        if ph:
            phase_ms[ph] += v["ms_per_step"]

    cpu = None
    if (not args.no_cpu_baseline and args.order == "workload" and args.ssqr is None
            and args.hptq is None and args.chmc is None and not args.no_clip):
        sample_rows = args.cpu_sample_rows or 64
        cpu = cpu_baseline(wl, host_inputs, sample_rows)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f64" if any(h.split8 for h in plan) else "f64",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.notes,
                   "layers": [f"{l.name} {l.rows}x{wl.input(l.hessian).dim}" for l in wl.layers],
                   "n_tokens": wl.n_tokens, "token_chunk": wl.token_chunk,
                   "bits": list(wl.bits), "group_size": wl.group_size,
                   "act_order": wl.act_order and args.order == "workload",
                   "clip": not args.no_clip,
                   "order": "min_pivot" if args.order == "min_pivot" else
                   ("act_order" if wl.act_order else "none"),
                   "damp": CHMC_DAMP if args.chmc is not None else wl.damp,
                   "weights_per_step": weights,
                   "hessian": {h.name: ("split8" if h.split8 else "exact") for h in plan},
                   "factor_form": {h.name: h.factor_form for h in plan},
                   "arithmetic": "Hessian: exact fp64 products, or (split8) int8 digit-slice "
                                 "products summed exactly in int32 and combined in fp64; "
                                 "fp64 Cholesky (and, outside the factor form, inverse) and "
                                 "sweep, fp32 MFMA lazy update"},
        "roofline": roofline,
        "ssqr": None if args.ssqr is None else {
            "target": args.ssqr, "iters": args.ssqr_iters, "sweeps_per_search": sweeps,
            "result": {k: [{"bits": r.layer.bits, "alpha": r.alpha,
                            "outlier_fraction": r.n_outliers / r.outlier_mask.numel()}
                           for r in v] for k, v in ssqr_last.items()}},
        "hptq": None if args.hptq is None else {
            "budget_bits_per_weight": args.hptq, "iters": args.ssqr_iters,
            "sweeps_per_search": sweeps,
            "result": {k: [{"alpha": r.alpha, "bits_per_weight": r.bpw} for r in v]
                       for k, v in hptq_last.items()}},
        "chmc": None if args.chmc is None else {
            "bpw_target": args.chmc, "sketch": "seeded Gaussian [in_features x rank]",
            "damp": CHMC_DAMP,
            "layers": [{"layer": name, "bits": b, "rank": q.rank,
                        "bits_per_weight": chmc_bpw(q.codes.shape[0], q.codes.shape[1], q.rank,
                                                    b, q.group_size)}
                       for v in chmc_last.values() for name, b, q in v]},
        "cpu_baseline": cpu,
        "step_repeats": step_repeats,
        "kernels": breakdown,
        "phases_device_ms_per_step": phase_ms,
        "quantize_only_weights_per_s": (weights / (phase_ms["quantize"] / 1000.0)
                                        if phase_ms["quantize"] > 0 else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
