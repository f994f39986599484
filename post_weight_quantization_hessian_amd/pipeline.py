"""One calibration input and the layers that read it, end to end on the GPU.

Holds every device buffer the three library calls need (the Hessian, the
workspaces, the act-order permutation, the factor U and one output set per
bit width), allocated once, and enqueues the whole hot path asynchronously
on the current stream:

    S  = sum over token chunks of X_c^T X_c        (first chunk overwrites S;
         exact fp64 products, or int8 digit slices on the matrix cores)
    perm, U = factor of the damped, act-ordered inverse Hessian
    codes, scales, zeros, g_idx, row_loss          for every bit width

Layers that read the same input are quantized together by stacking their
weight rows. Argument marshalling only: every step runs in the HIP library.
"""
from __future__ import annotations

from . import gptq as G

# The CHMC article's quantization damps the Hessian of the residual's GPTQ
# step with 0.05 (Anhang A, "dampening 0.05"; the same lambda as the
# activation energies of Schritt 1).
CHMC_DAMP = 0.05

# "auto" takes the int8 digit-slice Hessian from this many input features on
# (measured faster from 256 features at 2048 tokens; below, a handful of
# tiles, either is a few microseconds)
SPLIT8_MIN_DIM = 256

# "auto" sweeps in the factor form (no triangular inverse beyond the 128-wide
# diagonal blocks) from 768 features on. Measured per step, factor form
# against U: 70B-shape 599 against 722 ms, TinyLlama block 12.10 against
# 12.58 ms, Qwen MLP 4.82 against 5.34 ms; the 576-feature layer (five
# launch-bound panels) 0.517 against 0.502 ms, so smaller layers take U.
FACTOR_FORM_MIN_DIM = 768


def factor_form_mode(mode, dim):
    """True | False | 'auto' -> True when the plain sweep takes the factor form."""
    if mode == "auto":
        return dim >= FACTOR_FORM_MIN_DIM
    return bool(mode)


def hessian_mode(mode, dim):
    """'exact' | 'split8' | 'auto' -> True when the layer uses split8."""
    if mode == "auto":
        return dim >= SPLIT8_MIN_DIM
    if mode not in ("exact", "split8"):
        raise ValueError(f"hessian mode {mode!r}")
    return mode == "split8"


def torch_empty_bytes(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class LayerGroup:
    def __init__(self, dim, rows, *, max_chunk_tokens, bits, group_size, act_order, damp,
                 device, min_pivot=False, hessian="exact", clip=True, factor_form="auto"):
        import torch
        self.dim, self.rows = int(dim), int(rows)
        self.bits, self.group_size = tuple(bits), int(group_size)
        self.act_order, self.damp = bool(act_order), float(damp)
        self.min_pivot = bool(min_pivot)  # the min-pivot order instead of act-order
        self.clip = bool(clip)  # False: the no-clipping sweep (codes may leave [0, maxq])
        # the plain sweep in the factor form (U's diagonal blocks and the factor
        # of H beyond them), and so does the CHMC residual sweep; SSQR and HPTQ
        # take U itself
        self.factor_form = factor_form_mode(factor_form, self.dim)
        if self.min_pivot:
            self.act_order = False
        ng = -(-self.dim // self.group_size)
        self.S = torch.empty((self.dim, self.dim), dtype=torch.float64, device=device)
        self._swept = False  # quantize workspaces hold a status once enqueue ran
        self.split8 = hessian_mode(hessian, self.dim)
        hb = (G.hessian_split8_workspace_bytes if self.split8 else G.hessian_workspace_bytes)(
            self.dim, max_chunk_tokens)
        self.hws = torch.empty(max(hb, 1), dtype=torch.uint8, device=device)
        self.pws = torch.empty(G.prepare_workspace_bytes(self.dim), dtype=torch.uint8,
                               device=device)
        self.perm = torch.empty(self.dim, dtype=torch.int32, device=device)
        self.U = torch.empty((self.dim, self.dim), dtype=torch.float32, device=device)
        # one quantize workspace per bit width: each call clears the status
        # word of its workspace, and the statuses are read after the last call
        self.qws = [torch.empty(G.quantize_workspace_bytes(self.rows, self.dim, self.group_size),
                                dtype=torch.uint8, device=device) for _ in self.bits]
        self.outs = [G.QuantizedLayer(
            torch.empty((self.rows, self.dim), dtype=torch.uint8, device=device),
            torch.empty((self.rows, ng), dtype=torch.float16, device=device),
            torch.empty((self.rows, ng), dtype=torch.float16, device=device),
            torch.empty(self.dim, dtype=torch.int32, device=device),
            torch.empty(self.rows, dtype=torch.float64, device=device), b, self.group_size)
            for b in self.bits]

    def _factor(self, chunks, factor_form=False):
        n = 0
        self.n = 0
        for ci, c in enumerate(chunks):
            G.hessian_accumulate(self.S, c, workspace=self.hws, overwrite=(ci == 0),
                                 split8=self.split8)
            n += int(c.shape[0])
        self.n = n
        G.prepare_hinv(self.S, n, damp=self.damp, act_order=self.act_order,
                       workspace=self.pws, out=(self.perm, self.U), sync=False,
                       min_pivot=self.min_pivot, factor_form=factor_form)

    def enqueue(self, chunks, W):
        """The whole path for token chunks ``chunks`` (fp32 [n_c x dim] each)
        and stacked fp16 weights ``W`` [rows x dim], without synchronizing.
        The sweep runs in the factor form (no inverse of the factor beyond
        its 128-wide diagonal blocks) when ``factor_form`` says so. The bit
        widths run one after the other on the current stream (a side stream
        per extra bit width measured 599 -> 606 ms per 70B-shape step)."""
        self._factor(chunks, factor_form=self.factor_form)
        self._swept = True
        for bi, b in enumerate(self.bits):
            G.quantize_layer(W, self.U, self.perm if (self.act_order or self.min_pivot) else None,
                             bits=b,
                             group_size=self.group_size, workspace=self.qws[bi],
                             out=self.outs[bi], sync=False, clip=self.clip,
                             factor_form=self.factor_form)
        return self.outs

    def ssqr(self, chunks, W, target, iters=12):
        """Hessian and factor as in enqueue, then at every bit width the SSQR
        search for a target outlier fraction (synchronous: every probe reads
        its outlier count). Returns one SSQRLayer per bit width."""
        self._factor(chunks)
        perm = self.perm if (self.act_order or self.min_pivot) else None
        return [G.ssqr_search(W, self.U, perm, bits=b, group_size=self.group_size,
                              target=target, iters=iters) for b in self.bits]

    def hptq(self, chunks, W, budget, iters=12):
        """Hessian and factor as in enqueue, then at every bit width the HPTQ
        search for a bits-per-weight budget (synchronous). Returns one
        HPTQLayer per bit width."""
        self._factor(chunks)
        perm = self.perm if (self.act_order or self.min_pivot) else None
        return [G.hptq_search(W, self.U, perm, bits=b, group_size=self.group_size,
                              budget=budget, iters=iters) for b in self.bits]

    def chmc(self, chunks, W, layers, bpw, omega, damp=CHMC_DAMP):
        """Hessian, then the factor of H damped with ``damp`` (the CHMC
        article's 0.05 by default), then the CHMC layer (CHMC article,
        Methodik, Schritt 1-3) for each layer of the stack ``W`` (``layers``:
        (name, rows) in stacking order) and bit width, the rank from the budget
        ``bpw``, without synchronizing. The CHMC calls run on a side stream
        forked once S is complete: their frontends (which need only diag S and
        W) overlap with the factorization, and their sweeps wait for U. The
        outputs live in buffers of this group (one set per layer and bit
        width, reused by later calls). Returns [(name, bits, CHMCLayer)]."""
        import torch
        n = 0
        for ci, c in enumerate(chunks):
            G.hessian_accumulate(self.S, c, workspace=self.hws, overwrite=(ci == 0),
                                 split8=self.split8)
            n += int(c.shape[0])
        self.n = n
        main = torch.cuda.current_stream()
        if not hasattr(self, "cstream"):
            self.cstream = torch.cuda.Stream(device=W.device)
            self.cws = {}
            self.couts = {}
        fork = torch.cuda.Event()
        fork.record(main)
        G.prepare_hinv(self.S, n, damp=damp, act_order=self.act_order,
                       workspace=self.pws, out=(self.perm, self.U), sync=False,
                       min_pivot=self.min_pivot, factor_form=self.factor_form)
        perm = self.perm if (self.act_order or self.min_pivot) else None
        out, r0 = [], 0
        with torch.cuda.stream(self.cstream):
            self.cstream.wait_event(fork)
            for name, rows in layers:
                for b in self.bits:
                    r = G.chmc_rank(rows, self.dim, b, self.group_size, bpw)
                    key = (name, b, r)
                    if key not in self.cws:
                        self.cws[key] = torch_empty_bytes(
                            G.chmc_workspace_bytes(rows, self.dim, r), W.device)
                        self.couts[key] = G.chmc_outputs(rows, self.dim, r, b, self.group_size,
                                                         W.device)
                    G.chmc_layer(W[r0:r0 + rows], self.S, self.n, self.U, perm, omega, rank=r,
                                 bits=b, group_size=self.group_size, bpw_target=bpw,
                                 sync=False, workspace=self.cws[key], u_stream=main,
                                 out=self.couts[key], factor_form=self.factor_form)
                    out.append((name, b, self.couts[key]))
                r0 += rows
            join = torch.cuda.Event()
            join.record(self.cstream)
        main.wait_event(join)
        return out

    def check(self):
        """Synchronize and raise GPTQError if prepare or quantize reported one
        (a non-SPD Hessian, non-finite values, an invalid permutation)."""
        G.workspace_status(self.pws)
        for ws in getattr(self, "cws", {}).values():
            G.workspace_status(ws)
        if self._swept:  # (the SSQR search checks its own sweeps)
            for ws in self.qws:
                G.workspace_status(ws)
