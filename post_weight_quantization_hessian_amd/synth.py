"""Seeded synthetic inputs: layer weights and calibration activations.

This module only draws random numbers and shapes them into the workloads'
input laws; it holds none of the quantizer's arithmetic and is the one piece
of code that both the HIP path's callers and the CPU oracle's callers use, so
that both see the identical bytes.

Input laws (they stand in for real checkpoints and WikiText calibration
activations, which are not available here):

* Weights: iid Student-t (nu = 4) entries, each row rescaled to standard
  deviation 0.02, optional "outlier" input columns multiplied by a factor,
  then rounded to fp16.
* Calibration activations ("cone"): x = a*mu + V (sigma * z) + eps with a
  shared unit mean direction mu, an orthonormal rank-32 basis V with
  sigma_k ~ k^-1/2 (sum sigma_k^2 = 0.8), isotropic noise eps ~ N(0, 0.2/d),
  a = sqrt(c/(1-c)) for a target mean pairwise cosine c = 0.75, then one
  global factor so the mean per-coordinate second moment is 1. Optional
  per-channel log-normal multipliers exp(N(0, sigma^2)); optional SiLU-gated
  product silu(a) * b of two independent cone samples (the input of an MLP
  down projection).

Every tensor is drawn from numpy's PCG64 seeded with
SeedSequence([base_seed, workload_id, tensor_id, chunk_id]); base seed 42.
Token chunks are independent streams, so any chunk can be regenerated alone.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
import zlib

import numpy as np

BASE_SEED = 42
CONE_RANK = 32
CONE_COS = 0.75
CONE_RANK_ENERGY = 0.8
CONE_NOISE_ENERGY = 0.2
GEN_CHUNK = 8192


def _key(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def rng_for(workload: int, tensor: str, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([BASE_SEED, workload, _key(tensor), chunk])
    return np.random.Generator(np.random.PCG64(ss))


def weights(workload: int, tensor: str, rows: int, cols: int, *,
            row_std: float = 0.02, outlier_frac: float = 0.0,
            outlier_mult: float = 20.0) -> np.ndarray:
    """fp16 [rows x cols] weight matrix (Student-t nu=4, row std ``row_std``)."""
    rng = rng_for(workload, tensor)
    W = rng.standard_t(4.0, size=(rows, cols))
    sd = W.std(axis=1, keepdims=True)
    sd[sd == 0] = 1.0
    W = W / sd * row_std
    if outlier_frac > 0:
        k = max(1, int(round(outlier_frac * cols)))
        cols_sel = rng_for(workload, tensor + "/outliers").choice(cols, size=k, replace=False)
        W[:, cols_sel] *= outlier_mult
    return W.astype(np.float16)


def outlier_columns(workload: int, tensor: str, cols: int, outlier_frac: float) -> np.ndarray:
    k = max(1, int(round(outlier_frac * cols)))
    return np.sort(rng_for(workload, tensor + "/outliers").choice(cols, size=k, replace=False))


class ConeSpec:
    """Shared geometry (mean direction, basis, channel multipliers) of one
    activation tensor; token chunks are drawn independently from it."""

    def __init__(self, workload: int, tensor: str, dim: int, *,
                 lognormal_sigma: float = 0.0):
        rng = rng_for(workload, tensor + "/geometry")
        self.dim = dim
        mu = rng.standard_normal(dim)
        self.mu = mu / np.linalg.norm(mu)
        r = min(CONE_RANK, dim)
        V, _ = np.linalg.qr(rng.standard_normal((dim, r)))
        self.V = V
        sig = np.arange(1, r + 1, dtype=np.float64) ** -0.5
        self.sigma = sig * np.sqrt(CONE_RANK_ENERGY / np.sum(sig ** 2))
        self.a = np.sqrt(CONE_COS / (1.0 - CONE_COS))
        total = self.a ** 2 + CONE_RANK_ENERGY + CONE_NOISE_ENERGY
        self.gain = np.sqrt(dim / total)
        if lognormal_sigma > 0:
            self.chan = np.exp(lognormal_sigma * rng.standard_normal(dim))
        else:
            self.chan = None
        self.workload = workload
        self.tensor = tensor

    def chunk(self, chunk_id: int, n: int) -> np.ndarray:
        rng = rng_for(self.workload, self.tensor, chunk_id)
        z = rng.standard_normal((n, self.V.shape[1])) * self.sigma[None, :]
        x = rng.standard_normal((n, self.dim)) * np.sqrt(CONE_NOISE_ENERGY / self.dim)
        x += z @ self.V.T
        x += self.a * self.mu[None, :]
        x *= self.gain
        if self.chan is not None:
            x *= self.chan[None, :]
        return x.astype(np.float32)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def activations(workload: int, tensor: str, n_tokens: int, dim: int, *,
                kind: str = "cone", lognormal_sigma: float = 0.0,
                chunk: int = GEN_CHUNK, threads: int | None = None) -> np.ndarray:
    """fp32 [n_tokens x dim] calibration activations, generated in
    independent token chunks (parallel threads for large tensors)."""
    if kind == "cone":
        specs = [ConeSpec(workload, tensor, dim, lognormal_sigma=lognormal_sigma)]
    elif kind == "silu_gated":
        specs = [ConeSpec(workload, tensor + "/gate", dim, lognormal_sigma=lognormal_sigma),
                 ConeSpec(workload, tensor + "/up", dim, lognormal_sigma=lognormal_sigma)]
    else:
        raise ValueError(kind)
    out = np.empty((n_tokens, dim), dtype=np.float32)
    starts = list(range(0, n_tokens, chunk))

    def work(ci):
        s = starts[ci]
        n = min(chunk, n_tokens - s)
        if kind == "cone":
            out[s:s + n] = specs[0].chunk(ci, n)
        else:
            a = specs[0].chunk(ci, n).astype(np.float64)
            b = specs[1].chunk(ci, n).astype(np.float64)
            out[s:s + n] = (_silu(a) * b).astype(np.float32)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if len(starts) > 1 and threads > 1:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(len(starts))))
    else:
        for ci in range(len(starts)):
            work(ci)
    return out


def mean_pairwise_cosine(X: np.ndarray, sample: int = 512, seed: int = 0) -> float:
    """Mean cosine over distinct pairs of a token subsample (a statistic of
    the generated law, used to check it against the target)."""
    rng = np.random.default_rng(seed)
    idx = rng.choice(X.shape[0], size=min(sample, X.shape[0]), replace=False)
    Y = X[idx].astype(np.float64)
    Y /= np.linalg.norm(Y, axis=1, keepdims=True)
    C = Y @ Y.T
    m = C.shape[0]
    return float((C.sum() - np.trace(C)) / (m * (m - 1)))
