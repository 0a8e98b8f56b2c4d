"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws numbers and lays them out; it holds none of the method's
arithmetic (no scale, no rounding to codes, no packing). Both the HIP path
and the CPU oracle receive the same arrays from here.

Recipe (every tensor):
  * a ``numpy.random.Generator`` seeded by
    ``SeedSequence([2026, workload, layer, matrix, role, chunk])`` with role
    0 = weight, 1 = activation, 2 = outlier-channel draw;
  * float32 standard normals times sigma, rows drawn in chunks of
    ``CHUNK_ROWS`` so any row can be regenerated on its own;
  * optional per-input-channel multipliers (the activation/weight outlier
    channels the pages describe: a few fixed channels 10-100x larger);
  * conversion to bf16 with round-to-nearest-even, returned as uint16 bits.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 256
ROLE_WEIGHT, ROLE_ACT, ROLE_OUTLIER = 0, 1, 2


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(workload: int, k: int, count: int, layer: int = 0, matrix: int = 0) -> np.ndarray:
    """Sorted indices of ``count`` distinct input channels, drawn without replacement."""
    if count <= 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng(np.random.SeedSequence([2026, workload, layer, matrix, ROLE_OUTLIER]))
    return np.sort(rng.choice(k, size=count, replace=False))


def normal_bf16(seed: tuple, rows: int, cols: int, sigma: float = 1.0, col_mult=None,
                row_start: int = 0, row_stop: int | None = None, threads: int | None = None) -> np.ndarray:
    """Rows [row_start, row_stop) of a seeded rows x cols N(0, sigma^2) bf16 matrix.

    ``col_mult`` (optional, float32 [cols]) multiplies each column after
    drawing. Any row range gives the same values as the full draw; chunks are
    drawn on ``threads`` worker threads (default: up to 16).
    """
    if row_stop is None:
        row_stop = rows
    out = np.empty((row_stop - row_start, cols), np.uint16)
    c0 = row_start // CHUNK_ROWS
    c1 = (row_stop + CHUNK_ROWS - 1) // CHUNK_ROWS

    def one(c):
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        rng = np.random.default_rng(np.random.SeedSequence([*seed, c]))
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        blk *= np.float32(sigma)
        if col_mult is not None:
            blk *= col_mult[None, :]
        lo, hi = max(r0, row_start), min(r1, row_stop)
        out[lo - row_start:hi - row_start] = f32_to_bf16_bits(blk[lo - r0:hi - r0])

    nthreads = threads or min(16, os.cpu_count() or 1)
    if c1 - c0 <= 1 or nthreads <= 1:
        for c in range(c0, c1):
            one(c)
    else:
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(c0, c1)))
    return out


def normal_bf16_rows(seed: tuple, rows: int, cols: int, idx, sigma: float = 1.0, col_mult=None) -> np.ndarray:
    """Selected rows (any order) of the same seeded matrix as ``normal_bf16``."""
    idx = np.asarray(idx, np.int64)
    out = np.empty((idx.size, cols), np.uint16)
    for c in np.unique(idx // CHUNK_ROWS):
        sel = np.nonzero(idx // CHUNK_ROWS == c)[0]
        blk = normal_bf16(seed, rows, cols, sigma, col_mult, int(c) * CHUNK_ROWS,
                          min(rows, (int(c) + 1) * CHUNK_ROWS))
        out[sel] = blk[idx[sel] - int(c) * CHUNK_ROWS]
    return out


@dataclass(frozen=True)
class Linear:
    name: str
    n: int  # out features
    k: int  # in features


@dataclass
class Workload:
    """One of the five workloads: shapes, quantizer settings and input recipe."""
    index: int
    name: str
    linears: tuple
    layers: int
    bits: int
    symmetric: bool
    group: int
    batches: tuple = (1,)
    w_sigma: float = 0.02
    w_outlier_frac: float = 0.0     # fraction of input channels of W scaled
    w_outlier_mult: float = 1.0
    x_outlier_count: int = 0        # fixed activation outlier channels
    x_outlier_mults: tuple = ()
    tokens: int = 1
    distinct_layers: int = 1        # content-distinct layer sets (rest replicate addresses)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def weight_seed(self, layer: int, matrix: int) -> tuple:
        return (2026, self.index, layer % self.distinct_layers, matrix, ROLE_WEIGHT)

    def act_seed(self, k: int, batch: int) -> tuple:
        return (2026, self.index, k, batch, ROLE_ACT)

    def weight_col_mult(self, layer: int, matrix: int, k: int):
        if self.w_outlier_frac <= 0:
            return None
        cnt = int(round(self.w_outlier_frac * k))
        idx = outlier_channels(self.index, k, cnt, layer % self.distinct_layers, matrix)
        m = np.ones(k, np.float32)
        m[idx] = np.float32(self.w_outlier_mult)
        return m

    def act_col_mult(self, k: int):
        if self.x_outlier_count <= 0:
            return None
        idx = outlier_channels(self.index, k, self.x_outlier_count, layer=0, matrix=1000 + k)
        m = np.ones(k, np.float32)
        m[idx] = np.asarray(self.x_outlier_mults, np.float32)
        return m

    def weight(self, layer: int, matrix: int, rows=None) -> np.ndarray:
        lin = self.linears[matrix]
        seed = self.weight_seed(layer, matrix)
        cm = self.weight_col_mult(layer, matrix, lin.k)
        if rows is None:
            return normal_bf16(seed, lin.n, lin.k, self.w_sigma, cm)
        return normal_bf16_rows(seed, lin.n, lin.k, rows, self.w_sigma, cm)

    def activation(self, k: int, batch: int, rows=None) -> np.ndarray:
        seed = self.act_seed(k, batch)
        cm = self.act_col_mult(k)
        if rows is None:
            return normal_bf16(seed, batch, k, 1.0, cm)
        return normal_bf16_rows(seed, batch, k, rows, 1.0, cm)


LLAMA7B = (Linear("q", 4096, 4096), Linear("k", 4096, 4096), Linear("v", 4096, 4096),
           Linear("o", 4096, 4096), Linear("gate", 11008, 4096), Linear("up", 11008, 4096),
           Linear("down", 4096, 11008))
LLAMA70B = (Linear("q", 8192, 8192), Linear("k", 1024, 8192), Linear("v", 1024, 8192),
            Linear("o", 8192, 8192), Linear("gate", 28672, 8192), Linear("up", 28672, 8192),
            Linear("down", 8192, 28672))

WORKLOADS = {
    "single_4096": Workload(
        index=0, name="single_4096", linears=(Linear("w", 4096, 4096),), layers=1, bits=4,
        symmetric=False, group=128, batches=(1,),
        notes="one 4096x4096 W ~ N(0, 0.02^2), asymmetric INT4 G=128, batch-1 GEMV"),
    "llama7b_decode": Workload(
        index=1, name="llama7b_decode", linears=LLAMA7B, layers=32, bits=4, symmetric=True,
        group=128, batches=(1, 4, 16), w_outlier_frac=0.01, w_outlier_mult=20.0,
        distinct_layers=32,
        notes="Llama-2-7B-shaped 32-layer decode stack, 1% of input channels x20, symmetric INT4"),
    "llama70b_decode": Workload(
        index=2, name="llama70b_decode", linears=LLAMA70B, layers=80, bits=4, symmetric=False,
        group=128, batches=(1,), distinct_layers=1,
        notes="Llama-2-70B-shaped 80-layer batch-1 decode sweep, asymmetric INT4"),
    "prefill70b": Workload(
        index=3, name="prefill70b",
        linears=(Linear("o", 8192, 8192), Linear("gate", 28672, 8192), Linear("down", 8192, 28672)),
        layers=1, bits=4, symmetric=False, group=128, batches=(2048,), x_outlier_count=6,
        x_outlier_mults=(20.0, 28.0, 36.0, 44.0, 52.0, 60.0), tokens=2048,
        notes="M=2048 prefill, 70B-shaped layers, 6 activation channels x20..x60, asymmetric INT4"),
    "smoothquant": Workload(
        index=4, name="smoothquant", linears=(Linear("w", 8192, 8192),), layers=1, bits=8,
        symmetric=True, group=8192, batches=(512,), x_outlier_count=6,
        x_outlier_mults=(50.0,) * 6, tokens=512, extra={"alpha": 0.5},
        notes="SmoothQuant W8A8: X 512x8192 with 6 channels x50, W 8192x8192, alpha 0.5"),
    # AWQ's per-layer scale search: calibration activations with fixed outlier
    # channels (the salient channels the method protects) against the
    # Llama-2-7B layer shapes, asymmetric INT4 G = 128, alpha on a 21-point grid
    "awq7b": Workload(
        index=5, name="awq7b", linears=LLAMA7B, layers=1, bits=4, symmetric=False, group=128,
        batches=(512,), x_outlier_count=41, x_outlier_mults=(20.0,) * 41, tokens=512,
        extra={"n_grid": 20},
        notes="AWQ scale search: X 512 tokens with 41 channels x20, Llama-2-7B layer, asymmetric INT4 G=128"),
}
WORKLOAD_ORDER = ["single_4096", "llama7b_decode", "llama70b_decode", "prefill70b", "smoothquant"]


def tp8_share_weights(wl, layer: int):
    """One GPU's share (rank 0) of an 8-way tensor-parallel 70B layer, as
    bf16 host arrays: q|k|v and gate|up split along n (the first eighth of
    each of q, k, v, gate, up), o and down split along k on 128-aligned
    group boundaries (the first eighth of their input channels)."""
    names = [lin.name for lin in wl.linears]
    idx = {nm: names.index(nm) for nm in names}

    def head(nm):
        lin = wl.linears[idx[nm]]
        return wl.weight(layer, idx[nm], rows=np.arange(lin.n // 8))

    qkv = np.concatenate([head("q"), head("k"), head("v")], 0)
    gu = np.concatenate([head("gate"), head("up")], 0)
    o = wl.weight(layer, idx["o"])
    o = np.ascontiguousarray(o[:, : o.shape[1] // 8])
    down = wl.weight(layer, idx["down"])
    down = np.ascontiguousarray(down[:, : down.shape[1] // 8])
    return [qkv, o, gu, down]
