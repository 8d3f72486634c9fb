"""Seeded synthetic inputs for the FP8 down-projection workloads.

This module only draws random numbers and rounds them to BF16 storage; it
holds none of the method's arithmetic (no activation, scale, cast or GEMM).
Both the CPU oracle and the HIP library receive the same bytes from it.

Every generator uses numpy's PCG64 (``numpy.random.default_rng``) drawn in
float32, then rounds to BF16 with torch's round-to-nearest-even cast.  Large
tensors are drawn in row chunks, chunk ``c`` of stream ``s`` seeded with
``default_rng([s, c])``, so any row range can be regenerated on its own.

Workloads (shapes in row-major storage; the weight is stored [N x K], the
layout of a linear layer's weight):

  tiny      H0 [256 x 512] ~ N(0,1), seed 0; step t input H_t = bf16(H0 * 1.1^t),
            t = 0..3; W [128 x 512] ~ 0.02 N(0,1).
  gpt2      H0 [16384 x 3072] ~ N(0,1), seed 1 (8 sequences x 2048 tokens, MLP
            width 3072, model width 768); H_t = bf16(H0 * sqrt(r_t)), r_0 = 1,
            r_t = r_{t-1} (1 + u_t), u_t ~ U(-0.05, 0.05), so the squared-ReLU
            amax drifts by up to 5% a step; 16 steps; W [768 x 3072] ~ 0.02 N(0,1);
            dY [16384 x 768] with log-normal magnitudes (sigma 3), random signs.
  outlier   64 tensors X_k [4096 x 4096] ~ N(0,1), each with one entry set to
            +-bf16(1e5) = +-99840 at a seeded position, then X_64 = 8 * X_63
            (an 8x jump of the amax).
  fine      H [65536 x 4096] ~ Student-t (nu = 3); W [1024 x 4096] ~ 0.02 N(0,1).
  large     H [65536 x 16384] ~ N(0,1); W [4096 x 16384] ~ 0.02 N(0,1);
            dY [65536 x 4096] with log-normal magnitudes (sigma 3), random signs.

Up-projection inputs (for the quantizer fused into the up-projection's
epilogue): X [M x N] ~ N(0,1) (N is the model width) from seed + 4000, and
W1 [K x N] ~ N(0, 1/N) from seed + 5000, so that X W1^T has the scale of H.

Seeds: H from the workload seed, W from seed + 1000, dY from seed + 2000,
drift / positions / signs from seed + 3000, X from seed + 4000, W1 from
seed + 5000.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, List

import numpy as np
import torch

CHUNK_ROWS = 1024


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round a float32 array to BF16 (torch's RNE cast); return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rows_chunked(stream, rows: int, cols: int, draw: Callable, row0: int = 0,
                  nrows: int | None = None) -> np.ndarray:
    """Rows [row0, row0 + nrows) of a [rows x cols] float32 array drawn in chunks.

    ``stream`` is an int or a tuple of ints; chunk c uses default_rng([*stream, c]).
    """
    stream = list(stream) if isinstance(stream, (tuple, list)) else [stream]
    nrows = rows - row0 if nrows is None else nrows
    out = np.empty((nrows, cols), dtype=np.float32)
    c0 = row0 // CHUNK_ROWS
    c1 = (row0 + nrows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def chunk(c):
        r_lo = c * CHUNK_ROWS
        r_hi = min(rows, r_lo + CHUNK_ROWS)
        rng = np.random.default_rng(stream + [c])
        block = draw(rng, (r_hi - r_lo, cols))
        a = max(r_lo, row0)
        b = min(r_hi, row0 + nrows)
        out[a - row0:b - row0] = block[a - r_lo:b - r_lo]

    # chunks are independent streams, so drawing them on several threads
    # gives the same bytes as drawing them in order
    if c1 - c0 >= 8 and nrows * cols >= (1 << 24):
        with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(chunk, range(c0, c1)))
    else:
        for c in range(c0, c1):
            chunk(c)
    return out


def normal(stream: int, rows: int, cols: int, std: float = 1.0, **kw) -> np.ndarray:
    x = _rows_chunked(stream, rows, cols,
                      lambda g, shp: g.standard_normal(shp, dtype=np.float32), **kw)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def student_t(stream: int, rows: int, cols: int, nu: float = 3.0, **kw) -> np.ndarray:
    x = _rows_chunked(stream, rows, cols,
                      lambda g, shp: g.standard_t(nu, shp).astype(np.float32), **kw)
    return bf16_bits(x)


def signed_lognormal(stream: int, rows: int, cols: int, sigma: float = 3.0, **kw) -> np.ndarray:
    def draw(g, shp):
        mag = g.lognormal(0.0, sigma, shp)
        sign = np.where(g.integers(0, 2, shp, dtype=np.int8) == 1, -1.0, 1.0)
        return (mag * sign).astype(np.float32)

    return bf16_bits(_rows_chunked(stream, rows, cols, draw, **kw))


def scale_bf16(h_bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16(H * fp32(factor)): the float32 product rounded to BF16 by torch."""
    x = (h_bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return bf16_bits(x)


@dataclass
class Workload:
    name: str
    M: int
    K: int
    N: int
    steps: int
    act: str                    # "relu2" or "identity"
    mode: str                   # "tensor" or "group128"
    fmt: str = "e4m3"
    margin: float = 1.25
    initial_amax: float = 1.0
    hist_len: int = 1
    bf16_copy: bool = True
    seed: int = 0
    extra: Dict = field(default_factory=dict)

    # ----------------------------------------------------------- inputs
    def h0(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        if self.name == "fine":
            return student_t(self.seed, self.M, self.K, 3.0, row0=row0, nrows=nrows)
        return normal(self.seed, self.M, self.K, row0=row0, nrows=nrows)

    def step_factors(self) -> List[float]:
        """Per-step multiplier applied to H0 (tiny: 1.1^t; gpt2: sqrt of the drift)."""
        if self.name == "tiny":
            return [1.1 ** t for t in range(self.steps)]
        if self.name == "gpt2":
            rng = np.random.default_rng(self.seed + 3000)
            u = rng.uniform(-0.05, 0.05, self.steps)
            r = [1.0]
            for t in range(1, self.steps):
                r.append(r[-1] * (1.0 + u[t]))
            return [float(np.sqrt(v)) for v in r]
        return [1.0] * self.steps

    def h_step(self, t: int, h0: np.ndarray | None = None) -> np.ndarray:
        h0 = self.h0() if h0 is None else h0
        f = self.step_factors()[t]
        return h0.copy() if f == 1.0 else scale_bf16(h0, f)

    def weight(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        return normal(self.seed + 1000, self.N, self.K, std=0.02, row0=row0, nrows=nrows)

    def up_x(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        """Input X [M x N] of the up-projection (N = model width)."""
        return normal(self.seed + 4000, self.M, self.N, row0=row0, nrows=nrows)

    def up_weight(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        """Up-projection weight W1 [K x N], std 1/sqrt(N)."""
        return normal(self.seed + 5000, self.K, self.N, std=float(self.N) ** -0.5, row0=row0,
                      nrows=nrows)

    def da(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        """Gradient dA [M x K] of the activation (the dgrad GEMM's output shape):
        signed log-normal, sigma 1."""
        return signed_lognormal(self.seed + 6000, self.M, self.K, 1.0, row0=row0, nrows=nrows)

    def dy(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        return signed_lognormal(self.seed + 2000, self.M, self.N, 3.0, row0=row0, nrows=nrows)

    # ----------------------------------------------------------- accounting
    def quant_bytes_per_elem(self) -> float:
        """Algorithmic HBM bytes per element of the fused quantizer: read 2 (BF16),
        write 2 (BF16 copy, when kept) + 1 (FP8), plus 4 per 128 for group scales."""
        b = 2.0 + (2.0 if self.bf16_copy else 0.0) + 1.0
        if self.mode == "group128":
            b += 4.0 / 128.0
        return b

    def gemm_flops(self) -> int:
        return 2 * self.M * self.N * self.K


def outlier_tensor(k: int, seed: int = 2, rows: int = 4096, cols: int = 4096) -> np.ndarray:
    """X_k of the outlier workload (k = 0..64); X_64 = 8 * X_63 exactly."""
    if k == 64:
        x = outlier_tensor(63, seed, rows, cols)
        return scale_bf16(x, 8.0)
    h = normal((seed, k), rows, cols)
    rng = np.random.default_rng([seed + 3000, k])
    pos = int(rng.integers(0, rows * cols))
    sign = 1.0 if rng.integers(0, 2) == 0 else -1.0
    flat = h.reshape(-1)
    flat[pos] = bf16_bits(np.array([sign * 1e5], dtype=np.float32))[0]
    return h


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", M=256, K=512, N=128, steps=4, act="relu2", mode="tensor", seed=0),
    "gpt2": Workload("gpt2", M=16384, K=3072, N=768, steps=16, act="relu2", mode="tensor", seed=1),
    "outlier": Workload("outlier", M=4096, K=4096, N=0, steps=65, act="identity", mode="tensor",
                        bf16_copy=False, seed=2),
    "fine": Workload("fine", M=65536, K=4096, N=1024, steps=1, act="identity", mode="group128",
                     margin=1.0, bf16_copy=False, seed=3),
    "large": Workload("large", M=65536, K=16384, N=4096, steps=2, act="relu2", mode="tensor",
                      seed=4),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
