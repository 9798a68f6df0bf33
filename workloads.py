"""Seeded synthetic inputs for the Sparse-BitLinear hot path.

Both sides of every parity check (the CPU oracle and the HIP library) are fed
from here, so this module holds none of the method's arithmetic: it only draws
Gaussian numbers, rounds them to bf16 bit patterns and names the workload
shapes.  Every tensor gets its own PCG64 stream, ``default_rng([seed, stream])``,
so draws do not depend on the order in which tensors are requested.

bf16 tensors are returned as ``numpy.uint16`` bit patterns (row-major).

Workloads (shapes follow the pages' setting: Sparse-BitLinear replaces a
linear layer; T = tokens, R = output features, K = input features, the N:M
groups run along K):

  tiny     T=16,   R=256,  K=256,  2:4, fp32 output (parity case, seed 0)
  decode   T in {1,4,16}, R=K=4096, 2:4 and 6:8, bf16 output
  prefill  T=4096, R=6912, K=2560, 2:4, X has 1% outliers scaled x20
  train    T=8192, R=11008, K=4096, 6:8, dY ~ N(0, 1e-2)
  sweep    T=2048, R=K=8192, N:M in {2:4, 4:8, 6:8, 2:8, 1:4, 8:8}
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAM_W = 0
STREAM_X = 1
STREAM_DY = 2
STREAM_OUTLIERS = 3

SIGMA_W = 0.02
SIGMA_X = 1.0
SIGMA_DY = 1e-2


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite Gaussian draws; NaN is kept quiet for completeness.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def gaussian_bf16(shape, sigma: float, seed: int, stream: int) -> np.ndarray:
    """N(0, sigma^2) draws in float32, rounded to bf16 bits."""
    z = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(sigma))


def gaussian_bf16_with_outliers(shape, sigma: float, seed: int, stream: int,
                                frac: float, factor: float,
                                outlier_stream: int = STREAM_OUTLIERS) -> np.ndarray:
    """Gaussian draws where exactly round(frac*numel) distinct entries are scaled
    by ``factor`` before the bf16 rounding."""
    z = rng(seed, stream).standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    n = int(np.prod(shape))
    k = int(round(frac * n))
    pos = rng(seed, outlier_stream).choice(n, size=k, replace=False)
    flat = z.reshape(-1)
    flat[pos] *= np.float32(factor)
    return f32_to_bf16_bits(z)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    R: int
    K: int
    nm: tuple = ((2, 4),)
    out_dtype: str = "bf16"
    outliers: bool = False
    backward: bool = False
    Ts: tuple = field(default=())

    def weights(self, seed: int = 0) -> np.ndarray:
        return gaussian_bf16((self.R, self.K), SIGMA_W, seed, STREAM_W)

    def activations(self, seed: int = 0, T: int | None = None) -> np.ndarray:
        T = self.T if T is None else T
        if self.outliers:
            return gaussian_bf16_with_outliers((T, self.K), SIGMA_X, seed, STREAM_X, 0.01, 20.0)
        return gaussian_bf16((T, self.K), SIGMA_X, seed, STREAM_X)

    def upstream_grad(self, seed: int = 0, T: int | None = None) -> np.ndarray:
        T = self.T if T is None else T
        return gaussian_bf16((T, self.R), SIGMA_DY, seed, STREAM_DY)


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 256, ((2, 4),), "f32"),
    "decode": Workload("decode", 16, 4096, 4096, ((2, 4), (6, 8)), "bf16", Ts=(1, 4, 16)),
    "prefill": Workload("prefill", 4096, 6912, 2560, ((2, 4),), "bf16", outliers=True),
    "train": Workload("train", 8192, 11008, 4096, ((6, 8),), "bf16", backward=True),
    "sweep": Workload("sweep", 2048, 8192, 8192,
                      ((2, 4), (4, 8), (6, 8), (2, 8), (1, 4), (8, 8)), "bf16"),
}
