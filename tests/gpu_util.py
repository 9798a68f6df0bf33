"""Helpers for the GPU parity tests: moving seeded inputs to the device,
reading results back, and the comparison bars.

Comparison bars (the oracle is float64 / exact integer):
  * integer and byte outputs (meta, codes, Xq, int32 accumulators) and the
    scales s_w, s_x: bit-for-bit equal;
  * float32 Y: |y - y_ref| <= 1e-3 * |y_ref|  (y_ref == 0 exactly when acc == 0);
  * bf16 Y: |y - y_ref| <= (2^-8 + 2^-20) * |y_ref|  (one bf16 rounding of an
    fp32 value that is itself within 2^-23 of y_ref; 1e-3 is finer than the
    bf16 grid, so it cannot be asked of a bf16 output);
  * gradients: |g - g_ref| <= 1e-3 * (|A| @ |B|) elementwise, the bound of a
    float32 accumulation of that dot product with inputs rounded once.
"""
from __future__ import annotations

import numpy as np

BF16_REL = 2.0 ** -8 + 2.0 ** -20


def torch():
    import torch as _t
    return _t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(t.bfloat16)


def dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    tt = torch()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_rel(got: np.ndarray, ref: np.ndarray, rel: float, what: str):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = rel * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} bound {bound[tuple(i)]!r}")


def assert_abs_product(got: np.ndarray, ref: np.ndarray, absprod: np.ndarray, what: str, rel: float = 1e-3):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = rel * absprod
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} bound {bound[tuple(i)]!r}")
