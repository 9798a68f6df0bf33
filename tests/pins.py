"""Independent checks used to pin the oracle (plain loops and exact rationals).

Nothing here calls the oracle's own arithmetic: each check recomputes what it
verifies another way (brute-force enumeration, exact ``Fraction`` arithmetic,
bit-by-bit loops, torch autograd) and takes the function under test as an
argument, so ``test_oracle_mutations.py`` can pass in deliberately broken
copies and show that the check fails.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np


def _bf16_value(b: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, decoded from its fields."""
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** (-126 - 7)
    return sign * Fraction(128 + f) * Fraction(2) ** (e - 127 - 7)


def _f32_value(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ------------------------------------------------------------------ mask
def mask_matches_bruteforce(nm_mask, W, n, m) -> bool:
    """For every group: among all n-subsets of maximal exact sum of |w|, the
    lexicographically smallest index tuple must be the kept set."""
    R, K = W.shape
    got = nm_mask(W, n, m)
    for r in range(R):
        for g0 in range(0, K, m):
            mags = [abs(_bf16_value(int(W[r, g0 + p]))) for p in range(m)]
            best = None
            for comb in itertools.combinations(range(m), n):
                s = sum((mags[p] for p in comb), Fraction(0))
                if best is None or s > best[0] or (s == best[0] and comb < best[1]):
                    best = (s, comb)
            kept = tuple(p for p in range(m) if got[r, g0 + p])
            if kept != best[1]:
                return False
    return True


def mask_invariants(nm_mask, W, n, m) -> bool:
    got = nm_mask(W, n, m)
    R, K = W.shape
    mag = (W & 0x7FFF).astype(np.int64).reshape(R, K // m, m)   # |w| order = key order
    keep = got.reshape(R, K // m, m)
    if not (keep.sum(-1) == n).all():
        return False
    if n == m:
        return True
    big = np.where(keep, mag, 1 << 20).min(-1)
    small = np.where(keep, -1, mag).max(-1)
    if not (big >= small).all():
        return False
    # equal magnitudes across the boundary: survivor index must be lower
    for r, g in zip(*np.nonzero(big == small)):
        v = big[r, g]
        idx_keep = [p for p in range(m) if keep[r, g, p] and mag[r, g, p] == v]
        idx_drop = [p for p in range(m) if not keep[r, g, p] and mag[r, g, p] == v]
        if max(idx_keep) > min(idx_drop):
            return False
    return True


# ------------------------------------------------------------------ scale
def is_nearest_f32(round_fn, q: Fraction) -> bool:
    r = round_fn(q)
    if not np.isfinite(r):
        return False
    rf = Fraction(float(r))
    for nb in (np.nextafter(np.float32(r), np.float32(np.inf)),
               np.nextafter(np.float32(r), np.float32(-np.inf))):
        if not np.isfinite(nb):
            continue
        d_r, d_nb = abs(q - rf), abs(q - Fraction(float(nb)))
        if d_r > d_nb:
            return False
        if d_r == d_nb and (int(np.float32(r).view(np.uint32)) & 1):
            return False
    return True


def scale_matches_fsum(weight_scale, W) -> bool:
    """s_w must be the fp32 nearest to the exact mean |w| (floored at 1e-5).

    The exact sum is rebuilt from the bf16 bit fields with Python integers, and
    cross-checked against math.fsum of the float64 magnitudes.
    """
    flat = [int(b) for b in np.asarray(W, dtype=np.uint16).reshape(-1)]
    S = sum((abs(_bf16_value(b)) for b in flat), Fraction(0))
    fs = math.fsum(abs(float(_bf16_value(b))) for b in flat)
    if abs(Fraction(fs) - S) > S * Fraction(1, 2 ** 52):
        return False
    mean = S / len(flat)
    s = weight_scale(W)
    floor = _f32_value(np.float32(1e-5))
    if mean < floor:
        return Fraction(float(s)) == floor
    return is_nearest_f32(lambda _q: s, mean)


# ------------------------------------------------------------------ ternary
def ternary_matches_exact(W, s_w, got) -> bool:
    s = _f32_value(s_w)
    R, K = W.shape
    for r in range(R):
        for k in range(K):
            ratio = _bf16_value(int(W[r, k])) / s
            want = 0 if abs(ratio) <= Fraction(1, 2) else (1 if ratio > 0 else -1)
            if int(got[r, k]) != want:
                return False
    return True


# ------------------------------------------------------------------ packing
def pack_by_loops(codes, mask, n, m):
    R, K = codes.shape
    enc = {0: (0, 0), 1: (1, 0), -1: (1, 1)}
    cplanes, mplanes = [], []
    for r in range(R):
        cbits, mbits = [], []
        for k in range(K):
            mbits.append(1 if mask[r, k] else 0)
            if mask[r, k]:
                cbits.extend(enc[int(codes[r, k])])
        cplanes.append([sum(cbits[8 * i + j] << j for j in range(8)) for i in range(len(cbits) // 8)])
        mplanes.append([sum(mbits[8 * i + j] << j for j in range(8)) for i in range(K // 8)])
    cp = np.array(cplanes, dtype=np.uint8).reshape(R, -1)
    mp = np.array(mplanes, dtype=np.uint8).reshape(R, -1) if n < m else np.zeros((R, 0), np.uint8)
    return cp, mp


def unpack_by_loops(cp, mp, R, K, n, m):
    out = np.zeros((R, K), dtype=np.int8)
    dec = {0: 0, 1: 1, 3: -1}
    for r in range(R):
        j = 0
        for k in range(K):
            keep = True if n == m else bool((int(mp[r, k >> 3]) >> (k & 7)) & 1)
            if keep:
                b = 2 * j
                c = ((int(cp[r, b >> 3]) >> (b & 7)) & 1) | ((((int(cp[r, (b + 1) >> 3]) >> ((b + 1) & 7)) & 1)) << 1)
                out[r, k] = dec[c]
                j += 1
    return out


# ------------------------------------------------------------------ activations
def _round_half_even(q: Fraction) -> int:
    f = math.floor(q)
    d = q - f
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def act_quant_matches_exact(X, Xq, s_x) -> bool:
    """int8 codes equal round-half-even(127*x/a) computed exactly, a = max(absmax, 1e-5);
    s_x is the fp32 nearest to a/127.  When the 1e-5 floor is active (a has a
    24-bit significand) the fp32 quotient may sit on the other side of a half
    step than the exact one, so those rows only need to agree to within 1."""
    floor = _f32_value(np.float32(1e-5))
    T, K = X.shape
    for t in range(T):
        xs = [_bf16_value(int(b)) for b in X[t]]
        amax = max((abs(v) for v in xs), default=Fraction(0))
        a = max(amax, floor)
        for k in range(K):
            want = max(-127, min(127, _round_half_even(Fraction(127) * xs[k] / a)))
            if amax >= floor:
                if int(Xq[t, k]) != want:
                    return False
            elif abs(int(Xq[t, k]) - want) > 1:
                return False
        if not is_nearest_f32(lambda _q: s_x[t], a / 127):
            return False
    return True


# ------------------------------------------------------------------ backward
def backward_by_autograd(W, X, dY, codes, s_w, Xq, s_x, block_mask=None):
    """torch float64 autograd of the straight-through formulation
    w_eff = w + (s_w*Wt - w).detach(), x_hat = x + (s_x*Xq - x).detach().
    With block_mask (the blocked-gradient ablation) the weight path is
    w_eff = M * (w + (s_w*Wt - w).detach()): pruned weights get no gradient."""
    import torch

    def f64(bits):
        return torch.from_numpy((np.asarray(bits, np.uint16).astype(np.uint32) << 16)
                                .view(np.float32).astype(np.float64))

    w = f64(W).requires_grad_(True)
    x = f64(X).requires_grad_(True)
    w_q = float(s_w) * torch.from_numpy(codes.astype(np.float64))
    x_q = torch.from_numpy(s_x.astype(np.float64))[:, None] * torch.from_numpy(Xq.astype(np.float64))
    w_eff = w + (w_q - w).detach()
    if block_mask is not None:
        w_eff = torch.from_numpy(np.asarray(block_mask, dtype=np.float64)) * w_eff
    x_hat = x + (x_q - x).detach()
    y = x_hat @ w_eff.T
    y.backward(f64(dY))
    return x.grad.numpy(), w.grad.numpy()


# ------------------------------------------------------------------ ablation: mask from ternary weights
def mask_ternary_matches_bruteforce(mask_fn, W, s_w, n, m) -> bool:
    """Kept set per group = the lexicographically smallest n-subset among
    those of maximal sum of |q|, q the exact RoundClip(w / s_w) (|q| = 1 iff
    |w| / s_w > 1/2, computed with rationals)."""
    R, K = W.shape
    got = mask_fn(W, s_w, n, m)
    s = _f32_value(s_w)
    for r in range(R):
        for g0 in range(0, K, m):
            qs = [1 if abs(_bf16_value(int(W[r, g0 + p])) / s) > Fraction(1, 2) else 0 for p in range(m)]
            best = None
            for comb in itertools.combinations(range(m), n):
                t = sum(qs[p] for p in comb)
                if best is None or t > best[0] or (t == best[0] and comb < best[1]):
                    best = (t, comb)
            kept = tuple(p for p in range(m) if got[r, g0 + p])
            if kept != best[1]:
                return False
    return True


# ------------------------------------------------------------------ optimizer step
def round_binary(q: Fraction, p: int, emin: int = -126) -> Fraction:
    """Nearest number with a p-bit significand (ties to even significand),
    gradual underflow below 2^emin, for the rational q (no overflow check)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - (p - 1))
    k = a / ulp
    f = k.numerator // k.denominator
    rem = k - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return sign * f * ulp


def fma_matches_exact(fma_fn, a, b, c) -> bool:
    """fma_fn(a, b, c) equals the float32 nearest (ties to even) to the exact a*b + c."""
    got = np.asarray(fma_fn(a, b, c), dtype=np.float32).reshape(-1)
    A, B, C = (np.asarray(v, dtype=np.float32).reshape(-1) for v in (a, b, c))
    A, B, C = np.broadcast_arrays(A, B, C)
    for i in range(got.size):
        exact = _f32_value(A[i]) * _f32_value(B[i]) + _f32_value(C[i])
        if Fraction(float(got[i])) != round_binary(exact, 24):
            return False
    return True


def sgd_matches_exact(sgd_fn, W, G, lr) -> bool:
    """New weight = bf16 nearest (ties even) of the float32 nearest (ties even)
    of the exact w - lr * g, compared as exact values."""
    got = np.asarray(sgd_fn(W, G, lr), dtype=np.uint16)
    lrv = _f32_value(lr)
    for idx in np.ndindex(W.shape):
        exact = _bf16_value(int(W[idx])) - lrv * _f32_value(G[idx])
        want = round_binary(round_binary(exact, 24), 8)
        if _bf16_value(int(got[idx])) != want:
            return False
    return True


# ------------------------------------------------------------------ float outputs
def output_matches_exact(out_f32_fn, out_bf16_fn, acc, s_w, s_x) -> bool:
    """The float32 output is the float32 nearest (ties even) to the exact
    acc * c, where c is the float32 nearest to the exact s_w * s_x[t]; the
    bf16 output is the bf16 nearest (ties even) to that float32 value.  All
    compared as exact rational values."""
    got32 = np.asarray(out_f32_fn(acc, s_w, s_x), dtype=np.float32)
    got16 = np.asarray(out_bf16_fn(acc, s_w, s_x), dtype=np.uint16)
    sw = _f32_value(s_w)
    for t in range(acc.shape[0]):
        c = round_binary(sw * _f32_value(s_x[t]), 24)
        for r in range(acc.shape[1]):
            y = round_binary(Fraction(int(acc[t, r])) * c, 24)
            if Fraction(float(got32[t, r])) != y:
                return False
            if _bf16_value(int(got16[t, r])) != round_binary(y, 8):
                return False
    return True


# ------------------------------------------------------------------ decode plane
def d2_by_loops(codes):
    """Bit-by-bit construction of the decode plane: position 16w + 4k + b of a
    row goes to bits 8b + 6 - 2k (low) and 8b + 7 - 2k (high) of word w."""
    R, K = codes.shape
    enc = {0: 0, 1: 1, -1: 3}
    out = np.zeros((R, K // 4), dtype=np.uint8)
    for r in range(R):
        for w in range(K // 16):
            word = 0
            for k in range(4):
                for b in range(4):
                    word |= enc[int(codes[r, 16 * w + 4 * k + b])] << (8 * b + 6 - 2 * k)
            for i in range(4):
                out[r, 4 * w + i] = (word >> (8 * i)) & 0xFF
    return out


def d2_decode_matches(plane, codes) -> bool:
    """The decode the kernels use: (word << 2k) & 0xC0C0C0C0 holds positions
    4k .. 4k + 3 of the word as 64 * w, one signed byte each, in order."""
    R, K = codes.shape
    for r in range(R):
        for w in range(K // 16):
            word = int.from_bytes(bytes(plane[r, 4 * w: 4 * w + 4]), "little")
            for k in range(4):
                v = ((word << (2 * k)) & 0xC0C0C0C0) & 0xFFFFFFFF
                for b in range(4):
                    byte = (v >> (8 * b)) & 0xFF
                    sv = byte - 256 if byte >= 128 else byte
                    if sv != 64 * int(codes[r, 16 * w + 4 * k + b]):
                        return False
    return True


def j6_by_loops(eff):
    """Bit-by-bit construction of the joint 2:4 code planes from the written
    definition: per group the slots (i1, v1), (i2, v2) -- both nonzeros in
    increasing position, or the one nonzero twice with a zero second value, or
    position 0 with zeros -- then nib = i1 | i2 << 2 at bits 4(g % 2) of byte
    g / 2, and h (slot signs, or the single value's 2-bit code) at bits
    2(2b + o) of byte k of the 16-group word, group 16u + 8b + 2k + o."""
    R, K = eff.shape
    nib_plane = np.zeros((R, K // 8), dtype=np.uint8)
    h_plane = np.zeros((R, K // 16), dtype=np.uint8)
    for r in range(R):
        for g in range(K // 4):
            w = [int(v) for v in eff[r, 4 * g: 4 * g + 4]]
            nz = [p for p in range(4) if w[p] != 0]
            assert len(nz) <= 2
            if len(nz) == 2:
                i1, i2 = nz
                h = (1 if w[i1] < 0 else 0) + (2 if w[i2] < 0 else 0)
            elif len(nz) == 1:
                i1 = i2 = nz[0]
                h = 1 if w[i1] > 0 else 3
            else:
                i1 = i2 = 0
                h = 0
            nib_plane[r, g // 2] |= (i1 | (i2 << 2)) << (4 * (g % 2))
            u, rem = divmod(g, 16)
            b, rem = divmod(rem, 8)
            k, o = divmod(rem, 2)
            h_plane[r, 4 * u + k] |= h << (2 * (2 * b + o))
    return nib_plane, h_plane


def j6_slots_sum(nib_plane, h_plane, R, K):
    """The decode the kernels use, slot by slot: value v1 at i1 plus v2 at i2
    (i1 != i2: both +-1 from the sign bits; i1 == i2: v1 from the 2-bit code,
    v2 = 0).  Returns int8 [R, K]."""
    out = np.zeros((R, K), dtype=np.int8)
    code = {0: 0, 1: 1, 3: -1}
    for r in range(R):
        for g in range(K // 4):
            nib = (int(nib_plane[r, g // 2]) >> (4 * (g % 2))) & 15
            u, rem = divmod(g, 16)
            b, rem = divmod(rem, 8)
            k, o = divmod(rem, 2)
            h = (int(h_plane[r, 4 * u + k]) >> (2 * (2 * b + o))) & 3
            i1, i2 = nib & 3, nib >> 2
            if i1 != i2:
                out[r, 4 * g + i1] += -1 if h & 1 else 1
                out[r, 4 * g + i2] += -1 if h & 2 else 1
            else:
                out[r, 4 * g + i1] += code[h]
    return out
