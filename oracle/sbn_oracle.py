"""Plain CPU oracle for the Sparse-BitLinear hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

Every function writes out the plain definition of one step, in numpy (float64
unless noted), so it can be checked by eye against the pages.  The pages are
five web summaries of the paper "Sparse-BitNet: 1.58-bit LLMs are Naturally
Friendly to Semi-Structured Sparsity" (arXiv 2603.05168); they are cited as

  [ja]  gist.science, Japanese summary, section "技術概要" (technical overview)
  [de]  gist.science, German summary, section "Technische Zusammenfassung"
  [ko]  gist.science, Korean summary, section "기술 요약"
  [fr]  gist.science, French summary, section "Résumé technique"
  [abs] fugumt.com paper page, English abstract

followed by the numbered heading inside that section.

The pages give no formulas.  Where they are silent this oracle takes the
readings below (each is repeated at the function that uses it):

  * groups of M run along K, the input dimension, inside one output row;
  * the mask keeps exactly N entries per group, the N largest |w| of the
    master weights; equal magnitudes go to the lower index;
  * one per-tensor scale s_w = mean|W| over ALL master weights (the pages put
    quantization before masking), rounded once to fp32, floored at 1e-5;
  * ternary value = RoundClip(w / s_w, -1, 1), round half to even;
  * activations: per-token absmax to int8 in [-127, 127], decided in fp32 as
    rint((127*x) / a) with a = max(absmax, 1e-5), s_x = a/127 in fp32;
  * Y = s_w * s_x[t] * sum_k Xq[t,k] * Wt[r,k]; as float32, the token's
    scale is rounded once, fl32(s_w * s_x[t]), and each output is one float32
    product of the exact accumulator with it (bf16: that value rounded to
    nearest even);
  * dual STE: identity Jacobians through both quantizers and a dense
    gradient through the mask, so grad_X = dY @ (s_w*Wt) and
    grad_W = dY^T @ (s_x*Xq) covering every (r, k);
  * the two ablation variants ([de] §4 "Ablationsstudien", [fr] §5): the
    mask taken from |q| of the ternary weights (ties to the lower index),
    and grad_W blocked at pruned positions (grad_W * mask);
  * a decode plane (pack_d2, not on the pages): the effective ternary
    weights as one 2-bit code per position, for memory-bound decode;
  * a joint 2:4 code (pack_j6, not on the pages): each group of four
    effective 2:4 weights as one 6-bit code of its two (position, value)
    slots, 1.5 bits per weight, for memory-bound decode;
  * the master-weight optimizer step ([ja] §2.1: BF16 master weights are
    kept and receive the gradients; no optimizer is named): plain SGD,
    w' = bf16(fl32(w - lr*g)) with fl32 one rounding of the exact value
    (a float32 fused multiply-add) and bf16 round-half-to-even.

Tensor conventions: bf16 inputs are ``uint16`` bit patterns, row-major.
W is [R, K] (R output features, K input features), X is [T, K], Y is [T, R].

Packed weight format (the "explicit N:M metadata" the pages ask for):

  meta  plane: per row a K-bit bitstream, bit (g*M + p) set iff position p of
               group g survives; bit b lives in byte b >> 3 at bit b & 7.
               Row stride K/8 bytes.  Not stored when N == M.
  codes plane: per row the survivors' 2-bit codes in increasing k; the j-th
               survivor occupies bits 2j, 2j+1 (same bit order).  00 = 0,
               01 = +1, 11 = -1.  Row stride K*N/(4*M) bytes.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

S_FLOOR = np.float32(1e-5)       # floor of the weight scale and of the token absmax
QMAX = 127                       # symmetric int8 range [-127, 127]

__all__ = [
    "bf16_to_f64", "bf16_to_f32", "nm_mask", "absmean_exact", "round_to_f32",
    "weight_scale", "ternary_codes", "quant_then_mask", "packed_bytes",
    "pack_sbn1", "act_quant", "accumulate", "output", "backward",
    "forward", "S_FLOOR", "QMAX", "nm_mask_ternary", "fma_f32", "f32_to_bf16_rne",
    "sgd_update", "pack_d2", "unpack_d2", "output_f32", "output_bf16",
    "j6_group_code", "j6_group_weights", "pack_j6", "unpack_j6", "j6_bytes",
]


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact widening)."""
    return bf16_to_f32(bits).astype(np.float64)


def _check_finite(bits: np.ndarray) -> None:
    if np.any((np.asarray(bits, dtype=np.uint16) & 0x7F80) == 0x7F80):
        raise ValueError("non-finite bf16 input is outside the operator's contract")


# --------------------------------------------------------------------------- mask
def nm_mask(W_bits: np.ndarray, n: int, m: int) -> np.ndarray:
    """N:M magnitude mask of the master weights.  Returns bool [R, K].

    [de] §2 / [ko] §2.1 / [fr] §2: in every group of M consecutive weights
    the N largest magnitudes of the high-precision master weights are kept;
    [ja] §2.1: the magnitudes are those of the continuous weights before
    quantization.  Groups run along K inside one row.  Equal magnitudes are
    ordered by position, lower index first, which makes the selection unique.

    Definition: sort each group by (|w| descending, index ascending) with a
    stable sort and keep the first N.
    """
    _check_finite(W_bits)
    R, K = W_bits.shape
    assert K % m == 0 and 1 <= n <= m
    mag = np.abs(bf16_to_f64(W_bits)).reshape(R, K // m, m)
    order = np.argsort(-mag, axis=-1, kind="stable")      # stable: ties keep index order
    keep = np.zeros(mag.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :n], True, axis=-1)
    return keep.reshape(R, K)


def nm_mask_ternary(W_bits: np.ndarray, s_w: np.float32, n: int, m: int) -> np.ndarray:
    """Ablation variant of the mask: the N largest |q| of the TERNARY weights.

    [de] §4 ("Ablationsstudien") and [fr] §5 report that building the mask
    from the quantized ternary weights instead of the master weights makes
    training unstable; this is that variant, kept for the comparison.
    |q| is 0 or 1, so most groups hold ties; as in nm_mask, equal keys go
    to the lower index.  q = RoundClip(w / s_w, -1, 1) with the tensor's
    scale s_w (ternary_codes).

    Definition: stable sort each group by |q| descending and keep the first N.
    """
    _check_finite(W_bits)
    R, K = W_bits.shape
    assert K % m == 0 and 1 <= n <= m
    key = np.abs(ternary_codes(W_bits, s_w).astype(np.int64)).reshape(R, K // m, m)
    order = np.argsort(-key, axis=-1, kind="stable")
    keep = np.zeros(key.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :n], True, axis=-1)
    return keep.reshape(R, K)


# --------------------------------------------------------------------------- scale
def absmean_exact(W_bits: np.ndarray) -> Fraction:
    """Exact mean |w| over every entry of W, as a rational number.

    Scale domain: [ja] §2.1, [de] §2, [ko] §2.1 and [fr] §2 all quantize the
    master weights first and apply the mask afterwards, so the scale is taken
    over the whole dense tensor, before masking.  Every bf16 value is an exact
    binary fraction, so the sum is exact: count each magnitude pattern and add
    count * value with rational arithmetic.
    """
    _check_finite(W_bits)
    mag = (np.asarray(W_bits, dtype=np.uint16) & 0x7FFF).reshape(-1)
    counts = np.bincount(mag, minlength=0x8000)
    nz = np.nonzero(counts)[0]
    vals = bf16_to_f64(nz.astype(np.uint16))
    total = sum((Fraction(int(c)) * Fraction(float(v)) for c, v in zip(counts[nz], vals)),
                Fraction(0))
    return total / mag.size


def round_to_f32(q: Fraction) -> np.float32:
    """Nearest float32 to the rational q, ties to even (IEEE round-to-nearest).

    Handles zero, subnormals and overflow to infinity.
    """
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    num, den = a.numerator, a.denominator
    e = num.bit_length() - den.bit_length()          # a in [2^(e-1), 2^(e+1))
    if (num << max(0, -e)) < (den << max(0, e)):      # a < 2^e
        e -= 1                                         # now 2^e <= a < 2^(e+1)
    qe = max(e, -126) - 23                             # exponent of one ulp
    sn, sd = (num, den << qe) if qe >= 0 else (num << (-qe), den)
    k, r = divmod(sn, sd)
    if 2 * r > sd or (2 * r == sd and (k & 1)):
        k += 1
    val = Fraction(k) * (Fraction(2) ** qe)
    fmax = Fraction((1 << 24) - 1) * (Fraction(2) ** (127 - 23))
    out = np.float32(np.inf) if val > fmax else np.float32(float(val))
    return -out if neg else out


def weight_scale(W_bits: np.ndarray) -> np.float32:
    """s_w = max(fp32(mean|W|), 1e-5): one per-tensor absmean scale.

    The pages fix only the ternary set {-1, 0, +1} ([ja] §1, [de] §1,
    [fr] §1); the scale rule is the per-tensor absmean of 1.58-bit BitNet,
    rounded once to fp32 and floored at 1e-5 so that an all-zero tensor
    still has a positive scale.
    """
    s = round_to_f32(absmean_exact(W_bits))
    return np.float32(max(s, S_FLOOR))


# --------------------------------------------------------------------------- ternary
def ternary_codes(W_bits: np.ndarray, s_w: np.float32) -> np.ndarray:
    """RoundClip(w / s_w, -1, 1) with round-half-to-even, over all of W.  int8 [R, K].

    [ja] §1, [de] §1, [ko] §1, [fr] §1: 1.58-bit weights take values in
    {-1, 0, +1}.  The quotient is formed in float64; a bf16 w and an fp32
    s_w are far enough apart from the rounding boundary |w/s| = 1/2 that
    float64 decides it exactly (an exact half rounds to 0).
    """
    w = bf16_to_f64(W_bits)
    t = np.clip(np.rint(w / np.float64(s_w)), -1.0, 1.0)
    return t.astype(np.int8)


def quant_then_mask(W_bits: np.ndarray, n: int, m: int, mask_from: str = "master"):
    """Effective ternary weight W_t = mask (.) Q(W), plus the mask and s_w.

    [ja] §2.1 / [de] §2 / [ko] §2.1 / [fr] §2: quantize first, then apply
    the mask, so the discrete weights used at inference carry the N:M
    structure.  mask_from = "master" (the method) or "ternary" (the ablation
    variant, nm_mask_ternary).  Returns (codes int8 [R,K] with pruned
    entries 0, mask bool [R,K], s_w float32).
    """
    s_w = weight_scale(W_bits)
    q = ternary_codes(W_bits, s_w)
    if mask_from == "master":
        mask = nm_mask(W_bits, n, m)
    elif mask_from == "ternary":
        mask = nm_mask_ternary(W_bits, s_w, n, m)
    else:
        raise ValueError(mask_from)
    return np.where(mask, q, 0).astype(np.int8), mask, s_w


# --------------------------------------------------------------------------- packing
def packed_bytes(R: int, K: int, n: int, m: int):
    """(codes_bytes, meta_bytes) of the packed format for an R x K weight."""
    codes = R * (K // m) * n * 2 // 8
    meta = 0 if n == m else R * K // 8
    return codes, meta


def pack_sbn1(codes: np.ndarray, mask: np.ndarray, n: int, m: int):
    """Pack (mask, ternary codes) into the meta and codes planes.

    [ja] §2.1 / [fr] §2: the quantize-then-mask order yields explicit N:M
    metadata for inference.  The pages do not print a layout; the one used
    here is the per-row bitmap plus 2-bit survivor codes described in this
    module's docstring.
    """
    R, K = codes.shape
    c2 = np.where(codes == 1, 1, np.where(codes == -1, 3, 0)).astype(np.uint8)
    surv = c2[mask].reshape(R, (K // m) * n)            # row by row, increasing k
    bits = np.stack([surv & 1, (surv >> 1) & 1], axis=-1).reshape(R, -1)
    codes_plane = np.packbits(bits, axis=1, bitorder="little")
    if n == m:
        meta_plane = np.zeros((R, 0), dtype=np.uint8)
    else:
        meta_plane = np.packbits(mask.astype(np.uint8), axis=1, bitorder="little")
    return codes_plane, meta_plane


# --------------------------------------------------------------------------- decode plane
def pack_d2(codes: np.ndarray) -> np.ndarray:
    """Decode plane of an effective ternary weight (any N:M; pruned entries 0).

    Not a format of the pages: a byte-lean form for memory-bound decode (at
    6:8 the packed planes hold 2.5 bits per weight, a dense 2-bit ternary
    code 2).  Codes as in pack_sbn1 (00 = 0, 01 = +1, 11 = -1), one per
    position, no bitmap.  Row r is K/16 little-endian 32-bit words; word w
    holds positions 16w .. 16w + 15, position 16w + 4k + b (k, b in 0..3) in
    bits 8b + 6 - 2k (low) and 8b + 7 - 2k (high) -- so that shifting the word
    left by 2k and masking 0xC0C0C0C0 leaves positions 4k .. 4k + 3 as 64 * w,
    one per byte, in order.  Returns uint8 [R, K/4].
    """
    R, K = codes.shape
    assert K % 16 == 0
    c2 = np.where(codes == 1, 1, np.where(codes == -1, 3, 0)).astype(np.uint32)
    c = c2.reshape(R, K // 16, 4, 4)                    # [r, w, k, b]
    shift = 8 * np.arange(4)[None, None, None, :] + 6 - 2 * np.arange(4)[None, None, :, None]
    words = (c << shift.astype(np.uint32)).sum(axis=(2, 3)).astype(np.uint32)   # disjoint bit fields
    return words.astype("<u4").view(np.uint8).reshape(R, K // 4)


def unpack_d2(plane: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of pack_d2: int8 [R, K] ternary weights."""
    words = np.ascontiguousarray(plane[:, : K // 4]).view("<u4").reshape(R, K // 16, 1, 1)
    shift = 8 * np.arange(4)[None, None, None, :] + 6 - 2 * np.arange(4)[None, None, :, None]
    c = (words >> shift.astype(np.uint32)) & 3
    w = np.where(c == 1, 1, np.where(c == 3, -1, 0)).astype(np.int8)
    return w.reshape(R, K)


# --------------------------------------------------------------------------- joint 2:4 code
# Not a format of the pages: a byte-lean form of a 2:4 weight for memory-bound
# decode ([ja] §3.2 and [de] §4 "Geschwindigkeit" report decoding speed; a 2:4
# group of ternary weights has at most two nonzeros, so it is fixed by two
# (position, value) slots).  A group's code is 6 bits, c = nib | h << 4:
#   nib = i1 | i2 << 2, the positions (0..3) of slot 1 and slot 2;
#   if i1 != i2: slot values v1 = -1 if h & 1 else +1, v2 = -1 if h & 2 else +1;
#   if i1 == i2: v1 = 0, +1, -1 for h = 0, 1, 3 (h = 2 is not a code), v2 = 0;
# and the group's weights are v1 at i1 plus v2 at i2.  The canonical code of a
# group (the one pack_j6 writes): two nonzeros at i < j -> nib = i | j << 2
# with their signs in h; one nonzero at p -> nib = p | p << 2, h = 1 (+1) or
# 3 (-1); no nonzero -> c = 0.  33 groups, 33 canonical codes.

def j6_group_code(w4) -> int:
    """Canonical 6-bit code of one group of four effective ternary weights
    (at most two nonzeros)."""
    nz = [p for p in range(4) if w4[p] != 0]
    if len(nz) > 2:
        raise ValueError(f"group {list(w4)} has more than two nonzeros")
    if len(nz) == 2:
        i, j = nz
        h = (1 if w4[i] < 0 else 0) | (2 if w4[j] < 0 else 0)
        return (i | j << 2) | h << 4
    if len(nz) == 1:
        p = nz[0]
        return (p | p << 2) | (1 if w4[p] > 0 else 3) << 4
    return 0


def j6_group_weights(c: int) -> list:
    """The four weights a 6-bit code stands for: v1 at i1 plus v2 at i2."""
    nib, h = c & 15, c >> 4
    i1, i2 = nib & 3, nib >> 2
    w = [0, 0, 0, 0]
    if i1 != i2:
        w[i1] += -1 if h & 1 else 1
        w[i2] += -1 if h & 2 else 1
    else:
        if h == 2:
            raise ValueError(f"code {c:#x} is not a code (equal positions with h = 2)")
        w[i1] += {0: 0, 1: 1, 3: -1}[h]
    return w


def _j6_tables():
    # code of every ternary group (key sum (w_p + 1) * 3^p; -1 where > 2 nonzeros),
    # and the weights of every 6-bit code (a row of 99 where c is not a code)
    code = np.full(81, -1, dtype=np.int16)
    for key in range(81):
        w4 = [(key // 3 ** p) % 3 - 1 for p in range(4)]
        if sum(1 for v in w4 if v) <= 2:
            code[key] = j6_group_code(w4)
    weights = np.full((64, 4), 99, dtype=np.int8)
    for c in range(64):
        try:
            weights[c] = j6_group_weights(c)
        except ValueError:
            pass
    return code, weights


_J6_CODE, _J6_WEIGHTS = _j6_tables()


def j6_bytes(R: int, K: int):
    """(nibble-plane bytes, h-plane bytes) of an R x K weight: K/8 and K/16 per row."""
    return R * K // 8, R * K // 16


def pack_j6(codes: np.ndarray):
    """Joint 2:4 code of an effective 2:4 ternary weight (int8 [R, K], K a
    multiple of 64; every group of 4 with at most two nonzeros).

    Two planes, each row-major with the row strides below:
      nibble plane (K/8 bytes per row): the nib of group g in bits 4(g % 2)
        .. +3 of byte g / 2 -- as 32-bit little-endian words, word v holds
        groups 8v .. 8v + 7 at bits 4(g % 8), the index word of the 2:4
        matrix instruction for those 32 positions;
      h plane (K/16 bytes per row): word u (32-bit little-endian) holds the h
        of groups 16u .. 16u + 15; group 16u + 8b + 2k + o (b, o in 0..1,
        k in 0..3) in byte k at bits 2f, 2f + 1 with f = 2b + o.
    Returns (nibble_plane uint8 [R, K/8], h_plane uint8 [R, K/16]).
    """
    R, K = codes.shape
    assert K % 64 == 0
    key = ((codes.astype(np.int16) + 1).reshape(R, K // 4, 4) * np.array([1, 3, 9, 27], dtype=np.int16)).sum(-1)
    c = _J6_CODE[key]
    if (c < 0).any():
        raise ValueError("a group has more than two nonzeros")
    nib = (c & 15).astype(np.uint8)
    h = (c >> 4).astype(np.uint8)
    nib_plane = nib[:, 0::2] | (nib[:, 1::2] << 4)
    hh = h.reshape(R, K // 64, 2, 4, 2)                  # [r, u, b, k, o]
    f = 2 * np.arange(2)[:, None, None] + np.arange(2)[None, None, :]      # [b, 1, o] -> f = 2b + o
    byte = (hh.astype(np.uint32) << (2 * f)[None, None, :, :, :].astype(np.uint32)).sum(axis=(2, 4))   # [r, u, k]
    h_plane = byte.astype(np.uint8).reshape(R, K // 16)
    return nib_plane, h_plane


def unpack_j6(nib_plane: np.ndarray, h_plane: np.ndarray, R: int, K: int) -> np.ndarray:
    """Inverse of pack_j6 (any valid code, canonical or not): int8 [R, K]."""
    nib = np.stack([nib_plane & 15, nib_plane >> 4], axis=-1).reshape(R, K // 4)
    byte = h_plane.reshape(R, K // 64, 1, 4, 1).astype(np.uint32)          # [r, u, -, k, -]
    f = 2 * np.arange(2)[:, None, None] + np.arange(2)[None, None, :]
    h = (byte >> (2 * f)[None, None, :, :, :].astype(np.uint32)) & 3      # [r, u, b, k, o]
    c = nib.astype(np.int32) | (h.reshape(R, K // 4).astype(np.int32) << 4)
    w = _J6_WEIGHTS[c]
    if (w == 99).any():
        raise ValueError("not a code")
    return w.reshape(R, K).astype(np.int8)


# --------------------------------------------------------------------------- activations
def act_quant(X_bits: np.ndarray):
    """Per-token absmax int8 quantization.  Returns (Xq int8 [T,K], s_x float32 [T]).

    The pages do not describe the activation path.  Reading used: the
    1.58-bit BitNet convention of per-token absmax scaling into [-127, 127]:
    a = max(max_k |x|, 1e-5), q = rint((127*x) / a) (round half to even),
    s_x = a / 127.  The rounding decision is taken in float32, the precision
    the device kernel works in: 127*x is exact for bf16 x, and the quotient is
    one IEEE float32 division.
    """
    _check_finite(X_bits)
    x = bf16_to_f32(X_bits)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    a = np.maximum(amax, S_FLOOR).astype(np.float32)
    num = np.float32(QMAX) * x                          # float32, exact
    q = np.rint(num / a[:, None])                       # float32 IEEE division
    q = np.clip(q, -QMAX, QMAX).astype(np.int8)
    s_x = (a / np.float32(QMAX)).astype(np.float32)     # float32 IEEE division
    return q, s_x


# --------------------------------------------------------------------------- matmul
def accumulate(Xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """acc[t, r] = sum_k Xq[t, k] * Wt[r, k] as exact integers.  int64 [T, R].

    Sparse ternary matmul of the Sparse-BitLinear forward ([ja] §2.1,
    [de] §2).  The float64 matmul is exact here: every product and partial
    sum is an integer of magnitude at most 127*K < 2^53.
    """
    assert Xq.shape[1] == codes.shape[1] and Xq.shape[1] * QMAX < 2 ** 53
    acc = Xq.astype(np.float64) @ codes.astype(np.float64).T
    return acc.astype(np.int64)


def output(acc: np.ndarray, s_w: np.float32, s_x: np.ndarray) -> np.ndarray:
    """Y[t, r] = s_w * s_x[t] * acc[t, r], in float64 (the real value the
    float outputs approximate; tolerances are stated against it)."""
    return acc.astype(np.float64) * (np.float64(s_w) * s_x.astype(np.float64))[:, None]


def output_f32(acc: np.ndarray, s_w: np.float32, s_x: np.ndarray) -> np.ndarray:
    """The float32 output as the operator defines its rounding.  float32 [T, R].

    The pages fix no output precision.  Reading used: the dequantization
    scale of a token is formed once in float32, c[t] = fl32(s_w * s_x[t]),
    and each output is one float32 product y = fl32(fl32(acc) * c[t]).
    fl32(acc) is exact (|acc| <= 127*K < 2^24 for K <= 2^17), so y is fixed
    bit for bit by acc, s_w and s_x: every IEEE float32 multiplication
    rounds to nearest, ties to even.
    """
    assert np.abs(acc).max(initial=0) < 2 ** 24
    c = (np.float32(s_w) * np.asarray(s_x, dtype=np.float32)).astype(np.float32)   # float32 IEEE product
    return (acc.astype(np.float32) * c[:, None]).astype(np.float32)               # float32 IEEE product


def output_bf16(acc: np.ndarray, s_w: np.float32, s_x: np.ndarray) -> np.ndarray:
    """The bf16 output: output_f32 rounded to bf16, nearest, ties to even.
    uint16 bit patterns [T, R]."""
    return f32_to_bf16_rne(output_f32(acc, s_w, s_x))


def backward(dY_bits: np.ndarray, Xq: np.ndarray, s_x: np.ndarray,
             codes: np.ndarray, s_w: np.float32, grad_mask: np.ndarray | None = None):
    """Dual-STE backward.  Returns (grad_X [T,K], grad_W [R,K]) in float64.

    [ja] §2.1, [de] §2, [ko] §2.2, [fr] §2: straight-through estimators
    for the quantizers, and the gradient passes the mask densely so pruned
    master weights are still updated.  With identity Jacobians:
      grad_X = dY @ (s_w * Wt)        (through the sparse ternary weight)
      grad_W = dY^T @ (s_x * Xq)      (every (r, k), masked or not)
    No term for the derivative of s_w or s_x is taken.

    grad_mask (bool [R,K]) selects the ablation variant of [de] §4
    ("Ablationsstudien") and [fr] §5, gradients blocked for pruned weights:
    grad_W is multiplied by the mask.
    """
    dY = bf16_to_f64(dY_bits)
    W_eff = np.float64(s_w) * codes.astype(np.float64)
    X_hat = s_x.astype(np.float64)[:, None] * Xq.astype(np.float64)
    gW = dY.T @ X_hat
    if grad_mask is not None:
        gW = np.where(grad_mask, gW, 0.0)
    return dY @ W_eff, gW


# --------------------------------------------------------------------------- optimizer step
def fma_f32(a, b, c) -> np.ndarray:
    """fl32(a*b + c) for float32 inputs: the exact value rounded ONCE to
    float32, nearest, ties to even (an IEEE fused multiply-add).

    The product of two float32 values is exact in float64; the sum is formed
    in float64 together with its exact rounding error (Knuth's two-sum), so
    the float64 sum s and error e satisfy s + e = a*b + c exactly.  Rounding
    s to float32 is then the correct result unless s lies exactly halfway
    between two float32 values while e is not zero; in that case the exact
    value is on the side of e.  Results outside the float32 range are an
    error (the operator's inputs are finite).
    """
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a64 * b64                                   # exact: 48 significant bits
    s = p + c64
    bv = s - p
    e = (p - (s - bv)) + (c64 - bv)                 # s + e == p + c exactly
    with np.errstate(over="ignore"):
        f = s.astype(np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("float32 overflow in the update")
    # the float32 neighbour of f on the side of s, and the midpoint between them
    toward = np.where(s > f.astype(np.float64), np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    nb = np.nextafter(f, toward)
    mid = (f.astype(np.float64) + nb.astype(np.float64)) * 0.5   # exact in float64
    fix = (s != f.astype(np.float64)) & (s == mid) & (e != 0)
    up = np.maximum(f, nb)
    lo = np.minimum(f, nb)
    return np.where(fix, np.where(e > 0, up, lo), f).astype(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (an
    overflow to infinity is an error: every caller's inputs are finite)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if np.any((r & 0x7F80) == 0x7F80):
        raise ValueError("bf16 overflow")
    return r


def sgd_update(W_bits: np.ndarray, G: np.ndarray, lr) -> np.ndarray:
    """One SGD step on the BF16 master weights.  Returns the new bf16 bits.

    [ja] §2.1: BF16 master weights are kept during optimization and receive
    the (dense, dual-STE) gradients; [ja] §2.1 and [ko] §2.2: the mask is
    recomputed from the updated master weights at every step.  The pages
    name no optimizer; plain SGD is taken:
        w' = bf16(fl32(w - lr * g))
    with lr and g in float32, fl32 one rounding of the exact value (a fused
    multiply-add) and bf16 round-half-to-even.
    """
    _check_finite(W_bits)
    w = bf16_to_f32(W_bits)
    g = np.asarray(G, dtype=np.float32)
    assert g.shape == w.shape and np.all(np.isfinite(g))
    return f32_to_bf16_rne(fma_f32(-np.float32(lr), g, w))


def forward(W_bits: np.ndarray, X_bits: np.ndarray, n: int, m: int) -> dict:
    """All forward intermediates for one Sparse-BitLinear call."""
    codes, mask, s_w = quant_then_mask(W_bits, n, m)
    codes_plane, meta_plane = pack_sbn1(codes, mask, n, m)
    Xq, s_x = act_quant(X_bits)
    acc = accumulate(Xq, codes)
    return dict(codes=codes, mask=mask, s_w=s_w, codes_plane=codes_plane,
                meta_plane=meta_plane, Xq=Xq, s_x=s_x, acc=acc,
                y=output(acc, s_w, s_x))
