"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is a small rewrite of one oracle step with one error (a wrong
tie-break, a dropped term, a wrong sign or encoding, the wrong operand).  The
test asserts that the corresponding pin in ``pins.py`` rejects it, so a pin
that passes is known to be sensitive to that class of error.  Mutants live
only here, on the CPU; the oracle itself is never modified.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import pins
from workloads import f32_to_bf16_bits, gaussian_bf16

TIES = np.array([[0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x0000, 0x8000, 0x0000, 0x3C80,
                  0x3F80, 0xBF80, 0x3F80, 0x3D00, 0x0001, 0x8001, 0x0080, 0x0001]], dtype=np.uint16)


def _mask_highest_index_ties(W, n, m):
    R, K = W.shape
    mag = np.abs(O.bf16_to_f64(W)).reshape(R, K // m, m)[..., ::-1]
    order = np.argsort(-mag, axis=-1, kind="stable")[..., :n]
    keep = np.zeros(mag.shape, bool)
    np.put_along_axis(keep, order, True, axis=-1)
    return keep[..., ::-1].reshape(R, K)


def _mask_signed_not_abs(W, n, m):
    R, K = W.shape
    val = O.bf16_to_f64(W).reshape(R, K // m, m)
    order = np.argsort(-val, axis=-1, kind="stable")[..., :n]
    keep = np.zeros(val.shape, bool)
    np.put_along_axis(keep, order, True, axis=-1)
    return keep.reshape(R, K)


def _mask_smallest(W, n, m):
    R, K = W.shape
    mag = np.abs(O.bf16_to_f64(W)).reshape(R, K // m, m)
    order = np.argsort(mag, axis=-1, kind="stable")[..., :n]
    keep = np.zeros(mag.shape, bool)
    np.put_along_axis(keep, order, True, axis=-1)
    return keep.reshape(R, K)


@pytest.mark.parametrize("mutant", [_mask_highest_index_ties, _mask_signed_not_abs, _mask_smallest])
def test_mask_mutants_are_caught(mutant):
    W2 = gaussian_bf16((4, 32), 0.02, seed=1, stream=0)
    caught = (not pins.mask_matches_bruteforce(mutant, TIES, 2, 4)
              or not pins.mask_matches_bruteforce(mutant, W2, 2, 4)
              or not pins.mask_invariants(mutant, W2, 2, 4)
              or not pins.mask_matches_bruteforce(mutant, TIES, 3, 8))
    assert caught


def _scale_survivors_only(W):
    mask = O.nm_mask(W, 2, 4)
    vals = np.abs(O.bf16_to_f64(W))[mask]
    return np.float32(vals.mean())


def _scale_float32_sum(W):
    vals = np.abs(O.bf16_to_f32(W)).reshape(-1)
    acc = np.float32(0)
    for v in vals:                 # sequential float32 accumulation: rounding drift
        acc = np.float32(acc + v)
    return np.float32(max(acc / np.float32(vals.size), np.float32(1e-5)))


def _scale_max_not_mean(W):
    return np.float32(np.abs(O.bf16_to_f64(W)).max())


def _scale_no_floor(W):
    return O.round_to_f32(O.absmean_exact(W))


@pytest.mark.parametrize("mutant", [_scale_survivors_only, _scale_float32_sum, _scale_max_not_mean, _scale_no_floor])
def test_scale_mutants_are_caught(mutant):
    W = gaussian_bf16((128, 128), 0.02, seed=0, stream=0)
    Z = np.zeros((2, 8), np.uint16)
    assert (not pins.scale_matches_fsum(mutant, W)) or (not pins.scale_matches_fsum(mutant, Z))


def _ternary_ge(W, s):
    w = O.bf16_to_f64(W)
    h = float(s) / 2
    return np.where(w >= h, 1, np.where(w <= -h, -1, 0)).astype(np.int8)


def _ternary_half_up(W, s):
    w = O.bf16_to_f64(W) / float(s)
    return np.clip(np.floor(w + 0.5), -1, 1).astype(np.int8)


def _ternary_threshold_s(W, s):
    w = O.bf16_to_f64(W)
    return np.where(w > float(s), 1, np.where(w < -float(s), -1, 0)).astype(np.int8)


@pytest.mark.parametrize("mutant", [_ternary_ge, _ternary_half_up, _ternary_threshold_s])
def test_ternary_mutants_are_caught(mutant):
    s = np.float32(0.25)
    W = f32_to_bf16_bits(np.array([[0.125, -0.125, 0.1259765625, -0.1259765625, 0.2, 0.3]], np.float32))
    assert not pins.ternary_matches_exact(W, s, mutant(W, s))


def _pack_swapped_code_bits(codes, mask, n, m):
    cp, mp = O.pack_sbn1(-codes, mask, n, m)     # sign flipped: +1 <-> -1 encodings
    return cp, mp


def _pack_meta_big_endian(codes, mask, n, m):
    cp, mp = O.pack_sbn1(codes, mask, n, m)
    if n < m:
        mp = np.packbits(mask.astype(np.uint8), axis=1, bitorder="big")
    return cp, mp


@pytest.mark.parametrize("mutant", [_pack_swapped_code_bits, _pack_meta_big_endian])
def test_pack_mutants_are_caught(mutant):
    W = gaussian_bf16((4, 64), 0.02, seed=4, stream=0)
    codes, mask, _ = O.quant_then_mask(W, 2, 4)
    cp, mp = mutant(codes, mask, 2, 4)
    ecp, emp = pins.pack_by_loops(codes, mask, 2, 4)
    assert not (cp.tolist() == ecp.tolist() and mp.tolist() == emp.tolist())


def _aq_reading_reciprocal_multiply(X):
    """The other reading of the activation rounding, q = rint(fl32(x * fl32(127/a))):
    not the one the oracle takes (q = rint((127x)/a), one division), and the
    exact-rational pin tells the two apart."""
    x = O.bf16_to_f32(X)
    a = np.maximum(np.abs(x).max(1), np.float32(1e-5))
    q = np.clip(np.rint(x * (np.float32(127) / a)[:, None]), -127, 127).astype(np.int8)
    return q, (a / np.float32(127)).astype(np.float32)


def _aq_half_away(X):
    x = O.bf16_to_f32(X)
    a = np.maximum(np.abs(x).max(1), np.float32(1e-5))
    v = (np.float32(127) * x) / a[:, None]
    q = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8)
    return q, (a / np.float32(127)).astype(np.float32)


def _aq_scale_128(X):
    x = O.bf16_to_f32(X)
    a = np.maximum(np.abs(x).max(1), np.float32(1e-5))
    q = np.clip(np.rint((np.float32(128) * x) / a[:, None]), -128, 127).astype(np.int8)
    return q, (a / np.float32(128)).astype(np.float32)


@pytest.mark.parametrize("mutant", [_aq_reading_reciprocal_multiply, _aq_half_away, _aq_scale_128])
def test_act_quant_mutants_are_caught(mutant):
    X = f32_to_bf16_bits(np.array([[3.0, 1.5, -1.5, 0.75, 2.0, -1.0, 0.5, 0.25],
                                   [8.0, 4.0, -4.0, 1.5, 3.0, 0.0, 1.0, 2.0],
                                   [2.375, 1.1875, -1.1875, 0.5, 1.0, 2.0, 0.0, 0.25],
                                   [127.0, 62.5, 2.5, -2.5, 0.5, 1.5, -62.5, 0.0]], np.float32))
    q, s = mutant(X)
    assert not pins.act_quant_matches_exact(X, q, s)


def _bwd_masked_grad_w(dY, Xq, s_x, codes, s_w):
    gX, gW = O.backward(dY, Xq, s_x, codes, s_w)
    return gX, np.where(codes != 0, gW, 0.0)


def _bwd_raw_codes_no_scale(dY, Xq, s_x, codes, s_w):
    gX, gW = O.backward(dY, Xq, s_x, codes, s_w)
    return gX / float(s_w), gW


def _bwd_unscaled_activations(dY, Xq, s_x, codes, s_w):
    gX, _ = O.backward(dY, Xq, s_x, codes, s_w)
    return gX, O.bf16_to_f64(dY).T @ Xq.astype(np.float64)


@pytest.mark.parametrize("mutant", [_bwd_masked_grad_w, _bwd_raw_codes_no_scale, _bwd_unscaled_activations])
def test_backward_mutants_are_caught(mutant):
    W = gaussian_bf16((16, 64), 0.02, seed=8, stream=0)
    X = gaussian_bf16((4, 64), 1.0, seed=8, stream=1)
    dY = gaussian_bf16((4, 16), 1e-2, seed=8, stream=2)
    f = O.forward(W, X, 2, 4)
    gX, gW = mutant(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"])
    rX, rW = pins.backward_by_autograd(W, X, dY, f["codes"], f["s_w"], f["Xq"], f["s_x"])
    assert not (np.allclose(gX, rX, rtol=1e-9) and np.allclose(gW, rW, rtol=1e-9))


# ----------------------------------------------------------------- ablation variants
def _mask_ternary_highest_index_ties(W, s_w, n, m):
    R, K = W.shape
    key = np.abs(O.ternary_codes(W, s_w).astype(np.int64)).reshape(R, K // m, m)[..., ::-1]
    order = np.argsort(-key, axis=-1, kind="stable")[..., :n]
    keep = np.zeros(key.shape, bool)
    np.put_along_axis(keep, order, True, axis=-1)
    return keep[..., ::-1].reshape(R, K)


def _mask_ternary_uses_master(W, s_w, n, m):
    return O.nm_mask(W, n, m)


def _mask_ternary_half_scale(W, s_w, n, m):
    return O.nm_mask_ternary(W, np.float32(s_w * 2), n, m)


@pytest.mark.parametrize("mutant", [_mask_ternary_highest_index_ties, _mask_ternary_uses_master,
                                    _mask_ternary_half_scale])
def test_mask_ternary_mutants_are_caught(mutant):
    W = gaussian_bf16((6, 64), 0.02, seed=11, stream=0)
    s_w = O.weight_scale(W)
    assert not all(pins.mask_ternary_matches_bruteforce(mutant, W, s_w, n, m) for n, m in ((2, 4), (6, 8)))


def _bwd_blocked_by_codes(dY, Xq, s_x, codes, s_w, mask):
    return O.backward(dY, Xq, s_x, codes, s_w, grad_mask=(codes != 0))


def _bwd_blocked_not_applied(dY, Xq, s_x, codes, s_w, mask):
    return O.backward(dY, Xq, s_x, codes, s_w)


def _bwd_blocked_inverted(dY, Xq, s_x, codes, s_w, mask):
    return O.backward(dY, Xq, s_x, codes, s_w, grad_mask=~mask)


@pytest.mark.parametrize("mutant", [_bwd_blocked_by_codes, _bwd_blocked_not_applied, _bwd_blocked_inverted])
def test_backward_blocked_mutants_are_caught(mutant):
    W = gaussian_bf16((16, 64), 0.02, seed=13, stream=0)
    X = gaussian_bf16((4, 64), 1.0, seed=13, stream=1)
    dY = gaussian_bf16((4, 16), 1e-2, seed=13, stream=2)
    f = O.forward(W, X, 6, 8)
    gX, gW = mutant(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"], f["mask"])
    rX, rW = pins.backward_by_autograd(W, X, dY, f["codes"], f["s_w"], f["Xq"], f["s_x"], block_mask=f["mask"])
    assert not (np.allclose(gX, rX, rtol=1e-9) and np.allclose(gW, rW, rtol=1e-9))


# ----------------------------------------------------------------- optimizer step
def _fma_double_rounding(a, b, c):
    return (np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)
            + np.asarray(c, np.float32).astype(np.float64)).astype(np.float32)


def _fma_product_rounded(a, b, c):
    p = (np.asarray(a, np.float32) * np.asarray(b, np.float32)).astype(np.float32)
    return (p + np.asarray(c, np.float32)).astype(np.float32)


@pytest.mark.parametrize("mutant", [_fma_double_rounding, _fma_product_rounded])
def test_fma_mutants_are_caught(mutant):
    lr = np.float32(2.0 ** -24 * (1 + 2896 * 2.0 ** -23))
    g = np.float32(-(1 - 2895 * 2.0 ** -23))
    cases = [(-lr, g, np.float32(1.0))]
    # the float32 product rounds away information a fused operation keeps
    # (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 is a float32; the float32 product loses the 2^-24
    cases.append((np.float32(1 + 2.0 ** -12), np.float32(1 + 2.0 ** -12), np.float32(-1.0)))
    assert not all(pins.fma_matches_exact(mutant, a, b, c) for a, b, c in cases)
    assert all(pins.fma_matches_exact(O.fma_f32, a, b, c) for a, b, c in cases)


def _sgd_plus(W, G, lr):
    return O.f32_to_bf16_rne(O.fma_f32(np.float32(lr), G, O.bf16_to_f32(W)))


def _sgd_truncate(W, G, lr):
    v = O.fma_f32(-np.float32(lr), G, O.bf16_to_f32(W))
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _sgd_round_half_up(W, G, lr):
    v = O.fma_f32(-np.float32(lr), G, O.bf16_to_f32(W)).view(np.uint32).astype(np.uint64)
    return ((v + 0x8000) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mutant", [_sgd_plus, _sgd_truncate, _sgd_round_half_up])
def test_sgd_mutants_are_caught(mutant):
    W = gaussian_bf16((8, 40), 0.02, seed=14, stream=0)
    G = np.random.default_rng([14, 5]).standard_normal((8, 40)).astype(np.float32) * np.float32(1e-2)
    # plus an exact tie in the bf16 rounding: 1 + 2^-8 lands halfway between bf16 neighbours
    W = np.concatenate([W, f32_to_bf16_bits(np.full((1, 40), 1.0, np.float32))], axis=0)
    G = np.concatenate([G, np.full((1, 40), -2.0 ** -8, np.float32)], axis=0)
    assert not pins.sgd_matches_exact(mutant, W, G, np.float32(1.0))


# ----------------------------------------------------------------- decode plane
def _d2_position_major(codes):
    R, K = codes.shape
    c2 = np.where(codes == 1, 1, np.where(codes == -1, 3, 0)).astype(np.uint8)
    bits = np.stack([c2 & 1, (c2 >> 1) & 1], axis=-1).reshape(R, -1)
    return np.packbits(bits, axis=1, bitorder="little")          # the packed-plane order, not the decode order


def _d2_swapped_code(codes):
    return O.pack_d2(-codes)


@pytest.mark.parametrize("mutant", [_d2_position_major, _d2_swapped_code])
def test_d2_mutants_are_caught(mutant):
    W = gaussian_bf16((4, 64), 0.02, seed=17, stream=0)
    codes, _, _ = O.quant_then_mask(W, 6, 8)
    plane = mutant(codes)
    assert not (np.array_equal(plane, pins.d2_by_loops(codes)) and pins.d2_decode_matches(plane, codes))


# ------------------------------------------------------------------ float outputs
def _out_one_rounding(acc, s_w, s_x):
    y = acc.astype(np.float64) * np.float64(s_w) * s_x.astype(np.float64)[:, None]
    return y.astype(np.float32)


def _out_scale_acc_first(acc, s_w, s_x):
    y = (acc.astype(np.float32) * np.float32(s_w)).astype(np.float32)
    return (y * s_x.astype(np.float32)[:, None]).astype(np.float32)


def _out_bf16_truncated(acc, s_w, s_x):
    return (O.output_f32(acc, s_w, s_x).view(np.uint32) >> 16).astype(np.uint16)


def _out_bf16_half_up(acc, s_w, s_x):
    u = O.output_f32(acc, s_w, s_x).view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mutant", [_out_one_rounding, _out_scale_acc_first, _out_bf16_truncated,
                                    _out_bf16_half_up])
def test_output_mutants_are_caught(mutant):
    rng = np.random.default_rng(5)
    T, R = 24, 40
    acc = rng.integers(-127 * 4096, 127 * 4096 + 1, size=(T, R))
    acc[:, 0] = 1 << np.arange(T)                   # exact powers of two: bf16 ties of c itself
    s_w = np.float32(1 / 3)
    s_x = (np.float32(1.0) / np.arange(3, 3 + T, dtype=np.float32) / np.float32(127)).astype(np.float32)
    f32_fn, bf16_fn = O.output_f32, O.output_bf16
    if mutant in (_out_one_rounding, _out_scale_acc_first):
        f32_fn = mutant
        bf16_fn = lambda a, s, x: O.f32_to_bf16_rne(mutant(a, s, x))
    else:
        bf16_fn = mutant
    # power-of-two scales: acc = 257, 259, 770, 774 lie exactly half-way between two bf16 values
    acc2 = np.array([[257, 259, -257, 770, 774, 1, -3]])
    p2 = (np.float32(0.5), np.array([2.0 ** -7], dtype=np.float32))
    assert not (pins.output_matches_exact(f32_fn, bf16_fn, acc, s_w, s_x)
                and pins.output_matches_exact(f32_fn, bf16_fn, acc2, *p2))


# ----------------------------------------------------------------- joint 2:4 code
def _j6_h_fields_transposed(eff):
    nib, h = O.pack_j6(eff)
    R, K = eff.shape
    # f = 2o + b instead of 2b + o
    hh = np.zeros_like(h)
    for f_old, f_new in ((0, 0), (1, 2), (2, 1), (3, 3)):
        hh |= ((h >> (2 * f_old)) & 3) << (2 * f_new)
    return nib, hh


def _j6_nibbles_high_first(eff):
    nib, h = O.pack_j6(eff)
    return ((nib << 4) | (nib >> 4)).astype(np.uint8), h


def _j6_pair_sign_bits_swapped(eff):
    return O.pack_j6(_swap_pair_signs(eff))


def _swap_pair_signs(eff):
    # exchanges the two signs of every two-nonzero group (the slot-1 / slot-2 bits swapped)
    out = eff.copy()
    R, K = eff.shape
    for r in range(R):
        for g in range(K // 4):
            w = out[r, 4 * g: 4 * g + 4]
            nz = np.flatnonzero(w)
            if len(nz) == 2:
                w[nz[0]], w[nz[1]] = w[nz[1]], w[nz[0]]
    return out


def _j6_single_minus_as_2(eff):
    nib, h = O.pack_j6(eff)
    R, K = eff.shape
    out = h.copy()
    for g in range(K // 4):
        u, rem = divmod(g, 16)
        b, rem = divmod(rem, 8)
        k, o = divmod(rem, 2)
        f = 2 * b + o
        for r in range(R):
            w = eff[r, 4 * g: 4 * g + 4]
            if np.count_nonzero(w) == 1 and w.min() < 0:
                out[r, 4 * u + k] = (int(out[r, 4 * u + k]) & (0xFF ^ (3 << (2 * f)))) | (2 << (2 * f))
    return nib, out


@pytest.mark.parametrize("mutant", [_j6_h_fields_transposed, _j6_nibbles_high_first, _j6_pair_sign_bits_swapped,
                                    _j6_single_minus_as_2])
def test_j6_mutants_are_caught(mutant):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "j6_row_k64.json")))
    eff = np.array(g["rows"], dtype=np.int8)
    nib, h = mutant(eff)
    assert not (nib.tolist() == g["nib_plane"] and h.tolist() == g["h_plane"])
