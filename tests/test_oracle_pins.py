"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test compares the oracle with a hand-derived worked example, a brute-force
enumeration, a closed form, an invariant, a library routine or exact rational
arithmetic.  ``tests/test_oracle_mutations.py`` plants plausible mistakes in
copies of the oracle functions and shows that these checks catch them.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle as O
from workloads import f32_to_bf16_bits, gaussian_bf16, bf16_bits_to_f32
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HSET = settings(max_examples=60, derandomize=True, deadline=None,
                suppress_health_check=[HealthCheck.too_slow])


def f32_bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).reshape(1).view(np.uint32)[0])


# ----------------------------------------------------------------- worked example
def test_worked_example_1x8():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_1x8.json")))
    n, m = g["n"], g["m"]
    W = f32_to_bf16_bits(np.array([g["W"]], dtype=np.float32))
    X = f32_to_bf16_bits(np.array([g["X"]], dtype=np.float32))
    e = g["expect"]
    f = O.forward(W, X, n, m)
    assert f32_bits(f["s_w"]) == int(e["s_w_bits"], 16)
    assert f["mask"].astype(int).tolist() == [e["mask"]]
    assert O.ternary_codes(W, f["s_w"]).tolist() == [e["ternary_all"]]
    assert f["codes"].tolist() == [e["effective"]]
    assert f["meta_plane"].tolist() == [[int(b, 16) for b in e["meta_bytes"]]]
    assert f["codes_plane"].tolist() == [[int(b, 16) for b in e["codes_bytes"]]]
    assert f["Xq"].tolist() == [e["Xq"]]
    assert f32_bits(f["s_x"][0]) == int(e["s_x_bits"], 16)
    assert int(f["acc"][0, 0]) == e["acc"]
    # the float outputs, derived by hand with the token scale rounded once
    c = np.float32(f["s_w"]) * f["s_x"]
    assert f32_bits(c[0]) == int(e["scale_bits"], 16)
    assert f32_bits(O.output_f32(f["acc"], f["s_w"], f["s_x"])[0, 0]) == int(e["y_f32_bits"], 16)
    assert int(O.output_bf16(f["acc"], f["s_w"], f["s_x"])[0, 0]) == int(e["y_bf16_bits"], 16)
    # exact real value -51/127; the oracle applies the fp32 s_x (8/127 rounded),
    # so the two differ by at most that one fp32 rounding
    exact = Fraction(e["y_num"], e["y_den"])
    assert abs(Fraction(float(f["y"][0, 0])) - exact) <= abs(exact) * Fraction(1, 2 ** 23)


# ----------------------------------------------------------------- mask
# small bf16 alphabet: forces ties, +-0, subnormals and all-zero groups
ALPHABET = [0x0000, 0x8000, 0x0001, 0x8001, 0x3C00, 0xBC00, 0x3C80, 0xBC80,
            0x3D00, 0x3F80, 0xBF80, 0x3F81, 0x4000, 0x0080]


@st.composite
def small_w(draw, rows=(1, 3), groups=(1, 4)):
    m = draw(st.sampled_from([4, 8]))
    n = draw(st.integers(1, m))
    R = draw(st.integers(*rows))
    G = draw(st.integers(*groups))
    vals = draw(st.lists(st.sampled_from(ALPHABET), min_size=R * G * m, max_size=R * G * m))
    return np.array(vals, dtype=np.uint16).reshape(R, G * m), n, m


@HSET
@given(small_w())
def test_mask_matches_bruteforce_enumeration(case):
    W, n, m = case
    assert pins.mask_matches_bruteforce(O.nm_mask, W, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (3, 4), (4, 4), (2, 8), (4, 8), (6, 8), (8, 8), (3, 8)])
def test_mask_invariants_gaussian(n, m):
    W = gaussian_bf16((64, 512), 0.02, seed=7, stream=0)
    assert pins.mask_invariants(O.nm_mask, W, n, m)


def test_mask_dense_control_is_all_ones():
    W = gaussian_bf16((8, 64), 0.02, seed=1, stream=0)
    assert O.nm_mask(W, 8, 8).all() and O.nm_mask(W, 4, 4).all()


def test_mask_recovers_support_of_distinct_nonzeros():
    rng = np.random.default_rng(3)
    for n, m in [(2, 4), (6, 8), (1, 4), (2, 8)]:
        R, G = 5, 16
        vals = np.zeros((R, G, m), dtype=np.float32)
        support = np.zeros((R, G, m), dtype=bool)
        for r in range(R):
            for gi in range(G):
                pos = rng.choice(m, size=n, replace=False)
                mags = rng.choice(np.arange(1, 60), size=n, replace=False).astype(np.float32) / 64
                sgn = rng.choice([-1.0, 1.0], size=n).astype(np.float32)
                vals[r, gi, pos] = mags * sgn
                support[r, gi, pos] = True
        W = f32_to_bf16_bits(vals.reshape(R, G * m))
        assert (O.nm_mask(W, n, m) == support.reshape(R, G * m)).all()


# ----------------------------------------------------------------- scale
def test_round_to_f32_agrees_with_numpy_cast_on_doubles():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                         np.ldexp(rng.integers(1, 2 ** 30, 500).astype(np.float64), -150),
                         [1e-45, 1.4e-45, 7e-46, 3.4028235e38, 3.4028236e38, 1e39, -2.5e-40]])
    for x in xs:
        assert O.round_to_f32(Fraction(float(x))) == np.float32(x) or (
            np.isinf(np.float32(x)) and np.isinf(O.round_to_f32(Fraction(float(x)))))


@HSET
@given(st.integers(1, 2 ** 80), st.integers(1, 2 ** 60))
def test_round_to_f32_is_nearest_ties_even(num, den):
    assert pins.is_nearest_f32(O.round_to_f32, Fraction(num, den))


def test_round_to_f32_exact_ties():
    # 1 + 2^-24 is half-way between 1 and 1 + 2^-23 -> even (1.0)
    assert O.round_to_f32(Fraction(2 ** 24 + 1, 2 ** 24)) == np.float32(1.0)
    # 1 + 3*2^-24 is half-way between 1+2^-23 and 1+2^-22 -> even (1+2^-22)
    assert O.round_to_f32(Fraction(2 ** 24 + 3, 2 ** 24)) == np.float32(1 + 2 ** -22)
    assert O.round_to_f32(Fraction(-(2 ** 24 + 3), 2 ** 24)) == np.float32(-(1 + 2 ** -22))


def test_scale_closed_form_full_tiny_weight():
    W = gaussian_bf16((256, 256), 0.02, seed=0, stream=0)
    assert pins.scale_matches_fsum(O.weight_scale, W)


@HSET
@given(small_w(rows=(1, 4), groups=(1, 8)))
def test_scale_closed_form_small(case):
    W, _, _ = case
    assert pins.scale_matches_fsum(O.weight_scale, W)


def test_scale_gaussian_statistic():
    # E|w| for N(0, s^2) is s*sqrt(2/pi) = 0.015957691 at s = 0.02
    W = gaussian_bf16((1024, 1024), 0.02, seed=5, stream=0)
    assert abs(float(O.weight_scale(W)) - 0.02 * math.sqrt(2 / math.pi)) < 2e-4


def test_scale_floor_for_zero_weights():
    W = np.zeros((4, 16), dtype=np.uint16)
    assert O.weight_scale(W) == np.float32(1e-5)


# ----------------------------------------------------------------- ternary
def test_ternary_exact_boundaries():
    # scale 0.25 exactly: four entries of 0.25 give sum 1, mean over 4 = 0.25.
    # half scale is 0.125: |w| = 0.125 -> 0 (exact half, rounds to even 0)
    s = np.float32(0.25)
    vals = np.array([[0.125, -0.125, 0.1259765625, -0.1259765625, 0.12451171875, 0.375, -0.375, 1.0,
                      0.0, -0.0, 1e-30, 0.25]], dtype=np.float32)
    W = f32_to_bf16_bits(vals)
    got = O.ternary_codes(W, s)
    assert pins.ternary_matches_exact(W, s, got)
    assert got.tolist() == [[0, 0, 1, -1, 0, 1, -1, 1, 0, 0, 0, 1]]


@HSET
@given(small_w(rows=(1, 3), groups=(1, 6)))
def test_ternary_matches_exact_rational(case):
    W, n, m = case
    s = O.weight_scale(W)
    assert pins.ternary_matches_exact(W, s, O.ternary_codes(W, s))


def test_ternary_zero_fraction_gaussian_closed_form():
    # P(|w| <= E|w|/2) for Gaussian w = 2*Phi(sqrt(2/pi)/2) - 1 = 0.31010...
    W = gaussian_bf16((1024, 2048), 0.02, seed=9, stream=0)
    q = O.ternary_codes(W, O.weight_scale(W))
    phi = 0.5 * (1 + math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2)))
    assert abs((q == 0).mean() - (2 * phi - 1)) < 3e-3


def test_quant_then_mask_uses_dense_scale():
    W = gaussian_bf16((16, 64), 0.02, seed=2, stream=0)
    codes, mask, s_w = O.quant_then_mask(W, 2, 4)
    assert s_w == O.weight_scale(W)                      # scale over all of W
    full = O.ternary_codes(W, s_w)
    assert (codes == np.where(mask, full, 0)).all()
    assert (codes[~mask] == 0).all()


# ----------------------------------------------------------------- packing
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (3, 4), (4, 4), (2, 8), (4, 8), (6, 8), (8, 8)])
def test_pack_matches_bitwise_loop(n, m):
    W = gaussian_bf16((6, 64), 0.02, seed=n * 10 + m, stream=0)
    codes, mask, _ = O.quant_then_mask(W, n, m)
    cp, mp = O.pack_sbn1(codes, mask, n, m)
    ecp, emp = pins.pack_by_loops(codes, mask, n, m)
    assert cp.tolist() == ecp.tolist() and mp.tolist() == emp.tolist()
    assert (cp.nbytes, mp.nbytes) == O.packed_bytes(6, 64, n, m)
    assert (pins.unpack_by_loops(cp, mp, 6, 64, n, m) == codes).all()


# ----------------------------------------------------------------- activations
def test_act_quant_integer_identity():
    rng = np.random.default_rng(4)
    X = rng.integers(-127, 128, size=(8, 64)).astype(np.float32)
    X[:, 5] = 127.0
    Xq, s_x = O.act_quant(f32_to_bf16_bits(X))
    assert (Xq == X).all() and (s_x == np.float32(1.0)).all()


@HSET
@given(st.lists(st.sampled_from(ALPHABET + [0x3F40, 0xBF40, 0x4040, 0x42FE, 0x3DFF, 0x0100, 0x3727]),
                min_size=64, max_size=64), st.integers(1, 4))
def test_act_quant_decision_equals_exact_rational(vals, rows):
    X = np.array((vals * rows)[: 64 * rows], dtype=np.uint16).reshape(rows, 64)
    Xq, s_x = O.act_quant(X)
    assert pins.act_quant_matches_exact(X, Xq, s_x)


def test_act_quant_gaussian_with_outliers_matches_exact():
    from workloads import gaussian_bf16_with_outliers
    X = gaussian_bf16_with_outliers((32, 256), 1.0, 0, 1, 0.01, 20.0)
    Xq, s_x = O.act_quant(X)
    assert pins.act_quant_matches_exact(X, Xq, s_x)


def test_act_quant_half_ties_go_to_even():
    # a = 8: x*127/8 for x = 4 is 63.5 -> 64; x = 12/... construct 0.5 ties directly
    X = f32_to_bf16_bits(np.array([[4.0, 8.0, -4.0, 1.5, 3.0]], dtype=np.float32))
    Xq, _ = O.act_quant(X)
    # 127*4/8 = 63.5 -> 64 ; -63.5 -> -64 ; 127*1.5/8 = 23.8125 -> 24 ; 127*3/8 = 47.625 -> 48
    assert Xq.tolist() == [[64, 127, -64, 24, 48]]
    # a = 3: 1.5*127/3 = 63.5 -> 64 (tie with an inexact reciprocal)
    Xq, _ = O.act_quant(f32_to_bf16_bits(np.array([[3.0, 1.5, -1.5]], dtype=np.float32)))
    assert Xq.tolist() == [[127, 64, -64]]
    # a = 2.375: 127*1.1875/2.375 = 63.5 exactly; multiplying by a rounded
    # reciprocal of a would land just below the half and give 63
    Xq, _ = O.act_quant(f32_to_bf16_bits(np.array([[2.375, 1.1875, -1.1875]], dtype=np.float32)))
    assert Xq.tolist() == [[127, 64, -64]]
    # a = 127: q = rint(x); halves go to the even neighbour (62.5 -> 62, 2.5 -> 2)
    Xq, _ = O.act_quant(f32_to_bf16_bits(np.array([[127.0, 62.5, 2.5, -2.5, 0.5, 1.5, -62.5]], dtype=np.float32)))
    assert Xq.tolist() == [[127, 62, 2, -2, 0, 2, -62]]


def test_act_quant_zero_token():
    Xq, s_x = O.act_quant(np.zeros((2, 64), dtype=np.uint16))
    assert (Xq == 0).all() and s_x[0] == np.float32(np.float32(1e-5) / np.float32(127))


# ----------------------------------------------------------------- matmul + output
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 8), (1, 4)])
def test_accumulate_matches_int64_matmul_of_unpacked(n, m):
    W = gaussian_bf16((48, 128), 0.02, seed=3, stream=0)
    X = gaussian_bf16((9, 128), 1.0, seed=3, stream=1)
    f = O.forward(W, X, n, m)
    dense = pins.unpack_by_loops(f["codes_plane"], f["meta_plane"], 48, 128, n, m)
    ref = f["Xq"].astype(np.int64) @ dense.astype(np.int64).T      # numpy integer matmul
    assert (f["acc"] == ref).all()


def test_output_scaling_exact_rational():
    W = gaussian_bf16((8, 64), 0.02, seed=6, stream=0)
    X = gaussian_bf16((3, 64), 1.0, seed=6, stream=1)
    f = O.forward(W, X, 2, 4)
    for t in range(3):
        for r in range(8):
            exact = Fraction(int(f["acc"][t, r])) * Fraction(float(f["s_w"])) * Fraction(float(f["s_x"][t]))
            got = Fraction(float(f["y"][t, r]))
            assert abs(got - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_output_f32_and_bf16_match_exact_roundings():
    """Float outputs against exact rational arithmetic: one float32 rounding
    of s_w * s_x[t], one of acc times it, one bf16 rounding of that."""
    rng = np.random.default_rng(12)
    T, R = 24, 40
    acc = rng.integers(-127 * 4096, 127 * 4096 + 1, size=(T, R))
    acc[0, :4] = [0, 1, -1, 127 * 8192]
    s_w = np.float32(rng.uniform(0.005, 0.03))
    s_x = (rng.uniform(0.001, 0.2, size=T)).astype(np.float32)
    assert pins.output_matches_exact(O.output_f32, O.output_bf16, acc, s_w, s_x)
    # scales with many significant bits on both sides (products far from exact)
    s_x2 = np.float32(1.0) / np.arange(3, 3 + T, dtype=np.float32) / np.float32(127)
    assert pins.output_matches_exact(O.output_f32, O.output_bf16, acc, np.float32(1 / 3), s_x2)
    # c = 2^-8: 257, 259, 770 and 774 land half-way between two bf16 values (hand-derived:
    # 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6, 3 + 2^-7 -> 3, 3 + 3*2^-7 -> 3 + 2^-5 ... ties to even)
    acc2 = np.array([[257, 259, -257, 770, 774, 1, -3]])
    assert pins.output_matches_exact(O.output_f32, O.output_bf16, acc2, np.float32(0.5),
                                     np.array([2.0 ** -7], dtype=np.float32))
    assert O.output_bf16(acc2, np.float32(0.5), np.array([2.0 ** -7], np.float32)).tolist() == \
        [[0x3F80, 0x3F82, 0xBF80, 0x4040, 0x4042, 0x3B80, 0xBC40]]


def test_output_f32_within_rel_bound_of_real_value():
    """Two float32 roundings stay within 2^-23 relative of the real product."""
    W = gaussian_bf16((16, 256), 0.02, seed=13, stream=0)
    X = gaussian_bf16((8, 256), 1.0, seed=13, stream=1)
    f = O.forward(W, X, 2, 4)
    y32 = O.output_f32(f["acc"], f["s_w"], f["s_x"]).astype(np.float64)
    assert np.all(np.abs(y32 - f["y"]) <= 2.0 ** -23 * np.abs(f["y"]))


# ----------------------------------------------------------------- backward
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_backward_matches_torch_autograd_ste(n, m):
    W = gaussian_bf16((24, 64), 0.02, seed=8, stream=0)
    X = gaussian_bf16((5, 64), 1.0, seed=8, stream=1)
    dY = gaussian_bf16((5, 24), 1e-2, seed=8, stream=2)
    f = O.forward(W, X, n, m)
    gX, gW = O.backward(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"])
    rX, rW = pins.backward_by_autograd(W, X, dY, f["codes"], f["s_w"], f["Xq"], f["s_x"])
    assert np.allclose(gX, rX, rtol=1e-12, atol=1e-15)
    assert np.allclose(gW, rW, rtol=1e-12, atol=1e-15)
    # dense gradient through the mask: pruned positions receive gradient
    mask = f["mask"]
    assert np.abs(gW[~mask]).sum() > 0


# ----------------------------------------------------------------- ablation: mask from ternary weights
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (3, 4), (2, 8), (4, 8), (6, 8)])
def test_mask_ternary_matches_bruteforce(n, m):
    W = gaussian_bf16((6, 64), 0.02, seed=11, stream=0)
    s_w = O.weight_scale(W)
    assert pins.mask_ternary_matches_bruteforce(O.nm_mask_ternary, W, s_w, n, m)


def test_mask_ternary_worked_group():
    # s_w = 1: |q| = 1 iff |w| > 0.5.  Group [0.25, -0.75, 0.5, 1.0, 0.125, -2, 0, 0.75]
    # has |q| = [0, 1, 0, 1, 0, 1, 0, 1]: 2:8 keeps positions 1 and 3 (first two
    # nonzeros), 6:8 keeps the four nonzeros and the two lowest zeros (0, 2).
    W = f32_to_bf16_bits(np.array([[0.25, -0.75, 0.5, 1.0, 0.125, -2.0, 0.0, 0.75]], dtype=np.float32))
    one = np.float32(1.0)
    assert np.nonzero(O.nm_mask_ternary(W, one, 2, 8)[0])[0].tolist() == [1, 3]
    assert np.nonzero(O.nm_mask_ternary(W, one, 6, 8)[0])[0].tolist() == [0, 1, 2, 3, 5, 7]
    # the master-weight mask of the same group differs: 2:8 keeps -2 and 1.0
    assert np.nonzero(O.nm_mask(W, 2, 8)[0])[0].tolist() == [3, 5]


def test_quant_then_mask_ternary_variant_keeps_every_nonzero_when_room():
    # at 6:8 a group with at most six nonzero |q| keeps all of them
    W = gaussian_bf16((8, 64), 0.02, seed=12, stream=0)
    codes, mask, s_w = O.quant_then_mask(W, 6, 8, mask_from="ternary")
    q = O.ternary_codes(W, s_w)
    nz = (q != 0).reshape(8, 8, 8).sum(-1)
    lost = ((q != 0) & ~mask).reshape(8, 8, 8).sum(-1)
    assert (lost[nz <= 6] == 0).all() and (mask.reshape(8, 8, 8).sum(-1) == 6).all()
    assert np.array_equal(codes, np.where(mask, q, 0))


# ----------------------------------------------------------------- ablation: blocked gradient
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_backward_blocked_matches_torch_autograd(n, m):
    W = gaussian_bf16((24, 64), 0.02, seed=13, stream=0)
    X = gaussian_bf16((5, 64), 1.0, seed=13, stream=1)
    dY = gaussian_bf16((5, 24), 1e-2, seed=13, stream=2)
    f = O.forward(W, X, n, m)
    gX, gW = O.backward(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"], grad_mask=f["mask"])
    rX, rW = pins.backward_by_autograd(W, X, dY, f["codes"], f["s_w"], f["Xq"], f["s_x"], block_mask=f["mask"])
    assert np.allclose(gX, rX, rtol=1e-12, atol=1e-15)
    assert np.allclose(gW, rW, rtol=1e-12, atol=1e-15)
    assert (gW[~f["mask"]] == 0).all() and np.abs(gW[f["mask"]]).sum() > 0


# ----------------------------------------------------------------- optimizer step
def test_fma_f32_single_rounding_case():
    # w - lr*g = 1 + 2^-24 + 4688 * 2^-70: float64 rounds the sum onto the
    # float32 midpoint 1 + 2^-24 (a tie that goes to 1.0); the exact value is
    # above it, so the fused result is 1 + 2^-23.
    lr = np.float32(2.0 ** -24 * (1 + 2896 * 2.0 ** -23))
    g = np.float32(-(1 - 2895 * 2.0 ** -23))
    got = O.fma_f32(-lr, g, np.float32(1.0))
    assert float(got) == 1 + 2.0 ** -23
    assert pins.fma_matches_exact(O.fma_f32, -lr, g, np.float32(1.0))


def test_fma_f32_random_and_special():
    r = np.random.default_rng([21, 0])
    a = r.standard_normal(400).astype(np.float32) * np.float32(1e-3)
    b = r.standard_normal(400).astype(np.float32)
    c = f32_to_bf16_bits(r.standard_normal(400).astype(np.float32) * np.float32(0.02))
    c = bf16_bits_to_f32(c)
    assert pins.fma_matches_exact(O.fma_f32, a, b, c)
    # exact cases, zeros, and a subnormal result
    sa = np.array([0.5, 0.0, 1.0, 2.0 ** -70, -3.0], dtype=np.float32)
    sb = np.array([2.0, 5.0, -1.0, 2.0 ** -70, 0.0], dtype=np.float32)
    sc = np.array([0.0, -7.0, 1.0, 0.0, 0.0], dtype=np.float32)
    assert pins.fma_matches_exact(O.fma_f32, sa, sb, sc)
    assert O.fma_f32(sa, sb, sc).tolist()[:3] == [1.0, -7.0, 0.0]


def test_f32_to_bf16_rne_ties_and_examples():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -1.5, 0.0], dtype=np.float32)
    got = O.f32_to_bf16_rne(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6); just above a tie rounds up
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBFC0, 0x0000]


def test_sgd_update_matches_exact():
    W = gaussian_bf16((8, 40), 0.02, seed=14, stream=0)
    G = np.random.default_rng([14, 5]).standard_normal((8, 40)).astype(np.float32) * np.float32(1e-2)
    for lr in (np.float32(0.1), np.float32(3e-4), np.float32(1.0)):
        assert pins.sgd_matches_exact(O.sgd_update, W, G, lr)


def test_sgd_update_identities():
    W = gaussian_bf16((4, 64), 0.02, seed=15, stream=0)
    G = np.random.default_rng([15, 5]).standard_normal((4, 64)).astype(np.float32)
    assert np.array_equal(O.sgd_update(W, G, np.float32(0.0)), W)           # lr = 0
    assert np.array_equal(O.sgd_update(W, np.zeros_like(G), np.float32(0.5)), W)
    # w = 1, lr = 0.5, g = 1 -> 0.5 exactly; g = -2 -> 2.0
    one = f32_to_bf16_bits(np.array([[1.0, 1.0]], dtype=np.float32))
    out = O.sgd_update(one, np.array([[1.0, -2.0]], dtype=np.float32), np.float32(0.5))
    assert bf16_bits_to_f32(out).tolist() == [[0.5, 2.0]]


# ----------------------------------------------------------------- decode plane
@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 8), (1, 8)])
def test_d2_matches_bit_loops_and_decode(n, m):
    W = gaussian_bf16((5, 64), 0.02, seed=17, stream=0)
    codes, mask, sw = O.quant_then_mask(W, n, m)
    plane = O.pack_d2(codes)
    assert np.array_equal(plane, pins.d2_by_loops(codes))
    assert pins.d2_decode_matches(plane, codes)
    assert np.array_equal(O.unpack_d2(plane, 5, 64), codes)
    # the 2:4 bytes equal those of the packed planes; 6:8 is smaller
    cb, mb = O.packed_bytes(5, 64, n, m)
    assert plane.size == 5 * 64 // 4 and (plane.size < cb + mb if (n, m) == (6, 8) else True)


def test_d2_worked_word():
    # one row of 16: +1 at position 0, -1 at position 5 (k=1, b=1), +1 at 15 (k=3, b=3)
    codes = np.zeros((1, 16), np.int8)
    codes[0, 0], codes[0, 5], codes[0, 15] = 1, -1, 1
    # position 0 -> bits 6,7 of byte 0 (code 01 -> 0x40); position 5 -> bits 4,5 of byte 1
    # (code 11 -> 0x30); position 15 -> bits 0,1 of byte 3 (code 01 -> 0x01)
    assert O.pack_d2(codes).tolist() == [[0x40, 0x30, 0x00, 0x01]]


# ----------------------------------------------------------------- joint 2:4 code
def test_j6_worked_rows():
    g = json.load(open(os.path.join(GOLDEN, "j6_row_k64.json")))
    eff = np.array(g["rows"], dtype=np.int8)
    nib, h = O.pack_j6(eff)
    assert nib.tolist() == g["nib_plane"] and h.tolist() == g["h_plane"]
    assert np.array_equal(O.unpack_j6(nib, h, 2, g["K"]), eff)


def test_j6_groups_closed_form_count_and_round_trip():
    # a 2:4 group of effective ternary weights has 0, 1 or 2 nonzeros:
    # 1 + 4*2 + C(4,2)*4 = 33 groups, so 6 bits (64 >= 33 > 32) -- 1.5 bits per weight
    groups = [w for w in itertools.product((-1, 0, 1), repeat=4) if sum(1 for v in w if v) <= 2]
    assert len(groups) == 1 + 4 * 2 + math.comb(4, 2) * 4 == 33
    codes = [O.j6_group_code(w) for w in groups]
    assert len(set(codes)) == 33 and all(0 <= c < 64 for c in codes)
    for w, c in zip(groups, codes):
        assert O.j6_group_weights(c) == list(w)
    for w in itertools.product((-1, 0, 1), repeat=4):
        if sum(1 for v in w if v) > 2:
            with pytest.raises(ValueError):
                O.j6_group_code(w)


def test_j6_every_code_is_two_slots():
    # every 6-bit value is either not a code (equal positions with h = 2: four values)
    # or stands for at most two nonzeros, at the positions its nibble names
    bad = 0
    for c in range(64):
        i1, i2, h = c & 3, (c >> 2) & 3, c >> 4
        if i1 == i2 and h == 2:
            bad += 1
            with pytest.raises(ValueError):
                O.j6_group_weights(c)
            continue
        w = O.j6_group_weights(c)
        support = {p for p in range(4) if w[p] != 0}
        assert support <= {i1, i2} and len(support) <= 2
        assert O.j6_group_weights(O.j6_group_code(w)) == w          # canonical form stands for the same group
    assert bad == 4


def test_j6_all_sbn1_24_states():
    # every 2:4 packed state (two survivors, each code 0 / +1 / -1): 6 * 9 = 54 states,
    # whose effective groups the joint code must reproduce
    states = 0
    for pos in itertools.combinations(range(4), 2):
        for vals in itertools.product((0, 1, -1), repeat=2):
            eff = np.zeros((1, 64), dtype=np.int8)
            eff[0, list(pos)] = vals
            nib, h = O.pack_j6(eff)
            assert np.array_equal(O.unpack_j6(nib, h, 1, 64), eff)
            assert np.array_equal(pins.j6_slots_sum(nib, h, 1, 64), eff)
            states += 1
    assert states == 54


@pytest.mark.parametrize("R,K", [(3, 64), (5, 256), (2, 1024)])
def test_j6_matches_bit_loops_on_real_weights(R, K):
    W = gaussian_bf16((R, K), 0.02, seed=R + K, stream=0)
    eff, mask, sw = O.quant_then_mask(W, 2, 4)
    nib, h = O.pack_j6(eff)
    ln, lh = pins.j6_by_loops(eff)
    assert np.array_equal(nib, ln) and np.array_equal(h, lh)
    assert np.array_equal(pins.j6_slots_sum(nib, h, R, K), eff)
    assert np.array_equal(O.unpack_j6(nib, h, R, K), eff)
    # 1.5 bits per weight: 3/4 of the 2:4 packed planes
    cb, mb = O.packed_bytes(R, K, 2, 4)
    assert O.j6_bytes(R, K) == (nib.size, h.size) and 4 * (nib.size + h.size) == 3 * (cb + mb)
    # the GEMV through the code is the GEMV of the effective weights
    Xq, _ = O.act_quant(gaussian_bf16((3, K), 1.0, seed=K, stream=1))
    assert np.array_equal(O.accumulate(Xq, O.unpack_j6(nib, h, R, K)), O.accumulate(Xq, eff))
