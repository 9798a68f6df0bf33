"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bars (see gpu_util.py): meta, codes, s_w, Xq, s_x and int32 accumulators are
compared bit for bit; float32 and bf16 outputs bit for bit against the
oracle's rounding of the exact accumulator, and within the stated
tolerances of the real value.  Shapes
span several tiles with ragged tails in every dimension, the full workload
sizes (every output), all supported N:M ratios,
and the degenerate cases (zero weights, zero tokens, ties, subnormals,
magnitudes outside the fast summation window).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle as O
import sparse_linear_layers_02_amd as sbn
from gpu_util import (BF16_REL, assert_abs_product, assert_rel, bf16_bits_to_f64, dev, dev_bf16,
                      f32_bits, host)
from workloads import WORKLOADS, f32_to_bf16_bits, gaussian_bf16, gaussian_bf16_with_outliers

pytestmark = pytest.mark.gpu

ALL_NM = [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (6, 8), (7, 8), (8, 8)]


def gpu_pack(W_bits, n, m, ldw=None):
    import torch
    R, K = W_bits.shape
    if ldw is None:
        Wd = dev_bf16(W_bits)
    else:
        pad = np.full((R, ldw), 0x7F00, dtype=np.uint16)      # huge finite filler beyond K
        pad[:, :K] = W_bits
        Wd = dev_bf16(pad)[:, :K]
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(Wd, n, m)
    torch.cuda.synchronize()
    return codes, meta, s_w


def check_pack(W_bits, n, m, ldw=None, ref=None):
    R, K = W_bits.shape
    codes, meta, s_w = gpu_pack(W_bits, n, m, ldw)
    if ref is None:
        eff, mask, sw = O.quant_then_mask(W_bits, n, m)
        cp, mp = O.pack_sbn1(eff, mask, n, m)
    else:
        cp, mp, sw = ref
    assert f32_bits(host(s_w))[0] == f32_bits(sw), f"s_w {host(s_w)[0]!r} != {sw!r}"
    gc = host(codes)[: cp.size].reshape(cp.shape)
    assert np.array_equal(gc, cp), f"codes differ at {np.argwhere(gc != cp)[:3].tolist()}"
    if n < m:
        gm = host(meta)[: mp.size].reshape(mp.shape)
        assert np.array_equal(gm, mp), f"meta differ at {np.argwhere(gm != mp)[:3].tolist()}"
    return codes, meta, s_w


# ------------------------------------------------------------------ pack
@pytest.mark.parametrize("n,m", ALL_NM)
def test_pack_tiny_all_ratios(n, m):
    W = WORKLOADS["tiny"].weights(seed=0)
    check_pack(W, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 8), (1, 4)])
def test_pack_ragged_rows_and_leading_dim(n, m):
    W = gaussian_bf16((37, 192), 0.02, seed=3, stream=0)
    check_pack(W, n, m, ldw=200)


def special_weights(R=64, K=512, seed=11):
    rng = np.random.default_rng(seed)
    vals = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x2F80, 0xAF80,   # zeros, subnormals, 2^-32
            0x2F7F, 0x3C00, 0xBC00, 0x3C80, 0x4180, 0xC180, 0x4300, 0x7F7F,   # below 2^-32, ties, >= 16, max
            0xFF7F, 0x3F80, 0xBF80, 0x3F81]
    W = rng.choice(np.array(vals, dtype=np.uint16), size=(R, K))
    G = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    take = rng.random((R, K)) < 0.5
    return np.where(take, W, G).astype(np.uint16)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (3, 8), (4, 4)])
def test_pack_special_values_ties_and_extremes(n, m):
    check_pack(special_weights(), n, m)


def test_pack_gaussian_with_rare_tiny_weights():
    W = gaussian_bf16((128, 1024), 0.02, seed=5, stream=0)
    W[3, 7] = 0x0001          # subnormal
    W[9, 100] = 0x2000        # 2^-63
    W[50, 512] = 0x4200       # 32
    check_pack(W, 2, 4)


def test_pack_all_zero_weight():
    W = np.zeros((32, 128), dtype=np.uint16)
    codes, meta, s_w = check_pack(W, 2, 4)
    assert host(s_w)[0] == np.float32(1e-5)


def test_pack_exact_scale_ties_round_to_even():
    # one row of 64: the mean is a power-of-two fraction of the sum, so the sum
    # 1 + 2^-24 lands exactly half-way between two floats (-> even, down) and
    # 1 + 3*2^-24 half-way the other way (-> even, up)
    for extra in ([0x3380], [0x3400, 0x3380]):
        W = np.zeros((1, 64), dtype=np.uint16)
        W[0, 0] = 0x3F80
        W[0, 1:1 + len(extra)] = extra
        check_pack(W, 2, 4)


def test_pack_repeated_calls_reuse_workspace():
    W1 = gaussian_bf16((96, 256), 0.02, seed=1, stream=0)
    W2 = special_weights(48, 320, seed=2)
    for W in (W1, W2, W1):
        check_pack(W, 2, 4)


@functools.lru_cache(maxsize=None)
def full_ref(name, n, m):
    W = WORKLOADS[name].weights(seed=0)
    eff, mask, sw = O.quant_then_mask(W, n, m)
    cp, mp = O.pack_sbn1(eff, mask, n, m)
    return W, eff, cp, mp, sw


@pytest.mark.parametrize("name,n,m", [("prefill", 2, 4), ("train", 6, 8), ("decode", 2, 4), ("decode", 6, 8)])
def test_pack_full_size_bit_exact(name, n, m):
    W, eff, cp, mp, sw = full_ref(name, n, m)
    check_pack(W, n, m, ref=(cp, mp, sw))


# ------------------------------------------------------------------ act quant
def check_act_quant(X_bits, ldx=None):
    import torch
    T, K = X_bits.shape
    if ldx is None:
        Xd = dev_bf16(X_bits)
    else:
        pad = np.full((T, ldx), 0x7F00, dtype=np.uint16)
        pad[:, :K] = X_bits
        Xd = dev_bf16(pad)[:, :K]
    Xq, s_x = sbn.sbn_act_quant(Xd)
    torch.cuda.synchronize()
    rq, rs = O.act_quant(X_bits)
    gq = host(Xq)
    assert np.array_equal(gq, rq), f"Xq differ at {np.argwhere(gq != rq)[:3].tolist()}"
    assert np.array_equal(f32_bits(host(s_x)), f32_bits(rs))
    return Xq, s_x


@pytest.mark.parametrize("T,K", [(16, 256), (5, 64), (33, 2560), (7, 8192), (3, 16384)])
def test_act_quant_shapes(T, K):
    check_act_quant(gaussian_bf16((T, K), 1.0, seed=T, stream=1))


def test_act_quant_outliers_and_leading_dim():
    X = gaussian_bf16_with_outliers((40, 640), 1.0, 0, 1, 0.01, 20.0)
    check_act_quant(X, ldx=648)


def test_act_quant_half_ties_zero_and_tiny_rows():
    rows = [
        [127.0, 62.5, 2.5, -2.5, 0.5, 1.5, -62.5] + [0.0] * 57,
        [2.375, 1.1875, -1.1875] + [0.25] * 61,
        [3.0, 1.5, -1.5] + [1.0] * 61,
        [0.0] * 64,
        [1e-7, -3e-6, 2e-8] + [0.0] * 61,        # absmax below the 1e-5 floor
    ]
    X = f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    check_act_quant(X)


def test_act_quant_all_near_half_values():
    # every representable bf16 in [0.5, 1) against absmax 1: many near-half quotients
    vals = np.arange(0x3F00, 0x3F80, dtype=np.uint16)
    X = np.zeros((4, 192), dtype=np.uint16)
    X[:, : vals.size] = vals
    X[:, vals.size] = 0x3F80
    X[1] ^= 0x8000
    check_act_quant(X)


@pytest.mark.parametrize("name", ["prefill", "train"])
def test_act_quant_full_size(name):
    check_act_quant(WORKLOADS[name].activations(seed=0))


# ------------------------------------------------------------------ GEMM / GEMV
def forward_case(T, R, K, n, m, seed=0):
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=seed, stream=1)
    f = O.forward(W, X, n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(f["codes_plane"], f["meta_plane"], f["s_w"]))
    Xq = dev(f["Xq"])
    s_x = dev(f["s_x"])
    return f, Xq, s_x, codes, meta, s_w


def run_matmul(kind, Xq, s_x, codes, meta, s_w, R, n, m, ydt):
    """Runs the GEMM/GEMV; the output buffer's row stride is R rounded up to 8
    (the ABI's leading-dimension rule), and the padding columns must stay untouched."""
    import torch
    fn = sbn.sbn_sparse_ternary_gemm if kind == "gemm" else sbn.sbn_sparse_ternary_gemv
    T = Xq.shape[0]
    ldy = (R + 7) // 8 * 8
    dt = {sbn.SBN_F32: torch.float32, sbn.SBN_BF16: torch.bfloat16, sbn.SBN_I32_ACC: torch.int32}[ydt]
    full = torch.full((T, ldy), 77, dtype=dt, device=Xq.device)
    Y = full[:, :R]
    fn(Xq, s_x, codes, meta, s_w, R, n, m, ydt=ydt, Y=Y)
    torch.cuda.synchronize()
    if ldy > R:
        assert bool((full[:, R:] == 77).all()), "write past R"
    return host(Y.contiguous())


def assert_float_outputs(y32, yb, acc, sw, sx, what):
    """f32 Y and bf16 Y: bit for bit the operator's rounding of the exact
    accumulator (one float32 product with the token's float32 scale; bf16 its
    nearest-even rounding), and within the stated tolerances of the real value."""
    if y32 is not None:
        ref32 = O.output_f32(acc, sw, sx)
        bad = f32_bits(y32) != f32_bits(ref32)
        assert not bad.any(), f"{what} f32 Y: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
        assert_rel(y32, O.output(acc, sw, sx), 1e-3, f"{what} f32 Y")
    if yb is not None:
        refb = O.output_bf16(acc, sw, sx)
        bad = yb != refb
        assert not bad.any(), f"{what} bf16 Y: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
        assert_rel(bf16_bits_to_f64(yb), O.output(acc, sw, sx), BF16_REL, f"{what} bf16 Y")


def check_outputs(kind, f, Xq, s_x, codes, meta, s_w, R, n, m):
    acc = run_matmul(kind, Xq, s_x, codes, meta, s_w, R, n, m, sbn.SBN_I32_ACC)
    assert np.array_equal(acc.astype(np.int64), f["acc"]), \
        f"acc differ at {np.argwhere(acc != f['acc'])[:3].tolist()}"
    y32 = run_matmul(kind, Xq, s_x, codes, meta, s_w, R, n, m, sbn.SBN_F32)
    yb = run_matmul(kind, Xq, s_x, codes, meta, s_w, R, n, m, sbn.SBN_BF16)
    assert_float_outputs(y32, yb, f["acc"], f["s_w"], f["s_x"], kind)


def test_gemm_tiny_workload_fp32_output():
    wl = WORKLOADS["tiny"]
    W, X = wl.weights(0), wl.activations(0)
    f = O.forward(W, X, 2, 4)
    codes, meta, s_w = check_pack(W, 2, 4, ref=(f["codes_plane"], f["meta_plane"], f["s_w"]))
    check_outputs("gemm", f, dev(f["Xq"]), dev(f["s_x"]), codes, meta, s_w, 256, 2, 4)


@pytest.mark.parametrize("n,m", ALL_NM)
def test_gemm_ragged_all_ratios(n, m):
    T, R, K = 300, 520, 576          # two token tiles, three row tiles, K not a multiple of 128
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=n + 10 * m)
    check_outputs("gemm", f, Xq, s_x, codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("T,R,K", [(1, 16, 64), (5, 33, 128), (17, 33, 128), (257, 257, 640)])
def test_gemm_small_edges(T, R, K):
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, 2, 4, seed=T)
    check_outputs("gemm", f, Xq, s_x, codes, meta, s_w, R, 2, 4)
    if T <= 16:
        check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, R, 2, 4)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
@pytest.mark.parametrize("T", [100, 200, 497])
def test_gemm_token_tile_variants(T, n, m):
    # R = 96 row tiles - 37 rows: T = 497 keeps the 256-token block tile (192
    # tiles), T = 200 takes the 128-token tile and T = 100 the 64-token tile
    # (sparse; dense stops at 128), each with ragged rows and tokens
    R, K = 96 * 256 - 37, 256
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=T + n)
    check_outputs("gemm", f, Xq, s_x, codes, meta, s_w, R, n, m)


def test_gemm_extreme_activations():
    # Xq = +-127 everywhere on dense ternary +-1 weights: |acc| = 127*K at the limit of the range
    T, R, K, n, m = 32, 64, 2048, 8, 8
    W = f32_to_bf16_bits(np.where(np.random.default_rng(1).random((R, K)) < 0.5, 1.0, -1.0).astype(np.float32))
    X = f32_to_bf16_bits(np.where(np.random.default_rng(2).random((T, K)) < 0.5, 3.0, -3.0).astype(np.float32))
    f = O.forward(W, X, n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(f["codes_plane"], f["meta_plane"], f["s_w"]))
    check_outputs("gemm", f, dev(f["Xq"]), dev(f["s_x"]), codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (1, 4), (8, 8), (3, 8)])
@pytest.mark.parametrize("T", [1, 4, 16, 7])
def test_gemv_ragged(n, m, T):
    R, K = 600, 2560                 # K not a multiple of 1024: a short last range
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=T + n)
    check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("n,m", ALL_NM)
def test_gemv_all_ratios_short_k(n, m):
    f, Xq, s_x, codes, meta, s_w = forward_case(3, 40, 576, n, m, seed=7 * n + m)
    check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, 40, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
@pytest.mark.parametrize("K", [1024, 2048, 3072, 4096])
@pytest.mark.parametrize("T,R", [(1, 37), (5, 1000), (16, 203)])
def test_gemv_streamed_shapes(n, m, K, T, R):
    """The streamed decode kernels (K a multiple of 1024 up to 4096): one to four
    waves with a range, ragged R (rows past R read row R-1 and are dropped)."""
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=K + T + R)
    check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_gemv_streamed_ring_tail(n, m):
    """Many more row groups than blocks (at most 1024 blocks): each block walks
    five or more consecutive row groups through its ring, so the loads-in-flight
    count drains at the tail, outputs leave in one full group of four row groups
    and one partial group, and the last row group is ragged."""
    R, K, T = 1024 * 16 * 5 + 40, 1024, 3
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=5)
    check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("n,m,K", [(2, 4, 4096), (6, 8, 2048), (1, 4, 1024), (6, 8, 640)])
@pytest.mark.parametrize("count,R,T", [(3, 203, 5), (64, 48, 1)])
def test_gemv_batched_matches_oracle(n, m, K, count, R, T):
    """Several weights sharing the activations in one call (one launch for
    2:4 and 6:8 at K a multiple of 1024; otherwise one launch per weight):
    every output equals the oracle's for its own weight."""
    import torch
    X = gaussian_bf16((T, K), 1.0, seed=count + K, stream=1)
    Xq_h, s_x_h = O.act_quant(X)
    Xq, s_x = dev(Xq_h), dev(s_x_h)
    Ws = [gaussian_bf16((R, K), 0.02 * (1 + b % 3), seed=100 + b, stream=0) for b in range(count)]
    packed = [sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m) for W in Ws]
    codes = [p[0] for p in packed]
    metas = None if n == m else [p[1] for p in packed]
    s_ws = [p[2] for p in packed]
    for ydt in (sbn.SBN_I32_ACC, sbn.SBN_F32):
        Ys = sbn.sbn_sparse_ternary_gemv_batched(Xq, s_x, codes, metas, s_ws, R, n, m, ydt=ydt)
        torch.cuda.synchronize()
        for b in range(0, count, max(1, count // 8)):
            eff, _, sw = O.quant_then_mask(Ws[b], n, m)
            acc = O.accumulate(Xq_h, eff)
            got = host(Ys[b])
            if ydt == sbn.SBN_I32_ACC:
                assert np.array_equal(got.astype(np.int64), acc), f"weight {b}"
            else:
                assert_float_outputs(got, None, acc, sw, s_x_h, f"weight {b}")


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_gemv_decode_full_size(n, m):
    wl = WORKLOADS["decode"]
    W, eff, cp, mp, sw = full_ref("decode", n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(cp, mp, sw))
    for T in wl.Ts:
        X = wl.activations(seed=0, T=T)
        Xq_h, s_x_h = O.act_quant(X)
        acc = O.accumulate(Xq_h, eff)
        got = run_matmul("gemv", dev(Xq_h), dev(s_x_h), codes, meta, s_w, 4096, n, m, sbn.SBN_I32_ACC)
        assert np.array_equal(got.astype(np.int64), acc)
        yb = run_matmul("gemv", dev(Xq_h), dev(s_x_h), codes, meta, s_w, 4096, n, m, sbn.SBN_BF16)
        assert_float_outputs(None, yb, acc, sw, s_x_h, f"decode T={T}")


@pytest.mark.parametrize("name,n,m", [("prefill", 2, 4), ("train", 6, 8), ("sweep", 2, 4), ("sweep", 4, 8),
                                      ("sweep", 6, 8), ("sweep", 2, 8), ("sweep", 1, 4), ("sweep", 8, 8)])
def test_gemm_full_size_exact(name, n, m):
    """Every output of the GEMM at the full prefill, train-step and sweep
    shapes: the whole int32 accumulator equals the oracle's, and the bf16 Y
    equals the oracle's rounding of it, element by element."""
    wl = WORKLOADS[name]
    W, eff, cp, mp, sw = full_ref(name, n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(cp, mp, sw))
    X = wl.activations(seed=0)
    Xq_h, s_x_h = O.act_quant(X)
    Xq, s_x = check_act_quant(X)
    print(f"full-size GEMM {name} {n}:{m} T={wl.T} R={wl.R} K={wl.K}", flush=True)
    acc = run_matmul("gemm", Xq, s_x, codes, meta, s_w, wl.R, n, m, sbn.SBN_I32_ACC)
    ref = O.accumulate(Xq_h, eff)
    bad = acc.astype(np.int64) != ref
    assert not bad.any(), f"acc: {bad.sum()} of {bad.size} differ, first at {np.argwhere(bad)[0].tolist()}"
    del bad, acc
    yb = run_matmul("gemm", Xq, s_x, codes, meta, s_w, wl.R, n, m, sbn.SBN_BF16)
    assert_float_outputs(None, yb, ref, sw, s_x_h, f"{name} {n}:{m}")


def test_gemm_deterministic_and_matches_gemv():
    f, Xq, s_x, codes, meta, s_w = forward_case(16, 512, 1024, 2, 4, seed=4)
    a1 = run_matmul("gemm", Xq, s_x, codes, meta, s_w, 512, 2, 4, sbn.SBN_BF16)
    a2 = run_matmul("gemm", Xq, s_x, codes, meta, s_w, 512, 2, 4, sbn.SBN_BF16)
    g1 = run_matmul("gemv", Xq, s_x, codes, meta, s_w, 512, 2, 4, sbn.SBN_BF16)
    assert np.array_equal(a1, a2) and np.array_equal(a1, g1)


# ------------------------------------------------------------------ backward
def check_backward(T, R, K, n, m, seed=0, dxdt=None):
    import torch
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=seed, stream=1)
    dY = gaussian_bf16((T, R), 1e-2, seed=seed, stream=2)
    f = O.forward(W, X, n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(f["codes_plane"], f["meta_plane"], f["s_w"]))
    dxdt = sbn.SBN_F32 if dxdt is None else dxdt
    dX, dW = sbn.sbn_backward(dev_bf16(dY), dev(f["Xq"]), dev(f["s_x"]), codes, meta, s_w, n, m, dxdt=dxdt)
    torch.cuda.synchronize()
    gX, gW = O.backward(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"])
    dYf = np.abs(bf16_bits_to_f64(dY))
    boundX = dYf @ (float(f["s_w"]) * np.abs(f["codes"].astype(np.float64)))
    boundW = dYf.T @ (f["s_x"].astype(np.float64)[:, None] * np.abs(f["Xq"].astype(np.float64)))
    hx = host(dX)
    hx = bf16_bits_to_f64(hx) if dxdt == sbn.SBN_BF16 else hx
    if dxdt == sbn.SBN_BF16:
        assert_abs_product(hx, gX, boundX + np.abs(gX) * (2 ** -8 / 1e-3), "dX(bf16)")
    else:
        assert_abs_product(hx, gX, boundX, "dX")
    assert_abs_product(host(dW), gW, boundW, "dW")


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (8, 8), (1, 4)])
def test_backward_ragged(n, m):
    check_backward(96, 264, 320, n, m, seed=n + m)


def test_backward_multi_tile_and_bf16_dx():
    check_backward(300, 520, 576, 2, 4, seed=3)
    check_backward(40, 64, 128, 6, 8, seed=4, dxdt=sbn.SBN_BF16)


def test_backward_short_contraction():
    """One contraction step in both GEMMs (T <= 32 for dW, R <= 32 for dX), and
    two for dX (R = 56): fewer steps than the kernels' LDS stages."""
    check_backward(17, 24, 64, 2, 4, seed=5)
    check_backward(33, 56, 128, 6, 8, seed=6, dxdt=sbn.SBN_BF16)


def test_backward_train_size_full():
    """The train-step backward at full size (T=8192, R=11008, K=4096, 6:8):
    every element of dX and dW against the oracle within the abs-product bound."""
    import torch
    wl = WORKLOADS["train"]
    n, m = wl.nm[0]
    W, eff, cp, mp, sw = full_ref("train", n, m)
    codes, meta, s_w = check_pack(W, n, m, ref=(cp, mp, sw))
    X = wl.activations(seed=0)
    dY = wl.upstream_grad(seed=0)
    Xq_h, s_x_h = O.act_quant(X)
    print(f"full-size backward train {n}:{m}", flush=True)
    dX, dW = sbn.sbn_backward(dev_bf16(dY), dev(Xq_h), dev(s_x_h), codes, meta, s_w, n, m)
    torch.cuda.synchronize()
    gX, gW = O.backward(dY, Xq_h, s_x_h, eff, sw)
    dYa = np.abs(bf16_bits_to_f64(dY))
    bX = dYa @ (float(sw) * np.abs(eff.astype(np.float64)))
    assert_abs_product(host(dX), gX, bX, "dX")
    del gX, bX, dX
    bW = dYa.T @ (s_x_h.astype(np.float64)[:, None] * np.abs(Xq_h.astype(np.float64)))
    assert_abs_product(host(dW), gW, bW, "dW")


# ------------------------------------------------------------------ HIP graph replay
def test_graph_replays_match_eager():
    """The forward step (pack, act_quant, GEMM) captured as a HIP graph: every
    replay, with eager work and synchronisation between replays, reproduces
    the eager results bit for bit (the bench times such replays)."""
    import torch
    T, R, K, n, m = 300, 520, 576, 2, 4
    W = dev_bf16(gaussian_bf16((R, K), 0.02, seed=21, stream=0))
    X = dev_bf16(gaussian_bf16((T, K), 1.0, seed=21, stream=1))
    cb, mb = sbn.sbn_packed_bytes(R, K, n, m)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    s_w = torch.empty(1, dtype=torch.float32, device="cuda")
    Xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
    s_x = torch.empty(T, dtype=torch.float32, device="cuda")
    Y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    wsp = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_PACK, 0, R, K, n, m), dtype=torch.uint8, device="cuda")
    wsg = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, T, R, K, n, m), dtype=torch.uint8, device="cuda")

    def step():
        sbn.sbn_mask_ternarize_pack(W, n, m, codes=codes, meta=meta, s_w=s_w, ws=wsp)
        sbn.sbn_act_quant(X, Xq=Xq, s_x=s_x)
        sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, R, n, m, ydt=sbn.SBN_BF16, Y=Y, ws=wsg)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (codes, meta, s_w, Xq, s_x, Y)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (codes, meta, s_w, Xq, s_x, Y):
            t.zero_()                               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((codes, meta, s_w, Xq, s_x, Y), ref):
            assert torch.equal(a, b), f"replay {rep} differs"


@pytest.mark.parametrize("K", [128, 384, 640, 768, 896, 1600])
@pytest.mark.parametrize("T", [1, 7, 16])
def test_gemv_2_4_partial_ranges(K, T):
    """2:4 decode: K ranges of 512 positions with a short last range of one to
    three 128-position steps, and K = 64 mod 128 (the table path)."""
    f, Xq, s_x, codes, meta, s_w = forward_case(T, 40, K, 2, 4, seed=K + T)
    check_outputs("gemv", f, Xq, s_x, codes, meta, s_w, 40, 2, 4)


def _midpoint_weights(extra_bits=None):
    """256 x 256 bf16 weights whose exact mean |w| is 1 - 2^-15 + 2^-25: the
    midpoint between two adjacent fp32 values (65534 ones, one 2^-9, one 0);
    `extra_bits` replaces the zero to move the mean off the midpoint."""
    W = np.full((256, 256), 0x3F80, dtype=np.uint16)          # 1.0
    W[0, 0] = 0x3B00                                           # 2^-9
    W[0, 1] = 0x0000 if extra_bits is None else extra_bits
    return W


@pytest.mark.parametrize("extra", [None, 0x0001, 0x8001, 0x2F80])
def test_pack_scale_rounding_near_midpoint(extra):
    """s_w when mean |W| is exactly a midpoint between two floats (ties to
    even), a subnormal 2^-133 above it (rounds up, decided only by the exact
    comparison), and 2^-32 above it; against the oracle's exact rounding."""
    W = _midpoint_weights(extra)
    for n, m in [(2, 4), (6, 8)]:
        check_pack(W, n, m)
    sw = O.weight_scale(W)
    if extra is None:
        assert f32_bits(sw) == 0x3F7FFE00                      # the even neighbour
    elif extra in (0x0001, 0x8001):
        assert f32_bits(sw) == 0x3F7FFE01


@pytest.mark.parametrize("K", [128, 256, 384, 512, 1152])
def test_gemm_2_4_k_steps(K):
    """2:4 GEMM with one to nine K steps of 128, i.e. fewer steps than
    pipeline stages, exactly as many, and more; two token tiles and three row
    tiles with ragged tails."""
    T, R = 300, 520
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, 2, 4, seed=K)
    check_outputs("gemm", f, Xq, s_x, codes, meta, s_w, R, 2, 4)
