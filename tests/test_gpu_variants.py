"""GPU parity of the variants beside the path, through the C ABI, against the
CPU oracle: the two ablations (mask from the ternary weights; gradient
blocked at pruned positions), the SGD master-weight step fused with the
next pack, and the one-call forward.  Bars as in test_gpu_parity.py: packed planes, scales and updated
bf16 weights bit for bit; gradients within the float32 accumulation bound.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import sparse_linear_layers_02_amd as sbn
from gpu_util import assert_abs_product, bf16_bits_to_f64, dev, dev_bf16, f32_bits, host
from workloads import WORKLOADS, f32_to_bf16_bits, gaussian_bf16

pytestmark = pytest.mark.gpu

ALL_NM = [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (6, 8), (7, 8), (8, 8)]


def padded(bits: np.ndarray, ld: int | None, fill):
    """Device copy of a [R, K] array inside rows of ld entries (None: contiguous)."""
    R, K = bits.shape
    if ld is None:
        return dev_bf16(bits) if bits.dtype == np.uint16 else dev(bits)
    pad = np.full((R, ld), fill, dtype=bits.dtype)
    pad[:, :K] = bits
    return (dev_bf16(pad) if bits.dtype == np.uint16 else dev(pad))[:, :K]


def compare_planes(codes, meta, s_w, W_bits, n, m, mask_from):
    eff, mask, sw = O.quant_then_mask(W_bits, n, m, mask_from=mask_from)
    cp, mp = O.pack_sbn1(eff, mask, n, m)
    assert f32_bits(host(s_w))[0] == f32_bits(sw), f"s_w {host(s_w)[0]!r} != {sw!r}"
    gc = host(codes)[: cp.size].reshape(cp.shape)
    assert np.array_equal(gc, cp), f"codes differ at {np.argwhere(gc != cp)[:3].tolist()}"
    if n < m:
        gm = host(meta)[: mp.size].reshape(mp.shape)
        assert np.array_equal(gm, mp), f"meta differ at {np.argwhere(gm != mp)[:3].tolist()}"
    return eff, mask, sw


# ------------------------------------------------------------------ mask from the ternary weights
def check_pack_ternary(W_bits, n, m, ldw=None):
    import torch
    Wd = padded(W_bits, ldw, np.uint16(0x7F00))
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack_ex(Wd, n, m, sbn.SBN_MASK_FROM_TERNARY)
    torch.cuda.synchronize()
    return compare_planes(codes, meta, s_w, W_bits, n, m, "ternary")


@pytest.mark.parametrize("n,m", ALL_NM)
def test_pack_ternary_mask_all_ratios(n, m):
    W = gaussian_bf16((37, 320), 0.02, seed=n * 10 + m, stream=0)
    eff, mask, _ = check_pack_ternary(W, n, m)
    if n < m:   # the variant differs from the method's mask on Gaussian weights
        assert not np.array_equal(mask, O.nm_mask(W, n, m))


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (3, 8)])
def test_pack_ternary_mask_ties_zero_groups_and_leading_dim(n, m):
    rng = np.random.default_rng(7)
    W = gaussian_bf16((48, 256), 0.02, seed=7, stream=0)
    W[rng.random(W.shape) < 0.3] = 0           # many |q| = 0 ties, whole zero groups
    W[5, :] = 0x3C00                           # a row of equal values (all |q| = 1)
    check_pack_ternary(W, n, m, ldw=264)


def test_pack_ternary_flag_zero_is_the_method():
    import torch
    W = gaussian_bf16((64, 512), 0.02, seed=9, stream=0)
    Wd = dev_bf16(W)
    a = sbn.sbn_mask_ternarize_pack_ex(Wd, 6, 8, 0)
    b = sbn.sbn_mask_ternarize_pack(Wd, 6, 8)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("name,n,m", [("prefill", 2, 4), ("train", 6, 8)])
def test_pack_ternary_mask_full_size(name, n, m):
    check_pack_ternary(WORKLOADS[name].weights(seed=0), n, m)


# ------------------------------------------------------------------ blocked gradient
def check_backward_blocked(T, R, K, n, m, seed=0):
    import torch
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=seed, stream=1)
    dY = gaussian_bf16((T, R), 1e-2, seed=seed, stream=2)
    f = O.forward(W, X, n, m)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m)
    args = (dev_bf16(dY), dev(f["Xq"]), dev(f["s_x"]), codes, meta, s_w, n, m)
    dXb, dWb = sbn.sbn_backward_ex(*args, sbn.SBN_GRAD_W_MASKED)
    dXd, dWd = sbn.sbn_backward(*args)
    torch.cuda.synchronize()
    gX, gW = O.backward(dY, f["Xq"], f["s_x"], f["codes"], f["s_w"], grad_mask=f["mask"])
    dYf = np.abs(bf16_bits_to_f64(dY))
    boundW = dYf.T @ (f["s_x"].astype(np.float64)[:, None] * np.abs(f["Xq"].astype(np.float64)))
    hW = host(dWb)
    assert (hW[~f["mask"]] == 0.0).all(), "blocked dW is not exactly 0 at pruned positions"
    assert_abs_product(hW, gW, boundW, "blocked dW")
    # kept positions and dX are those of the dense-gradient call, bit for bit
    assert np.array_equal(hW[f["mask"]], host(dWd)[f["mask"]])
    assert np.array_equal(host(dXb), host(dXd))


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (1, 8), (8, 8)])
def test_backward_blocked_ragged(n, m):
    check_backward_blocked(96, 264, 320, n, m, seed=n + m)


def test_backward_blocked_multi_tile():
    check_backward_blocked(300, 520, 576, 6, 8, seed=5)


# ------------------------------------------------------------------ SGD step + pack
def sgd_case(R, K, seed, g_scale):
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    G = np.random.default_rng([seed, 9]).standard_normal((R, K)).astype(np.float32) * np.float32(g_scale)
    return W, G


def check_sgd(W_bits, G, lr, n, m, flags=0, ldw=None, ldg=None):
    import torch
    Wd = padded(W_bits, ldw, np.uint16(0x7F00))
    Gd = padded(G, ldg, np.float32(1e30))
    codes, meta, s_w = sbn.sbn_sgd_update_pack(Wd, Gd, lr, n, m, flags)
    torch.cuda.synchronize()
    want = O.sgd_update(W_bits, G, np.float32(lr))
    got = host(Wd)
    assert np.array_equal(got, want), f"updated W differs at {np.argwhere(got != want)[:3].tolist()}"
    mask_from = "ternary" if flags & sbn.SBN_MASK_FROM_TERNARY else "master"
    compare_planes(codes, meta, s_w, want, n, m, mask_from)
    return want


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (1, 4), (8, 8), (3, 8)])
def test_sgd_update_pack_ratios(n, m):
    W, G = sgd_case(45, 384, seed=n + 3 * m, g_scale=1e-2)
    for lr in (0.01, 3e-4):
        W = check_sgd(W, G, lr, n, m)


def test_sgd_update_pack_leading_dims_and_ternary_mask():
    W, G = sgd_case(33, 256, seed=4, g_scale=1e-2)
    check_sgd(W, G, 0.02, 6, 8, ldw=272, ldg=264)
    check_sgd(W, G, 0.02, 2, 4, flags=sbn.SBN_MASK_FROM_TERNARY, ldg=264)


def test_sgd_update_rounding_ties_and_identities():
    # lr = 1: w = 1 with g = -2^-8 gives the bf16 tie 1 + 2^-8 (-> 1.0), g = -3*2^-8
    # the tie 1 + 3*2^-8 (-> 1 + 2^-6); lr = 0 and g = 0 leave W unchanged
    W = gaussian_bf16((16, 128), 0.02, seed=6, stream=0)
    W[0, :4] = f32_to_bf16_bits(np.ones((1, 4), np.float32))[0]
    G = np.random.default_rng(6).standard_normal((16, 128)).astype(np.float32) * np.float32(1e-2)
    G[0, :4] = [-2.0 ** -8, -3 * 2.0 ** -8, 2.0 ** -9, 0.0]
    got = check_sgd(W, G, 1.0, 2, 4)
    assert bf16_bits_to_f64(got[0, :4]).tolist() == [1.0, 1 + 2.0 ** -6, 1.0, 1.0]
    check_sgd(W, G, 0.0, 2, 4)
    assert np.array_equal(check_sgd(W, np.zeros_like(G), 0.5, 6, 8), W)


def test_sgd_update_pack_repeated_steps():
    W, G = sgd_case(64, 512, seed=8, g_scale=5e-2)
    for step in range(3):
        W = check_sgd(W, G * np.float32(step + 1), 0.05, 6, 8)


def test_sgd_update_pack_train_size():
    wl = WORKLOADS["train"]
    n, m = wl.nm[0]
    W = wl.weights(seed=0)
    G = np.random.default_rng([0, 9]).standard_normal(W.shape).astype(np.float32) * np.float32(1e-2)
    check_sgd(W, G, 1e-2, n, m)


# ------------------------------------------------------------------ the one-call forward
def check_forward(T, R, K, n, m, flags=0, ldw=None, ldx=None, seed=0, ydt=None):
    import torch
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=seed, stream=1)
    Wd = padded(W, ldw, np.uint16(0x7F00))
    Xd = padded(X, ldx, np.uint16(0x7F00))
    ydt = sbn.SBN_I32_ACC if ydt is None else ydt
    codes, meta, s_w, Xq, s_x, Y = sbn.sbn_forward(Wd, Xd, n, m, flags, ydt=ydt)
    torch.cuda.synchronize()
    mask_from = "ternary" if flags & sbn.SBN_MASK_FROM_TERNARY else "master"
    eff, mask, sw = compare_planes(codes, meta, s_w, W, n, m, mask_from)
    xq, sx = O.act_quant(X)
    assert np.array_equal(host(Xq), xq)
    assert np.array_equal(f32_bits(host(s_x)), f32_bits(sx))
    acc = O.accumulate(xq, eff)
    check_forward_y(Y, ydt, acc, sw, sx)


def check_forward_y(Y, ydt, acc, sw, sx):
    """Y of the one-call forward: the int32 accumulator exactly; f32 / bf16 bit
    for bit the oracle's rounding of it, and within the stated tolerances."""
    got = host(Y)
    if ydt == sbn.SBN_I32_ACC:
        bad = got.astype(np.int64) != acc
        assert not bad.any(), f"acc: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
        return
    y = O.output(acc, sw, sx)
    if ydt == sbn.SBN_BF16:
        bad = got != O.output_bf16(acc, sw, sx)
        got = bf16_bits_to_f64(got)
        rel = 2.0 ** -8 + 2.0 ** -20
    else:
        bad = f32_bits(got) != f32_bits(O.output_f32(acc, sw, sx))
        rel = 1e-3
    assert not bad.any(), f"Y: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
    assert (np.abs(got - y) <= rel * np.abs(y)).all()


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8), (1, 8), (8, 8)])
def test_forward_matches_oracle(n, m):
    check_forward(37, 264, 320, n, m, seed=n + m)                 # T not a multiple of the 4 tokens per block


@pytest.mark.parametrize("K", [64, 2560, 8192, 16384])
def test_forward_token_lengths(K):
    # one, two and four 16-byte chunks per thread, and the two-pass quantizer beyond K = 8192
    check_forward(6, 40, K, 2, 4, seed=K)


def test_forward_leading_dims_flags_and_outputs():
    check_forward(21, 96, 256, 6, 8, ldw=264, ldx=272, seed=3)
    check_forward(19, 100, 192, 2, 4, ldw=200, ldx=208, seed=7)     # 2:4 with ragged rows, a 64-K tail step
    check_forward(21, 96, 256, 2, 4, flags=sbn.SBN_MASK_FROM_TERNARY, seed=4)
    check_forward(50, 520, 576, 2, 4, seed=5, ydt=sbn.SBN_BF16)
    check_forward(50, 520, 576, 6, 8, seed=6, ydt=sbn.SBN_F32)


@pytest.mark.parametrize("ydt", [sbn.SBN_I32_ACC, sbn.SBN_BF16])
@pytest.mark.parametrize("T,R,K,ldw,ldx", [(300, 520, 576, None, None), (17, 33, 128, None, None),
                                           (40, 100, 64, None, None), (257, 1000, 1152, 1160, 1168),
                                           (64, 7000, 384, None, None), (33, 264, 1664, None, None)])
def test_forward_wide_writes_operand(monkeypatch, T, R, K, ldw, ldx, ydt):
    """2:4 one-call forward with the wide GEMM tiles forced on: the pack's second
    pass writes the GEMM's weight operand and the GEMM reads the activations in
    place (no layout launch); planes, scales, Xq, s_x and Y against the oracle
    on ragged rows and tokens, a 64-position K tail, K = 64, padded rows and
    13 K steps split unevenly over two blocks."""
    monkeypatch.setenv("SBN_GEMM_TILE", "wide")
    print(f"forward, operand from pass 2: T={T} R={R} K={K} ldw={ldw} ldx={ldx} ydt={ydt}", flush=True)
    check_forward(T, R, K, 2, 4, ldw=ldw, ldx=ldx, seed=T + K, ydt=ydt)


def test_forward_launches_at_prefill_size():
    """The prefill-shape forward runs three kernels (pass 1, pass 2 with the
    quantizer and the weight operand, the wide GEMM); a 6:8 forward keeps the
    layout launch."""
    import torch
    wl = WORKLOADS["prefill"]
    W, X = dev_bf16(wl.weights(0)), dev_bf16(wl.activations(0))
    sbn.sbn_forward(W, X, 2, 4)
    torch.cuda.synchronize()
    for nm, want in (((2, 4), {"abs_sum", "mask_pack_quant", "gemm_smfmac_wide"}),
                     ((6, 8), {"abs_sum", "mask_pack", "act_quant", "layout_dense", "gemm_mfma"})):
        sbn.sbn_profile_reset()
        sbn.sbn_profile_enable(True)
        sbn.sbn_forward(W, X, *nm)
        torch.cuda.synchronize()
        sbn.sbn_profile_enable(False)
        got = set(sbn.sbn_profile_dump())
        assert got == want, f"{nm}: kernels {sorted(got)}"


def test_forward_prefill_size_equals_separate_calls():
    import torch
    wl = WORKLOADS["prefill"]
    W, X = dev_bf16(wl.weights(0)), dev_bf16(wl.activations(0))
    a = sbn.sbn_forward(W, X, 2, 4)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(W, 2, 4)
    Xq, s_x = sbn.sbn_act_quant(X)
    Y = sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, wl.R, 2, 4)
    torch.cuda.synchronize()
    for x, y in zip(a, (codes, meta, s_w, Xq, s_x, Y)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["prefill", "train"])
def test_forward_full_size_exact(name):
    """The one-call forward exactly as the benchmark runs it (full prefill
    shape at 2:4 and full train-step shape at 6:8, bf16 Y): planes, scales,
    Xq, s_x and every bf16 output against the oracle."""
    import torch
    wl = WORKLOADS[name]
    n, m = wl.nm[0]
    W, X = wl.weights(0), wl.activations(0)
    print(f"full-size forward {name} {n}:{m} T={wl.T} R={wl.R} K={wl.K}", flush=True)
    codes, meta, s_w, Xq, s_x, Y = sbn.sbn_forward(dev_bf16(W), dev_bf16(X), n, m, ydt=sbn.SBN_BF16)
    torch.cuda.synchronize()
    eff, mask, sw = compare_planes(codes, meta, s_w, W, n, m, "master")
    xq, sx = O.act_quant(X)
    assert np.array_equal(host(Xq), xq)
    assert np.array_equal(f32_bits(host(s_x)), f32_bits(sx))
    check_forward_y(Y, sbn.SBN_BF16, O.accumulate(xq, eff), sw, sx)


# ------------------------------------------------------------------ optional non-finite input check
def test_check_finite_rejects_nonfinite_inputs(monkeypatch):
    """SBN_CHECK_FINITE=1: a NaN or Inf in W, G, X or dY is rejected with
    SBN_ERR_VALUE before anything launches (outputs untouched); finite inputs
    give the unchecked results; without the variable nothing is scanned."""
    import torch
    R, K, T = 64, 256, 24
    W = gaussian_bf16((R, K), 0.02, seed=5, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=5, stream=1)
    dY = gaussian_bf16((T, R), 1e-2, seed=5, stream=2)
    ref = sbn.sbn_mask_ternarize_pack(dev_bf16(W), 2, 4)
    monkeypatch.setenv("SBN_CHECK_FINITE", "1")
    got = sbn.sbn_mask_ternarize_pack(dev_bf16(W), 2, 4)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ref, got))
    Xq, s_x = sbn.sbn_act_quant(dev_bf16(X))
    codes, meta, s_w = got

    def rejected(call):
        with pytest.raises(sbn.SbnError) as ei:
            call()
        assert ei.value.status == sbn.SBN_ERR_VALUE, str(ei.value)

    for bits, where in ((0x7FC0, (3, 100)), (0x7F80, (63, 255)), (0xFF80, (0, 0))):   # NaN, +Inf, -Inf
        Wb = W.copy(); Wb[where] = bits
        codes2 = torch.full_like(codes, 0x5A)
        rejected(lambda: sbn.sbn_mask_ternarize_pack(dev_bf16(Wb), 2, 4, codes=codes2))
        assert bool((codes2 == 0x5A).all()), "output touched"
        Xb = X.copy(); Xb[min(where[0], T - 1), where[1]] = bits
        rejected(lambda: sbn.sbn_act_quant(dev_bf16(Xb)))
        rejected(lambda: sbn.sbn_forward(dev_bf16(W), dev_bf16(Xb), 2, 4))
        dYb = dY.copy(); dYb[min(where[0], T - 1), min(where[1], R - 1)] = bits
        rejected(lambda: sbn.sbn_backward(dev_bf16(dYb), Xq, s_x, codes, meta, s_w, 2, 4))
    G = np.zeros((R, K), dtype=np.float32); G[7, 9] = np.inf
    rejected(lambda: sbn.sbn_sgd_update_pack(dev_bf16(W), dev(G), 0.1, 2, 4))
    # padding columns past K are not scanned
    Wp = np.full((R, K + 64), 0x7FC0, dtype=np.uint16); Wp[:, :K] = W
    got = sbn.sbn_mask_ternarize_pack(dev_bf16(Wp)[:, :K], 2, 4)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ref, got))
    monkeypatch.delenv("SBN_CHECK_FINITE")
    Wb = W.copy(); Wb[3, 100] = 0x7FC0
    sbn.sbn_mask_ternarize_pack(dev_bf16(Wb), 2, 4)        # outside the contract, but not rejected
    torch.cuda.synchronize()
