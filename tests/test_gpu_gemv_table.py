"""GPU parity of the table GEMV (the weights of one launch listed in a table in
device memory, any count): every output of every weight against the oracle
-- int32 accumulators bit for bit, float32 and bf16 outputs bit for bit
against the oracle's rounding of the exact accumulator -- for packed 2:4 and
6:8 weights and for decode planes, at small ragged shapes spanning one to
four waves' K ranges and more weights than one by-value launch holds, and at
the decode pool of the measured step (128 weights of 4096 x 4096, one launch
per ratio)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import sparse_linear_layers_02_amd as sbn
from gpu_util import dev, dev_bf16, f32_bits, host
from workloads import WORKLOADS, gaussian_bf16

pytestmark = pytest.mark.gpu

YDTS = (sbn.SBN_I32_ACC, sbn.SBN_F32, sbn.SBN_BF16)


def expect(acc, sw, sx, ydt):
    """The oracle's output of dtype ydt (as raw bits for the float outputs)."""
    if ydt == sbn.SBN_I32_ACC:
        return acc
    if ydt == sbn.SBN_F32:
        return f32_bits(O.output_f32(acc, sw, sx))
    return O.output_bf16(acc, sw, sx)


def got_bits(Y, ydt):
    h = host(Y.contiguous())
    if ydt == sbn.SBN_I32_ACC:
        return h.astype(np.int64)
    if ydt == sbn.SBN_F32:
        return f32_bits(h)
    return h


def weights(count, R, K, seed):
    return [gaussian_bf16((R, K), 0.02 * (1 + b % 3), seed=seed + b, stream=0) for b in range(count)]


def build_table(Ws, R, K, n, m, T, ydt, d2):
    import torch
    packed = [sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m) for W in Ws]
    s_ws = [p[2] for p in packed]
    ld = (R + 7) // 8 * 8
    dt = {sbn.SBN_F32: torch.float32, sbn.SBN_BF16: torch.bfloat16, sbn.SBN_I32_ACC: torch.int32}[ydt]
    fulls = [torch.full((T, ld), 77, dtype=dt, device="cuda") for _ in Ws]
    Ys = [f[:, :R] for f in fulls]
    if d2:
        planes = [sbn.sbn_repack_d2(p[0], p[1], R, K, n, m) for p in packed]
        tab = sbn.GemvTable.planes(planes, s_ws, R, K, T=T, ydt=ydt, Ys=Ys)
    else:
        tab = sbn.GemvTable([p[0] for p in packed], None if n == m else [p[1] for p in packed], s_ws, R, K, n, m,
                            T=T, ydt=ydt, Ys=Ys)
    return tab, fulls


def run_table(Xq, s_x, tab):
    import torch
    if tab.d2:
        sbn.sbn_ternary_gemv_d2_table(Xq, s_x, tab)
    else:
        sbn.sbn_sparse_ternary_gemv_table(Xq, s_x, tab)
    torch.cuda.synchronize()


@pytest.mark.parametrize("n,m,d2", [(2, 4, False), (6, 8, False), (2, 4, True), (6, 8, True), (1, 4, True)])
@pytest.mark.parametrize("count,R,K,T", [(1, 37, 1024, 1), (5, 203, 3072, 5), (130, 48, 1024, 16), (3, 1000, 4096, 2)])
def test_gemv_table_matches_oracle(n, m, d2, count, R, K, T):
    """Every weight's output in every dtype; the padding columns of each Y stay
    untouched.  130 weights is more than one by-value launch holds; R = 37
    and 203 leave ragged row groups; K = 1024 .. 4096 gives one to four waves
    a range."""
    Ws = weights(count, R, K, seed=1000 * n + 10 * count + K // 1024)
    X = gaussian_bf16((T, K), 1.0, seed=count + K + T, stream=1)
    xq, sx = O.act_quant(X)
    Xq, s_x = dev(xq), dev(sx)
    refs = []
    for W in Ws:
        eff, _, sw = O.quant_then_mask(W, n, m)
        refs.append((O.accumulate(xq, eff), sw))
    for ydt in YDTS:
        tab, fulls = build_table(Ws, R, K, n, m, T, ydt, d2)
        print(f"table gemv {n}:{m} d2={d2} count={count} R={R} K={K} T={T} ydt={ydt}", flush=True)
        run_table(Xq, s_x, tab)
        for b, (acc, sw) in enumerate(refs):
            got = got_bits(tab.Ys[b], ydt)
            want = expect(acc, sw, sx, ydt)
            bad = got != want
            assert not bad.any(), f"weight {b} ydt {ydt}: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
            if fulls[b].shape[1] > R:
                assert bool((fulls[b][:, R:] == 77).all()), f"weight {b}: write past R"


@pytest.mark.parametrize("K", [1024, 3072, 4096])
def test_gemv_table_one_token_kernel(K):
    """One token over 240 weights of R = 203 rows (3120 row groups, at least
    one for each of the 3072 resident waves of the one-token 2:4 kernel, which
    then takes the launch): every output in every dtype against the oracle,
    ragged last row group included, and the padding columns untouched.  Eight
    distinct weights, each listed 30 times with its own output."""
    import torch
    R, T, n, m, count = 203, 1, 2, 4, 240
    Wd = weights(8, R, K, seed=7000 + K // 1024)
    Ws = [Wd[b % 8] for b in range(count)]
    X = gaussian_bf16((T, K), 1.0, seed=K + 11, stream=1)
    xq, sx = O.act_quant(X)
    Xq, s_x = dev(xq), dev(sx)
    refs = []
    for W in Wd:
        eff, _, sw = O.quant_then_mask(W, n, m)
        refs.append((O.accumulate(xq, eff), sw))
    for ydt in YDTS:
        tab, fulls = build_table(Ws, R, K, n, m, T, ydt, False)
        print(f"one-token table gemv K={K} ydt={ydt}", flush=True)
        torch.cuda.synchronize()
        sbn.sbn_profile_reset()
        sbn.sbn_profile_enable(True, None)
        run_table(Xq, s_x, tab)
        sbn.sbn_profile_enable(False)
        assert "gemv_tok1_24" in sbn.sbn_profile_dump(), "the one-token kernel did not run"
        for b in range(count):
            acc, sw = refs[b % 8]
            got = got_bits(tab.Ys[b], ydt)
            want = expect(acc, sw, sx, ydt)
            bad = got != want
            assert not bad.any(), f"weight {b} ydt {ydt}: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
            assert bool((fulls[b][:, R:] == 77).all()), f"weight {b}: write past R"


def test_gemv_table_reused_with_new_activations():
    """A table is built once and called again with other activations: the
    second call's outputs are the oracle's for the new activations."""
    n, m, R, K, T, count = 2, 4, 96, 2048, 3, 4
    Ws = weights(count, R, K, seed=77)
    tab, _ = build_table(Ws, R, K, n, m, T, sbn.SBN_BF16, False)
    effs = [O.quant_then_mask(W, n, m) for W in Ws]
    for seed in (1, 2):
        xq, sx = O.act_quant(gaussian_bf16((T, K), 1.0, seed=seed, stream=1))
        run_table(dev(xq), dev(sx), tab)
        for b, (eff, _, sw) in enumerate(effs):
            want = O.output_bf16(O.accumulate(xq, eff), sw, sx)
            assert np.array_equal(host(tab.Ys[b].contiguous()), want), f"activations {seed}, weight {b}"


@pytest.mark.parametrize("n,m,d2", [(2, 4, False), (6, 8, False), (6, 8, True)])
def test_gemv_table_decode_pool_full_size(n, m, d2):
    """The measured decode step's launch: 128 weights of 4096 x 4096 in one
    table, bf16 outputs, T = 1 (and the other decode batch sizes).  Weight b
    is the decode workload's weight with its rows rotated by b, so each
    weight's outputs are the oracle's outputs of the base weight rotated by b
    (the scale, an absmean over the whole weight, is unchanged): every output
    of all 128 weights is checked, and a weight that read another entry's
    pointers would show rotated rows."""
    import torch
    wl = WORKLOADS["decode"]
    R, K, P = wl.R, wl.K, 128
    W0 = wl.weights(0)
    eff, _, sw = O.quant_then_mask(W0, n, m)
    Wd0 = dev_bf16(W0)
    packed = [sbn.sbn_mask_ternarize_pack(torch.roll(Wd0, shifts=b, dims=0), n, m) for b in range(P)]
    s_ws = [p[2] for p in packed]
    assert all(f32_bits(host(s))[0] == f32_bits(sw) for s in s_ws[:2])
    planes = [sbn.sbn_repack_d2(p[0], p[1], R, K, n, m) for p in packed] if d2 else None
    for T in wl.Ts:
        xq, sx = O.act_quant(wl.activations(seed=0, T=T))
        acc0 = O.accumulate(xq, eff)
        want0 = O.output_bf16(acc0, sw, sx)
        if d2:
            tab = sbn.GemvTable.planes(planes, s_ws, R, K, T=T)
        else:
            tab = sbn.GemvTable([p[0] for p in packed], [p[1] for p in packed], s_ws, R, K, n, m, T=T)
        print(f"table gemv decode pool {n}:{m} d2={d2} T={T}", flush=True)
        run_table(dev(xq), dev(sx), tab)
        for b in range(P):
            got = host(tab.Ys[b].contiguous())
            want = np.roll(want0, b, axis=1)
            bad = got != want
            assert not bad.any(), f"T={T} weight {b}: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
        del tab
