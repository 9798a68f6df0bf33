"""GPU parity of the joint 2:4 code: the repack of 2:4 packed planes into it
(both planes bit for bit against the oracle's pack_j6 of the effective
weights) and the decode GEMV on it, one weight and a device table of
weights (int32 accumulators, float32 and bf16 outputs bit for bit against
the oracle), at small ragged shapes, one to four waves' K ranges, and the
measured decode pool (128 weights of 4096 x 4096, one launch)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import sparse_linear_layers_02_amd as sbn
from gpu_util import dev, dev_bf16, f32_bits, host
from workloads import WORKLOADS, gaussian_bf16

pytestmark = pytest.mark.gpu


def packed_case(R, K, seed):
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    eff, mask, sw = O.quant_then_mask(W, 2, 4)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), 2, 4)
    return eff, sw, codes, meta, s_w


def check_repack(R, K, seed):
    import torch
    eff, sw, codes, meta, s_w = packed_case(R, K, seed)
    nib, hpl = sbn.sbn_repack_j6(codes, meta, R, K)
    torch.cuda.synchronize()
    wn, wh = O.pack_j6(eff)
    gn = host(nib)[: wn.size].reshape(wn.shape)
    gh = host(hpl)[: wh.size].reshape(wh.shape)
    assert np.array_equal(gn, wn), f"nibble plane differs at {np.argwhere(gn != wn)[:3].tolist()}"
    assert np.array_equal(gh, wh), f"h plane differs at {np.argwhere(gh != wh)[:3].tolist()}"
    return eff, sw, codes, meta, s_w, nib, hpl


@pytest.mark.parametrize("R,K", [(1, 64), (37, 64), (203, 320), (1000, 1024), (5, 4160)])
def test_repack_j6_matches_oracle(R, K):
    check_repack(R, K, seed=R + K)


def test_repack_j6_decode_size():
    check_repack(4096, 4096, seed=3)


def expect(acc, sw, sx, ydt):
    if ydt == sbn.SBN_I32_ACC:
        return acc
    if ydt == sbn.SBN_F32:
        return f32_bits(O.output_f32(acc, sw, sx))
    return O.output_bf16(acc, sw, sx)


def got_bits(Y, ydt):
    h = host(Y.contiguous())
    return h.astype(np.int64) if ydt == sbn.SBN_I32_ACC else (f32_bits(h) if ydt == sbn.SBN_F32 else h)


@pytest.mark.parametrize("K", [1024, 2048, 3072, 4096])
@pytest.mark.parametrize("T,R", [(1, 37), (5, 1000), (16, 203)])
def test_gemv_j6_matches_oracle(K, T, R):
    """Every output in every dtype; padding columns untouched; the bf16 output
    equals the packed-weight GEMV's."""
    import torch
    eff, sw, codes, meta, s_w, nib, hpl = check_repack(R, K, seed=K + T + R)
    xq, sx = O.act_quant(gaussian_bf16((T, K), 1.0, seed=K + R, stream=1))
    Xq, s_x = dev(xq), dev(sx)
    acc = O.accumulate(xq, eff)
    ld = (R + 7) // 8 * 8
    for ydt, dt in ((sbn.SBN_I32_ACC, torch.int32), (sbn.SBN_F32, torch.float32), (sbn.SBN_BF16, torch.bfloat16)):
        full = torch.full((T, ld), 77, dtype=dt, device="cuda")
        print(f"gemv_j6 K={K} T={T} R={R} ydt={ydt}", flush=True)
        sbn.sbn_ternary_gemv_j6(Xq, s_x, nib, hpl, s_w, R, ydt=ydt, Y=full[:, :R])
        torch.cuda.synchronize()
        got, want = got_bits(full[:, :R], ydt), expect(acc, sw, sx, ydt)
        bad = got != want
        assert not bad.any(), f"ydt {ydt}: {bad.sum()} differ, first at {np.argwhere(bad)[0].tolist()}"
        if ld > R:
            assert bool((full[:, R:] == 77).all()), "write past R"
    ref = sbn.sbn_sparse_ternary_gemv(Xq, s_x, codes, meta, s_w, R, 2, 4)
    yb = sbn.sbn_ternary_gemv_j6(Xq, s_x, nib, hpl, s_w, R)
    torch.cuda.synchronize()
    assert np.array_equal(host(yb.contiguous()), host(ref.contiguous()))


@pytest.mark.parametrize("count,R,K,T", [(1, 37, 1024, 1), (130, 48, 1024, 16), (5, 203, 4096, 3)])
def test_gemv_j6_table_matches_oracle(count, R, K, T):
    import torch
    xq, sx = O.act_quant(gaussian_bf16((T, K), 1.0, seed=count + K, stream=1))
    Xq, s_x = dev(xq), dev(sx)
    cases = [packed_case(R, K, seed=500 + b) for b in range(count)]
    planes = [sbn.sbn_repack_j6(c[2], c[3], R, K) for c in cases]
    tab = sbn.GemvTable.joint([p[0] for p in planes], [p[1] for p in planes], [c[4] for c in cases], R, K, T=T,
                              ydt=sbn.SBN_BF16)
    print(f"gemv_j6_table count={count} R={R} K={K} T={T}", flush=True)
    sbn.sbn_ternary_gemv_j6_table(Xq, s_x, tab)
    torch.cuda.synchronize()
    for b, c in enumerate(cases):
        want = O.output_bf16(O.accumulate(xq, c[0]), c[1], sx)
        got = host(tab.Ys[b].contiguous())
        assert np.array_equal(got, want), f"weight {b}: {(got != want).sum()} differ"


def test_gemv_j6_table_decode_pool_full_size():
    """The measured launch: 128 joint-coded weights of 4096 x 4096 in one table,
    bf16, every decode batch size; weight b is the decode weight with its rows
    rotated by b, so its outputs are the oracle's rotated by b (every output of
    every weight checked)."""
    import torch
    wl = WORKLOADS["decode"]
    R, K, P = wl.R, wl.K, 128
    W0 = wl.weights(0)
    eff, _, sw = O.quant_then_mask(W0, 2, 4)
    Wd0 = dev_bf16(W0)
    planes, s_ws = [], []
    for b in range(P):
        codes, meta, s_w = sbn.sbn_mask_ternarize_pack(torch.roll(Wd0, shifts=b, dims=0), 2, 4)
        planes.append(sbn.sbn_repack_j6(codes, meta, R, K))
        s_ws.append(s_w)
        del codes, meta
    for T in wl.Ts:
        xq, sx = O.act_quant(wl.activations(seed=0, T=T))
        want0 = O.output_bf16(O.accumulate(xq, eff), sw, sx)
        tab = sbn.GemvTable.joint([p[0] for p in planes], [p[1] for p in planes], s_ws, R, K, T=T)
        print(f"gemv_j6_table decode pool T={T}", flush=True)
        sbn.sbn_ternary_gemv_j6_table(dev(xq), dev(sx), tab)
        torch.cuda.synchronize()
        for b in range(P):
            got = host(tab.Ys[b].contiguous())
            bad = got != np.roll(want0, b, axis=1)
            assert not bad.any(), f"T={T} weight {b}: {bad.sum()} differ"
        del tab
