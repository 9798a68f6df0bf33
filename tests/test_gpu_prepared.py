"""GPU parity of the prepared GEMM weight: the GEMM on a weight operand built
once from the packed planes must give the oracle's int32 accumulators bit for
bit, and int32, float32 and bf16 outputs identical bit for bit to
sbn_sparse_ternary_gemm on the same planes, for every ratio, ragged shapes,
each token-tile width, and one prepared weight reused across calls."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import sparse_linear_layers_02_amd as sbn
from gpu_util import dev, dev_bf16, host
from workloads import WORKLOADS, gaussian_bf16

pytestmark = pytest.mark.gpu

ALL_NM = [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (6, 8), (7, 8), (8, 8)]
YDTS = (sbn.SBN_I32_ACC, sbn.SBN_F32, sbn.SBN_BF16)


def out_buffer(T, R, ydt, device):
    import torch
    ldy = (R + 7) // 8 * 8
    dt = {sbn.SBN_F32: torch.float32, sbn.SBN_BF16: torch.bfloat16, sbn.SBN_I32_ACC: torch.int32}[ydt]
    full = torch.full((T, ldy), 77, dtype=dt, device=device)
    return full, full[:, :R]


def run_both(Xq, s_x, codes, meta, prepared, s_w, R, n, m, ydt):
    """(prepared-path Y, per-call-expansion Y) as host arrays; padding columns untouched."""
    import torch
    T = Xq.shape[0]
    fa, Ya = out_buffer(T, R, ydt, Xq.device)
    fb, Yb = out_buffer(T, R, ydt, Xq.device)
    sbn.sbn_sparse_ternary_gemm_prepared(Xq, s_x, prepared, s_w, R, n, m, ydt=ydt, Y=Ya)
    sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, R, n, m, ydt=ydt, Y=Yb)
    torch.cuda.synchronize()
    if fa.shape[1] > R:
        assert bool((fa[:, R:] == 77).all()), "write past R"
    a, b = host(Ya.contiguous()), host(Yb.contiguous())
    return a, b


def as_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 or a.itemsize == 2 else a.view(np.uint32)


def check_prepared(T, R, K, n, m, seed=0, oracle=True):
    import torch
    W = gaussian_bf16((R, K), 0.02, seed=seed, stream=0)
    X = gaussian_bf16((T, K), 1.0, seed=seed, stream=1)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m)
    Xq, s_x = sbn.sbn_act_quant(dev_bf16(X))
    prepared = sbn.sbn_prepare_gemm_weight(codes, meta, R, K, n, m)
    torch.cuda.synchronize()
    for ydt in YDTS:
        a, b = run_both(Xq, s_x, codes, meta, prepared, s_w, R, n, m, ydt)
        assert np.array_equal(as_bits(a), as_bits(b)), \
            f"ydt {ydt}: prepared differs from per-call at {np.argwhere(as_bits(a) != as_bits(b))[:3].tolist()}"
        if oracle and ydt == sbn.SBN_I32_ACC:
            f = O.forward(W, X, n, m)
            assert np.array_equal(a.astype(np.int64), f["acc"]), \
                f"acc differ at {np.argwhere(a != f['acc'])[:3].tolist()}"
    return codes, meta, s_w, prepared


@pytest.mark.parametrize("n,m", ALL_NM)
def test_prepared_ragged_all_ratios(n, m):
    check_prepared(300, 520, 576, n, m, seed=n + 10 * m)   # two token tiles, three row tiles, short K


@pytest.mark.parametrize("T,R,K", [(1, 16, 64), (5, 33, 128), (17, 33, 128), (257, 257, 640)])
def test_prepared_small_edges(T, R, K):
    check_prepared(T, R, K, 2, 4, seed=T)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
@pytest.mark.parametrize("T", [497, 200, 100])
def test_prepared_token_tile_widths(T, n, m):
    # 96 row tiles less 37 rows: 256-, 128- and 64-token block tiles (dense stops at 128)
    check_prepared(T, 96 * 256 - 37, 256, n, m, seed=T + n, oracle=False)


def test_prepared_weight_reused_across_calls():
    """One prepared weight serves calls of different token counts; the planes
    it came from can be freed first."""
    import torch
    R, K, n, m = 520, 1024, 2, 4
    W = gaussian_bf16((R, K), 0.02, seed=3, stream=0)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m)
    prepared = sbn.sbn_prepare_gemm_weight(codes, meta, R, K, n, m)
    ref_planes = (codes.clone(), meta.clone())
    del codes, meta
    torch.cuda.synchronize()
    for T in (700, 33, 1):
        X = gaussian_bf16((T, K), 1.0, seed=T, stream=1)
        Xq, s_x = sbn.sbn_act_quant(dev_bf16(X))
        a, b = run_both(Xq, s_x, ref_planes[0], ref_planes[1], prepared, s_w, R, n, m, sbn.SBN_I32_ACC)
        f = O.forward(W, X, n, m)
        assert np.array_equal(a.astype(np.int64), f["acc"]), f"T={T}: acc differ"
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name,n,m", [("prefill", 2, 4), ("prefill", 6, 8)])
def test_prepared_full_size_equals_per_call(name, n, m):
    """At the prefill size the outputs equal the per-call-expansion GEMM's bit
    for bit (that GEMM is checked against the oracle at this size elsewhere)."""
    import torch
    wl = WORKLOADS[name]
    W, X = wl.weights(0), wl.activations(0)
    R, K = W.shape
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), n, m)
    Xq, s_x = sbn.sbn_act_quant(dev_bf16(X))
    prepared = sbn.sbn_prepare_gemm_weight(codes, meta, R, K, n, m)
    for ydt in (sbn.SBN_I32_ACC, sbn.SBN_BF16):
        a, b = run_both(Xq, s_x, codes, meta, prepared, s_w, R, n, m, ydt)
        assert np.array_equal(as_bits(a), as_bits(b)), f"ydt {ydt}: prepared differs from per-call"
    torch.cuda.synchronize()
