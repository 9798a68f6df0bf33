"""GPU parity of the wide-tile sparse GEMM (448 rows x 256 tokens per block,
the smfmac ratios 2:4, 1:4 and 2:8): forced on for ragged shapes that put
rows past the last tile, tokens past the last token tile and one to nine K
steps of 128 (odd and even step counts, a K tail), every int32 accumulator,
f32 and bf16 output bit for bit against the oracle, from packed planes and
from a prepared weight (the kernel then loads the activations straight from
row-major Xq, tokens past T and the bytes past Xq's end reading as zero); and
at the full prefill shape, where it is the default, the square 256 x 256
tiles forced on give the same outputs."""
from __future__ import annotations

import numpy as np
import pytest

import sparse_linear_layers_02_amd as sbn
from test_gpu_parity import check_outputs, forward_case, run_matmul
from test_gpu_prepared import check_prepared
from gpu_util import dev, dev_bf16
import oracle as O
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (2, 8)])
@pytest.mark.parametrize("T,R,K", [(300, 520, 576), (17, 33, 128), (513, 1000, 1152), (256, 448, 256),
                                   (64, 7000, 384), (40, 100, 64)])
def test_wide_tile_forced_matches_oracle(monkeypatch, T, R, K, n, m):
    monkeypatch.setenv("SBN_GEMM_TILE", "wide")
    print(f"wide GEMM {n}:{m} T={T} R={R} K={K}", flush=True)
    f, Xq, s_x, codes, meta, s_w = forward_case(T, R, K, n, m, seed=T + R + n)
    check_outputs("gemm", f, Xq, s_x, codes, meta, s_w, R, n, m)


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (2, 8)])
@pytest.mark.parametrize("T,R,K", [(300, 520, 576), (17, 33, 128), (259, 900, 64)])
def test_wide_tile_forced_prepared_weight(monkeypatch, T, R, K, n, m):
    monkeypatch.setenv("SBN_GEMM_TILE", "wide")
    print(f"wide GEMM on a prepared weight {n}:{m} T={T} R={R} K={K}", flush=True)
    check_prepared(T, R, K, n, m, seed=T + K + n)


def test_wide_and_square_tiles_agree_at_prefill_size(monkeypatch):
    wl = WORKLOADS["prefill"]
    W, X = wl.weights(0), wl.activations(0)
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(W), 2, 4)
    xq, sx = O.act_quant(X)
    outs = {}
    for tile in ("wide", "square"):
        monkeypatch.setenv("SBN_GEMM_TILE", tile)
        print(f"prefill GEMM, {tile} tiles", flush=True)
        outs[tile] = run_matmul("gemm", dev(xq), dev(sx), codes, meta, s_w, wl.R, 2, 4, sbn.SBN_BF16)
    assert np.array_equal(outs["wide"], outs["square"])
