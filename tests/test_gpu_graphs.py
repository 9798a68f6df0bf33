"""HIP-graph replays of the one-call forward with the backward, of the fused
SGD step, of the decode-plane GEMV and of the prepared-weight GEMM: every replay, with eager work and
synchronisation between replays, reproduces the eager results bit for bit
(the bench times such replays)."""
from __future__ import annotations

import numpy as np
import pytest

import sparse_linear_layers_02_amd as sbn
from gpu_util import dev, dev_bf16
from workloads import gaussian_bf16

pytestmark = pytest.mark.gpu


def replay_matches(step, outputs, before=None, reps=4):
    import torch
    if before:
        before()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        if before:
            before()
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    if before:
        before()
    with torch.cuda.graph(g):
        step()
    for rep in range(reps):
        for t in outputs:
            t.zero_()                               # eager work between replays
        if before:
            before()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_graph_forward_and_backward(n, m):
    import torch
    T, R, K = 300, 520, 576
    W = dev_bf16(gaussian_bf16((R, K), 0.02, seed=31, stream=0))
    X = dev_bf16(gaussian_bf16((T, K), 1.0, seed=31, stream=1))
    dY = dev_bf16(gaussian_bf16((T, R), 1e-2, seed=31, stream=2))
    cb, mb = sbn.sbn_packed_bytes(R, K, n, m)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    s_w = torch.empty(1, dtype=torch.float32, device="cuda")
    Xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
    s_x = torch.empty(T, dtype=torch.float32, device="cuda")
    Y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((R, K), dtype=torch.float32, device="cuda")
    wf = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_FORWARD, T, R, K, n, m), dtype=torch.uint8, device="cuda")
    wb = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_BACKWARD, T, R, K, n, m), dtype=torch.uint8, device="cuda")

    def step():
        sbn.sbn_forward(W, X, n, m, codes=codes, meta=meta, s_w=s_w, Xq=Xq, s_x=s_x, Y=Y, ws=wf)
        sbn.sbn_backward_ex(dY, Xq, s_x, codes, meta, s_w, n, m, sbn.SBN_GRAD_W_MASKED, dxdt=sbn.SBN_BF16, dX=dX,
                            dW=dW, ws=wb)

    replay_matches(step, [codes, meta, s_w, Xq, s_x, Y, dX, dW])


def test_graph_sgd_update_pack():
    import torch
    R, K = 264, 512
    W0 = dev_bf16(gaussian_bf16((R, K), 0.02, seed=32, stream=0))
    G = dev(np.random.default_rng([32, 9]).standard_normal((R, K)).astype(np.float32) * np.float32(1e-2))
    W = W0.clone()
    cb, mb = sbn.sbn_packed_bytes(R, K, 6, 8)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    s_w = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_PACK, 0, R, K, 6, 8), dtype=torch.uint8, device="cuda")

    def step():
        sbn.sbn_sgd_update_pack(W, G, 0.05, 6, 8, codes=codes, meta=meta, s_w=s_w, ws=ws)

    replay_matches(step, [W, codes, meta, s_w], before=lambda: W.copy_(W0))   # each replay updates W0 once


def test_graph_decode_plane_batched():
    import torch
    T, R, K, count = 4, 600, 2048, 5
    Xq, s_x = sbn.sbn_act_quant(dev_bf16(gaussian_bf16((T, K), 1.0, seed=33, stream=1)))
    d2s, sws = [], []
    for b in range(count):
        codes, meta, s_w = sbn.sbn_mask_ternarize_pack(dev_bf16(gaussian_bf16((R, K), 0.02, seed=40 + b, stream=0)), 6, 8)
        d2s.append(sbn.sbn_repack_d2(codes, meta, R, K, 6, 8))
        sws.append(s_w)
    Ys = [torch.empty((T, R), dtype=torch.bfloat16, device="cuda") for _ in range(count)]

    def step():
        sbn.sbn_ternary_gemv_d2_batched(Xq, s_x, d2s, sws, R, Ys=Ys)

    replay_matches(step, Ys)


@pytest.mark.parametrize("n,m", [(2, 4), (6, 8)])
def test_graph_prepare_and_prepared_gemm(n, m):
    """The weight preparation and two prepared GEMMs of different token counts
    in one graph."""
    import torch
    R, K = 520, 576
    W = dev_bf16(gaussian_bf16((R, K), 0.02, seed=34, stream=0))
    codes, meta, s_w = sbn.sbn_mask_ternarize_pack(W, n, m)
    pw = torch.empty(sbn.sbn_gemm_weight_bytes(R, K, n, m), dtype=torch.uint8, device="cuda")
    xs = [sbn.sbn_act_quant(dev_bf16(gaussian_bf16((T, K), 1.0, seed=T, stream=1))) for T in (300, 7)]
    Ys = [torch.empty((Xq.shape[0], R), dtype=torch.bfloat16, device="cuda") for Xq, _ in xs]

    def step():
        sbn.sbn_prepare_gemm_weight(codes, meta, R, K, n, m, prepared=pw)
        for (Xq, s_x), Y in zip(xs, Ys):
            sbn.sbn_sparse_ternary_gemm_prepared(Xq, s_x, pw, s_w, R, n, m, Y=Y)

    replay_matches(step, [pw] + Ys, before=lambda: pw.zero_())
