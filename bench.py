"""Throughput of the Sparse-BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--min-warmup-ms MS] [--steps-per-graph S]
                    [--workload prefill|train|sweep|decode|speedup]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM:
  prefill (default): mask/ternarize/pack W (per call), act_quant X, sparse
                     ternary GEMM -> bf16 Y (the one-call forward, sbn_forward).  T=4096, R=6912, K=2560, 2:4,
                     X with 1% outliers x20.
  train:             the same plus the dual-STE backward (dX, dW).
                     T=8192, R=11008, K=4096, 6:8, dY ~ N(0, 1e-2).
  sweep:             GEMM alone for N:M in {2:4, 4:8, 6:8, 2:8, 1:4, 8:8},
                     T=2048, R=K=8192, and the pack of W for each ratio
                     (one line per ratio is not the contract; the JSON line
                     carries the list).
  decode:            decode GEMV (T=1, R=K=4096) over pools of 128 distinct
                     packed weights per ratio (2:4 and 6:8), as batched calls
                     of 64 weights; `value` is GB/s of algorithmic bytes.  The
                     line also carries the same step on decode planes
                     (`decode_d2`: the weights repacked into dense 2-bit codes).
  speedup:           sparse against dense at several token counts: the
                     library's 2:4 and 6:8 calls against its own dense
                     ternary (8:8) call and the vendor library's dense bf16
                     and int8 GEMMs (hipBLASLt through torch), prefill shape
                     R=6912, K=2560 at T = 512..8192 and decode shape
                     R=K=4096 at T = 1, 4, 16 (pools above the Infinity
                     Cache); `value` is the 2:4 call's TOPS at T=4096.
`value` is dense-equivalent int8 TOPS of the whole step (2*T*R*K per
forward product; the train step counts its three products), timed over
--steps steps replayed from HIP graphs of --steps-per-graph (4) steps each,
the remainder as one-step replays (the library only enqueues kernels on the
caller's stream, so a step captures cleanly; one replay's host cost then
falls once per four steps), after --warmup steps and untimed
replays up to --min-warmup-ms (100 ms) from the start of the warmup, so the
part's clocks have settled.  One JSON line is printed.  The
same line carries:
  roofline      the dominant kernel's algorithmic ops (or bytes) per launch
                over its average launch time, timed with HIP events that the
                library records around that kernel alone on its own stream,
                against MI355X's published dense peak.  For the GEMM the ops
                are the products the method performs, 2*T*R*K*n/m (pruned
                positions are not work); the dense-equivalent rate and its
                fractions of the dense and 2:4-sparse int8 peaks sit beside it;
  decode_step   the other half of the metric, measured like `--workload
                decode`: GB/s of the batched decode GEMV step over both pools
                with the HBM roofline of each streamed kernel;
  decode_gemv   GB/s of the decode GEMV
                (R = K = 4096, T = 1, 2:4 and 6:8) over a pool of 128 distinct
                packed weights (twice the 256 MB Infinity Cache or more), three
                ways: (i) one call on a cold weight, (ii-a) the pool as
                separate calls replayed as four HIP graphs on four streams,
                (ii-b) the pool as batched calls of 64 weights sharing the
                activations (one launch each), replayed from a HIP graph;
  variants      (train) the SGD step fused with the next pack, and the two
                ablation switches (mask from the ternary weights; dW blocked
                at pruned positions), per kernel;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, with
                all of its BLAS threads and with one (median of 3 each).
Runs on more than one GPU are not supported: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-ternary GEMM dense-equiv int8 TOPS & decode GEMV GB/s, % of MI355X roofline"
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 matrix peak (2:4 structured headline excluded)
PEAK_INT8_SPARSE_TOPS = 10070.0  # the same with 2:4 structured sparsity, dense-equivalent
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-ms", type=float, default=100.0,
                    help="after the warmup steps, replay the step untimed until this much time has passed "
                         "(the part's clocks need tens of ms under load to settle)")
    ap.add_argument("--workload", default="prefill", choices=["prefill", "train", "sweep", "decode", "speedup"])
    ap.add_argument("--steps-per-graph", type=int, default=4,
                    help="prefill/train: steps captured back to back in one replayed HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode GEMV measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (scales the HBM byte counters)")
    return ap.parse_args()


def bf16_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def kernel_avg_ms(prof, name):
    cnt, ms = prof.get(name, (0, 0.0))
    return (ms / cnt if cnt else float("nan")), cnt


def gemv_kernel_name(step, n, m):
    """The name the decode GEMV launches of `step` carry: at 2:4 the library
    launches the one-token kernel (gemv_tok1_24) for one token over a large
    launch and the streamed kernel (gemv_stream_24) otherwise, and the same
    for the joint 2:4 code (n, m = "j", 6: gemv_tok1_j6 / gemv_stream_j6);
    6:8 is always gemv_stream_68."""
    if (n, m) not in ((2, 4), ("j", 6)):
        return f"gemv_stream_{n}{m}"
    prof = profile_pass(step, 1)
    tag = f"{n}{m}"
    return f"gemv_tok1_{tag}" if f"gemv_tok1_{tag}" in prof else f"gemv_stream_{tag}"


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source (the summary records the source hash)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)\s+source_sha256:\s*([0-9a-f]+)\s+source:\s*(\S+)", text)
    if not m:
        return None
    src = os.path.join(ROOT, m.group(3))
    if not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != m.group(2):
        return None
    return float(m.group(1))


GEMM_KERNELS = ("gemm_smfmac_wide", "gemm_smfmac", "gemm_mfma")


def gemm_name_in(prof, default="gemm_smfmac"):
    """The forward GEMM kernel a profile saw (the library picks the wide or the
    square sparse tiles, or the dense kernel, by shape)."""
    for nm in GEMM_KERNELS:
        if nm in prof:
            return nm
    return default


def gemm_roofline(gname, T, R, K, n, m, k_ms, launches, traffic):
    """Roofline of the forward GEMM: `achieved` counts the products the method
    performs, 2*T*R*K*n/m int8 ops (pruned positions are not work), against
    the dense int8 matrix peak.  For 2:4 on the structured-sparse instruction
    that fraction equals the dense-equivalent rate over the 2:4 instruction's
    dense-equivalent peak.  The dense-equivalent rate (2*T*R*K, pruned
    positions counted) and its fractions of both peaks are printed beside it."""
    dense_eq = 2 * T * R * K
    ops = dense_eq * n // m
    ach = ops / (k_ms * 1e-3) / 1e12
    de = dense_eq / (k_ms * 1e-3) / 1e12
    return {"kernel": gname, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_INT8_TOPS, 4), "traffic": traffic,
            "kernel_us": round(k_ms * 1e3, 3), "launches": launches, "ops_per_launch": ops,
            "dense_equivalent": {"TOPS": round(de, 2), "ops_per_launch": dense_eq,
                                 "frac_of_dense_int8_peak": round(de / PEAK_INT8_TOPS, 4),
                                 "frac_of_2_4_sparse_peak": round(de / PEAK_INT8_SPARSE_TOPS, 4)},
            "note": f"int8 multiply-adds count 2 ops; achieved = 2*T*R*K*{n}/{m} (the products the method "
                    "performs) per second over the dense int8 matrix peak"}


# ---------------------------------------------------------------------- steps
def make_forward_step(wl, n, m, with_backward=False):
    import torch
    import sparse_linear_layers_02_amd as sbn
    W = bf16_dev(wl.weights(0))
    X = bf16_dev(wl.activations(0))
    cb, mb = sbn.sbn_packed_bytes(wl.R, wl.K, n, m)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(max(mb, 16), dtype=torch.uint8, device="cuda")
    s_w = torch.empty(1, dtype=torch.float32, device="cuda")
    Xq = torch.empty((wl.T, wl.K), dtype=torch.int8, device="cuda")
    s_x = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    Y = torch.empty((wl.T, wl.R), dtype=torch.bfloat16, device="cuda")
    ws_fwd = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_FORWARD, wl.T, wl.R, wl.K, n, m), dtype=torch.uint8,
                         device="cuda")
    extra = {}
    if with_backward:
        dY = bf16_dev(wl.upstream_grad(0))
        dX = torch.empty((wl.T, wl.K), dtype=torch.bfloat16, device="cuda")
        dW = torch.empty((wl.R, wl.K), dtype=torch.float32, device="cuda")
        ws_bwd = torch.empty(sbn.sbn_workspace_bytes(sbn.SBN_OP_BACKWARD, wl.T, wl.R, wl.K, n, m),
                             dtype=torch.uint8, device="cuda")
        extra = dict(dY=dY, dX=dX, dW=dW, ws_bwd=ws_bwd)

    def step():
        # pack of W, quantization of X and the GEMM, as the one-call forward
        sbn.sbn_forward(W, X, n, m, ydt=sbn.SBN_BF16, codes=codes, meta=meta if mb else None, s_w=s_w, Xq=Xq,
                        s_x=s_x, Y=Y, ws=ws_fwd)
        if with_backward:
            sbn.sbn_backward(extra["dY"], Xq, s_x, codes, meta if mb else None, s_w, n, m, dxdt=sbn.SBN_BF16,
                             dX=extra["dX"], dW=extra["dW"], ws=extra["ws_bwd"])

    return step


def capture_graph(step):
    """One step captured as a HIP graph (the library only enqueues kernels on
    the current stream, so it captures cleanly); None if capture fails."""
    import torch
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        return g
    except Exception as e:                       # pragma: no cover - reported in the JSON line
        print(f"graph capture failed, timing eager launches: {e}", file=sys.stderr)
        return None


MIN_WARMUP_MS = 100.0


def time_steps(step, steps, warmup, kernel=None, use_graph=True, per_graph=1):
    """Timed region: `steps` steps between two synchronisations, replayed from
    HIP graphs when possible -- graphs of `per_graph` steps back to back (the
    host's cost of one replay, a few us, then falls once per `per_graph`
    steps, as it does for the layers of a model captured together), and the
    last steps % per_graph as one-step replays, so exactly `steps` steps run --
    after `warmup` steps and untimed replays until MIN_WARMUP_MS have passed
    (measured on this part: the decode step takes 290-320 us per step in its
    first 10 ms from idle and 262 us from about 25 ms on; the prefill step 100
    us, then 95 us).  Then the same number of eager steps with the library's
    HIP events around `kernel` (all kernels if None) give its average launch
    duration.  Returns (ms_per_step, wall_s, prof, mode)."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    t_warm = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = capture_graph(step) if use_graph else None
    run = g.replay if g is not None else step
    gm = None
    if g is not None and per_graph > 1:
        gm = capture_graph(lambda: [step() for _ in range(per_graph)])
    for _ in range(2):
        run()
        if gm is not None:
            gm.replay()
    torch.cuda.synchronize()
    while (time.perf_counter() - t_warm) * 1e3 < MIN_WARMUP_MS:
        for _ in range(4):
            run()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()                     # barrier (one rank) + sync on both sides
    t0 = time.perf_counter()
    e0.record()
    if gm is not None:
        for _ in range(steps // per_graph):
            gm.replay()
        for _ in range(steps % per_graph):
            run()
    else:
        for _ in range(steps):
            run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    return ms, wall, profile_pass(step, steps, kernel), ("graph" if g is not None else "eager")


def profile_pass(step, steps, kernel=None):
    """Eager steps with the library's HIP events around `kernel` (every kernel
    if None), recorded on the stream each launch goes to.  {name: (n, ms)}."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    torch.cuda.synchronize()
    sbn.sbn_profile_reset()
    sbn.sbn_profile_enable(True, kernel)
    torch.cuda._sleep(5_000_000)     # keep the GPU busy while the host queues the steps, so no
    for _ in range(steps):           # host submission delay falls between a kernel and its events
        step()
    torch.cuda.synchronize()
    sbn.sbn_profile_enable(False)
    return sbn.sbn_profile_dump()


# ---------------------------------------------------------------------- decode GEMV
def decode_gemv(n=2, m=4, T=1, reps=5):
    """Decode GEMV at R = K = 4096 over a pool of 128 distinct packed weights
    (537 MB at 2:4, 671 MB at 6:8: at least twice the 256 MB Infinity Cache, so
    every weight comes from HBM): (i) one call per cold weight, kernel time
    from the library's events; (ii-a) the pool as separate calls, replayed as
    four HIP graphs on four streams so launch ramps overlap; (ii-b) the pool
    as batched calls of 64 weights that share the activations (one launch
    each), replayed from a HIP graph of PASSES passes over the pool; (ii-c)
    the pool as one table call (its weights listed once in a device table:
    one launch), replayed from a HIP graph of PASSES passes.  Every steady
    mode replays its graphs untimed for 30 ms first (the clocks settle under
    load) and times at least 10 ms.  GB/s = algorithmic bytes (packed W +
    Xq + s_x + Y + s_w per weight) / time."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    wl = WORKLOADS["decode"]
    W = bf16_dev(wl.weights(0))
    codes0, meta0, s_w = sbn.sbn_mask_ternarize_pack(W, n, m)
    del W
    cb, mb = sbn.sbn_packed_bytes(wl.R, wl.K, n, m)
    per = cb + mb
    P, B = 128, 64
    assert P * per >= 2 * MALL_BYTES
    codes = [codes0.clone() for _ in range(P)]
    metas = [meta0.clone() for _ in range(P)]
    s_ws = [s_w.clone() for _ in range(P)]
    Xq, s_x = sbn.sbn_act_quant(bf16_dev(wl.activations(0, T=T)))
    Ys = [torch.empty((T, wl.R), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    algo = per + T * wl.K + 4 * T + 2 * T * wl.R + 4

    def call(i):
        sbn.sbn_sparse_ternary_gemv(Xq, s_x, codes[i], metas[i], s_ws[i], wl.R, n, m, Y=Ys[i])

    def batched(b0):
        sbn.sbn_sparse_ternary_gemv_batched(Xq, s_x, codes[b0:b0 + B], metas[b0:b0 + B], s_ws[b0:b0 + B], wl.R, n, m,
                                            Ys=Ys[b0:b0 + B])

    for i in range(P):
        call(i)
    # (i) cold single calls: kernel time from the library's events (gemv only)
    kname = gemv_kernel_name(lambda: call(0), n, m)
    prof = profile_pass(lambda: [call(i) for i in range(P)], 1, kname)
    kern_ms, kcnt = kernel_avg_ms(prof, kname)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def replay_ms(graphs, streams, calls):
        # untimed replays for at least 30 ms (clocks settle under load), then
        # enough timed replays for at least 10 ms
        t_warm = time.perf_counter()
        n_warm = 0
        while (time.perf_counter() - t_warm) * 1e3 < 30.0 or n_warm < 2:
            for g, s_ in zip(graphs, streams):
                with torch.cuda.stream(s_):
                    g.replay()
            for s_ in streams:
                s_.synchronize()
            n_warm += 1
        per = (time.perf_counter() - t_warm) * 1e3 / n_warm
        nrep = max(reps, int(10.0 / max(per, 1e-3)) + 1)
        torch.cuda.synchronize()
        e0.record()
        for s_ in streams:
            s_.wait_event(e0)
        for _ in range(nrep):
            for g, s_ in zip(graphs, streams):
                with torch.cuda.stream(s_):
                    g.replay()
        for s_ in streams:
            torch.cuda.current_stream().wait_stream(s_)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (nrep * calls)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            fn()
        return g

    # (ii-a) separate calls: four graphs (every 4th pool entry each) on four streams
    streams = [torch.cuda.Stream() for _ in range(4)]
    graphs = [capture(lambda b=b: [call(i) for i in range(b, P, 4)]) for b in range(4)]
    ss_ms = replay_ms(graphs, streams, P)
    del graphs
    # (ii-b) batched calls of B weights, one graph of PASSES passes over the pool on one stream
    gb = capture(lambda: [batched(b0) for _ in range(PASSES) for b0 in range(0, P, B)])
    bt_ms = replay_ms([gb], [streams[0]], P * PASSES)
    del gb
    # (ii-c) the pool as one table call (one launch), one graph of PASSES passes on one stream
    tab = sbn.GemvTable(codes, metas, s_ws, wl.R, wl.K, n, m, T=T, Ys=Ys)
    gt = capture(lambda: [sbn.sbn_sparse_ternary_gemv_table(Xq, s_x, tab) for _ in range(PASSES)])
    tb_ms = replay_ms([gt], [streams[0]], P * PASSES)
    del gt, tab
    frac = lambda ms_: round(algo / (ms_ * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    gbps = lambda ms_: round(algo / (ms_ * 1e-3) / 1e9, 1)
    return {
        "workload": f"decode R=K=4096 T={T} {n}:{m}", "algo_bytes_per_weight": algo,
        "pool_MiB": round(P * per / 2 ** 20, 1), "pool_weights": P,
        "single_call": {"kernel_us": round(kern_ms * 1e3, 3), "GBps": gbps(kern_ms), "frac_hbm": frac(kern_ms)},
        "steady_separate_calls_4streams": {"us_per_weight": round(ss_ms * 1e3, 3), "GBps": gbps(ss_ms),
                                           "frac_hbm": frac(ss_ms)},
        f"steady_batched_{B}": {"us_per_weight": round(bt_ms * 1e3, 3), "GBps": gbps(bt_ms), "frac_hbm": frac(bt_ms),
                                "launches_per_pool": P // B, "pool_passes_per_graph": PASSES},
        f"steady_table_{P}": {"us_per_weight": round(tb_ms * 1e3, 3), "GBps": gbps(tb_ms), "frac_hbm": frac(tb_ms),
                              "launches_per_pool": 1, "pool_passes_per_graph": PASSES},
    }


# ---------------------------------------------------------------------- sparse vs dense
SPEEDUP_T_PREFILL = (512, 1024, 2048, 4096, 8192)
SPEEDUP_T_DECODE = (1, 4, 16)
PER_GRAPH = 8                  # prefill calls per replayed graph in the speedup tables


def graph_ms(fn, reps, per=1):
    """Milliseconds per execution of fn (which only enqueues GPU work),
    replayed from a HIP graph of per executions back to back (eager launches
    if capture fails), so that the host's cost of one replay is spread."""
    import torch
    fn()
    torch.cuda.synchronize()
    body = fn if per == 1 else (lambda: [fn() for _ in range(per)])
    g = capture_graph(body)
    run = g.replay if g is not None else body
    t_warm = time.perf_counter()
    run()
    torch.cuda.synchronize()
    while (time.perf_counter() - t_warm) * 1e3 < 20.0:    # untimed replays: clocks settle under load
        run()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per)


def ternary_int8(W):
    """Dense ternary int8 copy of bf16 W [R, K] (absmean scale, no mask): the
    operand of the vendor int8 GEMM that the sparse calls are compared with."""
    import torch
    Wf = W.float()
    s = Wf.abs().mean().clamp_min(1e-5)
    return torch.clamp(torch.round(Wf / s), -1, 1).to(torch.int8)


def speedup_tables(reps):
    """Per-call times of the sparse 2:4 and 6:8 products against dense ones
    over the same activations: the library's dense ternary 8:8 call, and
    torch's bf16 matmul and int8 _int_mm (hipBLASLt).  Prefill: the prefill
    shape at several T, one call per timing, each library ratio both from the
    packed planes and on a weight operand prepared once.  Decode: R = K = 4096 at T = 1, 4,
    16, every weight of a pool of distinct weights at least twice the Infinity
    Cache, as separate calls in one graph (the library's calls also batched, 64
    weights per launch).  A product the vendor library refuses is null, with
    its error."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    out = {"prefill": [], "decode": []}
    # prefill shape
    wl = WORKLOADS["prefill"]
    R, K = wl.R, wl.K
    W = bf16_dev(wl.weights(0))
    Xall = bf16_dev(wl.activations(0, T=max(SPEEDUP_T_PREFILL)))
    packs = {(n, m): sbn.sbn_mask_ternarize_pack(W, n, m) for n, m in ((2, 4), (6, 8), (8, 8))}
    prepared = {nm: sbn.sbn_prepare_gemm_weight(c, mt, R, K, *nm) for nm, (c, mt, _) in packs.items()}
    Wq = ternary_int8(W)
    WqT = Wq.t()

    def vendor(fn):
        try:
            return graph_ms(fn, reps, PER_GRAPH), None
        except Exception as e:          # reported in the row
            return None, f"{type(e).__name__}: {str(e).splitlines()[0][:160]}"

    for T in SPEEDUP_T_PREFILL:
        X = Xall[:T]
        Xq, s_x = sbn.sbn_act_quant(X)
        row = {"T": T, "R": R, "K": K}
        ops = 2 * T * R * K
        for (n, m), (codes, meta, s_w) in packs.items():
            Y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(max(sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, T, R, K, n, m), 256), dtype=torch.uint8,
                             device="cuda")
            ms = graph_ms(lambda: sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, R, n, m, Y=Y, ws=ws),
                          reps, PER_GRAPH)
            row[f"sbn_{n}{m}_us"] = round(ms * 1e3, 2)
            ws = torch.empty(max(sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM_PREPARED, T, R, K, n, m), 256),
                             dtype=torch.uint8, device="cuda")
            pw = prepared[(n, m)]
            ms = graph_ms(lambda: sbn.sbn_sparse_ternary_gemm_prepared(Xq, s_x, pw, s_w, R, n, m, Y=Y, ws=ws),
                          reps, PER_GRAPH)
            row[f"sbn_{n}{m}_prepared_us"] = round(ms * 1e3, 2)
            del Y, ws
        Yb = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        ms, err = vendor(lambda: torch.matmul(X, W.t(), out=Yb))
        row["bf16_us"], row["bf16_error"] = (round(ms * 1e3, 2) if ms else None), err
        Yi = torch.empty((T, R), dtype=torch.int32, device="cuda")
        ms, err = vendor(lambda: torch._int_mm(Xq, WqT, out=Yi))
        row["int8_us"], row["int8_error"] = (round(ms * 1e3, 2) if ms else None), err
        del Yb, Yi
        for key in ("sbn_24", "sbn_68", "sbn_24_prepared", "sbn_68_prepared"):
            t = row[key + "_us"]
            dense = row["sbn_88_prepared_us" if key.endswith("prepared") else "sbn_88_us"]
            row[key + "_TOPS"] = round(ops / (t * 1e-6) / 1e12, 1)
            row[key + "_vs_dense_ternary"] = round(dense / t, 3)
            row[key + "_vs_bf16"] = round(row["bf16_us"] / t, 3) if row["bf16_us"] else None
            row[key + "_vs_int8"] = round(row["int8_us"] / t, 3) if row["int8_us"] else None
        out["prefill"].append({k: v for k, v in row.items() if v is not None or not k.endswith("_error")})
    del W, Xall, packs, prepared, Wq, WqT
    torch.cuda.empty_cache()

    # decode shape, pools above the Infinity Cache
    wl = WORKLOADS["decode"]
    R, K = wl.R, wl.K
    W = bf16_dev(wl.weights(0))
    pools = {}
    for n, m in ((2, 4), (6, 8), (8, 8)):
        codes0, meta0, s_w0 = sbn.sbn_mask_ternarize_pack(W, n, m)
        cb, mb = sbn.sbn_packed_bytes(R, K, n, m)
        P = -(-2 * MALL_BYTES // (cb + mb))
        pools[(n, m)] = dict(P=P, codes=[codes0.clone() for _ in range(P)],
                             metas=[(meta0.clone() if meta0 is not None else None) for _ in range(P)],
                             s_ws=[s_w0.clone() for _ in range(P)])
        del codes0, meta0
    Pb = -(-2 * MALL_BYTES // (2 * R * K))
    Wb = [W.clone() for _ in range(Pb)]
    Pi = -(-2 * MALL_BYTES // (R * K))
    Wi = [ternary_int8(W).t() for _ in range(Pi)]
    del W
    for T in SPEEDUP_T_DECODE:
        X = bf16_dev(wl.activations(0, T=T))
        Xq, s_x = sbn.sbn_act_quant(X)
        row = {"T": T, "R": R, "K": K}
        for (n, m), p in pools.items():
            P = p["P"]
            Ys = [torch.empty((T, R), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
            ws = torch.empty(max(sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMV, T, R, K, n, m), 256), dtype=torch.uint8,
                             device="cuda")
            ms = graph_ms(lambda: [sbn.sbn_sparse_ternary_gemv(Xq, s_x, p["codes"][i], p["metas"][i], p["s_ws"][i],
                                                                R, n, m, Y=Ys[i], ws=ws) for i in range(P)], reps)
            row[f"sbn_{n}{m}_us"] = round(ms * 1e3 / P, 3)
            if (n, m) != (8, 8):
                ms = graph_ms(lambda: [sbn.sbn_sparse_ternary_gemv_batched(
                    Xq, s_x, p["codes"][b:b + BATCH], p["metas"][b:b + BATCH], p["s_ws"][b:b + BATCH], R, n, m,
                    Ys=Ys[b:b + BATCH]) for b in range(0, P, BATCH)], reps)
                row[f"sbn_{n}{m}_batched_us"] = round(ms * 1e3 / P, 3)
                tab = sbn.GemvTable(p["codes"], p["metas"], p["s_ws"], R, K, n, m, T=T, Ys=Ys)
                ms = graph_ms(lambda: sbn.sbn_sparse_ternary_gemv_table(Xq, s_x, tab), reps)
                row[f"sbn_{n}{m}_table_us"] = round(ms * 1e3 / P, 3)
                del tab
            if (n, m) == (6, 8):                       # the same weights as decode planes (2 bits per weight)
                Pd = -(-2 * MALL_BYTES // (R * K // 4))
                d2s = [sbn.sbn_repack_d2(p["codes"][i % P], p["metas"][i % P], R, K, n, m) for i in range(Pd)]
                sds = [p["s_ws"][i % P] for i in range(Pd)]
                Yd = [torch.empty((T, R), dtype=torch.bfloat16, device="cuda") for _ in range(Pd)]
                ms = graph_ms(lambda: [sbn.sbn_ternary_gemv_d2_batched(
                    Xq, s_x, d2s[b:b + BATCH], sds[b:b + BATCH], R, Ys=Yd[b:b + BATCH])
                    for b in range(0, Pd, BATCH)], reps)
                row["sbn_68_d2_batched_us"] = round(ms * 1e3 / Pd, 3)
                tab = sbn.GemvTable.planes(d2s, sds, R, K, T=T, Ys=Yd)
                ms = graph_ms(lambda: sbn.sbn_ternary_gemv_d2_table(Xq, s_x, tab), reps)
                row["sbn_68_d2_table_us"] = round(ms * 1e3 / Pd, 3)
                del tab
                del d2s, sds, Yd
            del Ys, ws
        Yb = [torch.empty((T, R), dtype=torch.bfloat16, device="cuda") for _ in range(Pb)]
        ms, err = vendor(lambda: [torch.matmul(X, Wb[i].t(), out=Yb[i]) for i in range(Pb)])
        row["bf16_us"], row["bf16_error"] = (round(ms * 1e3 / Pb, 3) if ms else None), err
        Yi = [torch.empty((T, R), dtype=torch.int32, device="cuda") for _ in range(Pi)]
        ms, err = vendor(lambda: [torch._int_mm(Xq, Wi[i], out=Yi[i]) for i in range(Pi)])
        row["int8_us"], row["int8_error"] = (round(ms * 1e3 / Pi, 3) if ms else None), err
        del Yb, Yi
        for key in ("sbn_24", "sbn_68", "sbn_24_batched", "sbn_68_batched", "sbn_68_d2_batched", "sbn_24_table",
                    "sbn_68_table", "sbn_68_d2_table"):
            t = row[key + "_us"]
            row[key + "_vs_dense_ternary"] = round(row["sbn_88_us"] / t, 3)
            row[key + "_vs_bf16"] = round(row["bf16_us"] / t, 3) if row["bf16_us"] else None
            row[key + "_vs_int8"] = round(row["int8_us"] / t, 3) if row["int8_us"] else None
        row["pool_weights"] = {f"{n}:{m}": p["P"] for (n, m), p in pools.items()} | {"bf16": Pb, "int8": Pi}
        out["decode"].append({k: v for k, v in row.items() if v is not None or not k.endswith("_error")})
    return out


# ---------------------------------------------------------------------- variants beside the path
def variants_extras(wl, reps=10):
    """The SGD step fused with the next pack, and the two ablation switches, at
    the train shape, timed per kernel with the library's events:
      sgd_update_pack   sgd_abs_sum (W, G read, W written in place, exact sum
                        of the new |W|) + mask_pack, against the plain pack
                        (abs_sum + mask_pack); HBM roofline of the fused call
                        from its algorithmic bytes (W read twice and written
                        once, G read once, planes written);
      mask_from_ternary the pack with the mask from |q|;
      grad_w_masked     gemm_dw with dW blocked at pruned positions, against
                        the dense-gradient gemm_dw."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    n, m = wl.nm[0]
    R, K = wl.R, wl.K
    W = bf16_dev(wl.weights(0))
    G = torch.randn((R, K), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(0))
    G.mul_(1e-2)
    cb, mb = sbn.sbn_packed_bytes(R, K, n, m)
    codes = torch.empty(cb, dtype=torch.uint8, device="cuda")
    meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
    s_w = torch.empty(1, dtype=torch.float32, device="cuda")

    def kernels(fn_):
        fn_()
        torch.cuda.synchronize()
        prof = profile_pass(fn_, reps)
        return {k: v[1] / v[0] * 1e3 for k, v in prof.items() if v[0]}

    plain = kernels(lambda: sbn.sbn_mask_ternarize_pack(W, n, m, codes=codes, meta=meta, s_w=s_w))
    tern = kernels(lambda: sbn.sbn_mask_ternarize_pack_ex(W, n, m, sbn.SBN_MASK_FROM_TERNARY, codes=codes,
                                                          meta=meta, s_w=s_w))
    fused = kernels(lambda: sbn.sbn_sgd_update_pack(W, G, 1e-6, n, m, codes=codes, meta=meta, s_w=s_w))
    numel = R * K
    planes = cb + mb
    fused_bytes = numel * (2 + 4 + 2) + numel * 2 + planes
    f_us = fused["sgd_abs_sum"] + fused["mask_pack"]
    p_us = plain["abs_sum"] + plain["mask_pack"]
    # backward: the dW GEMM with and without the blocked-gradient flag
    X = bf16_dev(wl.activations(0))
    dY = bf16_dev(wl.upstream_grad(0))
    Xq, s_x = sbn.sbn_act_quant(X)
    sbn.sbn_mask_ternarize_pack(W, n, m, codes=codes, meta=meta, s_w=s_w)
    dW = torch.empty((R, K), dtype=torch.float32, device="cuda")
    dense = kernels(lambda: sbn.sbn_backward(dY, Xq, s_x, codes, meta, s_w, n, m, want_dX=False, dW=dW))
    blocked = kernels(lambda: sbn.sbn_backward_ex(dY, Xq, s_x, codes, meta, s_w, n, m, sbn.SBN_GRAD_W_MASKED,
                                                  want_dX=False, dW=dW))
    r = lambda x: round(x, 2)
    return {
        "shape": f"R={R} K={K} {n}:{m}",
        "sgd_update_pack": {"sgd_abs_sum_us": r(fused["sgd_abs_sum"]), "mask_pack_us": r(fused["mask_pack"]),
                            "total_us": r(f_us), "algo_bytes": fused_bytes,
                            "GBps": round(fused_bytes / (f_us * 1e-6) / 1e9, 1),
                            "frac_hbm": round(fused_bytes / (f_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                            "plain_pack_us": r(p_us),
                            "note": "W read twice and written once, G (float32) read once; an update followed "
                                    "by a separate pack reads W once more (2 bytes per weight)"},
        "mask_from_ternary": {"abs_sum_us": r(tern["abs_sum"]), "mask_pack_us": r(tern["mask_pack"]),
                              "plain_mask_pack_us": r(plain["mask_pack"])},
        "grad_w_masked": {"gemm_dw_us": r(blocked["gemm_dw"]), "dense_gemm_dw_us": r(dense["gemm_dw"])},
    }


# ---------------------------------------------------------------------- CPU baseline
def _median_runs(fn, runs=3):
    ts = sorted(fn() for _ in range(runs))
    return ts[len(ts) // 2]


def _oracle_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def cpu_baseline(wl, n, m, tokens, runs=3):
    """The oracle as it stands, on the host: pack the full W, quantize `tokens`
    tokens, accumulate them against every row, round the bf16 outputs.  Timed
    with all of the BLAS threads and with one (median of `runs` each).
    TOPS = 2*tokens*R*K / time."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    W = wl.weights(0)
    X = wl.activations(0)[:tokens]

    def once():
        t0 = time.perf_counter()
        eff, mask, sw = O.quant_then_mask(W, n, m)
        O.pack_sbn1(eff, mask, n, m)
        Xq, s_x = O.act_quant(X)
        O.output_bf16(O.accumulate(Xq, eff), sw, s_x)
        return time.perf_counter() - t0

    threads = _oracle_threads()
    dt = _median_runs(once, runs)
    with threadpool_limits(1):
        dt1 = _median_runs(once, runs)
    ops = 2 * tokens * wl.R * wl.K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "runs": runs, "statistic": "median",
            "single_thread": {"value": round(ops / dt1 / 1e12, 6), "cores": 1, "seconds": round(dt1, 3)},
            "nproc": os.cpu_count(),
            "sample": f"full W pack ({wl.R}x{wl.K}, {n}:{m}) + {tokens} of {wl.T} tokens through act_quant, "
                      f"the float64 matmul and the bf16 output rounding; ops = 2*{tokens}*R*K"}


# ---------------------------------------------------------------------- decode step
POOL = 128                     # weights per pool (one table launch per pool)
BATCH = 64                     # weights per by-value batched call (its maximum)
PASSES = 4                     # passes over a pool per replayed graph in decode_gemv's steady modes


def make_decode_step(T=1):
    """Decode step: every weight of two pools of POOL distinct R = K = 4096
    packed weights (2:4 and 6:8; 537 MB and 671 MB, each at least twice the
    Infinity Cache) multiplied by the same T activations, one table GEMV per
    pool (the pool's weights listed once in a device table: one launch each).
    Returns (step, bytes per step, per-launch bytes by kernel name, workload)."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    wl = WORKLOADS["decode"]
    W = bf16_dev(wl.weights(0))
    Xq, s_x = sbn.sbn_act_quant(bf16_dev(wl.activations(0, T=T)))
    tables, total, per_launch = [], 0, {}
    for n, m in wl.nm:
        codes0, meta0, s_w0 = sbn.sbn_mask_ternarize_pack(W, n, m)
        cb, mb = sbn.sbn_packed_bytes(wl.R, wl.K, n, m)
        per = cb + mb + T * wl.K + 4 * T + 2 * T * wl.R + 4
        tables.append(sbn.GemvTable([codes0.clone() for _ in range(POOL)], [meta0.clone() for _ in range(POOL)],
                                    [s_w0.clone() for _ in range(POOL)], wl.R, wl.K, n, m, T=T))
        total += POOL * per
        per_launch[f"gemv_stream_{n}{m}"] = POOL * per
    del W

    def step():
        for tab in tables:
            sbn.sbn_sparse_ternary_gemv_table(Xq, s_x, tab)

    return step, total, per_launch, wl


def make_decode_step_d2(T=1):
    """The decode step on decode planes: the same two pools (2:4 and 6:8 weights,
    POOL each) repacked once, outside the timed region, into the dense 2-bit
    decode plane (4.19 MB per weight for both ratios), one table GEMV per
    pool.  Returns (step, bytes per step, bytes per launch)."""
    import torch
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    wl = WORKLOADS["decode"]
    W = bf16_dev(wl.weights(0))
    Xq, s_x = sbn.sbn_act_quant(bf16_dev(wl.activations(0, T=T)))
    tables, total = [], 0
    per = wl.R * wl.K // 4 + T * wl.K + 4 * T + 2 * T * wl.R + 4
    for n, m in wl.nm:
        codes0, meta0, s_w0 = sbn.sbn_mask_ternarize_pack(W, n, m)
        d20 = sbn.sbn_repack_d2(codes0, meta0, wl.R, wl.K, n, m)
        tables.append(sbn.GemvTable.planes([d20.clone() for _ in range(POOL)], [s_w0.clone() for _ in range(POOL)],
                                           wl.R, wl.K, T=T))
        total += POOL * per
        del codes0, meta0, d20
    del W

    def step():
        for tab in tables:
            sbn.sbn_ternary_gemv_d2_table(Xq, s_x, tab)

    return step, total, POOL * per


def make_decode_pool_24(form, T=1):
    """The 2:4 pool of the decode step alone (POOL weights of R = K = 4096),
    as packed planes (form "packed") or as joint 2:4 codes (form "j6",
    repacked once outside the timed region), one table launch.  Returns
    (step, bytes per step)."""
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    wl = WORKLOADS["decode"]
    W = bf16_dev(wl.weights(0))
    Xq, s_x = sbn.sbn_act_quant(bf16_dev(wl.activations(0, T=T)))
    codes0, meta0, s_w0 = sbn.sbn_mask_ternarize_pack(W, 2, 4)
    del W
    rest = T * wl.K + 4 * T + 2 * T * wl.R + 4
    if form == "packed":
        tab = sbn.GemvTable([codes0.clone() for _ in range(POOL)], [meta0.clone() for _ in range(POOL)],
                            [s_w0.clone() for _ in range(POOL)], wl.R, wl.K, 2, 4, T=T)
        per = sum(sbn.sbn_packed_bytes(wl.R, wl.K, 2, 4)) + rest

        def step():
            sbn.sbn_sparse_ternary_gemv_table(Xq, s_x, tab)
    else:
        nib0, h0 = sbn.sbn_repack_j6(codes0, meta0, wl.R, wl.K)
        tab = sbn.GemvTable.joint([nib0.clone() for _ in range(POOL)], [h0.clone() for _ in range(POOL)],
                                  [s_w0.clone() for _ in range(POOL)], wl.R, wl.K, T=T)
        per = sum(sbn.sbn_j6_bytes(wl.R, wl.K)) + rest

        def step():
            sbn.sbn_ternary_gemv_j6_table(Xq, s_x, tab)
    return step, POOL * per


def measure_decode_j6(a):
    """The 2:4 pool as joint 2:4 codes (1.5 bits per weight) against the same
    pool as packed planes (2 bits per weight), each one table launch per step:
    time per pool, GB/s of each form's own bytes, and the joint code's HBM
    roofline (`gemv_stream_j6`)."""
    import torch
    res = {}
    for form in ("packed", "j6"):
        step, nbytes = make_decode_pool_24(form)
        kname = gemv_kernel_name(step, 2, 4) if form == "packed" else gemv_kernel_name(step, "j", 6)
        ms, _, _, mode = time_steps(step, a.steps, a.warmup, kernel=kname)
        k_ms, k_cnt = kernel_avg_ms(profile_pass(step, a.steps, kname), kname)
        ach = nbytes / (k_ms * 1e-3) / 1e9
        res[form] = {"ms_per_pool": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "launch": mode,
                     "bytes_per_pool": nbytes,
                     "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                                  "traffic": traffic_from_profiles(kname, "decode"), "kernel_us": round(k_ms * 1e3, 3),
                                  "launches": k_cnt, "bytes_per_launch": nbytes}}
        del step
        torch.cuda.empty_cache()
    res["speedup_vs_packed"] = round(res["packed"]["ms_per_pool"] / res["j6"]["ms_per_pool"], 3)
    res["weights_per_s"] = {f: round(POOL * 4096 * 4096 / (res[f]["ms_per_pool"] * 1e-3) / 1e12, 3)
                            for f in ("packed", "j6")}
    res["note"] = ("the 2:4 pool (128 weights of 4096 x 4096, T = 1, bf16 Y) as joint 2:4 codes, repacked once outside "
                   "the timed region, against the same weights as packed planes; weights_per_s in 1e12 weights/s")
    return res


def measure_decode_step(a, with_d2=True):
    """The decode half of the metric as one step: batched decode GEMVs over
    both pools (make_decode_step), timed like every step, with the HBM
    roofline of each streamed kernel (`roofline` 2:4, `roofline_68` 6:8) and,
    when asked, the same step on decode planes (`decode_d2`)."""
    import torch
    step, nbytes, per_launch, wl = make_decode_step(T=1)
    ms, wall, prof, mode = time_steps(step, a.steps, a.warmup)
    out = {"GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 4), "wall_s": round(wall, 4),
           "launch": mode, "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "config": {"workload": "decode", "T": 1, "R": wl.R, "K": wl.K, "nm": "2:4+6:8",
                      "pool_weights_per_ratio": POOL, "weights_per_launch": POOL,
                      "step": "one table decode GEMV per pool (both pools)", "y_dtype": "bf16", "seed": 0}}
    for key, (n, m) in (("roofline", (2, 4)), ("roofline_68", (6, 8))):
        kname = gemv_kernel_name(step, n, m)
        k_ms, k_cnt = kernel_avg_ms(profile_pass(step, a.steps, kname), kname)
        ach = per_launch[f"gemv_stream_{n}{m}"] / (k_ms * 1e-3) / 1e9
        out[key] = {"kernel": kname, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                    "traffic": traffic_from_profiles(kname, "decode"), "kernel_us": round(k_ms * 1e3, 3),
                    "launches": k_cnt, "bytes_per_launch": per_launch[f"gemv_stream_{n}{m}"],
                    "note": "algorithmic bytes: packed planes + activations + scales + bf16 outputs of the "
                            "weights of one launch"}
    out["stages_us"] = {k: round(v[1] / v[0] * 1e3, 3) for k, v in sorted(prof.items()) if v[0]}
    del step
    torch.cuda.empty_cache()
    if with_d2:
        step2, nbytes2, per_launch2 = make_decode_step_d2(T=1)
        ms2, _, _, mode2 = time_steps(step2, a.steps, a.warmup, kernel="gemv_stream_d2")
        k_ms, k_cnt = kernel_avg_ms(profile_pass(step2, a.steps, "gemv_stream_d2"), "gemv_stream_d2")
        ach = per_launch2 / (k_ms * 1e-3) / 1e9
        out["decode_d2"] = {
            "note": "the same step on decode planes (the pools' weights repacked once into dense 2-bit "
                    "ternary codes, 4.19 MB per weight for both ratios, against 4.19 / 5.24 MB packed); "
                    "the step's GB/s stays on the packed weights",
            "ms_per_step": round(ms2, 4), "GBps": round(nbytes2 / (ms2 * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes2 / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "speedup_vs_packed": round(ms / ms2, 3), "launch": mode2,
            "roofline": {"kernel": "gemv_stream_d2", "bound": "hbm", "achieved": round(ach, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": traffic_from_profiles("gemv_stream_d2", "decode"),
                         "kernel_us": round(k_ms * 1e3, 3), "launches": k_cnt, "bytes_per_launch": per_launch2}}
        del step2
        torch.cuda.empty_cache()
        out["decode_j6"] = measure_decode_j6(a)
    return out


def cpu_baseline_decode(wl, weights=POOL, runs=3):
    """The oracle's GEMV (float64 accumulate and bf16 output rounding) for one
    token against `weights` distinct R x K ternary weights per ratio, the
    effective weights prepared outside the timed region; all BLAS threads and
    one thread, median of `runs` each.  GB/s = the decode step's algorithmic
    bytes for those weights / time."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    X = wl.activations(0, T=1)
    Xq, s_x = O.act_quant(X)
    effs, nbytes = [], 0
    for n, m in wl.nm:
        eff, mask, sw = O.quant_then_mask(wl.weights(0), n, m)
        cb, mb = O.packed_bytes(wl.R, wl.K, n, m)
        effs += [(eff, sw)] * weights
        nbytes += weights * (cb + mb + wl.K + 4 + 2 * wl.R + 4)

    def once():
        t0 = time.perf_counter()
        for eff, sw in effs:
            O.output_bf16(O.accumulate(Xq, eff), sw, s_x)
        return time.perf_counter() - t0

    threads = _oracle_threads()
    dt = _median_runs(once, runs)
    with threadpool_limits(1):
        dt1 = _median_runs(once, runs)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "runs": runs, "statistic": "median",
            "single_thread": {"value": round(nbytes / dt1 / 1e9, 3), "cores": 1, "seconds": round(dt1, 3)},
            "nproc": os.cpu_count(),
            "sample": f"{weights} weights per ratio ({', '.join(f'{n}:{m}' for n, m in wl.nm)}) of {wl.R}x{wl.K}, "
                      f"one token, oracle accumulate + bf16 output; bytes = the packed-weight step's algorithmic "
                      f"bytes"}


# ---------------------------------------------------------------------- main
def main():
    a = parse()
    global MIN_WARMUP_MS
    MIN_WARMUP_MS = a.min_warmup_ms
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_linear_layers_02_amd as sbn
    from workloads import WORKLOADS
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sbn.lib()

    if a.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    out = {"metric": METRIC, "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "min_warmup_ms": a.min_warmup_ms}

    if a.workload in ("prefill", "train"):
        wl = WORKLOADS[a.workload]
        n, m = wl.nm[0]
        step = make_forward_step(wl, n, m, with_backward=(a.workload == "train"))
        ms, wall, prof, mode = time_steps(step, a.steps, a.warmup,          # every stage, for stages_us
                                          per_graph=a.steps_per_graph)
        gname = gemm_name_in(prof, "gemm_smfmac" if n <= 2 else "gemm_mfma")
        prof_g = profile_pass(step, a.steps, gname)                          # the roofline kernel alone
        nprod = 3 if a.workload == "train" else 1
        ops = 2 * wl.T * wl.R * wl.K * nprod
        out.update(value=round(ops / (ms * 1e-3) / 1e12, 3), unit="TOPS", ms_per_step=round(ms, 4),
                   wall_s=round(wall, 4), launch=mode, steps_per_graph=a.steps_per_graph if mode == "graph" else 1)
        out["config"] = {"workload": a.workload, "T": wl.T, "R": wl.R, "K": wl.K, "nm": f"{n}:{m}",
                         "step": "pack+act_quant+gemm" + ("+backward" if nprod == 3 else ""),
                         "y_dtype": "bf16", "seed": 0}
        g_ms, g_cnt = kernel_avg_ms(prof_g, gname)
        out["roofline"] = gemm_roofline(gname, wl.T, wl.R, wl.K, n, m, g_ms, g_cnt,
                                        traffic_from_profiles(gname, a.workload))
        out["stages_us"] = {k: round(v[1] / v[0] * 1e3, 3) for k, v in sorted(prof.items()) if v[0]}
        if a.workload == "train":
            for nm_, kname in (("dx", "gemm_dx"), ("dw", "gemm_dw")):
                k_ms, _ = kernel_avg_ms(profile_pass(step, max(2, a.steps // 4), kname), kname)
                fl = 2 * wl.T * wl.R * wl.K                     # the product the method computes
                ex = fl * (2 if kname == "gemm_dw" else 1)      # bf16 products executed (dW: hi and lo halves)
                out["roofline_" + nm_] = {"kernel": kname, "bound": "mfma", "achieved": round(fl / (k_ms * 1e-3) / 1e12, 2),
                                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                          "frac": round(fl / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                          "kernel_us": round(k_ms * 1e3, 3),
                                          "executed_TFLOPs": round(ex / (k_ms * 1e-3) / 1e12, 2),
                                          "executed_frac": round(ex / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                          "note": "achieved = 2*T*R*K (the method's product) per second; "
                                                  "executed counts the bf16 products run (dW runs hi and lo "
                                                  "halves of dY*s_x)"}
    elif a.workload == "decode":
        d = measure_decode_step(a, with_d2=not a.no_extras)
        out.update(value=d.pop("GBps"), unit="GB/s", ms_per_step=d.pop("ms_per_step"), wall_s=d.pop("wall_s"),
                   launch=d.pop("launch"))
        out["config"] = d.pop("config")
        out.update(d)
    elif a.workload == "speedup":
        tab = speedup_tables(a.steps)
        r = next(r for r in tab["prefill"] if r["T"] == 4096)
        out.update(value=r["sbn_24_TOPS"], unit="TOPS", ms_per_step=round(r["sbn_24_us"] * 1e-3, 4))
        out["config"] = {"workload": "speedup", "prefill": {"R": 6912, "K": 2560, "T": list(SPEEDUP_T_PREFILL)},
                         "decode": {"R": 4096, "K": 4096, "T": list(SPEEDUP_T_DECODE)},
                         "step": "one library call per product (sparse 2:4, 6:8; dense ternary 8:8) against "
                                 "torch bf16 matmul and int8 _int_mm"}
        out["speedup"] = tab
        out["roofline"] = None
    else:
        wl = WORKLOADS["sweep"]
        rows = []
        tot_ms = 0.0
        for (n, m) in wl.nm:
            W = bf16_dev(wl.weights(0))
            codes, meta, s_w = sbn.sbn_mask_ternarize_pack(W, n, m)
            Xq, s_x = sbn.sbn_act_quant(bf16_dev(wl.activations(0)))
            Y = torch.empty((wl.T, wl.R), dtype=torch.bfloat16, device="cuda")
            ms, wall, prof, mode = time_steps(
                lambda: sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, wl.R, n, m, Y=Y), a.steps, a.warmup)
            gname = gemm_name_in(prof, "gemm_smfmac" if sbn_uses_smfmac(n, m) else "gemm_mfma")
            g_ms, g_cnt = kernel_avg_ms(prof, gname)
            ops = 2 * wl.T * wl.R * wl.K
            ws_p = torch.empty(max(sbn.sbn_workspace_bytes(sbn.SBN_OP_PACK, 0, wl.R, wl.K, n, m), 256),
                               dtype=torch.uint8, device="cuda")
            pk_ms, _, pk_prof, _ = time_steps(
                lambda: sbn.sbn_mask_ternarize_pack(W, n, m, codes=codes, meta=meta, s_w=s_w, ws=ws_p), a.steps,
                a.warmup)
            pk_bytes = 2 * wl.R * wl.K + sum(sbn.sbn_packed_bytes(wl.R, wl.K, n, m))
            rows.append({"nm": f"{n}:{m}", "call_us": round(ms * 1e3, 2), "kernel_us": round(g_ms * 1e3, 2),
                         "TOPS_call": round(ops / (ms * 1e-3) / 1e12, 1),
                         "TOPS_kernel": round(ops / (g_ms * 1e-3) / 1e12, 1), "kernel": gname,
                         "roofline": gemm_roofline(gname, wl.T, wl.R, wl.K, n, m, g_ms, g_cnt, None),
                         "pack_us": round(pk_ms * 1e3, 2),
                         "pack_kernels_us": {k: round(v[1] / v[0] * 1e3, 2) for k, v in sorted(pk_prof.items())
                                             if v[0]},
                         "pack_GBps": round(pk_bytes / (pk_ms * 1e-3) / 1e9, 1),
                         "pack_frac_hbm": round(pk_bytes / (pk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
            tot_ms += ms
            del W, codes, meta, ws_p
        ops = 2 * wl.T * wl.R * wl.K * len(rows)
        out.update(value=round(ops / (tot_ms * 1e-3) / 1e12, 3), unit="TOPS", ms_per_step=round(tot_ms, 4))
        out["config"] = {"workload": "sweep", "T": wl.T, "R": wl.R, "K": wl.K, "step": "gemm for each N:M"}
        out["sweep"] = rows
        out["roofline"] = dict(next(r for r in rows if r["nm"] == "2:4")["roofline"], row="2:4")

    if not a.no_extras and a.workload not in ("decode", "speedup"):
        # the decode half of the metric beside the prefill / train / sweep line
        d = measure_decode_step(a, with_d2=False)
        out["decode_step"] = {k: d[k] for k in ("GBps", "frac_hbm", "ms_per_step", "launch", "config", "roofline",
                                                "roofline_68")}
        torch.cuda.empty_cache()
        out["decode_gemv"] = [decode_gemv(2, 4, 1), decode_gemv(6, 8, 1)]
        torch.cuda.empty_cache()
        out["decode_j6"] = measure_decode_j6(a)
    if not a.no_extras and a.workload == "train":
        out["variants"] = variants_extras(WORKLOADS["train"])

    if a.no_cpu_baseline or a.workload == "speedup":
        out["cpu_baseline"] = None
    elif a.workload == "decode":
        out["cpu_baseline"] = cpu_baseline_decode(WORKLOADS["decode"], weights=16)
    else:
        wl = WORKLOADS["prefill" if a.workload == "sweep" else a.workload]
        n, m = wl.nm[0]
        out["cpu_baseline"] = cpu_baseline(wl, n, m, tokens=min(wl.T, 4096 if a.workload == "prefill" else 512))
    print(json.dumps(out), flush=True)


def sbn_uses_smfmac(n, m):
    return n <= 2


if __name__ == "__main__":
    main()
