"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, reports sizes, and rejects bad arguments on the host before
any launch (fake, never-dereferenced device addresses are enough for that)."""
from __future__ import annotations

import ctypes

import pytest

import sparse_linear_layers_02_amd as sbn

OK, NULL, SHAPE, NM, ALIGN, WS, DTYPE, HIP, FLAGS, VALUE = range(10)
P = ctypes.c_void_p(0x100000)          # 16-byte aligned fake device address (never touched)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100004)        # misaligned


@pytest.fixture(scope="module")
def L():
    return sbn.lib()


def test_exports_every_header_symbol(L):
    names = sbn.header_symbols()
    assert len(names) == 33
    for nm in names:
        assert hasattr(L, nm), nm


def test_abi_version_and_status_strings(L):
    assert L.sbn_abi_version() == 2
    for s in range(10):
        assert L.sbn_status_string(s) != b"unknown status"
    assert L.sbn_status_string(99) == b"unknown status"


@pytest.mark.parametrize("R,K,n,m", [(256, 256, 2, 4), (4096, 4096, 6, 8), (7, 64, 1, 4), (3, 192, 8, 8),
                                     (11008, 4096, 6, 8)])
def test_packed_bytes(R, K, n, m):
    c, mt = sbn.sbn_packed_bytes(R, K, n, m)
    rnd = lambda x: (x + 15) // 16 * 16
    assert c == rnd(R * K * n // (4 * m))
    assert mt == (0 if n == m else rnd(R * K // 8))


@pytest.mark.parametrize("args,status", [
    ((0, 256, 2, 4), SHAPE), ((16, 100, 2, 4), SHAPE), ((16, 0, 2, 4), SHAPE),
    ((16, 256, 0, 4), NM), ((16, 256, 5, 4), NM), ((16, 256, 2, 6), NM),
    ((16, 1 << 19, 2, 4), SHAPE), ((1 << 20, 1 << 18, 2, 4), SHAPE),
])
def test_packed_bytes_errors(args, status):
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_packed_bytes(*args)
    assert e.value.status == status


def test_workspace_sizes():
    assert sbn.sbn_workspace_bytes(sbn.SBN_OP_ACT_QUANT, 16, 0, 256, 2, 4) == 0
    assert sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMV, 16, 4096, 4096, 2, 4) == 0
    assert sbn.sbn_workspace_bytes(sbn.SBN_OP_PACK, 0, 256, 256, 2, 4) >= 2304
    g24 = sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, 4096, 6912, 2560, 2, 4)
    assert g24 >= 6912 * 2560 // 2 + 6912 * 2560 // 8      # compressed values + indices
    g68 = sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, 8192, 11008, 4096, 6, 8)
    assert g68 >= 11008 * 4096                               # dense int8 operand
    b = sbn.sbn_workspace_bytes(sbn.SBN_OP_BACKWARD, 8192, 11008, 4096, 6, 8)
    assert b >= 2 * 11008 * 4096 + 2 * 4096 * 8192 + 4 * 11008 * 8192


def test_pack_validation(L):
    f = L.sbn_mask_ternarize_pack
    big = 1 << 20
    assert f(None, 16, 256, 256, 2, 4, P, P, P, P, big, None) == NULL
    assert f(P, 16, 256, 256, 2, 4, P, None, P, P, big, None) == NULL        # meta needed for n < m
    assert f(P, 16, 250, 256, 2, 4, P, P, P, P, big, None) == SHAPE
    assert f(P, 16, 256, 128, 2, 4, P, P, P, P, big, None) == SHAPE          # ldw < K
    assert f(P, 16, 256, 260, 2, 4, P, P, P, P, big, None) == ALIGN          # ldw % 8
    assert f(MIS, 16, 256, 256, 2, 4, P, P, P, P, big, None) == ALIGN
    assert f(P, 16, 256, 256, 3, 6, P, P, P, P, big, None) == NM
    assert f(P, 16, 256, 256, 2, 4, P, P, P, P, 16, None) == WS
    assert b"workspace" in L.sbn_last_error()


def test_act_quant_validation(L):
    f = L.sbn_act_quant
    assert f(None, 4, 256, 256, P, P, None) == NULL
    assert f(P, 0, 256, 256, P, P, None) == SHAPE
    assert f(P, 4, 96, 96, P, P, None) == SHAPE
    assert f(P, 4, 256, 255, P, P, None) == SHAPE
    assert f(P, 4, 256, 256, MIS, P, None) == ALIGN


@pytest.mark.parametrize("name", ["sbn_sparse_ternary_gemm", "sbn_sparse_ternary_gemv"])
def test_matmul_validation(L, name):
    f = getattr(L, name)
    big = 1 << 30
    args = dict(Xq=P, s_x=P, T=16, K=256, codes=P, meta=P, s_w=P, R=256, n=2, m=4, Y=P, ydt=1, ldy=256,
                ws=P2, wsb=big)

    def call(**kw):
        a = {**args, **kw}
        return f(a["Xq"], a["s_x"], a["T"], a["K"], a["codes"], a["meta"], a["s_w"], a["R"], a["n"], a["m"],
                 a["Y"], a["ydt"], a["ldy"], a["ws"], a["wsb"], None)

    assert call(Xq=None) == NULL
    assert call(meta=None) == NULL
    assert call(T=0) == SHAPE
    assert call(K=100) == SHAPE
    assert call(ldy=200) == SHAPE
    assert call(ldy=260) == ALIGN
    assert call(Y=MIS) == ALIGN
    assert call(n=9, m=8) == NM
    assert call(ydt=7) == DTYPE
    if name.endswith("gemm"):
        assert call(wsb=8) == WS
        assert call(ws=None) == NULL
    else:
        assert call(T=17) == SHAPE


def test_gemv_batched_validation(L):
    """Host arrays of device pointers; each weight is checked like a single call (error paths only)."""
    f = L.sbn_sparse_ternary_gemv_batched
    arr = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    three = lambda: arr(P, P, P)

    def call(codes=None, meta=None, s_w=None, Y=None, count=3, T=4, K=4096, n=2, m=4, ldy=256, ydt=1):
        return f(P, P, T, K, codes if codes is not None else three(), meta if meta is not None else three(),
                 s_w if s_w is not None else three(), 256, n, m, Y if Y is not None else three(), ydt, ldy, count, None)

    assert f(P, P, 4, 4096, None, three(), three(), 256, 2, 4, three(), 1, 256, 3, None) == NULL
    assert call(count=0) == SHAPE
    assert call(count=65) == SHAPE
    assert call(codes=arr(P, None, P)) == NULL                          # a NULL weight pointer
    assert call(meta=arr(P, P, MIS)) == ALIGN                           # a misaligned plane
    assert call(Y=arr(MIS, P, P)) == ALIGN
    assert call(T=17) == SHAPE
    assert call(K=100) == SHAPE
    assert call(n=5, m=4) == NM
    assert call(ydt=7) == DTYPE
    assert call(meta=arr(P, P, MIS)) == ALIGN and b"weight 2" in L.sbn_last_error()


def test_gemv_table_validation(L):
    """The table calls check what the host can see (the table's entries live in
    device memory); sbn_gemv_table_check checks a host copy of the entries."""
    f = L.sbn_sparse_ternary_gemv_table

    def call(table=P, count=3, T=4, K=4096, R=256, n=2, m=4, ydt=1, ldy=256):
        return f(P, P, T, K, table, count, R, n, m, ydt, ldy, None)

    assert call(table=None) == NULL
    assert f(None, P, 4, 4096, P, 3, 256, 2, 4, 1, 256, None) == NULL
    assert call(table=MIS) == ALIGN
    assert call(count=0) == SHAPE
    assert call(count=1 << 40) == SHAPE                     # count * ceil(R / 16) reaches 2^40
    assert call(T=17) == SHAPE
    assert call(K=2560) == SHAPE                            # not a multiple of 1024
    assert call(K=5120) == SHAPE                            # above 4096
    assert call(n=4, m=8) == NM                             # no streamed decoder for 4:8
    assert call(n=5, m=4) == NM
    assert call(ydt=7) == DTYPE
    assert call(ldy=250) == SHAPE
    g = L.sbn_ternary_gemv_d2_table
    assert g(P, P, 4, 4096, None, 3, 256, 1, 256, None) == NULL
    assert g(P, P, 4, 3000, P, 3, 256, 1, 256, None) == SHAPE
    assert g(P, P, 4, 4096, P, 0, 256, 1, 256, None) == SHAPE
    assert g(P, P, 4, 4096, MIS, 3, 256, 1, 256, None) == ALIGN
    c = L.sbn_gemv_table_check
    tab = lambda *rows: (ctypes.c_void_p * (4 * len(rows)))(*[p for r in rows for p in r])
    good = (P, P2, P, P2)
    assert c(tab(good, good), 2, 4, 4096, 256, 2, 4, 0, 1, 256) == OK
    assert c(tab(good, (None, P2, P, P2)), 2, 4, 4096, 256, 2, 4, 0, 1, 256) == NULL
    assert b"entry 1" in L.sbn_last_error()
    assert c(tab(good, (P, MIS, P, P2)), 2, 4, 4096, 256, 2, 4, 0, 1, 256) == ALIGN
    assert c(tab(good, (P, None, P, P2)), 2, 4, 4096, 256, 2, 4, 0, 1, 256) == NULL     # meta below n == m
    assert c(tab(good, (P, None, P, P2)), 2, 4, 4096, 256, 0, 0, 1, 1, 256) == OK       # planes: meta unused
    assert c(tab(good, (P, P, P, MIS)), 2, 4, 4096, 256, 2, 4, 0, 1, 256) == ALIGN      # Y
    assert c(tab(good), 1, 17, 4096, 256, 2, 4, 0, 1, 256) == SHAPE
    assert c(None, 1, 4, 4096, 256, 2, 4, 0, 1, 256) == NULL


def test_joint_code_validation(L):
    nb, hb = sbn.sbn_j6_bytes(4096, 4096)
    assert (nb, hb) == (4096 * 4096 // 8, 4096 * 4096 // 16)
    assert sbn.sbn_j6_bytes(3, 64) == (32, 16)                         # 24 and 12 rounded up to 16
    with pytest.raises(sbn.SbnError):
        sbn.sbn_j6_bytes(4, 100)
    f = L.sbn_repack_j6
    assert f(P, None, 16, 256, P2, P2, None) == NULL                   # meta is required (2:4 planes)
    assert f(P, P, 16, 250, P2, P2, None) == SHAPE
    assert f(P, P, 16, 256, P2, MIS, None) == ALIGN
    g = L.sbn_ternary_gemv_j6
    assert g(P, P, 17, 4096, P, P, P, 64, P, 1, 64, None) == SHAPE     # T > 16
    assert g(P, P, 4, 2560, P, P, P, 64, P, 1, 64, None) == SHAPE      # K not a multiple of 1024
    assert g(P, P, 4, 4096, P, None, P, 64, P, 1, 64, None) == NULL    # h plane
    assert g(P, P, 4, 4096, P, MIS, P, 64, P, 1, 64, None) == ALIGN
    assert g(P, P, 4, 4096, P, P, P, 64, P, 7, 64, None) == DTYPE
    t = L.sbn_ternary_gemv_j6_table
    assert t(P, P, 4, 4096, None, 3, 256, 1, 256, None) == NULL
    assert t(P, P, 4, 5120, P, 3, 256, 1, 256, None) == SHAPE
    assert t(P, P, 4, 4096, P, 0, 256, 1, 256, None) == SHAPE
    c = L.sbn_gemv_table_check
    tab = lambda *rows: (ctypes.c_void_p * (4 * len(rows)))(*[p for r in rows for p in r])
    good = (P, P2, P, P2)
    assert c(tab(good), 1, 4, 4096, 256, 2, 4, sbn.SBN_FORM_J6, 1, 256) == OK
    assert c(tab(good, (P, None, P, P2)), 2, 4, 4096, 256, 2, 4, sbn.SBN_FORM_J6, 1, 256) == NULL   # no h plane
    assert c(tab(good, (P, MIS, P, P2)), 2, 4, 4096, 256, 2, 4, sbn.SBN_FORM_J6, 1, 256) == ALIGN
    assert c(tab(good), 1, 4, 4096, 256, 2, 4, 7, 1, 256) == VALUE                                  # unknown form


def test_gemv_table_binding_checks_before_the_copy():
    """GemvTable checks every entry on the host and refuses mismatched outputs;
    the calls refuse activations whose shape is not the table's (CPU tensors:
    nothing is launched)."""
    import torch
    codes = [torch.zeros(4096 * 256 // 4, dtype=torch.uint8) for _ in range(2)]
    metas = [torch.zeros(4096 * 256 // 8, dtype=torch.uint8) for _ in range(2)]
    s_ws = [torch.ones(1, dtype=torch.float32) for _ in range(2)]
    tab = sbn.GemvTable(codes, metas, s_ws, 256, 4096, 2, 4, T=2)
    assert tab.count == 2 and tab.dev.shape == (8,) and tab.ldy == 256 and len(tab.Ys) == 2
    assert int(tab.dev[0]) == codes[0].data_ptr() and int(tab.dev[7]) == tab.Ys[1].data_ptr()
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_sparse_ternary_gemv_table(torch.zeros((3, 4096), dtype=torch.int8), torch.ones(3), tab)
    assert e.value.status == 2
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_ternary_gemv_d2_table(torch.zeros((2, 4096), dtype=torch.int8), torch.ones(2), tab)
    assert e.value.status == 2
    with pytest.raises(sbn.SbnError) as e:            # one Y with another row stride
        sbn.GemvTable(codes, metas, s_ws, 256, 4096, 2, 4, T=2,
                      Ys=[torch.empty((2, 256), dtype=torch.bfloat16), torch.empty((2, 264), dtype=torch.bfloat16)[:, :256]])
    assert e.value.status == 2
    with pytest.raises(sbn.SbnError) as e:            # 6:8 without its meta planes
        sbn.GemvTable(codes, None, s_ws, 256, 4096, 6, 8, T=2)
    assert e.value.status == 1
    with pytest.raises(sbn.SbnError) as e:
        sbn.GemvTable([], [], [], 256, 4096, 2, 4)
    assert e.value.status == 2


def test_backward_validation(L):
    f = L.sbn_backward
    big = 1 << 34

    def call(dY=P, T=64, R=256, Xq=P, s_x=P, K=256, codes=P, meta=P, s_w=P, n=2, m=4, dX=P, dxdt=0, dW=P, ws=P2,
             wsb=big):
        return f(dY, T, R, Xq, s_x, K, codes, meta, s_w, n, m, dX, dxdt, dW, ws, wsb, None)

    assert call(dY=None) == NULL
    assert call(ws=None) == NULL
    assert call(R=100) == SHAPE          # R % 8
    assert call(K=32) == SHAPE
    assert call(dxdt=2) == DTYPE
    assert call(dX=MIS) == ALIGN
    assert call(wsb=64) == WS


def test_profile_calls_without_launches(L):
    assert L.sbn_profile_enable(1, None) == OK
    assert L.sbn_profile_enable(1, b"gemm_smfmac") == OK
    assert L.sbn_profile_reset() == OK
    buf = ctypes.create_string_buffer(256)
    assert L.sbn_profile_dump(buf, 256) == OK and buf.value == b""
    assert L.sbn_profile_dump(None, 0) == NULL
    assert L.sbn_profile_enable(0, None) == OK


def test_pack_ex_and_sgd_validation(L):
    big = 1 << 20
    f = L.sbn_mask_ternarize_pack_ex
    assert f(P, 16, 256, 256, 2, 4, 4, P, P, P, P, big, None) == FLAGS          # unknown flag bit
    assert f(P, 16, 256, 256, 2, 4, 2, P, P, P, P, big, None) == FLAGS          # a backward flag
    assert f(None, 16, 256, 256, 2, 4, 1, P, P, P, P, big, None) == NULL
    g = L.sbn_sgd_update_pack
    nan = float("nan")
    assert g(P, 16, 256, 256, None, 256, 0.1, 2, 4, 0, P, P, P, P, big, None) == NULL     # no gradient
    assert g(P, 16, 256, 256, MIS, 256, 0.1, 2, 4, 0, P, P, P, P, big, None) == ALIGN
    assert g(P, 16, 256, 256, P2, 128, 0.1, 2, 4, 0, P, P, P, P, big, None) == SHAPE      # ldg < K
    assert g(P, 16, 256, 256, P2, 260, 0.1, 2, 4, 0, P, P, P, P, big, None) == ALIGN      # ldg % 8
    assert g(P, 16, 256, 256, P2, 256, nan, 2, 4, 0, P, P, P, P, big, None) == VALUE
    assert g(P, 16, 256, 256, P2, 256, float("inf"), 2, 4, 0, P, P, P, P, big, None) == VALUE
    assert g(P, 16, 256, 256, P2, 256, 0.1, 2, 4, 8, P, P, P, P, big, None) == FLAGS
    assert g(P, 16, 256, 256, P2, 256, 0.1, 2, 4, 0, P, P, P, P, 16, None) == WS
    assert b"workspace" in L.sbn_last_error()


def test_backward_ex_validation(L):
    f = L.sbn_backward_ex
    big = 1 << 30
    assert f(P, 16, 256, P, P, 256, P, P, P, 2, 4, P, 0, P, 1, P, big, None) == FLAGS      # a pack flag
    assert f(P, 16, 256, P, P, 256, P, None, P, 2, 4, P, 0, P, 2, P, big, None) == NULL    # meta needed
    assert f(P, 16, 250, P, P, 256, P, P, P, 2, 4, P, 0, P, 2, P, big, None) == SHAPE      # R % 8


def test_forward_validation(L):
    f = L.sbn_forward
    big = 1 << 30
    # W, R, K, ldw, X, T, ldx, n, m, flags, codes, meta, s_w, Xq, s_x, Y, ydt, ldy, ws, ws_bytes, stream
    assert f(None, 64, 256, 256, P, 16, 256, 2, 4, 0, P, P, P, P, P, P, 1, 64, P, big, None) == NULL
    assert f(P, 64, 256, 256, None, 16, 256, 2, 4, 0, P, P, P, P, P, P, 1, 64, P, big, None) == NULL
    assert f(P, 64, 256, 256, P, 16, 256, 2, 4, 0, P, None, P, P, P, P, 1, 64, P, big, None) == NULL
    assert f(P, 64, 256, 128, P, 16, 256, 2, 4, 0, P, P, P, P, P, P, 1, 64, P, big, None) == SHAPE   # ldw
    assert f(P, 64, 256, 256, P, 16, 260, 2, 4, 0, P, P, P, P, P, P, 1, 64, P, big, None) == ALIGN   # ldx
    assert f(P, 64, 256, 256, P, 16, 256, 2, 4, 2, P, P, P, P, P, P, 1, 64, P, big, None) == FLAGS
    assert f(P, 64, 256, 256, P, 16, 256, 2, 4, 0, P, P, P, P, P, P, 9, 64, P, big, None) == DTYPE
    assert f(P, 64, 256, 256, P, 16, 256, 2, 4, 0, P, P, P, P, P, P, 1, 64, P, 64, None) == WS
    need = sbn.sbn_workspace_bytes(sbn.SBN_OP_FORWARD, 16, 64, 256, 2, 4)
    assert need >= sbn.sbn_workspace_bytes(sbn.SBN_OP_PACK, 0, 64, 256, 2, 4) + \
        sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, 16, 64, 256, 2, 4)


def test_decode_plane_validation(L):
    big = 1 << 20
    assert sbn.sbn_decode_plane_bytes(4096, 4096) == 4096 * 4096 // 4
    assert sbn.sbn_decode_plane_bytes(7, 64) == 112
    f = L.sbn_repack_d2
    assert f(P, None, 16, 256, 6, 8, P2, None) == NULL            # meta needed below n == m
    assert f(P, None, 16, 250, 8, 8, P2, None) == SHAPE
    assert f(P, P, 16, 256, 3, 6, P2, None) == NM
    assert f(P, P, 16, 256, 6, 8, MIS, None) == ALIGN
    g = L.sbn_ternary_gemv_d2
    assert g(P, P, 17, 256, P, P, 64, P, 1, 64, None) == SHAPE     # T > 16
    assert g(P, P, 4, 256, None, P, 64, P, 1, 64, None) == NULL
    assert g(P, P, 4, 256, P, P, 64, P, 1, 60, None) == SHAPE      # ldy < R
    assert g(P, P, 4, 256, P, P, 64, P, 7, 64, None) == DTYPE


def test_prepared_weight_validation(L):
    assert sbn.sbn_gemm_weight_bytes(6912, 2560, 2, 4) >= 6912 * 2560 // 2
    assert sbn.sbn_gemm_weight_bytes(4096, 4096, 6, 8) >= 4096 * 4096
    # the GEMM on a prepared weight reads the activations in place: no workspace
    for n, m in ((2, 4), (1, 8), (6, 8), (8, 8)):
        assert sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM_PREPARED, 300, 0, 576, n, m) == 0
    # the GEMM from packed planes holds the expanded weight and the tiled activations
    assert sbn.sbn_workspace_bytes(sbn.SBN_OP_GEMM, 4096, 6912, 2560, 2, 4) == \
        sbn.sbn_gemm_weight_bytes(6912, 2560, 2, 4) + 4096 * 2560
    f = L.sbn_prepare_gemm_weight
    assert f(P, None, 16, 256, 2, 4, P2, None) == NULL
    assert f(P, P, 16, 250, 2, 4, P2, None) == SHAPE
    g = L.sbn_sparse_ternary_gemm_prepared
    assert g(P, P, 16, 256, None, P, 64, 2, 4, P2, 1, 64, P, 1 << 20, None) == NULL
    assert g(P, P, 16, 256, P, P, 64, 2, 4, P2, 1, 60, P, 1 << 20, None) == SHAPE


INJECT_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import sparse_linear_layers_02_amd as sbn
L = sbn.lib()
P, P2 = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
big = 1 << 30
calls = {
    "sbn_act_quant": lambda: L.sbn_act_quant(P, 16, 256, 256, P2, P2, None),
    "sbn_mask_ternarize_pack": lambda: L.sbn_mask_ternarize_pack(P, 16, 256, 256, 2, 4, P2, P2, P2, P2, big, None),
    "sbn_sparse_ternary_gemm": lambda: L.sbn_sparse_ternary_gemm(P, P, 16, 256, P, P, P, 64, 2, 4, P2, 1, 64, P2,
                                                                 big, None),
    "sbn_sparse_ternary_gemv": lambda: L.sbn_sparse_ternary_gemv(P, P, 4, 256, P, P, P, 64, 6, 8, P2, 1, 64, P2,
                                                                 big, None),
    "sbn_prepare_gemm_weight": lambda: L.sbn_prepare_gemm_weight(P, P, 64, 256, 2, 4, P2, None),
    "sbn_backward": lambda: L.sbn_backward(P, 16, 64, P, P, 256, P, P, P, 2, 4, P2, 1, P2, P2, big, None),
    "sbn_repack_d2": lambda: L.sbn_repack_d2(P, P, 64, 256, 2, 4, P2, None),
}
for name, call in calls.items():
    st = call()
    print(name, st, L.sbn_last_error().decode())
# validation still runs first
print("null", L.sbn_act_quant(None, 16, 256, 256, P2, P2, None))
"""


def test_injected_launch_failure_reports_hip_error(tmp_path):
    """SBN_TEST_INJECT_LAUNCH_FAILURE=1: every launch is replaced by a failure
    (nothing is launched), and each entry point returns SBN_ERR_HIP naming
    itself; a validation error still wins.  Runs in a child process (the
    variable is read once per process)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SBN_TEST_INJECT_LAUNCH_FAILURE="1", HIP_VISIBLE_DEVICES="")
    out = subprocess.run([sys.executable, "-c", INJECT_SCRIPT, root], env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 8, out.stdout
    for line in lines[:-1]:
        name, st, msg = line.split(" ", 2)
        assert int(st) == HIP, line
        assert msg.startswith(name + ":") and "injected" in msg, line
    assert lines[-1] == f"null {NULL}"


def test_huge_shapes_rejected_before_any_product(L):
    """Counts near the int64 range are rejected on the host: every product of
    two sizes is bounded by a division first (no signed overflow)."""
    huge = 1 << 50
    big = 1 << 62
    i64 = ctypes.c_int64
    sz = ctypes.c_size_t()
    assert L.sbn_packed_bytes(i64(huge), 256, 2, 4, ctypes.byref(sz), ctypes.byref(sz)) == SHAPE
    assert L.sbn_packed_bytes(i64(1 << 30), 1 << 18, 2, 4, ctypes.byref(sz), ctypes.byref(sz)) == SHAPE
    for op in (sbn.SBN_OP_PACK, sbn.SBN_OP_GEMM, sbn.SBN_OP_FORWARD, sbn.SBN_OP_BACKWARD):
        assert L.sbn_workspace_bytes(op, i64(16), i64(huge), 256, 2, 4, ctypes.byref(sz)) == SHAPE
    for op in (sbn.SBN_OP_GEMM, sbn.SBN_OP_GEMM_PREPARED, sbn.SBN_OP_FORWARD, sbn.SBN_OP_BACKWARD):
        assert L.sbn_workspace_bytes(op, i64(huge), i64(256), 256, 2, 4, ctypes.byref(sz)) == SHAPE
        assert L.sbn_workspace_bytes(op, i64(1 << 31), i64(256), 1 << 10, 2, 4, ctypes.byref(sz)) == SHAPE
    assert L.sbn_workspace_bytes(sbn.SBN_OP_BACKWARD, i64(1 << 30), i64(1 << 12), 64, 2, 4,
                                 ctypes.byref(sz)) == SHAPE                       # dY = T*R too large
    gemm = L.sbn_sparse_ternary_gemm
    call = lambda T, R, ldy: gemm(P, P, i64(T), 256, P, P, P, i64(R), 2, 4, P, 1, i64(ldy), P2, ctypes.c_size_t(big),
                                  None)
    assert call(16, huge, huge) == SHAPE
    assert call(huge, 256, 256) == SHAPE
    assert call(1 << 30, 256, 1 << 20) == SHAPE                                   # T*ldy reaches 2^40
    assert call(16, 256, 1 << 62) == SHAPE
    pack = L.sbn_mask_ternarize_pack
    assert pack(P, i64(huge), 256, 256, 2, 4, P, P, P, P, ctypes.c_size_t(big), None) == SHAPE
    assert pack(P, i64(1 << 24), 256, i64(1 << 20), 2, 4, P, P, P, P, ctypes.c_size_t(big), None) == SHAPE
    aq = L.sbn_act_quant
    assert aq(P, i64(huge), 256, 256, P, P, None) == SHAPE
    assert aq(P, i64(1 << 30), 256, i64(1 << 12), P, P, None) == SHAPE
    bwd = L.sbn_backward
    assert bwd(P, i64(huge), 256, P, P, 256, P, P, P, 2, 4, P, 0, P, P2, ctypes.c_size_t(big), None) == SHAPE
    assert bwd(P, 64, i64(huge), P, P, 256, P, P, P, 2, 4, P, 0, P, P2, ctypes.c_size_t(big), None) == SHAPE
    assert b"2^40" in L.sbn_last_error() or b"2^37" in L.sbn_last_error()


def test_binding_rejects_layouts_the_abi_cannot_see():
    """The binding checks what the C ABI has no argument for (element types,
    unit column strides, contiguity where no leading dimension is passed)
    before calling it: these fail on the host, with no device involved."""
    import torch
    X32 = torch.zeros((4, 256), dtype=torch.float32)
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_act_quant(X32)
    assert e.value.status == DTYPE
    Xq = torch.zeros((256, 4), dtype=torch.int8).t()               # non-contiguous, no ldx in the ABI
    s_x = torch.zeros(4, dtype=torch.float32)
    codes = torch.zeros(64, dtype=torch.uint8)
    s_w = torch.zeros(1, dtype=torch.float32)
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, codes, s_w, 16, 2, 4)
    assert e.value.status == SHAPE
    Xq = torch.zeros((4, 256), dtype=torch.int8)
    Ybad = torch.zeros((4, 16), dtype=torch.float32)               # bf16 requested
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_sparse_ternary_gemm(Xq, s_x, codes, codes, s_w, 16, 2, 4, ydt=sbn.SBN_BF16, Y=Ybad)
    assert e.value.status == DTYPE
    Wt = torch.zeros((256, 16), dtype=torch.bfloat16).t()          # column stride 16
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_mask_ternarize_pack(Wt, 2, 4)
    assert e.value.status == SHAPE
    dY = torch.zeros((4, 16), dtype=torch.float32)
    with pytest.raises(sbn.SbnError) as e:
        sbn.sbn_backward(dY, Xq, s_x, codes, codes, s_w, 2, 4)
    assert e.value.status == DTYPE


def test_noalloc_pack_validation(L):
    """The allocation-free pack validates like the pack and refuses weights
    beyond its fixed scratch (R*K above 2^28) before any launch."""
    f = L.sbn_mask_ternarize_pack_noalloc
    i64 = ctypes.c_int64
    assert f(None, 16, 256, 256, 2, 4, P, P, P, None) == NULL
    assert f(P, 16, 256, 256, 2, 4, P, None, P, None) == NULL
    assert f(P, 16, 250, 256, 2, 4, P, P, P, None) == SHAPE
    assert f(P, 16, 256, 260, 2, 4, P, P, P, None) == ALIGN
    assert f(P, 16, 256, 256, 3, 6, P, P, P, None) == NM
    assert f(P, i64(1 << 19), 1 << 10, 1 << 10, 2, 4, P, P, P, None) == WS       # R*K = 2^29
    assert b"2^28" in L.sbn_last_error()
    assert f(P, i64(1 << 50), 256, 256, 2, 4, P, P, P, None) == SHAPE
