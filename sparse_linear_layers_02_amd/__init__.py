"""Python binding of libsbn, the Sparse-BitLinear hot path for MI355X (gfx950).

Argument marshalling only: every function here checks nothing numerical
(only the tensor layouts the C ABI cannot see: dtypes, unit column strides,
contiguity where the ABI takes no leading dimension), allocates outputs
with PyTorch when the caller did not pass them, and calls
the C entry point of the same name in ``libsbn.so`` (declared in
``include/sbn.h``) with raw device pointers on the current HIP stream.  All
computation happens in the HIP kernels.  If the library is not built, import
of the binding still works but the first call raises ``SbnError``: there is no
fallback implementation.

Tensor conventions: bf16 tensors are ``torch.bfloat16`` (passed as bit
patterns), int8 ``torch.int8``, packed planes ``torch.uint8``, scales
``torch.float32``; all on the same CUDA (HIP) device, row-major.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsbn.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "sbn.h")

SBN_F32, SBN_BF16, SBN_I32_ACC = 0, 1, 2
SBN_FORM_PACKED, SBN_FORM_D2, SBN_FORM_J6 = 0, 1, 2     # the weight forms a GEMV table can hold
SBN_OP_PACK, SBN_OP_ACT_QUANT, SBN_OP_GEMM, SBN_OP_GEMV, SBN_OP_BACKWARD, SBN_OP_FORWARD = 0, 1, 2, 3, 4, 5
SBN_OP_GEMM_PREPARED = 6
SBN_FLAGS_NONE, SBN_MASK_FROM_TERNARY, SBN_GRAD_W_MASKED = 0, 1, 2
STATUS = {0: "SBN_OK", 1: "SBN_ERR_NULL", 2: "SBN_ERR_SHAPE", 3: "SBN_ERR_UNSUPPORTED_NM",
          4: "SBN_ERR_ALIGN", 5: "SBN_ERR_WORKSPACE", 6: "SBN_ERR_DTYPE", 7: "SBN_ERR_HIP",
          8: "SBN_ERR_FLAGS", 9: "SBN_ERR_VALUE"}
SBN_ERR_VALUE = 9


class SbnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()

_i64, _int, _sz, _vp, _u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32
_SIGNATURES = {
    "sbn_abi_version": ([], _int),
    "sbn_status_string": ([_int], ctypes.c_char_p),
    "sbn_last_error": ([], ctypes.c_char_p),
    "sbn_packed_bytes": ([_i64, _i64, _int, _int, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], _int),
    "sbn_workspace_bytes": ([_int, _i64, _i64, _i64, _int, _int, ctypes.POINTER(_sz)], _int),
    "sbn_mask_ternarize_pack": ([_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "sbn_mask_ternarize_pack_ex": ([_vp, _i64, _i64, _i64, _int, _int, _u32, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "sbn_sgd_update_pack": ([_vp, _i64, _i64, _i64, _vp, _i64, ctypes.c_float, _int, _int, _u32, _vp, _vp, _vp,
                             _vp, _sz, _vp], _int),
    "sbn_mask_ternarize_pack_noalloc": ([_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp], _int),
    "sbn_act_quant": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "sbn_sparse_ternary_gemm": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _int, _int, _vp, _int, _i64,
                                 _vp, _sz, _vp], _int),
    "sbn_sparse_ternary_gemv": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _int, _int, _vp, _int, _i64,
                                 _vp, _sz, _vp], _int),
    "sbn_gemm_weight_bytes": ([_i64, _i64, _int, _int, ctypes.POINTER(_sz)], _int),
    "sbn_prepare_gemm_weight": ([_vp, _vp, _i64, _i64, _int, _int, _vp, _vp], _int),
    "sbn_sparse_ternary_gemm_prepared": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _int, _int, _vp, _int, _i64, _vp, _sz,
                                          _vp], _int),
    "sbn_decode_plane_bytes": ([_i64, _i64, ctypes.POINTER(_sz)], _int),
    "sbn_repack_d2": ([_vp, _vp, _i64, _i64, _int, _int, _vp, _vp], _int),
    "sbn_ternary_gemv_d2": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _int, _i64, _vp], _int),
    "sbn_ternary_gemv_d2_batched": ([_vp, _vp, _i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64,
                                     ctypes.POINTER(_vp), _int, _i64, _i64, _vp], _int),
    "sbn_forward": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _int, _int, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _int,
                     _i64, _vp, _sz, _vp], _int),
    "sbn_sparse_ternary_gemv_batched": ([_vp, _vp, _i64, _i64, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                         ctypes.POINTER(_vp), _i64, _int, _int, ctypes.POINTER(_vp), _int,
                                         _i64, _i64, _vp], _int),
    "sbn_sparse_ternary_gemv_table": ([_vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _int, _int, _i64, _vp], _int),
    "sbn_ternary_gemv_d2_table": ([_vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _i64, _vp], _int),
    "sbn_gemv_table_check": ([_vp, _i64, _i64, _i64, _i64, _int, _int, _int, _int, _i64], _int),
    "sbn_j6_bytes": ([_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], _int),
    "sbn_repack_j6": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp], _int),
    "sbn_ternary_gemv_j6": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _int, _i64, _vp], _int),
    "sbn_ternary_gemv_j6_table": ([_vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _i64, _vp], _int),
    "sbn_backward": ([_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _int, _int, _vp, _int, _vp, _vp,
                      _sz, _vp], _int),
    "sbn_backward_ex": ([_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _int, _int, _vp, _int, _vp, _u32, _vp,
                         _sz, _vp], _int),
    "sbn_profile_enable": ([_int, ctypes.c_char_p], _int),
    "sbn_profile_reset": ([], _int),
    "sbn_profile_dump": ([ctypes.c_char_p, _sz], _int),
}


def header_symbols() -> list[str]:
    """Names of the functions declared in include/sbn.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:sbn_status|int|const char\*)\s+(sbn_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """The loaded libsbn.so (loaded once, signatures set)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise SbnError("load", 7, f"{LIB_PATH} is not built; run __graft_entry__.build()")
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGNATURES.items():
                f = getattr(L, name)
                f.argtypes, f.restype = args, res
            _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SbnError(fn, status, lib().sbn_last_error().decode())


# ------------------------------------------------------------------ host-only queries
def sbn_abi_version() -> int:
    return lib().sbn_abi_version()


def sbn_packed_bytes(R: int, K: int, n: int, m: int) -> tuple[int, int]:
    c, mt = _sz(), _sz()
    _check("sbn_packed_bytes", lib().sbn_packed_bytes(R, K, n, m, ctypes.byref(c), ctypes.byref(mt)))
    return c.value, mt.value


def sbn_workspace_bytes(op: int, T: int, R: int, K: int, n: int, m: int) -> int:
    b = _sz()
    _check("sbn_workspace_bytes", lib().sbn_workspace_bytes(op, T, R, K, n, m, ctypes.byref(b)))
    return b.value


# ------------------------------------------------------------------ device calls
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# Grow-only workspaces, one per (operation, device, stream): calls that share a
# workspace must be ordered on one stream (the ABI's rule), and a buffer is
# allocated while its stream is current, so the caching allocator hands its
# memory to later work on that stream only once this work is done.
_WS = {}


def _workspace(kind: str, nbytes: int, device, stream):
    torch = _torch()
    if nbytes == 0:
        return None
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (kind, str(device), s.cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


# Layout the C ABI assumes but cannot see: element types, unit column strides
# (row-major with a leading dimension), and fully contiguous tensors where the
# ABI takes no leading dimension.
_DT = {"bf16": "bfloat16", "i8": "int8", "u8": "uint8", "f32": "float32", "i32": "int32"}


def _req(t, name: str, dt: str, contiguous: bool = False, fn: str = "sbn") -> None:
    if t is None:
        return
    torch = _torch()
    if t.dtype != getattr(torch, _DT[dt]):
        raise SbnError(fn, 6, f"{name} must be {_DT[dt]}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise SbnError(fn, 2, f"{name} must be contiguous")
    if t.dim() == 2 and t.shape[1] > 1 and t.stride(1) != 1:
        raise SbnError(fn, 2, f"{name} must have unit column stride (row-major)")


def _pack_outputs(W, n: int, m: int, codes, meta, s_w, ws, stream=None, want_ws=True):
    torch = _torch()
    R, K = W.shape
    _req(W, "W", "bf16")
    for t, nm in ((codes, "codes"), (meta, "meta")):
        _req(t, nm, "u8", True)
    _req(s_w, "s_w", "f32", True)
    cb, mb = sbn_packed_bytes(R, K, n, m)
    dev = W.device
    if codes is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    if meta is None and mb:
        meta = torch.empty(mb, dtype=torch.uint8, device=dev)
    if s_w is None:
        s_w = torch.empty(1, dtype=torch.float32, device=dev)
    if want_ws and ws is None:
        ws = _workspace("pack", sbn_workspace_bytes(SBN_OP_PACK, 0, R, K, n, m), dev, stream)
    return codes, meta, s_w, ws


def sbn_mask_ternarize_pack(W, n: int, m: int, *, codes=None, meta=None, s_w=None, ws=None, stream=None):
    """Mask, ternarize and pack bf16 master weights W [R, K].  Returns (codes, meta, s_w)."""
    R, K = W.shape
    codes, meta, s_w, ws = _pack_outputs(W, n, m, codes, meta, s_w, ws, stream)
    _check("sbn_mask_ternarize_pack",
           lib().sbn_mask_ternarize_pack(_ptr(W), R, K, W.stride(0), n, m, _ptr(codes), _ptr(meta),
                                         _ptr(s_w), _ptr(ws), ws.numel() if ws is not None else 0,
                                         _stream(stream)))
    return codes, meta, s_w


def sbn_mask_ternarize_pack_ex(W, n: int, m: int, flags: int, *, codes=None, meta=None, s_w=None, ws=None,
                               stream=None):
    """sbn_mask_ternarize_pack with variant flags (SBN_MASK_FROM_TERNARY).  Returns (codes, meta, s_w)."""
    R, K = W.shape
    codes, meta, s_w, ws = _pack_outputs(W, n, m, codes, meta, s_w, ws, stream)
    _check("sbn_mask_ternarize_pack_ex",
           lib().sbn_mask_ternarize_pack_ex(_ptr(W), R, K, W.stride(0), n, m, flags, _ptr(codes), _ptr(meta),
                                            _ptr(s_w), _ptr(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)))
    return codes, meta, s_w


def sbn_mask_ternarize_pack_noalloc(W, n: int, m: int, *, codes=None, meta=None, s_w=None, stream=None):
    """sbn_mask_ternarize_pack on the library's fixed scratch (no workspace; R*K <= 2^28).
    Returns (codes, meta, s_w)."""
    R, K = W.shape
    codes, meta, s_w, _ = _pack_outputs(W, n, m, codes, meta, s_w, None, stream, want_ws=False)
    _check("sbn_mask_ternarize_pack_noalloc",
           lib().sbn_mask_ternarize_pack_noalloc(_ptr(W), R, K, W.stride(0), n, m, _ptr(codes), _ptr(meta),
                                                 _ptr(s_w), _stream(stream)))
    return codes, meta, s_w


def sbn_sgd_update_pack(W, G, lr: float, n: int, m: int, flags: int = 0, *, codes=None, meta=None, s_w=None,
                        ws=None, stream=None):
    """One SGD step W <- bf16(fma(-lr, G, W)) on bf16 W [R, K] (in place) with
    float32 G [R, K], then mask/ternarize/pack of the new W.  Returns (codes, meta, s_w)."""
    R, K = W.shape
    _req(G, "G", "f32")
    codes, meta, s_w, ws = _pack_outputs(W, n, m, codes, meta, s_w, ws, stream)
    _check("sbn_sgd_update_pack",
           lib().sbn_sgd_update_pack(_ptr(W), R, K, W.stride(0), _ptr(G), G.stride(0), float(lr), n, m, flags,
                                     _ptr(codes), _ptr(meta), _ptr(s_w), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream)))
    return codes, meta, s_w


def sbn_act_quant(X, *, Xq=None, s_x=None, stream=None):
    """Per-token absmax int8 quantization of bf16 X [T, K].  Returns (Xq, s_x)."""
    torch = _torch()
    T, K = X.shape
    _req(X, "X", "bf16")
    _req(Xq, "Xq", "i8", True)
    _req(s_x, "s_x", "f32", True)
    if Xq is None:
        Xq = torch.empty((T, K), dtype=torch.int8, device=X.device)
    if s_x is None:
        s_x = torch.empty(T, dtype=torch.float32, device=X.device)
    _check("sbn_act_quant",
           lib().sbn_act_quant(_ptr(X), T, K, X.stride(0), _ptr(Xq), _ptr(s_x), _stream(stream)))
    return Xq, s_x


_YT = {SBN_F32: "float32", SBN_BF16: "bfloat16", SBN_I32_ACC: "int32"}
_YD = {SBN_F32: "f32", SBN_BF16: "bf16", SBN_I32_ACC: "i32"}


def _req_matmul(fn, Xq, s_x, s_w, ydt, Y):
    _req(Xq, "Xq", "i8", True, fn)
    _req(s_x, "s_x", "f32", True, fn)
    _req(s_w, "s_w", "f32", True, fn)
    if ydt in _YD:
        _req(Y, "Y", _YD[ydt], False, fn)


def _matmul(name: str, Xq, s_x, codes, meta, s_w, R: int, n: int, m: int, ydt: int, Y, ws, stream):
    torch = _torch()
    T, K = Xq.shape
    _req_matmul(name, Xq, s_x, s_w, ydt, Y)
    _req(codes, "codes", "u8", True, name)
    _req(meta, "meta", "u8", True, name)
    if Y is None:                                    # row stride rounded up to 8 elements (the ABI's rule)
        Y = torch.empty((T, (R + 7) // 8 * 8), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R]
    op = SBN_OP_GEMM if name == "sbn_sparse_ternary_gemm" else SBN_OP_GEMV
    need = sbn_workspace_bytes(op, T, R, K, n, m)
    if ws is None:
        ws = _workspace("gemm", need, Xq.device, stream)
    fn = getattr(lib(), name)
    _check(name, fn(_ptr(Xq), _ptr(s_x), T, K, _ptr(codes), _ptr(meta), _ptr(s_w), R, n, m, _ptr(Y), ydt,
                    Y.stride(0), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return Y


def sbn_sparse_ternary_gemm(Xq, s_x, codes, meta, s_w, R: int, n: int, m: int, *, ydt: int = SBN_BF16,
                            Y=None, ws=None, stream=None):
    """Y [T, R] = s_w * s_x[t] * (Xq @ Wt^T) from the packed weight."""
    return _matmul("sbn_sparse_ternary_gemm", Xq, s_x, codes, meta, s_w, R, n, m, ydt, Y, ws, stream)


def sbn_sparse_ternary_gemv(Xq, s_x, codes, meta, s_w, R: int, n: int, m: int, *, ydt: int = SBN_BF16,
                            Y=None, ws=None, stream=None):
    """Decode form (T <= 16) of sbn_sparse_ternary_gemm."""
    return _matmul("sbn_sparse_ternary_gemv", Xq, s_x, codes, meta, s_w, R, n, m, ydt, Y, ws, stream)


def sbn_forward(W, X, n: int, m: int, flags: int = 0, *, ydt: int = SBN_BF16, codes=None, meta=None, s_w=None,
                Xq=None, s_x=None, Y=None, ws=None, stream=None):
    """The whole forward (pack of W, quantization of X, sparse ternary GEMM) in
    one call.  Returns (codes, meta, s_w, Xq, s_x, Y)."""
    torch = _torch()
    R, K = W.shape
    T = X.shape[0]
    _req(W, "W", "bf16", False, "sbn_forward")
    _req(X, "X", "bf16", False, "sbn_forward")
    _req_matmul("sbn_forward", Xq, s_x, s_w, ydt, Y)
    for t, nm in ((codes, "codes"), (meta, "meta")):
        _req(t, nm, "u8", True, "sbn_forward")
    cb, mb = sbn_packed_bytes(R, K, n, m)
    dev = W.device
    if codes is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    if meta is None and mb:
        meta = torch.empty(mb, dtype=torch.uint8, device=dev)
    if s_w is None:
        s_w = torch.empty(1, dtype=torch.float32, device=dev)
    if Xq is None:
        Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    if s_x is None:
        s_x = torch.empty(T, dtype=torch.float32, device=dev)
    if Y is None:                                    # row stride rounded up to 8 elements (the ABI's rule)
        Y = torch.empty((T, (R + 7) // 8 * 8), dtype=getattr(torch, _YT[ydt]), device=dev)[:, :R]
    need = sbn_workspace_bytes(SBN_OP_FORWARD, T, R, K, n, m)
    if ws is None:
        ws = _workspace("fwd", need, dev, stream)
    _check("sbn_forward",
           lib().sbn_forward(_ptr(W), R, K, W.stride(0), _ptr(X), T, X.stride(0), n, m, flags, _ptr(codes),
                             _ptr(meta), _ptr(s_w), _ptr(Xq), _ptr(s_x), _ptr(Y), ydt, Y.stride(0), _ptr(ws),
                             ws.numel(), _stream(stream)))
    return codes, meta, s_w, Xq, s_x, Y


def sbn_gemm_weight_bytes(R: int, K: int, n: int, m: int) -> int:
    b = _sz()
    _check("sbn_gemm_weight_bytes", lib().sbn_gemm_weight_bytes(R, K, n, m, ctypes.byref(b)))
    return b.value


def sbn_prepare_gemm_weight(codes, meta, R: int, K: int, n: int, m: int, *, prepared=None, stream=None):
    """The GEMM's weight operand, built once from the packed planes (uint8, opaque)."""
    torch = _torch()
    _req(codes, "codes", "u8", True, "sbn_prepare_gemm_weight")
    _req(meta, "meta", "u8", True, "sbn_prepare_gemm_weight")
    _req(prepared, "prepared", "u8", True, "sbn_prepare_gemm_weight")
    if prepared is None:
        prepared = torch.empty(sbn_gemm_weight_bytes(R, K, n, m), dtype=torch.uint8, device=codes.device)
    _check("sbn_prepare_gemm_weight",
           lib().sbn_prepare_gemm_weight(_ptr(codes), _ptr(meta), R, K, n, m, _ptr(prepared), _stream(stream)))
    return prepared


def sbn_sparse_ternary_gemm_prepared(Xq, s_x, prepared, s_w, R: int, n: int, m: int, *, ydt: int = SBN_BF16, Y=None,
                                     ws=None, stream=None):
    """sbn_sparse_ternary_gemm on a prepared weight operand.  Returns Y [T, R]."""
    torch = _torch()
    T, K = Xq.shape
    _req_matmul("sbn_sparse_ternary_gemm_prepared", Xq, s_x, s_w, ydt, Y)
    _req(prepared, "prepared", "u8", True, "sbn_sparse_ternary_gemm_prepared")
    if Y is None:                                    # row stride rounded up to 8 elements (the ABI's rule)
        Y = torch.empty((T, (R + 7) // 8 * 8), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R]
    need = sbn_workspace_bytes(SBN_OP_GEMM_PREPARED, T, R, K, n, m)
    if ws is None:
        ws = _workspace("gemm", need, Xq.device, stream)
    _check("sbn_sparse_ternary_gemm_prepared",
           lib().sbn_sparse_ternary_gemm_prepared(_ptr(Xq), _ptr(s_x), T, K, _ptr(prepared), _ptr(s_w), R, n, m,
                                                  _ptr(Y), ydt, Y.stride(0), _ptr(ws), ws.numel() if ws is not None else 0,
                                                  _stream(stream)))
    return Y


def sbn_decode_plane_bytes(R: int, K: int) -> int:
    b = _sz()
    _check("sbn_decode_plane_bytes", lib().sbn_decode_plane_bytes(R, K, ctypes.byref(b)))
    return b.value


def sbn_repack_d2(codes, meta, R: int, K: int, n: int, m: int, *, d2=None, stream=None):
    """Decode plane (uint8, sbn_decode_plane_bytes(R, K)) of a packed n:m weight."""
    torch = _torch()
    _req(codes, "codes", "u8", True, "sbn_repack_d2")
    _req(meta, "meta", "u8", True, "sbn_repack_d2")
    _req(d2, "d2", "u8", True, "sbn_repack_d2")
    if d2 is None:
        d2 = torch.empty(sbn_decode_plane_bytes(R, K), dtype=torch.uint8, device=codes.device)
    _check("sbn_repack_d2", lib().sbn_repack_d2(_ptr(codes), _ptr(meta), R, K, n, m, _ptr(d2), _stream(stream)))
    return d2


def sbn_ternary_gemv_d2(Xq, s_x, d2, s_w, R: int, *, ydt: int = SBN_BF16, Y=None, stream=None):
    """Decode GEMV (T <= 16) on a decode plane.  Returns Y [T, R]."""
    torch = _torch()
    T, K = Xq.shape
    _req_matmul("sbn_ternary_gemv_d2", Xq, s_x, s_w, ydt, Y)
    _req(d2, "d2", "u8", True, "sbn_ternary_gemv_d2")
    if Y is None:                                    # row stride rounded up to 8 elements (the ABI's rule)
        Y = torch.empty((T, (R + 7) // 8 * 8), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R]
    _check("sbn_ternary_gemv_d2", lib().sbn_ternary_gemv_d2(_ptr(Xq), _ptr(s_x), T, K, _ptr(d2), _ptr(s_w), R, _ptr(Y),
                                                          ydt, Y.stride(0), _stream(stream)))
    return Y


def sbn_ternary_gemv_d2_batched(Xq, s_x, d2s, s_ws, R: int, *, ydt: int = SBN_BF16, Ys=None, stream=None):
    """sbn_ternary_gemv_d2 over several planes sharing Xq (lists of tensors).  Returns the list of Y."""
    torch = _torch()
    T, K = Xq.shape
    count = len(d2s)
    for b in range(count):
        _req_matmul("sbn_ternary_gemv_d2_batched", Xq, s_x, s_ws[b], ydt, Ys[b] if Ys is not None else None)
        _req(d2s[b], "d2", "u8", True, "sbn_ternary_gemv_d2_batched")
    if Ys is None:
        ld = (R + 7) // 8 * 8
        Ys = [torch.empty((T, ld), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R] for _ in range(count)]
    arr = lambda ts: (_vp * max(count, 1))(*[t.data_ptr() for t in ts])
    _check("sbn_ternary_gemv_d2_batched",
           lib().sbn_ternary_gemv_d2_batched(_ptr(Xq), _ptr(s_x), T, K, arr(d2s), arr(s_ws), R, arr(Ys), ydt,
                                             Ys[0].stride(0) if count else R, count, _stream(stream)))
    return Ys


def sbn_sparse_ternary_gemv_batched(Xq, s_x, codes, metas, s_ws, R: int, n: int, m: int, *,
                                    ydt: int = SBN_BF16, Ys=None, stream=None):
    """sbn_sparse_ternary_gemv for several weights sharing Xq: codes, metas, s_ws
    (and Ys) are lists of tensors, one per weight.  Returns the list of Y."""
    torch = _torch()
    T, K = Xq.shape
    count = len(codes)
    for b in range(count):
        _req_matmul("sbn_sparse_ternary_gemv_batched", Xq, s_x, s_ws[b], ydt, Ys[b] if Ys is not None else None)
        _req(codes[b], "codes", "u8", True, "sbn_sparse_ternary_gemv_batched")
        _req(metas[b] if metas is not None else None, "meta", "u8", True, "sbn_sparse_ternary_gemv_batched")
    if Ys is None:                                   # row stride rounded up to 8 elements (the ABI's rule)
        ld = (R + 7) // 8 * 8
        Ys = [torch.empty((T, ld), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R] for _ in range(count)]
    arr = lambda ts: (_vp * max(count, 1))(*[None if t is None else t.data_ptr() for t in ts])
    metas_a = None if metas is None else arr(metas)
    _check("sbn_sparse_ternary_gemv_batched",
           lib().sbn_sparse_ternary_gemv_batched(_ptr(Xq), _ptr(s_x), T, K, arr(codes), metas_a, arr(s_ws), R, n, m,
                                                 arr(Ys), ydt, Ys[0].stride(0) if count else R, count,
                                                 _stream(stream)))
    return Ys


class GemvTable:
    """The weights of a table GEMV: per weight the device pointers of its
    packed planes (or decode plane), scale and output, in a table in device
    memory (sbn_gemv_entry: four pointers), built once and reused by every
    sbn_sparse_ternary_gemv_table / sbn_ternary_gemv_d2_table call.  The
    entries are checked on the host (sbn_gemv_table_check) before the copy;
    the object holds a reference to every tensor the table points at, so they
    stay alive as long as it does.  Ys: the outputs ([T, R] each, allocated
    with the row stride rounded up to 8 when not given)."""

    def __init__(self, codes, metas, s_ws, R: int, K: int, n: int, m: int, *, T: int = 1, ydt: int = SBN_BF16,
                 Ys=None, d2: bool = False, form: int = None):
        torch = _torch()
        if form is None:
            form = SBN_FORM_D2 if d2 else SBN_FORM_PACKED
        fn = {SBN_FORM_PACKED: "sbn_sparse_ternary_gemv_table", SBN_FORM_D2: "sbn_ternary_gemv_d2_table",
              SBN_FORM_J6: "sbn_ternary_gemv_j6_table"}[form]
        count = len(codes)
        if count < 1:
            raise SbnError(fn, 2, "a table needs at least one weight")
        for b in range(count):
            _req(codes[b], "codes", "u8", True, fn)
            _req(None if form == SBN_FORM_D2 or metas is None else metas[b], "meta", "u8", True, fn)
            _req(s_ws[b], "s_w", "f32", True, fn)
            if Ys is not None:
                if ydt in _YD:
                    _req(Ys[b], "Y", _YD[ydt], False, fn)
                if tuple(Ys[b].shape) != (T, R) or Ys[b].stride(0) != Ys[0].stride(0):
                    raise SbnError(fn, 2, f"every Y must be [{T}, {R}] with one row stride")
        dev = codes[0].device
        if Ys is None:
            ld = (R + 7) // 8 * 8
            Ys = [torch.empty((T, ld), dtype=getattr(torch, _YT[ydt]), device=dev)[:, :R] for _ in range(count)]
        ldy = Ys[0].stride(0)
        ptr = lambda t: 0 if t is None else t.data_ptr()
        host = (_vp * (4 * count))()
        for b in range(count):
            mt = None if form == SBN_FORM_D2 or metas is None else metas[b]
            host[4 * b: 4 * b + 4] = [ptr(codes[b]), ptr(mt), ptr(s_ws[b]), ptr(Ys[b])]
        _check("sbn_gemv_table_check", lib().sbn_gemv_table_check(host, count, T, K, R, n, m, form, ydt, ldy))
        flat = torch.tensor([0 if v is None else v for v in host], dtype=torch.int64)
        self.dev = flat.to(dev)                      # count x 4 pointers; 16-byte aligned (allocator)
        self.codes, self.metas, self.s_ws, self.Ys = list(codes), None if metas is None else list(metas), list(s_ws), Ys
        self.R, self.K, self.n, self.m, self.T, self.ydt, self.ldy = R, K, n, m, T, ydt, ldy
        self.count, self.form = count, form
        self.d2 = form == SBN_FORM_D2

    @classmethod
    def planes(cls, d2s, s_ws, R: int, K: int, *, T: int = 1, ydt: int = SBN_BF16, Ys=None):
        """A table of decode planes (sbn_repack_d2 outputs)."""
        return cls(d2s, None, s_ws, R, K, 0, 0, T=T, ydt=ydt, Ys=Ys, form=SBN_FORM_D2)

    @classmethod
    def joint(cls, nibs, hs, s_ws, R: int, K: int, *, T: int = 1, ydt: int = SBN_BF16, Ys=None):
        """A table of joint 2:4 codes (sbn_repack_j6 outputs: nibble and h planes)."""
        return cls(nibs, hs, s_ws, R, K, 2, 4, T=T, ydt=ydt, Ys=Ys, form=SBN_FORM_J6)


def _table_call(fn, Xq, s_x, table):
    T, K = Xq.shape
    _req(Xq, "Xq", "i8", True, fn)
    _req(s_x, "s_x", "f32", True, fn)
    if not isinstance(table, GemvTable):
        raise SbnError(fn, 2, "table must be a GemvTable")
    if (T, K) != (table.T, table.K) or Xq.device != table.dev.device:
        raise SbnError(fn, 2, f"Xq [{T}, {K}] on {Xq.device} does not match the table's T = {table.T}, "
                              f"K = {table.K} on {table.dev.device}")
    return T, K


def sbn_j6_bytes(R: int, K: int) -> tuple[int, int]:
    nb, hb = _sz(), _sz()
    _check("sbn_j6_bytes", lib().sbn_j6_bytes(R, K, ctypes.byref(nb), ctypes.byref(hb)))
    return nb.value, hb.value


def sbn_repack_j6(codes, meta, R: int, K: int, *, nib=None, hpl=None, stream=None):
    """2:4 packed planes -> joint 2:4 code planes.  Returns (nib, hpl)."""
    torch = _torch()
    for t, name in ((codes, "codes"), (meta, "meta"), (nib, "nib"), (hpl, "hpl")):
        _req(t, name, "u8", True, "sbn_repack_j6")
    nb, hb = sbn_j6_bytes(R, K)
    if nib is None:
        nib = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    if hpl is None:
        hpl = torch.empty(hb, dtype=torch.uint8, device=codes.device)
    _check("sbn_repack_j6", lib().sbn_repack_j6(_ptr(codes), _ptr(meta), R, K, _ptr(nib), _ptr(hpl), _stream(stream)))
    return nib, hpl


def sbn_ternary_gemv_j6(Xq, s_x, nib, hpl, s_w, R: int, *, ydt: int = SBN_BF16, Y=None, stream=None):
    """Decode GEMV (T <= 16) on a joint 2:4 code.  Returns Y [T, R]."""
    torch = _torch()
    T, K = Xq.shape
    _req_matmul("sbn_ternary_gemv_j6", Xq, s_x, s_w, ydt, Y)
    _req(nib, "nib", "u8", True, "sbn_ternary_gemv_j6")
    _req(hpl, "hpl", "u8", True, "sbn_ternary_gemv_j6")
    if Y is None:
        Y = torch.empty((T, (R + 7) // 8 * 8), dtype=getattr(torch, _YT[ydt]), device=Xq.device)[:, :R]
    _check("sbn_ternary_gemv_j6", lib().sbn_ternary_gemv_j6(_ptr(Xq), _ptr(s_x), T, K, _ptr(nib), _ptr(hpl), _ptr(s_w),
                                                          R, _ptr(Y), ydt, Y.stride(0), _stream(stream)))
    return Y


def sbn_ternary_gemv_j6_table(Xq, s_x, table, *, stream=None):
    """Decode GEMV of every weight of `table` (GemvTable.joint) against Xq, one
    launch.  Returns the table's list of Y."""
    fn = "sbn_ternary_gemv_j6_table"
    T, K = _table_call(fn, Xq, s_x, table)
    if table.form != SBN_FORM_J6:
        raise SbnError(fn, 2, "the table does not hold joint codes")
    _check(fn, lib().sbn_ternary_gemv_j6_table(_ptr(Xq), _ptr(s_x), T, K, table.dev.data_ptr(), table.count, table.R,
                                               table.ydt, table.ldy, _stream(stream)))
    return table.Ys


def sbn_sparse_ternary_gemv_table(Xq, s_x, table, *, stream=None):
    """Decode GEMV of every weight of `table` (a GemvTable of packed weights)
    against Xq, one launch.  Returns the table's list of Y."""
    fn = "sbn_sparse_ternary_gemv_table"
    T, K = _table_call(fn, Xq, s_x, table)
    if table.form != SBN_FORM_PACKED:
        raise SbnError(fn, 2, "the table does not hold packed weights")
    _check(fn, lib().sbn_sparse_ternary_gemv_table(_ptr(Xq), _ptr(s_x), T, K, table.dev.data_ptr(), table.count,
                                                   table.R, table.n, table.m, table.ydt, table.ldy, _stream(stream)))
    return table.Ys


def sbn_ternary_gemv_d2_table(Xq, s_x, table, *, stream=None):
    """Decode GEMV of every plane of `table` (GemvTable.planes) against Xq,
    one launch.  Returns the table's list of Y."""
    fn = "sbn_ternary_gemv_d2_table"
    T, K = _table_call(fn, Xq, s_x, table)
    if table.form != SBN_FORM_D2:
        raise SbnError(fn, 2, "the table does not hold decode planes")
    _check(fn, lib().sbn_ternary_gemv_d2_table(_ptr(Xq), _ptr(s_x), T, K, table.dev.data_ptr(), table.count, table.R,
                                               table.ydt, table.ldy, _stream(stream)))
    return table.Ys


def _backward(name, flags, dY, Xq, s_x, codes, meta, s_w, n, m, dxdt, want_dX, want_dW, dX, dW, ws, stream):
    torch = _torch()
    T, R = dY.shape
    K = Xq.shape[1]
    _req(dY, "dY", "bf16", True, name)
    _req(Xq, "Xq", "i8", True, name)
    _req(s_x, "s_x", "f32", True, name)
    _req(s_w, "s_w", "f32", True, name)
    _req(codes, "codes", "u8", True, name)
    _req(meta, "meta", "u8", True, name)
    _req(dX, "dX", "f32" if dxdt == SBN_F32 else "bf16", True, name)
    _req(dW, "dW", "f32", True, name)
    if want_dX and dX is None:
        dX = torch.empty((T, K), dtype=torch.float32 if dxdt == SBN_F32 else torch.bfloat16, device=dY.device)
    if want_dW and dW is None:
        dW = torch.empty((R, K), dtype=torch.float32, device=dY.device)
    need = sbn_workspace_bytes(SBN_OP_BACKWARD, T, R, K, n, m)
    if ws is None:
        ws = _workspace("bwd", need, dY.device, stream)
    args = [_ptr(dY), T, R, _ptr(Xq), _ptr(s_x), K, _ptr(codes), _ptr(meta), _ptr(s_w), n, m,
            _ptr(dX if want_dX else None), dxdt, _ptr(dW if want_dW else None)]
    if flags is not None:
        args.append(flags)
    args += [_ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)]
    _check(name, getattr(lib(), name)(*args))
    return (dX if want_dX else None), (dW if want_dW else None)


def sbn_backward(dY, Xq, s_x, codes, meta, s_w, n: int, m: int, *, dxdt: int = SBN_F32, want_dX: bool = True,
                 want_dW: bool = True, dX=None, dW=None, ws=None, stream=None):
    """Dual-STE backward.  Returns (dX [T, K] or None, dW [R, K] float32 or None)."""
    return _backward("sbn_backward", None, dY, Xq, s_x, codes, meta, s_w, n, m, dxdt, want_dX, want_dW, dX, dW,
                     ws, stream)


def sbn_backward_ex(dY, Xq, s_x, codes, meta, s_w, n: int, m: int, flags: int, *, dxdt: int = SBN_F32,
                    want_dX: bool = True, want_dW: bool = True, dX=None, dW=None, ws=None, stream=None):
    """sbn_backward with variant flags (SBN_GRAD_W_MASKED).  Returns (dX or None, dW or None)."""
    return _backward("sbn_backward_ex", flags, dY, Xq, s_x, codes, meta, s_w, n, m, dxdt, want_dX, want_dW, dX,
                     dW, ws, stream)


# ------------------------------------------------------------------ kernel timing
def sbn_profile_enable(on: bool = True, kernel: str | None = None) -> None:
    """Bracket library kernel launches (all, or only those named `kernel`) with
    HIP events on their stream."""
    _check("sbn_profile_enable", lib().sbn_profile_enable(1 if on else 0, kernel.encode() if kernel else None))


def sbn_profile_reset() -> None:
    _check("sbn_profile_reset", lib().sbn_profile_reset())


def sbn_profile_dump() -> dict:
    """{kernel name: (launches, total milliseconds)} since the last reset."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check("sbn_profile_dump", lib().sbn_profile_dump(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


__all__ = [
    "lib", "header_symbols", "SbnError", "sbn_abi_version", "sbn_packed_bytes", "sbn_workspace_bytes",
    "sbn_mask_ternarize_pack", "sbn_mask_ternarize_pack_noalloc", "sbn_act_quant", "sbn_sparse_ternary_gemm", "sbn_sparse_ternary_gemv",
    "sbn_backward", "sbn_backward_ex", "sbn_mask_ternarize_pack_ex", "sbn_sgd_update_pack", "sbn_forward",
    "sbn_decode_plane_bytes", "sbn_repack_d2", "sbn_ternary_gemv_d2", "sbn_ternary_gemv_d2_batched",
    "GemvTable", "sbn_sparse_ternary_gemv_table", "sbn_ternary_gemv_d2_table", "SBN_FORM_PACKED", "SBN_FORM_D2",
    "SBN_FORM_J6", "sbn_j6_bytes", "sbn_repack_j6", "sbn_ternary_gemv_j6", "sbn_ternary_gemv_j6_table",
    "sbn_gemm_weight_bytes", "sbn_prepare_gemm_weight", "sbn_sparse_ternary_gemm_prepared", "SBN_OP_GEMM_PREPARED",
    "SBN_ERR_VALUE",
    "SBN_FLAGS_NONE", "SBN_MASK_FROM_TERNARY", "SBN_GRAD_W_MASKED",
    "SBN_F32", "SBN_BF16", "SBN_I32_ACC", "SBN_OP_PACK", "SBN_OP_ACT_QUANT", "SBN_OP_GEMM",
    "SBN_OP_GEMV", "SBN_OP_BACKWARD", "SBN_OP_FORWARD", "sbn_profile_enable", "sbn_profile_reset", "sbn_profile_dump",
]
