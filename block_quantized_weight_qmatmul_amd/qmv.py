"""Python binding of the qmv C ABI (include/qmv.h): argument marshalling only.

Every computation runs in the HIP kernels of ``libqmv.so``; this module only
turns torch tensors (device memory, streams) into the pointers and sizes the
C functions take, and turns a negative status into an exception. There is no
fallback: if the library is missing, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqmv.so")

QMV_OK, QMV_EINVAL, QMV_EALIGN, QMV_EUNSUPPORTED, QMV_EHIP = 0, -1, -2, -3, -4
QMV_Q4_0, QMV_Q8_0, QMV_Q5_K, QMV_Q6_K = 2, 8, 13, 14
QMV_MAX_M = 16
BLOCK_BYTES = {QMV_Q4_0: 18, QMV_Q8_0: 34, QMV_Q5_K: 176, QMV_Q6_K: 210}
QTYPES = {"q4_0": QMV_Q4_0, "q8_0": QMV_Q8_0, "q5_k": QMV_Q5_K, "q6_k": QMV_Q6_K}

QMV_MAX_BATCH = 16

_lib = None


class Problem(ctypes.Structure):
    """C layout of qmv_problem (include/qmv.h)."""
    _fields_ = [("W", ctypes.c_void_p), ("ldw_bytes", ctypes.c_size_t), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int)]


class QmvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qmv status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqmv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m block_quantized_weight_qmatmul_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        for name in ("qmv_q4_0", "qmv_q8_0", "qmv_q5_k", "qmv_q6_k"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [P, S, P, S, P, S, I, I, I, P]
        L.qmv_id.restype = I
        L.qmv_id.argtypes = [I, P, S, S, I, P, S, P, I, I, P, S, I, I, P, P, P]
        L.qmv_id_swiglu.restype = I
        L.qmv_id_swiglu.argtypes = [I, P, S, S, I, P, S, P, I, I, P, S, I, I, P, P, P]
        L.qmv_moe_wsum.restype = I
        L.qmv_moe_wsum.argtypes = [P, S, P, I, I, I, P, S, P]
        L.qmv_moe_down.restype = I
        L.qmv_moe_down.argtypes = [I, P, S, S, I, P, S, P, P, I, I, P, S, I, I, P, P, P]
        L.qmv_affine4.restype = I
        L.qmv_affine4.argtypes = [P, S, P, P, S, P, S, P, S, I, I, I, P]
        L.qmv_affine4_id.restype = I
        L.qmv_affine4_id.argtypes = [P, S, S, P, P, S, S, I, P, S, P, I, I, P, S, I, I, P, P, P]
        L.qmv_gemm.restype = I
        L.qmv_gemm.argtypes = [I, P, S, P, S, P, S, I, I, I, P]
        L.qmv_batch.restype = I
        L.qmv_batch.argtypes = [I, ctypes.POINTER(Problem), I, P]
        L.qmv_ws.restype = I
        L.qmv_ws.argtypes = [I, P, S, P, S, P, S, I, I, I, P, S, P]
        L.qmv_ws_static.restype = I
        L.qmv_ws_static.argtypes = [I, P, S, P, S, P, S, I, I, I, P]
        L.qmv_ws_bytes.restype = S
        L.qmv_ws_bytes.argtypes = [I, I, I, I]
        L.qmv_last_error.restype = ctypes.c_char_p
        L.qmv_last_error.argtypes = []
        L.qmv_stream_read.restype = I
        L.qmv_stream_read.argtypes = [P, S, P, P]
        _lib = L
    return _lib


def _qt(qtype) -> int:
    return QTYPES[qtype] if isinstance(qtype, str) else int(qtype)


def last_error() -> str:
    return lib().qmv_last_error().decode()


def _check(status: int) -> None:
    if status != QMV_OK:
        raise QmvError(status, last_error())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


# ---------------------------------------------------------------------------
# Raw calls: pointers and sizes as integers, status returned (for tests of the
# argument checks and for callers that manage their own memory).
# ---------------------------------------------------------------------------
def raw_qmv(qtype: int, W: int, ldw: int, X: int, ldx: int, Y: int, ldy: int, M: int, N: int, K: int,
            stream: int = 0) -> int:
    f = {QMV_Q4_0: lib().qmv_q4_0, QMV_Q8_0: lib().qmv_q8_0, QMV_Q5_K: lib().qmv_q5_k, QMV_Q6_K: lib().qmv_q6_k}[qtype]
    return f(W, ldw, X, ldx, Y, ldy, M, N, K, stream)


def raw_qmv_ws(qtype: int, W: int, ldw: int, X: int, ldx: int, Y: int, ldy: int, M: int, N: int, K: int,
               ws: int, ws_bytes: int, stream: int = 0) -> int:
    return lib().qmv_ws(qtype, W, ldw, X, ldx, Y, ldy, M, N, K, ws, ws_bytes, stream)


def raw_qmv_ws_static(qtype: int, W: int, ldw: int, X: int, ldx: int, Y: int, ldy: int, M: int, N: int, K: int,
                      stream: int = 0) -> int:
    return lib().qmv_ws_static(qtype, W, ldw, X, ldx, Y, ldy, M, N, K, stream)


def raw_stream_read(src: int, nbytes: int, sink: int, stream: int = 0) -> int:
    return lib().qmv_stream_read(src, nbytes, sink, stream)


def stream_read(buf, sink, stream=None) -> None:
    """Read every byte of the device tensor buf once (the streaming-read
    reference of measurements); sink: a device int32 tensor of one element."""
    _check(raw_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def ws_bytes(qtype, M: int, N: int, K: int) -> int:
    """Workspace bytes qmv_ws uses for these sizes (0: it would not split K)."""
    return int(lib().qmv_ws_bytes(_qt(qtype), M, N, K))


def raw_qmv_id(qtype, W, expert_stride, ldw, n_experts, X, ldx, ids, n_tokens, top_k, Y, ldy, N, K,
               expert_scale=0, err_flag=0, stream=0) -> int:
    return lib().qmv_id(qtype, W, expert_stride, ldw, n_experts, X, ldx, ids, n_tokens, top_k, Y, ldy, N, K,
                        expert_scale, err_flag, stream)


def raw_qmv_id_swiglu(qtype, W, expert_stride, ldw, n_experts, G, ldg, ids, n_tokens, top_k, Y, ldy, N, K,
                      expert_scale=0, err_flag=0, stream=0) -> int:
    return lib().qmv_id_swiglu(qtype, W, expert_stride, ldw, n_experts, G, ldg, ids, n_tokens, top_k, Y, ldy, N, K,
                               expert_scale, err_flag, stream)


def raw_qmv_moe_wsum(Y, ldy, weights, n_tokens, top_k, N, out, ldo, stream=0) -> int:
    return lib().qmv_moe_wsum(Y, ldy, weights, n_tokens, top_k, N, out, ldo, stream)


def raw_qmv_moe_down(qtype, W, expert_stride, ldw, n_experts, G, ldg, ids, weights, n_tokens, top_k, out, ldo, N, K,
                     expert_scale=0, err_flag=0, stream=0) -> int:
    return lib().qmv_moe_down(qtype, W, expert_stride, ldw, n_experts, G, ldg, ids, weights, n_tokens, top_k, out,
                              ldo, N, K, expert_scale, err_flag, stream)


def raw_qmv_batch(qtype: int, problems, stream: int = 0) -> int:
    """problems: sequence of (W, ldw_bytes, x, y, N, K) integer tuples."""
    arr = (Problem * max(1, len(problems)))(*[Problem(*p) for p in problems])
    return lib().qmv_batch(qtype, arr, len(problems), stream)


# ---------------------------------------------------------------------------
# Tensor calls.
# ---------------------------------------------------------------------------
def _dense(qtype: int, W, X, Y, K: Optional[int], stream) -> None:
    """W: uint8 [N, ldw] (row stride W.stride(0) bytes); X: fp32 [M, K] or [K];
    Y: fp32 [M, N] or [N]."""
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D uint8 tensor with contiguous rows")
    N = W.shape[0]
    x2 = X if X.dim() == 2 else X.view(1, -1)
    y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    M = x2.shape[0]
    if K is None:
        K = x2.shape[1]
    if x2.stride(1) != 1 or y2.stride(1) != 1 or y2.shape[0] != M or y2.shape[1] != N:
        raise ValueError("X [M, K] and Y [M, N] need unit inner stride and matching M, N")
    st = raw_qmv(qtype, _ptr(W), W.stride(0), _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0), M, N, K,
                 _stream(stream))
    _check(st)


def qmv_ws(qtype, W, X, Y, workspace, K: Optional[int] = None, stream=None) -> None:
    """qmv_q4_0 / qmv_q8_0 with a caller workspace (a uint8 device tensor of at
    least ws_bytes(qtype, M, N, K) bytes, or None) -- see include/qmv.h."""
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a 2-D uint8 tensor with contiguous rows")
    x2 = X if X.dim() == 2 else X.view(1, -1)
    y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    M, N = x2.shape[0], W.shape[0]
    if K is None:
        K = x2.shape[1]
    if x2.stride(1) != 1 or y2.stride(1) != 1 or y2.shape[0] != M or y2.shape[1] != N:
        raise ValueError("X [M, K] and Y [M, N] need unit inner stride and matching M, N")
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(raw_qmv_ws(_qt(qtype), _ptr(W), W.stride(0), _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0), M, N, K,
                      _ptr(workspace), nb, _stream(stream)))


def qmv_q4_0(W, X, Y, K: Optional[int] = None, stream=None) -> None:
    """Y = deq(W) @ X per row, Q4_0 weights (see include/qmv.h)."""
    _dense(QMV_Q4_0, W, X, Y, K, stream)


def qmv_q8_0(W, X, Y, K: Optional[int] = None, stream=None) -> None:
    """Y = deq(W) @ X per row, Q8_0 weights (see include/qmv.h)."""
    _dense(QMV_Q8_0, W, X, Y, K, stream)


def qmv_q6_k(W, X, Y, K: Optional[int] = None, stream=None) -> None:
    """Y = deq(W) @ X per row, Q6_K super-blocks (see include/qmv.h)."""
    _dense(QMV_Q6_K, W, X, Y, K, stream)


def qmv_q5_k(W, X, Y, K: Optional[int] = None, stream=None) -> None:
    """Y = deq(W) @ X per row, Q5_K super-blocks (see include/qmv.h)."""
    _dense(QMV_Q5_K, W, X, Y, K, stream)


def raw_qmv_gemm(qtype: int, W: int, ldw: int, X: int, ldx: int, Y: int, ldy: int, M: int, N: int, K: int,
                 stream: int = 0) -> int:
    return lib().qmv_gemm(qtype, W, ldw, X, ldx, Y, ldy, M, N, K, stream)


def qmv_gemm(qtype, W, X, Y, K: Optional[int] = None, stream=None) -> None:
    """Y = deq(W) @ X per row for any number of rows M (see include/qmv.h).

    W: uint8 [N, ldw]; X: fp32 [M, K]; Y: fp32 [M, N]."""
    q = QTYPES[qtype] if isinstance(qtype, str) else int(qtype)
    if W.dim() != 2 or W.stride(1) != 1 or X.dim() != 2 or Y.dim() != 2:
        raise ValueError("W [N, ldw], X [M, K] and Y [M, N] must be 2-D")
    M, N = Y.shape
    K = X.shape[1] if K is None else K
    if X.shape[0] != M or W.shape[0] != N or X.stride(1) != 1 or Y.stride(1) != 1:
        raise ValueError("X [M, K] and Y [M, N] need unit inner stride and matching M, N")
    _check(raw_qmv_gemm(q, _ptr(W), W.stride(0), _ptr(X), X.stride(0), _ptr(Y), Y.stride(0), M, N, K,
                        _stream(stream)))


def raw_qmv_affine4(Wq, ldw, S, B, lds, X, ldx, Y, ldy, M, N, K, stream=0) -> int:
    return lib().qmv_affine4(Wq, ldw, S, B, lds, X, ldx, Y, ldy, M, N, K, stream)


def qmv_affine4(Wq, S, B, X, Y, stream=None) -> None:
    """Affine 4-bit product (see include/qmv.h): Wq int32/uint32 [N, >= K/8],
    S, B int16/uint16 bf16 bit patterns [N, >= K/32], X fp32 [M, K] or [K],
    Y fp32 [M, N] or [N]."""
    x2 = X if X.dim() == 2 else X.view(1, -1)
    y2 = Y if Y.dim() == 2 else Y.view(1, -1)
    M, K = x2.shape
    N = Wq.shape[0]
    if Wq.stride(1) != 1 or S.stride(1) != 1 or B.stride(1) != 1 or S.stride(0) != B.stride(0):
        raise ValueError("Wq, S and B need contiguous rows; S and B one row stride")
    _check(raw_qmv_affine4(_ptr(Wq), Wq.stride(0), _ptr(S), _ptr(B), S.stride(0), _ptr(x2), x2.stride(0), _ptr(y2),
                           y2.stride(0), M, N, K, _stream(stream)))


def qmv_affine4_id(Wq, S, B, X, ids, Y, N: int, K: int, expert_scale=None, err_flag=None, stream=None) -> None:
    """Expert-indexed affine 4-bit product: Wq [E, N, >= K/8] words, S, B [E, N, >= K/32]
    bf16 bit patterns, X fp32 [n_tokens, K], ids [n_tokens, top_k], Y fp32 [n_tokens*top_k, N]."""
    ids2 = ids if ids.dim() == 2 else ids.view(-1, 1)
    n_tokens, top_k = ids2.shape
    if S.stride() != B.stride() or Wq.stride(2) != 1 or S.stride(2) != 1 or not ids2.is_contiguous():
        raise ValueError("S and B need one layout, contiguous rows; ids contiguous")
    _check(lib().qmv_affine4_id(_ptr(Wq), Wq.stride(0), Wq.stride(1), _ptr(S), _ptr(B), S.stride(0), S.stride(1),
                                Wq.shape[0], _ptr(X), X.stride(0), _ptr(ids2), n_tokens, top_k, _ptr(Y), Y.stride(0),
                                N, K, _ptr(expert_scale), _ptr(err_flag), _stream(stream)))


def qmv_id(qtype, W, X, ids, Y, N: int, K: int, expert_scale=None, err_flag=None, stream=None) -> None:
    """Expert-indexed product (see include/qmv.h).

    W: uint8 [E, N, ldw] stacked experts (expert stride W.stride(0) bytes,
    row stride W.stride(1)); X: fp32 [n_tokens, K]; ids: uint32 or int32
    [n_tokens, top_k]; Y: fp32 [n_tokens * top_k, N].
    """
    q = QTYPES[qtype] if isinstance(qtype, str) else int(qtype)
    if W.dim() != 3 or W.stride(2) != 1:
        raise ValueError("W must be a 3-D uint8 tensor [E, N, ldw] with contiguous rows")
    ids2 = ids if ids.dim() == 2 else ids.view(-1, 1)
    n_tokens, top_k = ids2.shape
    if not ids2.is_contiguous():
        raise ValueError("ids must be contiguous")
    st = raw_qmv_id(q, _ptr(W), W.stride(0), W.stride(1), W.shape[0], _ptr(X), X.stride(0), _ptr(ids2),
                    n_tokens, top_k, _ptr(Y), Y.stride(0), N, K, _ptr(expert_scale), _ptr(err_flag),
                    _stream(stream))
    _check(st)


def _stack(W):
    if W.dim() != 3 or W.stride(2) != 1:
        raise ValueError("W must be a 3-D uint8 tensor [E, N, ldw] with contiguous rows")


def qmv_id_swiglu(qtype, W, G, ids, Y, N: int, K: int, expert_scale=None, err_flag=None, stream=None) -> None:
    """qmv_id on the SwiGLU of gate_up rows (see include/qmv.h).

    W: uint8 [E, N, ldw]; G: fp32 [n_tokens, >= 2K] (gate half first);
    ids: [n_tokens, top_k] (or [n_tokens]); Y: fp32 [n_tokens * top_k, N].
    """
    q = QTYPES[qtype] if isinstance(qtype, str) else int(qtype)
    _stack(W)
    ids2 = ids if ids.dim() == 2 else ids.view(-1, 1)
    if not ids2.is_contiguous():
        raise ValueError("ids must be contiguous")
    n_tokens, top_k = ids2.shape
    st = raw_qmv_id_swiglu(q, _ptr(W), W.stride(0), W.stride(1), W.shape[0], _ptr(G), G.stride(0), _ptr(ids2),
                           n_tokens, top_k, _ptr(Y), Y.stride(0), N, K, _ptr(expert_scale), _ptr(err_flag),
                           _stream(stream))
    _check(st)


def qmv_moe_wsum(Y, weights, out, top_k: int, stream=None) -> None:
    """out[t] = sum_s weights[t*top_k + s] * Y[t*top_k + s] (see include/qmv.h).

    Y: fp32 [n_tokens * top_k, N]; weights: fp32 contiguous [n_tokens * top_k]
    (any shape); out: fp32 [n_tokens, N]."""
    if not weights.is_contiguous() or Y.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("weights must be contiguous; Y and out need unit inner stride")
    n_tokens, N = out.shape
    if Y.shape[0] != n_tokens * top_k or Y.shape[1] != N or weights.numel() != n_tokens * top_k:
        raise ValueError("Y must be [n_tokens*top_k, N] and weights hold n_tokens*top_k values")
    _check(raw_qmv_moe_wsum(_ptr(Y), Y.stride(0), _ptr(weights), n_tokens, top_k, N, _ptr(out), out.stride(0),
                            _stream(stream)))


def qmv_moe_down(qtype, W, G, ids, weights, out, N: int, K: int, expert_scale=None, err_flag=None,
                 stream=None) -> None:
    """SwiGLU + expert-indexed down product + weighted sum, one launch (see include/qmv.h).

    W: uint8 [E, N, ldw]; G: fp32 [n_tokens * top_k, >= 2K]; ids: [n_tokens, top_k];
    weights: fp32 contiguous [n_tokens, top_k]; out: fp32 [n_tokens, N]."""
    q = QTYPES[qtype] if isinstance(qtype, str) else int(qtype)
    _stack(W)
    if ids.dim() != 2 or not ids.is_contiguous() or not weights.is_contiguous():
        raise ValueError("ids must be a contiguous [n_tokens, top_k] tensor and weights contiguous")
    n_tokens, top_k = ids.shape
    if weights.numel() != n_tokens * top_k:
        raise ValueError("weights must hold n_tokens*top_k values")
    st = raw_qmv_moe_down(q, _ptr(W), W.stride(0), W.stride(1), W.shape[0], _ptr(G), G.stride(0), _ptr(ids),
                          _ptr(weights), n_tokens, top_k, _ptr(out), out.stride(0), N, K, _ptr(expert_scale),
                          _ptr(err_flag), _stream(stream))
    _check(st)


def qmv_batch(qtype, problems, stream=None) -> None:
    """Several independent M = 1 products in one launch (see include/qmv.h).

    problems: sequence of (W, x, y) tensors with W uint8 [N, ldw] (row stride
    W.stride(0) bytes), x fp32 [K] and y fp32 [N].
    """
    q = QTYPES[qtype] if isinstance(qtype, str) else int(qtype)
    raw = []
    for W, x, y in problems:
        if W.dim() != 2 or W.stride(1) != 1 or x.dim() != 1 or y.dim() != 1:
            raise ValueError("each problem needs W [N, ldw] with contiguous rows, x [K] and y [N]")
        raw.append((_ptr(W), W.stride(0), _ptr(x), _ptr(y), W.shape[0], x.shape[0]))
    _check(raw_qmv_batch(q, raw, _stream(stream)))
