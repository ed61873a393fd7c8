"""CPU oracle for block-quantized weight mat-vec (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. The HIP library and its Python
binding never import it, and it imports nothing of theirs.

The arithmetic lives in ``qmv_oracle.c`` (plain C, fp64, optional OpenMP over
output rows); this module builds it with gcc when no build is present and
wraps it with ctypes. See the C file's header for what is computed and which
passages of the hf2q pages each part follows.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(hand-built blocks under ``tests/golden/``, the Q8_0 encoder from the hf2q
model page, closed forms, exact rational brute force and the expert-routing
signature). None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q4_0, Q8_0, Q5_K, Q6_K = 2, 8, 13, 14
QTYPES = {"q4_0": Q4_0, "q8_0": Q8_0, "q5_k": Q5_K, "q6_k": Q6_K}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q5_K: 176, Q6_K: 210}
BLOCK_ELEMS = {Q4_0: 32, Q8_0: 32, Q5_K: 256, Q6_K: 256}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P, S, I, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_double
        lib.oracle_f16_to_f64.restype = D
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_dequant_row.restype = I
        lib.oracle_dequant_row.argtypes = [I, P, I, P]
        lib.oracle_qmv.restype = I
        lib.oracle_qmv.argtypes = [I, P, S, P, S, I, I, I, P, P, S, I]
        lib.oracle_qmv_id.restype = I
        lib.oracle_qmv_id.argtypes = [I, P, S, S, I, P, S, P, I, I, P, I, I, P, P, S, I]
        lib.oracle_qmv_id_swiglu.restype = I
        lib.oracle_qmv_id_swiglu.argtypes = [I, P, S, S, I, P, S, P, I, I, P, I, I, P, P, S, I]
        lib.oracle_silu.restype = D
        lib.oracle_silu.argtypes = [D]
        lib.oracle_swiglu.restype = I
        lib.oracle_swiglu.argtypes = [P, S, I, I, P, S]
        lib.oracle_moe_wsum.restype = I
        lib.oracle_moe_wsum.argtypes = [P, P, S, P, I, I, I, P, P, S]
        lib.oracle_bf16_to_f64.restype = D
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_dequant_affine4_row.restype = I
        lib.oracle_dequant_affine4_row.argtypes = [P, P, P, I, P]
        lib.oracle_qmv_affine4.restype = I
        lib.oracle_qmv_affine4.argtypes = [P, S, P, P, S, P, S, I, I, I, P, P, S, I]
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _qt(qtype) -> int:
    return QTYPES[qtype] if isinstance(qtype, str) else int(qtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits) & 0xFFFF)


def dequant_row(qtype, row: np.ndarray, K: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    q = _qt(qtype)
    if row.size < K // BLOCK_ELEMS[q] * BLOCK_BYTES[q]:
        raise ValueError("row too short")
    out = np.empty(K, dtype=np.float64)
    if _load().oracle_dequant_row(q, _ptr(row), K, _ptr(out)) != 0:
        raise ValueError("bad arguments")
    return out


def qmv(qtype, W: np.ndarray, X: np.ndarray, N: Optional[int] = None, K: Optional[int] = None,
        nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Y, A = oracle of Y = W_deq @ X^T per row: W uint8 [N, ldw], X fp32 [M, K].

    Returns (Y, A), both fp64 [M, N].
    """
    W = np.ascontiguousarray(W, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, Kx = X.shape
    K = Kx if K is None else K
    N = W.shape[0] if N is None else N
    Y = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_qmv(_qt(qtype), _ptr(W), W.shape[1], _ptr(X), Kx, M, N, K,
                            _ptr(Y), _ptr(A), N, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_qmv failed ({rc})")
    return Y, A


def qmv_id(qtype, W: np.ndarray, X: np.ndarray, ids: np.ndarray, N: int, K: int,
           expert_scale: Optional[np.ndarray] = None, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Expert-indexed oracle. W uint8 [E, N, ldw] stacked; X fp32 [n_tokens, K];
    ids uint32 [n_tokens, top_k]. Returns (Y, A) fp64 [n_tokens*top_k, N]."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    if ids.ndim == 1:
        ids = ids[:, None]
    E, Nw, ldw = W.shape
    n_tokens, top_k = ids.shape
    if X.shape[0] != n_tokens:
        raise ValueError("X rows must equal n_tokens")
    es = None if expert_scale is None else np.ascontiguousarray(expert_scale, dtype=np.float32)
    P = n_tokens * top_k
    Y = np.empty((P, N), dtype=np.float64)
    A = np.empty((P, N), dtype=np.float64)
    rc = _load().oracle_qmv_id(_qt(qtype), _ptr(W), Nw * ldw, ldw, E, _ptr(X), X.shape[1], _ptr(ids),
                               n_tokens, top_k, None if es is None else _ptr(es), N, K,
                               _ptr(Y), _ptr(A), N, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_qmv_id failed ({rc})")
    return Y, A


def silu(z: float) -> float:
    """silu(z) = z / (1 + exp(-z)) in fp64."""
    return _load().oracle_silu(float(z))


def swiglu(G: np.ndarray, I: Optional[int] = None) -> np.ndarray:
    """H[r, i] = silu(G[r, i]) * G[r, I + i] in fp64; G fp32 [rows, >= 2I] (gate half first)."""
    G = np.ascontiguousarray(G, dtype=np.float32)
    if G.ndim == 1:
        G = G[None, :]
    rows, ldg = G.shape
    I = ldg // 2 if I is None else I
    H = np.empty((rows, I), dtype=np.float64)
    if _load().oracle_swiglu(_ptr(G), ldg, rows, I, _ptr(H), I) != 0:
        raise ValueError("bad arguments")
    return H


def qmv_id_swiglu(qtype, W: np.ndarray, G: np.ndarray, ids: np.ndarray, N: int, K: int,
                  expert_scale: Optional[np.ndarray] = None, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Expert-indexed product over SwiGLU rows: X[t] = silu(G[t, :K]) * G[t, K:2K].

    W uint8 [E, N, ldw]; G fp32 [n_tokens, >= 2K]; ids uint32 [n_tokens, top_k].
    Returns (Y, A) fp64 [n_tokens*top_k, N]."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    G = np.ascontiguousarray(G, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    if ids.ndim == 1:
        ids = ids[:, None]
    E, Nw, ldw = W.shape
    n_tokens, top_k = ids.shape
    if G.shape[0] != n_tokens:
        raise ValueError("G rows must equal n_tokens")
    es = None if expert_scale is None else np.ascontiguousarray(expert_scale, dtype=np.float32)
    P = n_tokens * top_k
    Y = np.empty((P, N), dtype=np.float64)
    A = np.empty((P, N), dtype=np.float64)
    rc = _load().oracle_qmv_id_swiglu(_qt(qtype), _ptr(W), Nw * ldw, ldw, E, _ptr(G), G.shape[1], _ptr(ids),
                                      n_tokens, top_k, None if es is None else _ptr(es), N, K,
                                      _ptr(Y), _ptr(A), N, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_qmv_id_swiglu failed ({rc})")
    return Y, A


def moe_wsum(Y: np.ndarray, w: np.ndarray, top_k: int, YA: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """out[t, n] = sum_s w[t*top_k + s] * Y[t*top_k + s, n] in slot order (fp64).

    Y fp64 [n_tokens*top_k, N]; w fp32 [n_tokens*top_k]. Returns (out, A) fp64
    [n_tokens, N]; A = sum_s |w| * YA when YA is given, else sum_s |w * Y|."""
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    P, N = Y.shape
    if P % top_k or w.size != P:
        raise ValueError("Y rows and w must hold n_tokens*top_k entries")
    T = P // top_k
    YA = None if YA is None else np.ascontiguousarray(YA, dtype=np.float64)
    out = np.empty((T, N), dtype=np.float64)
    A = np.empty((T, N), dtype=np.float64)
    rc = _load().oracle_moe_wsum(_ptr(Y), None if YA is None else _ptr(YA), N, _ptr(w), T, top_k, N,
                                 _ptr(out), _ptr(A), N)
    if rc != 0:
        raise ValueError(f"oracle_moe_wsum failed ({rc})")
    return out, A


def moe_down(qtype, W: np.ndarray, G: np.ndarray, ids: np.ndarray, w: np.ndarray, N: int, K: int,
             expert_scale: Optional[np.ndarray] = None, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The MoE down half of one layer: SwiGLU of each slot's gate_up row, the
    expert-indexed down product, then the routing-weighted sum over slots.

    G fp32 [n_tokens*top_k, >= 2K] (row t*top_k + s is slot s of token t);
    ids uint32 [n_tokens, top_k]; w fp32 [n_tokens, top_k]. Returns (out, A)
    fp64 [n_tokens, N]."""
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    if ids.ndim == 1:
        ids = ids[None, :]
    top_k = ids.shape[1]
    Y, YA = qmv_id_swiglu(qtype, W, G, ids.reshape(-1, 1), N, K, expert_scale=expert_scale, nthreads=nthreads)
    return moe_wsum(Y, np.asarray(w, dtype=np.float32).reshape(-1), top_k, YA=YA)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def dequant_affine4_row(wq: np.ndarray, scales: np.ndarray, biases: np.ndarray, K: int) -> np.ndarray:
    """Affine 4-bit row: uint32 words (code j at bits 4j), bf16 bit patterns of
    the group-of-32 scales and biases. Returns fp64 [K]."""
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    sc = np.ascontiguousarray(scales, dtype=np.uint16)
    bi = np.ascontiguousarray(biases, dtype=np.uint16)
    if wq.size < K // 8 or sc.size < K // 32 or bi.size < K // 32:
        raise ValueError("row too short")
    out = np.empty(K, dtype=np.float64)
    if _load().oracle_dequant_affine4_row(_ptr(wq), _ptr(sc), _ptr(bi), K, _ptr(out)) != 0:
        raise ValueError("bad arguments")
    return out


def qmv_affine4(Wq: np.ndarray, S: np.ndarray, B: np.ndarray, X: np.ndarray, nthreads: int = 0):
    """Y, A for affine 4-bit rows: Wq uint32 [N, >= K/8], S, B uint16 (bf16) [N, >= K/32],
    X fp32 [M, K]. Returns fp64 [M, N] each."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
    S = np.ascontiguousarray(S, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X[None, :]
    M, K = X.shape
    N = Wq.shape[0]
    if S.shape != B.shape or S.shape[0] != N:
        raise ValueError("scales and biases must be [N, groups]")
    Y = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_qmv_affine4(_ptr(Wq), Wq.shape[1], _ptr(S), _ptr(B), S.shape[1], _ptr(X), K, M, N, K,
                                    _ptr(Y), _ptr(A), N, nthreads)
    if rc != 0:
        raise ValueError(f"oracle_qmv_affine4 failed ({rc})")
    return Y, A


def max_threads() -> int:
    return _load().oracle_max_threads()
