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

Q4_0, Q8_0 = 2, 8
QTYPES = {"q4_0": Q4_0, "q8_0": Q8_0}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}

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
    if row.size < K // 32 * BLOCK_BYTES[q]:
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


def max_threads() -> int:
    return _load().oracle_max_threads()
