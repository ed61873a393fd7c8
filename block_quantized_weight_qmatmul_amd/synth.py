"""Seeded synthetic inputs for block-quantized mat-vec workloads.

This module only *draws* inputs: raw block bytes, activations, router ids and
per-expert scales. It contains none of the arithmetic of the dequantize-and-
multiply itself (no decoding of codes, no dot products), so that the CPU
oracle and the HIP path can both be fed from it without sharing any of the
computation they are compared on.

Block byte formats the generator writes (GGML-style, 32 weights per block):

* Q4_0, 18 bytes: a little-endian IEEE binary16 scale ``d`` in bytes [0, 2),
  then 16 bytes of packed 4-bit codes. Codes are drawn i.i.d. uniform over
  0..15 for every one of the 32 elements. Because every nibble is an
  independent uniform draw, this is the same as drawing each of the 16 code
  bytes uniformly over 0..255, which is what the generator does: it never
  needs to know which nibble holds which element.
* Q8_0, 34 bytes: the same binary16 scale, then 32 two's-complement int8
  codes drawn uniformly over -127..127 (the encoder on the hf2q model page,
  ``load_from_gguf`` lm_head Q8_0 block, never emits -128).

Scales are drawn as fp32 uniforms and rounded to binary16 with numpy's
round-to-nearest-even cast.

Seeds: ``numpy.random.default_rng([20261202, cfg, copy, tensor, part])``
with tensor ids 0 = scales, 1 = codes, 2 = activations, 3 = router logits,
4 = per-expert scale, 5 = gate_up rows, 6 = routing weights; ``part`` tells
apart several matrices of one config.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

ROOT_SEED = 20261202

T_SCALE, T_CODES, T_X, T_LOGITS, T_ESCALE, T_GATE_UP, T_RWEIGHT = 0, 1, 2, 3, 4, 5, 6

QK = 32  # weights per block
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "q5_k": 176, "q6_k": 210}
BLOCK_ELEMS = {"q4_0": 32, "q8_0": 32, "q5_k": 256, "q6_k": 256}
QTYPE_ID = {"q4_0": 2, "q8_0": 8, "q5_k": 13, "q6_k": 14}  # GGML type numbers

# Scale ranges and code ranges the workloads draw from.
Q4_0_D_RANGE = (0.001, 0.02)
Q8_0_D_RANGE = (0.0005, 0.01)


def rng(cfg: int, copy: int, tensor: int, part: int = 0) -> np.random.Generator:
    return np.random.default_rng([ROOT_SEED, cfg, copy, tensor, part])


def row_bytes(qtype: str, K: int) -> int:
    qk = BLOCK_ELEMS[qtype]
    if K % qk:
        raise ValueError(f"K={K} is not a multiple of {qk}")
    return K // qk * BLOCK_BYTES[qtype]


def _scales_f16_bytes(r: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    d32 = r.uniform(lo, hi, size=shape).astype(np.float32)
    d16 = d32.astype(np.float16)  # round-to-nearest-even
    return d16.astype("<f2").view(np.uint8).reshape(*shape, 2)


def make_weights(qtype: str, N: int, K: int, cfg: int, copy: int = 0, part: int = 0,
                 d_range: Tuple[float, float] | None = None, ldw: int | None = None) -> np.ndarray:
    """Return a uint8 array ``[N, ldw]`` of N rows, each K/32 blocks of ``qtype``.

    Bytes past the dense row length (when ``ldw`` exceeds it) are filled with
    0xA5 so that a reader that strays into the row padding gets garbage.
    """
    if qtype == "q6_k":
        return _make_q6_k(N, K, cfg, copy, part, d_range, ldw)
    if qtype == "q5_k":
        return _make_q5_k(N, K, cfg, copy, part, ldw)
    bb = BLOCK_BYTES[qtype]
    nb = K // QK
    dense = row_bytes(qtype, K)
    ldw = dense if ldw is None else ldw
    if ldw < dense:
        raise ValueError("ldw smaller than a dense row")
    if d_range is None:
        d_range = Q4_0_D_RANGE if qtype == "q4_0" else Q8_0_D_RANGE
    blocks = np.empty((N, nb, bb), dtype=np.uint8)
    blocks[..., 0:2] = _scales_f16_bytes(rng(cfg, copy, T_SCALE, part), (N, nb), *d_range)
    rc = rng(cfg, copy, T_CODES, part)
    if qtype == "q4_0":
        blocks[..., 2:] = rc.integers(0, 256, size=(N, nb, bb - 2), dtype=np.uint8)
    else:
        blocks[..., 2:] = rc.integers(-127, 128, size=(N, nb, bb - 2)).astype(np.int8).view(np.uint8)
    if ldw == dense:
        return blocks.reshape(N, dense)
    out = np.full((N, ldw), 0xA5, dtype=np.uint8)
    out[:, :dense] = blocks.reshape(N, dense)
    return out


Q6_K_D_RANGE = (1e-5, 5e-5)


def _make_q6_k(N, K, cfg, copy, part, d_range, ldw):
    """Q6_K rows: per 256-weight super-block, 192 bytes of code bits drawn
    uniformly (so every 6-bit code is uniform over 0..63), 16 int8 sub-block
    scales uniform over -128..127, and a binary16 scale d ~ U(d_range)
    (default 1e-5..5e-5, mostly binary16 subnormals, as small super-block
    scales are). Padding bytes past the dense row are 0xA5."""
    nb = K // 256
    dense = nb * 210
    ldw = dense if ldw is None else ldw
    if ldw < dense:
        raise ValueError("ldw smaller than a dense row")
    d_range = Q6_K_D_RANGE if d_range is None else d_range
    blocks = np.empty((N, nb, 210), dtype=np.uint8)
    rc = rng(cfg, copy, T_CODES, part)
    blocks[..., 0:192] = rc.integers(0, 256, size=(N, nb, 192), dtype=np.uint8)
    blocks[..., 192:208] = rc.integers(-128, 128, size=(N, nb, 16)).astype(np.int8).view(np.uint8)
    blocks[..., 208:210] = _scales_f16_bytes(rng(cfg, copy, T_SCALE, part), (N, nb), *d_range)
    if ldw == dense:
        return blocks.reshape(N, dense)
    out = np.full((N, ldw), 0xA5, dtype=np.uint8)
    out[:, :dense] = blocks.reshape(N, dense)
    return out


Q5_K_D_RANGE = (2e-5, 8e-5)
Q5_K_DMIN_RANGE = (2e-4, 1e-3)


def _make_q5_k(N, K, cfg, copy, part, ldw):
    """Q5_K rows: per 256-weight super-block, binary16 d ~ U[2e-5, 8e-5] and
    dmin ~ U[2e-4, 1e-3], and the 172 other bytes (packed 6-bit scales and
    minimums, code bits) drawn uniformly, so every 6-bit scale and minimum and
    every 5-bit code is uniform. Padding bytes past the dense row are 0xA5."""
    nb = K // 256
    dense = nb * 176
    ldw = dense if ldw is None else ldw
    if ldw < dense:
        raise ValueError("ldw smaller than a dense row")
    blocks = np.empty((N, nb, 176), dtype=np.uint8)
    rs = rng(cfg, copy, T_SCALE, part)
    blocks[..., 0:2] = _scales_f16_bytes(rs, (N, nb), *Q5_K_D_RANGE)
    blocks[..., 2:4] = _scales_f16_bytes(rs, (N, nb), *Q5_K_DMIN_RANGE)
    blocks[..., 4:] = rng(cfg, copy, T_CODES, part).integers(0, 256, size=(N, nb, 172), dtype=np.uint8)
    if ldw == dense:
        return blocks.reshape(N, dense)
    out = np.full((N, ldw), 0xA5, dtype=np.uint8)
    out[:, :dense] = blocks.reshape(N, dense)
    return out


def _bf16_rne(values) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even."""
    u = np.asarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def make_affine4(N: int, K: int, cfg: int, copy: int = 0, part: int = 0):
    """MLX affine 4-bit rows with groups of 32: (Wq uint32 [N, K/8], scales
    and biases as bf16 bit patterns uint16 [N, K/32]). Codes uniform over
    0..15 (uniform words), scales ~ U[0.002, 0.02] and biases ~ U[-0.16,
    -0.016] as fp32 rounded to bf16 (nearest even), so weights scale*q + bias
    straddle zero as affine-quantized weights do."""
    if K % 32:
        raise ValueError(f"K={K} is not a multiple of 32")
    wq = rng(cfg, copy, T_CODES, part).integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    r = rng(cfg, copy, T_SCALE, part)
    sc = _bf16_rne(r.uniform(0.002, 0.02, size=(N, K // 32)))
    bi = _bf16_rne(r.uniform(-0.16, -0.016, size=(N, K // 32)))
    return wq, sc, bi


def make_x(M: int, K: int, cfg: int, copy: int = 0, part: int = 0) -> np.ndarray:
    """Activations ``[M, K]`` fp32 drawn from N(0, 1)."""
    return rng(cfg, copy, T_X, part).standard_normal((M, K), dtype=np.float64).astype(np.float32)


def router_topk(T: int, n_experts: int, top_k: int, cfg: int, copy: int = 0, part: int = 0) -> np.ndarray:
    """Expert ids ``[T, top_k]`` uint32: the top_k largest of N(0,1) router logits.

    Ids come in descending logit order; equal logits go to the lower index
    (a stable argsort of the negated logits).
    """
    logits = rng(cfg, copy, T_LOGITS, part).standard_normal((T, n_experts)).astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :top_k].astype(np.uint32)


def expert_scale(n_experts: int, cfg: int, copy: int = 0, part: int = 0) -> np.ndarray:
    """Per-expert fp32 scale drawn from U[0.5, 1.5]."""
    return rng(cfg, copy, T_ESCALE, part).uniform(0.5, 1.5, size=n_experts).astype(np.float32)


# Standard deviation of one gate_up output for N(0,1) activations over
# K = 2816 inputs, Q4_0 codes uniform over 0..15 and d ~ U[0.001, 0.02]:
# E[(c - 8)^2] = 344/16 = 21.5, E[d^2] = (0.02^3 - 0.001^3) / (3 * 0.019)
# = 1.403e-4, so sqrt(2816 * 21.5 * 1.403e-4) = 2.91.
GATE_UP_STD = 2.9


def gate_up_rows(rows: int, inter: int, cfg: int, copy: int = 0, part: int = 0,
                 std: float = GATE_UP_STD) -> np.ndarray:
    """Stand-in gate_up outputs ``[rows, 2 * inter]`` fp32 drawn from N(0, std^2).

    Row p holds the gate half then the up half of one (token, slot) pair.
    """
    r = rng(cfg, copy, T_GATE_UP, part)
    return (r.standard_normal((rows, 2 * inter), dtype=np.float64) * std).astype(np.float32)


def routing_weights(T: int, top_k: int, cfg: int, copy: int = 0, part: int = 0) -> np.ndarray:
    """Routing weights ``[T, top_k]`` fp32: U[0, 1) draws divided by their
    per-token sum (positive, summing to 1 over a token's slots)."""
    u = rng(cfg, copy, T_RWEIGHT, part).random((T, top_k)) + 1e-3
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads. Each is a list of problems; a dense problem is
# (name, qtype, M, N, K) and the MoE workload lists its two id calls.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Dense:
    name: str
    qtype: str
    M: int
    N: int
    K: int

    @property
    def weight_bytes(self) -> int:
        return self.N * row_bytes(self.qtype, self.K)


@dataclasses.dataclass(frozen=True)
class MoeId:
    name: str
    qtype: str
    n_experts: int
    n_tokens: int   # rows of X handed to the call
    top_k: int      # experts per X row
    N: int
    K: int


CONFIGS: Dict[int, dict] = {
    0: {"name": "q4_0_m1_2048x2048",
        "problems": [Dense("proj", "q4_0", 1, 2048, 2048)]},
    1: {"name": "q4_0_m1_decode_layer_h4096",
        "problems": [Dense("q", "q4_0", 1, 4096, 4096), Dense("k", "q4_0", 1, 1024, 4096),
                     Dense("v", "q4_0", 1, 1024, 4096), Dense("o", "q4_0", 1, 4096, 4096),
                     Dense("gate", "q4_0", 1, 14336, 4096), Dense("up", "q4_0", 1, 14336, 4096),
                     Dense("down", "q4_0", 1, 4096, 14336)]},
    2: {"name": "q8_0_m1_4096x14336",
        "problems": [Dense("up", "q8_0", 1, 14336, 4096), Dense("down", "q8_0", 1, 4096, 14336)]},
    3: {"name": "q4_0_m16_k5120",
        "problems": [Dense("n5120", "q4_0", 16, 5120, 5120), Dense("n1024", "q4_0", 16, 1024, 5120),
                     Dense("n27648", "q4_0", 16, 27648, 5120)]},
    4: {"name": "q4_0_moe_id_e128_top8_h2816_i704"},
}

MOE = dict(n_experts=128, top_k=8, hidden=2816, inter=704)


def moe_calls(T: int) -> List[MoeId]:
    """The two id calls of one MoE FFN for T tokens.

    gate_up: X is [T, hidden], ids [T, top_k], output rows T*top_k of 2*inter.
    down: the slots are flattened (n_tokens = T*top_k, top_k = 1); X is the
    [T*top_k, inter] per-slot input and the output is [T*top_k, hidden].
    """
    E, k, h, i = MOE["n_experts"], MOE["top_k"], MOE["hidden"], MOE["inter"]
    return [MoeId("gate_up", "q4_0", E, T, k, 2 * i, h),
            MoeId("down", "q4_0", E, T * k, 1, h, i)]


def distinct(ids: np.ndarray) -> int:
    return int(np.unique(ids).size)


def dense_inputs(cfg: int, p: Dense, part: int, copy: int = 0, ldw: int | None = None):
    """(W bytes [N, ldw], X [M, K]) for one dense problem of a config."""
    W = make_weights(p.qtype, p.N, p.K, cfg, copy, part, ldw=ldw)
    X = make_x(p.M, p.K, cfg, copy, part)
    return W, X


def moe_inputs(T: int, copy: int = 0, cfg: int = 4):
    """All inputs of the MoE workload for T tokens.

    Returns a dict with the stacked gate_up and down weights (uint8
    [E, N, row_bytes]), the gate_up input X [T, hidden], the down input
    [T*top_k, inter], ids [T, top_k], the per-expert scale [E], stand-in
    gate_up output rows G_down [T*top_k, 2*inter] for the SwiGLU-fed down
    calls and the routing weights [T, top_k].
    """
    gu, dn = moe_calls(T)
    E = MOE["n_experts"]
    return {
        "W_gate_up": make_weights("q4_0", E * gu.N, gu.K, cfg, copy, part=0).reshape(E, gu.N, -1),
        "W_down": make_weights("q4_0", E * dn.N, dn.K, cfg, copy, part=1).reshape(E, dn.N, -1),
        "X_gate_up": make_x(T, gu.K, cfg, copy, part=0),
        "X_down": make_x(T * MOE["top_k"], dn.K, cfg, copy, part=1),
        "ids": router_topk(T, E, MOE["top_k"], cfg, copy),
        "expert_scale": expert_scale(E, cfg, copy),
        "G_down": gate_up_rows(T * MOE["top_k"], dn.K, cfg, copy),
        "weights": routing_weights(T, MOE["top_k"], cfg, copy),
    }
