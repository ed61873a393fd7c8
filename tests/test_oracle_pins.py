"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test ties one part of the oracle to something that does not come from the
oracle: hand-built blocks with hand-derived values (tests/golden/), the Q8_0
encoder printed on the hf2q model page, IEEE binary16 as numpy implements it,
closed forms, exact rational arithmetic on tiny inputs, and the expert-routing
signature. A plausible mistake in the oracle (swapped nibbles, a dropped -8,
a wrong byte order for the scale, a transposed operand, a wrong x or y row in
the expert-indexed call) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import read_blocks

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# binary16 scale decode: every bit pattern against numpy's IEEE binary16.
# --------------------------------------------------------------------------
def test_f16_decode_matches_ieee_binary16_for_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


# --------------------------------------------------------------------------
# Hand-built blocks (tests/golden/).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fixture,qtype", [("q4_0_blocks.txt", "q4_0"), ("q8_0_blocks.txt", "q8_0")])
def test_golden_blocks_dequantize_to_hand_derived_values(fixture, qtype):
    blocks = read_blocks(fixture)
    assert len(blocks) >= 4
    for label, raw, want in blocks:
        got = oracle.dequant_row(qtype, raw, 32)
        assert np.array_equal(got, want), (label, got, want)


@pytest.mark.parametrize("fixture,qtype", [("q4_0_blocks.txt", "q4_0"), ("q8_0_blocks.txt", "q8_0")])
def test_one_hot_x_picks_one_weight_exactly(fixture, qtype):
    """x = e_k gives y[n] = w[n, k]: one exact product, every other term is 0."""
    blocks = read_blocks(fixture)
    W = np.stack([raw for _, raw, _ in blocks])
    want = np.stack([v for _, _, v in blocks])
    for k in range(32):
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, k] = 1.0
        y, a = oracle.qmv(qtype, W, x)
        assert np.array_equal(y[0], want[:, k])
        assert np.array_equal(a[0], np.abs(want[:, k]))


def test_rows_of_x_map_to_rows_of_y():
    """X[m, k0 + m] = 1 for m < M gives Y[m, n] = w[n, k0 + m]."""
    blocks = read_blocks("q4_0_blocks.txt")
    W = np.stack([raw for _, raw, _ in blocks])
    want = np.stack([v for _, _, v in blocks])
    M, k0 = 16, 9
    X = np.zeros((M, 32), dtype=np.float32)
    for m in range(M):
        X[m, k0 + m] = 1.0
    Y, _ = oracle.qmv("q4_0", W, X)
    for m in range(M):
        assert np.array_equal(Y[m], want[:, k0 + m])


# --------------------------------------------------------------------------
# Q8_0: the encoder printed on the hf2q model page (`load_from_gguf`, the
# lm_head Q8_0 block), restated here, then decoded by the oracle.
# --------------------------------------------------------------------------
def page_q8_0_encode(block):
    """amax over the block; d = amax/127 (fp32); inv_d = 1/d; scale stored as
    binary16 bits low byte first; each code = round-half-away(v * inv_d)
    clamped to [-127, 127] and stored as an int8 byte."""
    v = np.asarray(block, dtype=np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    d = np.float32(amax / np.float32(127.0)) if amax > 0 else np.float32(0.0)
    inv_d = np.float32(np.float32(1.0) / d) if d != 0 else np.float32(0.0)
    bits = int(np.array(d, dtype=np.float32).astype(np.float16).view(np.uint16))
    out = [bits & 0xFF, bits >> 8]
    for vi in v:
        t = float(np.float32(vi * inv_d))
        q = math.copysign(math.floor(abs(t) + 0.5), t)
        q = int(max(-127.0, min(127.0, q)))
        out.append(q & 0xFF)
    return np.array(out, dtype=np.uint8), d


def test_q8_0_page_encoder_bytes_for_a_worked_block():
    # v_j = j - 16: amax = 16, d = 16/127 -> binary16 0x3008 (= 0.1259765625),
    # inv_d = 127/16 = 7.9375; code of -16 is -127, of 15 is round(119.0625) = 119.
    raw, d = page_q8_0_encode(np.arange(32, dtype=np.float32) - 16)
    assert raw[0] == 0x08 and raw[1] == 0x30
    assert raw[2] == 0x81  # -127
    assert raw[2 + 31] == 119
    assert raw[2 + 17] == 8 and raw[2 + 15] == 0xF8  # v = 1 -> 8, v = -1 -> -8
    got = oracle.dequant_row("q8_0", raw, 32)
    assert got[0] == -127 * 0.1259765625 and got[31] == 119 * 0.1259765625


def test_q8_0_page_encoder_round_trip_bound():
    r = np.random.default_rng(7)
    cases = [r.standard_normal(32) * s for s in (1e-3, 1.0, 50.0)]
    cases += [np.zeros(32), np.r_[np.zeros(31), 3.0], r.uniform(-1, 1, 32) * 1e-6]
    for v in cases:
        v = v.astype(np.float32)
        raw, d = page_q8_0_encode(v)
        d16 = float(np.float32(d).astype(np.float16))
        got = oracle.dequant_row("q8_0", raw, 32)
        bound = 127 * abs(d16 - float(d)) + float(d) * (0.5 + 1e-4)
        assert np.all(np.abs(got - v.astype(np.float64)) <= bound + 1e-300)


def test_q8_0_lm_head_size_closed_form():
    # The page sizes a Q8_0 lm_head of vocab 262144 x hidden 2816 at "784 MB"
    # (vs 1.47 GB in F16): 34 bytes per 32 weights.
    vocab, hidden = 262144, 2816
    q8 = vocab * hidden // 32 * oracle.BLOCK_BYTES[oracle.Q8_0]
    assert round(q8 / 1e6) == 784
    assert math.floor(vocab * hidden * 2 / 1e7) / 100 == 1.47  # the F16 size the page quotes
    assert oracle.BLOCK_BYTES[oracle.Q4_0] == 2 + 32 // 2


# --------------------------------------------------------------------------
# Closed forms and invariants of the dense product.
# --------------------------------------------------------------------------
def _const_blocks(qtype, N, K, code_byte, d_bits):
    bb = oracle.BLOCK_BYTES[oracle.QTYPES[qtype]]
    blk = np.full(bb, code_byte, dtype=np.uint8)
    blk[0], blk[1] = d_bits & 0xFF, d_bits >> 8
    return np.tile(blk, (N, K // 32))


@pytest.mark.parametrize("code", range(16))
def test_q4_0_constant_code_ones_closed_form(code):
    K, N = 4096, 3
    W = _const_blocks("q4_0", N, K, code | (code << 4), 0x3800)  # d = 0.5
    y, a = oracle.qmv("q4_0", W, np.ones((1, K), dtype=np.float32))
    assert np.all(y == K * (code - 8) * 0.5)
    assert np.all(a == K * abs(code - 8) * 0.5)


def test_q8_0_constant_code_ones_closed_form():
    K, N = 14336, 2
    for q in (-128, -127, -1, 0, 1, 127):
        W = _const_blocks("q8_0", N, K, q & 0xFF, 0x3400)  # d = 0.25
        y, a = oracle.qmv("q8_0", W, np.ones((1, K), dtype=np.float32))
        assert np.all(y == K * q * 0.25) and np.all(a == K * abs(q) * 0.25)


def test_q4_0_all_codes_eight_give_exact_zero():
    from block_quantized_weight_qmatmul_amd import synth
    W = synth.make_weights("q4_0", 5, 2048, cfg=99)
    W.reshape(5, -1, 18)[:, :, 2:] = 0x88
    y, a = oracle.qmv("q4_0", W, synth.make_x(2, 2048, cfg=99))
    assert np.all(y == 0) and np.all(a == 0)


def test_power_of_two_scaling_is_exact():
    from block_quantized_weight_qmatmul_amd import synth
    W = synth.make_weights("q4_0", 16, 1024, cfg=98)
    X = synth.make_x(3, 1024, cfg=98)
    y, _ = oracle.qmv("q4_0", W, X)
    y8, _ = oracle.qmv("q4_0", W, X * np.float32(8.0))
    assert np.array_equal(y8, 8.0 * y)


# --------------------------------------------------------------------------
# Brute force on tiny inputs in exact rational arithmetic.
# --------------------------------------------------------------------------
def _enc_q4_0(codes, d_bits):
    """Lay 32 codes out as the Q4_0 reading says: byte 2+j = code[j] | code[j+16] << 4."""
    return bytes([d_bits & 0xFF, d_bits >> 8] + [codes[j] | (codes[j + 16] << 4) for j in range(16)])


def _enc_q8_0(codes, d_bits):
    return bytes([d_bits & 0xFF, d_bits >> 8] + [c & 0xFF for c in codes])


def _f16_fraction(bits):
    return Fraction(float(np.array(bits, dtype=np.uint16).view(np.float16)))


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_brute_force_tiny_shapes_against_exact_rationals(qtype):
    r = np.random.default_rng(11)
    d_pool = [0x3C00, 0x3800, 0xC000, 0x0001, 0x03FF, 0x1234, 0x5A5A, 0xB555, 0x7BFF]
    for K in (32, 64):
        N, M = 16, 3
        nb = K // 32
        rows, dense = [], []
        for n in range(N):
            raw, vals = b"", []
            for b in range(nb):
                if qtype == "q4_0":
                    codes = [(n + 3 * b + j) % 16 for j in range(32)]  # every code at every position
                    ints = [c - 8 for c in codes]
                    enc = _enc_q4_0
                else:
                    codes = [int(c) for c in r.integers(-128, 128, 32)]
                    ints = codes
                    enc = _enc_q8_0
                d_bits = d_pool[(n + b) % len(d_pool)]
                raw += enc(codes, d_bits)
                d = _f16_fraction(d_bits)
                vals += [Fraction(i) * d for i in ints]
            rows.append(np.frombuffer(raw, dtype=np.uint8))
            dense.append(vals)
        W = np.stack(rows)
        X = r.standard_normal((M, K)).astype(np.float32)
        Y, A = oracle.qmv(qtype, W, X)
        for m in range(M):
            for n in range(N):
                prods = [dense[n][k] * Fraction(float(X[m, k])) for k in range(K)]
                exact = sum(prods)
                mag = sum(abs(p) for p in prods)
                bound = K * 2.0 ** -53 * float(mag)
                assert abs(Fraction(Y[m, n]) - exact) <= Fraction(bound), (K, m, n)
                assert abs(Fraction(A[m, n]) - mag) <= Fraction(bound)


def test_long_row_sum_within_fp64_bound_of_exactly_rounded_sum():
    """K = 14336: the oracle's fp64 sum is within K * 2^-53 * a of math.fsum of
    the exact products (each product of a binary16-scaled small integer and an
    fp32 value is exact in fp64)."""
    from block_quantized_weight_qmatmul_amd import synth
    K = 14336
    W = synth.make_weights("q4_0", 4, K, cfg=97)
    X = synth.make_x(1, K, cfg=97)
    Y, A = oracle.qmv("q4_0", W, X)
    for n in range(4):
        blk = W[n].reshape(-1, 18)
        d = blk[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
        lo = (blk[:, 2:] & 0x0F).astype(np.int64) - 8
        hi = (blk[:, 2:] >> 4).astype(np.int64) - 8
        w = (np.concatenate([lo, hi], axis=1) * d[:, None]).ravel()
        prods = w * X[0].astype(np.float64)
        exact = math.fsum(prods)
        assert abs(Y[0, n] - exact) <= K * 2.0 ** -53 * A[0, n]


# --------------------------------------------------------------------------
# Expert-indexed call.
# --------------------------------------------------------------------------
def _signature_stack(qtype, E, N, K):
    """Expert e: every scale is binary16(e + 1), every weight value is 1 * d."""
    bb = oracle.BLOCK_BYTES[oracle.QTYPES[qtype]]
    W = np.empty((E, N, K // 32, bb), dtype=np.uint8)
    for e in range(E):
        bits = int(np.array(e + 1, dtype=np.float16).view(np.uint16))
        W[e, :, :, 0], W[e, :, :, 1] = bits & 0xFF, bits >> 8
        W[e, :, :, 2:] = 0x99 if qtype == "q4_0" else 0x01
    return W.reshape(E, N, -1)


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_id_routing_signature_closed_form(qtype):
    E, N, K = 128, 8, 2816
    W = _signature_stack(qtype, E, N, K)
    ids = np.array([[127, 0, 5, 5], [64, 3, 127, 1], [0, 0, 0, 0]], dtype=np.uint32)  # repeats, duplicates
    X = np.ones((3, K), dtype=np.float32)
    Y, A = oracle.qmv_id(qtype, W, X, ids, N, K)
    for p, e in enumerate(ids.ravel()):
        assert np.all(Y[p] == (int(e) + 1) * K) and np.all(A[p] == (int(e) + 1) * K)
    sc = np.linspace(0.5, 1.5, E).astype(np.float32)
    Ys, _ = oracle.qmv_id(qtype, W, X, ids, N, K, expert_scale=sc)
    for p, e in enumerate(ids.ravel()):
        assert np.all(Ys[p] == float(sc[e]) * (int(e) + 1) * K)


def test_id_input_row_is_token_and_output_row_is_token_times_topk_plus_slot():
    E, N, K = 6, 4, 64
    W = _signature_stack("q4_0", E, N, K)
    ids = np.array([[1, 4], [2, 2], [5, 0]], dtype=np.uint32)
    X = np.stack([np.full(K, t + 1, dtype=np.float32) for t in range(3)])
    Y, _ = oracle.qmv_id("q4_0", W, X, ids, N, K)
    for t in range(3):
        for s in range(2):
            assert np.all(Y[t * 2 + s] == (t + 1) * (int(ids[t, s]) + 1) * K)


def test_id_flattened_down_call_matches_per_slot_dense_calls():
    """The down-projection form (n_tokens = T*top_k, top_k = 1) on expert e's
    slice equals a dense call on that slice (the dense call is pinned above)."""
    from block_quantized_weight_qmatmul_amd import synth
    E, N, K, P = 5, 24, 704, 7
    W = synth.make_weights("q4_0", E * N, K, cfg=96).reshape(E, N, -1)
    X = synth.make_x(P, K, cfg=96)
    ids = np.array([4, 0, 2, 2, 1, 4, 3], dtype=np.uint32)
    Y, _ = oracle.qmv_id("q4_0", W, X, ids[:, None], N, K)
    for p in range(P):
        yd, _ = oracle.qmv("q4_0", W[ids[p]], X[p:p + 1])
        assert np.array_equal(Y[p], yd[0])


def test_id_rejects_out_of_range_expert():
    W = _signature_stack("q4_0", 4, 2, 32)
    with pytest.raises(ValueError):
        oracle.qmv_id("q4_0", W, np.ones((1, 32), np.float32), np.array([[4]], np.uint32), 2, 32)


def test_dense_rejects_bad_shapes():
    W = np.zeros((2, 18), dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.qmv("q4_0", W, np.ones((1, 33), np.float32), K=33)
    with pytest.raises(ValueError):
        oracle.qmv("q4_0", W, np.ones((1, 64), np.float32))  # row shorter than K/32 blocks


# --------------------------------------------------------------------------
# MoE steps around the expert-indexed call: SwiGLU and the weighted sum.
# --------------------------------------------------------------------------
def _silu_tanh(z):
    """silu through the identity z * sigmoid(z) = (z / 2) * (1 + tanh(z / 2))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(0.5 * z))


def test_silu_closed_forms_limits_and_odd_part():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 0.5 * (1.0 + math.tanh(0.5))) <= 2.0 ** -52
    assert abs(oracle.silu(-1.0) - (-0.5) * (1.0 - math.tanh(0.5))) <= 2.0 ** -53
    # silu(z) = z * (1 - e^-z / (1 + e^-z)); at z = 40 the correction is
    # 4.2e-18, below half an ulp of 40, so the rounded value is 40 exactly.
    assert oracle.silu(40.0) == 40.0
    # e^800 overflows: the value is the limit, -0 (sign kept).
    v = oracle.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0
    assert math.isnan(oracle.silu(float("nan")))
    zs = np.linspace(-30.0, 30.0, 1201)
    for z in zs:
        s_pos, s_neg = oracle.silu(z), oracle.silu(-z)
        # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
        assert abs((s_pos - s_neg) - z) <= 4 * 2.0 ** -52 * max(1.0, abs(z))
        assert abs(s_pos - _silu_tanh(z)) <= 8 * 2.0 ** -52 * max(1.0, abs(z))


def test_swiglu_gate_is_the_first_half_of_each_row():
    G = np.array([[1.0, 2.0, 2.0, 1.0],
                  [0.0, 5.0, 7.0, -3.0],
                  [-2.0, 0.5, 0.0, 4.0]], dtype=np.float32)
    H = oracle.swiglu(G)
    want = np.array([[_silu_tanh(1.0) * 2.0, _silu_tanh(2.0) * 1.0],
                     [0.0, _silu_tanh(5.0) * -3.0],
                     [_silu_tanh(-2.0) * 0.0, _silu_tanh(0.5) * 4.0]])
    assert np.allclose(H, want, rtol=1e-15, atol=0)
    # swapped halves would give silu(2) * 1 = 1.7616 in place of silu(1) * 2 = 1.4621
    assert abs(H[0, 0] - 1.4621171572600098) < 1e-15
    assert H[1, 0] == 0.0 and H[2, 0] == 0.0


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_id_swiglu_with_saturated_gates_equals_id_on_scaled_up_rows(qtype):
    """Gate 40 gives silu = 40 exactly and gate -800 gives -0, so the SwiGLU
    rows are 40 * up (or 0) exactly; the product must then equal the pinned
    expert-indexed call on those rows bit for bit."""
    from block_quantized_weight_qmatmul_amd import synth
    E, N, K, T, k = 6, 12, 128, 3, 2
    W = synth.make_weights(qtype, E * N, K, cfg=95).reshape(E, N, -1)
    r = np.random.default_rng(95)
    up = r.integers(-100, 101, (T, K)).astype(np.float32)
    mask = r.random((T, K)) < 0.6
    gate = np.where(mask, 40.0, -800.0).astype(np.float32)
    G = np.concatenate([gate, up], axis=1)
    ids = np.array([[5, 1], [2, 2], [0, 4]], dtype=np.uint32)
    sc = np.array([0.5, 1.25, 2.0, 1.0, 0.75, 1.5], dtype=np.float32)
    Y, A = oracle.qmv_id_swiglu(qtype, W, G, ids, N, K, expert_scale=sc)
    X = np.where(mask, 40.0 * up, 0.0).astype(np.float32)
    Yr, Ar = oracle.qmv_id(qtype, W, X, ids, N, K, expert_scale=sc)
    assert np.array_equal(Y, Yr) and np.array_equal(A, Ar)


def test_weighted_sum_hand_derived_values():
    # two tokens, three slots, two columns; row p of Y is [2p + 1, 2p + 2]
    Y = np.arange(1, 13, dtype=np.float64).reshape(6, 2)
    w = np.array([0.5, 0.25, 2.0, 1.0, -1.0, 0.125], dtype=np.float32)
    out, A = oracle.moe_wsum(Y, w, 3)
    # token 0: 0.5*[1,2] + 0.25*[3,4] + 2*[5,6]; token 1: [7,8] - [9,10] + [11,12]/8
    assert np.array_equal(out, [[11.25, 14.0], [-0.625, -0.5]])
    assert np.array_equal(A, [[11.25, 14.0], [17.375, 19.5]])
    out1, _ = oracle.moe_wsum(Y, np.array([0, 1, 0, 0, 0, 1], np.float32), 3)
    assert np.array_equal(out1, [[3.0, 4.0], [11.0, 12.0]])


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_moe_down_composition_against_numpy_brute_force(qtype):
    """SwiGLU -> expert-indexed down -> weighted sum, against a numpy fp64
    evaluation that decodes the blocks itself and takes silu through tanh."""
    from block_quantized_weight_qmatmul_amd import synth
    E, N, K, T, k = 7, 10, 96, 3, 3
    W = synth.make_weights(qtype, E * N, K, cfg=94).reshape(E, N, -1)
    r = np.random.default_rng(94)
    G = (r.standard_normal((T * k, 2 * K)) * 2).astype(np.float32)
    ids = np.array([[6, 0, 3], [3, 3, 1], [2, 5, 4]], dtype=np.uint32)
    w = r.random((T, k)).astype(np.float32)
    sc = r.uniform(0.5, 1.5, E).astype(np.float32)
    out, A = oracle.moe_down(qtype, W, G, ids, w, N, K, expert_scale=sc)

    bb = oracle.BLOCK_BYTES[oracle.QTYPES[qtype]]

    def deq(mat):
        blk = mat.reshape(N, K // 32, bb)
        d = blk[:, :, 0:2].copy().view("<f2").astype(np.float64)[:, :, 0]
        if qtype == "q4_0":
            lo = (blk[:, :, 2:] & 0x0F).astype(np.int64) - 8
            hi = (blk[:, :, 2:] >> 4).astype(np.int64) - 8
            c = np.concatenate([lo, hi], axis=2)
        else:
            c = blk[:, :, 2:].view(np.int8).astype(np.int64)
        return (c * d[:, :, None]).reshape(N, K)

    for t in range(T):
        want = np.zeros(N)
        mag = np.zeros(N)
        for s in range(k):
            g = G[t * k + s].astype(np.float64)
            h = _silu_tanh(g[:K]) * g[K:]
            e = int(ids[t, s])
            prod = deq(W[e]) * h[None, :]
            want += float(w[t, s]) * float(sc[e]) * prod.sum(axis=1)
            mag += abs(float(w[t, s]) * float(sc[e])) * np.abs(prod).sum(axis=1)
        assert np.all(np.abs(out[t] - want) <= 1e-12 * mag + 1e-300), t
        assert np.allclose(A[t], mag, rtol=1e-12, atol=0)


# --------------------------------------------------------------------------
# Q6_K super-blocks (256 weights, 210 bytes).
# --------------------------------------------------------------------------
def _enc_q6_k(codes, scales, d_bits):
    """Lay out 256 six-bit codes, 16 int8 scales and a binary16 scale the way
    the GGML Q6_K super-block stores them, walking the storage bytes: ql byte
    64h + 32p + l holds code 128h + 32p + l in its low nibble and code
    128h + 32(p + 2) + l in its high nibble; qh byte 32h + l holds bits 4..5
    of codes 128h + 32g + l at bit 2g (g = 0..3)."""
    b = bytearray(210)
    for h in range(2):
        for p in range(2):
            for l in range(32):
                lo = codes[128 * h + 32 * p + l] & 15
                hi = codes[128 * h + 32 * (p + 2) + l] & 15
                b[64 * h + 32 * p + l] = lo | (hi << 4)
        for l in range(32):
            b[128 + 32 * h + l] = sum(((codes[128 * h + 32 * g + l] >> 4) & 3) << (2 * g) for g in range(4))
    b[192:208] = bytes(s & 0xFF for s in scales)
    b[208], b[209] = d_bits & 0xFF, d_bits >> 8
    return bytes(b)


def test_q6_k_lm_head_size_closed_form():
    # the pages: token_embd.weight as Q6_K [2816, 262144] is 605 MB
    from block_quantized_weight_qmatmul_amd import synth
    assert 262144 * (2816 // 256) * 210 == 605_552_640
    assert synth.row_bytes("q6_k", 2816) == 2310
    with pytest.raises(ValueError):
        oracle.dequant_row("q6_k", np.zeros(210, np.uint8), 128)  # K not a multiple of 256


def test_q6_k_hand_built_super_blocks():
    """Every code at every position, signed scales including -128, and
    normal, subnormal and negative super-block scales: weight i must be
    d * scale[i // 16] * (code_i - 32)."""
    r = np.random.default_rng(61)
    for trial, d_bits in enumerate([0x3C00, 0x3800, 0x0001, 0x03FF, 0xC400, 0x0000, 0x7BFF]):
        codes = [int(c) for c in r.permutation(np.repeat(np.arange(64), 4))]  # every code, 4 times
        scales = [int(v) for v in r.integers(-128, 128, 16)]
        scales[trial % 16] = -128
        raw = np.frombuffer(_enc_q6_k(codes, scales, d_bits), dtype=np.uint8)
        w = oracle.dequant_row("q6_k", raw, 256)
        d = float(np.array(d_bits, dtype=np.uint16).view(np.float16))
        want = np.array([d * scales[i // 16] * (codes[i] - 32) for i in range(256)])
        assert np.array_equal(w, want), trial


def test_q6_k_constant_codes_and_one_hot():
    raw = np.frombuffer(_enc_q6_k([33] * 256, [1] * 16, 0x3C00), dtype=np.uint8)
    W = np.tile(raw, (3, 2))  # 3 rows of K = 512
    x = np.random.default_rng(62).standard_normal((1, 512)).astype(np.float32)
    Y, A = oracle.qmv("q6_k", W, x)
    assert np.all(np.abs(Y[0] - math.fsum(x[0].astype(np.float64))) <= 512 * 2.0 ** -53 * A[0])
    from block_quantized_weight_qmatmul_amd import synth
    Wr = synth.make_weights("q6_k", 5, 512, cfg=62)
    for k in (0, 1, 127, 128, 255, 256, 300, 511):
        e = np.zeros((1, 512), np.float32)
        e[0, k] = 1.0
        Y, _ = oracle.qmv("q6_k", Wr, e)
        for n in range(5):
            assert Y[0, n] == oracle.dequant_row("q6_k", Wr[n], 512)[k]


def test_q6_k_brute_force_tiny_shapes_against_exact_rationals():
    r = np.random.default_rng(63)
    for K in (256, 512):
        N, M = 3, 2
        rows, dense = [], []
        for n in range(N):
            raw, vals = b"", []
            for sb in range(K // 256):
                codes = [int(c) for c in r.integers(0, 64, 256)]
                scales = [int(c) for c in r.integers(-128, 128, 16)]
                d_bits = [0x0123, 0x3555, 0x8C00][(n + sb) % 3]
                raw += _enc_q6_k(codes, scales, d_bits)
                d = _f16_fraction(d_bits)
                vals += [d * scales[i // 16] * (codes[i] - 32) for i in range(256)]
            rows.append(np.frombuffer(raw, dtype=np.uint8))
            dense.append(vals)
        W = np.stack(rows)
        X = r.standard_normal((M, K)).astype(np.float32)
        Y, A = oracle.qmv("q6_k", W, X)
        for m in range(M):
            for n in range(N):
                prods = [dense[n][k] * Fraction(float(X[m, k])) for k in range(K)]
                exact, mag = sum(prods), sum(abs(p) for p in prods)
                bound = Fraction(K * 2.0 ** -53 * float(mag))
                assert abs(Fraction(Y[m, n]) - exact) <= bound
                assert abs(Fraction(A[m, n]) - mag) <= bound


# --------------------------------------------------------------------------
# Q5_K super-blocks (256 weights, 176 bytes).
# --------------------------------------------------------------------------
def _enc_q5_k(codes, scales, mins, d_bits, dmin_bits):
    """Lay out 256 five-bit codes, eight 6-bit scales and minimums and the two
    binary16 scales the way the GGML Q5_K super-block stores them, walking
    the storage bytes: scale byte k (k < 4) = scale k | (scale k+4 >> 4) << 6;
    byte 4+k = min k | (min k+4 >> 4) << 6; byte 8+k = (scale k+4 & 15) |
    (min k+4 & 15) << 4; qh byte l holds bit 4 of code 32j + l at bit j; qs
    byte 32i + l = (code 64i + l & 15) | (code 64i + 32 + l & 15) << 4."""
    b = bytearray(176)
    b[0], b[1], b[2], b[3] = d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8
    for k in range(4):
        b[4 + k] = scales[k] | ((scales[k + 4] >> 4) << 6)
        b[8 + k] = mins[k] | ((mins[k + 4] >> 4) << 6)
        b[12 + k] = (scales[k + 4] & 15) | ((mins[k + 4] & 15) << 4)
    for l in range(32):
        b[16 + l] = sum(((codes[32 * j + l] >> 4) & 1) << j for j in range(8))
    for i in range(4):
        for l in range(32):
            b[48 + 32 * i + l] = (codes[64 * i + l] & 15) | ((codes[64 * i + 32 + l] & 15) << 4)
    return bytes(b)


def _q5_want(codes, scales, mins, d_bits, dmin_bits):
    d = Fraction(float(np.array(d_bits, dtype=np.uint16).view(np.float16)))
    dm = Fraction(float(np.array(dmin_bits, dtype=np.uint16).view(np.float16)))
    return [d * scales[i // 32] * codes[i] - dm * mins[i // 32] for i in range(256)]


def test_q5_k_hand_built_super_blocks():
    """Every code 0..31 eight times, every 6-bit scale and minimum value over
    the trials (high 2 bits included), normal, subnormal, negative and zero
    scales: weight i must be d * scale[i // 32] * q_i - dmin * min[i // 32]."""
    r = np.random.default_rng(71)
    pairs = [(0x3C00, 0x3800), (0x0001, 0x03FF), (0xC000, 0x2E66), (0x1234, 0x0000), (0x7BFF, 0x8001)]
    for trial, (db, mb) in enumerate(pairs * 2):
        codes = [int(c) for c in r.permutation(np.repeat(np.arange(32), 8))]
        scales = [int(v) for v in r.integers(0, 64, 8)]
        mins = [int(v) for v in r.integers(0, 64, 8)]
        scales[trial % 8], mins[(trial + 3) % 8] = 63, 63
        raw = np.frombuffer(_enc_q5_k(codes, scales, mins, db, mb), dtype=np.uint8)
        w = oracle.dequant_row("q5_k", raw, 256)
        want = [float(v) for v in _q5_want(codes, scales, mins, db, mb)]
        assert np.array_equal(w, np.array(want)), trial


def test_q5_k_brute_force_and_one_hot():
    r = np.random.default_rng(72)
    K, N = 512, 3
    rows, dense = [], []
    for n in range(N):
        raw, vals = b"", []
        for sb in range(K // 256):
            codes = [int(c) for c in r.integers(0, 32, 256)]
            scales = [int(c) for c in r.integers(0, 64, 8)]
            mins = [int(c) for c in r.integers(0, 64, 8)]
            db, mb = [(0x2A00, 0x1F00), (0x0040, 0x0123), (0x3555, 0x3000)][(n + sb) % 3]
            raw += _enc_q5_k(codes, scales, mins, db, mb)
            vals += _q5_want(codes, scales, mins, db, mb)
        rows.append(np.frombuffer(raw, dtype=np.uint8))
        dense.append(vals)
    W = np.stack(rows)
    X = r.standard_normal((2, K)).astype(np.float32)
    Y, A = oracle.qmv("q5_k", W, X)
    for m in range(2):
        for n in range(N):
            prods = [dense[n][k] * Fraction(float(X[m, k])) for k in range(K)]
            exact, mag = sum(prods), sum(abs(p) for p in prods)
            bound = Fraction(K * 2.0 ** -53 * float(mag))
            assert abs(Fraction(Y[m, n]) - exact) <= bound
            assert abs(Fraction(A[m, n]) - mag) <= bound
    for k in (0, 31, 32, 255, 256, 511):
        e = np.zeros((1, K), np.float32)
        e[0, k] = 1.0
        Y, _ = oracle.qmv("q5_k", W, e)
        assert all(Y[0, n] == float(dense[n][k]) for n in range(N))


# --------------------------------------------------------------------------
# MLX affine 4-bit, groups of 32 (codes eight to a 32-bit word, bf16 scale and
# bias per group).
# --------------------------------------------------------------------------
def _pack_words(codes):
    """codes [..., K] in 0..15 -> uint32 words [..., K/8], code j of a word in bits 4j."""
    c = np.asarray(codes, dtype=np.uint32).reshape(*np.shape(codes)[:-1], -1, 8)
    return np.bitwise_or.reduce(c << (4 * np.arange(8, dtype=np.uint32)), axis=-1).astype(np.uint32)


def _bf16_bits(values):
    """Truncate fp32 values to bf16 bit patterns (exactly representable inputs are kept)."""
    return (np.asarray(values, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    want = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_affine4_hand_built_rows():
    """Every code at every position of a word; scales and biases exactly
    representable in bf16 (signs, powers of two, subnormal): weight k must be
    scale[k // 32] * code_k + bias[k // 32]."""
    r = np.random.default_rng(81)
    K = 256
    for trial in range(6):
        codes = np.array([(k * 5 + k // 8 + trial) % 16 for k in range(K)])
        sc = np.array([0.5, -0.25, 3.0, 1.0 / 1024, -6.0, 2.0 ** -130, 0.75, 96.0], dtype=np.float32)[r.permutation(8)]
        bi = np.array([-1.0, 0.125, 0.0, -3.5, 2.0, -0.0, 7.0, 2.0 ** -128], dtype=np.float32)[r.permutation(8)]
        w = oracle.dequant_affine4_row(_pack_words(codes), _bf16_bits(sc), _bf16_bits(bi), K)
        want = [Fraction(float(sc[k // 32])) * int(codes[k]) + Fraction(float(bi[k // 32])) for k in range(K)]
        assert np.array_equal(w, np.array([float(v) for v in want])), trial


def test_affine4_brute_force_and_one_hot():
    r = np.random.default_rng(82)
    N, K = 3, 128
    codes = r.integers(0, 16, (N, K))
    sc = _bf16_bits(r.uniform(-0.05, 0.05, (N, K // 32)))
    bi = _bf16_bits(r.uniform(-0.3, 0.3, (N, K // 32)))
    Wq = _pack_words(codes)
    X = r.standard_normal((2, K)).astype(np.float32)
    Y, A = oracle.qmv_affine4(Wq, sc, bi, X)
    scf = (sc.astype(np.uint32) << 16).view(np.float32)
    bif = (bi.astype(np.uint32) << 16).view(np.float32)
    for m in range(2):
        for n in range(N):
            prods = [(Fraction(float(scf[n, k // 32])) * int(codes[n, k]) + Fraction(float(bif[n, k // 32])))
                     * Fraction(float(X[m, k])) for k in range(K)]
            exact, mag = sum(prods), sum(abs(p) for p in prods)
            bound = Fraction(K * 2.0 ** -53 * float(mag))
            assert abs(Fraction(Y[m, n]) - exact) <= bound
            assert abs(Fraction(A[m, n]) - mag) <= bound
    for k in (0, 7, 8, 31, 32, 127):
        e = np.zeros((1, K), np.float32)
        e[0, k] = 1.0
        Y, _ = oracle.qmv_affine4(Wq, sc, bi, e)
        for n in range(N):
            assert Y[0, n] == float(scf[n, k // 32]) * int(codes[n, k]) + float(bif[n, k // 32])
