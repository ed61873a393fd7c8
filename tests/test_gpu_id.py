"""GPU parity of qmv_id (expert-indexed product) against the CPU oracle.

Routing must be bit-exact: the signature weights make every output row equal
(e + 1) * K exactly for expert e, so a row that used the wrong expert, the
wrong activation row or the wrong output row is caught bit for bit.
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_id(qtype, W, X, ids, N, K, escale=None, err=False, ldy=None):
    ids2 = ids if ids.ndim == 2 else ids[:, None]
    P = ids2.size
    Yfull = torch.full((P, ldy or N), np.nan, dtype=torch.float32, device=DEV)
    Y = Yfull[:, :N]
    errd = torch.zeros(1, dtype=torch.int32, device=DEV) if err else None
    qmv.qmv_id(qtype, to_dev(W), to_dev(X), to_dev(ids2.astype(np.uint32)), Y, N, K,
               expert_scale=None if escale is None else to_dev(escale), err_flag=errd)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), (int(errd.item()) if err else None), Yfull.cpu().numpy()


def signature_stack(qtype, E, N, K):
    bb = synth.BLOCK_BYTES[qtype]
    W = np.empty((E, N, K // 32, bb), dtype=np.uint8)
    for e in range(E):
        bits = int(np.array(e + 1, dtype=np.float16).view(np.uint16))
        W[e, :, :, 0], W[e, :, :, 1] = bits & 0xFF, bits >> 8
        W[e, :, :, 2:] = 0x99 if qtype == "q4_0" else 0x01
    return W.reshape(E, N, -1)


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("K", [2816, 704, 96])
def test_routing_signature_bit_exact(qtype, K):
    E, N = 128, 72
    W = signature_stack(qtype, E, N, K)
    r = np.random.default_rng(K)
    ids = r.integers(0, E, size=(9, 8)).astype(np.uint32)
    ids[1] = ids[0]           # a token repeating another's experts
    ids[2, :] = 77            # one expert in every slot of a token
    ids[3, 5] = ids[3, 2]     # a duplicate inside a token
    X = np.ones((9, K), dtype=np.float32)
    y, _, _ = run_id(qtype, W, X, ids, N, K)
    want = ((ids.reshape(-1).astype(np.float64) + 1) * K).astype(np.float32)
    assert np.array_equal(y, np.repeat(want[:, None], N, axis=1))
    sc = np.linspace(0.5, 1.5, E).astype(np.float32)
    y, _, _ = run_id(qtype, W, X, ids, N, K, escale=sc)
    want = (sc[ids.reshape(-1)].astype(np.float64) * (ids.reshape(-1) + 1) * K).astype(np.float32)
    assert np.array_equal(y, np.repeat(want[:, None], N, axis=1))


def test_routing_signature_token_rows():
    """x row t = (t + 1) * ones: row t*top_k + s must be (t + 1)(e + 1)K."""
    E, N, K = 16, 40, 128
    W = signature_stack("q4_0", E, N, K)
    ids = np.array([[3, 9], [9, 3], [0, 15], [15, 15]], dtype=np.uint32)
    X = np.stack([np.full(K, t + 1, dtype=np.float32) for t in range(4)])
    y, _, _ = run_id("q4_0", W, X, ids, N, K)
    for t in range(4):
        for s in range(2):
            assert np.all(y[t * 2 + s] == (t + 1) * (int(ids[t, s]) + 1) * K)


def _moe_check(T, call_idx, sample_rows=None, escale=True):
    inp = synth.moe_inputs(T)
    call = synth.moe_calls(T)[call_idx]
    W = inp["W_gate_up"] if call.name == "gate_up" else inp["W_down"]
    X = inp["X_gate_up"] if call.name == "gate_up" else inp["X_down"]
    ids = inp["ids"] if call.name == "gate_up" else inp["ids"].reshape(-1, 1)
    sc = inp["expert_scale"] if escale else None
    y, _, _ = run_id("q4_0", W, X, ids, call.N, call.K, escale=sc)
    rows = np.arange(call.N) if sample_rows is None else sample_rows
    yo, a = oracle.qmv_id("q4_0", W[:, rows, :], X, ids, len(rows), call.K, expert_scale=sc)
    return assert_within_tol(y[:, rows], yo, a, f"moe T={T} {call.name}")


@pytest.mark.parametrize("call_idx", [0, 1])
def test_moe_t1_full(call_idx):
    print("ratio", _moe_check(1, call_idx))


@pytest.mark.parametrize("call_idx", [0, 1])
def test_moe_t32_full(call_idx):
    print("ratio", _moe_check(32, call_idx))


@pytest.mark.parametrize("call_idx", [0, 1])
def test_moe_t128_full(call_idx):
    """128 tokens (1024 pairs, 8 per expert on average): the matrix-core
    grouped kernel, every output element against the oracle."""
    print("ratio", _moe_check(128, call_idx))


def test_moe_without_expert_scale():
    _moe_check(1, 0, escale=False)


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_small_random_stack_against_oracle(qtype):
    E, N, K = 6, 100, 320
    W = synth.make_weights(qtype, E * N, K, cfg=80).reshape(E, N, -1)
    X = synth.make_x(5, K, cfg=80)
    ids = np.array([[0, 5, 2], [2, 2, 1], [4, 0, 3], [5, 5, 5], [1, 3, 0]], dtype=np.uint32)
    y, _, _ = run_id(qtype, W, X, ids, N, K)
    yo, a = oracle.qmv_id(qtype, W, X, ids, N, K)
    assert_within_tol(y, yo, a, qtype)


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("K", [2816, 704])
def test_one_expert_serving_many_pairs(qtype, K):
    """Slot 0 of all 24 tokens picks expert 3: its weights are streamed once
    for several passes of staged activation rows; every pair's own token row
    and output row must be used."""
    E, T, N = 16, 24, 136
    W = synth.make_weights(qtype, E * N, K, cfg=96, part=K).reshape(E, N, -1)
    X = synth.make_x(T, K, cfg=96, part=K)
    r = np.random.default_rng(K)
    ids = np.stack([np.full(T, 3), r.integers(0, E, T)], axis=1).astype(np.uint32)
    sc = synth.expert_scale(E, cfg=96)
    y, _, _ = run_id(qtype, W, X, ids, N, K, escale=sc)
    yo, a = oracle.qmv_id(qtype, W, X, ids, N, K, sc)
    assert_within_tol(y, yo, a, f"{qtype} K={K}")


def test_out_of_range_id_gives_nan_row_and_sets_flag():
    E, N, K = 8, 64, 256
    W = synth.make_weights("q4_0", E * N, K, cfg=81).reshape(E, N, -1)
    X = synth.make_x(2, K, cfg=81)
    ids = np.array([[1, 8], [3, 1000]], dtype=np.uint32)
    y, flag, _ = run_id("q4_0", W, X, ids, N, K, err=True)
    assert flag == 1
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[3]))
    good = np.array([[1], [3]], dtype=np.uint32)
    yo, a = oracle.qmv_id("q4_0", W, X, good, N, K)
    assert_within_tol(y[[0, 2]], yo, a, "valid rows")
    _, flag, _ = run_id("q4_0", W, X, np.array([[1, 2], [3, 4]], dtype=np.uint32), N, K, err=True)
    assert flag == 0


def test_out_of_range_ids_among_many_pairs():
    """More pairs than the few-pairs kernel takes: the grouped kernel writes
    NaN rows for ids out of range and serves the rest."""
    E, N, K = 12, 72, 192
    W = synth.make_weights("q4_0", E * N, K, cfg=83).reshape(E, N, -1)
    T, k = 40, 2  # 80 pairs
    X = synth.make_x(T, K, cfg=83)
    ids = np.random.default_rng(83).integers(0, E, size=(T, k)).astype(np.uint32)
    bad = [(3, 1), (17, 0), (39, 1)]
    for t, s in bad:
        ids[t, s] = E + 7 * t
    y, flag, _ = run_id("q4_0", W, X, ids, N, K, err=True)
    assert flag == 1
    badrows = [t * k + s for t, s in bad]
    assert np.all(np.isnan(y[badrows]))
    keep = np.ones(T * k, bool)
    keep[badrows] = False
    ids_ok = ids.copy()
    for t, s in bad:
        ids_ok[t, s] = 0
    yo, a = oracle.qmv_id("q4_0", W, X, ids_ok, N, K)
    assert_within_tol(y[keep], yo[keep], a[keep], "valid rows")


def test_more_experts_than_the_grouping_tables():
    """1100 experts (beyond what the grouped kernel's LDS tables index): the
    per-expert leader kernel serves the call."""
    E, N, K = 1100, 24, 128
    W = synth.make_weights("q8_0", E * N, K, cfg=84).reshape(E, N, -1)
    T, k = 40, 3
    X = synth.make_x(T, K, cfg=84)
    ids = np.random.default_rng(84).integers(0, E, size=(T, k)).astype(np.uint32)
    ids[5, 0] = ids[9, 2] = 1099
    y, _, _ = run_id("q8_0", W, X, ids, N, K)
    yo, a = oracle.qmv_id("q8_0", W, X, ids, N, K)
    assert_within_tol(y, yo, a, "1100 experts")


def test_many_pairs_split_across_launches_and_padded_ldy():
    E, N, K = 32, 48, 128
    W = synth.make_weights("q4_0", E * N, K, cfg=82).reshape(E, N, -1)
    T, k = 300, 4  # 1200 pairs > one launch's list
    X = synth.make_x(T, K, cfg=82)
    ids = np.random.default_rng(82).integers(0, E, size=(T, k)).astype(np.uint32)
    y, _, yfull = run_id("q4_0", W, X, ids, N, K, ldy=N + 5)
    yo, a = oracle.qmv_id("q4_0", W, X, ids, N, K)
    assert_within_tol(y, yo, a, "1200 pairs")
    assert np.all(np.isnan(yfull[:, N:]))


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("K", [2816, 704, 256])
def test_grouped_matrix_core_path(qtype, K):
    """Many pairs per expert take the matrix-core grouped kernel: 8 experts,
    160 tokens x top-4 = 640 pairs (about 80 per expert: several 16-pair
    blocks, the last ragged), N = 200 (a ragged 64-row tile), expert scales
    and padded output rows. K = 2816 splits K over four waves of an item,
    704 and 256 run one wave per item. A second call is bitwise equal."""
    E, T, k, N = 8, 160, 4, 200
    W = synth.make_weights(qtype, E * N, K, cfg=97, part=K).reshape(E, N, -1)
    X = synth.make_x(T, K, cfg=97, part=K)
    ids = np.random.default_rng(97 + K).integers(0, E, size=(T, k)).astype(np.uint32)
    sc = synth.expert_scale(E, cfg=97)
    y, _, yfull = run_id(qtype, W, X, ids, N, K, escale=sc, ldy=N + 3)
    yo, a = oracle.qmv_id(qtype, W, X, ids, N, K, sc)
    assert_within_tol(y, yo, a, f"{qtype} K={K}")
    assert np.all(np.isnan(yfull[:, N:]))
    y2, _, _ = run_id(qtype, W, X, ids, N, K, escale=sc, ldy=N + 3)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_grouped_matrix_core_bad_ids_and_two_launches():
    """1200 pairs over 16 experts (two launches of at most 1024 pairs, both
    on the matrix-core grouped kernel) with ids out of range: NaN rows, the
    flag set, every other row against the oracle."""
    E, N, K = 16, 72, 512
    W = synth.make_weights("q4_0", E * N, K, cfg=98).reshape(E, N, -1)
    T, k = 300, 4
    X = synth.make_x(T, K, cfg=98)
    ids = np.random.default_rng(98).integers(0, E, size=(T, k)).astype(np.uint32)
    bad = [(0, 3), (255, 0), (256, 1), (299, 3)]  # both launches
    for t, s_ in bad:
        ids[t, s_] = E + t
    y, flag, _ = run_id("q4_0", W, X, ids, N, K, err=True)
    assert flag == 1
    badrows = [t * k + s_ for t, s_ in bad]
    assert np.all(np.isnan(y[badrows]))
    keep = np.ones(T * k, bool)
    keep[badrows] = False
    ids_ok = ids.copy()
    for t, s_ in bad:
        ids_ok[t, s_] = 0
    yo, a = oracle.qmv_id("q4_0", W, X, ids_ok, N, K)
    assert_within_tol(y[keep], yo[keep], a[keep], "valid rows")


def test_zero_tokens_is_a_no_op():
    Y = torch.full((4, 8), 3.0, device=DEV)
    W = torch.zeros((2, 8, 18), dtype=torch.uint8, device=DEV)
    qmv.qmv_id("q4_0", W, torch.zeros((0, 32), device=DEV), torch.zeros((0, 2), dtype=torch.int32, device=DEV),
               Y, 8, 32)
    torch.cuda.synchronize()
    assert torch.all(Y == 3.0)


def test_deterministic_bitwise():
    inp = synth.moe_inputs(32)
    call = synth.moe_calls(32)[0]
    y1, _, _ = run_id("q4_0", inp["W_gate_up"], inp["X_gate_up"], inp["ids"], call.N, call.K)
    y2, _, _ = run_id("q4_0", inp["W_gate_up"], inp["X_gate_up"], inp["ids"], call.N, call.K)
    assert np.array_equal(y1, y2)


# --------------------------------------------------------------------------
# Q6_K experts (the pages' production MoE keeps gate_up experts as Q6_K).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(2816, 1408), (512, 300), (256, 77)])
def test_q6k_stack_against_oracle(K, N):
    E, T = 12, 5
    W = synth.make_weights("q6_k", E * N, K, cfg=83, part=K).reshape(E, N, -1)
    X = synth.make_x(T, K, cfg=83, part=K)
    ids = np.array([[0, 11, 2], [2, 2, 1], [4, 0, 3], [5, 5, 5], [11, 3, 0]], dtype=np.uint32)
    sc = synth.expert_scale(E, cfg=83)
    y, _, _ = run_id("q6_k", W, X, ids, N, K, escale=sc)
    yo, a = oracle.qmv_id("q6_k", W, X, ids, N, K, sc)
    assert_within_tol(y, yo, a, f"q6_k K={K}")


def test_q6k_moe_gate_up_t1_and_bad_id():
    """The gate_up call of one token, 128 Q6_K experts [1408, 2816], top-8;
    then an out-of-range id gives a NaN row and sets the flag."""
    E, N, K = 128, 1408, 2816
    W = synth.make_weights("q6_k", E * N, K, cfg=84).reshape(E, N, -1)
    X = synth.make_x(1, K, cfg=84)
    ids = synth.router_topk(1, E, 8, cfg=84)
    sc = synth.expert_scale(E, cfg=84)
    y, _, _ = run_id("q6_k", W, X, ids, N, K, escale=sc)
    yo, a = oracle.qmv_id("q6_k", W, X, ids, N, K, sc)
    print("ratio", assert_within_tol(y, yo, a, "q6_k gate_up T=1"))
    bad = ids.copy()
    bad[0, 3] = 128
    y2, flag, _ = run_id("q6_k", W, X, bad, N, K, escale=sc, err=True)
    assert flag == 1 and np.all(np.isnan(y2[3]))
    keep = [0, 1, 2, 4, 5, 6, 7]
    assert np.array_equal(y2[keep], y[keep])
