"""GPU parity of the MoE steps around the expert-indexed call against the CPU
oracle: the SwiGLU-fed down product (qmv_id_swiglu), the routing-weighted sum
(qmv_moe_wsum) and the one-launch down half (qmv_moe_down).

Inputs: the MoE workload's stacked Q4_0 weights (E = 128, hidden 2816,
intermediate 704), seeded stand-in gate_up rows N(0, 2.9^2), routing weights
that sum to 1 per token, and the per-expert scale U[0.5, 1.5].
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


def run_id_swiglu(qtype, W, G, ids, N, K, escale=None, err=False):
    ids2 = ids if ids.ndim == 2 else ids[:, None]
    Y = torch.full((ids2.size, N), np.nan, dtype=torch.float32, device=DEV)
    errd = torch.zeros(1, dtype=torch.int32, device=DEV) if err else None
    qmv.qmv_id_swiglu(qtype, to_dev(W), to_dev(G), to_dev(ids2.astype(np.uint32)), Y, N, K,
                      expert_scale=None if escale is None else to_dev(escale), err_flag=errd)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), (int(errd.item()) if err else None)


def run_moe_down(qtype, W, G, ids, w, N, K, escale=None, err=False, ldo=None):
    T = ids.shape[0]
    full = torch.full((T, ldo or N), np.nan, dtype=torch.float32, device=DEV)
    out = full[:, :N]
    errd = torch.zeros(1, dtype=torch.int32, device=DEV) if err else None
    qmv.qmv_moe_down(qtype, to_dev(W), to_dev(G), to_dev(ids.astype(np.uint32)), to_dev(w), out, N, K,
                     expert_scale=None if escale is None else to_dev(escale), err_flag=errd)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (int(errd.item()) if err else None), full.cpu().numpy()


def small_case(qtype, E, N, K, T, k, cfg):
    W = synth.make_weights(qtype, E * N, K, cfg=cfg, part=K).reshape(E, N, -1)
    G = synth.gate_up_rows(T * k, K, cfg=cfg, part=K)
    r = np.random.default_rng(cfg)
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.uint32)
    w = synth.routing_weights(T, k, cfg=cfg)
    sc = synth.expert_scale(E, cfg=cfg)
    return W, G, ids, w, sc


# --------------------------------------------------------------------------
# qmv_id_swiglu
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("K", [704, 2816, 96, 160])  # 96 and 160: K % 64 != 0, the generic kernel
def test_id_swiglu_small_stack(qtype, K):
    E, N, T = 6, 100, 5
    W = synth.make_weights(qtype, E * N, K, cfg=70, part=K).reshape(E, N, -1)
    G = synth.gate_up_rows(T, K, cfg=70, part=K)
    G[0, :8] = [-100, -89, -88, -30, 30, 88, 89, 100]  # gates where e^-z under/overflows in fp32
    ids = np.array([[0, 5, 2], [2, 2, 1], [4, 0, 3], [5, 5, 5], [1, 3, 0]], dtype=np.uint32)
    sc = synth.expert_scale(E, cfg=70)
    y, _ = run_id_swiglu(qtype, W, G, ids, N, K, escale=sc)
    yo, a = oracle.qmv_id_swiglu(qtype, W, G, ids, N, K, expert_scale=sc)
    assert_within_tol(y, yo, a, f"{qtype} K={K}")


@pytest.mark.parametrize("T", [1, 32])
def test_id_swiglu_moe_down_call(T):
    """The MoE down call fed by SwiGLU: (n_tokens = 8T, top_k = 1), every
    output element."""
    inp = synth.moe_inputs(T)
    dn = synth.moe_calls(T)[1]
    ids = inp["ids"].reshape(-1, 1)
    y, _ = run_id_swiglu("q4_0", inp["W_down"], inp["G_down"], ids, dn.N, dn.K, escale=inp["expert_scale"])
    yo, a = oracle.qmv_id_swiglu("q4_0", inp["W_down"], inp["G_down"], ids, dn.N, dn.K,
                                 expert_scale=inp["expert_scale"])
    print("ratio", assert_within_tol(y, yo, a, f"down T={T}"))


def test_id_swiglu_bad_id_nan_row_and_flag():
    E, N, K = 8, 64, 256
    W = synth.make_weights("q4_0", E * N, K, cfg=71).reshape(E, N, -1)
    G = synth.gate_up_rows(2, K, cfg=71)
    ids = np.array([[1, 8], [3, 2]], dtype=np.uint32)
    y, flag = run_id_swiglu("q4_0", W, G, ids, N, K, err=True)
    assert flag == 1 and np.all(np.isnan(y[1]))
    # row 0 = token 0 slot 0 (expert 1); rows 2, 3 = token 1 (experts 3, 2)
    yo, a = oracle.qmv_id_swiglu("q4_0", W, G[[0, 1, 1]], np.array([[1], [3], [2]], dtype=np.uint32), N, K)
    assert_within_tol(y[[0, 2, 3]], yo, a, "valid rows")


# --------------------------------------------------------------------------
# qmv_moe_wsum
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,k,N", [(1, 8, 2816), (32, 8, 2816), (3, 1, 257), (5, 3, 1), (2, 12, 1000)])
def test_wsum_against_oracle(T, k, N):
    r = np.random.default_rng(T * 1000 + k * 10 + N)
    Yn = (r.standard_normal((T * k, N)) * 3).astype(np.float32)
    w = synth.routing_weights(T, k, cfg=N)
    out = torch.full((T, N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_moe_wsum(to_dev(Yn), to_dev(w), out, k)
    torch.cuda.synchronize()
    ref, a = oracle.moe_wsum(Yn.astype(np.float64), w.reshape(-1), k)
    assert_within_tol(out.cpu().numpy(), ref, a, f"wsum T={T} k={k} N={N}")


def test_wsum_strided_rows_and_exact_small_integers():
    T, k, N = 2, 3, 2
    Yfull = torch.full((T * k, 7), 1e30, dtype=torch.float32, device=DEV)
    Yfull[:, :N] = torch.arange(1, 13, dtype=torch.float32, device=DEV).view(6, 2)
    w = torch.tensor([0.5, 0.25, 2.0, 1.0, -1.0, 0.125], device=DEV)
    ofull = torch.full((T, 5), 7.0, device=DEV)
    qmv.qmv_moe_wsum(Yfull[:, :N], w, ofull[:, :N], k)
    torch.cuda.synchronize()
    o = ofull.cpu().numpy()
    assert np.array_equal(o[:, :N], [[11.25, 14.0], [-0.625, -0.5]])
    assert np.all(o[:, N:] == 7.0)


# --------------------------------------------------------------------------
# qmv_moe_down (one launch)
# --------------------------------------------------------------------------
def test_moe_down_t1_full_workload():
    inp = synth.moe_inputs(1)
    dn = synth.moe_calls(1)[1]
    out, _, _ = run_moe_down("q4_0", inp["W_down"], inp["G_down"], inp["ids"], inp["weights"], dn.N, dn.K,
                             escale=inp["expert_scale"])
    ref, a = oracle.moe_down("q4_0", inp["W_down"], inp["G_down"], inp["ids"], inp["weights"], dn.N, dn.K,
                             expert_scale=inp["expert_scale"])
    print("ratio", assert_within_tol(out, ref, a, "moe_down T=1"))


@pytest.mark.parametrize("T", [4, 32])
def test_moe_down_full_shared_experts(T):
    inp = synth.moe_inputs(T)
    dn = synth.moe_calls(T)[1]
    ids = inp["ids"].copy()
    ids[1] = ids[0]  # token 1 picks token 0's experts
    out, _, _ = run_moe_down("q4_0", inp["W_down"], inp["G_down"], ids, inp["weights"], dn.N, dn.K,
                             escale=inp["expert_scale"])
    ref, a = oracle.moe_down("q4_0", inp["W_down"], inp["G_down"], ids, inp["weights"], dn.N, dn.K,
                             expert_scale=inp["expert_scale"])
    print("ratio", assert_within_tol(out, ref, a, f"moe_down T={T}"))


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("k,K,N", [(1, 704, 37), (2, 128, 300), (3, 192, 64), (8, 64, 1), (12, 256, 129),
                                   (8, 1920, 90), (16, 960, 50)])
def test_moe_down_shapes(qtype, k, K, N):
    """top_k below, at and above the eight waves of a workgroup (12 and 16:
    two slots per wave), every lanes-per-row choice, ragged N."""
    E, T = 20, 3
    W, G, ids, w, sc = small_case(qtype, E, N, K, T, k, cfg=k * 7 + K)
    out, _, _ = run_moe_down(qtype, W, G, ids, w, N, K, escale=sc)
    ref, a = oracle.moe_down(qtype, W, G, ids, w, N, K, expert_scale=sc)
    assert_within_tol(out, ref, a, f"{qtype} k={k} K={K} N={N}")


def test_moe_down_without_scale_padded_out_and_duplicate_slot():
    E, N, K, T, k = 10, 200, 704, 2, 8
    W, G, ids, w, _ = small_case("q4_0", E, N, K, T, k, cfg=72)
    ids[1, 3] = ids[1, 5]  # one expert in two slots of a token
    out, _, full = run_moe_down("q4_0", W, G, ids, w, N, K, ldo=N + 3)
    ref, a = oracle.moe_down("q4_0", W, G, ids, w, N, K)
    assert_within_tol(out, ref, a, "no scale")
    assert np.all(np.isnan(full[:, N:]))


def test_moe_down_bad_id_gives_nan_token_and_flag():
    E, N, K, T, k = 10, 64, 128, 3, 4
    W, G, ids, w, sc = small_case("q4_0", E, N, K, T, k, cfg=73)
    ids[1, 2] = 4000
    out, flag, _ = run_moe_down("q4_0", W, G, ids, w, N, K, escale=sc, err=True)
    assert flag == 1 and np.all(np.isnan(out[1]))
    keep = [0, 2]
    ref, a = oracle.moe_down("q4_0", W, G.reshape(T, k, -1)[keep].reshape(len(keep) * k, -1), ids[keep], w[keep],
                             N, K, expert_scale=sc)
    assert_within_tol(out[keep], ref, a, "valid tokens")
    _, flag, _ = run_moe_down("q4_0", W, G, np.zeros_like(ids), w, N, K, err=True)
    assert flag == 0


def test_moe_down_matches_two_call_path_and_is_deterministic():
    inp = synth.moe_inputs(1)
    dn = synth.moe_calls(1)[1]
    o1, _, _ = run_moe_down("q4_0", inp["W_down"], inp["G_down"], inp["ids"], inp["weights"], dn.N, dn.K,
                            escale=inp["expert_scale"])
    o2, _, _ = run_moe_down("q4_0", inp["W_down"], inp["G_down"], inp["ids"], inp["weights"], dn.N, dn.K,
                            escale=inp["expert_scale"])
    assert np.array_equal(o1, o2)
    y, _ = run_id_swiglu("q4_0", inp["W_down"], inp["G_down"], inp["ids"].reshape(-1, 1), dn.N, dn.K,
                         escale=inp["expert_scale"])
    out = torch.empty((1, dn.N), dtype=torch.float32, device=DEV)
    qmv.qmv_moe_wsum(to_dev(y), to_dev(inp["weights"]), out, 8)
    torch.cuda.synchronize()
    two = out.cpu().numpy()
    ref, a = oracle.moe_down("q4_0", inp["W_down"], inp["G_down"], inp["ids"], inp["weights"], dn.N, dn.K,
                             expert_scale=inp["expert_scale"])
    assert_within_tol(two, ref, a, "two-call path")
    print("fused vs two-call max |diff|", float(np.abs(o1 - two).max()))


def test_moe_down_zero_tokens_is_a_no_op():
    out = torch.full((1, 8), 3.0, device=DEV)
    W = torch.zeros((2, 8, 36), dtype=torch.uint8, device=DEV)
    qmv.qmv_moe_down("q4_0", W, torch.zeros((0, 128), device=DEV), torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                     torch.zeros((0, 2), device=DEV), out[:0], 8, 64)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
