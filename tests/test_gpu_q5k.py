"""GPU parity of qmv_q5_k (Q5_K super-blocks) against the CPU oracle.

Shapes: the pages' B9 group (gate and up 2816 -> 5760, router 2816 -> 128),
every lanes-per-row choice, padded rows, M = 1..16, one-hot activations
(one rounding of the exact weight), and Q5_K experts in the expert-indexed
call.
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(W, X, N, K, ldy=None):
    M = X.shape[0]
    Yfull = torch.full((M, ldy or N), np.nan, dtype=torch.float32, device=DEV)
    Y = Yfull[:, :N]
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    qmv.qmv_q5_k(Wd, Xd if M > 1 else Xd[0], Y if M > 1 else Y[0], K=K)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Yfull.cpu().numpy()


@pytest.mark.parametrize("N,K", [(5760, 2816), (128, 2816), (1000, 256), (77, 512), (2050, 4096), (64, 16384)])
def test_q5k_m1_against_oracle(N, K):
    W = synth.make_weights("q5_k", N, K, cfg=65, part=K)
    X = synth.make_x(1, K, cfg=65, part=K)
    y, _ = run(W, X, N, K)
    yo, a = oracle.qmv("q5_k", W, X)
    print("ratio", assert_within_tol(y, yo, a, f"N={N} K={K}"))


@pytest.mark.parametrize("M", [2, 5, 16])
def test_q5k_multi_row_padded(M):
    N, K = 700, 2816
    ldw = synth.row_bytes("q5_k", K) + 10
    W = synth.make_weights("q5_k", N, K, cfg=66, part=M, ldw=ldw)
    X = synth.make_x(M, K, cfg=66, part=M)
    y, full = run(W, X, N, K, ldy=N + 3)
    yo, a = oracle.qmv("q5_k", W, X)
    assert_within_tol(y, yo, a, f"M={M}")
    assert np.all(np.isnan(full[:, N:]))


def test_q5k_one_hot_is_one_rounding_of_the_weight():
    N, K = 96, 2816
    W = synth.make_weights("q5_k", N, K, cfg=67)
    ks = [0, 1, 31, 32, 127, 128, 255, 256, 1000, 2815]
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    y, _ = run(W, X, N, K)
    for i, k in enumerate(ks):
        want = np.array([oracle.dequant_row("q5_k", W[n], K)[k] for n in range(N)]).astype(np.float32)
        assert np.array_equal(y[i], want), k


def test_q5k_experts_in_the_id_call():
    E, N, K, T = 10, 300, 512, 4
    W = synth.make_weights("q5_k", E * N, K, cfg=68).reshape(E, N, -1)
    X = synth.make_x(T, K, cfg=68)
    ids = np.array([[0, 9], [3, 3], [7, 1], [2, 0]], dtype=np.uint32)
    sc = synth.expert_scale(E, cfg=68)
    Y = torch.full((T * 2, N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_id("q5_k", torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV),
               torch.from_numpy(ids.astype(np.int32)).to(DEV), Y, N, K, expert_scale=torch.from_numpy(sc).to(DEV))
    torch.cuda.synchronize()
    yo, a = oracle.qmv_id("q5_k", W, X, ids, N, K, sc)
    assert_within_tol(Y.cpu().numpy(), yo, a, "q5_k id")
