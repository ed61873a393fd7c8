"""GPU parity of the MLX affine 4-bit products (groups of 32, bf16 scale and
bias per group) against the CPU oracle: dense rows of every lane choice,
rows that are not a multiple of 128 weights (the MoE down width 704), M up
to 16, padded strides, one-hot rows, and stacked experts."""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def run(Wq, S, B, X, N):
    M = X.shape[0]
    Y = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_affine4(dev(Wq.view(np.int32)), dev(S.view(np.int16)), dev(B.view(np.int16)), dev(X), Y if M > 1 else Y[0])
    torch.cuda.synchronize()
    return Y.cpu().numpy()


@pytest.mark.parametrize("N,K,M", [(1408, 2816, 1), (2816, 704, 1), (300, 96, 1), (77, 4096, 1), (64, 16384, 1),
                                   (500, 704, 3), (257, 2816, 16)])
def test_affine4_against_oracle(N, K, M):
    Wq, S, B = synth.make_affine4(N, K, cfg=40, part=K)
    X = synth.make_x(M, K, cfg=40, part=K)
    y = run(Wq, S, B, X, N)
    yo, a = oracle.qmv_affine4(Wq, S, B, X)
    print("ratio", assert_within_tol(y, yo, a, f"N={N} K={K} M={M}"))


def test_affine4_padded_strides():
    N, K = 200, 704
    Wq, S, B = synth.make_affine4(N, K + 64, cfg=41)  # wider arrays: rows padded past K
    X = synth.make_x(1, K, cfg=41)
    y = run(Wq, S, B, X, N)
    yo, a = oracle.qmv_affine4(Wq, S, B, X)
    assert_within_tol(y, yo, a, "padded")


def test_affine4_one_hot_is_one_rounding_of_the_weight():
    N, K = 64, 704
    Wq, S, B = synth.make_affine4(N, K, cfg=42)
    ks = [0, 1, 7, 8, 31, 32, 127, 128, 640, 703]
    X = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    for i, k in enumerate(ks):
        y = run(Wq, S, B, X[i:i + 1], N)
        want = np.array([oracle.dequant_affine4_row(Wq[n], S[n], B[n], K)[k] for n in range(N)]).astype(np.float32)
        assert np.array_equal(y[0], want), k


@pytest.mark.parametrize("K,N", [(2816, 1408), (704, 2816)])
def test_affine4_experts_decode(K, N):
    """The MoE calls of one token over 32 affine experts: gate_up form (one x
    row, top-8) and down form (8 x rows, one slot each), with a bad id."""
    E = 32
    Wq, S, B = synth.make_affine4(E * N, K, cfg=43, part=K)
    Wq, S, B = Wq.reshape(E, N, -1), S.reshape(E, N, -1), B.reshape(E, N, -1)
    ids = synth.router_topk(1, E, 8, cfg=43, part=K)
    if K == 704:
        ids = ids.reshape(-1, 1)
    T = ids.shape[0]
    X = synth.make_x(T, K, cfg=43, part=K)
    sc = synth.expert_scale(E, cfg=43)
    Y = torch.full((ids.size, N), np.nan, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    qmv.qmv_affine4_id(dev(Wq.view(np.int32)), dev(S.view(np.int16)), dev(B.view(np.int16)), dev(X),
                       dev(ids.astype(np.int32)), Y, N, K, expert_scale=dev(sc), err_flag=err)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert int(err.item()) == 0
    for p, e in enumerate(ids.reshape(-1)):
        t = p // ids.shape[1]
        yo, a = oracle.qmv_affine4(Wq[e], S[e], B[e], X[t:t + 1])
        assert_within_tol(y[p:p + 1] / 1.0, yo * float(sc[e]), a * abs(float(sc[e])), f"pair {p}")
    bad = ids.copy()
    bad.reshape(-1)[1] = E + 5
    Y.fill_(0.0)
    qmv.qmv_affine4_id(dev(Wq.view(np.int32)), dev(S.view(np.int16)), dev(B.view(np.int16)), dev(X),
                       dev(bad.astype(np.int32)), Y, N, K, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1 and np.all(np.isnan(Y.cpu().numpy()[1]))
