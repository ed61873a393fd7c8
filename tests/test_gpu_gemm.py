"""GPU parity of qmv_gemm (any number of activation rows) against the oracle.

M spans one and several 16-row blocks with ragged tails; every weight type;
a prefill shape (M = 256 rows of a 4096 x 4096 Q4_0 matrix), every output element.
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(qtype, W, X, N, ldy=None):
    M = X.shape[0]
    Yfull = torch.full((M, ldy or N), np.nan, dtype=torch.float32, device=DEV)
    Y = Yfull[:, :N]
    qmv.qmv_gemm(qtype, torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV), Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Yfull.cpu().numpy()


@pytest.mark.parametrize("qtype,M,N,K", [("q4_0", 17, 300, 1088), ("q4_0", 33, 129, 4096), ("q4_0", 100, 64, 512),
                                         ("q4_0", 131, 1000, 2112), ("q4_0", 64, 128, 64), ("q8_0", 150, 260, 1088),
                                         ("q8_0", 40, 200, 1024), ("q6_k", 20, 150, 2816), ("q5_k", 21, 150, 2816),
                                         ("q4_0", 5, 77, 96)])
def test_gemm_against_oracle(qtype, M, N, K):
    W = synth.make_weights(qtype, N, K, cfg=90, part=M)
    X = synth.make_x(M, K, cfg=90, part=M)
    y, full = run(qtype, W, X, N, ldy=N + 2)
    yo, a = oracle.qmv(qtype, W, X)
    assert_within_tol(y, yo, a, f"{qtype} M={M}")
    assert np.all(np.isnan(full[:, N:]))


def test_gemm_prefill_shape_full():
    M, N, K = 256, 4096, 4096
    W = synth.make_weights("q4_0", N, K, cfg=91)
    X = synth.make_x(M, K, cfg=91)
    y, _ = run("q4_0", W, X, N)
    yo, a = oracle.qmv("q4_0", W, X)
    print("ratio", assert_within_tol(y, yo, a, "prefill"))


def test_gemm_row_blocks_agree_with_the_16_row_call_and_repeat_bitwise():
    """Rows 16..31 of a 40-row call and a 16-row dense call on those rows
    both meet the oracle (the 16-row call may split K, so the sums differ in
    order); a second 40-row call is bitwise identical to the first."""
    N, K = 256, 1024
    W = synth.make_weights("q4_0", N, K, cfg=92)
    X = synth.make_x(40, K, cfg=92)
    y, _ = run("q4_0", W, X, N)
    y2, _ = run("q4_0", W, X, N)
    assert np.array_equal(y, y2)
    Y16 = torch.empty((16, N), device=DEV)
    qmv.qmv_q4_0(torch.from_numpy(W).to(DEV), torch.from_numpy(X[16:32].copy()).to(DEV), Y16)
    torch.cuda.synchronize()
    yo, a = oracle.qmv("q4_0", W, X[16:32])
    assert_within_tol(y[16:32], yo, a, "rows 16..31 of the 40-row call")
    assert_within_tol(Y16.cpu().numpy(), yo, a, "16-row call")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_tiled_gemm_repeat_bitwise_and_unaligned_rows_fall_back(qtype):
    """The tiled kernel (>= 64 rows, 16-byte aligned X rows) repeats bitwise;
    the same product with X rows 4-byte aligned only (ldx = K + 1) goes
    through the 16-row blocks and also meets the oracle."""
    M, N, K = 200, 300, 1536
    W = synth.make_weights(qtype, N, K, cfg=93)
    X = synth.make_x(M, K, cfg=93)
    y1, _ = run(qtype, W, X, N)
    y2, _ = run(qtype, W, X, N)
    assert np.array_equal(y1, y2)
    yo, a = oracle.qmv(qtype, W, X)
    assert_within_tol(y1, yo, a, "tiled")
    Xp = torch.zeros((M, K + 1), dtype=torch.float32, device=DEV)
    Xp[:, :K] = torch.from_numpy(X).to(DEV)
    Y = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_gemm(qtype, torch.from_numpy(W).to(DEV), Xp[:, :K], Y)
    torch.cuda.synchronize()
    assert_within_tol(Y.cpu().numpy(), yo, a, "unaligned rows")
