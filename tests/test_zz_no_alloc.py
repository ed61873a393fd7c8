"""qmv_ws_static (the allocation-free variant of qmv_ws, whose K-segment
partial sums live in the library's static device scratch) against qmv_ws with
a caller workspace, through the C ABI: two calls in a row, the second
smaller, each bit for bit equal to qmv_ws (same kernels, same plan) and
within the tolerance of the oracle."""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _args(W, X, Y):
    return (W.data_ptr(), W.stride(0), X.data_ptr(), X.stride(0), Y.data_ptr(), Y.stride(0), X.shape[0], W.shape[0],
            X.shape[1])


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_static_scratch_matches_caller_workspace(qtype):
    q = qmv.QTYPES[qtype]
    st = torch.cuda.current_stream().cuda_stream
    # second call smaller in every dimension: it must not read what the first left behind
    for i, (M, N, K) in enumerate([(16, 5120, 5120), (7, 1000, 2048)]):
        W = synth.make_weights(qtype, N, K, cfg=73, part=i)
        X = synth.make_x(M, K, cfg=73, part=i)
        nb = qmv.ws_bytes(qtype, M, N, K)
        assert 0 < nb <= qmv.lib().qmv_ws_bytes(q, M, N, K) <= (4 << 20)
        Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
        Ys = torch.full((M, N), np.nan, device=DEV)
        Yw = torch.full((M, N), np.nan, device=DEV)
        ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device=DEV)
        assert qmv.raw_qmv_ws_static(q, *_args(Wd, Xd, Ys), st) == qmv.QMV_OK, qmv.last_error()
        assert qmv.raw_qmv_ws(q, *_args(Wd, Xd, Yw), ws.data_ptr(), nb, st) == qmv.QMV_OK, qmv.last_error()
        torch.cuda.synchronize()
        ys, yw = Ys.cpu().numpy(), Yw.cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), yw.view(np.uint32)), f"call {i}: static scratch != workspace"
        yo, a = oracle.qmv(qtype, W, X)
        assert_within_tol(ys, yo, a, f"{qtype} call {i} M={M} N={N} K={K}")


def test_static_scratch_rejects_and_passes_through():
    """M = 1 and many-row calls need no scratch (plain kernels); an unsupported
    qtype is rejected on the host."""
    st = torch.cuda.current_stream().cuda_stream
    W = synth.make_weights("q4_0", 300, 1024, cfg=72)
    X = synth.make_x(1, 1024, cfg=72)
    Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
    Y = torch.empty((1, 300), device=DEV)
    assert qmv.raw_qmv_ws_static(qmv.QMV_Q4_0, *_args(Wd, Xd, Y), st) == qmv.QMV_OK
    torch.cuda.synchronize()
    yo, a = oracle.qmv("q4_0", W, X)
    assert_within_tol(Y.cpu().numpy(), yo, a, "M = 1")
    assert qmv.raw_qmv_ws_static(qmv.QMV_Q6_K, *_args(Wd, Xd, Y), st) == qmv.QMV_EUNSUPPORTED
