"""GPU parity of qmv_ws (the dense product with a caller workspace that lets
calls of few output rows split K over workgroups) against the CPU oracle,
and against the workspace-free call."""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_ws(qtype, W, X, ws=True, ldy=None):
    M, N, K = X.shape[0], W.shape[0], X.shape[1]
    nb = qmv.ws_bytes(qtype, M, N, K)
    wsd = torch.empty(max(nb, 256) + 256, dtype=torch.uint8, device=DEV) if ws else None
    Yfull = torch.full((M, ldy or N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_ws(qtype, torch.from_numpy(np.ascontiguousarray(W)).to(DEV), torch.from_numpy(X).to(DEV),
               Yfull[:, :N], wsd)
    torch.cuda.synchronize()
    return Yfull.cpu().numpy()[:, :N], Yfull.cpu().numpy(), nb


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_ws_m16_workload_full(qtype):
    """Config 3's shapes (M = 16, K = 5120), every output element."""
    for part, p in enumerate(synth.CONFIGS[3]["problems"]):
        W = synth.make_weights(qtype, p.N, p.K, cfg=3, part=part)
        X = synth.make_x(p.M, p.K, cfg=3, part=part)
        y, _, nb = run_ws(qtype, W, X)
        yo, a = oracle.qmv(qtype, W, X)
        r = assert_within_tol(y, yo, a, f"{qtype} N={p.N}")
        print(f"{qtype} N={p.N}: workspace {nb} B, max ratio {r:.3g}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", [(2, 64, 5120), (5, 300, 1088), (16, 17, 64), (16, 4100, 2112), (9, 1000, 14336),
                                   (16, 129, 704)])
def test_ws_shapes_and_padded_y(qtype, M, N, K):
    W = synth.make_weights(qtype, N, K, cfg=77, part=M)
    X = synth.make_x(M, K, cfg=77, part=M)
    y, full, _ = run_ws(qtype, W, X, ldy=N + 3)
    yo, a = oracle.qmv(qtype, W, X)
    assert_within_tol(y, yo, a, f"{qtype} M={M} N={N} K={K}")
    assert np.all(np.isnan(full[:, N:]))


def test_ws_repeat_bitwise_and_reuse():
    """Two calls with one workspace give the same bits; a call of other sizes
    in between leaves nothing behind."""
    W = synth.make_weights("q4_0", 1024, 5120, cfg=76)
    X = synth.make_x(16, 5120, cfg=76)
    W2 = synth.make_weights("q4_0", 300, 2048, cfg=76, part=1)
    X2 = synth.make_x(7, 2048, cfg=76, part=1)
    nb = max(qmv.ws_bytes("q4_0", 16, 1024, 5120), qmv.ws_bytes("q4_0", 7, 300, 2048))
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = []
    for Wi, Xi in ((W, X), (W2, X2), (W, X)):
        Y = torch.empty((Xi.shape[0], Wi.shape[0]), device=DEV)
        qmv.qmv_ws("q4_0", torch.from_numpy(Wi).to(DEV), torch.from_numpy(Xi).to(DEV), Y, ws)
        torch.cuda.synchronize()
        out.append(Y.cpu().numpy())
    assert np.array_equal(out[0].view(np.uint32), out[2].view(np.uint32))
    yo, a = oracle.qmv("q4_0", W2, X2)
    assert_within_tol(out[1], yo, a, "in-between call")


def test_ws_without_workspace_is_the_plain_call():
    W = synth.make_weights("q8_0", 777, 1536, cfg=75)
    X = synth.make_x(16, 1536, cfg=75)
    y, _, _ = run_ws("q8_0", W, X, ws=False)
    Y = torch.empty((16, 777), device=DEV)
    qmv.qmv_q8_0(torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV), Y)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(np.uint32), Y.cpu().numpy().view(np.uint32))


def test_ws_graph_replays():
    """Captured with its workspace, replayed three times with eager work in
    between: every replay gives the eager bits."""
    W = synth.make_weights("q4_0", 5120, 5120, cfg=74)
    X = synth.make_x(16, 5120, cfg=74)
    Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
    ws = torch.empty(qmv.ws_bytes("q4_0", 16, 5120, 5120), dtype=torch.uint8, device=DEV)
    Y = torch.empty((16, 5120), device=DEV)
    qmv.qmv_ws("q4_0", Wd, Xd, Y, ws)
    torch.cuda.synchronize()
    eager = Y.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        qmv.qmv_ws("q4_0", Wd, Xd, Y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        Y.fill_(np.nan)
        ws.fill_(0xFF)  # the workspace needs no initialisation
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().view(np.uint32), eager.view(np.uint32)), rep
