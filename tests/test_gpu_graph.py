"""Calls captured into a HIP graph and replayed (needs an MI355X).

Every call can be captured as it is: the library allocates nothing, so a
captured call runs the same kernels as an eager one. Each replay is checked
against the oracle and bit for bit against the eager result, with eager work
and synchronisations between replays.
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_graph_replays_dense_and_batch():
    # M = 1; M = 16 with few tiles (K split over the waves of a tile); ragged
    # steps; M = 16 at N = 27648, K = 5120 (one wave per tile over all of K)
    cases = [(1, 300, 4096), (16, 64, 5120), (7, 700, 1088), (16, 27648, 5120)]
    data = []
    for i, (M, N, K) in enumerate(cases):
        W = synth.make_weights("q4_0", N, K, cfg=91, part=i)
        X = synth.make_x(M, K, cfg=91, part=i)
        data.append((W, X, torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV),
                     torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)))
    # batch of two M = 1 problems
    Wb = [synth.make_weights("q4_0", 256, 2048, cfg=91, part=10 + k) for k in range(2)]
    xb = synth.make_x(1, 2048, cfg=91, part=10)[0]
    Wbd = [torch.from_numpy(w).to(DEV) for w in Wb]
    xbd = torch.from_numpy(xb).to(DEV)
    ybd = [torch.full((256,), np.nan, dtype=torch.float32, device=DEV) for _ in range(2)]

    def calls():
        for _, _, Wd, Xd, Yd in data:
            qmv.qmv_q4_0(Wd, Xd, Yd)
        qmv.qmv_batch("q4_0", [(Wbd[k], xbd, ybd[k]) for k in range(2)])

    # eager reference (the same kernels as in the graph)
    calls()
    torch.cuda.synchronize()
    eager = [d[4].cpu().numpy().copy() for d in data]
    eager_b = [y.cpu().numpy().copy() for y in ybd]
    refs = [oracle.qmv("q4_0", W, X) for W, X, _, _, _ in data]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()

    first = None
    for rep in range(3):
        for _, _, _, _, Yd in data:
            Yd.fill_(np.nan)  # eager work between replays
        for y in ybd:
            y.fill_(np.nan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        outs = [d[4].cpu().numpy().copy() for d in data]
        for y, e, (yo, a), (M, N, K) in zip(outs, eager, refs, cases):
            assert_within_tol(y, yo, a, f"replay {rep} M={M} N={N} K={K}")
            assert np.array_equal(y.view(np.uint32), e.view(np.uint32)), f"replay {rep} M={M} N={N}: not the eager bits"
        for k in range(2):
            assert np.array_equal(ybd[k].cpu().numpy().view(np.uint32), eager_b[k].view(np.uint32))
        if first is None:
            first = outs
        else:
            for a_, b_ in zip(first, outs):
                assert np.array_equal(a_.view(np.uint32), b_.view(np.uint32))


def test_graph_replays_id():
    E, T, N, K = 16, 6, 96, 704
    W = synth.make_weights("q4_0", E * N, K, cfg=90).reshape(E, N, -1)
    X = synth.make_x(T, K, cfg=90)
    ids = synth.router_topk(T, E, 4, cfg=90)
    Wd, Xd = torch.from_numpy(W).to(DEV), torch.from_numpy(X).to(DEV)
    idd = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    Y = torch.full((T * 4, N), np.nan, dtype=torch.float32, device=DEV)
    qmv.qmv_id("q4_0", Wd, Xd, idd, Y, N, K)
    torch.cuda.synchronize()
    eager = Y.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        qmv.qmv_id("q4_0", Wd, Xd, idd, Y, N, K)
    torch.cuda.synchronize()
    yo, a = oracle.qmv_id("q4_0", W, X, ids, N, K)
    for rep in range(3):
        Y.fill_(np.nan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y = Y.cpu().numpy()
        assert np.array_equal(y.view(np.uint32), eager.view(np.uint32))
        assert_within_tol(y, yo, a, f"id replay {rep}")


def test_graph_replays_moe_ffn():
    """One MoE FFN token in a graph: gate_up id, then the one-launch down half;
    and the two-call down half (SwiGLU-fed id, weighted sum) beside it."""
    E, T, k, H, I = 16, 2, 4, 512, 192
    Wgu = synth.make_weights("q4_0", E * 2 * I, H, cfg=89, part=0).reshape(E, 2 * I, -1)
    Wdn = synth.make_weights("q4_0", E * H, I, cfg=89, part=1).reshape(E, H, -1)
    X = synth.make_x(T, H, cfg=89)
    ids = synth.router_topk(T, E, k, cfg=89)
    w = synth.routing_weights(T, k, cfg=89)
    sc = synth.expert_scale(E, cfg=89)
    d = {n: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
         for n, v in dict(Wgu=Wgu, Wdn=Wdn, X=X, ids=ids.astype(np.int32), w=w, sc=sc).items()}
    G = torch.full((T * k, 2 * I), np.nan, dtype=torch.float32, device=DEV)
    out1 = torch.full((T, H), np.nan, dtype=torch.float32, device=DEV)
    Yd = torch.full((T * k, H), np.nan, dtype=torch.float32, device=DEV)
    out2 = torch.full((T, H), np.nan, dtype=torch.float32, device=DEV)

    def calls():
        qmv.qmv_id("q4_0", d["Wgu"], d["X"], d["ids"], G, 2 * I, H)
        qmv.qmv_moe_down("q4_0", d["Wdn"], G, d["ids"], d["w"], out1, H, I, expert_scale=d["sc"])
        qmv.qmv_id_swiglu("q4_0", d["Wdn"], G, d["ids"].view(-1, 1), Yd, H, I, expert_scale=d["sc"])
        qmv.qmv_moe_wsum(Yd, d["w"], out2, k)

    calls()
    torch.cuda.synchronize()
    eager = [t.cpu().numpy().copy() for t in (G, out1, out2)]
    # the down half against the oracle, fed the gate_up rows the GPU produced
    ref, a = oracle.moe_down("q4_0", Wdn, eager[0], ids, w, H, I, expert_scale=sc)
    assert_within_tol(eager[1], ref, a, "eager one-launch")
    assert_within_tol(eager[2], ref, a, "eager two-call")
    gu, ga = oracle.qmv_id("q4_0", Wgu, X, ids, 2 * I, H)
    assert_within_tol(eager[0], gu, ga, "eager gate_up")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (G, out1, Yd, out2):
            t.fill_(np.nan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e, name in zip((G, out1, out2), eager, ("gate_up", "one-launch", "two-call")):
            assert np.array_equal(t.cpu().numpy().view(np.uint32), e.view(np.uint32)), f"replay {rep} {name}"
