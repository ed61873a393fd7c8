"""GPU parity of qmv_batch for the super-block types (Q5_K, Q6_K) against
the CPU oracle.

The pages' B9 group (FFN gate and up 2816 -> 5760 and the router 2816 -> 128
in Q5_K, one concurrent group of dispatches: gpu_full_attn.rs,
`encode_one_layer`, block B9) goes out as one launch: problems that share x
and K stream as one virtual matrix of row tiles. Ragged row counts, padded
row strides, problems with another x or K (separate launches), N = 0 and
K = 0 are covered. The batch picks its lane-group width for all rows
together, so its sums may be ordered differently from a single call's: both
are checked against the oracle, not against each other bit for bit.
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SINGLE = {"q5_k": qmv.qmv_q5_k, "q6_k": qmv.qmv_q6_k}

GROUPS = {
    # name: (K, [N or (N, row padding in bytes)])
    "b9_k2816": (2816, [5760, 5760, 128]),
    "ragged_k2816": (2816, [5, 300, 13, 1, 64, 7]),
    "padded_k4096": (4096, [(100, 2), (37, 6), (513, 0)]),
    "many_tiles_k256": (256, [20000, 8, 8, 3000]),
    "sixteen_k512": (512, [3 + 17 * i for i in range(16)]),
}


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
@pytest.mark.parametrize("group", sorted(GROUPS))
def test_kq_batch_shared_input(qtype, group):
    K, Ns = GROUPS[group]
    X = synth.make_x(1, K, cfg=91, part=K)
    xd = torch.from_numpy(X[0]).to(DEV)
    host, dev = [], []
    for i, N in enumerate(Ns):
        N, pad = N if isinstance(N, tuple) else (N, 0)
        W = synth.make_weights(qtype, N, K, cfg=91, part=i + 1, ldw=synth.row_bytes(qtype, K) + pad)
        host.append(W)
        dev.append((torch.from_numpy(W).to(DEV), xd, torch.full((N,), np.nan, device=DEV)))
    qmv.qmv_batch(qtype, dev)
    torch.cuda.synchronize()
    for i, (W, (Wd, _, y)) in enumerate(zip(host, dev)):
        yo, a = oracle.qmv(qtype, W, X)
        assert_within_tol(y.cpu().numpy()[None, :], yo, a, f"{qtype} {group} problem {i}")
        ys = torch.full((W.shape[0],), np.nan, device=DEV)
        SINGLE[qtype](Wd, xd, ys, K=K)
        torch.cuda.synchronize()
        assert_within_tol(ys.cpu().numpy()[None, :], yo, a, f"{qtype} {group} problem {i} (single call)")


def test_kq_batch_repeat_is_bitwise():
    K, Ns = GROUPS["b9_k2816"]
    X = synth.make_x(1, K, cfg=92)
    xd = torch.from_numpy(X[0]).to(DEV)
    dev = [(torch.from_numpy(synth.make_weights("q5_k", N, K, cfg=92, part=i)).to(DEV), xd,
            torch.empty(N, device=DEV)) for i, N in enumerate(Ns)]
    outs = []
    for _ in range(2):
        qmv.qmv_batch("q5_k", dev)
        torch.cuda.synchronize()
        outs.append([y.clone() for _, _, y in dev])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_kq_batch_mixed_inputs_and_empty_sums():
    """Problems on two different x (and K) and K = 0 in one call: the problems
    on the first x go out as one launch, the rest one by one."""
    specs = [(700, 2816, 0), (33, 2816, 0), (90, 1024, 1), (5, 0, 0), (128, 2816, 0)]
    xs = [synth.make_x(1, 2816, cfg=93, part=0), synth.make_x(1, 1024, cfg=93, part=1)]
    xds = [torch.from_numpy(x[0]).to(DEV) for x in xs]
    host, dev = [], []
    for i, (N, K, xi) in enumerate(specs):
        if K:
            W = synth.make_weights("q6_k", N, K, cfg=93, part=i + 2)
            xd = xds[xi]
        else:
            W = np.zeros((N, 210), np.uint8)
            xd = xds[0][:0]
        host.append((W, xs[xi], K))
        dev.append((torch.from_numpy(W).to(DEV), xd, torch.full((N,), np.nan, device=DEV)))
    qmv.qmv_batch("q6_k", dev)
    torch.cuda.synchronize()
    for i, ((W, X, K), (_, _, y)) in enumerate(zip(host, dev)):
        if K == 0:
            assert torch.all(y == 0), f"problem {i}: K = 0 must give zeros"
            continue
        yo, a = oracle.qmv("q6_k", W, X)
        assert_within_tol(y.cpu().numpy()[None, :], yo, a, f"mixed problem {i}")
