"""GPU parity of qmv_q4_0 / qmv_q8_0 against the CPU oracle (needs an MI355X).

Every comparison is element by element at |gpu - oracle| <= 1e-4 * a + 1e-6
(a = sum_k |w_k x_k| from the oracle), or bit-exact where the exact result is
representable (one-hot and identity activations, all-zero weights).
"""
import numpy as np
import pytest

import oracle
from block_quantized_weight_qmatmul_amd import qmv, synth
from golden_io import read_blocks
from helpers import assert_within_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FN = {"q4_0": qmv.qmv_q4_0, "q8_0": qmv.qmv_q8_0}


def run(qtype, W, X, K=None, ldy=None, y_fill=np.nan):
    """Run the GPU kernel on host arrays W [N, ldw] uint8 and X [M, K] fp32."""
    Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    M, N = X.shape[0], W.shape[0]
    Yfull = torch.full((M, ldy or N), y_fill, dtype=torch.float32, device=DEV)
    Y = Yfull[:, :N]
    FN[qtype](Wd, Xd, Y, K=K)
    torch.cuda.synchronize()
    return Yfull.cpu().numpy()[:, :N], Yfull.cpu().numpy()


def check(qtype, W, X, what, rows=None):
    y, _ = run(qtype, W, X)
    if rows is None:
        yo, a = oracle.qmv(qtype, W, X)
        return assert_within_tol(y, yo, a, what)
    yo, a = oracle.qmv(qtype, W[rows], X)
    return assert_within_tol(y[:, rows], yo, a, what)


# --------------------------------------------------------------------------
# The workloads at full size.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_m1_workloads_full_size(cfg):
    for part, p in enumerate(synth.CONFIGS[cfg]["problems"]):
        W, X = synth.dense_inputs(cfg, p, part)
        print(f"cfg{cfg} {p.name} {p.qtype} M={p.M} N={p.N} K={p.K}", flush=True)
        r = check(p.qtype, W, X, f"cfg{cfg}/{p.name}")
        print(f"  max ratio {r:.3g}")


def test_m16_workload_full():
    """Config 3 (M = 16, K = 5120, N = 5120 / 1024 / 27648): every output
    element against the oracle."""
    cfg = 3
    for part, p in enumerate(synth.CONFIGS[cfg]["problems"]):
        W, X = synth.dense_inputs(cfg, p, part)
        print(f"cfg3 {p.name} M={p.M} N={p.N} K={p.K}", flush=True)
        r = check(p.qtype, W, X, f"cfg3/{p.name}")
        print(f"  max ratio {r:.3g}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_m16_rows_match_m1_kernel(qtype):
    """Each row of an M = 16 product matches the M = 1 kernel's output for
    that activation row within the tolerance (a from the oracle), on the
    config 3 shapes (Q8_0: the same shapes with 34-byte blocks)."""
    cfg = 3
    for part, p in enumerate(synth.CONFIGS[cfg]["problems"]):
        W = synth.make_weights(qtype, p.N, p.K, cfg=cfg, part=part) if qtype == "q8_0" else \
            synth.dense_inputs(cfg, p, part)[0]
        X = synth.dense_inputs(cfg, p, part)[1]
        y16, _ = run(qtype, W, X)
        Wd = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
        y1 = np.empty_like(y16)
        for m in range(p.M):
            Y1 = torch.full((1, p.N), np.nan, dtype=torch.float32, device=DEV)
            FN[qtype](Wd, torch.from_numpy(np.ascontiguousarray(X[m:m + 1])).to(DEV), Y1)
            torch.cuda.synchronize()
            y1[m] = Y1.cpu().numpy()[0]
        _, a = oracle.qmv(qtype, W, X)
        r = assert_within_tol(y16, y1.astype(np.float64), a, f"{qtype} cfg3/{p.name}: M=16 vs M=1")
        print(f"{qtype} {p.name}: max |M=16 - M=1| / tol = {r:.3g}")


# --------------------------------------------------------------------------
# Exact cases.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fixture,qtype", [("q4_0_blocks.txt", "q4_0"), ("q8_0_blocks.txt", "q8_0")])
@pytest.mark.parametrize("nblk", [1, 2, 64])
def test_one_hot_is_bit_exact(fixture, qtype, nblk):
    """Rows of hand-built blocks; x = e_k picks w[n, k] exactly (K = 32*nblk,
    so both the generic (K=32) and the fast (K % 64 == 0) kernels are hit)."""
    blocks = read_blocks(fixture)
    rows = [np.concatenate([raw] * nblk) for _, raw, _ in blocks]
    want = np.stack([np.tile(v, nblk) for _, _, v in blocks])
    W = np.stack(rows)
    K = 32 * nblk
    for k in sorted({0, 1, 15, 16, 17, 31, K - 1, K // 2 + 3}):
        X = np.zeros((1, K), dtype=np.float32)
        X[0, k] = 1.0
        y, _ = run(qtype, W, X)
        assert np.array_equal(y[0], want[:, k].astype(np.float32)), (k, y[0], want[:, k])


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_identity_rows_m16_bit_exact(qtype):
    N, K = 40, 256
    W = synth.make_weights(qtype, N, K, cfg=90)
    M, k0 = 16, 37
    X = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        X[m, k0 + m] = 1.0
    y, _ = run(qtype, W, X)
    deq = np.stack([oracle.dequant_row(qtype, W[n], K) for n in range(N)])
    for m in range(M):
        assert np.array_equal(y[m], deq[:, k0 + m].astype(np.float32))


@pytest.mark.parametrize("K", [2048, 4096, 96])
def test_all_codes_eight_give_exact_zero(K):
    W = synth.make_weights("q4_0", 300, K, cfg=91)
    W.reshape(300, -1, 18)[:, :, 2:] = 0x88
    X = synth.make_x(1, K, cfg=91) * np.float32(1e4)
    y, _ = run("q4_0", W, X)
    assert np.all(y == 0)


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_deterministic_bitwise(qtype):
    W, X = synth.dense_inputs(1, synth.Dense("gate", qtype, 1, 14336, 4096), part=4)
    y1, _ = run(qtype, W, X)
    y2, _ = run(qtype, W, X)
    assert np.array_equal(y1, y2)


# --------------------------------------------------------------------------
# Ragged, strided, misaligned and boundary shapes (fast and generic kernels).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("N,K", [(1, 64), (3, 32), (17, 96), (1000, 2080), (4097, 128), (257, 704),
                                 (63, 2816), (129, 15360), (65, 16384), (5, 30720)])
def test_ragged_shapes(qtype, N, K):
    W = synth.make_weights(qtype, N, K, cfg=92, part=N)
    X = synth.make_x(1, K, cfg=92, part=K)
    check(qtype, W, X, f"{qtype} N={N} K={K}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("N,K", [(32768, 1024), (33001, 2816), (40000, 8192)])
def test_m1_large_matrices_narrow_lane_groups(qtype, N, K):
    """Large M = 1 calls take 16 lanes per row (N >= 32768, 1024 <= K <= 8192);
    a ragged last tile included."""
    W = synth.make_weights(qtype, N, K, cfg=96, part=N % 97)
    X = synth.make_x(1, K, cfg=96, part=K)
    check(qtype, W, X, f"{qtype} N={N} K={K}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("pad", [2, 4, 64])
def test_padded_row_stride(qtype, pad):
    N, K = 515, 1024
    ldw = synth.row_bytes(qtype, K) + pad
    W = synth.make_weights(qtype, N, K, cfg=93, ldw=ldw)
    X = synth.make_x(1, K, cfg=93)
    check(qtype, W, X, f"{qtype} pad={pad}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_weights_at_2_byte_offset(qtype):
    N, K = 300, 512
    W = synth.make_weights(qtype, N, K, cfg=94)
    X = synth.make_x(1, K, cfg=94)
    buf = torch.zeros(W.size + 64, dtype=torch.uint8, device=DEV)
    Wd = buf[2:2 + W.size].view(N, -1)
    Wd.copy_(torch.from_numpy(W))
    Y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    FN[qtype](Wd, torch.from_numpy(X).to(DEV), Y)
    torch.cuda.synchronize()
    yo, a = oracle.qmv(qtype, W, X)
    assert_within_tol(Y.cpu().numpy(), yo, a, "offset 2")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [2, 3, 7, 16])
def test_multi_row_x_with_strides(qtype, M):
    N, K = 777, 1536
    W = synth.make_weights(qtype, N, K, cfg=95, part=M)
    Xfull = synth.make_x(M, K + 40, cfg=95, part=M)
    Xd = torch.from_numpy(Xfull).to(DEV)[:, 8:8 + K]
    Yfull = torch.full((M, N + 9), np.nan, dtype=torch.float32, device=DEV)
    FN[qtype](torch.from_numpy(W).to(DEV), Xd, Yfull[:, :N])
    torch.cuda.synchronize()
    y = Yfull.cpu().numpy()
    yo, a = oracle.qmv(qtype, W, np.ascontiguousarray(Xfull[:, 8:8 + K]))
    assert_within_tol(y[:, :N], yo, a, f"M={M}")
    assert np.all(np.isnan(y[:, N:]))  # the row padding of Y is left alone


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [5, 16])
@pytest.mark.parametrize("N,K", [(64, 5120), (4100, 2112), (300, 1088), (27, 64), (16400, 704), (65552, 256)])
def test_multi_row_launch_shapes_and_ragged_steps(qtype, M, N, K):
    """M >= 2 on the matrix cores: few tiles (K split over 4 or 2 waves of a
    tile), many tiles (one wave per tile, workgroups of 4 and 8 waves), K not
    a multiple of the 256-column step, N not a multiple of 16."""
    W = synth.make_weights(qtype, N, K, cfg=94, part=M)
    X = synth.make_x(M, K, cfg=94, part=M)
    check(qtype, W, X, f"{qtype} M={M} N={N} K={K}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_multi_row_dynamic_range(qtype):
    """Activations spanning e^-60..e^60 (about 2^-87..2^87), a different
    scale in every row and every 512 columns."""
    M, N, K = 16, 384, 3072
    W = synth.make_weights(qtype, N, K, cfg=93)
    r = np.random.default_rng(93)
    X = synth.make_x(M, K, cfg=93) * np.exp(r.uniform(-40, 40, (M, K)))
    X *= np.exp(r.uniform(-20, 20, (M, K // 512, 1))).repeat(512, axis=2).reshape(M, K)
    check(qtype, W, X.astype(np.float32), "dynamic range M=16")


@pytest.mark.parametrize("outlier", [1e9, 1e10, 1e30, 3.3e38])
def test_multi_row_outlier_on_a_zero_weight(outlier):
    """One huge activation on a column whose weights are all exactly zero
    (code 8): the other columns must keep their full precision, so the
    result meets the tolerance built from the small terms alone."""
    M, N, K = 16, 96, 2048
    W = synth.make_weights("q4_0", N, K, cfg=88)
    col = 517
    blk = W.reshape(N, K // 32, 18)
    q = blk[:, col // 32, 2 + (col % 32) % 16]
    blk[:, col // 32, 2 + (col % 32) % 16] = (q & 0x0F) | 0x80 if col % 32 >= 16 else (q & 0xF0) | 0x08
    X = synth.make_x(M, K, cfg=88)
    X[:, col] = np.float32(outlier)
    X[3, col + 1] = np.float32(outlier)  # one row also has it on a nonzero weight
    r = check("q4_0", W, X, f"outlier {outlier:g}")
    print(f"outlier {outlier:g}: max ratio {r:.3g}")


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M", [1, 16])
def test_non_finite_activations_propagate(qtype, M):
    """x = +inf at one column: y is +-inf where that column's weight is
    nonzero (sign of the weight) and NaN where it is zero (0 * inf); a NaN in
    x makes its row NaN; in Q4_0 a finite x beyond the largest bf16 (3.39e38)
    is an ordinary value (in Q8_0 the unscaled block sum, up to 127 |x|,
    would leave the fp32 range: the stated limit is |x| < 2^116)."""
    N, K = 200, 1024
    W = synth.make_weights(qtype, N, K, cfg=87)
    deq = np.stack([oracle.dequant_row(qtype, W[n], K) for n in range(N)])
    X = synth.make_x(M, K, cfg=87) * np.float32(1e-3)
    k_inf = 300
    X[0, k_inf] = np.inf
    if M > 1:
        X[1, 5] = np.nan
        if qtype == "q4_0":
            X[2, 700] = np.float32(3.395e38)
            X[3, 701] = np.float32(-3.4e38)
        else:
            X[2, 700] = np.float32(2.0**115)
            X[3, 701] = np.float32(-(2.0**115))
    y, _ = run(qtype, W, X)
    w = deq[:, k_inf]
    assert np.array_equal(np.isnan(y[0]), w == 0), "NaN exactly where the weight is zero"
    nz = w != 0
    assert np.all(np.isinf(y[0][nz])) and np.array_equal(np.sign(y[0][nz]), np.sign(w[nz]))
    if M > 1:
        assert np.all(np.isnan(y[1]))
        rows = [m for m in range(M) if m not in (0, 1)]
        yo, a = oracle.qmv(qtype, W, X[rows])
        assert_within_tol(y[rows], yo, a, f"{qtype} finite rows")


def test_multi_row_deterministic_bitwise():
    M, N, K = 16, 200, 5120  # K split over the waves of a tile
    W = synth.make_weights("q4_0", N, K, cfg=92)
    X = synth.make_x(M, K, cfg=92)
    y1, _ = run("q4_0", W, X)
    y2, _ = run("q4_0", W, X)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_k_zero_writes_zeros_and_empty_calls_do_nothing():
    Y = torch.full((3, 10), 7.0, dtype=torch.float32, device=DEV)
    W = torch.zeros((10, 2), dtype=torch.uint8, device=DEV)
    X = torch.zeros((3, 4), dtype=torch.float32, device=DEV)
    qmv.qmv_q4_0(W, X, Y, K=0)
    torch.cuda.synchronize()
    assert torch.all(Y == 0)
    Y.fill_(7.0)
    qmv.qmv_q8_0(W[:0], X, Y[:, :0], K=0)  # N = 0
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0)


def test_large_dynamic_range_activations():
    N, K = 512, 4096
    W = synth.make_weights("q4_0", N, K, cfg=89)
    r = np.random.default_rng(89)
    X = (synth.make_x(1, K, cfg=89) * np.exp(r.uniform(-40, 40, K))).astype(np.float32)
    check("q4_0", W, X, "dynamic range")


# --------------------------------------------------------------------------
# Batched launch (qmv_batch).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
def test_batch_decode_layer_set_against_oracle(qtype):
    """The decode-layer projection set as one batch; Q, K and V share x."""
    probs = synth.CONFIGS[1]["problems"]
    host, dev = [], []
    xq = synth.make_x(1, 4096, cfg=1, part=0)
    for part, p in enumerate(probs):
        W = synth.make_weights(qtype, p.N, p.K, cfg=1, part=part)
        X = xq if p.name in ("q", "k", "v") else synth.make_x(1, p.K, cfg=1, part=part)
        host.append((W, X))
    xs_dev = {}
    for W, X in host:
        key = id(X)
        if key not in xs_dev:
            xs_dev[key] = torch.from_numpy(X[0]).to(DEV)
        dev.append((torch.from_numpy(W).to(DEV), xs_dev[key], torch.full((W.shape[0],), np.nan, device=DEV)))
    qmv.qmv_batch(qtype, dev)
    torch.cuda.synchronize()
    for (W, X), (_, _, y), p in zip(host, dev, probs):
        yo, a = oracle.qmv(qtype, W, X)
        assert_within_tol(y.cpu().numpy()[None, :], yo, a, f"batch {p.name}")


SHARED_GROUPS = {
    # name: (K, [N per problem]) -- every problem of a group reads one x
    "qkv_h4096": (4096, [4096, 1024, 1024]),
    "gate_up_h4096": (4096, [14336, 14336]),
    "ragged_k2816": (2816, [5, 300, 13, 1, 64, 7]),
    "sixteen_k704": (704, [3 + 17 * i for i in range(16)]),
    "down_k14336": (14336, [1000, 24]),
    # row strides padded by 12 bytes (4-byte aligned) and by 2 bytes (the
    # second problem then takes the generic kernel, the others the fast one)
    "padded_k4096": (4096, [(100, 12), (37, 2), (513, 0)]),
    # more 8-row tiles (1027) than workgroups: a workgroup's stride jumps
    # from the second problem over the three one-tile problems to the last
    "stride_skips_k4096": (4096, [4096, 8, 8, 8, 4096]),
}


@pytest.mark.parametrize("qtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("group", sorted(SHARED_GROUPS))
def test_batch_shared_input_groups(qtype, group):
    """Problems that share one x (a layer's Q/K/V, its gate/up) stream as one
    virtual matrix of row tiles; ragged row counts end tiles early, a tile
    never spans two problems."""
    K, Ns = SHARED_GROUPS[group]
    X = synth.make_x(1, K, cfg=81, part=0)
    xd = torch.from_numpy(X[0]).to(DEV)
    host, dev = [], []
    for i, N in enumerate(Ns):
        N, pad = N if isinstance(N, tuple) else (N, 0)
        W = synth.make_weights(qtype, N, K, cfg=81, part=i + 1, ldw=synth.row_bytes(qtype, K) + pad)
        host.append(W)
        dev.append((torch.from_numpy(W).to(DEV), xd, torch.full((N,), np.nan, device=DEV)))
    qmv.qmv_batch(qtype, dev)
    torch.cuda.synchronize()
    for i, (W, (_, _, y)) in enumerate(zip(host, dev)):
        yo, a = oracle.qmv(qtype, W, X)
        assert_within_tol(y.cpu().numpy()[None, :], yo, a, f"{group} problem {i}")
        # the same rows through the single-problem call, bit for bit
        ys = torch.full((W.shape[0],), np.nan, device=DEV)
        FN[qtype](dev[i][0], xd[None, :], ys[None, :])
        torch.cuda.synchronize()
        assert torch.equal(ys, y), f"{group} problem {i}: batch differs from the single call"


def test_batch_mixed_fast_and_fallback_problems():
    """Problems the fast kernel takes and ones it does not (odd blocks per
    row, 2-byte row stride, K = 0) in one call."""
    specs = [(300, 4096, None), (7, 96, None), (129, 1024, synth.row_bytes("q4_0", 1024) + 2), (64, 2816, None),
             (5, 0, 18)]
    host, dev = [], []
    for i, (N, K, ldw) in enumerate(specs):
        if K:
            W = synth.make_weights("q4_0", N, K, cfg=79, part=i, ldw=ldw)
            X = synth.make_x(1, K, cfg=79, part=i)
        else:
            W = np.zeros((N, ldw), np.uint8)
            X = np.zeros((1, 4), np.float32)
        host.append((W, X, K))
        dev.append((torch.from_numpy(W).to(DEV), torch.from_numpy(X[0]).to(DEV)[:K] if K else torch.from_numpy(X[0]).to(DEV)[:0],
                    torch.full((N,), np.nan, device=DEV)))
    qmv.qmv_batch("q4_0", dev)
    torch.cuda.synchronize()
    for (W, X, K), (_, _, y) in zip(host, dev):
        if K == 0:
            assert torch.all(y == 0)
            continue
        yo, a = oracle.qmv("q4_0", W, X)
        assert_within_tol(y.cpu().numpy()[None, :], yo, a, f"mixed K={K}")
