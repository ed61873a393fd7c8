"""The C-ABI library loads, exports what include/qmv.h declares, and rejects
bad arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from block_quantized_weight_qmatmul_amd import qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(qmv.LIB_PATH):
        from block_quantized_weight_qmatmul_amd import build
        build.build()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qmv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(qmv_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"qmv_q4_0", "qmv_q8_0", "qmv_q5_k", "qmv_q6_k", "qmv_gemm", "qmv_affine4", "qmv_affine4_id", "qmv_id", "qmv_id_swiglu", "qmv_moe_wsum", "qmv_moe_down",
            "qmv_batch", "qmv_ws", "qmv_ws_bytes", "qmv_last_error", "qmv_stream_read"} <= set(names)
    L = ctypes.CDLL(qmv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


# Fake, never dereferenced device addresses: every case below is rejected on
# the host before anything touches them.
W, X, Y = 0x10000000, 0x20000000, 0x30000000
Q4, Q8 = qmv.QMV_Q4_0, qmv.QMV_Q8_0


@pytest.mark.parametrize("args,status,msg", [
    ((Q4, W, 18 * 4, X, 128, Y, 16, 17, 16, 128), qmv.QMV_EUNSUPPORTED, "M=17"),
    ((Q4, W, 18 * 4, X, 128, Y, 16, -1, 16, 128), qmv.QMV_EUNSUPPORTED, "M=-1"),
    ((Q4, W, 18 * 4, X, 128, Y, 16, 1, -2, 128), qmv.QMV_EINVAL, "N=-2"),
    ((Q4, W, 18 * 4, X, 128, Y, 16, 1, 16, 100), qmv.QMV_EINVAL, "K=100"),
    ((Q4, 0, 18 * 4, X, 128, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "W is NULL"),
    ((Q4, W, 18 * 4, 0, 128, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "X is NULL"),
    ((Q4, W, 18 * 4, X, 128, 0, 16, 1, 16, 128), qmv.QMV_EINVAL, "Y is NULL"),
    ((Q4, W, 18 * 4 - 2, X, 128, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "ldw_bytes"),
    ((Q8, W, 18 * 4, X, 128, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "ldw_bytes"),
    ((Q4, W, 18 * 4 + 1, X, 128, Y, 16, 1, 16, 128), qmv.QMV_EALIGN, "2-byte"),
    ((Q4, W + 1, 18 * 4, X, 128, Y, 16, 1, 16, 128), qmv.QMV_EALIGN, "2-byte"),
    ((Q4, W, 18 * 4, X + 2, 128, Y, 16, 1, 16, 128), qmv.QMV_EALIGN, "4-byte"),
    ((Q4, W, 18 * 4, X, 127, Y, 16, 2, 16, 128), qmv.QMV_EINVAL, "ldx"),
    ((Q4, W, 18 * 4, X, 128, Y, 15, 2, 16, 128), qmv.QMV_EINVAL, "ldy"),
    ((Q4, W, 18 * 4, X, 128, W + 8, 16, 1, 16, 128), qmv.QMV_EINVAL, "overlaps"),
    ((Q4, W, 18 * 4, X, 128, X + 64, 16, 1, 16, 128), qmv.QMV_EINVAL, "overlaps"),
])
def test_dense_argument_checks(args, status, msg):
    q, *rest = args
    assert qmv.raw_qmv(q, *rest) == status
    assert msg in qmv.last_error()


WS = 0x50000000


@pytest.mark.parametrize("args,status,msg", [
    ((Q4, W, 18 * 160, X, 5120, Y, 1024, 16, 1024, 5120, WS, 1000), qmv.QMV_EINVAL, "workspace_bytes=1000"),
    ((Q4, W, 18 * 160, X, 5120, Y, 1024, 16, 1024, 5120, WS + 16, 1 << 26), qmv.QMV_EINVAL, "256-byte aligned"),
    ((Q4, W, 18 * 160, X, 5120, Y, 1024, 16, 1024, 5120, Y + 256, 1 << 26), qmv.QMV_EINVAL, "not overlap"),
    ((qmv.QMV_Q6_K, W, 18 * 160, X, 5120, Y, 1024, 16, 1024, 5120, WS, 1 << 26), qmv.QMV_EUNSUPPORTED, "qtype"),
    ((Q4, W, 18 * 160, X, 5120, Y, 1024, 17, 1024, 5120, WS, 1 << 26), qmv.QMV_EUNSUPPORTED, "M=17"),
])
def test_ws_argument_checks(args, status, msg):
    q, *rest = args
    assert qmv.raw_qmv_ws(q, *rest) == status
    assert msg in qmv.last_error()


def test_ws_bytes_query():
    """Partial sums of S K segments, S * M * N * 4 bytes, for calls with few
    output rows; 0 where the call does not split K."""
    n = qmv.ws_bytes("q4_0", 16, 1024, 5120)
    assert n > 0 and n % (16 * 1024 * 4) == 0 and n // (16 * 1024 * 4) <= 5120 // 256
    assert qmv.ws_bytes("q8_0", 16, 5120, 5120) % (16 * 5120 * 4) == 0
    assert qmv.ws_bytes("q4_0", 1, 1024, 5120) == 0          # M = 1
    assert qmv.ws_bytes("q4_0", 16, 1024, 5120 + 32) == 0     # K % 64 != 0 (generic kernel)
    assert qmv.ws_bytes("q6_k", 16, 1024, 5120) == 0
    assert qmv.ws_bytes("q4_0", 17, 1024, 5120) == 0


def test_empty_calls_are_no_ops_without_touching_memory():
    # M = 0 or N = 0: nothing to do, pointers may be NULL, no HIP call made.
    assert qmv.raw_qmv(Q4, 0, 0, 0, 0, 0, 0, 0, 16, 128) == qmv.QMV_OK
    assert qmv.raw_qmv(Q8, 0, 0, 0, 0, 0, 0, 1, 0, 128) == qmv.QMV_OK
    assert qmv.raw_qmv_id(Q4, 0, 0, 0, 4, 0, 0, 0, 0, 2, 0, 0, 16, 32) == qmv.QMV_OK


def _id(**kw):
    a = dict(qtype=Q4, W=W, es=18 * 16, ldw=18, E=4, X=X, ldx=32, ids=0x40000000, nt=1, k=2, Y=Y, ldy=16,
             N=16, K=32, sc=0, err=0)
    a.update(kw)
    return qmv.raw_qmv_id(a["qtype"], a["W"], a["es"], a["ldw"], a["E"], a["X"], a["ldx"], a["ids"], a["nt"],
                          a["k"], a["Y"], a["ldy"], a["N"], a["K"], a["sc"], a["err"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(qtype=3), qmv.QMV_EUNSUPPORTED, "qtype"),
    (dict(E=0), qmv.QMV_EINVAL, "n_experts"),
    (dict(k=0), qmv.QMV_EINVAL, "top_k"),
    (dict(k=4096), qmv.QMV_EUNSUPPORTED, "top_k"),
    (dict(nt=-1), qmv.QMV_EINVAL, "n_tokens"),
    (dict(K=48), qmv.QMV_EINVAL, "K=48"),
    (dict(ldw=16), qmv.QMV_EINVAL, "ldw_bytes"),
    (dict(es=18 * 15), qmv.QMV_EINVAL, "expert_stride"),
    (dict(ldx=31), qmv.QMV_EINVAL, "ldx"),
    (dict(ldy=15), qmv.QMV_EINVAL, "ldy"),
    (dict(ids=0), qmv.QMV_EINVAL, "NULL"),
    (dict(es=18 * 16 + 1), qmv.QMV_EALIGN, "2-byte"),
    (dict(ids=0x40000002), qmv.QMV_EALIGN, "4-byte"),
    (dict(err=0x50000001), qmv.QMV_EALIGN, "4-byte"),
    (dict(Y=W + 18 * 20), qmv.QMV_EINVAL, "overlaps"),
    (dict(Y=0x40000000 - 4), qmv.QMV_EINVAL, "overlaps"),
    (dict(qtype=qmv.QMV_Q6_K), qmv.QMV_EINVAL, "multiple of 256"),
    (dict(qtype=qmv.QMV_Q6_K, K=256, ldw=208, es=210 * 16, ldx=256), qmv.QMV_EINVAL, "ldw_bytes"),
    (dict(qtype=qmv.QMV_Q6_K, K=16640, ldw=210 * 65, es=210 * 65 * 16, ldx=16640), qmv.QMV_EUNSUPPORTED, "Q6_K"),
])
def test_id_argument_checks(kw, status, msg):
    assert _id(**kw) == status
    assert msg in qmv.last_error()


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(qmv, "_lib", None)
    monkeypatch.setattr(qmv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        qmv.lib()


def _bp(**kw):
    d = dict(W=W, ldw=18 * 4, x=X, y=Y, N=16, K=128)
    d.update(kw)
    return (d["W"], d["ldw"], d["x"], d["y"], d["N"], d["K"])


@pytest.mark.parametrize("probs,status,msg", [
    ([_bp(K=100)], qmv.QMV_EINVAL, "K=100"),
    ([_bp(N=-1)], qmv.QMV_EINVAL, "N=-1"),
    ([_bp(), _bp(ldw=18 * 3, y=Y + 4096)], qmv.QMV_EINVAL, "problem 1: ldw_bytes"),
    ([_bp(W=W + 1)], qmv.QMV_EALIGN, "2-byte"),
    ([_bp(y=Y + 2)], qmv.QMV_EALIGN, "4-byte"),
    ([_bp(x=0)], qmv.QMV_EINVAL, "NULL"),
    ([_bp(), _bp(y=Y + 32)], qmv.QMV_EINVAL, "overlaps"),          # two outputs overlap
    ([_bp(), _bp(W=Y - 8, y=Y + 4096)], qmv.QMV_EINVAL, "overlaps"),  # output 0 overlaps W of problem 1
    ([_bp()] * 17, qmv.QMV_EINVAL, "n_problems"),
])
def test_batch_argument_checks(probs, status, msg):
    assert qmv.raw_qmv_batch(Q4, probs) == status
    assert msg in qmv.last_error()


@pytest.mark.parametrize("probs,status,msg", [
    ([_bp(K=128, ldw=176)], qmv.QMV_EINVAL, "multiple of 256"),
    ([_bp(K=16640, ldw=176 * 65)], qmv.QMV_EUNSUPPORTED, "exceeds"),
    ([_bp(K=512, ldw=176 * 2 - 2)], qmv.QMV_EINVAL, "ldw_bytes"),
    ([_bp(K=512, ldw=176 * 2 + 1)], qmv.QMV_EALIGN, "2-byte"),
])
def test_batch_super_block_argument_checks(probs, status, msg):
    """Q5_K batches: K a multiple of 256 up to 16384, rows of K/256 super-blocks."""
    assert qmv.raw_qmv_batch(qmv.QMV_Q5_K, probs) == status
    assert msg in qmv.last_error()


def test_batch_bad_qtype_and_empty():
    assert qmv.raw_qmv_batch(5, [_bp()]) == qmv.QMV_EUNSUPPORTED
    assert qmv.raw_qmv_batch(Q4, []) == qmv.QMV_OK
    assert qmv.raw_qmv_batch(Q8, [_bp(N=0, W=0, x=0, ldw=34 * 4)]) == qmv.QMV_OK  # N = 0: nothing to launch


def _sw(**kw):
    a = dict(qtype=Q4, W=W, es=18 * 16, ldw=18, E=4, G=X, ldg=64, ids=0x40000000, nt=1, k=2, Y=Y, ldy=16,
             N=16, K=32, sc=0, err=0)
    a.update(kw)
    return qmv.raw_qmv_id_swiglu(a["qtype"], a["W"], a["es"], a["ldw"], a["E"], a["G"], a["ldg"], a["ids"], a["nt"],
                                 a["k"], a["Y"], a["ldy"], a["N"], a["K"], a["sc"], a["err"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(ldg=63), qmv.QMV_EINVAL, "qmv_id_swiglu: ldx=63 < 2K=64"),
    (dict(qtype=3), qmv.QMV_EUNSUPPORTED, "qmv_id_swiglu: qtype"),
    (dict(G=X + 2), qmv.QMV_EALIGN, "4-byte"),
    (dict(Y=X + 4 * 60), qmv.QMV_EINVAL, "overlaps"),  # Y inside G's second half
    (dict(K=48), qmv.QMV_EINVAL, "K=48"),
    (dict(qtype=qmv.QMV_Q6_K, K=256, ldw=210, es=210 * 16, ldg=512), qmv.QMV_EUNSUPPORTED, "qtype 14"),
])
def test_id_swiglu_argument_checks(kw, status, msg):
    assert _sw(**kw) == status
    assert msg in qmv.last_error()


def _ws(**kw):
    a = dict(Y=Y, ldy=16, w=0x40000000, nt=2, k=4, N=16, out=0x50000000, ldo=16)
    a.update(kw)
    return qmv.raw_qmv_moe_wsum(a["Y"], a["ldy"], a["w"], a["nt"], a["k"], a["N"], a["out"], a["ldo"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(k=0), qmv.QMV_EINVAL, "top_k"),
    (dict(nt=-1), qmv.QMV_EINVAL, "n_tokens"),
    (dict(N=-1), qmv.QMV_EINVAL, "N=-1"),
    (dict(ldy=15), qmv.QMV_EINVAL, "ldy"),
    (dict(ldo=15), qmv.QMV_EINVAL, "ldo"),
    (dict(w=0), qmv.QMV_EINVAL, "NULL"),
    (dict(out=Y + 4 * 16 * 7), qmv.QMV_EINVAL, "overlaps"),  # out starts in Y's last row
    (dict(out=0x50000002), qmv.QMV_EALIGN, "4-byte"),
])
def test_moe_wsum_argument_checks(kw, status, msg):
    assert _ws(**kw) == status
    assert msg in qmv.last_error()


def _md(**kw):
    a = dict(qtype=Q4, W=W, es=36 * 16, ldw=36, E=4, G=X, ldg=128, ids=0x40000000, w=0x48000000, nt=1, k=8,
             out=Y, ldo=16, N=16, K=64, sc=0, err=0)
    a.update(kw)
    return qmv.raw_qmv_moe_down(a["qtype"], a["W"], a["es"], a["ldw"], a["E"], a["G"], a["ldg"], a["ids"], a["w"],
                                a["nt"], a["k"], a["out"], a["ldo"], a["N"], a["K"], a["sc"], a["err"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(qtype=3), qmv.QMV_EUNSUPPORTED, "qtype"),
    (dict(K=32, ldw=18, es=18 * 16, ldg=64), qmv.QMV_EUNSUPPORTED, "K % 64"),
    (dict(K=0), qmv.QMV_EUNSUPPORTED, "K=0"),
    (dict(k=65), qmv.QMV_EUNSUPPORTED, "staging limit"),
    (dict(k=16, K=1024, ldw=18 * 32, es=18 * 32 * 16, ldg=2048), qmv.QMV_EUNSUPPORTED, "staging limit"),
    (dict(ldg=127), qmv.QMV_EINVAL, "ldg"),
    (dict(ldo=15), qmv.QMV_EINVAL, "ldo"),
    (dict(w=0), qmv.QMV_EINVAL, "NULL"),
    (dict(es=36 * 15), qmv.QMV_EINVAL, "expert_stride"),
    (dict(ldw=38, es=38 * 16), qmv.QMV_EUNSUPPORTED, "4-byte aligned W"),
    (dict(w=0x48000002), qmv.QMV_EALIGN, "4-byte"),
    (dict(out=X + 4 * 100), qmv.QMV_EINVAL, "overlaps"),
])
def test_moe_down_argument_checks(kw, status, msg):
    assert _md(**kw) == status
    assert msg in qmv.last_error()


def test_moe_empty_calls_are_no_ops():
    assert qmv.raw_qmv_moe_wsum(0, 0, 0, 0, 8, 16, 0, 0) == qmv.QMV_OK
    assert qmv.raw_qmv_moe_down(Q4, 0, 0, 0, 4, 0, 0, 0, 0, 0, 8, 0, 0, 16, 64) == qmv.QMV_OK
    assert qmv.raw_qmv_id_swiglu(Q4, 0, 0, 0, 4, 0, 0, 0, 0, 2, 0, 0, 16, 32) == qmv.QMV_OK


Q6 = qmv.QMV_Q6_K


@pytest.mark.parametrize("args,status,msg", [
    ((Q6, W, 210, X, 256, Y, 16, 17, 16, 256), qmv.QMV_EUNSUPPORTED, "M=17"),
    ((Q6, W, 210, X, 256, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "multiple of 256"),
    ((Q6, W, 208, X, 256, Y, 16, 1, 16, 256), qmv.QMV_EINVAL, "ldw_bytes"),
    ((Q6, W, 211, X, 256, Y, 16, 1, 16, 256), qmv.QMV_EALIGN, "2-byte"),
    ((Q6, W + 1, 210, X, 256, Y, 16, 1, 16, 256), qmv.QMV_EALIGN, "2-byte"),
    ((Q6, W, 210 * 64, X, 16384, Y, 16, 1, 16, 16640), qmv.QMV_EUNSUPPORTED, "exceeds"),
    ((Q6, W, 210, X, 256, W + 8, 16, 1, 16, 256), qmv.QMV_EINVAL, "overlaps"),
    ((Q6, W, 210, X, 255, Y, 16, 2, 16, 256), qmv.QMV_EINVAL, "ldx"),
])
def test_q6k_argument_checks(args, status, msg):
    q, *rest = args
    assert qmv.raw_qmv(q, *rest) == status
    assert msg in qmv.last_error()


Q5 = qmv.QMV_Q5_K


@pytest.mark.parametrize("args,status,msg", [
    ((Q5, W, 176, X, 256, Y, 16, 1, 16, 128), qmv.QMV_EINVAL, "multiple of 256"),
    ((Q5, W, 174, X, 256, Y, 16, 1, 16, 256), qmv.QMV_EINVAL, "K/256*176"),
    ((Q5, W + 1, 176, X, 256, Y, 16, 1, 16, 256), qmv.QMV_EALIGN, "2-byte"),
    ((Q5, W, 176, X, 256, W + 8, 16, 1, 16, 256), qmv.QMV_EINVAL, "overlaps"),
    ((Q5, W, 176 * 65, X, 16640, Y, 16, 1, 16, 16640), qmv.QMV_EUNSUPPORTED, "exceeds"),
])
def test_q5k_argument_checks(args, status, msg):
    q, *rest = args
    assert qmv.raw_qmv(q, *rest) == status
    assert msg in qmv.last_error()


@pytest.mark.parametrize("args,status,msg", [
    ((5, W, 18 * 4, X, 128, Y, 16, 40, 16, 128), qmv.QMV_EUNSUPPORTED, "qtype"),
    ((Q4, W, 18 * 4, X, 128, Y, 16, -1, 16, 128), qmv.QMV_EINVAL, "M=-1"),
    ((Q4, W, 18 * 4, X, 127, Y, 16, 40, 16, 128), qmv.QMV_EINVAL, "ldx"),
    ((Q4, W, 18 * 4, X, 128, Y, 15, 40, 16, 128), qmv.QMV_EINVAL, "ldy"),
    ((Q4, W, 18 * 4, X, 128, X + 4 * 128 * 39, 16, 40, 16, 128), qmv.QMV_EINVAL, "overlaps"),
    ((qmv.QMV_Q6_K, W, 210, X, 256, Y, 16, 40, 16, 128), qmv.QMV_EINVAL, "multiple of 256"),
])
def test_gemm_argument_checks(args, status, msg):
    assert qmv.raw_qmv_gemm(*args) == status
    assert msg in qmv.last_error()


def test_gemm_empty_is_a_no_op():
    assert qmv.raw_qmv_gemm(Q4, 0, 0, 0, 0, 0, 0, 0, 16, 128) == qmv.QMV_OK


def _a4(**kw):
    a = dict(Wq=W, ldw=88, S=X, B=X + 4096, lds=22, X=Y, ldx=704, Y=0x40000000, ldy=16, M=1, N=16, K=704)
    a.update(kw)
    return qmv.raw_qmv_affine4(a["Wq"], a["ldw"], a["S"], a["B"], a["lds"], a["X"], a["ldx"], a["Y"], a["ldy"],
                               a["M"], a["N"], a["K"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=700), qmv.QMV_EINVAL, "multiple of 32"),
    (dict(ldw=87), qmv.QMV_EINVAL, "ldw"),
    (dict(lds=21), qmv.QMV_EINVAL, "lds"),
    (dict(M=17), qmv.QMV_EUNSUPPORTED, "M=17"),
    (dict(K=16416, ldw=2052, lds=513, ldx=16416), qmv.QMV_EUNSUPPORTED, "exceeds"),
    (dict(Wq=W + 2), qmv.QMV_EALIGN, "aligned"),
    (dict(S=X + 1), qmv.QMV_EALIGN, "aligned"),
    (dict(Y=X + 8), qmv.QMV_EINVAL, "overlaps"),
    (dict(B=0), qmv.QMV_EINVAL, "NULL"),
])
def test_affine4_argument_checks(kw, status, msg):
    assert _a4(**kw) == status
    assert msg in qmv.last_error()


@pytest.mark.parametrize("args,status,msg", [
    ((0, 4096, 64), qmv.QMV_EINVAL, "NULL src"),
    ((64, 4096, 0), qmv.QMV_EINVAL, "NULL src or sink"),
    ((72, 4096, 64), qmv.QMV_EALIGN, "16-byte aligned"),
    ((64, 4100, 64), qmv.QMV_EALIGN, "16-byte aligned"),
    ((64, 4096, 66), qmv.QMV_EALIGN, "sink 4-byte aligned"),
])
def test_stream_read_argument_checks(args, status, msg):
    assert qmv.raw_stream_read(*args) == status
    assert msg in qmv.last_error()


def test_stream_read_empty_is_a_no_op():
    assert qmv.raw_stream_read(0, 0, 0) == qmv.QMV_OK
