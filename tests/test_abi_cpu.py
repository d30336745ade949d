"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/q4k.h declares, and rejects invalid arguments on the host with the
documented status codes before anything is launched.

Every call below fails a host-side check, so no device pointer is ever
dereferenced; the fake addresses are never touched."""
import ctypes
import os
import re

import pytest

import gemm_q4_super_amd as q4k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EALIGN, ESHAPE, EWORKSPACE = 0, -1, -2, -3, -4
A = 0x10000          # a 256-byte aligned fake address (never dereferenced)


def _declared():
    src = open(os.path.join(ROOT, "include", "q4k.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q[46]k_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return q4k.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared()
    assert set(declared) == set(q4k.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_int8_gemm_library_exports_the_same_calls():
    """libq4k_gemm_int8.so (the GEMM's int8 contraction) is the same library
    apart from the GEMM object: same entry points, same host checks."""
    L8 = q4k.lib_gemm_int8()
    for name in _declared():
        assert hasattr(L8, name), name
    P = q4k._lib.GemmProblem
    arr = (P * 1)(P(A, A, 16))
    need = L8.q4k_gemm_workspace_bytes()
    assert need == q4k.lib().q4k_gemm_workspace_bytes()
    assert L8.q4k_gemm(None, 16, 512, A, A, A, 16, A, None, 0, None) == EINVAL
    assert L8.q4k_gemm_batch(arr, 1, 500, A, A, A, 16, None, 0, None) == ESHAPE
    assert L8.q4k_gemm_batch(arr, 1, 512, A, A, A, 16, A, need - 1, None) == EWORKSPACE


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert q4k.q4k_status_string(st) != "unknown status"
    assert q4k.q4k_status_string(7) == "unknown status"


def test_gemv_gemm_argument_checks(L):
    for gemm in (False, True):
        good = dict(w=A, N=16, K=512, codes=A, scales=A, sums=A, M=1, y=A)

        def call(**kw):
            a = dict(good, **kw)
            args = (a["w"], a["N"], a["K"], a["codes"], a["scales"], a["sums"], a["M"], a["y"])
            if gemm:
                return L.q4k_gemm(*args, None, 0, None)
            return L.q4k_gemv(*args, None)
        assert call(w=None) == EINVAL
        assert call(codes=None) == EINVAL
        assert call(y=None) == EINVAL
        assert call(K=100) == ESHAPE
        assert call(K=0) == ESHAPE
        assert call(K=288) == ESHAPE
        assert call(N=0) == ESHAPE
        assert call(M=0) == ESHAPE
        assert call(N=1 << 25) == ESHAPE
        assert call(w=A + 8) == EALIGN
        assert call(codes=A + 4) == EALIGN
        assert call(y=A + 2) == EALIGN
    # the GEMV takes at most 8 activation rows
    assert L.q4k_gemv(A, 16, 512, A, A, A, 9, A, None) == ESHAPE


def test_q6k_gemv_argument_checks(L):
    f = L.q6k_gemv
    assert f(None, 16, 512, A, A, 1, A, None) == EINVAL
    assert f(A, 16, 512, None, A, 1, A, None) == EINVAL
    assert f(A, 16, 512, A, None, 1, A, None) == EINVAL
    assert f(A, 16, 512, A, A, 1, None, None) == EINVAL
    assert f(A, 16, 500, A, A, 1, A, None) == ESHAPE
    assert f(A, 16, 0, A, A, 1, A, None) == ESHAPE
    assert f(A, 0, 512, A, A, 1, A, None) == ESHAPE
    assert f(A, 16, 512, A, A, 0, A, None) == ESHAPE
    assert f(A, 16, 512, A, A, 9, A, None) == ESHAPE
    assert f(A, 16, 12544, A, A, 1, A, None) == ESHAPE    # K beyond 48 super-blocks
    assert f(A, 16, 12288, A, A, 8, A, None) == ESHAPE    # staged rows beyond any LDS
    assert f(A + 8, 16, 512, A, A, 1, A, None) == EALIGN
    assert f(A, 16, 512, A + 8, A, 1, A, None) == EALIGN
    assert f(A, 16, 512, A, A + 2, 1, A, None) == EALIGN
    assert f(A, 16, 512, A, A, 1, A + 2, None) == EALIGN


def test_q6k_quantize_gemv_argument_checks(L):
    f = L.q6k_quantize_gemv
    assert f(None, 16, 512, A, 1, A, None) == EINVAL
    assert f(A, 16, 512, None, 1, A, None) == EINVAL
    assert f(A, 16, 512, A, 1, None, None) == EINVAL
    assert f(A, 16, 500, A, 1, A, None) == ESHAPE
    assert f(A, 16, 512, A, 9, A, None) == ESHAPE
    assert f(A, 16, 12288, A, 8, A, None) == ESHAPE
    assert f(A, 0, 512, A, 1, A, None) == ESHAPE
    assert f(A + 4, 16, 512, A, 1, A, None) == EALIGN
    assert f(A, 16, 512, A + 4, 1, A, None) == EALIGN


def test_quantize_gemv_argument_checks(L):
    f = L.q4k_quantize_gemv
    assert f(None, 16, 512, A, 1, A, None) == EINVAL
    assert f(A, 16, 512, None, 1, A, None) == EINVAL
    assert f(A, 16, 500, A, 1, A, None) == ESHAPE
    assert f(A, 16, 512, A, 9, A, None) == ESHAPE
    assert f(A, 16, 16384, A, 8, A, None) == ESHAPE     # staged rows beyond any LDS
    assert f(A, 16, 65536, A, 1, A, None) == ESHAPE     # more columns than 16 waves take
    assert f(A, 0, 512, A, 1, A, None) == ESHAPE
    assert f(A + 4, 16, 512, A, 1, A, None) == EALIGN
    assert f(A, 16, 512, A + 4, 1, A, None) == EALIGN


def test_quantize_gemv_residual_argument_checks(L):
    f = L.q4k_quantize_gemv_residual
    B = 0x20000                          # disjoint from A's [M][N] fp32 range below
    assert f(None, 16, 512, A, 1, B, A, None) == EINVAL
    assert f(A, 16, 512, A, 1, None, A, None) == EINVAL
    assert f(A, 16, 512, A, 1, B, None, None) == EINVAL
    assert f(A, 16, 500, A, 1, B, A, None) == ESHAPE
    assert f(A, 16, 512, A, 9, B, A, None) == ESHAPE
    assert f(A, 16, 16384, A, 8, B, A, None) == ESHAPE  # staged rows beyond any LDS
    assert f(A, 16, 512, A, 1, B + 2, A, None) == EALIGN
    assert f(A + 4, 16, 512, A, 1, B, A, None) == EALIGN
    # residual partly overlapping y (not the same buffer) is rejected
    assert f(A, 16, 512, A, 2, A + 4, A, None) == EINVAL
    assert f(A, 16, 512, A, 2, A, A + 124, None) == EINVAL


def test_quantize_gemv_batch_argument_checks(L):
    f = L.q4k_quantize_gemv_batch
    P = q4k._lib.GemvProblem

    def call(probs, K=512, M=1):
        arr = (P * max(len(probs), 1))(*[P(*p) for p in probs])
        return f(arr, len(probs), K, M, None)
    good = (A, A, A, 16)
    assert f(None, 1, 512, 1, None) == EINVAL
    assert call([]) == ESHAPE
    assert call([good] * 9) == ESHAPE
    assert call([good], K=500) == ESHAPE
    assert call([good], M=9) == ESHAPE
    assert call([good], K=16384, M=8) == ESHAPE
    assert call([good, (A, A, A, 0)]) == ESHAPE
    assert call([good, (None, A, A, 16)]) == EINVAL
    assert call([good, (A, A, None, 16)]) == EINVAL
    assert call([good, (A + 4, A, A, 16)]) == EALIGN
    assert call([good, (A, A + 4, A, 16)]) == EALIGN
    assert call([good, (A, A, A + 2, 16)]) == EALIGN


def test_q6k_gemv_batch_argument_checks(L):
    f, g = L.q6k_gemv_batch, L.q6k_quantize_gemv_batch
    P = q4k._lib.GemvProblem

    def arr(probs):
        return (P * max(len(probs), 1))(*[P(*p) for p in probs])

    def call(probs, K=512, M=1, codes=A, scales=A):
        return f(arr(probs), len(probs), K, codes, scales, M, None)

    def callq(probs, K=512, M=1):
        return g(arr(probs), len(probs), K, M, None)
    good = (A, A, A, 16)
    assert f(None, 1, 512, A, A, 1, None) == EINVAL
    assert call([good], codes=None) == EINVAL
    assert call([good], scales=None) == EINVAL
    assert call([]) == ESHAPE
    assert call([good] * 9) == ESHAPE
    assert call([good], K=500) == ESHAPE
    assert call([good], M=9) == ESHAPE
    assert call([good], K=12544) == ESHAPE              # K beyond 48 super-blocks
    assert call([good], K=12288, M=8) == ESHAPE         # staged rows beyond any LDS
    assert call([good, (A, A, A, 0)]) == ESHAPE
    assert call([good, (None, A, A, 16)]) == EINVAL
    assert call([good, (A, A, None, 16)]) == EINVAL
    assert call([good], codes=A + 8) == EALIGN
    assert call([good], scales=A + 2) == EALIGN
    assert call([good, (A + 4, A, A, 16)]) == EALIGN
    assert call([good, (A, A, A + 2, 16)]) == EALIGN
    assert g(None, 1, 512, 1, None) == EINVAL
    assert callq([]) == ESHAPE
    assert callq([good] * 9) == ESHAPE
    assert callq([good], K=500) == ESHAPE
    assert callq([good], M=9) == ESHAPE
    assert callq([good], K=12288, M=8) == ESHAPE
    assert callq([good, (A, None, A, 16)]) == EINVAL
    assert callq([good, (A, A + 4, A, 16)]) == EALIGN


def test_gemm_batch_argument_checks(L):
    f = L.q4k_gemm_batch
    P = q4k._lib.GemmProblem

    def call(probs, K=512, M=1, codes=A):
        arr = (P * max(len(probs), 1))(*[P(*p) for p in probs])
        return f(arr, len(probs), K, codes, A, A, M, None, 0, None)
    good = (A, A, 16)
    assert f(None, 1, 512, A, A, A, 1, None, 0, None) == EINVAL
    assert call([]) == ESHAPE
    assert call([good] * 9) == ESHAPE
    assert call([good], K=500) == ESHAPE
    assert call([good], M=0) == ESHAPE
    assert call([good], codes=None) == EINVAL
    assert call([good], codes=A + 4) == EALIGN
    assert call([good, (A, A, 0)]) == ESHAPE
    assert call([good, (None, A, 16)]) == EINVAL
    assert call([good, (A, None, 16)]) == EINVAL
    assert call([good, (A + 4, A, 16)]) == EALIGN
    assert call([good, (A, A + 2, 16)]) == EALIGN


def test_gemm_workspace_checks(L):
    """The GEMM workspace is optional; when given it must hold
    q4k_gemm_workspace_bytes() bytes and be 256-byte aligned."""
    need = int(L.q4k_gemm_workspace_bytes())
    assert need == 65536 + 2 * 256 * 128 * 128 * 4
    args = (A, 16, 512, A, A, A, 1, A)
    assert L.q4k_gemm(*args, None, 16, None) == EWORKSPACE
    assert L.q4k_gemm(*args, A, need - 1, None) == EWORKSPACE
    assert L.q4k_gemm(*args, A + 16, need, None) == EALIGN
    P = q4k._lib.GemmProblem
    arr = (P * 1)(P(A, A, 16))
    assert L.q4k_gemm_batch(arr, 1, 512, A, A, A, 1, A, need - 1, None) == EWORKSPACE
    assert L.q4k_gemm_batch(arr, 1, 512, A, A, A, 1, A + 128, need, None) == EALIGN


def test_ceiling_argument_checks(L):
    assert L.q4k_ceiling_stream_read(None, 1024, 1, A, None) == EINVAL
    assert L.q4k_ceiling_stream_read(A, 1024, 1, None, None) == EINVAL
    assert L.q4k_ceiling_stream_read(A, 1000, 1, A, None) == ESHAPE
    assert L.q4k_ceiling_stream_read(A, 1024, 0, A, None) == ESHAPE
    assert L.q4k_ceiling_stream_read(A + 4, 1024, 1, A, None) == EALIGN
    assert L.q4k_ceiling_empty(0, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 16, 1, 3, None, None) == EINVAL
    assert L.q4k_ceiling_mfma_valu(0, 16, 1, 3, A, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 0, 1, 3, A, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 16, 65, 3, A, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 16, 1, 0, A, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 16, 1, 4, A, None) == ESHAPE
    assert L.q4k_ceiling_mfma_valu(1, 16, 1, 3, A + 2, None) == EALIGN


def test_quantize_argument_checks(L):
    f = L.q4k_quantize_act
    assert f(None, 1, 32, None, A, A, A, None) == EINVAL
    assert f(A, 1, 31, None, A, A, A, None) == ESHAPE
    assert f(A, 0, 32, None, A, A, A, None) == ESHAPE
    assert f(A + 4, 1, 32, None, A, A, A, None) == EALIGN
    assert f(A, 1, 32, A + 4, A, A, A, None) == EALIGN


def test_moe_argument_checks(L):
    f = L.q4k_moe_gemv
    ws = q4k.q4k_moe_workspace_bytes(16, 8, 64, 1024)
    assert ws >= 16 * 8 * 1024 * 4
    assert q4k.q4k_moe_workspace_bytes(1, 9, 8, 1024) == 0
    assert q4k.q4k_moe_workspace_bytes(0, 1, 8, 1024) == 0
    assert q4k.q4k_moe_workspace_bytes(4097, 1, 8, 1024) == 0
    assert q4k.q4k_moe_workspace_bytes(1, 1, 4097, 1024) == 0
    stride = 1024 * 8 * 144

    def call(**kw):
        a = dict(w=A, E=64, stride=stride, N=1024, K=2048, ids=A, rw=A, T=16, topk=8,
                 codes=A, scales=A, sums=A, aps=0, y=A, ws=A, wsb=ws)
        a.update(kw)
        return f(a["w"], a["E"], a["stride"], a["N"], a["K"], a["ids"], a["rw"], a["T"],
                 a["topk"], a["codes"], a["scales"], a["sums"], a["aps"], a["y"], a["ws"],
                 a["wsb"], None)
    assert call(ids=None) == EINVAL
    assert call(aps=2) == EINVAL
    assert call(topk=65) == ESHAPE
    assert call(T=600, topk=8) == ESHAPE
    assert call(topk=0) == ESHAPE
    assert call(T=0) == ESHAPE
    assert call(stride=stride - 16) == ESHAPE
    assert call(stride=stride + 8) == ESHAPE
    assert call(K=2000) == ESHAPE
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=ws - 1) == EWORKSPACE
    assert call(ws=A + 16) == EALIGN
    assert call(w=A + 4) == EALIGN


def test_moe_ffn_argument_checks(L):
    f = L.q4k_moe_ffn
    H, F, E, T, topk = 2048, 1024, 64, 16, 8
    ws = q4k.q4k_moe_ffn_workspace_bytes(T, topk, E, H, F)
    assert ws >= T * topk * (2 * F + H) * 4
    assert q4k.q4k_moe_ffn_workspace_bytes(1, 9, 8, H, F) == 0
    assert q4k.q4k_moe_ffn_workspace_bytes(1, 1, 8, 0, F) == 0
    sgu, sd = F * (H // 256) * 144, H * (F // 256) * 144

    def call(**kw):
        a = dict(wg=A, wu=A, wd=A, E=E, sgu=sgu, sd=sd, H=H, F=F, ids=A, rw=A, T=T, topk=topk,
                 x=A, y=A, ws=A, wsb=ws)
        a.update(kw)
        return f(a["wg"], a["wu"], a["wd"], a["E"], a["sgu"], a["sd"], a["H"], a["F"],
                 a["ids"], a["rw"], a["T"], a["topk"], a["x"], a["y"], a["ws"], a["wsb"], None)
    assert call(rw=None) == EINVAL          # the layer's output is the routed sum
    assert call(wu=None) == EINVAL
    assert call(x=None) == EINVAL
    assert call(H=2000) == ESHAPE
    assert call(F=1000) == ESHAPE
    assert call(topk=65) == ESHAPE
    assert call(T=600) == ESHAPE
    assert call(sgu=sgu - 16) == ESHAPE
    assert call(sd=sd + 8) == ESHAPE
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=ws - 1) == EWORKSPACE
    assert call(ws=A + 16) == EALIGN
    assert call(x=A + 4) == EALIGN
    assert call(wd=A + 4) == EALIGN


def test_attn_argument_checks(L):
    ws = int(L.q4k_attn_workspace_bytes(1, 32, 8))
    assert ws >= 4096
    assert L.q4k_attn_workspace_bytes(1, 30, 8) == 0
    f = L.q4k_attn_decode
    ok = (A, 1, 32, 8, 128, A, A, A, A, 1024, 1024, 0.088, A, A, ws, None)

    def call(**kw):
        names = ("q", "M", "n_head", "n_kv", "hd", "kc", "ks", "vc", "vs", "cap", "n_ctx",
                 "scale", "out", "ws", "wsb", "stream")
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])

    assert call(q=None) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(hd=64) == ESHAPE
    assert call(M=0) == ESHAPE and call(M=9) == ESHAPE
    assert call(n_head=30) == ESHAPE            # not a multiple of n_kv
    assert call(n_head=72, n_kv=8) == ESHAPE    # groups of 9
    assert call(n_ctx=0) == ESHAPE
    assert call(M=4, n_ctx=3) == ESHAPE         # a token would see no position
    assert call(n_ctx=1025) == ESHAPE           # beyond the capacity
    assert call(q=A + 4) == EALIGN
    assert call(kc=A + 8) == EALIGN
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=ws - 1) == EWORKSPACE
    assert call(ws=A + 128) == EALIGN
    s = L.q4k_kv_store
    ok_s = (A, A, 1, 8, 128, 0, 16, A, A, A, A, None)
    assert s(None, *ok_s[1:]) == EINVAL
    assert s(*ok_s[:4], 64, *ok_s[5:]) == ESHAPE
    assert s(*ok_s[:5], 16, *ok_s[6:]) == ESHAPE          # pos0 + M > cap
    assert s(*ok_s[:5], -1, *ok_s[6:]) == ESHAPE
    assert s(A + 4, *ok_s[1:]) == EALIGN
    assert s(*ok_s[:7], A + 8, *ok_s[8:]) == EALIGN


def test_q6k_gemm_argument_checks(L):
    f = L.q6k_gemm
    need = int(L.q4k_gemm_workspace_bytes())
    ok = (A, 16, 512, A, A, 1, A, A, need, None)
    assert f(None, *ok[1:]) == EINVAL
    assert f(*ok[:3], None, *ok[4:]) == EINVAL
    assert f(*ok[:4], None, *ok[5:]) == EINVAL
    assert f(*ok[:6], None, *ok[7:]) == EINVAL
    assert f(A, 16, 500, *ok[3:]) == ESHAPE
    assert f(A, 0, 512, *ok[3:]) == ESHAPE
    assert f(*ok[:5], 0, *ok[6:]) == ESHAPE
    assert f(A + 8, *ok[1:]) == EALIGN
    assert f(*ok[:3], A + 8, *ok[4:]) == EALIGN
    assert f(*ok[:4], A + 2, *ok[5:]) == EALIGN
    assert f(*ok[:7], None, 16, None) == EWORKSPACE
    assert f(*ok[:7], A, need - 1, None) == EWORKSPACE
    assert f(*ok[:7], A + 16, need, None) == EALIGN
