"""CPU oracle for the Q4_K x Q8 products -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrapper over `q4k_oracle.c` (plain C, fp64 products,
bit-exact fp32 activation quantizer), built single-threaded and, for the
full-size checks and the all-core CPU baseline, with OpenMP over the output
rows of each product (the same arithmetic per output).  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import this package; the GPU product
path neither imports it nor shares any code with it.

`build()` compiles the C file with gcc (no fast-math, no FMA contraction) into
`liboracle.so` and `liboracle_omp.so` next to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4k_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QK, SB_BYTES, QB = 256, 144, 32

_P = ctypes.c_void_p
_I = ctypes.c_int64


_OMP_PATH = os.path.join(_HERE, "liboracle_omp.so")
_omp = None
_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc, single-threaded and with OpenMP over output
    rows.  Returns the single-threaded library's path."""
    for path, extra in ((_LIB_PATH, []), (_OMP_PATH, ["-fopenmp"])):
        if force or not os.path.exists(path):
            tmp = path + ".tmp"
            subprocess.check_call(["gcc"] + _FLAGS + extra + ["-o", tmp, _SRC, "-lm"])
            os.replace(tmp, path)
    return _LIB_PATH


_SIG = {
    "oracle_unpack_q4k": [_P, _P, _P, _P, _P, _P],
    "oracle_dequant_row": [_P, _I, _P],
    "oracle_quantize_act": [_P, _I, _I, _P, _P, _P],
    "oracle_swiglu": [_P, _P, _I, _P],
    "oracle_matvec": [_P, _I, _I, _P, _P, _I, _P, _I, _P],
    "oracle_subblock_dots": [_P, _I, _P, _I, _P, _I, _P],
    "oracle_matvec_intform": [_P, _I, _P, _P, _P, _I, _P, _I, _P],
    "oracle_moe_matvec": [_P, _I, _I, _I, _I, _P, _P, _I, _I, _P, _P,
                          ctypes.c_int, _P],
    "oracle_moe_layer": [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I,
                         _P, _P, _P, _P, _P, _P, _P, _P],
    "oracle_unpack_q6k": [_P, _P, _P, _P],
    "oracle_q6k_dequant_row": [_P, _I, _P],
    "oracle_q6k_matvec": [_P, _I, _I, _P, _P, _I, _P, _I, _P],
    "oracle_kv_quantize": [_P, _I, _I, _P, _P],
    "oracle_attn_int8kv": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I,
                           ctypes.c_double, _P],
}


def _open(path):
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    for name, args in _SIG.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _open(_LIB_PATH)
    return _lib


def _load_omp():
    global _omp
    if _omp is None:
        _omp = _open(_OMP_PATH)
    return _omp


def threads(parallel: bool = True) -> int:
    """Threads the oracle uses: 1 single-threaded, or the OpenMP team size."""
    return int((_load_omp() if parallel else _load()).oracle_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def unpack_q4k(sb: np.ndarray):
    """Fields of one 144-byte super-block: (d, dmin, sc[8], mn[8], q[256])."""
    sb = _c(sb, np.uint8).reshape(SB_BYTES)
    d, dmin = ctypes.c_double(), ctypes.c_double()
    sc = np.zeros(8, np.int32)
    mn = np.zeros(8, np.int32)
    q = np.zeros(QK, np.int32)
    _load().oracle_unpack_q4k(_ptr(sb), ctypes.addressof(d), ctypes.addressof(dmin),
                              _ptr(sc), _ptr(mn), _ptr(q))
    return d.value, dmin.value, sc, mn, q


def dequant(w: np.ndarray, K: int) -> np.ndarray:
    """fp64 [N, K] dequantized weights of packed Q4_K rows."""
    w = _c(w, np.uint8)
    N = w.size // (K // QK * SB_BYTES)
    w = w.reshape(N, -1)
    out = np.zeros((N, K), np.float64)
    for n in range(N):
        _load().oracle_dequant_row(_ptr(w[n]), K, _ptr(out[n]))
    return out


def quantize_act(x: np.ndarray):
    """Q8 of fp32 [M, K]: (codes int8 [M, K], scales fp32 [M, K/32], sums int32 [M, K/32])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    codes = np.zeros((M, K), np.int8)
    scales = np.zeros((M, K // QB), np.float32)
    sums = np.zeros((M, K // QB), np.int32)
    _load().oracle_quantize_act(_ptr(x), M, K, _ptr(codes), _ptr(scales), _ptr(sums))
    return codes, scales, sums


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g, u = _c(g, np.float32), _c(u, np.float32)
    h = np.zeros_like(g)
    _load().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def _rows(rows, N):
    if rows is None:
        return np.arange(N, dtype=np.int64)
    return _c(rows, np.int64)


def matvec(w, N, K, codes, scales, rows=None, parallel=False) -> np.ndarray:
    """fp64 [M, len(rows)]: y[m, r] = sum_k w[rows[r], k] * xhat[m, k].
    parallel=True runs the output rows on all host cores (same arithmetic)."""
    codes, scales = _c(codes, np.int8), _c(scales, np.float32)
    M = codes.size // K
    r = _rows(rows, N)
    y = np.zeros((M, r.size), np.float64)
    (_load_omp() if parallel else _load()).oracle_matvec(_ptr(_c(w, np.uint8)), N, K, _ptr(codes), _ptr(scales), M,
                          _ptr(r), r.size, _ptr(y))
    return y


def matvec_residual(w, N, K, codes, scales, residual, rows=None) -> np.ndarray:
    """fp64 [M, len(rows)]: residual[m, rows[r]] + matvec(...)[m, r] -- the
    decode step's residual-stream update with the add taken into the GEMV
    ("genie-ai-runtime ...", section 4, Path C).  residual is [M, N]."""
    y = matvec(w, N, K, codes, scales, rows)
    res = np.asarray(residual, np.float64).reshape(y.shape[0], N)
    return res[:, _rows(rows, N)] + y


def matvec_intform(w, N, K, codes, scales, sums, rows=None) -> np.ndarray:
    codes, scales, sums = _c(codes, np.int8), _c(scales, np.float32), _c(sums, np.int32)
    M = codes.size // K
    r = _rows(rows, N)
    y = np.zeros((M, r.size), np.float64)
    _load().oracle_matvec_intform(_ptr(_c(w, np.uint8)), K, _ptr(codes), _ptr(scales),
                                  _ptr(sums), M, _ptr(r), r.size, _ptr(y))
    return y


def subblock_dots(w, N, K, codes, rows=None) -> np.ndarray:
    """int32 [M, len(rows), K/32] sub-block dots D = sum q*c."""
    codes = _c(codes, np.int8)
    M = codes.size // K
    r = _rows(rows, N)
    D = np.zeros((M, r.size, K // QB), np.int32)
    _load().oracle_subblock_dots(_ptr(_c(w, np.uint8)), K, _ptr(codes), M, _ptr(r),
                                 r.size, _ptr(D))
    return D


def moe_matvec(w, n_experts, expert_stride, N, K, ids, route_w, codes, scales,
               act_per_slot: bool) -> np.ndarray:
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    rw = None if route_w is None else _c(route_w, np.float32)
    codes, scales = _c(codes, np.int8), _c(scales, np.float32)
    y = np.zeros((T if rw is not None else T * topk, N), np.float64)
    _load().oracle_moe_matvec(_ptr(_c(w, np.uint8)), n_experts, expert_stride, N, K,
                              _ptr(ids), _ptr(rw), T, topk, _ptr(codes), _ptr(scales),
                              int(act_per_slot), _ptr(y))
    return y


def moe_layer(w_gate, w_up, w_down, n_experts, H, F, ids, route_w, x, parallel=False):
    """Whole routed-expert FFN layer.  Returns dict with y (fp64 [T, H]) and the
    intermediates g, u, h (fp32 [T*topk, F]) and hc/hs/hsum (Q8 of h).
    parallel=True runs each product's output rows on all host cores."""
    ids, rw, x = _c(ids, np.int32), _c(route_w, np.float32), _c(x, np.float32)
    T, topk = ids.shape
    P = T * topk
    stride_gu = F * (H // QK) * SB_BYTES
    stride_dn = H * (F // QK) * SB_BYTES
    out = dict(g=np.zeros((P, F), np.float32), u=np.zeros((P, F), np.float32),
               h=np.zeros((P, F), np.float32), hc=np.zeros((P, F), np.int8),
               hs=np.zeros((P, F // QB), np.float32), hsum=np.zeros((P, F // QB), np.int32),
               y=np.zeros((T, H), np.float64))
    (_load_omp() if parallel else _load()).oracle_moe_layer(
                             _ptr(_c(w_gate, np.uint8)), _ptr(_c(w_up, np.uint8)),
                             _ptr(_c(w_down, np.uint8)), n_experts, stride_gu, stride_dn,
                             H, F, _ptr(ids), _ptr(rw), T, topk, _ptr(x),
                             _ptr(out["g"]), _ptr(out["u"]), _ptr(out["h"]),
                             _ptr(out["hc"]), _ptr(out["hs"]), _ptr(out["hsum"]),
                             _ptr(out["y"]))
    return out


# ------------------------------------------------------------------ Q6_K ----

Q6_SB_BYTES = 210


def unpack_q6k(sb: np.ndarray):
    """Fields of one 210-byte Q6_K super-block: (d, sc[16] int32, q[256] int32)."""
    sb = _c(sb, np.uint8)
    d = ctypes.c_double()
    sc = np.zeros(16, np.int32)
    q = np.zeros(256, np.int32)
    _load().oracle_unpack_q6k(_ptr(sb), ctypes.addressof(d), _ptr(sc), _ptr(q))
    return d.value, sc, q


def q6k_dequant(w: np.ndarray, K: int) -> np.ndarray:
    """fp64 [N, K] weights of Q6_K rows (uint8 [N, K/256*210])."""
    w = _c(w, np.uint8).reshape(-1, K // QK * Q6_SB_BYTES)
    out = np.zeros((w.shape[0], K), np.float64)
    for n in range(w.shape[0]):
        _load().oracle_q6k_dequant_row(_ptr(w[n]), K, _ptr(out[n]))
    return out


def q6k_matvec(w, N, K, codes, scales, rows=None, parallel=False) -> np.ndarray:
    """fp64 [M, len(rows)]: y[m, r] = sum_k w[rows[r], k] * xhat[m, k], Q6_K weights."""
    codes, scales = _c(codes, np.int8), _c(scales, np.float32)
    M = codes.size // K
    r = _rows(rows, N)
    y = np.zeros((M, r.size), np.float64)
    (_load_omp() if parallel else _load()).oracle_q6k_matvec(_ptr(_c(w, np.uint8)), N, K, _ptr(codes), _ptr(scales), M,
                              _ptr(r), r.size, _ptr(y))
    return y


# --------------------------------------------------------- INT8 KV cache ----

def kv_quantize(x: np.ndarray):
    """Q8 of fp32 vectors [..., hd], one scale per vector (a cache entry of one
    position and kv-head).  Returns (codes int8 [..., hd], scales fp32 [...])."""
    x = _c(x, np.float32)
    hd = x.shape[-1]
    R = x.size // hd
    codes = np.zeros(x.shape, np.int8)
    scales = np.zeros(x.shape[:-1], np.float32)
    _load().oracle_kv_quantize(_ptr(x), R, hd, _ptr(codes), _ptr(scales))
    return codes, scales


def attn_int8kv(q, kc, ks, vc, vs, n_ctx, scale, parallel=False) -> np.ndarray:
    """fp64 [M, n_head, hd] decode attention over one layer's INT8 cache.

    q fp32 [M, n_head, hd]; kc, vc int8 [n_kv, cap, hd]; ks, vs fp32 [n_kv, cap].
    Query token m sees the first n_ctx - (M - 1 - m) positions.  parallel=True
    runs the (token, head) pairs on all host cores (same arithmetic)."""
    q = _c(q, np.float32)
    M, n_head, hd = q.shape
    kc, vc = _c(kc, np.int8), _c(vc, np.int8)
    ks, vs = _c(ks, np.float32), _c(vs, np.float32)
    n_kv, cap, _ = kc.shape
    out = np.zeros((M, n_head, hd), np.float64)
    (_load_omp() if parallel else _load()).oracle_attn_int8kv(
        _ptr(q), M, n_head, n_kv, hd, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
        cap, n_ctx, float(scale), _ptr(out))
    return out
