"""ctypes marshalling for libq4k.so.  No arithmetic of the products lives here."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libq4k.so")
lib_gemm_int8_path = os.path.join(_HERE, "libq4k_gemm_int8.so")

EXPORTED_SYMBOLS = (
    "q4k_quantize_act",
    "q4k_gemv",
    "q4k_quantize_gemv",
    "q4k_quantize_gemv_residual",
    "q4k_quantize_gemv_batch",
    "q4k_gemm",
    "q4k_gemm_batch",
    "q4k_gemm_workspace_bytes",
    "q4k_gemm_batch_noalloc",
    "q4k_moe_gemv",
    "q4k_moe_workspace_bytes",
    "q4k_moe_ffn",
    "q4k_moe_ffn_workspace_bytes",
    "q6k_gemv",
    "q6k_quantize_gemv",
    "q6k_gemv_batch",
    "q6k_quantize_gemv_batch",
    "q6k_gemm",
    "q4k_kv_store",
    "q4k_attn_workspace_bytes",
    "q4k_attn_decode",
    "q4k_ceiling_stream_read",
    "q4k_ceiling_empty",
    "q4k_ceiling_mfma_valu",
    "q4k_status_string",
)

_P = ctypes.c_void_p
_I = ctypes.c_int64
_lib = None
_lib_int8 = None


class GemvProblem(ctypes.Structure):
    """Mirror of q4k_gemv_problem."""
    _fields_ = [("w", _P), ("x", _P), ("y", _P), ("N", _I)]


class GemmProblem(ctypes.Structure):
    """Mirror of q4k_gemm_problem."""
    _fields_ = [("w", _P), ("y", _P), ("N", _I)]


class Q4KError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, q4k_status_string(status), status))


def _load(path):
    try:
        import torch  # noqa: F401  -- load torch's HIP runtime first (same soname)
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError("%s not built: run `python -m gemm_q4_super_amd.build` "
                           "(or __graft_entry__.build())" % os.path.basename(path))
    return _declare(ctypes.CDLL(path))


def lib():
    """The loaded library (raises if libq4k.so has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(lib_path)
    return _lib


def lib_gemm_int8():
    """The same library with the prefill GEMM's int8 contraction
    (libq4k_gemm_int8.so; raises if it has not been built)."""
    global _lib_int8
    if _lib_int8 is None:
        _lib_int8 = _load(lib_gemm_int8_path)
    return _lib_int8


def _declare(L):
    """Argument and result types of every exported call."""
    L.q4k_quantize_act.argtypes = [_P, _I, _I, _P, _P, _P, _P, _P]
    L.q4k_gemv.argtypes = [_P, _I, _I, _P, _P, _P, _I, _P, _P]
    L.q4k_gemm.argtypes = [_P, _I, _I, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P]
    L.q4k_gemm_batch.argtypes = [ctypes.POINTER(GemmProblem), ctypes.c_int, _I, _P, _P, _P,
                                 _I, _P, ctypes.c_size_t, _P]
    L.q4k_gemm_batch_noalloc.argtypes = [ctypes.POINTER(GemmProblem), ctypes.c_int, _I, _P,
                                         _P, _P, _I, _P]
    L.q4k_gemm_batch_noalloc.restype = ctypes.c_int
    L.q4k_gemm_workspace_bytes.argtypes = []
    L.q4k_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.q4k_quantize_gemv.argtypes = [_P, _I, _I, _P, _I, _P, _P]
    L.q4k_quantize_gemv_residual.argtypes = [_P, _I, _I, _P, _I, _P, _P, _P]
    L.q4k_quantize_gemv_batch.argtypes = [ctypes.POINTER(GemvProblem), ctypes.c_int, _I,
                                          _I, _P]
    L.q4k_moe_gemv.argtypes = [_P, _I, _I, _I, _I, _P, _P, _I, _I, _P, _P, _P,
                               ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
    L.q4k_moe_workspace_bytes.argtypes = [_I, _I, _I, _I]
    L.q4k_moe_workspace_bytes.restype = ctypes.c_size_t
    L.q4k_moe_ffn.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _P, _P, _P,
                              ctypes.c_size_t, _P]
    L.q4k_moe_ffn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    L.q4k_moe_ffn_workspace_bytes.restype = ctypes.c_size_t
    L.q6k_gemv.argtypes = [_P, _I, _I, _P, _P, _I, _P, _P]
    L.q6k_quantize_gemv.argtypes = [_P, _I, _I, _P, _I, _P, _P]
    L.q6k_gemv_batch.argtypes = [ctypes.POINTER(GemvProblem), ctypes.c_int, _I, _P, _P, _I, _P]
    L.q6k_quantize_gemv_batch.argtypes = [ctypes.POINTER(GemvProblem), ctypes.c_int, _I, _I,
                                          _P]
    L.q6k_gemm.argtypes = [_P, _I, _I, _P, _P, _I, _P, _P, ctypes.c_size_t, _P]
    L.q4k_kv_store.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.q4k_attn_workspace_bytes.argtypes = [_I, _I, _I]
    L.q4k_attn_workspace_bytes.restype = ctypes.c_size_t
    L.q4k_attn_decode.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I,
                                  ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
    L.q4k_ceiling_stream_read.argtypes = [_P, _I, _I, _P, _P]
    L.q4k_ceiling_stream_read.restype = ctypes.c_int
    L.q4k_ceiling_empty.argtypes = [_I, _P]
    L.q4k_ceiling_empty.restype = ctypes.c_int
    L.q4k_ceiling_mfma_valu.argtypes = [_I, _I, ctypes.c_int, ctypes.c_int, _P, _P]
    L.q4k_ceiling_mfma_valu.restype = ctypes.c_int
    L.q4k_status_string.argtypes = [ctypes.c_int]
    L.q4k_status_string.restype = ctypes.c_char_p
    for name in ("q4k_quantize_act", "q4k_gemv", "q4k_quantize_gemv",
                 "q4k_quantize_gemv_residual",
                 "q4k_quantize_gemv_batch", "q4k_gemm", "q4k_gemm_batch", "q4k_moe_gemv",
                 "q4k_moe_ffn", "q6k_gemv", "q6k_quantize_gemv", "q6k_gemv_batch",
                 "q6k_quantize_gemv_batch", "q6k_gemm", "q4k_kv_store",
                 "q4k_attn_decode"):
        getattr(L, name).restype = ctypes.c_int
    return L


def q4k_status_string(status: int) -> str:
    return lib().q4k_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(st, what):
    if st != 0:
        raise Q4KError(st, what)


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def q4k_quantize_act(x, gate=None, out=None):
    """Q8 of fp32 x [M, K] (or silu(gate)*x).  Returns (codes, scales, sums)."""
    import torch
    _dev(x, "x"); _dev(gate, "gate")
    M, K = x.shape
    if out is None:
        codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
        scales = torch.empty((M, K // 32), dtype=torch.float32, device=x.device)
        sums = torch.empty((M, K // 32), dtype=torch.int32, device=x.device)
    else:
        codes, scales, sums = out
    _check(lib().q4k_quantize_act(_ptr(x), M, K, _ptr(gate), _ptr(codes), _ptr(scales),
                                  _ptr(sums), _stream(x)), "q4k_quantize_act")
    return codes, scales, sums


def _matrix_call(fn, what, w, N, K, codes, scales, sums, y):
    import torch
    for t, n in ((w, "w"), (codes, "codes"), (scales, "scales"), (sums, "sums")):
        _dev(t, n)
    M = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check(fn(_ptr(w), N, K, _ptr(codes), _ptr(scales), _ptr(sums), M, _ptr(y),
              _stream(codes)), what)
    return y


def q4k_gemv(w, N, K, codes, scales, sums, y=None):
    return _matrix_call(lib().q4k_gemv, "q4k_gemv", w, N, K, codes, scales, sums, y)


def q6k_gemv(w, N, K, codes, scales, y=None):
    """Q6_K weights (N rows x K/256*210 bytes) times prepared Q8 rows (M <= 8)."""
    import torch
    for t, n in ((w, "w"), (codes, "codes"), (scales, "scales")):
        _dev(t, n)
    M = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check(lib().q6k_gemv(_ptr(w), N, K, _ptr(codes), _ptr(scales), M, _ptr(y), _stream(codes)),
           "q6k_gemv")
    return y


def q6k_quantize_gemv(w, N, K, x, y=None):
    """Q8-quantize fp32 x [M, K] and multiply by Q6_K W^T in one launch."""
    import torch
    _dev(w, "w"); _dev(x, "x")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q6k_quantize_gemv(_ptr(w), N, K, _ptr(x), M, _ptr(y), _stream(x)),
           "q6k_quantize_gemv")
    return y


def q6k_gemv_batch(problems, K, codes, scales, ys=None):
    """Several Q6_K GEMVs on the same prepared Q8 rows in one launch.

    `problems` is a sequence of (w, N); returns the list of outputs y_i [M, N_i]
    (or fills `ys`)."""
    import torch
    problems = list(problems)
    if not problems:
        raise ValueError("q6k_gemv_batch: empty batch")
    _dev(codes, "codes"); _dev(scales, "scales")
    M = codes.shape[0]
    if ys is None:
        ys = [torch.empty((M, N), dtype=torch.float32, device=codes.device) for _, N in problems]
    arr = (GemvProblem * len(problems))()
    for i, ((w, N), y) in enumerate(zip(problems, ys)):
        _dev(w, "w")
        arr[i] = GemvProblem(_ptr(w), None, _ptr(y), N)
    _check(lib().q6k_gemv_batch(arr, len(problems), K, _ptr(codes), _ptr(scales), M,
                                _stream(codes)), "q6k_gemv_batch")
    return ys


def q6k_quantize_gemv_batch(problems, K, ys=None):
    """Several Q6_K quantize-and-GEMV products with the same K and M in one
    launch.  `problems` is a sequence of (w, N, x) with fp32 x [M, K]; returns
    the list of outputs y_i [M, N_i] (or fills `ys`)."""
    import torch
    problems = list(problems)
    if not problems:
        raise ValueError("q6k_quantize_gemv_batch: empty batch")
    M = problems[0][2].shape[0]
    if ys is None:
        ys = [torch.empty((M, N), dtype=torch.float32, device=x.device) for _, N, x in problems]
    arr = (GemvProblem * len(problems))()
    for i, ((w, N, x), y) in enumerate(zip(problems, ys)):
        _dev(w, "w"); _dev(x, "x")
        if x.shape[0] != M:
            raise ValueError("q6k_quantize_gemv_batch: every x must have the same M")
        arr[i] = GemvProblem(_ptr(w), _ptr(x), _ptr(y), N)
    _check(lib().q6k_quantize_gemv_batch(arr, len(problems), K, M, _stream(problems[0][2])),
           "q6k_quantize_gemv_batch")
    return ys


def q4k_quantize_gemv(w, N, K, x, y=None):
    """Q8-quantize fp32 x [M, K] and multiply by W^T in one launch."""
    import torch
    _dev(w, "w"); _dev(x, "x")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q4k_quantize_gemv(_ptr(w), N, K, _ptr(x), M, _ptr(y), _stream(x)),
           "q4k_quantize_gemv")
    return y


def q4k_quantize_gemv_residual(w, N, K, x, residual, y=None):
    """y = residual + Q8(x) W^T in one launch (fp32 x [M, K], residual [M, N]).

    With y=None the sum goes to a new tensor; y=residual updates it in place."""
    import torch
    _dev(w, "w"); _dev(x, "x"); _dev(residual, "residual")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q4k_quantize_gemv_residual(_ptr(w), N, K, _ptr(x), M, _ptr(residual), _ptr(y),
                                            _stream(x)),
           "q4k_quantize_gemv_residual")
    return y


def q4k_quantize_gemv_batch(problems, K, ys=None):
    """Several quantize-and-GEMV products with the same K and M in one launch.

    `problems` is a sequence of (w, N, x) with fp32 x [M, K]; returns the list
    of outputs y_i [M, N_i] (or fills `ys`)."""
    import torch
    problems = list(problems)
    if not problems:
        raise ValueError("q4k_quantize_gemv_batch: empty batch")
    M = problems[0][2].shape[0]
    if ys is None:
        ys = [torch.empty((M, N), dtype=torch.float32, device=x.device) for _, N, x in problems]
    arr = (GemvProblem * len(problems))()
    for i, ((w, N, x), y) in enumerate(zip(problems, ys)):
        _dev(w, "w"); _dev(x, "x")
        if x.shape[0] != M:
            raise ValueError("q4k_quantize_gemv_batch: every x must have the same M")
        arr[i] = GemvProblem(_ptr(w), _ptr(x), _ptr(y), N)
    _check(lib().q4k_quantize_gemv_batch(arr, len(problems), K, M, _stream(problems[0][2])),
           "q4k_quantize_gemv_batch")
    return ys


_GEMM_WS = {}


def gemm_workspace(device):
    """A zero-filled GEMM workspace for `device`, made once and reused: every
    call leaves its counters zero again.  Calls on several streams at once
    must pass workspaces of their own."""
    import torch
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _GEMM_WS.get(key)
    if ws is None:
        ws = torch.zeros(int(lib().q4k_gemm_workspace_bytes()), dtype=torch.uint8, device=dev)
        _GEMM_WS[key] = ws
    return ws


def _gemm_ws(workspace, device):
    """(pointer, bytes) of the workspace argument: "auto" -> the cached one,
    None -> no workspace (whole tiles only), else a uint8 device tensor."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a device tensor")
        workspace = gemm_workspace(device)
    _dev(workspace, "workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def q4k_gemm(w, N, K, codes, scales, sums, y=None, workspace="auto", library=None):
    import torch
    for t, n in ((w, "w"), (codes, "codes"), (scales, "scales"), (sums, "sums")):
        _dev(t, n)
    M = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    wp, wb = _gemm_ws(workspace, codes.device)
    _check((library or lib()).q4k_gemm(_ptr(w), N, K, _ptr(codes), _ptr(scales), _ptr(sums), M,
                                       _ptr(y), wp, wb, _stream(codes)), "q4k_gemm")
    return y


def q4k_gemm_batch(problems, K, codes, scales, sums, ys=None, workspace="auto", library=None):
    """Several prefill GEMMs against the same Q8 rows in one launch.

    `problems` is a sequence of (w, N); returns the list of outputs y_i [M, N_i]
    (or fills `ys`).  `library` (for q4k_gemm too): lib_gemm_int8() runs the
    int8 contraction; default lib()."""
    import torch
    problems = list(problems)
    if not problems:
        raise ValueError("q4k_gemm_batch: empty batch")
    for t, n in ((codes, "codes"), (scales, "scales"), (sums, "sums")):
        _dev(t, n)
    M = codes.shape[0]
    if ys is None:
        ys = [torch.empty((M, N), dtype=torch.float32, device=codes.device) for _, N in problems]
    arr = (GemmProblem * len(problems))()
    for i, ((w, N), y) in enumerate(zip(problems, ys)):
        _dev(w, "w")
        arr[i] = GemmProblem(_ptr(w), _ptr(y), N)
    wp, wb = _gemm_ws(workspace, codes.device)
    _check((library or lib()).q4k_gemm_batch(arr, len(problems), K, _ptr(codes), _ptr(scales),
                                             _ptr(sums), M, wp, wb, _stream(codes)),
           "q4k_gemm_batch")
    return ys


def q4k_moe_workspace_bytes(T, topk, n_experts, N) -> int:
    return int(lib().q4k_moe_workspace_bytes(T, topk, n_experts, N))


def q4k_moe_gemv(w, n_experts, expert_stride, N, K, ids, route_w, codes, scales, sums,
                 act_per_slot, workspace=None, y=None):
    import torch
    for t, n in ((w, "w"), (ids, "ids"), (route_w, "route_w"), (codes, "codes"),
                 (scales, "scales"), (sums, "sums")):
        _dev(t, n)
    T, topk = ids.shape
    if workspace is None:
        nbytes = q4k_moe_workspace_bytes(T, topk, n_experts, N)
        workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=codes.device)
    if y is None:
        rows = T if route_w is not None else T * topk
        y = torch.empty((rows, N), dtype=torch.float32, device=codes.device)
    _check(lib().q4k_moe_gemv(_ptr(w), n_experts, expert_stride, N, K, _ptr(ids),
                              _ptr(route_w), T, topk, _ptr(codes), _ptr(scales), _ptr(sums),
                              int(act_per_slot), _ptr(y), _ptr(workspace),
                              workspace.numel(), _stream(codes)), "q4k_moe_gemv")
    return y


def q4k_moe_ffn_workspace_bytes(T, topk, n_experts, H, F) -> int:
    return int(lib().q4k_moe_ffn_workspace_bytes(T, topk, n_experts, H, F))


def q4k_moe_ffn(w_gate, w_up, w_down, n_experts, stride_gate_up, stride_down, H, F, ids,
                route_w, x, workspace=None, y=None):
    import torch
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"), (ids, "ids"),
                 (route_w, "route_w"), (x, "x")):
        _dev(t, n)
    T, topk = ids.shape
    if workspace is None:
        nbytes = q4k_moe_ffn_workspace_bytes(T, topk, n_experts, H, F)
        workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _check(lib().q4k_moe_ffn(_ptr(w_gate), _ptr(w_up), _ptr(w_down), n_experts, stride_gate_up,
                             stride_down, H, F, _ptr(ids), _ptr(route_w), T, topk, _ptr(x),
                             _ptr(y), _ptr(workspace), workspace.numel(), _stream(x)),
           "q4k_moe_ffn")
    return y


def q6k_gemm(w, N, K, codes, scales, y=None, workspace="auto"):
    """Q6_K prefill GEMM: y [M, N] = Q8 rows (codes, scales) x W^T."""
    import torch
    for t, n in ((w, "w"), (codes, "codes"), (scales, "scales")):
        _dev(t, n)
    M = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    wp, wb = _gemm_ws(workspace, codes.device)
    _check(lib().q6k_gemm(_ptr(w), N, K, _ptr(codes), _ptr(scales), M, _ptr(y), wp, wb,
                          _stream(codes)), "q6k_gemm")
    return y


# ------------------------------------------------------------ INT8 KV cache --

def q4k_kv_store(k, v, pos0, k_codes, k_scales, v_codes, v_scales):
    """Quantize fp32 k, v [M, n_kv, 128] into cache positions pos0..pos0+M-1 of
    k_codes/v_codes int8 [n_kv, cap, 128] and k_scales/v_scales fp32 [n_kv, cap]."""
    for t, n in ((k, "k"), (v, "v"), (k_codes, "k_codes"), (k_scales, "k_scales"),
                 (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, n)
    M, n_kv, hd = k.shape
    cap = k_codes.shape[1]
    _check(lib().q4k_kv_store(_ptr(k), _ptr(v), M, n_kv, hd, pos0, cap, _ptr(k_codes),
                              _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _stream(k)),
           "q4k_kv_store")


def q4k_attn_workspace_bytes(M, n_head, n_kv) -> int:
    return int(lib().q4k_attn_workspace_bytes(M, n_head, n_kv))


_ATTN_WS = {}


def attn_workspace(device, nbytes):
    """A zero-filled attention workspace of at least `nbytes` for `device`,
    reused across calls (every call leaves its counters zero)."""
    import torch
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _ATTN_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(int(nbytes), dtype=torch.uint8, device=dev)
        _ATTN_WS[key] = ws
    return ws


def q4k_attn_decode(q, k_codes, k_scales, v_codes, v_scales, n_ctx, scale, out=None,
                    workspace="auto"):
    """Decode attention of q fp32 [M, n_head, 128] over the first n_ctx positions
    of one layer's INT8 cache (token m sees n_ctx - (M - 1 - m) positions)."""
    import torch
    for t, n in ((q, "q"), (k_codes, "k_codes"), (k_scales, "k_scales"), (v_codes, "v_codes"),
                 (v_scales, "v_scales")):
        _dev(t, n)
    M, n_head, hd = q.shape
    n_kv, cap, _ = k_codes.shape
    if out is None:
        out = torch.empty_like(q)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a device tensor")
        workspace = attn_workspace(q.device, q4k_attn_workspace_bytes(M, n_head, n_kv))
    _dev(workspace, "workspace")
    _check(lib().q4k_attn_decode(_ptr(q), M, n_head, n_kv, hd, _ptr(k_codes), _ptr(k_scales),
                                 _ptr(v_codes), _ptr(v_scales), cap, n_ctx, float(scale),
                                 _ptr(out), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(q)),
           "q4k_attn_decode")
    return out
