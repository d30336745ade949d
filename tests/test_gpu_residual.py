"""GPU parity of q4k_quantize_gemv_residual (y = residual + Q8(x) W^T, the add
inside the GEMV) against q4k_quantize_gemv and the CPU oracle.

The product must be the one q4k_quantize_gemv computes, so y equals the fp32
sum of residual and that output bit for bit.  Against the oracle's fp64
residual + W x the error bound is the GEMV's, max(2e-3 |W x|, 1e-4), plus the
half-ulp rounding of the final fp32 add (<= 2^-24 |y|).
"""
import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import ABS_TOL, REL_TOL, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    import torch
    assert torch.cuda.is_available()
    import gemm_q4_super_amd as m
    m.lib()
    return m


def _check_oracle(y, r, w, N, K, x, oracle_lib, rows, what):
    rc, rs, _ = oracle_lib.quantize_act(x)
    mv = oracle_lib.matvec(w, N, K, rc, rs, rows=rows)
    ref = oracle_lib.matvec_residual(w, N, K, rc, rs, r, rows=rows)
    ys = np.asarray(y if rows is None else y[:, rows], np.float64)
    tol = np.maximum(REL_TOL * np.abs(mv), ABS_TOL) + 2.0 ** -24 * np.abs(ys)
    bad = np.abs(ys - ref) > tol
    assert not bad.any(), "%s: %d elements out of tolerance" % (what, bad.sum())


@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (37, 512, 2), (1000, 2560, 1), (2560, 4096, 1),
                                   (2560, 9728, 1), (2560, 9728, 3), (4096, 2560, 1),
                                   (129, 3840, 7), (2049, 1280, 5), (40000, 2560, 1),
                                   (64, 32768, 1), (17, 2560, 8), (4096, 4096, 8),
                                   (2560, 9728, 4), (2560, 9728, 8)])
def test_residual_equals_gemv_plus_residual(q4k, oracle_lib, N, K, M):
    """Out of place: bits of fp32(residual + q4k_quantize_gemv), and the oracle."""
    import torch
    print("residual N=%d K=%d M=%d" % (N, K, M), flush=True)
    w = qi.make_q4k_bytes(N, K, 9100 + N + K)
    x = qi.make_act(M, K, 9200 + M + K)
    r = qi.make_act(M, N, 9300 + M + N)
    wd, xd, rd = to_dev(w), to_dev(x), to_dev(r)
    y0 = q4k.q4k_quantize_gemv(wd, N, K, xd)
    y = q4k.q4k_quantize_gemv_residual(wd, N, K, xd, rd)
    torch.cuda.synchronize()
    y0, y = y0.cpu().numpy(), y.cpu().numpy()
    assert (rd.cpu().numpy() == r).all()                      # residual left as it was
    assert (y.view(np.uint32) == (y0 + r).view(np.uint32)).all()
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
    _check_oracle(y, r, w, N, K, x, oracle_lib, rows, "residual N=%d K=%d M=%d" % (N, K, M))


@pytest.mark.parametrize("N,K,M", [(2560, 4096, 1), (2560, 9728, 1), (300, 2560, 4)])
def test_residual_in_place(q4k, oracle_lib, N, K, M):
    """y = residual (the residual stream updated in place) gives the same bits
    as the out-of-place call; residual = -(W x) cancels to exact zeros."""
    import torch
    w = qi.make_q4k_bytes(N, K, 9400 + N + K)
    x = qi.make_act(M, K, 9500 + M + K)
    r = qi.make_act(M, N, 9600 + M + N)
    wd, xd = to_dev(w), to_dev(x)
    out = q4k.q4k_quantize_gemv_residual(wd, N, K, xd, to_dev(r))
    stream_buf = to_dev(r)
    same = q4k.q4k_quantize_gemv_residual(wd, N, K, xd, stream_buf, y=stream_buf)
    assert same.data_ptr() == stream_buf.data_ptr()
    neg = -q4k.q4k_quantize_gemv(wd, N, K, xd)
    zero = q4k.q4k_quantize_gemv_residual(wd, N, K, xd, neg, y=neg)
    torch.cuda.synchronize()
    assert (stream_buf.cpu().numpy().view(np.uint32) == out.cpu().numpy().view(np.uint32)).all()
    assert (zero.cpu().numpy() == 0).all()


def test_residual_writes_only_its_output(q4k, oracle_lib):
    """Output and residual as views inside larger buffers: nothing outside the
    output view changes, and the residual view is only read."""
    import torch
    N, K, M = 37, 512, 2
    w = qi.make_q4k_bytes(N, K, 9700)
    x = qi.make_act(M, K, 9701)
    r = qi.make_act(M, N, 9702)
    buf = torch.full((M * N + 64,), 12345.0, device="cuda")
    rbuf = torch.full((M * N + 64,), -7.0, device="cuda")
    rbuf[16:16 + M * N] = to_dev(r).reshape(-1)
    y = buf[32:32 + M * N].view(M, N)
    q4k.q4k_quantize_gemv_residual(to_dev(w), N, K, to_dev(x), rbuf[16:16 + M * N].view(M, N), y=y)
    torch.cuda.synchronize()
    b, rb = buf.cpu().numpy(), rbuf.cpu().numpy()
    assert (b[:32] == 12345.0).all() and (b[32 + M * N:] == 12345.0).all()
    assert (rb[:16] == -7.0).all() and (rb[16 + M * N:] == -7.0).all()
    assert (rb[16:16 + M * N] == r.reshape(-1)).all()
    _check_oracle(y.cpu().numpy(), r, w, N, K, x, oracle_lib, None, "residual into a view")


def test_residual_in_place_graph_replays(q4k):
    """The decode-step use: the o (2560 x 4096) and down (2560 x 9728)
    products add into one residual stream in place, captured in a HIP graph
    and replayed three times with eager work between the replays.  After each
    replay the stream must hold, bit for bit, the fp32 sums built on the host
    from the two products' q4k_quantize_gemv outputs."""
    import torch
    shapes = [(2560, 4096), (2560, 9728)]
    ws = [to_dev(qi.make_q4k_bytes(N, K, 9800 + i)) for i, (N, K) in enumerate(shapes)]
    xs = [to_dev(qi.make_act(1, K, 9810 + i)) for i, (N, K) in enumerate(shapes)]
    r0 = qi.make_act(1, 2560, 9820)
    ys = [q4k.q4k_quantize_gemv(w, N, K, x).cpu().numpy() for w, x, (N, K) in zip(ws, xs, shapes)]
    resid = to_dev(r0)
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for w, x, (N, K) in zip(ws, xs, shapes):
            q4k.q4k_quantize_gemv_residual(w, N, K, x, resid, y=resid)
    torch.cuda.synchronize()
    assert (resid.cpu().numpy() == r0).all()          # capture launched nothing
    expect = r0.copy()
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        for y in ys:
            expect = (expect + y).astype(np.float32)
        got = resid.cpu().numpy()
        assert (got.view(np.uint32) == expect.view(np.uint32)).all(), "replay %d" % k
        _ = torch.ones(1024, device="cuda").sum().item()   # eager work between replays
