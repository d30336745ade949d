"""GPU parity of q6k_gemv (Q6_K weights x prepared Q8 rows) and of
q6k_quantize_gemv (fp32 rows quantized inside) against the CPU oracle.

Outputs must be within |gpu - oracle| <= max(2e-3 |oracle|, 1e-4) elementwise,
and exactly equal in the integer-exposing case where the sub-block dots pass
unrounded to the output.  Shapes with an odd number of super-blocks per row
put every other row's super-blocks at addresses 2 (mod 4), the case the
kernel's byte shifting covers.
"""
import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    import torch
    assert torch.cuda.is_available()
    import gemm_q4_super_amd as m
    m.lib()
    return m


def _q6k(q4k, w, N, K, x, oracle_lib, rows=None):
    import torch
    codes, scales, _ = oracle_lib.quantize_act(x)
    y = q4k.q6k_gemv(to_dev(w), N, K, to_dev(codes), to_dev(scales))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle_lib.q6k_matvec(w, N, K, codes, scales, rows=rows)
    return (y if rows is None else y[:, rows]), ref


@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (9, 768), (33, 2560), (100, 4096),
                                 (257, 1280), (1000, 2560), (65, 3328)])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_q6k_gemv_shapes_and_tails(q4k, oracle_lib, N, K, M):
    w, _ = qi.make_q6k(N, K, 500 + N + K)
    x = qi.make_act(M, K, 600 + M + K)
    x[0, :32] = 0.0                      # an all-zero activation block
    y, ref = _q6k(q4k, w, N, K, x, oracle_lib)
    assert_close(y, ref, "q6k_gemv N=%d K=%d M=%d" % (N, K, M))


def test_q6k_gemv_integer_exposing_bit_exact(q4k, oracle_lib):
    """d = 1, one scale 1 per super-block, integer activations with a 127 in
    every block (so the Q8 scale is 1 and codes = x): y is the integer dot of
    that 16-weight sub-block with (q - 32), exact in fp32."""
    rng = np.random.default_rng(21)
    N, K = 40, 768
    f = qi.draw_q6k_fields(N, K, 700)
    f.d[:] = np.float16(1.0)
    f.sc[:] = 0
    for n in range(N):
        for b in range(K // 256):
            f.sc[n, b, rng.integers(0, 16)] = 1
    w = qi.pack_q6k(f)
    x = rng.integers(-127, 128, size=(3, K)).astype(np.float32)
    x[:, ::32] = 127.0
    y, ref = _q6k(q4k, w, N, K, x, oracle_lib)
    assert np.abs(ref).max() < 2 ** 24
    assert (y == ref).all()


def test_q6k_gemv_all_ones_closed_form(q4k, oracle_lib):
    N, K = 50, 1024
    w, f = qi.make_q6k(N, K, 710)
    x = np.ones((1, K), np.float32)
    y, _ = _q6k(q4k, w, N, K, x, oracle_lib)
    j = np.arange(256) // 16
    wf = (f.d.astype(np.float64)[:, :, None] * f.sc.astype(np.float64)[:, :, j] *
          (f.q.astype(np.float64) - 32.0)).reshape(N, K)
    d_a = float(np.float32(1.0) / np.float32(127.0))
    assert_close(y[0], 127.0 * d_a * wf.sum(axis=1), "all-ones closed form")


def test_q6k_gemv_zero_scales_exact_zero(q4k, oracle_lib):
    N, K = 24, 512
    f = qi.draw_q6k_fields(N, K, 720)
    f.d[: N // 2] = 0
    f.sc[N // 2:] = 0
    w = qi.pack_q6k(f)
    y, _ = _q6k(q4k, w, N, K, qi.make_act(2, K, 721), oracle_lib)
    assert (y == 0).all()


@pytest.mark.parametrize("proj", range(7))
def test_q6k_gemv_qwen3_4b_shapes_sampled(q4k, oracle_lib, proj):
    """The decode projection shapes at full size, sampled rows against the oracle."""
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    w = qi.make_q6k_bytes(N, K, 730 + proj)
    rows = np.unique(np.r_[0, 1, N - 1, np.random.default_rng(proj).integers(0, N, 60)])
    for M in (1, 3, 8):
        x = qi.make_act(M, K, 740 + proj + M)
        y, ref = _q6k(q4k, w, N, K, x, oracle_lib, rows=rows)
        assert_close(y, ref, "q6k %s M=%d" % (name, M))


def test_q6k_gemv_writes_only_its_output(q4k, oracle_lib):
    import torch
    N, K, M = 37, 512, 2
    w, _ = qi.make_q6k(N, K, 750)
    codes, scales, _ = oracle_lib.quantize_act(qi.make_act(M, K, 751))
    buf = torch.full((M * N + 64,), 12345.0, device="cuda")
    y = buf[32:32 + M * N].view(M, N)
    q4k.q6k_gemv(to_dev(w), N, K, to_dev(codes), to_dev(scales), y=y)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert (b[:32] == 12345.0).all() and (b[32 + M * N:] == 12345.0).all()
    assert_close(y.cpu().numpy(), oracle_lib.q6k_matvec(w, N, K, codes, scales), "q6k into a view")


@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (9, 768, 1), (33, 2560, 1), (100, 4096, 2),
                                   (257, 1280, 3), (65, 3328, 5), (40, 4096, 8), (2560, 9728, 3),
                                   (4096, 2560, 1), (2560, 9728, 4), (2560, 9728, 8),
                                   (300, 11264, 8), (200, 12288, 7)])
def test_q6k_quantize_gemv_bit_identical_to_two_step(q4k, oracle_lib, N, K, M):
    """One launch (quantize inside) equals q4k_quantize_act followed by
    q6k_gemv bit for bit, and the oracle within tolerance."""
    import torch
    w = qi.make_q6k_bytes(N, K, 800 + N + K)
    x = qi.make_act(M, K, 810 + M + K)
    x[0, 32:64] = 0.0
    wd, xd = to_dev(w), to_dev(x)
    y1 = q4k.q6k_quantize_gemv(wd, N, K, xd)
    c, s, _ = q4k.q4k_quantize_act(xd)
    y2 = q4k.q6k_gemv(wd, N, K, c, s)
    torch.cuda.synchronize()
    y1, y2 = y1.cpu().numpy(), y2.cpu().numpy()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
    rc, rs, _ = oracle_lib.quantize_act(x)
    ref = oracle_lib.q6k_matvec(w, N, K, rc, rs, rows=rows)
    assert_close(y1 if rows is None else y1[:, rows], ref, "q6k_quantize_gemv N=%d K=%d M=%d" % (N, K, M))


_Q6_BATCHES = {
    # name: (K, [N_i]) -- the decode launch groups, and eight ragged products
    "qkv": (2560, [4096, 1024, 1024]),
    "gate_up": (2560, [9728, 9728]),
    "eight_ragged": (768, [1, 7, 33, 100, 257, 8, 9, 1000]),
}


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("name", sorted(_Q6_BATCHES))
def test_q6k_gemv_batch_bit_identical_to_single(q4k, oracle_lib, name, M):
    """q6k_gemv_batch (one launch, shared prepared rows) equals q6k_gemv on
    each product bit for bit; q6k_quantize_gemv_batch (each product its own
    fp32 rows) equals q6k_quantize_gemv likewise; sampled rows within the
    tolerance of the oracle."""
    import torch
    K, Ns = _Q6_BATCHES[name]
    ws = [to_dev(qi.make_q6k_bytes(N, K, 5100 + 31 * i + N)) for i, N in enumerate(Ns)]
    x = qi.make_act(M, K, 5200 + M + K)
    codes, scales, _ = oracle_lib.quantize_act(x)
    dc, ds = to_dev(codes), to_dev(scales)
    ys = q4k.q6k_gemv_batch(list(zip(ws, Ns)), K, dc, ds)
    singles = [q4k.q6k_gemv(w, N, K, dc, ds) for w, N in zip(ws, Ns)]
    xs = [to_dev(qi.make_act(M, K, 5300 + 7 * i + M)) for i in range(len(Ns))]
    yq = q4k.q6k_quantize_gemv_batch([(w, N, xi) for w, N, xi in zip(ws, Ns, xs)], K)
    sq = [q4k.q6k_quantize_gemv(w, N, K, xi) for w, N, xi in zip(ws, Ns, xs)]
    torch.cuda.synchronize()
    for i, (w, N) in enumerate(zip(ws, Ns)):
        assert torch.equal(ys[i].view(torch.int32), singles[i].view(torch.int32)), "%s %d" % (name, i)
        assert torch.equal(yq[i].view(torch.int32), sq[i].view(torch.int32)), "%s fused %d" % (name, i)
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N + i).integers(0, N, 12)])
        ref = oracle_lib.q6k_matvec(w.cpu().numpy(), N, K, codes, scales, rows=rows)
        assert_close(ys[i].cpu().numpy()[:, rows], ref, "q6k_gemv_batch %s product %d" % (name, i))
