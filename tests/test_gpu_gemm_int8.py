"""GPU parity of the prefill GEMM's int8 contraction (libq4k_gemm_int8.so:
v_mfma_i32_32x32x32_i8 on the 4-bit quants and the Q8 codes, exact int32
sub-block dots, fp32 epilogue) against the CPU oracle, beside the default fp16
contraction of libq4k.so.

  - integer-exposing weights (d = 1, dmin = 0, one-hot sub-block scale) and
    integer activations reproduce the oracle's int32 sub-block dots exactly;
  - random inputs over tails and tile edges, outlier activation blocks and
    every output of a full 512-row layer within max(2e-3 |oracle|, 1e-4);
  - repeated calls give the same bits and leave the split counters zero;
    without a workspace a batched call equals the single calls bit for bit;
  - both contractions agree to fp32 rounding of the same exact block sums.
Calls with M <= 8 run the GEMV kernels in both libraries, so the cases here
have M > 8.
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
    m.lib_gemm_int8()
    return m


def _gemm(q4k, w, N, K, codes, scales, sums, library, workspace="auto"):
    import torch
    y = q4k.q4k_gemm(to_dev(w), N, K, to_dev(codes), to_dev(scales), to_dev(sums),
                     workspace=workspace, library=library)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run(q4k, oracle_lib, w, N, K, x, rows=None, workspace="auto"):
    codes, scales, sums = oracle_lib.quantize_act(x)
    y = _gemm(q4k, w, N, K, codes, scales, sums, q4k.lib_gemm_int8(), workspace)
    ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows, parallel=True)
    if rows is not None:
        y = y[:, rows]
    return y, ref


def _close_where_no_cancellation(oracle_lib, y, ref, x, w, K, label):
    # outputs that cancel to below 2^-10 of sum |w x| are held to 2^-20 of that
    # sum instead (the contraction's error scales with sum |w x|, not |y|)
    codes, scales, _ = oracle_lib.quantize_act(x)
    xhat = np.abs(codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=1))
    mag = xhat @ np.abs(oracle_lib.dequant(w, K)).T
    cancel = mag > 2.0 ** 10 * np.abs(ref)
    assert cancel.mean() < 0.01
    assert_close(y[~cancel], ref[~cancel], label)
    assert (np.abs(y - ref)[cancel] <= 2.0 ** -20 * mag[cancel]).all()


@pytest.mark.parametrize("M,N,K", [(9, 33, 512), (63, 64, 256), (64, 65, 768), (65, 100, 2560),
                                   (129, 127, 4096), (512, 96, 9728), (200, 260, 6144),
                                   (300, 2560, 4096)])
def test_int8_gemm_shapes_and_tails(q4k, oracle_lib, M, N, K):
    w, _ = qi.make_q4k(N, K, 6000 + N + K)
    x = qi.make_act(M, K, 7000 + M + N)
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 50)])
    for ws in ("auto", None):
        y, ref = _run(q4k, oracle_lib, w, N, K, x, rows=rows, workspace=ws)
        assert_close(y, ref, "int8 gemm M=%d N=%d K=%d ws=%s" % (M, N, K, ws))


def test_int8_gemm_integer_exposing_bit_exact(q4k, oracle_lib):
    rng = np.random.default_rng(23)
    N, K, M = 96, 512, 70
    for j0 in range(8):
        f = qi.draw_q4k_fields(N, K, 600 + j0)
        f.d[:] = np.float16(1.0); f.dmin[:] = np.float16(0.0)
        f.sc[:] = 0; f.sc[:, :, j0] = 1
        w = qi.pack_q4k(f)
        x = rng.integers(-126, 127, size=(M, K)).astype(np.float32)
        x.reshape(M, K // 32, 32)[:, :, 0] = rng.choice([-127.0, 127.0], size=(M, K // 32))
        y, ref = _run(q4k, oracle_lib, w, N, K, x)
        D = oracle_lib.subblock_dots(w, N, K, oracle_lib.quantize_act(x)[0])
        assert (y == D[:, :, j0] + D[:, :, 8 + j0]).all()
        assert (y == ref).all()


@pytest.mark.parametrize("spread", [12, 20])
def test_int8_gemm_outlier_blocks(q4k, oracle_lib, spread):
    """The fp16 contraction's outlier case: block scales inside one
    super-block 2^spread apart (a tenth of the blocks large) and every 17th
    row scaled by 1e4."""
    N, K, M = 520, 2560, 150
    w = qi.make_q4k_bytes(N, K, 8900 + spread)
    rng = np.random.default_rng(8901)
    x = qi.make_act(M, K, 8902 + spread)
    blocks = x.reshape(M, K // 32, 32)
    big = rng.random((M, K // 32)) < 0.1
    blocks[big] *= np.float32(2.0 ** (spread / 2))
    blocks[~big] *= np.float32(2.0 ** (-spread / 2))
    x[::17] *= np.float32(1e4)
    y, ref = _run(q4k, oracle_lib, w, N, K, x)
    _close_where_no_cancellation(oracle_lib, y, ref, x, w, K, "int8 gemm outlier blocks 2^%d" % spread)


def test_int8_gemm_full_layer_every_output(q4k, oracle_lib):
    M, N, K = 512, 1024, 2560
    w, _ = qi.make_q4k(N, K, qi.weight_seed(2, 0, 0))
    x = qi.make_act(M, K, qi.act_seed(30000))
    y, ref = _run(q4k, oracle_lib, w, N, K, x)
    assert_close(y, ref, "int8 gemm 512 x 1024 x 2560, every output")


def test_int8_gemm_deterministic_batch_and_close_to_fp16(q4k, oracle_lib):
    import torch
    M, K = 512, 2560
    shapes = ((1024, 9000), (640, 9001))
    ws_ = [(qi.make_q4k(N, K, s)[0], N) for N, s in shapes]
    x = qi.make_act(M, K, 9100)
    codes, scales, sums = (to_dev(a) for a in oracle_lib.quantize_act(x))
    i8 = q4k.lib_gemm_int8()
    dev_w = [(to_dev(w), N) for w, N in ws_]
    a = [q4k.q4k_gemm(w, N, K, codes, scales, sums, library=i8) for w, N in dev_w]
    b = q4k.q4k_gemm_batch(dev_w, K, codes, scales, sums, library=i8)
    c = q4k.q4k_gemm_batch(dev_w, K, codes, scales, sums, library=i8)
    a0 = [q4k.q4k_gemm(w, N, K, codes, scales, sums, library=i8, workspace=None) for w, N in dev_w]
    b0 = q4k.q4k_gemm_batch(dev_w, K, codes, scales, sums, library=i8, workspace=None)
    f16 = q4k.q4k_gemm_batch(dev_w, K, codes, scales, sums)
    torch.cuda.synchronize()
    ws = q4k.gemm_workspace("cuda")
    assert int(ws[:65536].view(torch.int32).abs().sum().item()) == 0
    for (w, N), ya, yb, yc, ya0, yb0, yf in zip(ws_, a, b, c, a0, b0, f16):
        # the same call twice: the same bits; without a workspace (no split
        # tiles) the batched and single calls give the same bits too; with one,
        # the split of tiles differs between them (fp32 rounding of the parts)
        assert torch.equal(yb, yc) and torch.equal(ya0, yb0)
        assert_close(ya.cpu().numpy(), yb.cpu().numpy().astype(np.float64), "int8 single vs batch")
        # both contractions form the same exact block sums; they differ only in
        # where the fp32 roundings of the scales fall
        # (each within (K/32) * 2^-24 * sum |w x| of the exact value)
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
        qc, qs, _ = oracle_lib.quantize_act(x)
        ref = oracle_lib.matvec(w, N, K, qc, qs, rows=rows, parallel=True)
        assert_close(ya.cpu().numpy()[:, rows], ref, "int8 batch N=%d" % N)
        xhat = np.abs(qc.astype(np.float64) * np.repeat(qs.astype(np.float64), 32, axis=1))
        mag = xhat @ np.abs(oracle_lib.dequant(w, K)[rows]).T
        diff = np.abs(ya.cpu().numpy()[:, rows].astype(np.float64) - yf.cpu().numpy()[:, rows])
        assert (diff <= 2.0 ** -16 * mag).all()
