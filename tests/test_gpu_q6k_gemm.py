"""GPU parity of q6k_gemm (the Q6_K prefill GEMM on the matrix cores) against
the CPU oracle.

fp32 outputs within |gpu - oracle| <= max(2e-3 |oracle|, 1e-4).  Beyond random
inputs (ragged N, M across tile edges, odd super-block counts that put every
other row at addresses 2 mod 4):
  - integer-exposing weights (d = 1, small scales) and integer activations with
    a +-127 in every block pass the integer dot unrounded to the output: the
    operand layout, both weight parts and the scale index are checked bit for
    bit;
  - extreme scales (-128, 127) with extreme quants (0, 63) stay exact in the
    fp16 operands;
  - an all-ones activation gives the closed form 127 * fl32(1/127) * row sum;
  - the seven Qwen3-4B projection shapes at a 512-token prefill, sampled rows;
  - repeated calls give the same bits, with or without a workspace.
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


def _gemm(q4k, w, N, K, codes, scales, workspace="auto"):
    import torch
    y = q4k.q6k_gemm(to_dev(w), N, K, to_dev(codes), to_dev(scales), workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (37, 512, 5), (129, 768, 33), (300, 2560, 65),
                                   (1000, 1280, 130), (257, 3328, 200), (64, 4096, 300),
                                   (2048, 256, 17), (130, 9728, 64)])
def test_q6k_gemm_shapes_and_tails(q4k, oracle_lib, N, K, M):
    print("q6k_gemm N=%d K=%d M=%d" % (N, K, M), flush=True)
    w = qi.make_q6k_bytes(N, K, 900 + N + K)
    x = qi.make_act(M, K, 910 + M + K)
    x[0, :32] = 0.0
    codes, scales, _ = oracle_lib.quantize_act(x)
    y = _gemm(q4k, w, N, K, codes, scales)
    ref = oracle_lib.q6k_matvec(w, N, K, codes, scales, parallel=True)
    assert_close(y, ref, "q6k_gemm N=%d K=%d M=%d" % (N, K, M))


def test_q6k_gemm_integer_exposing_bit_exact(q4k, oracle_lib):
    rng = np.random.default_rng(31)
    N, K, M = 160, 768, 70
    f = qi.draw_q6k_fields(N, K, 930)
    f.d[:] = np.float16(1.0)
    f.sc[:] = rng.integers(-3, 4, size=f.sc.shape).astype(np.int8)
    w = qi.pack_q6k(f)
    x = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    x[:, ::32] = 127.0
    codes, scales, _ = oracle_lib.quantize_act(x)
    assert (scales == 1.0).all()
    y = _gemm(q4k, w, N, K, codes, scales)
    ref = oracle_lib.q6k_matvec(w, N, K, codes, scales)
    assert np.abs(ref).max() < 2 ** 24
    assert (y == ref).all()


def test_q6k_gemm_extreme_scales_and_quants(q4k, oracle_lib):
    rng = np.random.default_rng(32)
    N, K, M = 200, 1280, 90
    f = qi.draw_q6k_fields(N, K, 940)
    f.sc[:] = rng.choice(np.array([-128, 127, -127, 1], np.int8), size=f.sc.shape)
    f.q[:] = rng.choice(np.array([0, 63, 31, 32], np.uint8), size=f.q.shape)
    w = qi.pack_q6k(f)
    x = qi.make_act(M, K, 941)
    codes, scales, _ = oracle_lib.quantize_act(x)
    y = _gemm(q4k, w, N, K, codes, scales)
    assert_close(y, oracle_lib.q6k_matvec(w, N, K, codes, scales, parallel=True),
                 "q6k_gemm extreme scales")


def test_q6k_gemm_all_ones_closed_form(q4k, oracle_lib):
    N, K, M = 300, 1024, 40
    w, f = qi.make_q6k(N, K, 950)
    codes, scales, _ = oracle_lib.quantize_act(np.ones((M, K), np.float32))
    y = _gemm(q4k, w, N, K, codes, scales)
    j = np.arange(256) // 16
    wf = (f.d.astype(np.float64)[:, :, None] * f.sc.astype(np.float64)[:, :, j] *
          (f.q.astype(np.float64) - 32.0)).reshape(N, K)
    d_a = float(np.float32(1.0) / np.float32(127.0))
    want = np.broadcast_to(127.0 * d_a * wf.sum(axis=1), (M, N))
    assert_close(y, want, "q6k_gemm all-ones closed form")


@pytest.mark.parametrize("proj", range(7))
def test_q6k_gemm_qwen3_4b_m512_sampled(q4k, oracle_lib, proj):
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    M = 512
    print("q6k_gemm %s M=%d" % (name, M), flush=True)
    w = qi.make_q6k_bytes(N, K, 960 + proj)
    codes, scales, _ = oracle_lib.quantize_act(qi.make_act(M, K, 970 + proj))
    y = _gemm(q4k, w, N, K, codes, scales)
    rows = np.unique(np.r_[0, 1, N - 1, np.random.default_rng(proj).integers(0, N, 60)])
    ref = oracle_lib.q6k_matvec(w, N, K, codes, scales, rows=rows, parallel=True)
    assert_close(y[:, rows], ref, "q6k_gemm %s" % name)


def test_q6k_gemm_deterministic_with_and_without_workspace(q4k, oracle_lib):
    N, K, M = 2560, 9728, 512
    w = qi.make_q6k_bytes(N, K, 980)
    codes, scales, _ = oracle_lib.quantize_act(qi.make_act(M, K, 981))
    a = _gemm(q4k, w, N, K, codes, scales)
    b = _gemm(q4k, w, N, K, codes, scales)
    c = _gemm(q4k, w, N, K, codes, scales, workspace=None)
    assert (a.view(np.uint32) == b.view(np.uint32)).all()
    # split tiles add their parts in another grouping: fp32 rounding of the
    # sums, a few units of 2^-24 of the outputs' magnitude
    assert np.abs(c - a).max() <= 2e-6 * np.abs(a).max()
