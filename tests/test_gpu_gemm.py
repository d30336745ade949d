"""GPU parity of q4k_gemm (matrix-core prefill GEMM) against the CPU oracle.

fp32 outputs within |gpu - oracle| <= max(2e-3 |oracle|, 1e-4); the
integer-exposing cases (d = 1, dmin = 0, one-hot sub-block scale, integer
activations with a +-127 per block) must reproduce the exact int32 sub-block
dots through the fp32 output, which also pins the matrix-core operand and
result layouts.
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


def _run(q4k, oracle_lib, w, N, K, x, rows=None):
    import torch
    codes, scales, sums = oracle_lib.quantize_act(x)
    y = q4k.q4k_gemm(to_dev(w), N, K, to_dev(codes), to_dev(scales), to_dev(sums))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
    if rows is not None:
        y = y[:, rows]
    return y, ref


def test_gemm_single_1024(q4k, oracle_lib):
    w, _ = qi.make_q4k(1024, 1024, qi.weight_seed(0, 0, 0))
    for M in (1, 2, 5, 16):
        x = qi.make_act(M, 1024, qi.act_seed(M))
        y, ref = _run(q4k, oracle_lib, w, 1024, 1024, x)
        assert_close(y, ref, "gemm 1024x1024 M=%d" % M)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 33, 512), (63, 64, 256), (64, 65, 768),
                                   (65, 100, 2560), (100, 1000, 1280), (129, 127, 4096),
                                   (512, 96, 9728), (7, 4099, 256), (200, 260, 6144)])
def test_gemm_shapes_and_tails(q4k, oracle_lib, M, N, K):
    w, _ = qi.make_q4k(N, K, 3000 + N + K)
    x = qi.make_act(M, K, 4000 + M + N)
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 50)])
    y, ref = _run(q4k, oracle_lib, w, N, K, x, rows=rows)
    assert_close(y, ref, "gemm M=%d N=%d K=%d" % (M, N, K))


def test_gemm_integer_exposing_bit_exact(q4k, oracle_lib):
    rng = np.random.default_rng(19)
    N, K, M = 96, 512, 70
    for j0 in range(8):
        f = qi.draw_q4k_fields(N, K, 500 + j0)
        f.d[:] = np.float16(1.0); f.dmin[:] = np.float16(0.0)
        f.sc[:] = 0; f.sc[:, :, j0] = 1
        w = qi.pack_q4k(f)
        x = rng.integers(-126, 127, size=(M, K)).astype(np.float32)
        x.reshape(M, K // 32, 32)[:, :, 0] = rng.choice([-127.0, 127.0], size=(M, K // 32))
        y, ref = _run(q4k, oracle_lib, w, N, K, x)
        D = oracle_lib.subblock_dots(w, N, K, oracle_lib.quantize_act(x)[0])
        assert (y == D[:, :, j0] + D[:, :, 8 + j0]).all()
        assert (y == ref).all()
        # mins only: y = -(S_j0 of super-block 0 + S_j0 of super-block 1)
        f.q[:] = 0; f.sc[:] = 0; f.dmin[:] = np.float16(1.0); f.mn[:] = 0; f.mn[:, :, j0] = 1
        y, ref = _run(q4k, oracle_lib, qi.pack_q4k(f), N, K, x)
        assert (y == ref).all()


def test_gemm_matches_gemv_small_m(q4k, oracle_lib):
    import torch
    N, K = 777, 2560
    w, _ = qi.make_q4k(N, K, 44)
    for M in (1, 4, 8):
        x = qi.make_act(M, K, 45 + M)
        codes, scales, sums = (to_dev(a) for a in oracle_lib.quantize_act(x))
        wd = to_dev(w)
        a = q4k.q4k_gemm(wd, N, K, codes, scales, sums)
        b = q4k.q4k_gemv(wd, N, K, codes, scales, sums)
        torch.cuda.synchronize()
        assert_close(a.cpu().numpy(), b.cpu().numpy().astype(np.float64), "gemm vs gemv M=%d" % M)


@pytest.mark.parametrize("proj", range(7))
def test_gemm_qwen3_4b_prefill_shapes_sampled(q4k, oracle_lib, proj):
    """M = 512 prompt tokens against each full-size projection; 40 random weight
    rows plus the first and last, all 512 activation rows."""
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 0, proj))
    x = qi.make_act(512, K, qi.act_seed(5000 + proj))
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(proj).integers(0, N, 40)])
    y, ref = _run(q4k, oracle_lib, w, N, K, x, rows=rows)
    assert_close(y, ref, "gemm %s M=512" % name)


@pytest.mark.parametrize("M,N,offset", [(512, 1024, 1), (129, 1023, 0), (129, 1023, 3)])
def test_gemm_split_k_output_layouts(q4k, oracle_lib, M, N, offset):
    """Few output tiles, so K is split and the parts add into a zero-filled y:
    y 16-byte aligned or only 4-byte aligned, M*N a multiple of 4 or not.  The
    floats around y stay untouched."""
    import torch
    K = 2560
    w, _ = qi.make_q4k(N, K, 7100 + N)
    x = qi.make_act(M, K, 7200 + M)
    codes, scales, sums = oracle_lib.quantize_act(x)
    buf = torch.full((M * N + 8,), 7.0, dtype=torch.float32, device="cuda")
    y = buf[offset:offset + M * N].view(M, N)
    q4k.q4k_gemm(to_dev(w), N, K, to_dev(codes), to_dev(scales), to_dev(sums), y=y)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[:offset] == 7.0).all() and (got[offset + M * N:] == 7.0).all()
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
    ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
    assert_close(got[offset:offset + M * N].reshape(M, N)[:, rows], ref,
                 "gemm split M=%d N=%d offset=%d" % (M, N, offset))


_GEMM_BATCHES = {
    # name: (M, K, [N_i])
    "qkv_m512": (512, 2560, [4096, 1024, 1024]),
    "gate_up_m512": (512, 2560, [9728, 9728]),
    "ragged_m129": (129, 768, [1000, 33, 1, 257]),
    "eight_m40": (40, 512, [100, 200, 300, 1, 64, 65, 127, 128]),
    "m7_pair": (7, 1024, [513, 1023]),
}


@pytest.mark.parametrize("name", sorted(_GEMM_BATCHES))
def test_gemm_batch_matches_single_and_oracle(q4k, oracle_lib, name):
    """Each product of a batched launch agrees with its own q4k_gemm call (to
    fp32 rounding: the K split may differ) and with the oracle on sampled rows."""
    import torch
    M, K, Ns = _GEMM_BATCHES[name]
    ws = [qi.make_q4k_bytes(N, K, 7300 + 17 * i + N) for i, N in enumerate(Ns)]
    x = qi.make_act(M, K, 7400 + M)
    codes, scales, sums = oracle_lib.quantize_act(x)
    dc, ds, dsu = to_dev(codes), to_dev(scales), to_dev(sums)
    dws = [to_dev(w) for w in ws]
    ys = q4k.q4k_gemm_batch(list(zip(dws, Ns)), K, dc, ds, dsu)
    singles = [q4k.q4k_gemm(w, N, K, dc, ds, dsu) for w, N in zip(dws, Ns)]
    torch.cuda.synchronize()
    for i, (w, N, y, y1) in enumerate(zip(ws, Ns, ys, singles)):
        a, b = y.cpu().numpy(), y1.cpu().numpy().astype(np.float64)
        assert_close(a, b, "%s product %d vs single" % (name, i))
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N + i).integers(0, N, 12)])
        ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
        assert_close(a[:, rows], ref, "%s product %d vs oracle" % (name, i))


def test_gemm_batch_leaves_other_memory_untouched(q4k, oracle_lib):
    """Outputs of a batch packed into one buffer with gaps: the gaps keep their
    values (no product writes outside its own y)."""
    import torch
    M, K, Ns = 70, 512, [300, 5, 129]
    ws = [to_dev(qi.make_q4k_bytes(N, K, 7500 + N)) for N in Ns]
    codes, scales, sums = (to_dev(a) for a in oracle_lib.quantize_act(qi.make_act(M, K, 75)))
    gap = 64
    total = sum(M * N for N in Ns) + gap * (len(Ns) + 1)
    buf = torch.full((total,), -3.0, dtype=torch.float32, device="cuda")
    ys, off = [], gap
    for N in Ns:
        ys.append(buf[off:off + M * N].view(M, N))
        off += M * N + gap
    q4k.q4k_gemm_batch(list(zip(ws, Ns)), K, codes, scales, sums, ys=ys)
    torch.cuda.synchronize()
    host, off = buf.cpu().numpy(), 0
    for N in Ns:
        assert (host[off:off + gap] == -3.0).all()
        off += gap + M * N
    assert (host[off:] == -3.0).all()
