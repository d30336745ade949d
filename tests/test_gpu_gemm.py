"""GPU parity of q4k_gemm / q4k_gemm_batch (matrix-core prefill GEMM) against
the CPU oracle.

fp32 outputs within |gpu - oracle| <= max(2e-3 |oracle|, 1e-4).  Beyond random
inputs the cases pin what the format and the mathematics fix:
  - integer-exposing weights (d = 1, dmin = 0, one-hot sub-block scale) and
    integer activations with a +-127 per block reproduce the exact int32
    sub-block dots through the fp32 output (operand and result layouts);
  - an all-ones activation gives 127 * fl32(1/127) * (row sum of the
    dequantized weights), the closed form;
  - scaling d and dmin by 2^k and x by 2^k' scales y by exactly 2^(k+k');
  - activations with outlier blocks (block scales 2^12 apart inside one
    super-block) stay within tolerance;
  - every output of one full 512 x 2560 x 9728 layer (the down projection at a
    512-token prefill) is checked, split across workgroups as the benchmark
    launches it;
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


def _gemm(q4k, w, N, K, codes, scales, sums, workspace="auto"):
    import torch
    y = q4k.q4k_gemm(to_dev(w), N, K, to_dev(codes), to_dev(scales), to_dev(sums),
                     workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run(q4k, oracle_lib, w, N, K, x, rows=None, workspace="auto"):
    codes, scales, sums = oracle_lib.quantize_act(x)
    y = _gemm(q4k, w, N, K, codes, scales, sums, workspace)
    ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows, parallel=True)
    if rows is not None:
        y = y[:, rows]
    return y, ref


def _counters_zero(q4k):
    import torch
    ws = q4k.gemm_workspace("cuda")
    torch.cuda.synchronize()
    return int(ws[:65536].view(torch.int32).abs().sum().item()) == 0


def test_gemm_single_1024(q4k, oracle_lib):
    w, _ = qi.make_q4k(1024, 1024, qi.weight_seed(0, 0, 0))
    for M in (1, 2, 5, 16):
        x = qi.make_act(M, 1024, qi.act_seed(M))
        for ws in ("auto", None):
            y, ref = _run(q4k, oracle_lib, w, 1024, 1024, x, workspace=ws)
            assert_close(y, ref, "gemm 1024x1024 M=%d ws=%s" % (M, ws))


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (3, 33, 512), (63, 64, 256), (64, 65, 768),
                                   (65, 100, 2560), (100, 1000, 1280), (129, 127, 4096),
                                   (512, 96, 9728), (7, 4099, 256), (200, 260, 6144),
                                   (300, 2560, 4096)])
def test_gemm_shapes_and_tails(q4k, oracle_lib, M, N, K):
    w, _ = qi.make_q4k(N, K, 3000 + N + K)
    x = qi.make_act(M, K, 4000 + M + N)
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 50)])
    for ws in ("auto", None):
        y, ref = _run(q4k, oracle_lib, w, N, K, x, rows=rows, workspace=ws)
        assert_close(y, ref, "gemm M=%d N=%d K=%d ws=%s" % (M, N, K, ws))
    assert _counters_zero(q4k)


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


@pytest.mark.parametrize("proj", [0, 3, 4, 6])
def test_gemm_all_ones_closed_form(q4k, oracle_lib, proj):
    """x = 1 everywhere: codes 127, scale fl32(1/127), S = 32*127, so
    y[m][n] = 127 * fl32(1/127) * sum_k w[n][k] for every m (full projection
    shapes, M = 130 rows: a ragged tail in M)."""
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 1, proj))
    M = 130
    x = np.ones((M, K), np.float32)
    codes, scales, sums = oracle_lib.quantize_act(x)
    assert (codes == 127).all() and (scales == np.float32(1.0) / np.float32(127.0)).all()
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(proj).integers(0, N, 200)])
    wsum = oracle_lib.dequant(w.reshape(N, -1)[rows], K).sum(axis=1)
    closed = 127.0 * float(np.float32(1.0) / np.float32(127.0)) * wsum
    for ws in ("auto", None):
        y = _gemm(q4k, w, N, K, codes, scales, sums, ws)
        assert_close(y[:, rows], np.broadcast_to(closed, (M, rows.size)),
                     "all-ones %s ws=%s" % (name, ws))
    # whole tiles: every activation row is the same, so is every row of y
    assert (y == y[0]).all()


def test_gemm_power_of_two_scaling_exact(q4k, oracle_lib):
    """d, dmin -> 2^3 * (d, dmin) and x -> 2^-5 * x scale y by exactly 2^-2 (every
    value stays fp16-normal / fp32-normal, so every rounding scales with it)."""
    N, K, M = 300, 2560, 200
    f = qi.draw_q4k_fields(N, K, 8800)
    x = qi.make_act(M, K, 8801)
    w0 = qi.pack_q4k(f)
    f.d = (f.d.astype(np.float32) * 8).astype(np.float16)
    f.dmin = (f.dmin.astype(np.float32) * 8).astype(np.float16)
    w1 = qi.pack_q4k(f)
    c0, s0, u0 = oracle_lib.quantize_act(x)
    c1, s1, u1 = oracle_lib.quantize_act(x * np.float32(2.0 ** -5))
    assert (c0 == c1).all() and (s1 == s0 * np.float32(2.0 ** -5)).all()
    y0 = _gemm(q4k, w0, N, K, c0, s0, u0)
    y1 = _gemm(q4k, w1, N, K, c1, s1, u1)
    assert (y1 == y0 * np.float32(0.25)).all()
    assert_close(y0, oracle_lib.matvec(w0, N, K, c0, s0, parallel=True), "pow2 base")


@pytest.mark.parametrize("spread", [12, 16, 20])
def test_gemm_outlier_blocks(q4k, oracle_lib, spread):
    """Activation rows whose block scales inside one super-block differ by
    2^spread (a few outlier channels next to small ones), plus whole rows
    scaled by 1e4, against the oracle.  Some outputs are sums of terms far
    larger than the result itself; fp32 accumulation in any order cannot meet
    a 2e-3 relative bar on those, so outputs that cancel by more than 2^10
    (sum of |w x^| over |y|) are held to the fp32 accumulation bound
    2^-20 * sum |w x^| instead, and every other output to the bar.  Fewer than
    1 % of the outputs cancel that much."""
    N, K, M = 520, 2560, 150
    w = qi.make_q4k_bytes(N, K, 8900 + spread)
    rng = np.random.default_rng(8901)
    x = qi.make_act(M, K, 8902 + spread)
    blocks = x.reshape(M, K // 32, 32)
    big = rng.random((M, K // 32)) < 0.1
    blocks[big] *= np.float32(2.0 ** (spread / 2))
    blocks[~big] *= np.float32(2.0 ** (-spread / 2))
    x[::17] *= np.float32(1e4)
    codes, scales, sums = oracle_lib.quantize_act(x)
    s = scales.reshape(M, K // 256, 8)
    ratio = s.max(axis=2) / np.maximum(s.min(axis=2), np.float32(1e-30))
    assert (ratio >= 2.0 ** (spread - 2)).any()
    y, ref = _run(q4k, oracle_lib, w, N, K, x)
    xhat = np.abs(codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 32, axis=1))
    mag = xhat @ np.abs(oracle_lib.dequant(w, K)).T
    cancel = mag > 2.0 ** 10 * np.abs(ref)
    assert cancel.mean() < 0.01
    assert_close(y[~cancel], ref[~cancel], "outlier blocks 2^%d" % spread)
    assert (np.abs(y - ref)[cancel] <= 2.0 ** -20 * mag[cancel]).all()


def test_gemm_full_layer_every_output(q4k, oracle_lib):
    """The down projection of a 512-token prefill, 512 x 2560 x 9728: every one
    of the 1.3 M outputs against the oracle, with the workspace (tiles split
    across workgroups, as the benchmark runs it) and without."""
    name, K, N = qi.QWEN3_4B_LAYER[6]
    w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 0, 6))
    x = qi.make_act(512, K, qi.act_seed(20006))
    codes, scales, sums = oracle_lib.quantize_act(x)
    ref = oracle_lib.matvec(w, N, K, codes, scales, parallel=True)
    for ws in ("auto", None):
        y = _gemm(q4k, w, N, K, codes, scales, sums, ws)
        assert_close(y, ref, "full %s layer ws=%s" % (name, ws))


def test_gemm_deterministic(q4k, oracle_lib):
    """Repeated calls give identical bits, split (workspace) or not; the
    counters are zero after every call."""
    import torch
    M, K, Ns = 512, 4096, [2560]
    w = to_dev(qi.make_q4k_bytes(Ns[0], K, 9100))
    codes, scales, sums = (to_dev(a) for a in oracle_lib.quantize_act(qi.make_act(M, K, 9101)))
    for ws in ("auto", None):
        a = q4k.q4k_gemm(w, Ns[0], K, codes, scales, sums, workspace=ws)
        outs = [q4k.q4k_gemm(w, Ns[0], K, codes, scales, sums, workspace=ws) for _ in range(4)]
        torch.cuda.synchronize()
        for b in outs:
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "ws=%s" % ws
    assert _counters_zero(q4k)


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
    """M = 512 prompt tokens against each full-size projection; 100 random
    weight rows plus the first and last, all 512 activation rows."""
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 0, proj))
    x = qi.make_act(512, K, qi.act_seed(5000 + proj))
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(proj).integers(0, N, 100)])
    y, ref = _run(q4k, oracle_lib, w, N, K, x, rows=rows)
    assert_close(y, ref, "gemm %s M=512" % name)


@pytest.mark.parametrize("M,N,offset", [(512, 1024, 1), (129, 1023, 0), (129, 1023, 3)])
def test_gemm_output_layouts(q4k, oracle_lib, M, N, offset):
    """Few output tiles, so tiles are split across workgroups: y 16-byte
    aligned or only 4-byte aligned, N a multiple of 4 or not.  The floats
    around y stay untouched."""
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
                 "gemm M=%d N=%d offset=%d" % (M, N, offset))


_GEMM_BATCHES = {
    # name: (M, K, [N_i])
    "qkv_m512": (512, 2560, [4096, 1024, 1024]),
    "gate_up_m512": (512, 2560, [9728, 9728]),
    "ragged_m129": (129, 768, [1000, 33, 1, 257]),
    "eight_m40": (40, 512, [100, 200, 300, 1, 64, 65, 127, 128]),
    "m7_pair": (7, 1024, [513, 1023]),
    # up to 8 rows: the matrix-core GEMV over all products in one launch
    # where the launch's rows favour it (products found by tile index)
    "qkv_m4": (4, 2560, [4096, 1024, 1024]),
    "eight_m3": (3, 512, [100, 200, 300, 1, 64, 65, 127, 2048]),
    "eight_m8": (8, 768, [16, 17, 1, 300, 33, 48, 1000, 5]),
}


@pytest.mark.parametrize("name", sorted(_GEMM_BATCHES))
def test_gemm_batch_matches_single_and_oracle(q4k, oracle_lib, name):
    """Each product of a batched launch agrees with its own q4k_gemm call (to
    fp32 rounding: the split of tiles may differ; bit for bit without a
    workspace) and with the oracle on sampled rows."""
    import torch
    M, K, Ns = _GEMM_BATCHES[name]
    ws = [qi.make_q4k_bytes(N, K, 7300 + 17 * i + N) for i, N in enumerate(Ns)]
    x = qi.make_act(M, K, 7400 + M)
    codes, scales, sums = oracle_lib.quantize_act(x)
    dc, ds, dsu = to_dev(codes), to_dev(scales), to_dev(sums)
    dws = [to_dev(w) for w in ws]
    ys = q4k.q4k_gemm_batch(list(zip(dws, Ns)), K, dc, ds, dsu)
    singles = [q4k.q4k_gemm(w, N, K, dc, ds, dsu) for w, N in zip(dws, Ns)]
    ys0 = q4k.q4k_gemm_batch(list(zip(dws, Ns)), K, dc, ds, dsu, workspace=None)
    singles0 = [q4k.q4k_gemm(w, N, K, dc, ds, dsu, workspace=None) for w, N in zip(dws, Ns)]
    torch.cuda.synchronize()
    for i, (w, N, y, y1, z, z1) in enumerate(zip(ws, Ns, ys, singles, ys0, singles0)):
        assert torch.equal(z.view(torch.int32), z1.view(torch.int32)), "%s %d" % (name, i)
        a, b = y.cpu().numpy(), y1.cpu().numpy().astype(np.float64)
        assert_close(a, b, "%s product %d vs single" % (name, i))
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N + i).integers(0, N, 12)])
        ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
        assert_close(a[:, rows], ref, "%s product %d vs oracle" % (name, i))
        assert_close(z.cpu().numpy()[:, rows], ref, "%s product %d (no workspace)" % (name, i))


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


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_gemm_few_rows_run_the_gemv_bit_for_bit(q4k, oracle_lib, M):
    """Up to 8 rows q4k_gemm and q4k_gemm_batch run the streaming GEMV: the
    same bits as q4k_gemv, the batch (q|k|v of one layer, one launch) the same
    as the products one by one, and the oracle within tolerance."""
    import torch
    K = 2560
    shapes = [4096, 1024, 1024]
    ws = [qi.make_q4k_bytes(N, K, 3000 + N + M) for N in shapes]
    x = qi.make_act(M, K, 3100 + M)
    codes, scales, sums = oracle_lib.quantize_act(x)
    dc, dsc, dsu = to_dev(codes), to_dev(scales), to_dev(sums)
    dws = [to_dev(w) for w in ws]
    ys = q4k.q4k_gemm_batch([(w, N) for w, N in zip(dws, shapes)], K, dc, dsc, dsu)
    for w, dw, N, yb in zip(ws, dws, shapes, ys):
        y1 = q4k.q4k_gemm(dw, N, K, dc, dsc, dsu)
        y2 = q4k.q4k_gemv(dw, N, K, dc, dsc, dsu)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
        assert torch.equal(yb.view(torch.int32), y2.view(torch.int32))
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
        ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
        assert_close(y1.cpu().numpy()[:, rows], ref, "gemm M=%d N=%d" % (M, N))
