"""GPU parity of q4k_quantize_act and q4k_gemv against the CPU oracle.

Q8 codes, scales and sums must be bit-exact; GEMV outputs must be within
|gpu - oracle| <= max(2e-3 |oracle|, 1e-4) elementwise, and exactly equal in the
integer-exposing cases where the sub-block dots pass unrounded to the output.
"""
import json
import os

import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def q4k():
    import torch
    assert torch.cuda.is_available()
    import gemm_q4_super_amd as m
    m.lib()
    return m


def _gpu_quant(q4k, x, gate=None):
    import torch
    c, s, su = q4k.q4k_quantize_act(to_dev(x), None if gate is None else to_dev(gate))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), su.cpu().numpy()


def _gemv(q4k, w, N, K, x, oracle_lib, rows=None, use_gemm=False):
    import torch
    codes, scales, sums = oracle_lib.quantize_act(x)
    fn = q4k.q4k_gemm if use_gemm else q4k.q4k_gemv
    y = fn(to_dev(w), N, K, to_dev(codes), to_dev(scales), to_dev(sums))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle_lib.matvec(w, N, K, codes, scales, rows=rows)
    if rows is not None:
        y = y[:, rows]
    return y, ref


# -------------------------------------------------------------- quantizer ----

@pytest.mark.parametrize("M,K,scale", [(1, 1024, 1.0), (3, 2560, 1.0), (512, 4096, 1.0),
                                       (7, 9728, 1e-3), (2, 32, 300.0), (5, 96, 1.0)])
def test_quantize_bit_exact(q4k, oracle_lib, M, K, scale):
    x = qi.make_act(M, K, 77 + M) * np.float32(scale)
    x[0, :32] = 0.0                    # an all-zero block
    if K >= 96:
        x[-1, 64:96] = np.float32(-2.5)  # all-equal block: codes -127
    c, s, su = _gpu_quant(q4k, x)
    rc, rs, rsu = oracle_lib.quantize_act(x)
    assert (c == rc).all() and (su == rsu).all()
    assert (s.view(np.uint32) == rs.view(np.uint32)).all()


def test_quantize_golden_ties(q4k):
    cases = json.load(open(os.path.join(GOLDEN, "q8_ties.json")))["cases"]
    x = np.array([c["x"] for c in cases], np.float32)
    c, s, su = _gpu_quant(q4k, x)
    for i, case in enumerate(cases):
        assert c[i].tolist() == case["codes"]
        assert float(s[i, 0]) == case["scale"] and int(su[i, 0]) == case["sum"]


def test_quantize_near_rounding_boundaries(q4k, oracle_lib):
    """Quotients placed within a few ulps of k+1/2 decide codes by the last bit
    of the IEEE division; GPU and oracle must agree on every one."""
    rng = np.random.default_rng(5)
    rows = []
    for _ in range(256):
        amax = np.float32(rng.uniform(0.5, 8.0))
        s = amax / np.float32(127)
        blk = np.zeros(32, np.float32)
        blk[0] = amax
        for i in range(1, 32):
            k = int(rng.integers(0, 126))
            x0 = np.float32((k + 0.5) * float(s))
            blk[i] = np.float32(x0 + int(rng.integers(-3, 4)) * np.spacing(x0)) * rng.choice([-1, 1])
        rows.append(blk)
    x = np.stack(rows).reshape(8, -1)
    c, sc, su = _gpu_quant(q4k, x)
    rc, rs, rsu = oracle_lib.quantize_act(x)
    assert (c == rc).all() and (su == rsu).all() and (sc == rs).all()


def _wide_range_blocks(rng, nblk, emin, emax):
    """Blocks whose max|x| spans 2^emin .. 2^emax (subnormal to near overflow),
    each value placed within a few ulps of (k + 1/2) * scale, so every code is
    decided by the last bit of a correctly rounded quotient at that magnitude."""
    out = np.zeros((nblk, 32), np.float32)
    for b in range(nblk):
        amax = np.float32(np.ldexp(rng.uniform(1.0, 2.0), int(rng.integers(emin, emax + 1))))
        if amax == 0:
            amax = np.float32(np.ldexp(1.0, -149))
        s = amax / np.float32(127)
        out[b, 0] = amax
        for i in range(1, 32):
            x0 = np.float32((int(rng.integers(0, 127)) + 0.5) * float(s))
            x0 = np.float32(x0 + int(rng.integers(-3, 4)) * np.spacing(x0))
            out[b, i] = x0 * rng.choice([-1, 1])
    return out


def test_quantize_wide_range_scales(q4k, oracle_lib):
    """Scales from subnormal to ~2.7e36, including the tiny scales that take the
    IEEE division branch, agree with the oracle bit for bit."""
    rng = np.random.default_rng(11)
    x = _wide_range_blocks(rng, 512, -149, 127).reshape(16, -1)
    x[3, 64:96] = np.float32(np.ldexp(1.0, -149))     # all-equal subnormal block
    x[5, :32] = 0.0
    x[5, 1] = np.float32(-0.0)                          # zeros of both signs
    c, sc, su = _gpu_quant(q4k, x)
    rc, rs, rsu = oracle_lib.quantize_act(x)
    assert (c == rc).all() and (su == rsu).all()
    assert (sc.view(np.uint32) == rs.view(np.uint32)).all()


def test_quantize_gemv_wide_range_scales_bit_identical(q4k, oracle_lib):
    """The quantizer inside the fused GEMV gives the same codes as
    q4k_quantize_act for scales far from those of ordinary activations."""
    import torch
    N, K = 300, 2560
    rng = np.random.default_rng(12)
    x = _wide_range_blocks(rng, K // 32, -140, 60).reshape(1, K)
    w = qi.make_q4k_bytes(N, K, 4242)
    wd, xd = to_dev(w), to_dev(x)
    y1 = q4k.q4k_quantize_gemv(wd, N, K, xd)
    c, s, su = q4k.q4k_quantize_act(xd)
    y2 = q4k.q4k_gemv(wd, N, K, c, s, su)
    torch.cuda.synchronize()
    rc, rs, rsu = oracle_lib.quantize_act(x)
    assert (c.cpu().numpy() == rc).all() and (su.cpu().numpy() == rsu).all()
    assert (y1.cpu().numpy().view(np.uint32) == y2.cpu().numpy().view(np.uint32)).all()


def test_quantize_swiglu_bit_exact(q4k, oracle_lib):
    M, K = 16, 1024
    g = qi.make_act(M, K, 5) * np.float32(4.0)
    u = qi.make_act(M, K, 6) * np.float32(4.0)
    c, s, su = _gpu_quant(q4k, u, gate=g)
    rc, rs, rsu = oracle_lib.quantize_act(oracle_lib.swiglu(g, u))
    # h is evaluated in fp64 and rounded once on both sides; the two exp()
    # implementations may differ by an ulp of fp64, which flips the fp32 h (and
    # possibly a code) with probability ~1e-9 per element.
    assert (c == rc).all() and (su == rsu).all() and (s == rs).all()


# ------------------------------------------------------------------- GEMV ----

def test_gemv_single_1024(q4k, oracle_lib):
    """1024 x 1024 Q4_K weight (4 super-blocks per row), batch 1, all outputs."""
    w, _ = qi.make_q4k(1024, 1024, qi.weight_seed(0, 0, 0))
    x = qi.make_act(1, 1024, qi.act_seed(0))
    y, ref = _gemv(q4k, w, 1024, 1024, x, oracle_lib)
    assert_close(y, ref, "gemv 1024x1024")


@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (9, 768), (33, 2560), (100, 4096),
                                 (257, 9728), (1000, 1280), (4097, 2560), (63, 6144)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_gemv_shapes_and_tails(q4k, oracle_lib, N, K, M):
    w, _ = qi.make_q4k(N, K, 1000 + N + K)
    x = qi.make_act(M, K, 2000 + N + M)
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 60)])
    y, ref = _gemv(q4k, w, N, K, x, oracle_lib, rows=rows)
    assert_close(y, ref, "gemv N=%d K=%d M=%d" % (N, K, M))


def test_gemv_integer_exposing_bit_exact(q4k, oracle_lib):
    """d=1, dmin=0, one-hot sub-block scale, integer activations with a +-127 in
    every block: each output is an exact integer sub-block dot (< 2^24)."""
    rng = np.random.default_rng(9)
    N, K, M = 64, 256, 4
    for j0 in range(8):
        f = qi.draw_q4k_fields(N, K, 300 + j0)
        f.d[:] = np.float16(1.0); f.dmin[:] = np.float16(0.0)
        f.sc[:] = 0; f.sc[:, :, j0] = 1
        w = qi.pack_q4k(f)
        x = rng.integers(-126, 127, size=(M, K)).astype(np.float32)
        x.reshape(M, 8, 32)[:, :, 0] = rng.choice([-127.0, 127.0], size=(M, 8))
        y, ref = _gemv(q4k, w, N, K, x, oracle_lib)
        D = oracle_lib.subblock_dots(w, N, K, oracle_lib.quantize_act(x)[0])
        assert (y == D[:, :, j0]).all()
        assert (y == ref).all()
        # mins only: y = -S_j0
        f.q[:] = 0; f.sc[:] = 0; f.dmin[:] = np.float16(1.0); f.mn[:] = 0; f.mn[:, :, j0] = 1
        y, ref = _gemv(q4k, qi.pack_q4k(f), N, K, x, oracle_lib)
        assert (y == ref).all()


def test_gemv_all_ones_closed_form(q4k, oracle_lib):
    N, K = 512, 2560
    w, f = qi.make_q4k(N, K, 17)
    x = np.ones((1, K), np.float32)
    y, ref = _gemv(q4k, w, N, K, x, oracle_lib)
    jj = np.arange(256) // 32
    wf = (f.d.astype(np.float64)[:, :, None] * f.sc[:, :, jj] * f.q
          - f.dmin.astype(np.float64)[:, :, None] * f.mn[:, :, jj]).reshape(N, K)
    closed = 127.0 * float(np.float32(1) / np.float32(127)) * wf.sum(axis=1)
    assert_close(y[0], closed, "all-ones")
    assert_close(y, ref, "all-ones vs oracle")


def test_gemv_zero_scales_exact_zero(q4k, oracle_lib):
    f = qi.draw_q4k_fields(40, 512, 8)
    f.d[:] = 0; f.dmin[:] = 0
    y, _ = _gemv(q4k, qi.pack_q4k(f), 40, 512, qi.make_act(3, 512, 1), oracle_lib)
    assert (y == 0).all()


def test_gemv_power_of_two_scaling_bit_identical(q4k, oracle_lib):
    N, K = 300, 2560
    w, f = qi.make_q4k(N, K, 12)
    x = qi.make_act(2, K, 13)
    y, _ = _gemv(q4k, w, N, K, x, oracle_lib)
    f.d = (f.d * np.float16(4)).astype(np.float16)
    f.dmin = (f.dmin * np.float16(4)).astype(np.float16)
    y4, _ = _gemv(q4k, qi.pack_q4k(f), N, K, x, oracle_lib)
    assert (y4 == 4 * y).all()


@pytest.mark.parametrize("proj", range(7))
def test_gemv_qwen3_4b_shapes_sampled(q4k, oracle_lib, proj):
    """Full-size decode projections; 64 random rows plus the first and last
    checked against the oracle (M = 1 and M = 8)."""
    name, K, N = qi.QWEN3_4B_LAYER[proj]
    w = qi.make_q4k_bytes(N, K, qi.weight_seed(1, 0, proj))
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(proj).integers(0, N, 64)])
    for M in (1, 8):
        x = qi.make_act(M, K, qi.act_seed(proj * 10 + M))
        y, ref = _gemv(q4k, w, N, K, x, oracle_lib, rows=rows)
        assert_close(y, ref, "gemv %s M=%d" % (name, M))


# ------------------------------------------------- fused quantize + GEMV ----

@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (37, 512, 2), (1000, 2560, 1), (4096, 2560, 1),
                                   (2560, 4096, 1), (2560, 9728, 1), (9728, 2560, 1),
                                   (300, 4096, 8), (129, 6144, 5), (2048, 16384, 2),
                                   (64, 32768, 1), (16, 256, 2), (17, 2560, 3), (1000, 2560, 4),
                                   (33, 1024, 6), (129, 3840, 7), (4097, 4096, 8),
                                   (2560, 4096, 8), (1024, 2560, 8), (2048, 512, 4),
                                   (4096, 768, 3), (2049, 1280, 5), (2500, 3328, 6),
                                   # the down projection's width at small batches, and the
                                   # widest rows the LDS takes per M
                                   (2560, 9728, 4), (2560, 9728, 8), (1000, 12288, 6),
                                   (300, 15872, 8), (500, 31744, 4), (64, 49152, 1)])
def test_quantize_gemv_bit_identical_to_two_step(q4k, oracle_lib, N, K, M):
    """One launch (quantize inside the GEMV) equals q4k_quantize_act followed
    by q4k_gemv bit for bit, and the oracle within tolerance.  For M = 2..8 the
    second call runs the matrix-core GEMV, the first the streaming one: the two
    must form every super-block term and row sum the same way."""
    import torch
    w = qi.make_q4k_bytes(N, K, 7000 + N + K)
    x = qi.make_act(M, K, 8000 + M + K)
    x[0, :32] = 0.0
    wd, xd = to_dev(w), to_dev(x)
    y1 = q4k.q4k_quantize_gemv(wd, N, K, xd)
    c, s, su = q4k.q4k_quantize_act(xd)
    y2 = q4k.q4k_gemv(wd, N, K, c, s, su)
    torch.cuda.synchronize()
    y1, y2 = y1.cpu().numpy(), y2.cpu().numpy()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
    rc, rs, _ = oracle_lib.quantize_act(x)
    ref = oracle_lib.matvec(w, N, K, rc, rs, rows=rows)
    assert_close(y1 if rows is None else y1[:, rows], ref, "quantize_gemv N=%d K=%d M=%d" % (N, K, M))


@pytest.mark.parametrize("N,K,M", [(2560, 4096, 8), (4096, 2560, 4), (2100, 1536, 5)])
def test_gemv_unaligned_scales_same_bits(q4k, oracle_lib, N, K, M):
    """Q8 scales and sums that are only 4-byte aligned take the streaming GEMV
    instead of the matrix-core one; both give the same bits."""
    import torch
    w = qi.make_q4k_bytes(N, K, 7700 + N + M)
    x = qi.make_act(M, K, 7800 + K + M)
    wd = to_dev(w)
    c, s, su = q4k.q4k_quantize_act(to_dev(x))
    s_buf = torch.empty(s.numel() + 1, dtype=torch.float32, device="cuda")
    su_buf = torch.empty(su.numel() + 1, dtype=torch.int32, device="cuda")
    s_off, su_off = s_buf[1:].view(s.shape), su_buf[1:].view(su.shape)
    s_off.copy_(s)
    su_off.copy_(su)
    assert s_off.data_ptr() % 16 == 4 and su_off.data_ptr() % 16 == 4
    y1 = q4k.q4k_gemv(wd, N, K, c, s, su)
    y2 = q4k.q4k_gemv(wd, N, K, c, s_off, su_off)
    torch.cuda.synchronize()
    y1, y2 = y1.cpu().numpy(), y2.cpu().numpy()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 40)])
    rc, rs, _ = oracle_lib.quantize_act(x)
    assert_close(y1[:, rows], oracle_lib.matvec(w, N, K, rc, rs, rows=rows),
                 "gemv N=%d K=%d M=%d" % (N, K, M))


# ------------------------------------------- batched quantize + GEMV ----

_BATCHES = {
    "qkv": (2560, 1, [4096, 1024, 1024]),
    "gate_up": (2560, 1, [9728, 9728]),
    "qkv_m2": (2560, 2, [4096, 1024, 1024]),
    "ragged_m3": (512, 3, [1, 37, 300, 4097, 8, 9]),
    "eight_m1": (1024, 1, [5, 17, 64, 129, 1000, 2048, 3, 700]),
    "eight_m2_t2": (768, 2, [1000, 1000, 1000, 1000, 70, 1, 33, 2]),
    "m8": (4096, 8, [300, 257]),
    "single": (9728, 1, [2560]),
    "down_m8": (9728, 8, [2560, 1000]),
}


@pytest.mark.parametrize("name", sorted(_BATCHES))
def test_quantize_gemv_batch_bit_identical_to_single(q4k, oracle_lib, name):
    """Each product of a batched launch equals q4k_quantize_gemv on it alone
    bit for bit (also where the batch's size picks a different row tiling),
    and the oracle within tolerance."""
    import torch
    K, M, Ns = _BATCHES[name]
    ws = [qi.make_q4k_bytes(N, K, 9100 + i + N) for i, N in enumerate(Ns)]
    xs = [qi.make_act(M, K, 9300 + i + M) for i in range(len(Ns))]
    xs[0][0, :32] = 0.0
    wd = [to_dev(w) for w in ws]
    xd = [to_dev(x) for x in xs]
    yb = q4k.q4k_quantize_gemv_batch([(w, N, x) for w, N, x in zip(wd, Ns, xd)], K)
    ys = [q4k.q4k_quantize_gemv(w, N, K, x) for w, N, x in zip(wd, Ns, xd)]
    torch.cuda.synchronize()
    for i, N in enumerate(Ns):
        a, b = yb[i].cpu().numpy(), ys[i].cpu().numpy()
        assert a.shape == (M, N)
        assert (a.view(np.uint32) == b.view(np.uint32)).all(), "problem %d" % i
        rows = None if N <= 300 else np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 24)])
        rc, rs, _ = oracle_lib.quantize_act(xs[i])
        ref = oracle_lib.matvec(ws[i], N, K, rc, rs, rows=rows)
        assert_close(a if rows is None else a[:, rows], ref, "batch %s problem %d" % (name, i))


@pytest.mark.parametrize("group", ["qkv", "o", "gate_up", "down"])
def test_quantize_gemv_batch_row_shard_bit_identical(q4k, oracle_lib, group):
    """One GPU's share of an 8-way row shard of a decode launch group: the
    first N/8 rows of each matrix (a prefix of its bytes) give, row for row,
    the same bits as the full launch (a row's sum does not depend on the
    launch shape), and the oracle within tolerance."""
    import torch
    idx = {"qkv": (0, 1, 2), "o": (3,), "gate_up": (4, 5), "down": (6,)}[group]
    K = qi.QWEN3_4B_LAYER[idx[0]][1]
    Ns = [qi.QWEN3_4B_LAYER[p][2] for p in idx]
    ws = [qi.make_q4k_bytes(N, K, qi.weight_seed(1, 5, p)) for N, p in zip(Ns, idx)]
    xs = [qi.make_act(1, K, qi.act_seed(500 + p)) for p in idx]
    wd = [to_dev(w) for w in ws]
    xd = [to_dev(x) for x in xs]
    full = q4k.q4k_quantize_gemv_batch([(w, N, x) for w, N, x in zip(wd, Ns, xd)], K)
    shard = q4k.q4k_quantize_gemv_batch([(w, N // 8, x) for w, N, x in zip(wd, Ns, xd)], K)
    torch.cuda.synchronize()
    for i, N in enumerate(Ns):
        a, b = shard[i].cpu().numpy(), full[i].cpu().numpy()[:, :N // 8]
        assert (a.view(np.uint32) == b.view(np.uint32)).all(), "%s problem %d" % (group, i)
        rows = np.unique(np.r_[0, N // 8 - 1, np.random.default_rng(N).integers(0, N // 8, 24)])
        rc, rs, _ = oracle_lib.quantize_act(xs[i])
        ref = oracle_lib.matvec(ws[i], N, K, rc, rs, rows=rows)
        assert_close(a[:, rows], ref, "shard %s problem %d" % (group, i))


def test_quantize_gemv_batch_leaves_other_memory_untouched(q4k):
    """Outputs are written only inside each [M, N_i] block: guard words around
    every output survive."""
    import torch
    K, M, Ns = 512, 2, [3, 40, 9]
    pad = 64
    buf = torch.full((sum(M * N + 2 * pad for N in Ns),), 12345.0, device="cuda")
    probs, views, off = [], [], 0
    for i, N in enumerate(Ns):
        off += pad
        y = buf[off:off + M * N].view(M, N)
        views.append((off, M * N))
        off += M * N + pad
        probs.append((to_dev(qi.make_q4k_bytes(N, K, 50 + i)), N, to_dev(qi.make_act(M, K, 60 + i))))
    q4k.q4k_quantize_gemv_batch(probs, K, ys=[buf[o:o + n].view(M, -1) for o, n in views])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    mask = np.ones(h.shape, bool)
    for o, n in views:
        mask[o:o + n] = False
    assert (h[mask] == 12345.0).all()
