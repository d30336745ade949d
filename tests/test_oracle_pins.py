"""Pins of the CPU oracle against what the Q4_K/Q8 formats and the mathematics fix.

None of these compares the oracle with itself: each checks it against a value
worked out by hand (tests/golden), a closed form, an exact invariant, or a
brute force from the unpacked fields that never goes through the oracle's
byte decoding.  A plausible mistake anywhere in the oracle (a swapped nibble, a
wrong 6-bit scale index, a dropped or sign-flipped min term, round-half-away
instead of half-even, reciprocal instead of division, a wrong expert or slot in
the routed sum) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import q4k_inputs as qi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _block_bytes(b):
    sb = np.zeros(144, np.uint8)
    sb[0:2] = np.array([int(b["d_bits"], 16)], "<u2").view(np.uint8)
    sb[2:4] = np.array([int(b["dmin_bits"], 16)], "<u2").view(np.uint8)
    sb[4:16] = np.array(b["scale_bytes"], np.uint8)
    for k, v in b["qs"].items():
        sb[16 + int(k)] = v
    return sb


def _fields_to_w(f: qi.Q4KFields) -> np.ndarray:
    """fp64 weights straight from the drawn fields (no byte decoding)."""
    N, nsb, _ = f.q.shape
    j = np.arange(256) // 32
    d = f.d.astype(np.float64)[:, :, None]
    dm = f.dmin.astype(np.float64)[:, :, None]
    w = d * f.sc.astype(np.float64)[:, :, j] * f.q - dm * f.mn.astype(np.float64)[:, :, j]
    return w.reshape(N, nsb * 256)


# ---------------------------------------------------------------- format ----

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_golden_superblock_unpack(oracle_lib, idx):
    b = _load("q4k_superblock_handbuilt.json")["blocks"][idx]
    sb = _block_bytes(b)
    d, dmin, sc, mn, q = oracle_lib.unpack_q4k(sb)
    assert d == b["d"] and dmin == b["dmin"]
    assert sc.tolist() == b["sc"] and mn.tolist() == b["mn"]
    expect_q = np.zeros(256, np.int32)
    for k, v in b["q_nonzero"].items():
        expect_q[int(k)] = v
    assert q.tolist() == expect_q.tolist()
    w = oracle_lib.dequant(sb, 256)[0]
    for k, v in b["w_expected"].items():
        assert w[int(k)] == v, (k, w[int(k)], v)
    if "row_sum" in b:
        assert w.sum() == b["row_sum"]


def test_golden_residual_matvec(oracle_lib):
    """y = residual + W x with one-hot Q8 rows (code 1, scale 1) picks single
    hand-worked weights of the golden blocks: y[m, n] = w_n[k_m] + r[m, n]
    exactly.  Distinct k per row and r per (m, n) catch a transposed residual
    or a row / column mix-up."""
    blocks = _load("q4k_superblock_handbuilt.json")["blocks"][:2]
    w = np.concatenate([_block_bytes(b) for b in blocks])
    ks = sorted(set(int(k) for k in blocks[0]["w_expected"]) &
                set(int(k) for k in blocks[1]["w_expected"]))[:3]
    assert len(ks) >= 2
    M, N, K = len(ks), 2, 256
    codes = np.zeros((M, K), np.int8)
    for m, k in enumerate(ks):
        codes[m, k] = 1
    scales = np.ones((M, K // 32), np.float32)
    r = np.array([[0.25 * (1 + m) - 4.0 * n for n in range(N)] for m in range(M)])
    y = oracle_lib.matvec_residual(w, N, K, codes, scales, r)
    for m, k in enumerate(ks):
        for n in range(N):
            assert y[m, n] == blocks[n]["w_expected"][str(k)] + r[m, n]
    assert (oracle_lib.matvec_residual(w, N, K, codes, scales, r, rows=[1]) == y[:, 1:]).all()


def test_generator_pack_roundtrip(oracle_lib):
    for seed in range(20):
        f = qi.draw_q4k_fields(3, 512, seed)
        if seed == 1:
            f.q[:] = 15; f.sc[:] = 63; f.mn[:] = 63
        if seed == 2:
            f.q[:] = 0; f.sc[:] = 0; f.mn[:] = 0
            f.d[:] = 0; f.dmin[:] = 0
        if seed == 3:
            f.d[:] = np.float16(65504); f.dmin[:] = np.float16(1.0)
        w = qi.pack_q4k(f)
        for n in range(3):
            for b in range(2):
                d, dmin, sc, mn, q = oracle_lib.unpack_q4k(w[n, b * 144:(b + 1) * 144])
                assert d == float(f.d[n, b]) and dmin == float(f.dmin[n, b])
                assert (sc == f.sc[n, b]).all() and (mn == f.mn[n, b]).all()
                assert (q == f.q[n, b]).all()


def test_fast_bytes_generator_is_valid_q4k(oracle_lib):
    w = qi.make_q4k_bytes(5, 512, 7)
    for n in range(5):
        for b in range(2):
            d, dmin, sc, mn, q = oracle_lib.unpack_q4k(w[n, b * 144:(b + 1) * 144])
            assert 1e-4 * 0.99 <= d <= 1e-3 * 1.01 and 1e-4 * 0.99 <= dmin <= 1e-3 * 1.01
            assert sc.max() <= 63 and mn.max() <= 63 and q.max() <= 15


# ------------------------------------------------------------- quantizer ----

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_golden_q8_cases(oracle_lib, idx):
    c = _load("q8_ties.json")["cases"][idx]
    codes, scales, sums = oracle_lib.quantize_act(np.array(c["x"], np.float32)[None])
    assert codes[0].tolist() == c["codes"]
    assert float(scales[0, 0]) == c["scale"]
    assert int(sums[0, 0]) == c["sum"]


def test_q8_roundtrip_bound_and_invariants(oracle_lib):
    x = qi.make_act(64, 1024, 3) * np.float32(3.0)
    x[5, 64:96] = 0.0
    codes, scales, sums = oracle_lib.quantize_act(x)
    xb = x.reshape(64, 32, 32).astype(np.float64)
    cb = codes.reshape(64, 32, 32).astype(np.int64)
    s = scales.astype(np.float64)[:, :, None]
    # round trip: |x - s*c| <= s*(1/2 + 2^-17)
    assert (np.abs(xb - s * cb) <= s * (0.5 + 2.0 ** -17)).all()
    nz = np.abs(xb).max(axis=2) > 0
    assert (np.abs(cb).max(axis=2)[nz] == 127).all()
    assert (cb[~nz] == 0).all() and (scales[~nz] == 0).all()
    assert (cb.sum(axis=2) == sums).all()
    assert np.abs(cb).max() <= 127
    # scale is max|x| / 127 in fp32 (division, not reciprocal-multiply)
    amax = np.abs(x.reshape(64, 32, 32)).max(axis=2)
    assert (scales == amax / np.float32(127)).all()
    # power-of-two scaling: codes unchanged, scale scales exactly
    for k in (-3, 5):
        c2, s2, su2 = oracle_lib.quantize_act(x * np.float32(2.0 ** k))
        assert (c2 == codes).all() and (su2 == sums).all()
        assert (s2 == scales * np.float32(2.0 ** k)).all()


def test_q8_uses_division_not_reciprocal(oracle_lib):
    """Build blocks whose quotient x/s sits next to a rounding boundary, where
    fl(x/s) and fl(x*fl(1/s)) round to different codes, and check the oracle
    follows the IEEE division."""
    rng = np.random.default_rng(11)
    found = 0
    for _ in range(2000):
        amax = np.float32(rng.uniform(0.5, 8.0))
        s = amax / np.float32(127)
        r = np.float32(1) / s
        k = int(rng.integers(0, 126))
        x0 = np.float32((k + 0.5) * float(s))
        for step in range(-4, 5):
            x = x0 if step == 0 else np.float32(x0 + step * np.spacing(x0))
            by_div = np.rint(x / s)
            by_rcp = np.rint(x * r)
            if by_div != by_rcp:
                blk = np.zeros(32, np.float32)
                blk[0], blk[1] = amax, x
                codes, scales, _ = oracle_lib.quantize_act(blk[None])
                assert scales[0, 0] == s
                assert codes[0, 1] == int(by_div) and codes[0, 0] == 127
                found += 1
        if found >= 5:
            break
    assert found >= 5


# -------------------------------------------------------------- products ----

@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (3, 512, 2), (3, 256, 3), (5, 768, 1)])
def test_matvec_vs_field_brute_force(oracle_lib, N, K, M):
    for seed in range(0, 40):
        w, f = qi.make_q4k(N, K, seed)
        x = qi.make_act(M, K, 1000 + seed)
        codes, scales, sums = oracle_lib.quantize_act(x)
        xhat = scales.astype(np.float64).repeat(32, axis=1) * codes
        y_bf = xhat @ _fields_to_w(f).T
        y = oracle_lib.matvec(w, N, K, codes, scales)
        y2 = oracle_lib.matvec_intform(w, N, K, codes, scales, sums)
        mag = np.abs(xhat) @ np.abs(_fields_to_w(f)).T
        assert (np.abs(y - y_bf) <= 1e-12 * mag).all()
        assert (np.abs(y2 - y_bf) <= 1e-12 * mag).all()


def test_subblock_dots_vs_integer_brute_force(oracle_lib):
    N, K, M = 4, 512, 3
    w, f = qi.make_q4k(N, K, 5)
    codes, _, _ = oracle_lib.quantize_act(qi.make_act(M, K, 6))
    D = oracle_lib.subblock_dots(w, N, K, codes)
    q = f.q.reshape(N, K // 32, 32).astype(np.int64)
    c = codes.reshape(M, K // 32, 32).astype(np.int64)
    expect = np.einsum("njk,mjk->mnj", q, c)
    assert (D == expect).all()


def test_all_ones_activation_closed_form(oracle_lib):
    N, K = 6, 1024
    w, f = qi.make_q4k(N, K, 21)
    x = np.ones((1, K), np.float32)
    codes, scales, sums = oracle_lib.quantize_act(x)
    assert (codes == 127).all() and (sums == 32 * 127).all()
    assert (scales == np.float32(1) / np.float32(127)).all()
    rowsum = _fields_to_w(f).sum(axis=1)
    y = oracle_lib.matvec(w, N, K, codes, scales)[0]
    expect = 127.0 * float(np.float32(1) / np.float32(127)) * rowsum
    assert np.allclose(y, expect, rtol=1e-12, atol=0)
    # (1 + delta) with |delta| < 6e-8 relative to the plain row sum
    assert np.allclose(y, rowsum, rtol=6e-8, atol=0)


def _integer_activation(rng, M, K):
    x = rng.integers(-126, 127, size=(M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 0] = rng.choice([-127.0, 127.0], size=(M, K // 32))
    return x


def test_integer_exposing_special_case(oracle_lib):
    """d=1, dmin=0, one-hot sub-block scale j0, integer x with a +-127 per block:
    activation scale is exactly 1, codes equal x, and y equals the integer dot of
    sub-block j0's quants with x."""
    rng = np.random.default_rng(3)
    N, K, M = 4, 256, 2
    for j0 in range(8):
        f = qi.draw_q4k_fields(N, K, 100 + j0)
        f.d[:] = np.float16(1.0); f.dmin[:] = np.float16(0.0)
        f.sc[:] = 0; f.sc[:, :, j0] = 1
        w = qi.pack_q4k(f)
        x = _integer_activation(rng, M, K)
        codes, scales, sums = oracle_lib.quantize_act(x)
        assert (scales == 1.0).all() and (codes == x).all()
        y = oracle_lib.matvec(w, N, K, codes, scales)
        qj = f.q[:, 0, 32 * j0:32 * j0 + 32].astype(np.int64)
        expect = x[:, 32 * j0:32 * j0 + 32].astype(np.int64) @ qj.T
        assert (y == expect).all()
        # mins-only variant: q = 0, sc = 0, dmin = 1, one-hot mn -> y = -S_j0
        f.q[:] = 0; f.sc[:] = 0; f.dmin[:] = np.float16(1.0)
        f.mn[:] = 0; f.mn[:, :, j0] = 1
        y = oracle_lib.matvec(qi.pack_q4k(f), N, K, codes, scales)
        assert (y == -sums[:, j0][:, None]).all()


def test_power_of_two_scaling_is_exact(oracle_lib):
    N, K = 5, 512
    w, f = qi.make_q4k(N, K, 31)
    x = qi.make_act(2, K, 32)
    codes, scales, _ = oracle_lib.quantize_act(x)
    y = oracle_lib.matvec(w, N, K, codes, scales)
    f.d = (f.d * np.float16(2)).astype(np.float16)
    f.dmin = (f.dmin * np.float16(2)).astype(np.float16)
    y2 = oracle_lib.matvec(qi.pack_q4k(f), N, K, codes, scales)
    assert (y2 == 2 * y).all()
    c4, s4, _ = oracle_lib.quantize_act(x * np.float32(4))
    y4 = oracle_lib.matvec(w, N, K, c4, s4)
    assert (y4 == 4 * y).all()


def test_zero_scales_and_zero_blocks(oracle_lib):
    N, K = 3, 512
    f = qi.draw_q4k_fields(N, K, 41)
    f.d[:] = 0; f.dmin[:] = 0
    x = qi.make_act(1, K, 42)
    codes, scales, _ = oracle_lib.quantize_act(x)
    assert (oracle_lib.matvec(qi.pack_q4k(f), N, K, codes, scales) == 0).all()
    # a zero activation block contributes exactly nothing
    w, f = qi.make_q4k(N, K, 43)
    x2 = x.copy(); x2[0, 32:64] = 0
    c2, s2, _ = oracle_lib.quantize_act(x2)
    wf = _fields_to_w(f)
    xhat = s2.astype(np.float64).repeat(32, axis=1) * c2
    assert (xhat[0, 32:64] == 0).all()
    y = oracle_lib.matvec(w, N, K, c2, s2)[0]
    mag = np.abs(xhat) @ np.abs(wf).T
    assert (np.abs(y - (xhat @ wf.T)[0]) <= 1e-12 * mag[0]).all()


# ----------------------------------------------------------------- SwiGLU ----

def test_swiglu_identities(oracle_lib):
    g = np.linspace(-30, 30, 2001).astype(np.float32)
    one = np.ones_like(g)
    h = oracle_lib.swiglu(g, one).astype(np.float64)
    hn = oracle_lib.swiglu(-g, one).astype(np.float64)
    # silu(g) - silu(-g) = g
    assert np.allclose(h - hn, g, rtol=0, atol=4 * np.spacing(np.float32(30)))
    assert oracle_lib.swiglu(np.zeros(1, np.float32), np.ones(1, np.float32))[0] == 0
    big = np.array([40.0, 60.0], np.float32)
    assert (oracle_lib.swiglu(big, np.float32([2.0, -3.0])) == big * np.float32([2.0, -3.0])).all()
    # silu(g) at g = ln(3): sigma = 3/4 exactly, so h = 0.75 * ln(3)
    g3 = np.float32(np.log(3.0))
    assert abs(float(oracle_lib.swiglu(np.array([g3]), np.ones(1, np.float32))[0])
               - 0.75 * float(g3)) <= 1e-7


# ------------------------------------------------------------ routed MoE ----

def _experts(E, N, K, seed0):
    ws = [qi.make_q4k(N, K, seed0 + e) for e in range(E)]
    return np.concatenate([w for w, _ in ws], axis=0), [f for _, f in ws]


def test_moe_matvec_gathers_the_right_expert_and_row(oracle_lib):
    E, N, K, T, topk = 4, 64, 256, 3, 2
    w, fields = _experts(E, N, K, 500)
    stride = N * K // 256 * 144
    ids = np.array([[2, 0], [1, 3], [3, 2]], np.int32)
    x = qi.make_act(T * topk, K, 9)
    codes, scales, _ = oracle_lib.quantize_act(x)
    xhat = scales.astype(np.float64).repeat(32, axis=1) * codes
    # per-slot activation rows
    y = oracle_lib.moe_matvec(w, E, stride, N, K, ids, None, codes, scales, True)
    for t in range(T):
        for s in range(topk):
            wf = _fields_to_w(fields[ids[t, s]])
            ref = xhat[t * topk + s] @ wf.T
            mag = np.abs(xhat[t * topk + s]) @ np.abs(wf).T
            assert (np.abs(y[t * topk + s] - ref) <= 1e-12 * mag).all()
    # per-token activation rows, weighted sum in slot order
    rw = np.array([[0.25, 0.75], [1.0, 0.0], [0.5, 0.5]], np.float32)
    y = oracle_lib.moe_matvec(w, E, stride, N, K, ids, rw, codes[:T], scales[:T], False)
    for t in range(T):
        ref = sum(float(rw[t, s]) * (xhat[t] @ _fields_to_w(fields[ids[t, s]]).T)
                  for s in range(topk))
        mag = sum(abs(float(rw[t, s])) * (np.abs(xhat[t]) @ np.abs(_fields_to_w(fields[ids[t, s]])).T)
                  for s in range(topk))
        assert (np.abs(y[t] - ref) <= 1e-12 * mag).all()


def test_moe_layer_identical_experts_reduce_to_dense(oracle_lib):
    """All experts equal: every slot computes the same down product, so the layer
    equals (sum of routing weights) x the dense gate/up/SwiGLU/down chain."""
    E, H, F, T, topk = 4, 256, 256, 2, 3
    wg, _ = qi.make_q4k(F, H, 1); wu, _ = qi.make_q4k(F, H, 2); wd, _ = qi.make_q4k(H, F, 3)
    ids = np.array([[0, 3, 1], [2, 1, 0]], np.int32)
    rw = np.array([[0.2, 0.3, 0.5], [0.6, 0.1, 0.3]], np.float32)
    x = qi.make_act(T, H, 4)
    out = oracle_lib.moe_layer(np.tile(wg, (E, 1)), np.tile(wu, (E, 1)), np.tile(wd, (E, 1)),
                               E, H, F, ids, rw, x)
    xc, xs, _ = oracle_lib.quantize_act(x)
    g = oracle_lib.matvec(wg, F, H, xc, xs).astype(np.float32)
    u = oracle_lib.matvec(wu, F, H, xc, xs).astype(np.float32)
    h = oracle_lib.swiglu(g, u)
    hc, hs, _ = oracle_lib.quantize_act(h)
    z = oracle_lib.matvec(wd, H, F, hc, hs)
    for t in range(T):
        assert (out["g"][t * topk:(t + 1) * topk] == g[t]).all()
        ref = sum(float(rw[t, s]) for s in range(topk)) * z[t]
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-12 * np.abs(z[t]).max())


# ------------------------------------------------------------------ Q6_K ----

def _q6k_block_bytes(b):
    sb = np.zeros(210, np.uint8)
    for k, v in b["ql"].items():
        sb[int(k)] = v
    for k, v in b["qh"].items():
        sb[128 + int(k)] = v
    sb[192:208] = np.array(b["sc"], np.int8).view(np.uint8)
    sb[208:210] = np.array([int(b["d_bits"], 16)], "<u2").view(np.uint8)
    return sb


def _q6k_fields_to_w(f: qi.Q6KFields) -> np.ndarray:
    """fp64 Q6_K weights straight from the drawn fields (no byte decoding)."""
    N, nsb, _ = f.q.shape
    j = np.arange(256) // 16
    w = (f.d.astype(np.float64)[:, :, None] * f.sc.astype(np.float64)[:, :, j] *
         (f.q.astype(np.float64) - 32.0))
    return w.reshape(N, nsb * 256)


def test_q6k_golden_superblock_unpack(oracle_lib):
    b = _load("q6k_superblock_handbuilt.json")["blocks"][0]
    sb = _q6k_block_bytes(b)
    d, sc, q = oracle_lib.unpack_q6k(sb)
    assert d == b["d"] and sc.tolist() == b["sc"]
    expect_q = np.zeros(256, np.int32)
    for k, v in b["q_nonzero"].items():
        expect_q[int(k)] = v
    assert q.tolist() == expect_q.tolist()
    w = oracle_lib.q6k_dequant(sb, 256)[0]
    for k, v in b["w_expected"].items():
        assert w[int(k)] == v, (k, w[int(k)], v)
    assert w.sum() == b["row_sum"]


def test_q6k_generator_pack_roundtrip(oracle_lib):
    for seed in range(12):
        f = qi.draw_q6k_fields(3, 512, 100 + seed)
        if seed == 1:
            f.q[:] = 63; f.sc[:] = 127
        if seed == 2:
            f.q[:] = 0; f.sc[:] = -128; f.d[:] = 0
        if seed == 3:
            f.d[:] = np.float16(65504)
        w = qi.pack_q6k(f)
        for n in range(3):
            for b in range(2):
                d, sc, q = oracle_lib.unpack_q6k(w[n, b * 210:(b + 1) * 210])
                assert d == float(f.d[n, b])
                assert (sc == f.sc[n, b]).all() and (q == f.q[n, b]).all()


def test_q6k_fast_bytes_generator_is_valid(oracle_lib):
    w = qi.make_q6k_bytes(4, 512, 9)
    seen_neg = False
    for n in range(4):
        for b in range(2):
            d, sc, q = oracle_lib.unpack_q6k(w[n, b * 210:(b + 1) * 210])
            assert 1e-4 * 0.99 <= d <= 1e-3 * 1.01
            assert q.min() >= 0 and q.max() <= 63
            seen_neg |= bool((sc < 0).any())
    assert seen_neg   # scales are signed


@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (3, 512, 2), (2, 768, 3)])
def test_q6k_matvec_vs_field_brute_force(oracle_lib, N, K, M):
    for seed in range(4):
        w, f = qi.make_q6k(N, K, 200 + seed)
        x = qi.make_act(M, K, 300 + seed)
        codes, scales, _ = oracle_lib.quantize_act(x)
        wf = _q6k_fields_to_w(f)
        assert np.array_equal(oracle_lib.q6k_dequant(w, K), wf)
        xh = scales.astype(np.float64).repeat(32, axis=1) * codes.astype(np.float64)
        ref = xh @ wf.T
        y = oracle_lib.q6k_matvec(w, N, K, codes, scales)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_q6k_all_ones_activation_closed_form(oracle_lib):
    w, f = qi.make_q6k(4, 512, 5)
    codes, scales, _ = oracle_lib.quantize_act(np.ones((1, 512), np.float32))
    assert (codes == 127).all()
    d_a = float(np.float32(1.0) / np.float32(127.0))
    y = oracle_lib.q6k_matvec(w, 4, 512, codes, scales)[0]
    expect = 127.0 * d_a * _q6k_fields_to_w(f).sum(axis=1)
    assert np.allclose(y, expect, rtol=1e-12, atol=0)


def test_q6k_integer_exposing_special_case(oracle_lib):
    """d = 1 and one scale = 1: y is the integer dot of one 16-weight sub-block
    with (q - 32), exact."""
    rng = np.random.default_rng(11)
    for j in (0, 5, 9, 15):
        f = qi.draw_q6k_fields(1, 256, 400 + j)
        f.d[:] = np.float16(1.0)
        f.sc[:] = 0
        f.sc[0, 0, j] = 1
        w = qi.pack_q6k(f)
        x = rng.integers(-127, 128, size=(1, 256)).astype(np.float32)
        x[0, ::32] = 127.0          # every block's max is 127: scale 1, codes = x
        codes, scales, _ = oracle_lib.quantize_act(x)
        assert (scales == 1.0).all() and (codes == x).all()
        e = np.arange(16 * j, 16 * j + 16)
        expect = float(((f.q[0, 0, e].astype(np.int64) - 32) * x[0, e].astype(np.int64)).sum())
        assert oracle_lib.q6k_matvec(w, 1, 256, codes, scales)[0, 0] == expect


def test_q6k_zero_scale_gives_zero(oracle_lib):
    f = qi.draw_q6k_fields(2, 512, 12)
    f.d[0] = 0
    f.sc[1] = 0
    w = qi.pack_q6k(f)
    codes, scales, _ = oracle_lib.quantize_act(qi.make_act(2, 512, 13))
    y = oracle_lib.q6k_matvec(w, 2, 512, codes, scales)
    assert (y == 0).all()


# ------------------------------------------------- INT8 KV cache, attention --
# Cache entries and decode attention of genie-ai-runtime's Path I (section 4,
# "Memory-first: making every byte count").

def _golden_kv(case, hd):
    x = np.zeros(hd, np.float32)
    for k, v in case["x"].items():
        x[int(k)] = v
    codes = np.zeros(hd, np.int64)
    for k, v in case["codes"].items():
        codes[int(k)] = v
    return x, codes


@pytest.mark.parametrize("idx", range(3))
def test_kv_quantize_golden(oracle_lib, idx):
    g = _load("kv_int8_handbuilt.json")
    c = g["cases"][idx]
    x, want = _golden_kv(c, g["head_dim"])
    codes, scales = oracle_lib.kv_quantize(x[None])
    assert codes[0].astype(np.int64).tolist() == want.tolist()
    assert float(scales[0]) == c["scale"]


def test_kv_quantize_roundtrip_bound(oracle_lib):
    k, v = qi.make_kv(40, 8, 128, 5)
    x = np.concatenate([k, 7.0 * v]).reshape(-1, 128)
    x[3] = 0.0
    codes, scales = oracle_lib.kv_quantize(x)
    s = scales.astype(np.float64)[:, None]
    c = codes.astype(np.int64)
    assert (np.abs(x - s * c) <= s * (0.5 + 2.0 ** -17)).all()
    amax = np.abs(x).max(axis=1)
    assert (scales == amax / np.float32(127)).all()
    nz = amax > 0
    assert (np.abs(c).max(axis=1)[nz] == 127).all()
    assert (c[~nz] == 0).all()


def _cache(rng, n_kv, cap, hd=128):
    kc = rng.integers(-127, 128, size=(n_kv, cap, hd)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(n_kv, cap, hd)).astype(np.int8)
    ks = rng.uniform(0.001, 0.03, size=(n_kv, cap)).astype(np.float32)
    vs = rng.uniform(0.001, 0.03, size=(n_kv, cap)).astype(np.float32)
    return kc, ks, vc, vs


def test_attn_zero_query_is_mean_of_visible_values(oracle_lib):
    rng = np.random.default_rng(1)
    kc, ks, vc, vs = _cache(rng, 2, 40)
    n_ctx, M = 37, 3
    q = np.zeros((M, 4, 128), np.float32)
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, n_ctx, 0.088)
    vhat = vs.astype(np.float64)[:, :, None] * vc
    for m in range(M):
        L = n_ctx - (M - 1 - m)
        for h in range(4):
            np.testing.assert_allclose(out[m, h], vhat[h // 2, :L].mean(axis=0), rtol=1e-12, atol=1e-15)


def test_attn_one_hot_query_selects_one_position(oracle_lib):
    rng = np.random.default_rng(2)
    kc, ks, vc, vs = _cache(rng, 1, 64)
    j, t_star = 17, 41
    kc[0, :, j] = 0
    kc[0, t_star, j] = 127
    ks[0, t_star] = 1.0
    q = np.zeros((1, 1, 128), np.float32)
    q[0, 0, j] = 100.0
    # score gap 100*127*0.0884 > 1100: e^-1100 is 0 in fp64
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, 64, 128 ** -0.5)
    assert (out[0, 0] == vs[0, t_star].astype(np.float64) * vc[0, t_star]).all()


def test_attn_two_positions_logistic_form(oracle_lib):
    rng = np.random.default_rng(3)
    kc, ks, vc, vs = _cache(rng, 1, 2)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32) * 4
    scale = 128 ** -0.5
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, 2, scale)
    kh = ks.astype(np.float64)[0, :, None] * kc[0]
    vh = vs.astype(np.float64)[0, :, None] * vc[0]
    s0, s1 = (scale * (kh @ q[0, 0].astype(np.float64))).tolist()
    want = vh[1] + (vh[0] - vh[1]) / (1.0 + np.exp(s1 - s0))
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-12, atol=1e-14)


def test_attn_grouped_heads_read_their_own_kv_head(oracle_lib):
    # n_head = 8 over n_kv = 4: head h reads kv head h // 2.  Each kv head g has
    # its key spike at its own position t_g, so head h must return v[g][t_g].
    rng = np.random.default_rng(4)
    kc, ks, vc, vs = _cache(rng, 4, 32)
    kc[:, :, 0] = 0
    t = [3, 29, 11, 20]
    for g in range(4):
        kc[g, t[g], 0] = 127
        ks[g, t[g]] = 1.0
    q = np.zeros((1, 8, 128), np.float32)
    q[0, :, 0] = 100.0
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, 32, 128 ** -0.5)
    for h in range(8):
        g = h // 2
        assert (out[0, h] == vs[g, t[g]].astype(np.float64) * vc[g, t[g]]).all(), h


def test_attn_causal_rows_equal_shorter_single_queries(oracle_lib):
    rng = np.random.default_rng(5)
    kc, ks, vc, vs = _cache(rng, 2, 50)
    q = qi.make_query(4, 8, 128, 6)
    n_ctx = 45
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, n_ctx, 0.09)
    for m in range(4):
        one = oracle_lib.attn_int8kv(q[m:m + 1], kc, ks, vc, vs, n_ctx - 3 + m, 0.09)
        assert (out[m] == one[0]).all()


def test_attn_position_permutation_and_convex_hull(oracle_lib):
    rng = np.random.default_rng(7)
    kc, ks, vc, vs = _cache(rng, 1, 30)
    q = qi.make_query(1, 3, 128, 8, gain=3.0)
    out = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, 30, 0.0884)
    perm = rng.permutation(30)
    outp = oracle_lib.attn_int8kv(q, kc[:, perm], ks[:, perm], vc[:, perm], vs[:, perm], 30, 0.0884)
    np.testing.assert_allclose(outp, out, rtol=1e-12, atol=1e-15)
    vh = vs.astype(np.float64)[0, :, None] * vc[0]
    assert (out[0] <= vh.max(axis=0) + 1e-15).all() and (out[0] >= vh.min(axis=0) - 1e-15).all()
    # positions beyond n_ctx are never read
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, 25:], vc2[:, 25:] = 99, -99
    a = oracle_lib.attn_int8kv(q, kc, ks, vc, vs, 25, 0.0884)
    b = oracle_lib.attn_int8kv(q, kc2, ks, vc2, vs, 25, 0.0884)
    assert (a == b).all()
