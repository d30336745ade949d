"""GPU parity of the routed-expert path (q4k_moe_gemv and the SwiGLU variant of
q4k_quantize_act) against the CPU oracle, on the 8B-A1B-style layer shape:
64 experts, hidden 2048, expert FFN 1024 (gate/up 2048->1024, down 1024->2048),
top-8 routing with softmax weights, T = 1 and 16 tokens.

Stage by stage the expected values are exact or within the fp32 tolerance:
  gate/up grouped GEMV             -> tolerance vs oracle g, u
  Q8 of SwiGLU(oracle g, oracle u) -> bit-exact vs oracle codes/scales/sums
  down grouped GEMV + routed sum   -> tolerance vs oracle y (on the oracle's Q8(h))
The whole chain run on the GPU's own intermediates is compared with a bound
that admits the one place where two correct answers exist: an element of h
whose quotient h/scale lies next to a rounding boundary may round either way
when g and u differ in their last fp32 bits.
"""
import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu

E, H, F, TOPK = qi.MOE_EXPERTS, qi.MOE_HIDDEN, qi.MOE_FFN, qi.MOE_TOPK


@pytest.fixture(scope="module")
def q4k():
    import torch
    assert torch.cuda.is_available()
    import gemm_q4_super_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def layer():
    wg = np.concatenate([qi.make_q4k_bytes(F, H, qi.expert_seed(0, e, 0)) for e in range(E)])
    wu = np.concatenate([qi.make_q4k_bytes(F, H, qi.expert_seed(0, e, 1)) for e in range(E)])
    wd = np.concatenate([qi.make_q4k_bytes(H, F, qi.expert_seed(0, e, 2)) for e in range(E)])
    return wg, wu, wd


STRIDE_GU = F * (H // 256) * 144
STRIDE_D = H * (F // 256) * 144


def _moe(q4k, w, N, K, ids, rw, codes, scales, sums, act_per_slot, stride):
    import torch
    y = q4k.q4k_moe_gemv(to_dev(w), E, stride, N, K, to_dev(ids),
                         None if rw is None else to_dev(rw), to_dev(codes), to_dev(scales),
                         to_dev(sums), act_per_slot)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("T", [1, 16])
def test_moe_gate_up_per_slot(q4k, oracle_lib, layer, T):
    wg, wu, _ = layer
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(T))
    x = qi.make_act(T, H, qi.act_seed(60000 + T))
    c, s, su = oracle_lib.quantize_act(x)
    for w in (wg, wu):
        y = _moe(q4k, w, F, H, ids, None, c, s, su, 0, STRIDE_GU)
        ref = oracle_lib.moe_matvec(w, E, STRIDE_GU, F, H, ids, None, c, s, False)
        assert_close(y, ref, "moe gate/up T=%d" % T)


@pytest.mark.parametrize("T", [1, 16])
def test_moe_down_weighted_sum(q4k, oracle_lib, layer, T):
    _, _, wd = layer
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(100 + T))
    h = qi.make_act(T * TOPK, F, qi.act_seed(61000 + T)) * np.float32(20.0)
    c, s, su = oracle_lib.quantize_act(h)
    y = _moe(q4k, wd, H, F, ids, rw, c, s, su, 1, STRIDE_D)
    ref = oracle_lib.moe_matvec(wd, E, STRIDE_D, H, F, ids, rw, c, s, True)
    assert_close(y, ref, "moe down T=%d" % T)
    # per-slot form of the same call
    y = _moe(q4k, wd, H, F, ids, None, c, s, su, 1, STRIDE_D)
    ref = oracle_lib.moe_matvec(wd, E, STRIDE_D, H, F, ids, None, c, s, True)
    assert_close(y, ref, "moe down per slot T=%d" % T)


def test_moe_many_tokens_one_expert_and_bad_ids(q4k, oracle_lib):
    """20 tokens all routed to expert 3 in slot 0 (more pairs than one 8-row
    chunk), a repeated expert across slots of different tokens, and ids out of
    range, which are skipped (zero rows / no contribution)."""
    n_exp, N, K, T, topk = 8, 96, 512, 20, 2
    w = np.concatenate([qi.make_q4k_bytes(N, K, 900 + e) for e in range(n_exp)])
    stride = N * (K // 256) * 144
    ids = np.zeros((T, topk), np.int32)
    ids[:, 0] = 3
    ids[:, 1] = np.arange(T) % n_exp
    ids[ids[:, 1] == 3, 1] = 5
    ids[4, 1] = -1
    ids[7, 1] = n_exp          # out of range
    rw = np.full((T, topk), 0.5, np.float32)
    x = qi.make_act(T, K, 77)
    c, s, su = oracle_lib.quantize_act(x)
    import torch
    y = q4k.q4k_moe_gemv(to_dev(w), n_exp, stride, N, K, to_dev(ids), None, to_dev(c),
                         to_dev(s), to_dev(su), 0)
    y2 = q4k.q4k_moe_gemv(to_dev(w), n_exp, stride, N, K, to_dev(ids), to_dev(rw), to_dev(c),
                          to_dev(s), to_dev(su), 0)
    torch.cuda.synchronize()
    y, y2 = y.cpu().numpy(), y2.cpu().numpy()
    valid = (ids >= 0) & (ids < n_exp)
    safe = np.where(valid, ids, 0)
    ref = oracle_lib.moe_matvec(w, n_exp, stride, N, K, safe, None, c, s, False)
    ref[~valid.ravel()] = 0.0
    assert_close(y, ref, "per-slot with bad ids")
    assert (y[~valid.ravel()] == 0).all()
    ref2 = (ref.reshape(T, topk, N) * 0.5).sum(axis=1)
    assert_close(y2, ref2, "weighted with bad ids")


def test_swiglu_quantize_bit_exact_on_oracle_gu(q4k, oracle_lib, layer):
    import torch
    wg, wu, wd = layer
    T = 16
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(7))
    x = qi.make_act(T, H, qi.act_seed(62000))
    out = oracle_lib.moe_layer(wg, wu, wd, E, H, F, ids, rw, x)
    c, s, su = q4k.q4k_quantize_act(to_dev(out["u"]), to_dev(out["g"]))
    torch.cuda.synchronize()
    assert (c.cpu().numpy() == out["hc"]).all()
    assert (s.cpu().numpy() == out["hs"]).all()
    assert (su.cpu().numpy() == out["hsum"]).all()


def _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y, ids, rw, wd, H_, F_, what):
    """y (a whole layer computed on the GPU, whose intermediates are g, u and
    Q8(h) = hc, hs) against the oracle layer `ref`: g and u within the fp32
    tolerance; h codes equal except +-1 where the oracle's quotient h/scale
    lies within what the measured g, u differences can move it of a rounding
    boundary; y within the tolerance plus what those flips and scale shifts
    can move it."""
    T, topk = ids.shape
    P = T * topk
    assert_close(g, ref["g"], what + " g")
    assert_close(u, ref["u"], what + " u")
    g0, u0 = ref["g"].astype(np.float64), ref["u"].astype(np.float64)
    dg, du = np.abs(g - g0), np.abs(u - u0)
    sig = 1.0 / (1.0 + np.exp(-g0))
    dh = np.abs(sig * (1.0 + g0 * (1.0 - sig))) * dg * np.abs(u0) + np.abs(g0 * sig) * du + dg * du
    # plus one fp32 ulp of h: both sides round their (different) h to fp32
    dh = dh + np.spacing(np.abs(ref["h"])).astype(np.float64)
    dh = dh.reshape(P, F_ // 32, 32) + 1e-12
    amax = np.abs(ref["h"].astype(np.float64)).reshape(P, F_ // 32, 32).max(axis=2)
    amax = np.maximum(amax, 1e-30)[:, :, None]
    q = ref["h"].reshape(P, F_ // 32, 32).astype(np.float64) * 127.0 / amax
    dq = 127.0 * dh / amax + np.abs(q) * dh.max(axis=2, keepdims=True) / amax
    frac = np.abs(q - np.floor(q) - 0.5)
    diff = (hc.astype(np.int64) - ref["hc"].astype(np.int64)).reshape(P, F_ // 32, 32)
    mism = diff != 0
    assert (np.abs(diff) <= 1).all()
    assert (frac[mism] <= 2.0 * dq[mism] + 1e-6).all(), "code flip away from a boundary"
    dscale = np.abs(hs.astype(np.float64) - ref["hs"])
    # scale = fl32(amax / 127): amax moves by at most max dh, plus one ulp of the scale
    assert (dscale <= 1.01 * dh.max(axis=2) / 127.0
            + np.spacing(ref["hs"]).astype(np.float64) + 1e-12).all()
    W = {e: np.abs(oracle_lib.dequant(wd[e * H_:(e + 1) * H_], F_)) for e in np.unique(ids)}
    extra = np.zeros((T, H_))
    for t in range(T):
        for s_ in range(topk):
            p = t * topk + s_
            d_blk = np.maximum(ref["hs"][p], hs[p]).astype(np.float64).repeat(32)
            flips = mism[p].ravel().astype(np.float64)
            shift = dscale[p].repeat(32) * 127.0
            extra[t] += abs(float(rw[t, s_])) * (W[ids[t, s_]] @ (flips * d_blk + shift))
    err = np.abs(y.astype(np.float64) - ref["y"])
    tol = np.maximum(2e-3 * np.abs(ref["y"]), 1e-4) + 1.01 * extra
    assert (err <= tol).all(), what + ": y outside tolerance + admitted-flip bound"
    return int(mism.sum()), float(err.max())


def _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_):
    """The six-call chain; returns (g, u, hc, hs, y) on the host."""
    import torch
    sgu, sd = F_ * (H_ // 256) * 144, H_ * (F_ // 256) * 144
    xc, xs, xsu = q4k.q4k_quantize_act(x)
    g = q4k.q4k_moe_gemv(dwg, n_exp, sgu, F_, H_, dids, None, xc, xs, xsu, 0)
    u = q4k.q4k_moe_gemv(dwu, n_exp, sgu, F_, H_, dids, None, xc, xs, xsu, 0)
    hc, hs, hsu = q4k.q4k_quantize_act(u, g)
    y = q4k.q4k_moe_gemv(dwd, n_exp, sd, H_, F_, dids, drw, hc, hs, hsu, 1)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (g, u, hc, hs, y))


@pytest.mark.parametrize("T", [1, 16])
def test_moe_layer_chain(q4k, oracle_lib, layer, T):
    """The whole layer on the GPU's own intermediates."""
    wg, wu, wd = layer
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(T))
    x = qi.make_act(T, H, qi.act_seed(63000 + T))
    ref = oracle_lib.moe_layer(wg, wu, wd, E, H, F, ids, rw, x)
    g, u, hc, hs, y = _chain_parts(q4k, to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids),
                                   to_dev(rw), to_dev(x), E, H, F)
    flips, err = _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y, ids, rw, wd, H, F, "chain")
    print("chain: %d h-code flips, max y err %.3g" % (flips, err))


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_moe_ffn_vs_oracle(q4k, oracle_lib, layer, T):
    """q4k_moe_ffn (for T <= 2 with Q8 and SwiGLU inside the GEMV kernels) on
    the chain test's inputs against the oracle layer, with the same
    flip-aware bound; the bound's intermediates are the chain's, which the
    fused layer equals bit for bit (asserted here too)."""
    import torch
    wg, wu, wd = layer
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(T))
    x = qi.make_act(T, H, qi.act_seed(63000 + T))
    ref = oracle_lib.moe_layer(wg, wu, wd, E, H, F, ids, rw, x)
    dwg, dwu, dwd, dids, drw, dx = (to_dev(a) for a in (wg, wu, wd, ids, rw, x))
    g, u, hc, hs, y2 = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, dx, E, H, F)
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, E, STRIDE_GU, STRIDE_D, H, F, dids, drw, dx)
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y1, ids, rw, wd, H, F, "moe_ffn T=%d" % T)


def _chain(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_):
    import torch
    y = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_)[4]
    return torch.from_numpy(y)


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_moe_ffn_bit_identical_to_chain(q4k, layer, T):
    """The fused layer (gate|up in one launch; for T <= 2 x quantized and
    SwiGLU + Q8 formed inside the GEMV kernels, beyond that by the quantizer
    kernel) equals the six-call chain bit for bit; the chain itself is checked
    against the oracle by test_moe_layer_chain."""
    import torch
    wg, wu, wd = layer
    ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(200 + T))
    x = to_dev(qi.make_act(T, H, qi.act_seed(64000 + T)))
    dwg, dwu, dwd, dids, drw = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids), to_dev(rw)
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, E, STRIDE_GU, STRIDE_D, H, F, dids, drw, x)
    y2 = _chain(q4k, dwg, dwu, dwd, dids, drw, x, E, H, F)
    torch.cuda.synchronize()
    y1, y2 = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.isfinite(y1).all()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()


def test_moe_ffn_repeated_and_bad_ids_and_two_passes(q4k, oracle_lib):
    """Small experts with K spanning several passes (H = 3072: 12 columns per
    row), 20 tokens on one expert (several pair chunks), a repeated expert and
    out-of-range ids: fused equals chain bit for bit."""
    import torch
    n_exp, H_, F_, T, topk = 6, 3072, 512, 20, 2
    wg = np.concatenate([qi.make_q4k_bytes(F_, H_, 1300 + e) for e in range(n_exp)])
    wu = np.concatenate([qi.make_q4k_bytes(F_, H_, 1400 + e) for e in range(n_exp)])
    wd = np.concatenate([qi.make_q4k_bytes(H_, F_, 1500 + e) for e in range(n_exp)])
    ids = np.zeros((T, topk), np.int32)
    ids[:, 0] = 2
    ids[:, 1] = np.arange(T) % n_exp
    ids[ids[:, 1] == 2, 1] = 4
    ids[3, 1] = -5
    ids[9, 1] = n_exp
    rw = np.random.default_rng(3).standard_normal((T, topk)).astype(np.float32)
    x = to_dev(qi.make_act(T, H_, 91))
    dwg, dwu, dwd, dids, drw = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids), to_dev(rw)
    sgu, sd = F_ * (H_ // 256) * 144, H_ * (F_ // 256) * 144
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, n_exp, sgu, sd, H_, F_, dids, drw, x)
    g, u, hc, hs, y2 = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_)
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    assert np.isfinite(y1).all()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    # against the oracle: a skipped pair (out-of-range id) adds nothing, which
    # the oracle's layer gives with routing weight 0 on any valid expert; the
    # skipped pairs' g, u and h are not compared
    bad = (ids < 0) | (ids >= n_exp)
    ids_o, rw_o = np.where(bad, 0, ids).astype(np.int32), np.where(bad, 0, rw).astype(np.float32)
    ref = oracle_lib.moe_layer(wg, wu, wd, n_exp, H_, F_, ids_o, rw_o, x.cpu().numpy())
    keep = ~bad.ravel()
    for k in ("g", "u", "h", "hc", "hs"):
        ref[k] = np.where(keep[:, None], ref[k], 0).astype(ref[k].dtype)
    g[~keep] = 0.0
    u[~keep] = 0.0
    hc[~keep] = 0
    hs[~keep] = 0.0
    _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y1, ids_o, rw_o, wd, H_, F_,
                        "moe_ffn repeated/bad ids")


@pytest.mark.parametrize("topk,F_,bad", [(1, 512, None), (3, 1024, 1), (6, 512, 4), (8, 1024, 7)])
def test_moe_ffn_one_token(q4k, oracle_lib, topk, F_, bad):
    """One token: gate|up forms Q8(h) in its workgroups and the down launch
    sums the slots inside each workgroup (4- and 8-slot forms, 2 and 4 waves,
    gate|up over several passes at H = 3072, an out-of-range id): equal to the
    chain bit for bit and close to the oracle."""
    import torch
    n_exp, H_ = 9, 3072
    wg = np.concatenate([qi.make_q4k_bytes(F_, H_, 2300 + e) for e in range(n_exp)])
    wu = np.concatenate([qi.make_q4k_bytes(F_, H_, 2400 + e) for e in range(n_exp)])
    wd = np.concatenate([qi.make_q4k_bytes(H_, F_, 2500 + e) for e in range(n_exp)])
    ids = np.random.default_rng(topk).permutation(n_exp)[:topk].astype(np.int32)[None, :]
    if bad is not None:
        ids[0, bad % topk] = n_exp + 3
    rw = np.random.default_rng(10 + topk).standard_normal((1, topk)).astype(np.float32)
    x = to_dev(qi.make_act(1, H_, 92 + topk))
    dwg, dwu, dwd, dids, drw = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids), to_dev(rw)
    sgu, sd = F_ * (H_ // 256) * 144, H_ * (F_ // 256) * 144
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, n_exp, sgu, sd, H_, F_, dids, drw, x)
    y1b = q4k.q4k_moe_ffn(dwg, dwu, dwd, n_exp, sgu, sd, H_, F_, dids, drw, x)
    g, u, hc, hs, y2 = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_)
    torch.cuda.synchronize()
    y1, y1b = y1.cpu().numpy(), y1b.cpu().numpy()
    assert np.isfinite(y1).all()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    assert (y1.view(np.uint32) == y1b.view(np.uint32)).all()
    keep = ((ids >= 0) & (ids < n_exp)).ravel()
    ids_o = np.where(keep[None, :], ids, 0).astype(np.int32)
    rw_o = np.where(keep[None, :], rw, 0).astype(np.float32)
    ref = oracle_lib.moe_layer(wg, wu, wd, n_exp, H_, F_, ids_o, rw_o, x.cpu().numpy())
    for k in ("g", "u", "h", "hc", "hs"):
        ref[k] = np.where(keep[:, None], ref[k], 0).astype(ref[k].dtype)
    g[~keep] = 0.0
    u[~keep] = 0.0
    hc[~keep] = 0
    hs[~keep] = 0.0
    _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y1, ids_o, rw_o, wd, H_, F_,
                        "moe_ffn one token topk=%d F=%d" % (topk, F_))


@pytest.mark.parametrize("T,topk,F_", [(2, 4, 512), (3, 8, 1024), (1, 8, 2048), (40, 8, 512),
                                       (32, 8, 1024), (3, 12, 512), (1, 10, 512)])
def test_moe_ffn_launch_forms(q4k, oracle_lib, T, topk, F_):
    """Every form q4k_moe_ffn picks: two tokens (Q8(h) from the gate|up launch,
    the row-block down launch), three (the quantizer, then the row-block down
    launch), one token on a wide FFN and more than 256 pairs (the grouped
    launches with the routed sum by the last workgroup), and exactly 256
    pairs (the row-block down launch at its limit); and more than 8 slots per
    token (the slot sums take 8 slots per step: a second, partial step), in
    the row-block down launch (T = 3) and, one token past the one-token
    down launch's 8 slots, in the routed sum by the last workgroup: equal to
    the chain bit for bit and close to the oracle."""
    import torch
    n_exp, H_ = 12, 512
    wg = np.concatenate([qi.make_q4k_bytes(F_, H_, 3300 + e) for e in range(n_exp)])
    wu = np.concatenate([qi.make_q4k_bytes(F_, H_, 3400 + e) for e in range(n_exp)])
    wd = np.concatenate([qi.make_q4k_bytes(H_, F_, 3500 + e) for e in range(n_exp)])
    ids, rw = qi.make_routing(T, n_exp, topk, 900 + T)
    x = to_dev(qi.make_act(T, H_, 93 + T))
    dwg, dwu, dwd, dids, drw = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids), to_dev(rw)
    sgu, sd = F_ * (H_ // 256) * 144, H_ * (F_ // 256) * 144
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, n_exp, sgu, sd, H_, F_, dids, drw, x)
    g, u, hc, hs, y2 = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_)
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    assert np.isfinite(y1).all()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    ref = oracle_lib.moe_layer(wg, wu, wd, n_exp, H_, F_, ids, rw, x.cpu().numpy(), parallel=True)
    _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y1, ids, rw, wd, H_, F_,
                        "moe_ffn T=%d topk=%d F=%d" % (T, topk, F_))


def test_moe_ffn_many_experts(q4k, oracle_lib):
    """2048 small experts (H = F = 256: one column per row) at 256 pairs: the
    once-per-call grouping and the row-block down launch scan more experts
    than threads; equal to the chain bit for bit and close to the oracle."""
    import torch
    n_exp, H_, F_, T, topk = 2048, 256, 256, 32, 8
    wg = qi.make_q4k_bytes(n_exp * F_, H_, 4100)
    wu = qi.make_q4k_bytes(n_exp * F_, H_, 4101)
    wd = qi.make_q4k_bytes(n_exp * H_, F_, 4102)
    ids, rw = qi.make_routing(T, n_exp, topk, 4103)
    ids[5, 3] = ids[5, 2]                      # a token routing twice to one expert
    x = to_dev(qi.make_act(T, H_, 4104))
    dwg, dwu, dwd, dids, drw = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(ids), to_dev(rw)
    sgu, sd = F_ * (H_ // 256) * 144, H_ * (F_ // 256) * 144
    y1 = q4k.q4k_moe_ffn(dwg, dwu, dwd, n_exp, sgu, sd, H_, F_, dids, drw, x)
    g, u, hc, hs, y2 = _chain_parts(q4k, dwg, dwu, dwd, dids, drw, x, n_exp, H_, F_)
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    assert np.isfinite(y1).all()
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()
    ref = oracle_lib.moe_layer(wg, wu, wd, n_exp, H_, F_, ids, rw, x.cpu().numpy(), parallel=True)
    _assert_layer_close(oracle_lib, ref, g, u, hc, hs, y1, ids, rw, wd, H_, F_, "moe_ffn 2048 experts")


def test_moe_routed_sum_in_launch_reuses_workspace(q4k, oracle_lib):
    """The weighted sum is formed inside the down launch by the last
    workgroup of each row block: one zero-filled workspace serves repeated
    calls at T = 1, 16, 1 (its counters are back at zero after each), the
    bits repeat, and q4k_moe_gemv with routing weights equals the sum of its
    per-slot products in slot order."""
    import torch
    E, H, F, topk = qi.MOE_EXPERTS, qi.MOE_HIDDEN, qi.MOE_FFN, qi.MOE_TOPK
    wg = np.concatenate([qi.make_q4k_bytes(F, H, qi.expert_seed(5, e, 0)) for e in range(E)])
    wu = np.concatenate([qi.make_q4k_bytes(F, H, qi.expert_seed(5, e, 1)) for e in range(E)])
    wd = np.concatenate([qi.make_q4k_bytes(H, F, qi.expert_seed(5, e, 2)) for e in range(E)])
    dwg, dwu, dwd = to_dev(wg), to_dev(wu), to_dev(wd)
    sgu, sd = F * (H // 256) * 144, H * (F // 256) * 144
    nbytes = max(q4k.q4k_moe_ffn_workspace_bytes(T, topk, E, H, F) for T in (1, 16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for T in (1, 16, 1):
        ids, rw = qi.make_routing(T, E, topk, qi.routing_seed(50 + T))
        x = to_dev(qi.make_act(T, H, 60 + T))
        y = q4k.q4k_moe_ffn(dwg, dwu, dwd, E, sgu, sd, H, F, to_dev(ids), to_dev(rw), x,
                            workspace=ws)
        torch.cuda.synchronize()
        assert (ws[:256].cpu().numpy() == 0).all()
        outs.append(y.cpu().numpy())
        if T == 16:
            ref = oracle_lib.moe_layer(wg, wu, wd, E, H, F, ids, rw, x.cpu().numpy(),
                                       parallel=True)
            assert_close(outs[-1], ref["y"], "moe_ffn T=16 shared workspace")
    assert (outs[0].view(np.uint32) == outs[2].view(np.uint32)).all()
    # q4k_moe_gemv: weighted sum in the launch = slot-ordered fma of its products
    T = 4
    ids, rw = qi.make_routing(T, E, topk, qi.routing_seed(77))
    codes, scales, sums = oracle_lib.quantize_act(qi.make_act(T * topk, F, 78))
    args = (dwd, E, sd, H, F, to_dev(ids))
    z = q4k.q4k_moe_gemv(*args, None, to_dev(codes), to_dev(scales), to_dev(sums), True)
    y = q4k.q4k_moe_gemv(*args, to_dev(rw), to_dev(codes), to_dev(scales), to_dev(sums), True)
    torch.cuda.synchronize()
    z, y = z.cpu().numpy(), y.cpu().numpy()
    # v = fma(rw, z, v) per slot in order; a product of two fp32 is exact in
    # fp64, so each step is the fp64 sum rounded once to fp32 (up to a rare
    # double rounding: at most one unit in the last place)
    want = np.zeros((T, H), np.float32)
    for t in range(T):
        for s in range(topk):
            want[t] = (np.float64(rw[t, s]) * z[t * topk + s].astype(np.float64) +
                       want[t].astype(np.float64)).astype(np.float32)
    ulps = np.abs(y.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, ulps.max()
