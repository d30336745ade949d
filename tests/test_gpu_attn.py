"""GPU parity of the INT8 KV cache (q4k_kv_store) and the decode attention over
it (q4k_attn_decode) against the CPU oracle.

  - cache entries: codes and scales bit for bit equal to the oracle's, on
    N(0, 1) vectors, hand-worked ties, all-zero vectors, and magnitudes whose
    scale is subnormal, tiny or near the top of the fp32 range; entries
    outside the written positions are untouched;
  - attention: every output within max(2e-3 |oracle|, 1e-4) of the fp64
    oracle on caches the oracle quantized, over Qwen3-4B's grouping (32 query
    heads on 8 kv heads) and groups of 1, 2, 3 and 8, one to eight query
    tokens (causal rows), contexts from 1 position to 16384 with ragged tails,
    a capacity beyond the context, peaked scores, and all-equal scores;
  - repeated calls give the same bits and leave the workspace counters zero.
"""
import json
import os

import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu

HD = 128
SCALE = HD ** -0.5


@pytest.fixture(scope="module")
def q4k():
    import torch
    assert torch.cuda.is_available()
    import gemm_q4_super_amd as m
    m.lib()
    return m


def _empty_cache(n_kv, cap, fill=0x55):
    import torch
    kc = torch.full((n_kv, cap, HD), fill, dtype=torch.int8, device="cuda")
    vc = torch.full((n_kv, cap, HD), -fill, dtype=torch.int8, device="cuda")
    ks = torch.full((n_kv, cap), 7.0, dtype=torch.float32, device="cuda")
    vs = torch.full((n_kv, cap), -7.0, dtype=torch.float32, device="cuda")
    return kc, ks, vc, vs


def test_kv_store_bit_exact(q4k, oracle_lib):
    import torch
    n_kv, cap, pos0 = 8, 40, 5
    k, v = qi.make_kv(12, n_kv, HD, 11)
    k[1, 2] = 0.0                                   # all-zero vector
    v[2, 3] *= np.float32(1e-38)                    # subnormal scale
    k[3, 4] *= np.float32(1e-30)                    # scale below 2^-100
    v[4, 5] = np.float32(3e38) * np.tanh(v[4, 5])   # scale near the fp32 top
    k[5, 6] *= np.float32(1e35)
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "kv_int8_handbuilt.json")))
    for i, c in enumerate(g["cases"]):
        x = np.zeros(HD, np.float32)
        for key, val in c["x"].items():
            x[int(key)] = val
        k[6 + i, 0] = x
        v[6 + i, 7] = -x
    kc, ks, vc, vs = _empty_cache(n_kv, cap)
    q4k.q4k_kv_store(to_dev(k), to_dev(v), pos0, kc, ks, vc, vs)
    torch.cuda.synchronize()
    for which, x, codes, scales, fill, sfill in ((0, k, kc, ks, 0x55, 7.0), (1, v, vc, vs, -0x55, -7.0)):
        want_c, want_s = oracle_lib.kv_quantize(x)          # [12, n_kv, HD], [12, n_kv]
        got_c = codes.cpu().numpy()
        got_s = scales.cpu().numpy()
        written = slice(pos0, pos0 + 12)
        assert (got_c[:, written] == want_c.transpose(1, 0, 2)).all(), which
        assert (got_s[:, written].view(np.uint32) == want_s.T.view(np.uint32)).all(), which
        rest = np.ones(cap, bool)
        rest[written] = False
        assert (got_c[:, rest] == fill).all() and (got_s[:, rest] == sfill).all()


def _oracle_cache(oracle_lib, n_kv, cap, n_ctx, seed, zero_k=False):
    k, v = qi.make_kv(cap, n_kv, HD, seed)
    if zero_k:
        k[:] = 0.0
    kc, ks = oracle_lib.kv_quantize(k)
    vc, vs = oracle_lib.kv_quantize(v)
    # head-major [n_kv, cap, ...]; positions >= n_ctx hold data the call must not read
    return (np.ascontiguousarray(kc.transpose(1, 0, 2)), np.ascontiguousarray(ks.T),
            np.ascontiguousarray(vc.transpose(1, 0, 2)), np.ascontiguousarray(vs.T))


def _attn(q4k, q, cache, n_ctx, scale=SCALE, workspace="auto"):
    import torch
    kc, ks, vc, vs = (to_dev(a) for a in cache)
    out = q4k.q4k_attn_decode(to_dev(q), kc, ks, vc, vs, n_ctx, scale, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # (n_head, n_kv, M, n_ctx, cap, gain)
    (32, 8, 1, 1, 1, 1.0),
    (32, 8, 1, 7, 16, 1.0),
    (32, 8, 1, 32, 32, 1.0),
    (32, 8, 1, 33, 64, 1.0),
    (32, 8, 1, 100, 100, 1.0),
    (32, 8, 1, 1024, 1024, 1.0),
    (32, 8, 1, 1031, 1100, 1.0),
    (32, 8, 1, 1024, 1024, 8.0),
    (32, 8, 2, 300, 300, 1.0),
    (32, 8, 4, 100, 128, 3.0),
    (32, 8, 8, 4097, 4100, 1.0),
    (8, 8, 1, 513, 513, 1.0),       # one query head per kv head
    (4, 2, 3, 77, 80, 2.0),         # groups of 2
    (6, 2, 1, 200, 200, 1.0),       # groups of 3: a partly filled query block
    (64, 8, 8, 2000, 2000, 1.0),    # groups of 8, 64 query vectors per kv head
    (32, 8, 1, 16384, 16384, 1.0),  # the long-context decode
    (32, 8, 1, 2048, 2048, 1.0),    # short contexts: 8 to 16 chunks of 256 positions
    (32, 8, 1, 3000, 3072, 2.0),
    (32, 8, 2, 4096, 4096, 1.0),
]


@pytest.mark.parametrize("n_head,n_kv,M,n_ctx,cap,gain", CASES)
def test_attn_vs_oracle(q4k, oracle_lib, n_head, n_kv, M, n_ctx, cap, gain):
    print("attn n_head=%d n_kv=%d M=%d n_ctx=%d cap=%d gain=%g" % (n_head, n_kv, M, n_ctx, cap, gain),
          flush=True)
    cache = _oracle_cache(oracle_lib, n_kv, cap, n_ctx, seed=1000 + n_ctx)
    q = qi.make_query(M, n_head, HD, seed=2000 + n_ctx, gain=gain)
    got = _attn(q4k, q, cache, n_ctx)
    ref = oracle_lib.attn_int8kv(q, *cache, n_ctx, SCALE, parallel=True)
    assert_close(got, ref, "attn")


def test_attn_equal_scores_is_mean(q4k, oracle_lib):
    # all-zero keys: every score is 0 and each output is the mean of the values
    cache = _oracle_cache(oracle_lib, 8, 700, 700, seed=5, zero_k=True)
    q = qi.make_query(2, 32, HD, seed=6)
    got = _attn(q4k, q, cache, 700)
    ref = oracle_lib.attn_int8kv(q, *cache, 700, SCALE)
    assert_close(got, ref, "attn equal scores")


def test_attn_deterministic_and_counters_left_zero(q4k, oracle_lib):
    import torch
    nbytes = q4k.q4k_attn_workspace_bytes(1, 32, 8)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    cache = _oracle_cache(oracle_lib, 8, 3000, 3000, seed=9)
    q = qi.make_query(1, 32, HD, seed=10)
    a = _attn(q4k, q, cache, 3000, workspace=ws)
    assert (ws[:4096].cpu().numpy() == 0).all()
    b = _attn(q4k, q, cache, 2999, workspace=ws)
    c = _attn(q4k, q, cache, 3000, workspace=ws)
    assert (ws[:4096].cpu().numpy() == 0).all()
    assert (a.view(np.uint32) == c.view(np.uint32)).all()
    assert_close(b, oracle_lib.attn_int8kv(q, *cache, 2999, SCALE, parallel=True), "attn 2999")


def test_attn_store_then_read(q4k, oracle_lib):
    """Cache written by q4k_kv_store, position by position as decode does, then
    read by q4k_attn_decode: equal to the oracle on the oracle's own cache."""
    import torch
    n_kv, cap, n_ctx = 8, 96, 90
    k, v = qi.make_kv(n_ctx, n_kv, HD, 21)
    kc, ks, vc, vs = _empty_cache(n_kv, cap)
    dk, dv = to_dev(k), to_dev(v)
    q4k.q4k_kv_store(dk[:64], dv[:64], 0, kc, ks, vc, vs)     # a prompt of 64
    for t in range(64, n_ctx):                                 # then one token at a time
        q4k.q4k_kv_store(dk[t:t + 1], dv[t:t + 1], t, kc, ks, vc, vs)
    q = qi.make_query(1, 32, HD, seed=22)
    out = q4k.q4k_attn_decode(to_dev(q), kc, ks, vc, vs, n_ctx, SCALE)
    torch.cuda.synchronize()
    okc, oks = oracle_lib.kv_quantize(k)
    ovc, ovs = oracle_lib.kv_quantize(v)
    cache = (okc.transpose(1, 0, 2), oks.T, ovc.transpose(1, 0, 2), ovs.T)
    ref = oracle_lib.attn_int8kv(q, *cache, n_ctx, SCALE)
    assert_close(out.cpu().numpy(), ref, "attn after store")
