"""Seeded synthetic inputs for the Q4_K x Q8 matrix products.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It draws random numbers and encodes Q4_K fields into bytes; it holds
none of the arithmetic of the products themselves (no dequantisation, no
activation quantisation, no dot products), so neither side can borrow the
other's maths through it.

Q4_K super-block (public GGUF format; the pages name "Q4_K_M" weights but do not
print the layout, see "genie-ai-runtime ..." section 0 and section 3, Path E):
one super-block covers 256 consecutive weights of one row in 144 bytes:

    bytes 0..1    d      fp16, scale applied to the 6-bit sub-block scales
    bytes 2..3    dmin   fp16, scale applied to the 6-bit sub-block mins
    bytes 4..15   12 bytes holding eight 6-bit scales sc[j] and eight mins mn[j]
    bytes 16..143 128 bytes of 4-bit quants

Weight value: w = d*sc[j]*q - dmin*mn[j], j = element // 32.

Field distributions follow the synthetic workloads: quants uniform 0..15,
scales and mins uniform 0..63, d and dmin uniform in [1e-4, 1e-3] rounded to
fp16 (the stored fp16 is the truth); activations N(0, 1) fp32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK = 256            # weights per super-block
SB_BYTES = 144      # bytes per super-block
QBLK = 32           # activation block (and weight sub-block) length

# Qwen3-4B-shaped projections: (name, K, N) for y = x W^T with W of N rows x K cols.
QWEN3_4B_LAYER = (
    ("q", 2560, 4096),
    ("k", 2560, 1024),
    ("v", 2560, 1024),
    ("o", 4096, 2560),
    ("gate", 2560, 9728),
    ("up", 2560, 9728),
    ("down", 9728, 2560),
)
QWEN3_4B_LAYERS = 36

# Qwen3-4B attention: 32 query heads sharing 8 kv heads, head_dim 128.
QWEN3_4B_HEADS = 32
QWEN3_4B_KV_HEADS = 8
QWEN3_4B_HEAD_DIM = 128

# 8B-A1B-style routed-expert layer.
MOE_EXPERTS = 64
MOE_HIDDEN = 2048
MOE_FFN = 1024
MOE_TOPK = 8


@dataclass
class Q4KFields:
    """Unpacked Q4_K fields of an N x K matrix (nsb = K // 256 super-blocks per row)."""
    q: np.ndarray      # uint8 [N, nsb, 256], 0..15, in element order
    sc: np.ndarray     # uint8 [N, nsb, 8],   0..63
    mn: np.ndarray     # uint8 [N, nsb, 8],   0..63
    d: np.ndarray      # float16 [N, nsb]
    dmin: np.ndarray   # float16 [N, nsb]

    @property
    def shape(self):
        n, nsb, _ = self.q.shape
        return n, nsb * QK


def draw_q4k_fields(N: int, K: int, seed: int,
                    d_range=(1e-4, 1e-3)) -> Q4KFields:
    """Draw the Q4_K fields of an N x K matrix from a seeded PCG64 stream."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    nsb = K // QK
    q = rng.integers(0, 16, size=(N, nsb, QK), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(N, nsb, 8), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(N, nsb, 8), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, nsb)).astype(np.float16)
    dmin = rng.uniform(d_range[0], d_range[1], size=(N, nsb)).astype(np.float16)
    return Q4KFields(q=q, sc=sc, mn=mn, d=d, dmin=dmin)


def pack_q4k(f: Q4KFields) -> np.ndarray:
    """Encode fields into GGUF Q4_K bytes: uint8 [N, nsb*144], rows contiguous.

    Scale/min packing of the 12 bytes B[0..11]:
      j < 4 : low 6 bits of B[j] = sc[j], low 6 bits of B[j+4] = mn[j]
      j >= 4: low nibble of B[j+4] = sc[j] & 15, high nibble = mn[j] & 15,
              top 2 bits of B[j-4] = sc[j] >> 4, top 2 bits of B[j] = mn[j] >> 4
    Quants: for group g (elements 64g..64g+63), byte 32g+l holds element
    64g+l in its low nibble and element 64g+32+l in its high nibble.
    """
    q, sc, mn = f.q.astype(np.uint16), f.sc.astype(np.uint16), f.mn.astype(np.uint16)
    if q.max(initial=0) > 15 or sc.max(initial=0) > 63 or mn.max(initial=0) > 63:
        raise ValueError("field out of range")
    N, nsb, _ = q.shape
    out = np.zeros((N, nsb, SB_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = f.d.astype("<f2").view(np.uint8).reshape(N, nsb, 2)
    out[:, :, 2:4] = f.dmin.astype("<f2").view(np.uint8).reshape(N, nsb, 2)
    B = np.zeros((N, nsb, 12), dtype=np.uint16)
    for j in range(4):
        B[..., j] = sc[..., j] | ((sc[..., j + 4] >> 4) << 6)
        B[..., j + 4] = mn[..., j] | ((mn[..., j + 4] >> 4) << 6)
        B[..., j + 8] = (sc[..., j + 4] & 15) | ((mn[..., j + 4] & 15) << 4)
    out[:, :, 4:16] = B.astype(np.uint8)
    qg = q.reshape(N, nsb, 4, 2, 32)               # [group, half, l]
    qs = qg[:, :, :, 0, :] | (qg[:, :, :, 1, :] << 4)
    out[:, :, 16:] = qs.reshape(N, nsb, 128).astype(np.uint8)
    return out.reshape(N, nsb * SB_BYTES)


def make_q4k(N: int, K: int, seed: int) -> tuple[np.ndarray, Q4KFields]:
    """Packed bytes and fields of a seeded N x K Q4_K matrix."""
    f = draw_q4k_fields(N, K, seed)
    return pack_q4k(f), f


def make_q4k_bytes(N: int, K: int, seed: int) -> np.ndarray:
    """Packed Q4_K bytes of a seeded N x K matrix, drawn directly as bytes.

    Because quants (0..15), scales and mins (0..63) are uniform over power-of-two
    ranges, every one of the 140 scale/min/quant bytes of a super-block is a
    uniform byte, so this has the same field distribution as `make_q4k` at a
    fraction of the cost; only d and dmin are drawn as fp16 values.  Used for the
    multi-gigabyte sweeps; the small cases use `make_q4k`.
    """
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    nsb = K // QK
    out = np.frombuffer(rng.bytes(N * nsb * SB_BYTES), dtype=np.uint8)
    out = out.reshape(N, nsb, SB_BYTES).copy()
    dd = rng.uniform(1e-4, 1e-3, size=(N, nsb, 2)).astype("<f2")
    out[:, :, 0:4] = dd.view(np.uint8).reshape(N, nsb, 4)
    return out.reshape(N, nsb * SB_BYTES)


# Q6_K super-block (public GGUF format; real "Q4_K_M" files keep some tensors in
# Q6_K, and the decode kernels genie's "Path G" targets are Q6_K ones --
# "genie-ai-runtime ...", section 6, "The negatives I kept" -- but the pages do
# not print the layout):
# 256 weights of one row in 210 bytes:
#
#     bytes 0..127    ql   low 4 bits of the 6-bit quants
#     bytes 128..191  qh   high 2 bits of the 6-bit quants
#     bytes 192..207  sc   int8 scale per 16 weights
#     bytes 208..209  d    fp16
#
# Weight value: w = d*sc[e // 16]*(q[e] - 32).  Element e = 128h + 32t + l
# (h < 2, t < 4, l < 32) keeps its low 4 bits in ql[64h + 32(t % 2) + l] (low
# nibble for t < 2, high nibble for t >= 2) and its high 2 bits in bits 2t, 2t+1
# of qh[32h + l].
Q6_SB_BYTES = 210


@dataclass
class Q6KFields:
    """Unpacked Q6_K fields of an N x K matrix (nsb = K // 256 super-blocks per row)."""
    q: np.ndarray      # uint8 [N, nsb, 256], 0..63, in element order
    sc: np.ndarray     # int8  [N, nsb, 16]
    d: np.ndarray      # float16 [N, nsb]


def draw_q6k_fields(N: int, K: int, seed: int, d_range=(1e-4, 1e-3)) -> Q6KFields:
    """Draw the Q6_K fields of an N x K matrix: quants uniform 0..63, scales
    uniform over all int8 values, d uniform in d_range rounded to fp16."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    nsb = K // QK
    q = rng.integers(0, 64, size=(N, nsb, QK), dtype=np.uint8)
    sc = rng.integers(-128, 128, size=(N, nsb, 16), dtype=np.int16).astype(np.int8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, nsb)).astype(np.float16)
    return Q6KFields(q=q, sc=sc, d=d)


def pack_q6k(f: Q6KFields) -> np.ndarray:
    """Encode fields into GGUF Q6_K bytes: uint8 [N, nsb*210], rows contiguous."""
    q = f.q.astype(np.uint16)
    if q.max(initial=0) > 63:
        raise ValueError("field out of range")
    N, nsb, _ = q.shape
    out = np.zeros((N, nsb, Q6_SB_BYTES), dtype=np.uint8)
    qq = q.reshape(N, nsb, 2, 4, 32)                  # [half h, part t, l]
    lo, hi = qq & 15, qq >> 4
    ql = np.zeros((N, nsb, 2, 2, 32), dtype=np.uint16)   # [h, t % 2, l]
    ql[:, :, :, 0, :] = lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4)
    ql[:, :, :, 1, :] = lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)
    qh = hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4) | (hi[:, :, :, 3, :] << 6)
    out[:, :, 0:128] = ql.reshape(N, nsb, 128).astype(np.uint8)
    out[:, :, 128:192] = qh.reshape(N, nsb, 64).astype(np.uint8)
    out[:, :, 192:208] = f.sc.astype(np.int8).view(np.uint8)
    out[:, :, 208:210] = f.d.astype("<f2").view(np.uint8).reshape(N, nsb, 2)
    return out.reshape(N, nsb * Q6_SB_BYTES)


def make_q6k(N: int, K: int, seed: int) -> tuple[np.ndarray, Q6KFields]:
    """Packed bytes and fields of a seeded N x K Q6_K matrix."""
    f = draw_q6k_fields(N, K, seed)
    return pack_q6k(f), f


def make_q6k_bytes(N: int, K: int, seed: int) -> np.ndarray:
    """Packed Q6_K bytes of a seeded N x K matrix, drawn directly as bytes: every
    quant bit and scale byte is uniform, so uniform bytes give the field
    distribution of `make_q6k`; only d is drawn as an fp16 value."""
    if K % QK:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    nsb = K // QK
    out = np.frombuffer(rng.bytes(N * nsb * Q6_SB_BYTES), dtype=np.uint8)
    out = out.reshape(N, nsb, Q6_SB_BYTES).copy()
    dd = rng.uniform(1e-4, 1e-3, size=(N, nsb)).astype("<f2")
    out[:, :, 208:210] = dd.view(np.uint8).reshape(N, nsb, 2)
    return out.reshape(N, nsb * Q6_SB_BYTES)


def make_act(M: int, K: int, seed: int) -> np.ndarray:
    """fp32 [M, K] activations drawn from N(0, 1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, K), dtype=np.float32)


def make_routing(T: int, n_experts: int, topk: int, seed: int):
    """Per token: `topk` distinct expert ids drawn uniformly (in draw order) and
    routing weights = softmax of `topk` N(0, 1) logits, in fp32.

    Returns (ids int32 [T, topk], weights fp32 [T, topk]).  The weights are an
    input of the routed layer, shared by both sides.
    """
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(n_experts, size=topk, replace=False)
                    for _ in range(T)]).astype(np.int32).reshape(T, topk)
    logits = rng.standard_normal((T, topk), dtype=np.float32)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def make_kv(n_pos: int, n_kv: int, hd: int, seed: int):
    """fp32 keys and values [n_pos, n_kv, hd], each drawn from N(0, 1) (the
    per-head vectors after the model's q/k normalisation have unit-scale
    elements)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_pos, n_kv, hd), dtype=np.float32)
    v = rng.standard_normal((n_pos, n_kv, hd), dtype=np.float32)
    return k, v


def make_query(M: int, n_head: int, hd: int, seed: int, gain: float = 1.0) -> np.ndarray:
    """fp32 queries [M, n_head, hd] drawn from gain * N(0, 1); a larger gain
    gives peakier attention."""
    rng = np.random.default_rng(seed)
    return (gain * rng.standard_normal((M, n_head, hd))).astype(np.float32)


# Seed scheme of the synthetic workloads.
def weight_seed(workload: int, layer: int, proj: int) -> int:
    return 1000 * workload + 10 * layer + proj


def expert_seed(layer: int, expert: int, which: int) -> int:
    """which: 0 = gate, 1 = up, 2 = down."""
    return 40000 + 1000 * layer + 3 * expert + which


def act_seed(call_index: int) -> int:
    return 900000 + call_index


def routing_seed(layer: int) -> int:
    return 700000 + layer


def kv_seed(layer: int) -> int:
    return 800000 + layer


def query_seed(layer: int) -> int:
    return 850000 + layer
