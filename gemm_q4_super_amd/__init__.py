"""Q4_K x Q8 matrix products on AMD MI355X (gfx950).

Python binding of libq4k.so (C ABI in include/q4k.h).  The binding only
marshals arguments: PyTorch supplies device memory and the current stream;
every step of the computation runs in the library's HIP kernels.  There is no
CPU or PyTorch fallback: if the library is missing, importing the binding's
functions raises.

Functions carry the C names:
    q4k_quantize_act(x, gate=None)                   -> (codes, scales, sums)
    q4k_gemv(w, N, K, codes, scales, sums)           -> y [M, N]   (M <= 8)
    q4k_quantize_gemv(w, N, K, x)                    -> y [M, N]   (fp32 x, one launch)
    q4k_quantize_gemv_residual(w, N, K, x, r[, y=r]) -> r + Q8(x) W^T (residual add inside)
    q4k_quantize_gemv_batch([(w, N, x), ...], K)     -> [y, ...]   (<= 8 products, one launch)
    q4k_gemm(w, N, K, codes, scales, sums, workspace="auto") -> y [M, N]
    q4k_gemm_batch([(w, N), ...], K, codes, scales, sums, workspace="auto")
                                                     -> [y, ...] (<= 8 products, one launch)
        (both take library=lib_gemm_int8() for the GEMM's int8 contraction)
    gemm_workspace(device)                           -> the zero-filled GEMM workspace reused
                                                        by workspace="auto"
    q4k_moe_gemv(w, n_experts, stride, N, K, ids, route_w, codes, scales, sums,
                 act_per_slot, workspace=None)       -> y
    q4k_moe_ffn(w_gate, w_up, w_down, n_experts, stride_gate_up, stride_down, H, F,
                ids, route_w, x, workspace=None)     -> y [T, H]  (whole expert FFN layer)
    q6k_gemv(w, N, K, codes, scales)                 -> y [M, N]   (Q6_K weights, M <= 8)
    q6k_quantize_gemv(w, N, K, x)                    -> y [M, N]   (Q6_K, fp32 x, one launch)
    q6k_gemv_batch([(w, N)...], K, codes, scales)    -> [y_i]      (Q6_K, one launch)
    q6k_quantize_gemv_batch([(w, N, x)...], K)       -> [y_i]      (Q6_K, fp32 x, one launch)
    q6k_gemm(w, N, K, codes, scales, workspace="auto") -> y [M, N] (Q6_K prefill GEMM)
    q4k_kv_store(k, v, pos0, k_codes, k_scales, v_codes, v_scales)
                                                     (INT8 KV cache entries of M positions)
    q4k_attn_decode(q, k_codes, k_scales, v_codes, v_scales, n_ctx, scale, workspace="auto")
                                                     -> out [M, n_head, 128]
"""
from ._lib import (  # noqa: F401
    Q4KError,
    attn_workspace,
    gemm_workspace,
    lib,
    lib_gemm_int8,
    lib_path,
    q4k_gemm,
    q4k_gemm_batch,
    q4k_kv_store,
    q4k_attn_decode,
    q4k_attn_workspace_bytes,
    q4k_gemv,
    q4k_moe_ffn,
    q4k_moe_ffn_workspace_bytes,
    q4k_moe_gemv,
    q4k_moe_workspace_bytes,
    q4k_quantize_act,
    q4k_quantize_gemv,
    q4k_quantize_gemv_batch,
    q4k_quantize_gemv_residual,
    q4k_status_string,
    q6k_gemm,
    q6k_gemv,
    q6k_gemv_batch,
    q6k_quantize_gemv,
    q6k_quantize_gemv_batch,
    EXPORTED_SYMBOLS,
)
