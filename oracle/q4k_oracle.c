/*
 * CPU oracle for the Q4_K x Q8 matrix products -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C: the definition of what the GPU path computes,
 * written out without blocking, fusion or reordering.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load this library; the
 * product path never calls it and shares no code, header or table with it.
 *
 * What is computed (sources):
 *  - Weights: Q4_K super-blocks (public GGUF format; the pages name the
 *    Q4_K_M weight format -- "genie-ai-runtime: a Jetson edge LLM inference
 *    engine that beats llama.cpp", section 0 and section 3 "The tensor-core
 *    kernel (Path E)" -- but do not print its bytes).  256 weights of one row
 *    in 144 bytes: fp16 d, fp16 dmin, twelve bytes of 6-bit sub-block scales
 *    and mins, 128 bytes of 4-bit quants.  w = d*sc[j]*q - dmin*mn[j] with
 *    j = element/32, evaluated exactly in fp64.
 *  - Activations: Q8 blocks of 32 values (format of the 1024x1024 single-GEMV
 *    workload): amax = max|x|, scale = fl32(amax/127), code =
 *    clamp(round-half-even(fl32(x/scale)), -127, 127), block sum = sum of codes;
 *    an all-zero block has scale 0 and codes 0.  Evaluated in fp32, bit for bit.
 *    The value used downstream is scale*code, exact in fp64.
 *  - Product: y[m][n] = sum_k w[n][k] * xhat[m][k] in fp64 (y = x W^T, the
 *    "K->N" projection naming).  This is the decode GEMV of section 2 ("The
 *    target hardware (and the roofline that dictates strategy)") and the
 *    prefill GEMM of section 3, which only regroup this sum.
 *  - A second, integer-structured form of the same sum (per 32-element
 *    sub-block integer dots D = sum q*c, then the scales and the min term),
 *    used to check that regrouping and to export D for bit-exact checks.
 *  - Routed experts (the mixture-of-experts layer of "I'm making LLMs work on
 *    small and old devices", intro and "Lessons"): per token, the selected
 *    experts' gate/up products, SwiGLU h = silu(g)*u (the pages name no
 *    activation; SwiGLU is the reading), Q8 of h, the expert's down product,
 *    and the routing-weighted sum in slot order.
 *
 *  - Q6_K weights (public GGUF format; real Q4_K_M files keep some tensors in
 *    Q6_K and the decode kernels of genie's "Path G" -- section 6, "The
 *    negatives I kept" -- are Q6_K ones, but the pages do not print the
 *    bytes): 256 weights of one row in
 *    210 bytes, ql[128] low 4 bits and qh[64] high 2 bits of 6-bit quants,
 *    int8 scales per 16 weights, fp16 d; w = d*sc[e/16]*(q - 32), exact in
 *    fp64; the same fp64 product against Q8 activations.
 *  - INT8 KV cache and decode attention (genie's Path I, section 4, "Memory-
 *    first: making every byte count"): each (layer, position, kv-head) vector
 *    of head_dim values is kept as int8 codes with one fp32 absmax scale,
 *    quantized by the Q8 rule above over the whole vector.  Attention is the
 *    transformer's scaled dot-product softmax attention (the pages name the
 *    model, Qwen3-4B, not the formula) with grouped kv heads, read from the
 *    dequantized cache scale*code and evaluated in fp64.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 *
 * Built twice from this one file: single-threaded (liboracle.so) and with
 * OpenMP over the output rows of the products (liboracle_omp.so, for the
 * full-size checks and the all-core CPU baseline).  The arithmetic of every
 * output is the same sequential loop in both.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define QK 256
#define SB_BYTES 144
#define QB 32

/* IEEE binary16 -> double, exact, from the encoding's definition. */
static double half_bits_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Unpack one 144-byte super-block into its fields. */
void oracle_unpack_q4k(const uint8_t *sb, double *d, double *dmin,
                       int32_t *sc, int32_t *mn, int32_t *q)
{
    const uint8_t *B = sb + 4;
    const uint8_t *qs = sb + 16;
    *d = half_bits_to_double((uint16_t)(sb[0] | (sb[1] << 8)));
    *dmin = half_bits_to_double((uint16_t)(sb[2] | (sb[3] << 8)));
    for (int j = 0; j < 4; ++j) {
        sc[j] = B[j] & 63;
        mn[j] = B[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (B[j + 4] & 15) | ((B[j - 4] >> 6) << 4);
        mn[j] = (B[j + 4] >> 4) | ((B[j] >> 6) << 4);
    }
    for (int e = 0; e < QK; ++e) {
        int g = e / 64, r = e % 64;
        q[e] = r < 32 ? (qs[32 * g + r] & 15) : (qs[32 * g + r - 32] >> 4);
    }
}

/* Dequantize one row of K weights (K/256 super-blocks) into fp64. */
void oracle_dequant_row(const uint8_t *row, int64_t K, double *w)
{
    int32_t sc[8], mn[8], q[QK];
    double d, dmin;
    for (int64_t b = 0; b < K / QK; ++b) {
        oracle_unpack_q4k(row + b * SB_BYTES, &d, &dmin, sc, mn, q);
        for (int e = 0; e < QK; ++e) {
            int j = e / QB;
            w[b * QK + e] = d * sc[j] * q[e] - dmin * mn[j];
        }
    }
}

/* Q8 quantization of M rows of K fp32 values, bit for bit in fp32. */
void oracle_quantize_act(const float *x, int64_t M, int64_t K,
                         int8_t *codes, float *scales, int32_t *sums)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t blk = 0; blk < K / QB; ++blk) {
            const float *xb = x + m * K + blk * QB;
            int8_t *cb = codes + m * K + blk * QB;
            float amax = 0.0f;
            for (int i = 0; i < QB; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            float dq = amax / 127.0f;
            int32_t s = 0;
            for (int i = 0; i < QB; ++i) {
                int c = 0;
                if (dq != 0.0f) {
                    float t = xb[i] / dq;
                    float r = rintf(t); /* round half to even (default mode) */
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (int)r;
                }
                cb[i] = (int8_t)c;
                s += c;
            }
            scales[m * (K / QB) + blk] = dq;
            sums[m * (K / QB) + blk] = s;
        }
    }
}

/* SwiGLU in fp64 from fp32 inputs, rounded once to fp32:
 * h = g / (1 + exp(-g)) * u. */
void oracle_swiglu(const float *g, const float *u, int64_t n, float *h)
{
    for (int64_t i = 0; i < n; ++i) {
        double gd = (double)g[i];
        h[i] = (float)(gd / (1.0 + exp(-gd)) * (double)u[i]);
    }
}

/* y[m][r] = sum_k w[n_r][k] * scale[m][k/32] * code[m][k], fp64, for the rows
 * n_r listed in `rows` (all N rows when rows == NULL, nrows == N). */
void oracle_matvec(const uint8_t *w, int64_t N, int64_t K,
                   const int8_t *codes, const float *scales, int64_t M,
                   const int64_t *rows, int64_t nrows, double *y)
{
    int64_t row_bytes = K / QK * SB_BYTES;
    (void)N;
    /* Output rows are independent; a build with OpenMP takes them in parallel
     * (each row's sum is the same sequential loop either way). */
#pragma omp parallel
    {
        double *wr = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t n = rows ? rows[r] : r;
            oracle_dequant_row(w + n * row_bytes, K, wr);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double xh = (double)scales[m * (K / QB) + k / QB] * (double)codes[m * K + k];
                    acc += wr[k] * xh;
                }
                y[m * nrows + r] = acc;
            }
        }
        free(wr);
    }
}

/* Threads the OpenMP runtime would use (1 in a build without OpenMP). */
int oracle_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Integer sub-block dots D[m][r][j] = sum_{i<32} q[n_r][32j+i] * code[m][32j+i]. */
void oracle_subblock_dots(const uint8_t *w, int64_t K, const int8_t *codes,
                          int64_t M, const int64_t *rows, int64_t nrows,
                          int32_t *D)
{
    int64_t row_bytes = K / QK * SB_BYTES, nsub = K / QB;
    int32_t sc[8], mn[8], q[QK];
    double d, dmin;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t *row = w + rows[r] * row_bytes;
        for (int64_t b = 0; b < K / QK; ++b) {
            oracle_unpack_q4k(row + b * SB_BYTES, &d, &dmin, sc, mn, q);
            for (int64_t m = 0; m < M; ++m)
                for (int j = 0; j < 8; ++j) {
                    int32_t acc = 0;
                    for (int i = 0; i < QB; ++i)
                        acc += q[QB * j + i] * codes[m * K + b * QK + QB * j + i];
                    D[(m * nrows + r) * nsub + b * 8 + j] = acc;
                }
        }
    }
}

/* The same product in the integer-structured form:
 * y = sum_b [ d * sum_j sc_j * a_j * D_j  -  dmin * sum_j mn_j * a_j * S_j ],
 * a_j = activation scale, S_j = activation code sum, all in fp64. */
void oracle_matvec_intform(const uint8_t *w, int64_t K, const int8_t *codes,
                           const float *scales, const int32_t *sums, int64_t M,
                           const int64_t *rows, int64_t nrows, double *y)
{
    int64_t row_bytes = K / QK * SB_BYTES, nsub = K / QB;
    int32_t sc[8], mn[8], q[QK];
    double d, dmin;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t *row = w + rows[r] * row_bytes;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t b = 0; b < K / QK; ++b) {
                oracle_unpack_q4k(row + b * SB_BYTES, &d, &dmin, sc, mn, q);
                double main_t = 0.0, min_t = 0.0;
                for (int j = 0; j < 8; ++j) {
                    int32_t Dj = 0;
                    for (int i = 0; i < QB; ++i)
                        Dj += q[QB * j + i] * codes[m * K + b * QK + QB * j + i];
                    double a = scales[m * nsub + b * 8 + j];
                    main_t += sc[j] * a * Dj;
                    min_t += mn[j] * a * sums[m * nsub + b * 8 + j];
                }
                acc += d * main_t - dmin * min_t;
            }
            y[m * nrows + r] = acc;
        }
    }
}

/* Routed-expert product.  Experts are matrices of N rows x K columns at
 * `expert_stride` bytes from each other.  For token t and slot s the expert is
 * ids[t*topk+s]; its activation row is t (act_per_slot == 0) or t*topk+s
 * (act_per_slot == 1).  With route_w == NULL the output is per slot,
 * y[(t*topk+s)][n]; otherwise y[t][n] = sum_s route_w[t*topk+s] * (slot product),
 * summed in slot order. */
void oracle_moe_matvec(const uint8_t *w, int64_t n_experts, int64_t expert_stride,
                       int64_t N, int64_t K, const int32_t *ids,
                       const float *route_w, int64_t T, int64_t topk,
                       const int8_t *codes, const float *scales,
                       int act_per_slot, double *y)
{
    double *tmp = (double *)malloc(sizeof(double) * N);
    (void)n_experts;
    if (route_w)
        memset(y, 0, sizeof(double) * T * N);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t s = 0; s < topk; ++s) {
            int64_t e = ids[t * topk + s];
            int64_t arow = act_per_slot ? t * topk + s : t;
            oracle_matvec(w + e * expert_stride, N, K, codes + arow * K,
                          scales + arow * (K / QB), 1, NULL, N, tmp);
            if (route_w) {
                double rw = route_w[t * topk + s];
                for (int64_t n = 0; n < N; ++n)
                    y[t * N + n] += rw * tmp[n];
            } else {
                memcpy(y + (t * topk + s) * N, tmp, sizeof(double) * N);
            }
        }
    }
    free(tmp);
}

/* Whole routed-expert FFN layer: Q8(x) -> gate/up per slot (fp64, rounded to
 * fp32) -> SwiGLU -> Q8(h) -> down per slot -> routing-weighted sum.
 * Intermediates g, u, h (fp32 [T*topk][F]) and the Q8 of h are written out when
 * the pointers are non-NULL.  y is fp64 [T][H]. */
void oracle_moe_layer(const uint8_t *w_gate, const uint8_t *w_up,
                      const uint8_t *w_down, int64_t n_experts,
                      int64_t stride_gu, int64_t stride_down,
                      int64_t H, int64_t F, const int32_t *ids,
                      const float *route_w, int64_t T, int64_t topk,
                      const float *x, float *g_out, float *u_out, float *h_out,
                      int8_t *hc_out, float *hs_out, int32_t *hsum_out,
                      double *y)
{
    int64_t P = T * topk;
    int8_t *xc = (int8_t *)malloc(T * H);
    float *xs = (float *)malloc(sizeof(float) * T * (H / QB));
    int32_t *xsum = (int32_t *)malloc(sizeof(int32_t) * T * (H / QB));
    double *gd = (double *)malloc(sizeof(double) * P * F);
    double *ud = (double *)malloc(sizeof(double) * P * F);
    float *g = (float *)malloc(sizeof(float) * P * F);
    float *u = (float *)malloc(sizeof(float) * P * F);
    float *h = (float *)malloc(sizeof(float) * P * F);
    int8_t *hc = (int8_t *)malloc(P * F);
    float *hs = (float *)malloc(sizeof(float) * P * (F / QB));
    int32_t *hsum = (int32_t *)malloc(sizeof(int32_t) * P * (F / QB));

    oracle_quantize_act(x, T, H, xc, xs, xsum);
    oracle_moe_matvec(w_gate, n_experts, stride_gu, F, H, ids, NULL, T, topk, xc, xs, 0, gd);
    oracle_moe_matvec(w_up, n_experts, stride_gu, F, H, ids, NULL, T, topk, xc, xs, 0, ud);
    for (int64_t i = 0; i < P * F; ++i) {
        g[i] = (float)gd[i];
        u[i] = (float)ud[i];
    }
    oracle_swiglu(g, u, P * F, h);
    oracle_quantize_act(h, P, F, hc, hs, hsum);
    oracle_moe_matvec(w_down, n_experts, stride_down, H, F, ids, route_w, T, topk, hc, hs, 1, y);

    if (g_out) memcpy(g_out, g, sizeof(float) * P * F);
    if (u_out) memcpy(u_out, u, sizeof(float) * P * F);
    if (h_out) memcpy(h_out, h, sizeof(float) * P * F);
    if (hc_out) memcpy(hc_out, hc, P * F);
    if (hs_out) memcpy(hs_out, hs, sizeof(float) * P * (F / QB));
    if (hsum_out) memcpy(hsum_out, hsum, sizeof(int32_t) * P * (F / QB));
    free(xc); free(xs); free(xsum); free(gd); free(ud); free(g); free(u); free(h);
    free(hc); free(hs); free(hsum);
}

/* ---------------------------------------------------------------- Q6_K -- */

#define Q6_SB_BYTES 210

/* Unpack one 210-byte Q6_K super-block: element e = 128h + 32t + l takes its
 * low 4 bits from ql[64h + 32(t%2) + l] (low nibble for t < 2, high for t >= 2)
 * and its high 2 bits from bits 2t..2t+1 of qh[32h + l]. */
void oracle_unpack_q6k(const uint8_t *sb, double *d, int32_t *sc, int32_t *q)
{
    const uint8_t *ql = sb, *qh = sb + 128;
    *d = half_bits_to_double((uint16_t)(sb[208] | (sb[209] << 8)));
    for (int j = 0; j < 16; ++j)
        sc[j] = (int8_t)sb[192 + j];
    for (int e = 0; e < QK; ++e) {
        int h = e / 128, t = (e % 128) / 32, l = e % 32;
        int lo = ql[64 * h + 32 * (t % 2) + l];
        lo = t < 2 ? (lo & 15) : (lo >> 4);
        int hi = (qh[32 * h + l] >> (2 * t)) & 3;
        q[e] = lo | (hi << 4);
    }
}

/* Dequantize one Q6_K row of K weights into fp64. */
void oracle_q6k_dequant_row(const uint8_t *row, int64_t K, double *w)
{
    int32_t sc[16], q[QK];
    double d;
    for (int64_t b = 0; b < K / QK; ++b) {
        oracle_unpack_q6k(row + b * Q6_SB_BYTES, &d, sc, q);
        for (int e = 0; e < QK; ++e)
            w[b * QK + e] = d * sc[e / 16] * (q[e] - 32);
    }
}

/* y[m][r] = sum_k w[n_r][k] * scale[m][k/32] * code[m][k] for Q6_K weights,
 * fp64, rows as in oracle_matvec. */
void oracle_q6k_matvec(const uint8_t *w, int64_t N, int64_t K,
                       const int8_t *codes, const float *scales, int64_t M,
                       const int64_t *rows, int64_t nrows, double *y)
{
    int64_t row_bytes = K / QK * Q6_SB_BYTES;
    (void)N;
#pragma omp parallel
    {
        double *wr = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t n = rows ? rows[r] : r;
            oracle_q6k_dequant_row(w + n * row_bytes, K, wr);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double xh = (double)scales[m * (K / QB) + k / QB] * (double)codes[m * K + k];
                    acc += wr[k] * xh;
                }
                y[m * nrows + r] = acc;
            }
        }
        free(wr);
    }
}

/* ------------------------------------------------------- INT8 KV cache -- */

/* Q8 of R vectors of hd fp32 values, one scale per vector (the cache entry of
 * one position and kv-head): scale = fl32(amax/127), code =
 * clamp(rne(fl32(x/scale)), -127, 127); an all-zero vector has scale 0 and
 * codes 0.  Evaluated in fp32, bit for bit. */
void oracle_kv_quantize(const float *x, int64_t R, int64_t hd, int8_t *codes, float *scales)
{
    for (int64_t r = 0; r < R; ++r) {
        const float *xr = x + r * hd;
        float amax = 0.0f;
        for (int64_t i = 0; i < hd; ++i) {
            float a = fabsf(xr[i]);
            if (a > amax)
                amax = a;
        }
        float d = amax / 127.0f;
        for (int64_t i = 0; i < hd; ++i) {
            int c = 0;
            if (d != 0.0f) {
                float t = xr[i] / d;
                float v = rintf(t);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                c = (int)v;
            }
            codes[r * hd + i] = (int8_t)c;
        }
        scales[r] = d;
    }
}

/* Decode attention of M query tokens over one layer's INT8 cache, in fp64.
 *   q      fp32 [M][n_head][hd]   (keys and queries already position-encoded)
 *   kc, vc int8 [n_kv][cap][hd],  ks, vs fp32 [n_kv][cap]
 *   out    fp64 [M][n_head][hd]
 * Query token m sits at position n_ctx - M + m and sees the positions
 * t < n_ctx - (M - 1 - m) (causal).  Head h reads kv head h / (n_head/n_kv).
 * s_t = scale * sum_i q[i] * ks[t]*kc[t][i];  p = softmax(s) over the visible
 * t;  out[i] = sum_t p_t * vs[t]*vc[t][i]. */
void oracle_attn_int8kv(const float *q, int64_t M, int64_t n_head, int64_t n_kv, int64_t hd,
                        const int8_t *kc, const float *ks, const int8_t *vc, const float *vs,
                        int64_t cap, int64_t n_ctx, double scale, double *out)
{
    const int64_t group = n_head / n_kv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t mh = 0; mh < M * n_head; ++mh) {
        const int64_t m = mh / n_head, h = mh % n_head, g = h / group;
        const int64_t L = n_ctx - (M - 1 - m);
        const float *qv = q + mh * hd;
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        double smax = -INFINITY;
        for (int64_t t = 0; t < L; ++t) {
            const int8_t *kr = kc + (g * cap + t) * hd;
            const double kscale = (double)ks[g * cap + t];
            double dot = 0.0;
            for (int64_t i = 0; i < hd; ++i)
                dot += (double)qv[i] * (kscale * (double)kr[i]);
            s[t] = scale * dot;
            if (s[t] > smax)
                smax = s[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            s[t] = exp(s[t] - smax);
            denom += s[t];
        }
        double *o = out + mh * hd;
        for (int64_t i = 0; i < hd; ++i)
            o[i] = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int8_t *vr = vc + (g * cap + t) * hd;
            const double w = s[t] / denom * (double)vs[g * cap + t];
            for (int64_t i = 0; i < hd; ++i)
                o[i] += w * (double)vr[i];
        }
        free(s);
    }
}
