// Small-batch GEMV on the matrix cores (q4k_gemv with M = 2..8 prepared Q8
// rows): y[m][n] = sum_k Q8(x)[m][k] * W[n][k], W in Q4_K.
//
// Verifying a few draft tokens in one pass reads every weight once for up to
// M activation rows ("genie-ai-runtime ...", speculative decoding), so the
// launch is still a weight stream; what limits the vector-unit GEMV at M > 2
// is how few weight bytes a wave can keep in flight once it holds M rows of
// activations and accumulators.  Here the integer sub-block dots run on
// v_mfma_i32_16x16x64_i8 and a wave keeps 16 rows x CPW super-blocks
// (2.3 KB each) in flight.
//
// One super-block column of a 16-row tile is four matrix instructions t = 0..3:
//  * weight operand (column n = lane % 16 = weight row, k-group q = lane / 16):
//    groups q = 0, 1 ("X") carry sub-block t, groups 2, 3 ("Y") sub-block 7 - t,
//    16 elements each: one nibble of every byte of a 16-byte quant chunk;
//  * activation operand (row i = lane % 16): rows 0-7 are activation rows
//    m = 0..7 holding the X sub-block's codes in groups 0, 1 and zeros in 2, 3;
//    rows 8-15 the same rows with the Y sub-block's codes in groups 2, 3
//    (zeros come from a zero slot in LDS; rows m >= M read it too);
//  * so the int32 result is the exact sub-block dot D for (row n, act row m):
//    lane (n, q) gets m = 4 (q % 2) .. +3, sub-block t (q < 2) or 7 - t.
// The fp32 epilogue rebuilds the streaming GEMV's super-block term
// T = (u0 + u2) + (u7 + u5), u_j = fma(a_j, f_j, RN(a_k f_k)), k = j ^ 1,
// f_j = fma(d sc_j, D_j, -RN(dmin mn_j S_j)) (superblock_term in q4k_device.h):
// X lanes form u0 + u2 from t = 0..3, Y lanes u7 + u5 (t = 0..3 are sub-blocks
// 7, 6, 5, 4), both halves go to LDS, and each row adds X + Y per column in
// column order.  Same values, operations and order as the streaming GEMV, so
// both paths give the same bits.
//
// A launch takes up to kMaxGemvBatch products with the same K and M (a
// launch group such as q|k|v): workgroups are dealt out over the products'
// tiles in order, each finding its product from its tile index (the first
// product's arguments lead the argument block, preloaded into registers); a
// one-product launch has its own entry kernel with no table.
//
// Workgroup: one 16-row tile and all K/256 columns; wave w owns columns
// [w CPW, (w + 1) CPW).  A wave stages its columns' Q8 codes, scales and sums
// in LDS (loads issued before its weight loads; no workgroup barrier before
// the dots), then issues all 3 CPW weight loads of 16 bytes per lane (header,
// two quant chunks), then runs the matrix instructions column by column.
#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kCodeRow = 272;   // LDS bytes per (column, activation row): 256 codes + 16 (bank spread)
constexpr int kMaxLds = 160 * 1024;
constexpr int kMaxCpw = 3;      // columns per wave, at most (16 waves: K up to 48 super-blocks)

// LDS layout of one workgroup (bytes): per column [M][272] codes + a 16-byte
// zero slot; then scales [nsb][8 j][8 m] and sums (as float) the same; then the
// half terms [16 rows][nsb][2][8 m].
__host__ __device__ constexpr int col_stride(int M) { return M * kCodeRow + 16; }
__host__ __device__ constexpr size_t mfma_lds_bytes(int M, int nsb) {
    return (size_t)nsb * (col_stride(M) + 2 * 256 + 16 * 64);
}

// Products 1.. of one launch: weights, outputs, rows, and the first tile of
// each (tile0[count] = all tiles; entry 0 unused, product 0 travels in the
// leading kernel arguments).
struct MfmaSet {
    const uint8_t *w[kMaxGemvBatch];
    float *y[kMaxGemvBatch];
    int N[kMaxGemvBatch];
    int tile0[kMaxGemvBatch + 1];
    int count;
};

// One workgroup: the 16-row tile of rows row_base.. of one product.
template <int CPW>
__device__ __forceinline__ void gemv_mfma_tile(
    const uint8_t *__restrict__ w, float *__restrict__ y, const int N, const int row_base,
    const int8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ sums, int nsb, int M) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nw = blockDim.x >> 6;
    const int n = lane & 15;           // weight row of the tile (operand column / output column)
    const int q = lane >> 4;           // k-group
    const bool Yh = q >= 2;            // this lane's sub-blocks: 7-t (Y) or t (X)
    const int K = nsb * 256, nblk = nsb * 8;
    const int cs = col_stride(M);
    uint8_t *lcodes = lds;
    float *la = reinterpret_cast<float *>(lds + (size_t)nsb * cs);   // [nsb][8 j][8 m]
    float *ls = la + (size_t)nsb * 64;
    float *lterm = ls + (size_t)nsb * 64;                             // [16][nsb][2][8]
    const int wcol0 = wave * CPW;
    const int ncols = min(CPW, nsb - wcol0);   // >= 1 (the host sizes the workgroup)

    // ---- staging loads (branch-free: lanes and columns past the data load a
    // clamped address and store nothing):
    // codes, per column ceil(M/4) loads of 4 rows x 256 bytes; scales and sums,
    // 16 bytes per lane, two columns per load (lanes 32i..32i+31: column 2k+i,
    // pieces 0..2M-1 scales, 2M..4M-1 sums, piece = row m = p/2, sub-blocks 4(p%2)..+3)
    const int cm0 = min(lane >> 4, M - 1), cm1 = min((lane >> 4) + 4, M - 1);
    const int co = 16 * (lane & 15);
    const int sp = lane & 31;
    const bool s_sum = sp >= 2 * M, s_live = sp < 4 * M;
    const int s_m = min((s_sum ? sp - 2 * M : sp) >> 1, M - 1), s_h = sp & 1;
    const uint8_t *s_src = s_sum ? reinterpret_cast<const uint8_t *>(sums)
                                 : reinterpret_cast<const uint8_t *>(scales);
    constexpr int kSP = (CPW + 1) / 2;
    i32x4 cv0[CPW], cv1[CPW], sv[kSP];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int b = min(wcol0 + c, nsb - 1);
        cv0[c] = *reinterpret_cast<const i32x4 *>(codes + (int64_t)cm0 * K + 256 * b + co);
        if (M > 4) cv1[c] = *reinterpret_cast<const i32x4 *>(codes + (int64_t)cm1 * K + 256 * b + co);
    }
#pragma unroll
    for (int k = 0; k < kSP; ++k) {
        const int b = min(wcol0 + 2 * k + (lane >> 5), nsb - 1);
        sv[k] = *reinterpret_cast<const i32x4 *>(s_src + 4 * ((int64_t)s_m * nblk + 8 * b + 4 * s_h));
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- weight loads, all of them before any arithmetic (clamped rows and columns:
    // rows past N read row N-1 and are never written; columns past nsb are skipped).
    // A 64-bit scalar base for the workgroup's rows plus 32-bit offsets.
    const int64_t row_bytes = (int64_t)nsb * 144;
    const uint8_t *__restrict__ wb = w + (int64_t)row_base * row_bytes;
    // quant chunk of chunk set s: X lanes pair s (chunk 2s + q), Y lanes pair 3 - s
    const unsigned ch0 = Yh ? 4u + q : (unsigned)q, ch1 = 2u + q;
    const unsigned rr = (unsigned)(min(row_base + n, N - 1) - row_base);
    u32x4 hd[CPW], w0[CPW], w1[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const unsigned b = (unsigned)min(wcol0 + c, nsb - 1);
        const unsigned off = __umul24(rr, (unsigned)row_bytes) + b * 144u;
        hd[c] = load_weights16(wb + off);
        w0[c] = load_weights16(wb + (off + 16u + 16u * ch0));
        w1[c] = load_weights16(wb + (off + 16u + 16u * ch1));
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- LDS stores of the staged columns (this wave reads only its own columns)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        if (c >= ncols) continue;   // wave-uniform
        uint8_t *cb = lcodes + (size_t)(wcol0 + c) * cs;
        if ((lane >> 4) < M) *reinterpret_cast<i32x4 *>(cb + (lane >> 4) * kCodeRow + co) = cv0[c];
        if (M > 4 && (lane >> 4) + 4 < M)
            *reinterpret_cast<i32x4 *>(cb + ((lane >> 4) + 4) * kCodeRow + co) = cv1[c];
        if (lane == 0) *reinterpret_cast<i32x4 *>(cb + M * kCodeRow) = i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kSP; ++k) {
        const int c = 2 * k + (lane >> 5);
        if (s_live && c < ncols) {
            float *dst = (s_sum ? ls : la) + (size_t)(wcol0 + c) * 64 + 4 * s_h * 8 + s_m;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[8 * e] = s_sum ? (float)sv[k][e] : __int_as_float(sv[k][e]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();

    // Per-lane LDS offsets by instruction t: activation operand (codes of the
    // lane's operand row, or the zero slot) and the scales / sums of its output
    // rows m = 4 (q % 2) .. +3 for its sub-block.
    const int ma = n & 7;
    const bool valid = ((n < 8) == !Yh) && ma < M;
    int aoff[4], soff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int j = Yh ? 7 - t : t;
        aoff[t] = valid ? ma * kCodeRow + 32 * j + 16 * (q & 1) : M * kCodeRow;
        soff[t] = j * 8 + 4 * (q & 1);
    }
    const int sh_even = Yh ? 4 : 0, sh_odd = 4 - sh_even;   // nibble of instructions t even / odd
    const int tofs = (Yh ? 8 : 0) + 4 * (q & 1);            // half-term slot of this lane

#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        if (c >= ncols) break;   // wave-uniform
        const int b = wcol0 + c;
        const uint8_t *cb = lcodes + (size_t)b * cs;
        const float *lab = la + (size_t)b * 64;
        const float *lsb = ls + (size_t)b * 64;

        // activation operands, scales and sums of the column
        i32x4 aw[4];
        f32x4 a4[4], s4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            aw[t] = *reinterpret_cast<const i32x4 *>(cb + aoff[t]);
            a4[t] = *reinterpret_cast<const f32x4 *>(lab + soff[t]);
            s4[t] = *reinterpret_cast<const f32x4 *>(lsb + soff[t]);
        }
        {
            // the four sub-block dots of the column
            i32x4 D[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 src = (t < 2) ? w0[c] : w1[c];
                const int shv = (t & 1) ? sh_odd : sh_even;
                i32x4 bw;
#pragma unroll
                for (int k = 0; k < 4; ++k) bw[k] = (int)((src[k] >> shv) & 0x0F0F0F0Fu);
                D[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[t], bw, i32x4{0, 0, 0, 0}, 0, 0, 0);
            }

            // scales of the lane's 4 sub-blocks, byte t = sub-block t (X) or 7 - t
            // (Y: the bytes of sub-blocks 4..7 reversed)
            const u32x4 h = hd[c];
            const float d = half_lo(h.x), dmin = half_hi(h.x);
            const unsigned scX = h.y & 0x3F3F3F3Fu, mnX = h.z & 0x3F3F3F3Fu;
            const unsigned scY =
                __builtin_bswap32((h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u));
            const unsigned mnY =
                __builtin_bswap32(((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u));
            const unsigned scb = Yh ? scY : scX, mnb = Yh ? mnY : mnX;

            float f[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float ds = d * (float)((scb >> (8 * t)) & 0xFFu);
                const float dm = dmin * (float)((mnb >> (8 * t)) & 0xFFu);
#pragma unroll
                for (int r = 0; r < 4; ++r) f[t][r] = subblock_factor(ds, D[t][r], dm, s4[t][r]);
            }
            f32x4 half;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma clang fp contract(off)
                const float uA = fmaf(a4[0][r], f[0][r], a4[1][r] * f[1][r]);
                const float uB = fmaf(a4[2][r], f[2][r], a4[3][r] * f[3][r]);
                half[r] = uA + uB;
            }
            *reinterpret_cast<f32x4 *>(lterm + ((size_t)n * nsb + b) * 16 + tofs) = half;
        }
    }
    __syncthreads();

    // ---- a row adds (X + Y) per column in column order (the streaming GEMV's order)
    for (int i = threadIdx.x; i < 16 * M; i += 64 * nw) {
        const int r = i / M, m = i % M;
        const float *ts = lterm + (size_t)r * nsb * 16 + m;   // row r of the workgroup
        float t = 0.0f;
        for (int b = 0; b < nsb; ++b) {
#pragma clang fp contract(off)
            t += ts[(size_t)b * 16] + ts[(size_t)b * 16 + 8];
        }
        const int row = row_base + r;
        if (row < N) y[(int64_t)m * N + row] = t;
    }
}

// One product per launch.
template <int CPW>
__global__ __launch_bounds__(1024) void gemv_mfma_kernel(
    const uint8_t *__restrict__ w, float *__restrict__ y, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const int32_t *__restrict__ sums, int N, int nsb, int M) {
    gemv_mfma_tile<CPW>(w, y, N, (int)blockIdx.x * 16, codes, scales, sums, nsb, M);
}

// Several products per launch: the first one's arguments lead (preloaded into
// registers), the others come from the table.
template <int CPW>
__global__ __launch_bounds__(1024) void gemv_mfma_batch_kernel(
    const uint8_t *w0, float *y0, int N0, int tiles0, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const int32_t *__restrict__ sums, int nsb, int M,
    const MfmaSet set) {
    if ((int)blockIdx.x < tiles0) {                // uniform
        gemv_mfma_tile<CPW>(w0, y0, N0, (int)blockIdx.x * 16, codes, scales, sums, nsb, M);
        return;
    }
    int pi = 1;
    while (pi + 1 < set.count && (int)blockIdx.x >= set.tile0[pi + 1]) ++pi;
    gemv_mfma_tile<CPW>(set.w[pi], set.y[pi], set.N[pi], ((int)blockIdx.x - set.tile0[pi]) * 16,
                        codes, scales, sums, nsb, M);
}

template <int CPW>
hipError_t launch_cpw(const MfmaSet &set, int nsb, const int8_t *codes, const float *scales,
                      const int32_t *sums, int M, hipStream_t stream) {
    const int waves = (nsb + CPW - 1) / CPW;
    if (set.count == 1)
        hipLaunchKernelGGL((gemv_mfma_kernel<CPW>), dim3(set.tile0[1]), dim3(64 * waves),
                           mfma_lds_bytes(M, nsb), stream, set.w[0], set.y[0], codes, scales, sums,
                           set.N[0], nsb, M);
    else
        hipLaunchKernelGGL((gemv_mfma_batch_kernel<CPW>), dim3(set.tile0[set.count]), dim3(64 * waves),
                           mfma_lds_bytes(M, nsb), stream, set.w[0], set.y[0], set.N[0], set.tile0[1],
                           codes, scales, sums, nsb, M, set);
    return hipGetLastError();
}

}  // namespace

bool gemv_mfma_fits(int64_t K, int64_t M, const void *scales, const void *sums) {
    const int64_t nsb = K / kQK;
    return reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(sums) % 16 == 0 && M >= 2 && M <= 8 &&
           nsb <= 16 * kMaxCpw && mfma_lds_bytes((int)M, (int)nsb) <= (size_t)kMaxLds;
}

// Where the matrix-core GEMV beats the streaming one, measured on MI355X over
// the decode projections (N = 1024 .. 9728, K = 2560 .. 9728) for M = 2..8:
// from M = 3 on wide products; below N = 2048 a 16-row tile per workgroup
// leaves most CUs idle, and the streaming GEMV keeps up until M = 5 (N = 1024,
// M = 3: 3.45 against 3.77 us); at M = 2 the streaming GEMV's lighter vector
// work wins.
// N: the rows of the launch (all its products').
bool gemv_mfma_preferred(int64_t N, int64_t K, int64_t M, const void *scales, const void *sums) {
    if (!gemv_mfma_fits(K, M, scales, sums)) return false;
    return M >= 3 && (N >= 2048 || M >= 5);
}

hipError_t launch_gemv_mfma_batch(const GemvProblem *probs, int count, int64_t K,
                                  const int8_t *codes, const float *scales, const int32_t *sums,
                                  int64_t M, hipStream_t stream) {
    if (count < 1 || count > kMaxGemvBatch) return hipErrorInvalidValue;
    MfmaSet set = {};
    set.count = count;
    for (int p = 0; p < count; ++p) {
        set.w[p] = static_cast<const uint8_t *>(probs[p].w);
        set.y[p] = probs[p].y;
        set.N[p] = (int)probs[p].N;
        set.tile0[p + 1] = set.tile0[p] + (int)((probs[p].N + 15) / 16);
    }
    const int nsb = (int)(K / kQK);
    // columns per wave: the fewest that keep the workgroup within 8 waves, and
    // at most 3 (up to 16 waves): past 24 columns more waves issue the loads
    // sooner (2560 x 9728: 10.1 us at 13 waves against 11.3 at 8)
    const int cpw = std::min((nsb + 7) / 8, kMaxCpw);
    switch (cpw) {
    case 1: return launch_cpw<1>(set, nsb, codes, scales, sums, (int)M, stream);
    case 2: return launch_cpw<2>(set, nsb, codes, scales, sums, (int)M, stream);
    case 3: return launch_cpw<3>(set, nsb, codes, scales, sums, (int)M, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_mfma(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                            const float *scales, const int32_t *sums, int64_t M, float *y,
                            hipStream_t stream) {
    const GemvProblem p = {w, nullptr, y, N};
    return launch_gemv_mfma_batch(&p, 1, K, codes, scales, sums, M, stream);
}

}  // namespace q4k
