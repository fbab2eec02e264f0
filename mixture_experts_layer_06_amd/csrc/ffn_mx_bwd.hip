// Backward of the MXFP8 expert computation ("Scalable Training of
// Mixture-of-Experts Models with Megatron Core": section 5.1 runs the expert
// GEMMs in low precision and keeps the router in FP32; section 5.3.3 gives
// MXFP8 as 1 x 32 blocks with E8M0 scales; section 5.4 aligns dimensions to
// 32 by padding the routing map). Every GEMM takes both operands in MXFP8,
// blocked along its own reduction axis:
//   gu   = Q_h(X) Q_h(W1)           the first projection recomputed in fp32
//                                    from the forward's codes (selective
//                                    recomputation: nothing but the routing
//                                    is kept from the forward), act = silu(g) u
//   dY   = row weight * dL/dout     fp32, built inside the quantisers
//   dact = Q_h(dY) Q_h(W2)          input gradient of the second projection
//   dgu  = SwiGLU backward           fp32, at the recomputed g and u
//   dX   = Q_2F(dgu) Q_2F(W1)       input gradient of the first projection
//   dW2  = Q_tok(dY)^T Q_tok(act)   weight gradients: reductions over each
//   dW1  = Q_tok(dgu)^T Q_tok(X)    expert's tokens, blocked from its first row
// Every quantised operand is thus formed from fp32 values as exact as the
// forward's (MXFP8's block rounding turns a bf16 rounding of its inputs
// into flipped E4M3 roundings). W2 and W1 blocked along h and 2F are the
// transposed codes of
// moe_mx_quantize_t ([E][F][h] and [E][h][2F]). Token-blocked operands are
// stored transposed, [N][Pc]: each expert's segment starts at a padded
// column poffs[e] and is completed with zero columns to a multiple of 128
// (one k-step), so a k-step never mixes two experts and the padding adds
// nothing; the blocks of 32 start at the segment's first token. act and dgu
// exist only inside the passes that quantise them (fp32 in LDS): act along
// the tokens, dgu along 2F and along the tokens.
//
// The five products run on the forward's MXFP8 grouped GEMM (mx_gemm_rows:
// 256 x 256 tiles of v_mfma_scale_f32_32x32x64_f8f6f4, one persistent block
// per compute unit, k-step t + 1 written to LDS while k-step t is multiplied
// and t + 2 is loaded): the recomputation and the input gradients by token
// segments, the weight gradients by each expert's k-range of the transposed
// operands (mx_gemm_kseg), all with fp32 accumulation.
#include <type_traits>

#include "mx_common.hpp"

namespace moe {
namespace {

// poffs[e] = sum over e' < e of count_e' rounded up to 128 (one block of
// 256 threads, E <= 256).
__global__ __launch_bounds__(256) void mx_pad_offsets_kernel(const int32_t *__restrict__ offs, int E,
                                                             int32_t *__restrict__ poffs) {
    __shared__ int s[256];
    const int t = threadIdx.x;
    const int v = t < E ? ((offs[t + 1] - offs[t] + 127) / 128) * 128 : 0;
    s[t] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int add = t >= d ? s[t - d] : 0;
        __syncthreads();
        s[t] += add;
        __syncthreads();
    }
    if (t == 0) poffs[0] = 0;
    if (t < E) poffs[t + 1] = s[t];
}

// Blocks of 32 consecutive rows of one column to transposed codes, one
// thread per (column n, block). Segments: source rows r0_s + i (through
// `gather` when given), i < n_s, either the token segments (offs; block
// starts at padded column poffs[s] + 32 b of codes row n, stride ld) or
// uniform segments of seg_rows rows (offs null; segment s is the matrix
// [N][ld] at s * N * ld codes, its block b at column 32 b of row n). Rows past
// n_s, up to the segment's padded end, are zeros. Block index pb: padded
// column / 32 over all segments. With token segments, the last 128 columns
// of each codes row (from ld - 128) get zero codes and zero scale bytes: a
// k-step of zeros for the weight gradients. With row_w, segment row r's
// values are multiplied by row_w[r] (in fp32) before quantising.
template <typename TE>
__global__ __launch_bounds__(256) void mx_quantize_cols_kernel(const TE *__restrict__ src, int64_t src_ld,
                                                               const int32_t *__restrict__ gather,
                                                               const float *__restrict__ row_w,
                                                               const int32_t *__restrict__ offs,
                                                               const int32_t *__restrict__ poffs, int nseg,
                                                               int seg_rows, int N, int64_t ld,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
    const int pb = blockIdx.x;
    const int n = blockIdx.y * blockDim.x + threadIdx.x;
    int s, local, nrows, r0;
    int64_t cbase;   // codes offset of the block's first element in row n = 0
    if (offs) {
        const int p = 32 * pb;
        cbase = p;
        if (p >= poffs[nseg]) {
            if (p < ld - 128) return;
            s = local = r0 = nrows = 0;   // the zero k-step
        } else {
            int lo = 0, hi = nseg - 1;   // largest s with poffs[s] <= p
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (poffs[mid] <= p) lo = mid;
                else hi = mid - 1;
            }
            s = lo;
            local = p - poffs[s];
            r0 = offs[s];
            nrows = offs[s + 1] - r0;
        }
    } else {
        const int per = seg_rows / 32;
        s = pb / per;
        local = 32 * (pb - s * per);
        r0 = s * seg_rows;
        nrows = seg_rows;
        cbase = static_cast<int64_t>(s) * N * ld + local;   // segment s: the matrix [N][ld] at s N ld
    }
    if (n >= N) return;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int li = local + i;
        float x = 0.0f;
        if (li < nrows) {
            const int64_t r = gather ? gather[r0 + li] : r0 + li;
            x = Elem<TE>::load(src, r * src_ld + n);
            if (row_w) x *= row_w[r0 + li];
        }
        v[i] = x;
        amax = fmaxf(amax, fabsf(x));
    }
    const int ex = mx_block_exponent(amax);
    u32x4 out[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t word = e4m3_word(ldexpf(v[4 * w], -ex), ldexpf(v[4 * w + 1], -ex),
                                        ldexpf(v[4 * w + 2], -ex), ldexpf(v[4 * w + 3], -ex));
        out[w >> 2][w & 3] = word;
    }
    const int64_t ce = cbase + static_cast<int64_t>(n) * ld;
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + ce);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[ce / 32] = static_cast<uint8_t>(ex + 127);
}

// The same quantisation by tiles of 128 rows x 64 columns: the block reads
// the tile's (gathered) rows with 16-byte loads along the columns into LDS
// (bf16 sources as bf16, with the tile's row weights beside them; fp32
// sources weighted as fp32), then wave w quantises the tile's 32-row block w
// with one lane per column, so that each column's codes of the tile (128
// bytes) and its four scale bytes are written by one block. Consecutive
// blocks take consecutive column groups of one row tile, so that the blocks
// running together read whole source rows. Needs N % 64 == 0, a 16-byte
// aligned source with 16-byte aligned rows, and tiles that do not straddle
// segments: token segments padded to 128 rows (poffs), or uniform segments
// (tile t of segment s covers its rows 128 t.., the 32-row blocks past
// seg_rows are skipped).
constexpr int kQtRows = 128, kQtCols = 64;
template <typename TE>
__global__ __launch_bounds__(256) void mx_quantize_cols_tile_kernel(const TE *__restrict__ src, int64_t src_ld,
                                                                    const int32_t *__restrict__ gather,
                                                                    const float *__restrict__ row_w,
                                                                    const int32_t *__restrict__ offs,
                                                                    const int32_t *__restrict__ poffs, int nseg,
                                                                    int seg_rows, int N, int64_t ld,
                                                                    uint8_t *__restrict__ codes,
                                                                    uint8_t *__restrict__ scales) {
    constexpr bool kHalf = sizeof(TE) == 2;
    constexpr int kVec = 16 / static_cast<int>(sizeof(TE));   // elements per 16-byte load
    constexpr int kLpr = kQtCols / kVec;                      // lanes per tile row
    constexpr int kRpp = 256 / kLpr;                          // rows per pass
    constexpr int kPasses = kQtRows / kRpp;
    constexpr int kLd = kQtCols + kVec;                       // LDS row stride (elements), 16 bytes of padding
    typedef typename std::conditional<kHalf, bf16_t, float>::type TL;
    __shared__ __attribute__((aligned(16))) TL T[kQtRows * kLd];
    __shared__ float s_w[kQtRows];
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * kQtCols, tb = blockIdx.y;
    int local, nrows, r0, nblk;
    int64_t cbase;
    if (offs) {
        const int p = kQtRows * tb;
        cbase = p;
        nblk = 4;
        if (p >= poffs[nseg]) {
            if (p != ld - kQtRows) return;
            local = r0 = nrows = 0;   // the zero k-step
        } else {
            int lo = 0, hi = nseg - 1;   // largest s with poffs[s] <= p
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (poffs[mid] <= p) lo = mid;
                else hi = mid - 1;
            }
            local = p - poffs[lo];
            r0 = offs[lo];
            nrows = offs[lo + 1] - r0;
        }
    } else {
        const int tps = (seg_rows + kQtRows - 1) / kQtRows;
        const int sg = tb / tps;
        local = kQtRows * (tb - sg * tps);
        r0 = sg * seg_rows;
        nrows = seg_rows;
        cbase = static_cast<int64_t>(sg) * N * ld + local;   // segment s: [N][ld] at s N ld
        nblk = min(4, (seg_rows - local) / 32);
    }
    const int c = tid % kLpr, rr0 = tid / kLpr;
    u32x4 q[kPasses];
    float wrow[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
        const int li = local + rr0 + kRpp * i;
        q[i] = u32x4{0u, 0u, 0u, 0u};
        wrow[i] = 1.0f;
        if (li < nrows) {
            const int64_t r = gather ? gather[r0 + li] : r0 + li;
            q[i] = *reinterpret_cast<const u32x4 *>(src + r * src_ld + n0 + kVec * c);
            if (row_w) wrow[i] = row_w[r0 + li];
        }
    }
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
        TL *dst = T + (rr0 + kRpp * i) * kLd + kVec * c;
        if constexpr (kHalf) {
            *reinterpret_cast<u32x4 *>(dst) = q[i];
            if (c == 0) s_w[rr0 + kRpp * i] = wrow[i];
        } else {
            *reinterpret_cast<float4 *>(dst) =
                make_float4(__uint_as_float(q[i][0]) * wrow[i], __uint_as_float(q[i][1]) * wrow[i],
                            __uint_as_float(q[i][2]) * wrow[i], __uint_as_float(q[i][3]) * wrow[i]);
        }
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63;
    if (w >= nblk) return;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if constexpr (kHalf)
            v[i] = bf16_to_f32(T[(32 * w + i) * kLd + lane]) * s_w[32 * w + i];
        else
            v[i] = T[(32 * w + i) * kLd + lane];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const int ex = mx_block_exponent(amax);
    u32x4 out[2];
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
        const uint32_t word = e4m3_word(ldexpf(v[4 * wd], -ex), ldexpf(v[4 * wd + 1], -ex),
                                        ldexpf(v[4 * wd + 2], -ex), ldexpf(v[4 * wd + 3], -ex));
        out[wd >> 2][wd & 3] = word;
    }
    const int64_t ce = cbase + static_cast<int64_t>(n0 + lane) * ld + 32 * w;
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + ce);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[ce / 32] = static_cast<uint8_t>(ex + 127);
}

// The padded token rows of column-quantisation tile tb (positions 128 tb ..):
// segment rows r0 + local + i for local + i < nrows; for the zero k-step at
// columns ld - 128, no rows. False for a tile past the segments otherwise.
__device__ __forceinline__ bool qt_tile(const int32_t *__restrict__ offs, const int32_t *__restrict__ poffs, int nseg,
                                        int64_t ld, int tb, int &local, int &r0, int &nrows) {
    const int p = kQtRows * tb;
    if (p >= poffs[nseg]) {
        if (p != ld - kQtRows) return false;
        local = r0 = nrows = 0;
        return true;
    }
    int lo = 0, hi = nseg - 1;   // largest s with poffs[s] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (poffs[mid] <= p) lo = mid;
        else hi = mid - 1;
    }
    local = p - poffs[lo];
    r0 = offs[lo];
    nrows = offs[lo + 1] - r0;
    return true;
}

// One 32-block of fp32 values v (amax their largest magnitude) to 32 codes
// at codes[ce..] and its scale byte at scales[ce / 32].
__device__ __forceinline__ void mx_store_block(const float (&v)[32], float amax, uint8_t *__restrict__ codes,
                                               uint8_t *__restrict__ scales, int64_t ce) {
    const int ex = mx_block_exponent(amax);
    u32x4 out[2];
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
        const uint32_t word = e4m3_word(ldexpf(v[4 * wd], -ex), ldexpf(v[4 * wd + 1], -ex),
                                        ldexpf(v[4 * wd + 2], -ex), ldexpf(v[4 * wd + 3], -ex));
        out[wd >> 2][wd & 3] = word;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + ce);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[ce / 32] = static_cast<uint8_t>(ex + 127);
}

// Rows 32 w .. 32 w + 31 of column c of an fp32 LDS tile (row stride tld)
// as one block along the tokens.
__device__ __forceinline__ void qt_col_block(const float *T, int tld, int c, int w, uint8_t *__restrict__ codes,
                                             uint8_t *__restrict__ scales, int64_t ce) {
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] = T[(32 * w + i) * tld + c];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    mx_store_block(v, amax, codes, scales, ce);
}

// The activation act = silu(g) u of the recomputed pre-activations (g | u)
// [P][2F] (fp32, the expression of the forward's epilogue), quantised along
// the tokens straight away: tiles of 128 padded token rows x 64 columns of
// F as in mx_quantize_cols_tile_kernel (codes [F][ld], zero padding rows
// and zero k-step included), so act itself is never stored.
__global__ __launch_bounds__(256) void mx_act_cols_kernel(const float *__restrict__ gu, int F,
                                                          const int32_t *__restrict__ offs,
                                                          const int32_t *__restrict__ poffs, int nseg, int64_t ld,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    constexpr int kLd = kQtCols + 4;
    __shared__ __attribute__((aligned(16))) float T[kQtRows * kLd];
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * kQtCols, tb = blockIdx.y;
    int local, r0, nrows;
    if (!qt_tile(offs, poffs, nseg, ld, tb, local, r0, nrows)) return;
    const int c = tid & 15, rr0 = tid >> 4;   // 16 lanes of 4 columns per row, 16 rows per pass
#pragma unroll
    for (int i = 0; i < kQtRows / 16; ++i) {
        const int li = local + rr0 + 16 * i;
        float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (li < nrows) {
            const float *row = gu + static_cast<int64_t>(r0 + li) * 2 * F;
            const float4 g = *reinterpret_cast<const float4 *>(row + n0 + 4 * c);
            const float4 u = *reinterpret_cast<const float4 *>(row + F + n0 + 4 * c);
            a = make_float4(g.x / (1.0f + expf(-g.x)) * u.x, g.y / (1.0f + expf(-g.y)) * u.y,
                            g.z / (1.0f + expf(-g.z)) * u.z, g.w / (1.0f + expf(-g.w)) * u.w);
        }
        *reinterpret_cast<float4 *>(T + (rr0 + 16 * i) * kLd + 4 * c) = a;
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63;
    qt_col_block(T, kLd, lane, w, codes, scales, kQtRows * static_cast<int64_t>(tb) + (n0 + lane) * ld + 32 * w);
}

// The SwiGLU backward at the recomputed (g | u), fp32 (dg = dact u s (1 + g
// (1 - s)), du = dact g s, s = sigmoid(g), the expressions of the unfused
// pass), quantised at once both ways: along 2F into row codes [P][2F] (for
// the input gradient) and along the tokens into codes [2F][ld] (for the
// first weight gradient). Tiles of 128 padded token rows x 32 columns of F
// (kDguCols): the tile's 32 dg and 32 du columns in LDS (35 KB, four blocks
// per compute unit), then each valid row's two 32-column blocks and each
// column's four 32-row blocks; dgu itself is never stored.
constexpr int kDguCols = 32;
__global__ __launch_bounds__(256) void mx_dgu_quant_kernel(const float *__restrict__ dact,
                                                           const float *__restrict__ gu, int F,
                                                           const int32_t *__restrict__ offs,
                                                           const int32_t *__restrict__ poffs, int nseg, int64_t ld,
                                                           uint8_t *__restrict__ row_codes,
                                                           uint8_t *__restrict__ row_scales,
                                                           uint8_t *__restrict__ tok_codes,
                                                           uint8_t *__restrict__ tok_scales) {
    constexpr int kLd = 2 * kDguCols + 4;
    __shared__ __attribute__((aligned(16))) float T[kQtRows * kLd];
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * kDguCols, tb = blockIdx.y;
    int local, r0, nrows;
    if (!qt_tile(offs, poffs, nseg, ld, tb, local, r0, nrows)) return;
    const int c = tid & 7, rr0 = tid >> 3;   // 8 lanes of 4 columns per row, 32 rows per pass
#pragma unroll
    for (int i = 0; i < kQtRows / 32; ++i) {
        const int li = local + rr0 + 32 * i;
        float dg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, du[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (li < nrows) {
            const int64_t p = r0 + li;
            const float4 d4 = *reinterpret_cast<const float4 *>(dact + p * F + n0 + 4 * c);
            const float4 g4 = *reinterpret_cast<const float4 *>(gu + p * 2 * F + n0 + 4 * c);
            const float4 u4 = *reinterpret_cast<const float4 *>(gu + p * 2 * F + F + n0 + 4 * c);
            const float da[4] = {d4.x, d4.y, d4.z, d4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w},
                        uv[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float sg = 1.0f / (1.0f + expf(-gv[q]));
                dg[q] = da[q] * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
                du[q] = da[q] * gv[q] * sg;
            }
        }
        float *trow = T + (rr0 + 32 * i) * kLd + 4 * c;
        *reinterpret_cast<float4 *>(trow) = make_float4(dg[0], dg[1], dg[2], dg[3]);
        *reinterpret_cast<float4 *>(trow + kDguCols) = make_float4(du[0], du[1], du[2], du[3]);
    }
    __syncthreads();
    // along 2F: row i, block b (0: the dg columns n0 .., 1: the du columns F + n0 ..)
    {
        const int i = tid >> 1, b = tid & 1;
        if (local + i < nrows) {
            float v[32];
            float amax = 0.0f;
            const float *src = T + i * kLd + kDguCols * b;
#pragma unroll
            for (int k = 0; k < 32; k += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(src + k);
                v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
            }
#pragma unroll
            for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
            mx_store_block(v, amax, row_codes, row_scales,
                           static_cast<int64_t>(r0 + local + i) * 2 * F + (b ? F + n0 : n0));
        }
    }
    // along the tokens: wave w takes the 32-row block w of the tile's 64 columns
    const int w = tid >> 6, lane = tid & 63;
    const int gcol = lane < kDguCols ? n0 + lane : F + n0 + lane - kDguCols;
    qt_col_block(T, kLd, lane, w, tok_codes, tok_scales,
                 kQtRows * static_cast<int64_t>(tb) + static_cast<int64_t>(gcol) * ld + 32 * w);
}

// Rows of 32-blocks along K of a gathered, row-weighted source: row p of
// the result is row_w[p] * src[gather[p]] (fp32), quantised by the same
// rule as mx_quantize_kernel; one thread per block.
template <typename TE>
__global__ __launch_bounds__(256) void mx_quantize_rows_gather_kernel(const TE *__restrict__ src,
                                                                      const int32_t *__restrict__ gather,
                                                                      const float *__restrict__ row_w, int64_t nrows,
                                                                      int K, uint8_t *__restrict__ codes,
                                                                      uint8_t *__restrict__ scales) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int kb = K / 32;
    if (b >= nrows * kb) return;
    const int64_t p = b / kb;
    const int c0 = static_cast<int>(b - p * kb) * 32;
    const float w = row_w[p];
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) load8(src + static_cast<int64_t>(gather[p]) * K + c0 + 8 * c, v + 8 * c);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] *= w;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const int ex = mx_block_exponent(amax);
    u32x4 out[2];
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
        const uint32_t word = e4m3_word(ldexpf(v[4 * wd], -ex), ldexpf(v[4 * wd + 1], -ex),
                                        ldexpf(v[4 * wd + 2], -ex), ldexpf(v[4 * wd + 3], -ex));
        out[wd >> 2][wd & 3] = word;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[b] = static_cast<uint8_t>(ex + 127);
}

template <typename TE>
void launch_quantize_cols(const TE *src, int64_t src_ld, const int32_t *gather, const float *row_w,
                          const int32_t *offs, const int32_t *poffs, int nseg, int seg_rows, int64_t padded_rows,
                          int N, int64_t ld, uint8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t nb = padded_rows / 32;
    if (nb == 0 || N == 0) return;
    constexpr int kVec = 16 / static_cast<int>(sizeof(TE));
    const int64_t tiles = offs ? padded_rows / kQtRows
                               : static_cast<int64_t>(nseg) * ((seg_rows + kQtRows - 1) / kQtRows);
    if (N % kQtCols == 0 && aligned16(src) && src_ld % kVec == 0 && tiles <= 65535) {
        hipLaunchKernelGGL(mx_quantize_cols_tile_kernel<TE>,
                           dim3(static_cast<unsigned>(N / kQtCols), static_cast<unsigned>(tiles)), dim3(256), 0, s,
                           src, src_ld, gather, row_w, offs, poffs, nseg, seg_rows, N, ld, codes, scales);
        return;
    }
    hipLaunchKernelGGL(mx_quantize_cols_kernel<TE>, dim3(static_cast<unsigned>(nb), static_cast<unsigned>((N + 255) / 256)),
                       dim3(256), 0, s, src, src_ld, gather, row_w, offs, poffs, nseg, seg_rows, N, ld, codes,
                       scales);
}


// Workspace of the backward: sub-buffers at 256-byte boundaries.
struct MxBwdLayout {
    int64_t Pc;   // padded token columns of the token-blocked (transposed) operands
    int64_t ldT;  // their row stride: Pc and a last k-step of zeros (the weight gradients' zero step)
    size_t poffs, gu, dy_c, dy_s, dyT_c, dyT_s, actT_c, actT_s, dact, dgu_c, dgu_s, dguT_c, dguT_s, xT_c,
        xT_s;
    size_t total;
};

MxBwdLayout mx_bwd_layout(int64_t P, int64_t h, int64_t F, int E) {
    MxBwdLayout L{};
    L.Pc = ((P + 127 * static_cast<int64_t>(E)) + 127) / 128 * 128;
    L.ldT = L.Pc + 128;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at += (bytes + 255) & ~static_cast<size_t>(255);
        return o;
    };
    const size_t Pz = static_cast<size_t>(P), hz = static_cast<size_t>(h), Fz = static_cast<size_t>(F),
                 Pcz = static_cast<size_t>(L.ldT);
    L.poffs = take(static_cast<size_t>(E + 1) * 4);
    L.gu = take(Pz * 2 * Fz * 4);
    L.dy_c = take(Pz * hz);
    L.dy_s = take(Pz * hz / 32);
    L.dyT_c = take(hz * Pcz);
    L.dyT_s = take(hz * Pcz / 32);
    L.actT_c = take(Fz * Pcz);
    L.actT_s = take(Fz * Pcz / 32);
    L.dact = take(Pz * Fz * 4);
    L.dgu_c = take(Pz * 2 * Fz);
    L.dgu_s = take(Pz * 2 * Fz / 32);
    L.dguT_c = take(2 * Fz * Pcz);
    L.dguT_s = take(2 * Fz * Pcz / 32);
    L.xT_c = take(hz * Pcz);
    L.xT_s = take(hz * Pcz / 32);
    L.total = at;
    return L;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_mx_quantize_t(const void *src, int dtype, int64_t batch, int64_t R, int64_t C, uint8_t *codes,
                                 uint8_t *scales, void *stream) {
    clear_error();
    MOE_CHECK_ARG(batch >= 0 && R > 0 && C > 0, MOE_ERR_INVALID_ARG, "moe_mx_quantize_t: bad sizes");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_mx_quantize_t: bad dtype %d", dtype);
    MOE_CHECK_ARG(batch == 0 || (src && codes && scales), MOE_ERR_INVALID_ARG, "moe_mx_quantize_t: null pointer");
    MOE_CHECK_ARG(R % 32 == 0 && R < (int64_t(1) << 30) && C < (int64_t(1) << 30) &&
                      batch * (R / 32) < (int64_t(1) << 31) && (C + 255) / 256 <= 65535,
                  MOE_ERR_UNSUPPORTED, "moe_mx_quantize_t: need R %% 32 == 0 and sizes below the launch limits");
    MOE_CHECK_ARG(batch == 0 || (aligned16(codes) && (R % 16 == 0)), MOE_ERR_INVALID_ARG,
                  "moe_mx_quantize_t: codes must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    const int64_t rows = batch * R;
    if (dtype == MOE_DTYPE_BF16)
        launch_quantize_cols(static_cast<const bf16_t *>(src), C, nullptr, nullptr, nullptr, nullptr,
                             static_cast<int>(batch), static_cast<int>(R), rows, static_cast<int>(C), R, codes, scales,
                             s);
    else
        launch_quantize_cols(static_cast<const float *>(src), C, nullptr, nullptr, nullptr, nullptr,
                             static_cast<int>(batch), static_cast<int>(R), rows, static_cast<int>(C), R, codes, scales,
                             s);
    return check_launch("moe_mx_quantize_t");
}

extern "C" size_t moe_grouped_ffn_bwd_mx_workspace_size(int64_t P, int64_t h, int64_t F, int E) {
    if (P < 0 || h <= 0 || F <= 0 || E <= 0) return 0;
    return mx_bwd_layout(P, h, F, E).total;
}

extern "C" int moe_grouped_ffn_bwd_mx(const void *grad_out, const float *row_w, const void *x, const uint8_t *x_codes,
                                      const uint8_t *x_scales, const int32_t *sorted_token, int64_t T, int64_t P,
                                      int64_t h, int64_t F, int E, const int32_t *offsets, int act_kind,
                                      const uint8_t *w1_codes, const uint8_t *w1_scales, const uint8_t *w1t_codes,
                                      const uint8_t *w1t_scales, const uint8_t *w2t_codes,
                                      const uint8_t *w2t_scales, void *grad_x_perm, float *grad_w1, float *grad_w2,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(offsets && w1_codes && w1_scales && w1t_codes && w1t_scales && w2t_codes && w2t_scales &&
                      grad_w1 && grad_w2 &&
                      (P == 0 || (grad_out && row_w && x && x_codes && x_scales && sorted_token && grad_x_perm)),
                  MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_mx: null required pointer");
    MOE_CHECK_ARG(P >= 0 && T >= 0 && h > 0 && F > 0 && E > 0 && (P == 0 || T > 0), MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_bwd_mx: bad sizes");
    MOE_CHECK_ARG(act_kind == MOE_ACT_SWIGLU, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_bwd_mx: SwiGLU experts only");
    MOE_CHECK_ARG(h % 128 == 0 && F % 128 == 0 && E <= 256, MOE_ERR_UNSUPPORTED,
                  "moe_grouped_ffn_bwd_mx: need h %% 128 == 0, F %% 128 == 0, E <= 256");
    const MxBwdLayout L = mx_bwd_layout(P, h, F, E);
    MOE_CHECK_ARG(P < (int64_t(1) << 31) && T * h < (int64_t(1) << 31) && P * h < (int64_t(1) << 31) &&
                      2 * P * F < (int64_t(1) << 31) && 2 * F * h < (int64_t(1) << 31) && L.ldT / 128 <= 65535,
                  MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_bwd_mx: sizes too large");
    MOE_CHECK_ARG(workspace && workspace_bytes >= L.total, MOE_ERR_WORKSPACE,
                  "moe_grouped_ffn_bwd_mx: needs moe_grouped_ffn_bwd_mx_workspace_size bytes of workspace");
    const void *ptrs[] = {grad_out, x, x_codes, w1_codes, w1t_codes, w2t_codes, grad_x_perm, grad_w1, grad_w2,
                          workspace};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(p == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn_bwd_mx: tensor, code and workspace pointers must be 16-byte aligned");
    const void *sp[] = {x_scales, w1_scales, w1t_scales, w2t_scales};
    for (const void *p : sp)
        MOE_CHECK_ARG((reinterpret_cast<uintptr_t>(p) & 3u) == 0, MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn_bwd_mx: scale pointers must be 4-byte aligned");
    hipStream_t s = as_stream(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *poffs = reinterpret_cast<int32_t *>(ws + L.poffs);
    const bf16_t *G = static_cast<const bf16_t *>(grad_out);
    const int hh = static_cast<int>(h), FF = static_cast<int>(F);
    float *gu = reinterpret_cast<float *>(ws + L.gu);

    hipLaunchKernelGGL(mx_pad_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, E, poffs);
    if (P > 0) {
        // gu = Q_h(X) Q_h(W1) in fp32 (the forward's codes); act = silu(g) u
        // quantised along the tokens as it is formed
        int st = mx_gemm_rows(x_codes, x_scales, sorted_token, static_cast<int>(T), offsets, E, P, w1_codes,
                              w1_scales, 2 * FF, hh, gu, true, s, "moe_grouped_ffn_bwd_mx recompute");
        if (st != MOE_OK) return st;
        const dim3 qt_grid(static_cast<unsigned>(F / kQtCols), static_cast<unsigned>(L.ldT / kQtRows));
        hipLaunchKernelGGL(mx_act_cols_kernel, qt_grid, dim3(256), 0, s, static_cast<const float *>(gu), FF, offsets,
                           poffs, E, L.ldT, ws + L.actT_c, ws + L.actT_s);
        // dY = row_w * dL/dout along h (rows) and along the tokens; the
        // token rows along the tokens
        hipLaunchKernelGGL(mx_quantize_rows_gather_kernel<bf16_t>, dim3(static_cast<unsigned>((P * (h / 32) + 255) / 256)),
                           dim3(256), 0, s, G, sorted_token, row_w, P, hh, ws + L.dy_c, ws + L.dy_s);
        launch_quantize_cols(G, h, sorted_token, row_w, offsets, poffs, E, 0, L.ldT, hh, L.ldT, ws + L.dyT_c,
                             ws + L.dyT_s, s);
        launch_quantize_cols(static_cast<const bf16_t *>(x), h, sorted_token, nullptr, offsets, poffs, E, 0, L.ldT, hh,
                             L.ldT, ws + L.xT_c, ws + L.xT_s, s);
        // dact = Q_h(dY) Q_h(W2)
        st = mx_gemm_rows(ws + L.dy_c, ws + L.dy_s, nullptr, 0, offsets, E, P, w2t_codes, w2t_scales, FF, hh,
                          ws + L.dact, true, s, "moe_grouped_ffn_bwd_mx dact");
        if (st != MOE_OK) return st;
        // dgu quantised along 2F (rows) and along the tokens as it is formed
        hipLaunchKernelGGL(mx_dgu_quant_kernel, dim3(static_cast<unsigned>(F / kDguCols), qt_grid.y), dim3(256), 0, s,
                           reinterpret_cast<const float *>(ws + L.dact),
                           static_cast<const float *>(gu), FF, offsets, poffs, E, L.ldT, ws + L.dgu_c, ws + L.dgu_s,
                           ws + L.dguT_c, ws + L.dguT_s);
        // dX = Q_2F(dgu) Q_2F(W1)
        st = mx_gemm_rows(ws + L.dgu_c, ws + L.dgu_s, nullptr, 0, offsets, E, P, w1t_codes, w1t_scales, hh,
                          2 * FF, grad_x_perm, false, s, "moe_grouped_ffn_bwd_mx dX");
        if (st != MOE_OK) return st;
    }
    // dW2 = Q_tok(dY)^T Q_tok(act), dW1 = Q_tok(dgu)^T Q_tok(X): every
    // expert's tiles run (zeros when it has no tokens)
    const int st2 = mx_gemm_kseg(ws + L.dyT_c, ws + L.dyT_s, hh, ws + L.actT_c, ws + L.actT_s, FF, L.ldT, poffs, E,
                                 grad_w2, s, "moe_grouped_ffn_bwd_mx dW2");
    if (st2 != MOE_OK) return st2;
    const int st1 = mx_gemm_kseg(ws + L.dguT_c, ws + L.dguT_s, 2 * FF, ws + L.xT_c, ws + L.xT_s, hh, L.ldT, poffs, E,
                                 grad_w1, s, "moe_grouped_ffn_bwd_mx dW1");
    if (st1 != MOE_OK) return st1;
    return check_launch("moe_grouped_ffn_bwd_mx");
}
