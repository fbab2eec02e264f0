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
// nothing; the blocks of 32 start at the segment's first token.
//
// mx_gemm_nt: C[m][n] = sum_k A[m][k] B[n][k] on E4M3 codes with one E8M0
// scale per 32 values of k. Tiles of 128 x 128 (m x n); four waves of 64 x
// 64 (2 x 2 v_mfma_scale_f32_32x32x64_f8f6f4 per k-sub of 64); k-steps of
// 128 bytes staged global -> VGPR -> LDS in two stages, one barrier per
// k-step, the next k-step loaded while the current one is multiplied. The
// n side is the instruction's A operand, so a lane's four consecutive
// accumulators are four consecutive n of one m (one 16-byte store). Operand
// layout of the instruction and the LDS swizzle as in the forward kernel:
// lane half g supplies chunks 4s + g and 4s + 2 + g of k-sub s and the scale
// of block 2s + g (its row's scale word shifted right by 8 g, opsel 2s).
//  - rows mode (recomputation, input gradients): A is the token rows [P][K]
//    cut into the experts' segments (offsets), or with a_gather the rows
//    a_gather[r] of an unpermuted [T][K]; B is expert g's matrix [N][K];
//    C [P][N].
//  - k-segment mode (weight gradients): A [M][Pc] and B [N][Pc] are shared;
//    expert g reduces over its columns [poffs[g], poffs[g+1]); C is expert
//    g's [M][N], all zeros for an expert without tokens.
#include <type_traits>

#include "mx_common.hpp"

namespace moe {
namespace {

constexpr int kNtT = 128;                     // tile rows, m and n
constexpr int kNtK = 128;                     // bytes (fp8 values) of a row per k-step
constexpr int kNtRegion = kNtT * kNtK;        // one operand tile of a stage
constexpr int kNtStage = 2 * kNtRegion + 2 * kNtT * 4;   // + a scale word per row of each side

struct MxNtArgs {
    const uint8_t *A, *As;   // m side: codes [.][lda], scales [.][lda/32]
    const uint8_t *B, *Bs;   // n side
    void *C;
    const int32_t *offs;     // rows mode: segment offsets [E+1]; k-segment mode: padded offsets [E+1]
    const int32_t *a_gather; // rows mode: A row of segment row r is a_gather[r] (or null: r)
    int E, M, N, K;          // M: k-segment mode only; K: rows mode only
    int64_t lda, ldb;        // row strides of the codes (bytes)
    int64_t b_stride;        // rows mode: bytes between the experts' B matrices
    int n_tiles, m_tiles;
};

__device__ __forceinline__ v8i nt_frag(const uint8_t *R, int row, int sub, int lhi) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(R + mswz(row, 4 * sub + lhi));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(R + mswz(row, 4 * sub + 2 + lhi));
    v8i f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
}

// The four scaled MFMAs of k-sub S of the stage at LB.
template <int S>
__device__ __forceinline__ void nt_ksub(floatx16 (&acc)[2][2], const uint8_t *LB, int rn, int rm, int lhi,
                                        const uint32_t (&SA)[2], const uint32_t (&SB)[2]) {
    v8i fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = nt_frag(LB, rn + 32 * i, S, lhi);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = nt_frag(LB + kNtRegion, rm + 32 * j, S, lhi);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 2 * S, SA[i],
                                                                        2 * S, SB[j]);
}

template <bool KSEG, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void mx_gemm_nt(MxNtArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t LS[2][kNtStage];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wn = wave & 1, wm = wave >> 1;
    int g, mrows, n0, k0, nk;
    int64_t m0;   // first A row of the tile
    const uint8_t *Bg = a.B, *Bsg = a.Bs;
    if constexpr (KSEG) {
        const int per = a.m_tiles * a.n_tiles;
        g = static_cast<int>(blockIdx.x) / per;
        const int r = static_cast<int>(blockIdx.x) - g * per;
        const int mt = r / a.n_tiles, nt = r - mt * a.n_tiles;
        m0 = static_cast<int64_t>(mt) * kNtT;
        mrows = min(kNtT, a.M - mt * kNtT);
        n0 = nt * kNtT;
        const int p0 = a.offs[g], p1 = a.offs[g + 1];
        k0 = p0 / kNtK;
        nk = (p1 - p0) / kNtK;
    } else {
        GGArgs gg{};
        gg.offsets = a.offs;
        gg.E = a.E;
        gg.n_tiles = a.n_tiles;
        const int total = build_tile_prefix(gg, kNtT, s_cum, s_tmp);
        if (static_cast<int>(blockIdx.x) >= total) return;   // the whole block
        const TileInfo ti = decode_tile(gg, s_cum, blockIdx.x, kNtT);
        g = ti.seg;
        m0 = static_cast<int64_t>(ti.row0) + ti.m0;
        mrows = min(kNtT, ti.M - ti.m0);
        n0 = ti.n_tile * kNtT;
        k0 = 0;
        nk = a.K / kNtK;
        Bg = a.B + static_cast<int64_t>(g) * a.b_stride;
        Bsg = a.Bs + static_cast<int64_t>(g) * (a.b_stride / 32);
    }
    g = __builtin_amdgcn_readfirstlane(g);
    nk = __builtin_amdgcn_readfirstlane(nk);
    k0 = __builtin_amdgcn_readfirstlane(k0);

    // rows this thread stages: chunk c of rows rb + 32 j (clamped to valid
    // rows; rows past them are computed and never stored), and one scale
    // word: the n-side row tid (tid < 128) or the m-side row tid - 128
    const int c = tid & 7, rb = tid >> 3;
    const uint8_t *pa[4], *pb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ra = min(rb + 32 * j, mrows - 1), rbn = min(n0 + rb + 32 * j, a.N - 1);
        const int64_t arow = KSEG || a.a_gather == nullptr ? m0 + ra : a.a_gather[m0 + ra];
        pa[j] = a.A + arow * a.lda + 16 * c;
        pb[j] = Bg + static_cast<int64_t>(rbn) * a.ldb + 16 * c;
    }
    int64_t srow;   // the row whose scale word this thread stages
    if (tid < kNtT) {
        srow = min(n0 + tid, a.N - 1);
    } else {
        const int64_t r = m0 + min(tid - kNtT, mrows - 1);
        srow = KSEG || a.a_gather == nullptr ? r : a.a_gather[r];
    }
    const uint32_t *ps = tid < kNtT ? reinterpret_cast<const uint32_t *>(Bsg + srow * (a.ldb / 32))
                                    : reinterpret_cast<const uint32_t *>(a.As + srow * (a.lda / 32));
    u32x4 RA[4], RB[4];
    uint32_t RS = 0;
    auto load = [&](int t) {
        const int64_t off = static_cast<int64_t>(k0 + t) * kNtK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            RA[j] = *reinterpret_cast<const u32x4 *>(pa[j] + off);
            RB[j] = *reinterpret_cast<const u32x4 *>(pb[j] + off);
        }
        RS = ps[k0 + t];
    };
    auto store = [&](uint8_t *S) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<u32x4 *>(S + mswz(rb + 32 * j, c)) = RB[j];
            *reinterpret_cast<u32x4 *>(S + kNtRegion + mswz(rb + 32 * j, c)) = RA[j];
        }
        reinterpret_cast<uint32_t *>(S + 2 * kNtRegion)[tid] = RS;
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    const int rn = 64 * wn + l32, rm = 64 * wm + l32;
    if (nk > 0) {
        load(0);
        store(LS[0]);
        __syncthreads();
        for (int t = 0; t < nk; ++t) {
            const uint8_t *cur = LS[t & 1];
            if (t + 1 < nk) load(t + 1);
            const uint32_t *W = reinterpret_cast<const uint32_t *>(cur + 2 * kNtRegion);
            uint32_t SA[2], SB[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) SA[i] = W[rn + 32 * i] >> (8 * lhi);
#pragma unroll
            for (int j = 0; j < 2; ++j) SB[j] = W[kNtT + rm + 32 * j] >> (8 * lhi);
            nt_ksub<0>(acc, cur, rn, rm, lhi, SA, SB);
            nt_ksub<1>(acc, cur, rn, rm, lhi, SA, SB);
            // the other stage was last read in step t - 1, before the
            // barrier that ended it
            if (t + 1 < nk) store(LS[(t + 1) & 1]);
            __syncthreads();
        }
    }

    // accumulator q of MFMA (i, j): n = n0 + 64 wn + 32 i + 8 (q/4) + 4 lhi +
    // q%4, m = 64 wm + 32 j + l32 within the tile
    const int64_t crow = KSEG ? static_cast<int64_t>(g) * a.M + m0 : m0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int ml = 64 * wm + 32 * j + l32;
        if (ml >= mrows) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = n0 + 64 * wn + 32 * i + 8 * gq + 4 * lhi;
                if (n >= a.N) continue;
                const int64_t e = (crow + ml) * a.N + n;
                if constexpr (OUT_BF16) {
                    uint2 o;
                    o.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
                    o.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    *reinterpret_cast<uint2 *>(static_cast<bf16_t *>(a.C) + e) = o;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.C) + e) =
                        make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                                    acc[i][j][4 * gq + 3]);
                }
            }
    }
}

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
// column / 32 over all segments. With row_w, segment row r's values are
// multiplied by row_w[r] (in fp32) before quantising.
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
        if (p >= poffs[nseg]) return;
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
        cbase = p;
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
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) word |= e4m3_code(ldexpf(v[4 * w + q], -ex)) << (8 * q);
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
        if (p >= poffs[nseg]) return;
        int lo = 0, hi = nseg - 1;   // largest s with poffs[s] <= p
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (poffs[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        local = p - poffs[lo];
        r0 = offs[lo];
        nrows = offs[lo + 1] - r0;
        cbase = p;
        nblk = 4;
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
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) word |= e4m3_code(ldexpf(v[4 * wd + k], -ex)) << (8 * k);
        out[wd >> 2][wd & 3] = word;
    }
    const int64_t ce = cbase + static_cast<int64_t>(n0 + lane) * ld + 32 * w;
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + ce);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[ce / 32] = static_cast<uint8_t>(ex + 127);
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
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) word |= e4m3_code(ldexpf(v[4 * wd + q], -ex)) << (8 * q);
        out[wd >> 2][wd & 3] = word;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[b] = static_cast<uint8_t>(ex + 127);
}

// act = silu(g) u from the recomputed fp32 pre-activations (g | u) [P][2F];
// four columns per thread.
__global__ __launch_bounds__(256) void mx_swiglu_act_kernel(const float *__restrict__ gu, int64_t P, int F,
                                                            float *__restrict__ act) {
    const int64_t nq = P * (F / 4);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nq;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t p = i / (F / 4);
        const int f = static_cast<int>(i - p * (F / 4)) * 4;
        const float4 g = *reinterpret_cast<const float4 *>(gu + p * 2 * F + f);
        const float4 u = *reinterpret_cast<const float4 *>(gu + p * 2 * F + F + f);
        *reinterpret_cast<float4 *>(act + p * F + f) =
            make_float4(g.x / (1.0f + expf(-g.x)) * u.x, g.y / (1.0f + expf(-g.y)) * u.y,
                        g.z / (1.0f + expf(-g.z)) * u.z, g.w / (1.0f + expf(-g.w)) * u.w);
    }
}

// dgu = SwiGLU backward of dact at the recomputed pre-activations (g | u),
// fp32: dg = dact u s (1 + g (1 - s)), du = dact g s, s = sigmoid(g); four
// columns per thread.
__global__ __launch_bounds__(256) void mx_swiglu_bwd_kernel(const float *__restrict__ dact,
                                                            const float *__restrict__ gu, int64_t P, int F,
                                                            float *__restrict__ dgu) {
    const int64_t nq = P * (F / 4);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nq;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t p = i / (F / 4);
        const int f = static_cast<int>(i - p * (F / 4)) * 4;
        const float4 d = *reinterpret_cast<const float4 *>(dact + p * F + f);
        const float4 g4 = *reinterpret_cast<const float4 *>(gu + p * 2 * F + f);
        const float4 u4 = *reinterpret_cast<const float4 *>(gu + p * 2 * F + F + f);
        const float da[4] = {d.x, d.y, d.z, d.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w}, uv[4] = {u4.x, u4.y, u4.z, u4.w};
        float dg[4], du[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sg = 1.0f / (1.0f + expf(-gv[q]));
            dg[q] = da[q] * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
            du[q] = da[q] * gv[q] * sg;
        }
        *reinterpret_cast<float4 *>(dgu + p * 2 * F + f) = make_float4(dg[0], dg[1], dg[2], dg[3]);
        *reinterpret_cast<float4 *>(dgu + p * 2 * F + F + f) = make_float4(du[0], du[1], du[2], du[3]);
    }
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

inline unsigned grid_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192); }

template <bool KSEG, bool OUT_BF16>
void launch_nt(MxNtArgs a, int64_t P, hipStream_t s) {
    a.n_tiles = (a.N + kNtT - 1) / kNtT;
    int64_t grid;
    if (KSEG) {
        a.m_tiles = (a.M + kNtT - 1) / kNtT;
        grid = static_cast<int64_t>(a.E) * a.m_tiles * a.n_tiles;
    } else {
        grid = (P / kNtT + a.E) * static_cast<int64_t>(a.n_tiles);   // upper bound; extra blocks exit
    }
    if (grid > 0) hipLaunchKernelGGL((mx_gemm_nt<KSEG, OUT_BF16>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
}

// Workspace of the backward: sub-buffers at 256-byte boundaries.
struct MxBwdLayout {
    int64_t Pc;   // columns of the token-blocked (transposed) operands
    size_t poffs, gu, act, dy_c, dy_s, dyT_c, dyT_s, actT_c, actT_s, dact, dgu, dgu_c, dgu_s, dguT_c, dguT_s, xT_c,
        xT_s;
    size_t total;
};

MxBwdLayout mx_bwd_layout(int64_t P, int64_t h, int64_t F, int E) {
    MxBwdLayout L{};
    L.Pc = ((P + 127 * static_cast<int64_t>(E)) + 127) / 128 * 128;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at += (bytes + 255) & ~static_cast<size_t>(255);
        return o;
    };
    const size_t Pz = static_cast<size_t>(P), hz = static_cast<size_t>(h), Fz = static_cast<size_t>(F),
                 Pcz = static_cast<size_t>(L.Pc);
    L.poffs = take(static_cast<size_t>(E + 1) * 4);
    L.gu = take(Pz * 2 * Fz * 4);
    L.act = take(Pz * Fz * 4);
    L.dy_c = take(Pz * hz);
    L.dy_s = take(Pz * hz / 32);
    L.dyT_c = take(hz * Pcz);
    L.dyT_s = take(hz * Pcz / 32);
    L.actT_c = take(Fz * Pcz);
    L.actT_s = take(Fz * Pcz / 32);
    L.dact = take(Pz * Fz * 4);
    L.dgu = take(Pz * 2 * Fz * 4);
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
    MOE_CHECK_ARG(P < (int64_t(1) << 31) && T < (int64_t(1) << 31) && 2 * F * h < (int64_t(1) << 31) &&
                      L.Pc / 32 < (int64_t(1) << 31),
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
    float *act = reinterpret_cast<float *>(ws + L.act);
    float *dgu = reinterpret_cast<float *>(ws + L.dgu);

    hipLaunchKernelGGL(mx_pad_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, E, poffs);
    if (P > 0) {
        // gu = Q_h(X) Q_h(W1) in fp32 (the forward's codes), act = silu(g) u
        MxNtArgs r1{};
        r1.A = x_codes;
        r1.As = x_scales;
        r1.a_gather = sorted_token;
        r1.B = w1_codes;
        r1.Bs = w1_scales;
        r1.C = gu;
        r1.offs = offsets;
        r1.E = E;
        r1.N = 2 * FF;
        r1.K = hh;
        r1.lda = h;
        r1.ldb = h;
        r1.b_stride = 2 * F * h;
        launch_nt<false, false>(r1, P, s);
        hipLaunchKernelGGL(mx_swiglu_act_kernel, dim3(grid_for(P * (F / 4))), dim3(256), 0, s, gu, P, FF, act);
        // dY = row_w * dL/dout along h (rows) and along the tokens; the
        // activation and the token rows along the tokens
        hipLaunchKernelGGL(mx_quantize_rows_gather_kernel<bf16_t>, dim3(static_cast<unsigned>((P * (h / 32) + 255) / 256)),
                           dim3(256), 0, s, G, sorted_token, row_w, P, hh, ws + L.dy_c, ws + L.dy_s);
        launch_quantize_cols(G, h, sorted_token, row_w, offsets, poffs, E, 0, L.Pc, hh, L.Pc, ws + L.dyT_c,
                             ws + L.dyT_s, s);
        launch_quantize_cols(static_cast<const float *>(act), F, nullptr, nullptr, offsets, poffs, E, 0, L.Pc, FF,
                             L.Pc, ws + L.actT_c, ws + L.actT_s, s);
        launch_quantize_cols(static_cast<const bf16_t *>(x), h, sorted_token, nullptr, offsets, poffs, E, 0, L.Pc, hh,
                             L.Pc, ws + L.xT_c, ws + L.xT_s, s);
        // dact = Q_h(dY) Q_h(W2)
        MxNtArgs d2{};
        d2.A = ws + L.dy_c;
        d2.As = ws + L.dy_s;
        d2.B = w2t_codes;
        d2.Bs = w2t_scales;
        d2.C = ws + L.dact;
        d2.offs = offsets;
        d2.E = E;
        d2.N = FF;
        d2.K = hh;
        d2.lda = h;
        d2.ldb = h;
        d2.b_stride = F * h;
        launch_nt<false, false>(d2, P, s);
        // dgu, then along 2F (rows) and along the tokens
        hipLaunchKernelGGL(mx_swiglu_bwd_kernel, dim3(grid_for(P * (F / 4))), dim3(256), 0, s,
                           reinterpret_cast<const float *>(ws + L.dact), static_cast<const float *>(gu), P, FF, dgu);
        launch_quantize(static_cast<const float *>(dgu), P, 2 * F, ws + L.dgu_c, ws + L.dgu_s, s);
        launch_quantize_cols(static_cast<const float *>(dgu), 2 * F, nullptr, nullptr, offsets, poffs, E, 0, L.Pc,
                             2 * FF, L.Pc, ws + L.dguT_c, ws + L.dguT_s, s);
        // dX = Q_2F(dgu) Q_2F(W1)
        MxNtArgs d1{};
        d1.A = ws + L.dgu_c;
        d1.As = ws + L.dgu_s;
        d1.B = w1t_codes;
        d1.Bs = w1t_scales;
        d1.C = grad_x_perm;
        d1.offs = offsets;
        d1.E = E;
        d1.N = hh;
        d1.K = 2 * FF;
        d1.lda = 2 * F;
        d1.ldb = 2 * F;
        d1.b_stride = 2 * F * h;
        launch_nt<false, true>(d1, P, s);
    }
    // dW2 = Q_tok(dY)^T Q_tok(act), dW1 = Q_tok(dgu)^T Q_tok(X): every
    // expert's tiles run (zeros when it has no tokens)
    MxNtArgs w2{};
    w2.A = ws + L.dyT_c;
    w2.As = ws + L.dyT_s;
    w2.B = ws + L.actT_c;
    w2.Bs = ws + L.actT_s;
    w2.C = grad_w2;
    w2.offs = poffs;
    w2.E = E;
    w2.M = hh;
    w2.N = FF;
    w2.lda = L.Pc;
    w2.ldb = L.Pc;
    launch_nt<true, false>(w2, P, s);
    MxNtArgs w1{};
    w1.A = ws + L.dguT_c;
    w1.As = ws + L.dguT_s;
    w1.B = ws + L.xT_c;
    w1.Bs = ws + L.xT_s;
    w1.C = grad_w1;
    w1.offs = poffs;
    w1.E = E;
    w1.M = 2 * FF;
    w1.N = hh;
    w1.lda = L.Pc;
    w1.ldb = L.Pc;
    launch_nt<true, false>(w1, P, s);
    return check_launch("moe_grouped_ffn_bwd_mx");
}
