// Backward of the grouped bf16 SwiGLU FFN: four grouped GEMMs per step
// (other expert kinds and fp32: ffn_bwd_generic.hip).
//
//   dact   = dY W2[e]                      (per segment; + SwiGLU backward)
//   dg     = dact * u * silu'(g),  du = dact * silu(g)
//   dX     = [dg du] W1[e]                 (per segment)
//   dW2[e] = dY_e^T act_e                  (K = tokens of expert e)
//   dW1[e] = [dg du]_e^T X_e               (K = tokens of expert e)
//
// with silu'(g) = s (1 + g (1 - s)), s = sigma(g). The forward these derive
// from is the SwiGLU expert of "Mixture-of-Experts from Architecture to
// Large-Scale Training" (section 2.5) run as one grouped GEMM over experts
// ("Scalable Training of Mixture-of-Experts Models with Megatron Core",
// section 2.1 stage 3).
//
// One kernel template serves all four, built like the forward kernel: 4
// waves, 128 x 128 (or 64 x 128) wave tiles of v_mfma_f32_32x32x16_bf16
// accumulators, 64-deep k-steps staged global -> VGPR -> LDS one k-step ahead,
// the LDS reads, LDS writes and global loads of each k-step interleaved
// between its MFMAs. Operands whose storage has K as the slow index (the
// weights [K][cols] of the two data-gradient GEMMs, the activations
// [tokens][cols] of the two weight-gradient GEMMs) are copied to LDS as they
// are, K rows of 256 contiguous columns, and read out with
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column
// of a 4-row block: two such reads give a lane the 8 consecutive k of its
// MFMA row. Weight-gradient tiles cover the whole K range of their expert
// (no split-K, so results are deterministic), rows past the expert's tokens
// read as zero (buffer range), tiles are ordered heaviest expert first, and
// experts without tokens get zero gradients.
#include "gemm_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// kDgradSwiGLUW: the SwiGLU backward of an activation scaled by a per-row
// weight p (row_w): d(p a)/da = p, and the row's dL/dp = <dact, a> is summed
// per tile into dp_part.
enum BwdKind { kDgradSwiGLU = 0, kDgradPlain = 1, kWgrad = 2, kDgradSwiGLUW = 3 };

struct BGArgs {
    const bf16_t *A;          // MFMA "A": K-major storage, element (k, a) at A[k * lda + a]
    const bf16_t *B;          // MFMA "B": dgrad: row-major [P][K]; wgrad: K-major like A
    void *C;                  // dgrad: [P][a_dim] bf16 (plain); wgrad: [E][b_dim][a_dim] fp32
    const bf16_t *GU;         // SwiGLU backward: pre-activations [P][2 a_dim]
    bf16_t *dGU;              // SwiGLU backward: output [P][2 a_dim]
    const int32_t *offsets;   // [E+1]
    int E;
    int a_dim;                // rows of the A operand = columns of C
    int b_dim;                // wgrad: rows of the B operand = rows of C
    int K;                    // dgrad: reduction length
    int lda, ldb;             // storage row strides (elements)
    int64_t a_expert_stride;  // dgrad: elements between experts' weights; wgrad: 0
    int n_tiles_a, n_tiles_b;
    int grid;
    const float *row_w;       // kDgradSwiGLUW: [P] per-row weights of the activation
    float *dp_part;           // kDgradSwiGLUW: [P][n_tiles_a] per-tile sums of <dact, a>
};

constexpr int kBK = 64, kTile = 256, kRegion = kTile * kBK, kStage = 2 * kRegion;

// Row-major token region [256 rows][64 k]: chunk c of row r at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz_k(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 7)) << 3); }
// K-row region [64 k][256 cols]: 16-byte chunk q of row k at q ^ ((k & 3) << 2),
// so the 4 rows x 4 chunks that 32 lanes of a transposing read touch fall in
// 16 different bank groups.
__device__ __forceinline__ int swz_mn(int k, int col) {
    return k * kTile + (((col >> 3) ^ ((k & 3) << 2)) << 3) + (col & 7);
}

// MFMA operand for rows c0..c0+31 (columns of the K-row region) and
// k = 16 ks .. 16 ks + 15: lane group g = lane / 16 covers rows
// c0 + 16 (g & 1) .. +15 and k 8 (g >> 1) .. +7; lane j of the group names
// row 4-block j / 4, chunk j % 4, and receives column j of each 4-row block.
__device__ __forceinline__ bf16x8_t frag_mn(const bf16_t *R, int c0, int ks, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int k = ks * 16 + 8 * (g >> 1) + (j >> 2);
    const int col = c0 + 16 * (g & 1) + 4 * (j & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(R + swz_mn(k, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(R + swz_mn(k + 4, col)));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Even spread of NRD fragment reads and NWR (write, load) pairs over the NMF
// MFMAs of a quarter.
template <int NMF, int NRD, int NWR, int Q = 0>
__device__ __forceinline__ void sched_quarter() {
    if constexpr (Q < NMF) {
        MOE_SGB(kSgMfma, 1);
        constexpr int r = (Q + 1) * NRD / NMF - Q * NRD / NMF;
        if constexpr (r > 0) MOE_SGB(kSgDsRead, r);
        constexpr int w = (Q + 1) * NWR / NMF - Q * NWR / NMF;
        if constexpr (w > 0) {
            MOE_SGB(kSgDsWrite, w);
            MOE_SGB(kSgVmemRead, w);
        }
        sched_quarter<NMF, NRD, NWR, Q + 1>();
    }
}

// One output tile. dgrad: token rows [row0, row0 + rows) of P (all of one
// expert e), columns [a0, a0 + 256) of C, K = a.K. wgrad: rows [b0, b0 + 256)
// of C = dW[e], columns [a0, a0 + 256), K = the nk_tok tokens of expert e
// starting at row0. FULL (HALF = false): wave w owns columns 128 (w % 2) ..
// and rows 128 (w / 2) ..; HALF: columns 64 w .. +63, rows 0..127.
template <int KIND, bool ODD, bool HALF>
__device__ __forceinline__ void bwd_tile(const BGArgs &a, int e, int a0, int b0, int row0, int rows,
                                         int nk_tok, bf16_t *LB0, bf16_t *LB1, float (*s_dp)[kTile]) {
    constexpr bool WG = KIND == kWgrad;
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    constexpr int XB = WG ? 8 : (HALF ? 4 : 8);     // B chunks per thread per k-step
    constexpr int NMF = NI * NJ;
    constexpr int NRD = 2 * NI + (WG ? 2 : 1) * NJ;
    constexpr int NWR = (8 + XB) / 2;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int acol0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int brow0 = HALF ? 0 : (wave >> 1) * 128;

    // reduction length in k-steps (wgrad: at least one, so that an expert
    // without tokens gets zeros); rows past the expert's tokens read as zero
    const int Krows = WG ? nk_tok : a.K;
    int nk = (Krows + kBK - 1) / kBK;
    if (WG) nk = max(1, nk);
    nk = __builtin_amdgcn_readfirstlane(nk);

    // A: K-row storage; thread t moves chunk t % 32 of k-rows t / 32 + 8 j
    const bf16_t *abase = WG ? a.A + static_cast<int64_t>(row0) * a.lda
                             : a.A + static_cast<int64_t>(e) * a.a_expert_stride;
    const int ca = tid & 31, kr0 = tid >> 5;
    const int acol = min(a0 + 8 * ca, a.a_dim - 8);
    const int va0 = (kr0 * a.lda + acol) * 2;
    const int vstep_a = 16 * a.lda;                     // 8 rows, bytes
    const int offa = swz_mn(kr0, 8 * ca);              // + 8 j rows
    // B: wgrad K-row storage like A; dgrad row-major token rows rb + 32 j
    const bf16_t *bbase = a.B + static_cast<int64_t>(row0) * a.ldb;
    int vb[XB];
    int offb;
    if (WG) {
        const int bcol = min(b0 + 8 * ca, a.b_dim - 8);
        vb[0] = (kr0 * a.ldb + bcol) * 2;
#pragma unroll
        for (int j = 1; j < XB; ++j) vb[j] = vb[0] + j * 16 * a.ldb;
        offb = swz_mn(kr0, 8 * ca);
    } else {
        const int chunk = tid & 7, rb = tid >> 3;
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int r = rb + 32 * j;
            vb[j] = ((r < rows ? r : rows - 1) * a.ldb + chunk * 8) * 2;
        }
        offb = swz_k(rb, chunk);
    }
    const __amdgpu_buffer_rsrc_t rb_tok = make_rsrc(bbase);   // dgrad B (k advances within rows)

    floatx16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    u32x4 RA[8], RB[XB];
    bf16x8_t fa0[NI], fb0[NJ], fa1[NI], fb1[NJ];

// K-row operands: a resource over the k-step's remaining rows, so rows past
// the end read as zero
#define MOE_KROWS_RSRC(BASE, LD, KT)                                                              \
    make_rsrc((BASE) + static_cast<int64_t>(KT) * kBK * (LD),                                   \
              static_cast<uint32_t>(max(0, Krows - (KT) * kBK)) * static_cast<uint32_t>(LD) * 2u)
#define MOE_LD(KT, H)                                                                             \
    do {                                                                                        \
        const __amdgpu_buffer_rsrc_t ra_ = MOE_KROWS_RSRC(abase, a.lda, KT);                    \
        _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                            \
            RA[j] = __builtin_amdgcn_raw_buffer_load_b128(ra_, va0 + j * vstep_a, 0, 0);        \
        if (WG) {                                                                               \
            const __amdgpu_buffer_rsrc_t rbk_ = MOE_KROWS_RSRC(bbase, a.ldb, KT);               \
            _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                        \
                RB[j] = __builtin_amdgcn_raw_buffer_load_b128(rbk_, vb[j], 0, 0);               \
        } else {                                                                                \
            _Pragma("unroll") for (int j = (XB / 2) * (H); j < (XB / 2) * (H) + XB / 2; ++j)    \
                RB[j] = __builtin_amdgcn_raw_buffer_load_b128(rb_tok, vb[j], (KT) * kBK * 2, 0); \
        }                                                                                       \
    } while (0)
#define MOE_WR(LB, H)                                                                             \
    do {                                                                                        \
        _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                            \
            *reinterpret_cast<u32x4 *>((LB) + offa + j * 8 * kTile) = RA[j];                     \
        if (WG) {                                                                               \
            _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                        \
                *reinterpret_cast<u32x4 *>((LB) + kRegion + offb + j * 8 * kTile) = RB[j];       \
        } else {                                                                                \
            _Pragma("unroll") for (int j = (XB / 2) * (H); j < (XB / 2) * (H) + XB / 2; ++j)    \
                *reinterpret_cast<u32x4 *>((LB) + kRegion + offb + j * 32 * kBK) = RB[j];        \
        }                                                                                       \
    } while (0)
#define MOE_RD(FA, FB, LB, KS)                                                                    \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < NI; ++i) FA[i] = frag_mn((LB), acol0 + 32 * i, (KS), lane); \
        if (WG) {                                                                               \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                      \
                FB[j] = frag_mn((LB) + kRegion, brow0 + 32 * j, (KS), lane);                    \
        } else {                                                                                \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                      \
                FB[j] = *reinterpret_cast<const bf16x8_t *>((LB) + kRegion +                    \
                                                            swz_k(brow0 + 32 * j + l32, (KS) * 2 + lhi)); \
        }                                                                                       \
    } while (0)
#define MOE_MF(FA, FB)                                                                            \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < NI; ++i)                                          \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                    \
                if constexpr (WG)                                                               \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FB[j], FA[i], acc[i][j], 0, 0, 0); \
                else                                                                            \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0); \
            }                                                                                   \
    } while (0)
#define MOE_STEP(CUR, NXT, T)                                                                     \
    do {                                                                                        \
        const int kk_ = (T) + 2 < nk ? (T) + 2 : nk - 1;                                        \
        MOE_MF(fa0, fb0); MOE_RD(fa1, fb1, CUR, 1);                                             \
        sched_quarter<NMF, NRD, 0>(); __builtin_amdgcn_sched_barrier(0);                        \
        MOE_MF(fa1, fb1); MOE_RD(fa0, fb0, CUR, 2); MOE_WR(NXT, 0); MOE_LD(kk_, 0);             \
        sched_quarter<NMF, NRD, NWR>(); __builtin_amdgcn_sched_barrier(0);                      \
        MOE_MF(fa0, fb0); MOE_RD(fa1, fb1, CUR, 3); MOE_WR(NXT, 1); MOE_LD(kk_, 1);             \
        sched_quarter<NMF, NRD, NWR>(); __builtin_amdgcn_sched_barrier(0);                      \
        MOE_LDS_BARRIER();                                                                      \
        MOE_MF(fa1, fb1); MOE_RD(fa0, fb0, NXT, 0);                                             \
        sched_quarter<NMF, NRD, 0>(); __builtin_amdgcn_sched_barrier(0);                        \
    } while (0)

    MOE_LD(0, 0);
    MOE_LD(0, 1);
    MOE_LDS_BARRIER();   // every wave is done reading the previous tile's stages
    MOE_WR(LB0, 0);
    MOE_WR(LB0, 1);
    {
        const int k1 = nk > 1 ? 1 : 0;
        MOE_LD(k1, 0);
        MOE_LD(k1, 1);
    }
    MOE_LDS_BARRIER();
    MOE_RD(fa0, fb0, LB0, 0);
    // pairs of k-steps, then the odd one (dgrad: known at compile time;
    // wgrad: the expert's token count decides)
    for (int t = 0; t + 1 < nk; t += 2) {
        MOE_STEP(LB0, LB1, t);
        MOE_STEP(LB1, LB0, t + 1);
    }
    if (ODD || (WG && (nk & 1))) MOE_STEP(LB0, LB1, nk - 1);
#undef MOE_KROWS_RSRC
#undef MOE_LD
#undef MOE_WR
#undef MOE_RD
#undef MOE_MF
#undef MOE_STEP

    // ------------------------------------------------------------ epilogue
    if constexpr (WG) {
        // The weight-gradient products run with the operands swapped, so
        // lane l holds column acol0 + 32 i + l % 32 of rows
        // brow0 + 32 j + 8 (v / 4) + 4 (l / 32) + v % 4: each store writes two
        // whole 128-byte row pieces of the fp32 tile.
        float *Ce = static_cast<float *>(a.C) + static_cast<int64_t>(e) * a.b_dim * a.a_dim;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int col = a0 + acol0 + 32 * i + l32;
            if (col >= a.a_dim) continue;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = b0 + brow0 + 32 * j + 8 * (v >> 2) + 4 * lhi + (v & 3);
                    // streamed past the caches: nothing reads the tile again here
                    if (row < a.b_dim)
                        __builtin_nontemporal_store(acc[i][j][v], Ce + static_cast<int64_t>(row) * a.a_dim + col);
                }
        }
        return;
    }
    float dpacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) dpacc[j] = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int bl = brow0 + j * 32 + l32;   // row of C within the tile
        if (!WG && bl >= rows) continue;
        if (WG && b0 + bl >= a.b_dim) continue;
        const float pw = KIND == kDgradSwiGLUW ? a.row_w[row0 + bl] : 1.0f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int col = a0 + acol0 + i * 32 + 8 * gq + 4 * lhi;
                if (col >= a.a_dim) continue;
                if (KIND == kWgrad) {
                    const float4 o = make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                                                 acc[i][j][4 * gq + 3]);
                    float *C = static_cast<float *>(a.C) + (static_cast<int64_t>(e) * a.b_dim + b0 + bl) * a.a_dim + col;
                    *reinterpret_cast<float4 *>(C) = o;
                } else if (KIND == kDgradPlain) {
                    uint2 o;
                    o.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
                    o.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    bf16_t *C = static_cast<bf16_t *>(a.C) + (static_cast<int64_t>(row0) + bl) * a.a_dim + col;
                    *reinterpret_cast<uint2 *>(C) = o;
                } else {
                    const int64_t r = static_cast<int64_t>(row0) + bl;
                    const bf16_t *gr = a.GU + r * 2 * a.a_dim;
                    const uint2 gv = *reinterpret_cast<const uint2 *>(gr + col);
                    const uint2 uv = *reinterpret_cast<const uint2 *>(gr + a.a_dim + col);
                    const float g[4] = {bf16lo(gv.x), bf16hi(gv.x), bf16lo(gv.y), bf16hi(gv.y)};
                    const float u[4] = {bf16lo(uv.x), bf16hi(uv.x), bf16lo(uv.y), bf16hi(uv.y)};
                    float dg[4], du[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float d = acc[i][j][4 * gq + q];
                        // hardware exp and reciprocal (a few ulp): with the
                        // IEEE divide the epilogue needs so many registers
                        // that the accumulators get spilled inside the k-loop
                        const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g[q]));
                        if (KIND == kDgradSwiGLUW) {
                            dpacc[j] = fmaf(d, g[q] * s * u[q], dpacc[j]);
                            d *= pw;
                        }
                        dg[q] = d * u[q] * (s * (1.0f + g[q] * (1.0f - s)));
                        du[q] = d * (g[q] * s);
                    }
                    bf16_t *dr = a.dGU + r * 2 * a.a_dim;
                    uint2 og, ou;
                    og.x = pack_bf16x2(dg[0], dg[1]);
                    og.y = pack_bf16x2(dg[2], dg[3]);
                    ou.x = pack_bf16x2(du[0], du[1]);
                    ou.y = pack_bf16x2(du[2], du[3]);
                    *reinterpret_cast<uint2 *>(dr + col) = og;
                    *reinterpret_cast<uint2 *>(dr + a.a_dim + col) = ou;
                }
            }
        }
    }
    if constexpr (KIND == kDgradSwiGLUW) {
        // <dact, a> of each row: this lane's columns, then its partner half
        // (lane ^ 32), then the waves sharing the row in a fixed order
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float v = dpacc[j] + __shfl_xor(dpacc[j], 32);
            if (lhi == 0) s_dp[HALF ? wave : (wave & 1)][brow0 + j * 32 + l32] = v;
        }
        __syncthreads();
        const int r = threadIdx.x;
        if (r < rows) {
            const float v = HALF ? ((s_dp[0][r] + s_dp[1][r]) + s_dp[2][r]) + s_dp[3][r] : s_dp[0][r] + s_dp[1][r];
            a.dp_part[static_cast<int64_t>(row0 + r) * a.n_tiles_a + a0 / kTile] = v;
        }
    }
}

// ODD (data-gradient GEMMs only): K / 64 is odd.
template <int KIND, bool ODD>
__global__ __launch_bounds__(256, 1) void bwd_gemm(BGArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t LB0[kStage];
    __shared__ __attribute__((aligned(16))) bf16_t LB1[kStage];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    __shared__ int s_order[256];
    __shared__ float s_dp[KIND == kDgradSwiGLUW ? 4 : 1][kTile];
    const int tid = threadIdx.x;

    int total;
    if (KIND == kWgrad) {
        // experts by decreasing token count (ties: lower index first)
        s_tmp[tid] = tid < a.E ? a.offsets[tid + 1] - a.offsets[tid] : -1;
        __syncthreads();
        if (tid < a.E) {
            const int m = s_tmp[tid];
            int rank = 0;
            for (int e = 0; e < a.E; ++e) {
                const int me = s_tmp[e];
                rank += (me > m) || (me == m && e < tid);
            }
            s_order[rank] = tid;
        }
        __syncthreads();
        total = a.E * a.n_tiles_a * a.n_tiles_b;
    } else {
        GGArgs g{};
        g.offsets = a.offsets;
        g.E = a.E;
        g.n_tiles = a.n_tiles_a;
        total = build_tile_prefix(g, kTile, s_cum, s_tmp);
    }
    total = __builtin_amdgcn_readfirstlane(total);

    const int cu = xcd_block_index(blockIdx.x, a.grid);
    for (int L0 = 0; L0 < total; L0 += a.grid) {
        // wgrad: experts by decreasing size, and every other round of tiles
        // in reverse block order, so that the blocks' token totals even out
        const int L = KIND == kWgrad && ((L0 / a.grid) & 1) ? L0 + a.grid - 1 - cu : L0 + cu;
        if (L >= total) continue;
        if (KIND == kWgrad) {
            const int per = a.n_tiles_a * a.n_tiles_b;
            const int e = s_order[L / per];
            const int local = L % per;
            const int row0 = a.offsets[e];
            bwd_tile<KIND, false, false>(a, e, (local % a.n_tiles_a) * kTile, (local / a.n_tiles_a) * kTile, row0,
                                         0, a.offsets[e + 1] - row0, LB0, LB1, s_dp);
        } else {
            GGArgs g{};
            g.offsets = a.offsets;
            g.E = a.E;
            g.n_tiles = a.n_tiles_a;
            const TileInfo ti = decode_tile(g, s_cum, L, kTile);
            const int rows = min(kTile, ti.M - ti.m0);
            if (rows > kTile / 2)
                bwd_tile<KIND, ODD, false>(a, ti.seg, ti.n_tile * kTile, 0, ti.row0 + ti.m0, rows, 0, LB0, LB1,
                                           s_dp);
            else
                bwd_tile<KIND, ODD, true>(a, ti.seg, ti.n_tile * kTile, 0, ti.row0 + ti.m0, rows, 0, LB0, LB1,
                                          s_dp);
        }
    }
}

template <int KIND>
int launch_bwd(BGArgs a, int64_t P, hipStream_t s, const char *what) {
    a.n_tiles_a = (a.a_dim + kTile - 1) / kTile;
    int64_t upper;
    if (KIND == kWgrad) {
        a.n_tiles_b = (a.b_dim + kTile - 1) / kTile;
        upper = static_cast<int64_t>(a.E) * a.n_tiles_a * a.n_tiles_b;
    } else {
        a.n_tiles_b = 1;
        upper = (P / kTile + a.E) * static_cast<int64_t>(a.n_tiles_a);
    }
    int64_t grid = num_cus();
    if (grid > upper) grid = upper;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    if (KIND != kWgrad && ((a.K / kBK) & 1))
        hipLaunchKernelGGL((bwd_gemm<KIND, true>), dim3(a.grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_gemm<KIND, false>), dim3(a.grid), dim3(256), 0, s, a);
    return check_launch(what);
}

}  // namespace

// Plain grouped GEMMs of the backward kernel for other callers (the router's
// dense backward). Weight-gradient form: C[s] [b_dim][a_dim] (fp32) =
// B_s^T A_s over the rows of segment s (A [rows][a_dim], B [rows][b_dim],
// both K-major with row strides lda, ldb). Data-gradient form: C [P][a_dim]
// (bf16) = B A, B [P][K] row-major (stride ldb), A [K][a_dim] (stride lda),
// over the segments of offsets (all with the same A).
int bwd_wgrad_segments(const bf16_t *A, int lda, int a_dim, const bf16_t *B, int ldb, int b_dim,
                       const int32_t *offsets, int nseg, int64_t rows, float *C, hipStream_t s) {
    BGArgs w{};
    w.A = A;
    w.B = B;
    w.C = C;
    w.offsets = offsets;
    w.E = nseg;
    w.a_dim = a_dim;
    w.b_dim = b_dim;
    w.lda = lda;
    w.ldb = ldb;
    return launch_bwd<kWgrad>(w, rows, s, "wgrad gemm");
}

int bwd_dgrad_plain(const bf16_t *B, int ldb, const bf16_t *A, int lda, int a_dim, int K, const int32_t *offsets,
                    int nseg, int64_t P, bf16_t *C, hipStream_t s) {
    BGArgs d{};
    d.A = A;
    d.B = B;
    d.C = C;
    d.offsets = offsets;
    d.E = nseg;
    d.a_dim = a_dim;
    d.K = K;
    d.lda = lda;
    d.ldb = ldb;
    d.a_expert_stride = 0;
    return launch_bwd<kDgradPlain>(d, P, s, "dgrad gemm");
}

}  // namespace moe

using namespace moe;

namespace {

// act[r][f] = bf16(silu(g) * u * p_r) from the saved pre-activations, with
// the forward epilogue's expression (p = 1 without row weights): one 8-column
// piece per thread.
__global__ __launch_bounds__(256) void swiglu_recompute_kernel(const bf16_t *__restrict__ gu,
                                                               const float *__restrict__ row_w, int F,
                                                               bf16_t *__restrict__ act, int64_t npieces) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = F >> 3;
    const int64_t r = idx / nv;
    const int v = static_cast<int>(idx - r * nv);
    const bf16_t *gr = gu + r * 2 * F + 8 * v;
    float g[8], u[8], o[8];
    load8(gr, g);
    load8(gr + F, u);
    const float p = row_w ? row_w[r] : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = silu_fast(g[i]) * u[i] * p;
    store8(act + r * F + 8 * v, o);
}

// grad_row_w[r] = sum of the row's per-tile partials, tiles ascending.
__global__ __launch_bounds__(256) void dp_reduce_kernel(const float *__restrict__ part, int nt, int64_t P,
                                                        float *__restrict__ grad_row_w) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r >= P) return;
    float s = 0.0f;
    for (int t = 0; t < nt; ++t) s += part[r * nt + t];
    grad_row_w[r] = s;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int check_bwd_args(const char *what, const void *grad_y, const void *x_perm, const void *gu, int dtype, int64_t P,
                   int64_t h, int64_t F, int E, const int32_t *offsets, int act_kind, const void *w1,
                   const void *w2, const void *grad_gu, const void *grad_x_perm, const float *grad_w1,
                   const float *grad_w2, bool bf16_swiglu_only) {
    MOE_CHECK_ARG(offsets && w1 && w2 && grad_w1 && grad_w2 &&
                      (P == 0 || (grad_y && x_perm && gu && grad_gu && grad_x_perm)),
                  MOE_ERR_INVALID_ARG, "%s: null required pointer", what);
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG, "%s: bad dtype %d", what,
                  dtype);
    MOE_CHECK_ARG(act_kind == MOE_ACT_GELU || act_kind == MOE_ACT_SWIGLU, MOE_ERR_INVALID_ARG,
                  "%s: bad activation %d", what, act_kind);
    MOE_CHECK_ARG(P >= 0 && h > 0 && F > 0 && E > 0, MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    MOE_CHECK_ARG(!bf16_swiglu_only || (dtype == MOE_DTYPE_BF16 && act_kind == MOE_ACT_SWIGLU), MOE_ERR_UNSUPPORTED,
                  "%s: bf16 SwiGLU experts only", what);
    MOE_CHECK_ARG(h % 64 == 0 && F % 64 == 0 && E <= 256, MOE_ERR_UNSUPPORTED,
                  "%s: need h %% 64 == 0, F %% 64 == 0, E <= 256", what);
    MOE_CHECK_ARG(P < (int64_t(1) << 31) && h < (int64_t(1) << 20) && F < (int64_t(1) << 20) &&
                      P * (2 * F > h ? 2 * F : h) < (int64_t(1) << 31),
                  MOE_ERR_UNSUPPORTED, "%s: sizes too large", what);
    const void *ptrs[] = {grad_y, x_perm, gu, w1, w2, grad_gu, grad_x_perm, grad_w1, grad_w2};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(aligned16(p), MOE_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", what);
    return MOE_OK;
}

// The four GEMMs of the backward; with row_w, the data gradient of the
// activation uses the weighted SwiGLU backward and leaves per-tile partials of
// dL/dp in dp_part.
int ffn_bwd_gemms(const bf16_t *dY, const bf16_t *X, const bf16_t *H, const void *gu, int64_t P, int64_t h,
                  int64_t F, int E, const int32_t *offsets, const void *w1, const void *w2, bf16_t *dGU,
                  void *grad_x_perm, float *grad_w1, float *grad_w2, const float *row_w, float *dp_part,
                  hipStream_t s) {
    const int hi = static_cast<int>(h), Fi = static_cast<int>(F);

    // dact = dY W2[e] with the SwiGLU backward fused: A = W2[e] as [h][F]
    BGArgs d2{};
    d2.A = static_cast<const bf16_t *>(w2);
    d2.B = dY;
    d2.GU = static_cast<const bf16_t *>(gu);
    d2.dGU = dGU;
    d2.offsets = offsets;
    d2.E = E;
    d2.a_dim = Fi;
    d2.K = hi;
    d2.lda = Fi;
    d2.ldb = hi;
    d2.a_expert_stride = static_cast<int64_t>(h) * F;
    d2.row_w = row_w;
    d2.dp_part = dp_part;
    int st = row_w ? launch_bwd<kDgradSwiGLUW>(d2, P, s, "moe_grouped_ffn_bwd dact")
                   : launch_bwd<kDgradSwiGLU>(d2, P, s, "moe_grouped_ffn_bwd dact");
    if (st != MOE_OK) return st;

    // dX = [dg du] W1[e]: A = W1[e] as [2F][h]
    BGArgs d1{};
    d1.A = static_cast<const bf16_t *>(w1);
    d1.B = dGU;
    d1.C = grad_x_perm;
    d1.offsets = offsets;
    d1.E = E;
    d1.a_dim = hi;
    d1.K = 2 * Fi;
    d1.lda = hi;
    d1.ldb = 2 * Fi;
    d1.a_expert_stride = 2 * static_cast<int64_t>(F) * h;
    st = launch_bwd<kDgradPlain>(d1, P, s, "moe_grouped_ffn_bwd dx");
    if (st != MOE_OK) return st;

    // dW2[e] = dY_e^T act_e: rows h (B = dY), columns F (A = act)
    BGArgs w2g{};
    w2g.A = H;
    w2g.B = dY;
    w2g.C = grad_w2;
    w2g.offsets = offsets;
    w2g.E = E;
    w2g.a_dim = Fi;
    w2g.b_dim = hi;
    w2g.lda = Fi;
    w2g.ldb = hi;
    st = launch_bwd<kWgrad>(w2g, P, s, "moe_grouped_ffn_bwd dW2");
    if (st != MOE_OK) return st;

    // dW1[e] = [dg du]_e^T X_e: rows 2F (B = dGU), columns h (A = X)
    BGArgs w1g{};
    w1g.A = X;
    w1g.B = dGU;
    w1g.C = grad_w1;
    w1g.offsets = offsets;
    w1g.E = E;
    w1g.a_dim = hi;
    w1g.b_dim = 2 * Fi;
    w1g.lda = hi;
    w1g.ldb = 2 * Fi;
    return launch_bwd<kWgrad>(w1g, P, s, "moe_grouped_ffn_bwd dW1");
}

}  // namespace

extern "C" int moe_grouped_ffn_bwd(const void *grad_y, const void *x_perm, const void *act,
                                   const void *gu, int dtype, int64_t P, int64_t h, int64_t F, int E,
                                   const int32_t *offsets, int act_kind, const void *w1,
                                   const void *w2, void *grad_gu, void *grad_x_perm, float *grad_w1,
                                   float *grad_w2, float *grad_b1, float *grad_b2, void *stream) {
    clear_error();
    int st = check_bwd_args("moe_grouped_ffn_bwd", grad_y, x_perm, gu, dtype, P, h, F, E, offsets, act_kind, w1,
                            w2, grad_gu, grad_x_perm, grad_w1, grad_w2, false);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(P == 0 || (act && aligned16(act)), MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_bwd: act must be a 16-byte aligned pointer");
    hipStream_t s = as_stream(stream);
    if (dtype != MOE_DTYPE_BF16 || act_kind != MOE_ACT_SWIGLU)
        return ffn_bwd_generic(grad_y, x_perm, act, gu, dtype, P, h, F, E, offsets, act_kind, w1, w2, grad_gu,
                               grad_x_perm, grad_w1, grad_w2, grad_b1, grad_b2, s);
    st = ffn_bwd_gemms(static_cast<const bf16_t *>(grad_y), static_cast<const bf16_t *>(x_perm),
                       static_cast<const bf16_t *>(act), gu, P, h, F, E, offsets, w1, w2,
                       static_cast<bf16_t *>(grad_gu), grad_x_perm, grad_w1, grad_w2, nullptr, nullptr, s);
    if (st != MOE_OK) return st;
    if (grad_b2) st = segment_colsums_bf16(grad_y, static_cast<int>(h), offsets, E, grad_b2, s, "moe_grouped_ffn_bwd db2");
    if (st != MOE_OK) return st;
    if (grad_b1)
        st = segment_colsums_bf16(grad_gu, static_cast<int>(2 * F), offsets, E, grad_b1, s, "moe_grouped_ffn_bwd db1");
    return st;
}

extern "C" size_t moe_grouped_ffn_bwd_recompute_workspace_size(int64_t P, int64_t F, int weighted) {
    if (P <= 0 || F <= 0) return 0;
    const size_t act = align256(static_cast<size_t>(P) * static_cast<size_t>(F) * sizeof(bf16_t));
    const size_t nt = static_cast<size_t>((F + kTile - 1) / kTile);
    return act + (weighted ? static_cast<size_t>(P) * nt * sizeof(float) : 0);
}

extern "C" int moe_grouped_ffn_bwd_recompute(const void *grad_y, const void *x_perm, const void *gu, int dtype,
                                             int64_t P, int64_t h, int64_t F, int E, const int32_t *offsets,
                                             int act_kind, const void *w1, const void *w2, const float *row_w,
                                             void *grad_gu, void *grad_x_perm, float *grad_w1, float *grad_w2,
                                             float *grad_row_w, void *workspace, size_t workspace_bytes,
                                             void *stream) {
    clear_error();
    int st = check_bwd_args("moe_grouped_ffn_bwd_recompute", grad_y, x_perm, gu, dtype, P, h, F, E, offsets,
                            act_kind, w1, w2, grad_gu, grad_x_perm, grad_w1, grad_w2, true);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG((row_w == nullptr) == (grad_row_w == nullptr), MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_bwd_recompute: row_w and grad_row_w go together");
    const size_t need = moe_grouped_ffn_bwd_recompute_workspace_size(P, F, row_w != nullptr);
    MOE_CHECK_ARG(need == 0 || (workspace && workspace_bytes >= need && aligned16(workspace)), MOE_ERR_WORKSPACE,
                  "moe_grouped_ffn_bwd_recompute: a 16-byte aligned workspace of %zu bytes is needed", need);
    hipStream_t s = as_stream(stream);
    bf16_t *H = static_cast<bf16_t *>(workspace);
    float *dp_part = row_w ? reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                       align256(static_cast<size_t>(P) * F * sizeof(bf16_t)))
                           : nullptr;
    if (P > 0) {
        const int64_t npieces = P * (F / 8);
        hipLaunchKernelGGL(swiglu_recompute_kernel, dim3(static_cast<unsigned>((npieces + 255) / 256)), dim3(256),
                           0, s, static_cast<const bf16_t *>(gu), row_w, static_cast<int>(F), H, npieces);
        st = check_launch("moe_grouped_ffn_bwd_recompute act");
        if (st != MOE_OK) return st;
    }
    st = ffn_bwd_gemms(static_cast<const bf16_t *>(grad_y), static_cast<const bf16_t *>(x_perm), H, gu, P, h, F, E,
                       offsets, w1, w2, static_cast<bf16_t *>(grad_gu), grad_x_perm, grad_w1, grad_w2, row_w,
                       dp_part, s);
    if (st != MOE_OK || !row_w || P == 0) return st;
    hipLaunchKernelGGL(dp_reduce_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0, s, dp_part,
                       static_cast<int>((F + kTile - 1) / kTile), P, grad_row_w);
    return check_launch("moe_grouped_ffn_bwd_recompute dp");
}
