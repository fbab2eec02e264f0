// Expert computation: one grouped GEMM launch per projection over all
// experts' ragged segments ("Scalable Training of Mixture-of-Experts Models
// with Megatron Core", section 2.1 stage 3: all local experts in a single
// grouped GEMM call). SwiGLU experts without bias ("Mixture-of-Experts from
// Architecture to Large-Scale Training", section 2.5: gate, up and down
// matrices) or GELU(erf) experts with biases ("emerging-techniques-moe-
// training", Quick Start).
//
// bf16 kernel, CDNA4 (gfx950), one persistent launch per projection:
// - every expert segment (and the shared expert's rows) is cut into tiles of
//   256 token rows (the last one shorter); tiles are 256 weight rows wide; the
//   tile list is built on the device from the segment offsets, numbered
//   m-fastest (consecutive tiles share a weight panel) and mapped so that the
//   blocks of one XCD take consecutive tiles (their shared panels stay in that
//   XCD's L2);
// - 4 waves per block, one per SIMD, each with a 128 x 128 (or, for tiles of
//   at most 128 token rows, 64 x 128) slice of v_mfma_f32_32x32x16_bf16
//   accumulators in AGPRs; the weight tile is the MFMA "A" operand, so a
//   lane's accumulators are runs of 4 consecutive output columns of one token
//   row;
// - operands move global -> VGPR -> LDS one k-step ahead of their use, with
//   the LDS reads, LDS writes and global loads of a k-step interleaved
//   between its MFMAs (details at the kernel);
// - SwiGLU: the weight tile interleaves 32-row blocks of gate rows and up rows
//   of the same 32 output columns, so each lane holds the gate and up values
//   of the same output element and applies silu(g) * u in registers; GELU and
//   biases are applied in the same epilogue.
#include "gemm_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Tile: 256 weight rows (n) x up to 256 token rows (m), 4 waves (256
// threads, one wave per SIMD). Full tiles (more than 128 token rows): wave w
// owns weight rows [128 (w%2), +128) and token rows [128 (w/2), +128), i.e.
// 4 x 4 MFMA subtiles of 32 x 32 (256 accumulators). Half tiles (at most 128
// token rows): wave w owns weight rows [64 w, +64) and token rows [0, 128),
// 2 x 4 subtiles. Token rows past the tile's count are computed from a
// clamped (valid) row and never stored.
//
// MFMA v_mfma_f32_32x32x16_bf16: lane l supplies row l%32, k = 8(l/32)..+7
// of each operand; accumulator element i of lane l is row
// 8(i/4) + 4(l/32) + i%4 (weight row) and column l%32 (token row).
//
// k-steps of kBK = 64: an LDS stage holds 256 weight rows and 256 token rows
// of 64 bf16 (128-byte rows, eight 16-byte chunks; chunk c of row r sits at
// chunk c ^ ((r >> 1) & 7), which keeps both the 16-byte row-chunk writes and
// the MFMA fragment reads free of bank conflicts). Two stages alternate. Each
// thread moves 8 weight chunks and 8 (half tile: 4) token chunks per k-step,
// rows rb + 32 j, chunk tid % 8, with raw buffer loads (a uniform base per
// tile and a 32-bit per-lane offset) into VGPRs, then ds_write_b128.
//
// One k-step t reads stage t%2 in four quarters (k = 16 each). Fragments for
// quarter q+1 are read during the MFMAs of quarter q. During quarters 1 and
// 2 the VGPRs holding k-step t+1 are written to stage (t+1)%2 and refilled
// with k-step t+2 from global memory, so a global load has about one k-step
// of MFMA work to land. After quarter 2: wait for this wave's LDS traffic,
// s_barrier (stage (t+1)%2 complete, stage t%2 no longer read), then the
// MFMAs of quarter 3 run while quarter 0 of the next stage is read.
// sched_group_barrier fixes the interleaving inside each quarter; the last
// k-step of a tile runs the same code (its extra loads re-read the last
// k-step, its extra writes go to a stage nobody reads again).
constexpr int kBK = 64;
constexpr int kTile = 256;
constexpr int kRegion = kTile * kBK;   // elements of one operand region of a stage
constexpr int kStage = 2 * kRegion;

__device__ __forceinline__ int swz(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 7)) << 3); }

// Epilogue of a tile: bias, activation, rounding, stores (C and, for SwiGLU
// with a.GU, the pre-activations). acc as laid out by gemm_tile; JONLY >= 0:
// token subtile JONLY of the wave only.
template <int MODE, bool HALF, int JONLY = -1>
__device__ __forceinline__ void store_tile(const GGArgs &a, const TileInfo &ti,
                                           floatx16 (&acc)[HALF ? 2 : 4][4], int wave, int lane);

// Split workspace: an int header of 64 KB ([0..2] the plan: split tiles,
// pieces per tile, k-steps per piece; from int 64, 8 ints per split tile:
// seg, m0, n_tile, M, row0, shared), then fp32 partial tiles of kPartFloats
// each, piece p of split tile t at index t * s + p.
constexpr int kWsHeaderFloats = 16384;
constexpr int kWsMaxSplitTiles = (kWsHeaderFloats - 64) / 8;
constexpr int kPartFloats = 256 * 256;

// One tile over k-steps [k0, k0 + nks), then the epilogue; or, for a piece
// of a split tile (part != null), its raw fp32 accumulators to part:
// element e = 16 (i*4 + j) + q of thread tid's accumulators, in float4
// groups, at float4 index (e/4) * 256 + tid.
template <int MODE, bool ODD, bool HALF>
__device__ __forceinline__ void gemm_tile(const GGArgs &a, const TileInfo &ti, bf16_t *LB0, bf16_t *LB1,
                                          int k0, int nks, float *part) {
    constexpr int NI = HALF ? 2 : 4;    // 32-row weight subtiles per wave
    constexpr int NJ = 4;               // 32-row token subtiles per wave
    constexpr int XJ = HALF ? 4 : 8;    // token chunks per thread per k-step
    constexpr int NMF = NI * NJ;        // MFMAs per quarter
    constexpr int NRD = NI + NJ;        // fragment reads per quarter
    constexpr int NWR = 4 + XJ / 2;     // chunk writes (and loads) per heavy quarter
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    // uniform by construction; say so, so that they live in SGPRs (buffer
    // load offsets and loop bounds)
    k0 = __builtin_amdgcn_readfirstlane(k0);
    const int K = a.K, nk = __builtin_amdgcn_readfirstlane(nks);
    const int chunk = tid & 7, rb = tid >> 3;
    const int so = swz(rb, chunk);      // + 32 j rows: same swizzle
    const int rows = min(kTile, ti.M - ti.m0);
    const int nb_rows = (MODE & 7) == kModeSwiGLU ? 2 * a.N_out : a.N_out;

    const bf16_t *wseg = ti.shared ? static_cast<const bf16_t *>(a.B_sh)
                                   : static_cast<const bf16_t *>(a.B) + static_cast<int64_t>(ti.seg) * nb_rows * K;
    // token rows: rows m0.. of the segment, or (gather) the rows of A that
    // a.gather names for them; a resource over all of A then, so that an
    // out-of-range index reads zeros instead of faulting
    const bool gather = a.gather != nullptr && !ti.shared;
    const bf16_t *xbase = gather ? static_cast<const bf16_t *>(a.A)
                                 : (ti.shared ? static_cast<const bf16_t *>(a.A_sh)
                                              : static_cast<const bf16_t *>(a.A) + static_cast<int64_t>(ti.row0) * K) +
                                       static_cast<int64_t>(ti.m0) * K;
    // weight rows of the tile: SwiGLU j even -> gate rows f, j odd -> up rows
    // N_out + f, f = n_tile*128 + (j/2)*32 + rb; plain: n_tile*256 + rb + 32 j
    const int wfirst = (MODE & 7) == kModeSwiGLU ? ti.n_tile * (kTile / 2) : ti.n_tile * kTile;
    const __amdgpu_buffer_rsrc_t rwg = make_rsrc(wseg + static_cast<int64_t>(wfirst) * K);
    const __amdgpu_buffer_rsrc_t rwu =
        make_rsrc(wseg + static_cast<int64_t>((MODE & 7) == kModeSwiGLU ? a.N_out + wfirst : wfirst) * K);
    const __amdgpu_buffer_rsrc_t rx =
        gather ? make_rsrc(xbase, static_cast<uint32_t>(a.a_rows) * static_cast<uint32_t>(K) * 2u) : make_rsrc(xbase);
    int wv[8], xv[XJ];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int rl = (MODE & 7) == kModeSwiGLU ? (j >> 1) * 32 + rb : rb + 32 * j;   // row past the base
        const int lim = (MODE & 7) == kModeSwiGLU ? a.N_out : nb_rows;
        wv[j] = ((wfirst + rl < lim ? rl : 0) * K + chunk * 8) * 2;            // base row is valid
    }
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
        const int r = rb + 32 * j;
        int m = r < rows ? r : rows - 1;
        if (gather) m = a.gather[ti.row0 + ti.m0 + m];
        xv[j] = (m * K + chunk * 8) * 2;
    }

    floatx16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    u32x4 RW[8], RX[XJ];
    bf16x8_t fa0[NI], fb0[NJ], fa1[NI], fb1[NJ];

#define MOE_LD(KT, H)                                                                           \
    do {                                                                                      \
        _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                          \
            RW[j] = __builtin_amdgcn_raw_buffer_load_b128((j & 1) ? rwu : rwg, wv[j], (k0 + (KT)) * kBK * 2, 0); \
        _Pragma("unroll") for (int j = (XJ / 2) * (H); j < (XJ / 2) * (H) + XJ / 2; ++j)      \
            RX[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xv[j], (k0 + (KT)) * kBK * 2, 0); \
    } while (0)
#define MOE_WR(LB, H)                                                                           \
    do {                                                                                      \
        _Pragma("unroll") for (int j = 4 * (H); j < 4 * (H) + 4; ++j)                          \
            *reinterpret_cast<u32x4 *>((LB) + so + j * 32 * kBK) = RW[j];                      \
        _Pragma("unroll") for (int j = (XJ / 2) * (H); j < (XJ / 2) * (H) + XJ / 2; ++j)      \
            *reinterpret_cast<u32x4 *>((LB) + kRegion + so + j * 32 * kBK) = RX[j];           \
    } while (0)
#define MOE_RD(FA, FB, LB, KS)                                                                  \
    do {                                                                                      \
        const int ch_ = (KS) * 2 + lhi;                                                       \
        _Pragma("unroll") for (int i = 0; i < NI; ++i)                                        \
            FA[i] = *reinterpret_cast<const bf16x8_t *>((LB) + swz(wrow0 + i * 32 + l32, ch_)); \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                        \
            FB[j] = *reinterpret_cast<const bf16x8_t *>((LB) + kRegion + swz(tok0 + j * 32 + l32, ch_)); \
    } while (0)
#define MOE_MF(FA, FB)                                                                          \
    do {                                                                                      \
        _Pragma("unroll") for (int i = 0; i < NI; ++i)                                        \
            _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                    \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[i], FB[j], acc[i][j], 0, 0, 0); \
    } while (0)
// quarter with fragment reads only
#define MOE_PAT_LIGHT()                                                                         \
    do {                                                                                      \
        _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                     \
            MOE_SGB(kSgMfma, 1);                                                              \
            if ((HALF && q < NRD) || (!HALF && (q & 1))) MOE_SGB(kSgDsRead, 1);               \
        }                                                                                     \
    } while (0)
// quarter with fragment reads, chunk writes and global loads
#define MOE_PAT_HEAVY()                                                                         \
    do {                                                                                      \
        _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                     \
            MOE_SGB(kSgMfma, 1);                                                              \
            if (HALF) {                                                                       \
                if (q < NRD) MOE_SGB(kSgDsRead, 1);                                           \
                if (q < NWR) { MOE_SGB(kSgDsWrite, 1); MOE_SGB(kSgVmemRead, 1); }             \
            } else if (q & 1) {                                                               \
                MOE_SGB(kSgDsWrite, 1); MOE_SGB(kSgVmemRead, 1);                              \
            } else {                                                                          \
                MOE_SGB(kSgDsRead, 1);                                                        \
            }                                                                                 \
        }                                                                                     \
    } while (0)
#define MOE_STEP(CUR, NXT, T)                                                                   \
    do {                                                                                      \
        const int kk_ = (T) + 2 < nk ? (T) + 2 : nk - 1;                                      \
        MOE_MF(fa0, fb0); MOE_RD(fa1, fb1, CUR, 1);                                           \
        MOE_PAT_LIGHT(); __builtin_amdgcn_sched_barrier(0);                                   \
        MOE_MF(fa1, fb1); MOE_RD(fa0, fb0, CUR, 2); MOE_WR(NXT, 0); MOE_LD(kk_, 0);           \
        MOE_PAT_HEAVY(); __builtin_amdgcn_sched_barrier(0);                                   \
        MOE_MF(fa0, fb0); MOE_RD(fa1, fb1, CUR, 3); MOE_WR(NXT, 1); MOE_LD(kk_, 1);           \
        MOE_PAT_HEAVY(); __builtin_amdgcn_sched_barrier(0);                                   \
        MOE_LDS_BARRIER();                                                                    \
        MOE_MF(fa1, fb1); MOE_RD(fa0, fb0, NXT, 0);                                           \
        MOE_PAT_LIGHT(); __builtin_amdgcn_sched_barrier(0);                                   \
    } while (0)

    // prologue: k-step 0 into stage 0, k-step 1 into the VGPRs
    MOE_LD(0, 0);
    MOE_LD(0, 1);
    MOE_LDS_BARRIER();   // every wave is done reading the previous tile's stages
    MOE_WR(LB0, 0);
    MOE_WR(LB0, 1);
    {
        // issued one by one in the loop's order: the wait counter counts
        // loads in issue order, and the loop's waits are derived from the
        // order these arrive in at its first iteration (any other order here
        // makes every iteration wait for loads issued a quarter earlier)
        const int k1 = nk > 1 ? 1 : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 4 * h; j < 4 * h + 4; ++j) {
                RW[j] = __builtin_amdgcn_raw_buffer_load_b128((j & 1) ? rwu : rwg, wv[j], (k0 + k1) * kBK * 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = (XJ / 2) * h; j < (XJ / 2) * h + XJ / 2; ++j) {
                RX[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xv[j], (k0 + k1) * kBK * 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    MOE_LDS_BARRIER();
    MOE_RD(fa0, fb0, LB0, 0);
    if (ODD) {
        for (int t = 0; t + 1 < nk; t += 2) {
            MOE_STEP(LB0, LB1, t);
            MOE_STEP(LB1, LB0, t + 1);
        }
        MOE_STEP(LB0, LB1, nk - 1);
    } else {
        for (int t = 0; t < nk; t += 2) {
            MOE_STEP(LB0, LB1, t);
            MOE_STEP(LB1, LB0, t + 1);
        }
    }
#undef MOE_LD
#undef MOE_WR
#undef MOE_RD
#undef MOE_MF
#undef MOE_PAT_LIGHT
#undef MOE_PAT_HEAVY
#undef MOE_STEP

    if (part) {
        float4 *P4 = reinterpret_cast<float4 *>(part);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    P4[((i * NJ + j) * 4 + q) * 256 + tid] =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        return;
    }
    store_tile<MODE, HALF>(a, ti, acc, wave, lane);
}

template <int MODE, bool HALF, int JONLY>
__device__ __forceinline__ void store_tile(const GGArgs &a, const TileInfo &ti,
                                           floatx16 (&acc)[HALF ? 2 : 4][4], int wave, int lane) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    const int rows = min(kTile, ti.M - ti.m0);
    const int nb_rows = (MODE & 7) == kModeSwiGLU ? 2 * a.N_out : a.N_out;
    const int64_t crow0 = static_cast<int64_t>(ti.row0) + ti.m0;
    bf16_t *Cseg = ti.shared ? static_cast<bf16_t *>(a.C_sh) + static_cast<int64_t>(ti.m0) * a.N_out
                             : static_cast<bf16_t *>(a.C) + crow0 * a.N_out;
    // pre-activations kept for the backward: SwiGLU [rows][2 N_out] (g, u),
    // GELU [rows][N_out] (with the bias)
    bf16_t *GUseg = nullptr;
    if ((MODE & 7) == kModeSwiGLU || (MODE & 7) == kModeGELU) {
        const int gw = (MODE & 7) == kModeSwiGLU ? 2 * a.N_out : a.N_out;
        if (ti.shared)
            GUseg = a.GU_sh ? static_cast<bf16_t *>(a.GU_sh) + static_cast<int64_t>(ti.m0) * gw : nullptr;
        else
            GUseg = a.GU ? static_cast<bf16_t *>(a.GU) + crow0 * gw : nullptr;
    }
    const bf16_t *bias = (a.bias && !ti.shared)
                             ? static_cast<const bf16_t *>(a.bias) + static_cast<int64_t>(ti.seg) * nb_rows
                             : nullptr;
    const float *roww = (MODE & kRowW) && !ti.shared ? a.row_w + crow0 : nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (JONLY >= 0 && j != JONLY) continue;
        const int m = tok0 + j * 32 + l32;
        if (m >= rows) continue;
        const float rw = roww ? roww[m] : 1.0f;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int nl = 8 * gq + 4 * lhi;   // row offset inside a 32-row subtile
            if ((MODE & 7) == kModeSwiGLU) {
#pragma unroll
                for (int p = 0; p < NI / 2; ++p) {
                    const int f = ti.n_tile * (kTile / 2) + wrow0 / 2 + p * 32 + nl;
                    if (f >= a.N_out) continue;
                    float g[4], u[4], hv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        g[q] = acc[2 * p][j][4 * gq + q];
                        u[q] = acc[2 * p + 1][j][4 * gq + q];
                        if (bias) {
                            g[q] += bf16_to_f32(bias[f + q]);
                            u[q] += bf16_to_f32(bias[a.N_out + f + q]);
                        }
                        hv[q] = silu_fast(g[q]) * u[q] * rw;
                    }
                    uint2 o;
                    o.x = pack_bf16x2(hv[0], hv[1]);
                    o.y = pack_bf16x2(hv[2], hv[3]);
                    *reinterpret_cast<uint2 *>(Cseg + static_cast<int64_t>(m) * a.N_out + f) = o;
                    if (GUseg) {
                        uint2 og, ou;
                        og.x = pack_bf16x2(g[0], g[1]);
                        og.y = pack_bf16x2(g[2], g[3]);
                        ou.x = pack_bf16x2(u[0], u[1]);
                        ou.y = pack_bf16x2(u[2], u[3]);
                        bf16_t *gr = GUseg + static_cast<int64_t>(m) * 2 * a.N_out;
                        *reinterpret_cast<uint2 *>(gr + f) = og;
                        *reinterpret_cast<uint2 *>(gr + a.N_out + f) = ou;
                    }
                }
            } else if ((MODE & 7) == kModeF32Out) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int n = ti.n_tile * kTile + wrow0 + i * 32 + nl;
                    if (n >= a.N_out) continue;
                    float *Cf = static_cast<float *>(a.C) + (crow0 + m) * a.N_out + n;
                    if (n + 4 <= a.N_out && (a.N_out & 3) == 0) {
                        *reinterpret_cast<float4 *>(Cf) = make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1],
                                                                      acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (n + q < a.N_out) Cf[q] = acc[i][j][4 * gq + q];
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int n = ti.n_tile * kTile + wrow0 + i * 32 + nl;
                    if (n >= a.N_out) continue;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[q] = acc[i][j][4 * gq + q];
                        if (bias) v[q] += bf16_to_f32(bias[n + q]);
                    }
                    if ((MODE & 7) == kModeGELU) {
                        if (GUseg) {
                            uint2 og;
                            og.x = pack_bf16x2(v[0], v[1]);
                            og.y = pack_bf16x2(v[2], v[3]);
                            *reinterpret_cast<uint2 *>(GUseg + static_cast<int64_t>(m) * a.N_out + n) = og;
                        }
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = gelu_erf_f(v[q]) * rw;
                    }
                    uint2 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(Cseg + static_cast<int64_t>(m) * a.N_out + n) = o;
                }
            }
        }
    }
}

// Work split. With T tiles and G persistent blocks, floor(T / G) rounds run
// whole tiles. When a workspace is given and the last round would leave at
// least half of the blocks idle, its rem tiles are cut along k into s pieces
// of ps k-steps each (ps even), so that the last round keeps up to G blocks
// busy; split_reduce then sums each tile's pieces in piece order
// (deterministic) and runs the epilogue. Every block derives the same plan
// from the segment offsets.
struct SplitPlan {
    int full, s, ps, items;   // whole tiles, pieces per split tile, k-steps per piece, work items
};

__device__ __forceinline__ SplitPlan split_plan(const GGArgs &a, int total, int nk, bool odd) {
    SplitPlan p{total, 0, 0, total};
    const int G = a.grid, rem = total % G;
    if (odd || a.ws == nullptr || rem == 0 || 2 * rem > G || nk < 4) return p;
    int s = min(G / rem, nk / 2);
    const int ps = 2 * ((nk + 2 * s - 1) / (2 * s));
    s = (nk + ps - 1) / ps;
    if (s < 2 || rem * s > a.ws_tiles || rem > kWsMaxSplitTiles) return p;
    p.full = total - rem;
    p.s = s;
    p.ps = ps;
    p.items = p.full + rem * s;
    return p;
}

// ODD: the number of k-steps K / 64 is odd (no split then).
template <int MODE, bool ODD>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16(GGArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t LB0[kStage];
    __shared__ __attribute__((aligned(16))) bf16_t LB1[kStage];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    const int total = __builtin_amdgcn_readfirstlane(build_tile_prefix(a, kTile, s_cum, s_tmp));
    const int nk = a.K / kBK;
    const SplitPlan sp = split_plan(a, total, nk, ODD);
    int *hdr = reinterpret_cast<int *>(a.ws);
    if (hdr && blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[0] = sp.s ? total - sp.full : 0;
        hdr[1] = sp.s;
        hdr[2] = sp.ps;
    }
    for (int w = xcd_block_index(blockIdx.x, a.grid); w < sp.items; w += a.grid) {
        int L = w, k0 = 0, nks = nk;
        float *part = nullptr;
        if (sp.s && w >= sp.full) {
            const int q = w - sp.full;
            L = sp.full + q / sp.s;
            k0 = (q % sp.s) * sp.ps;
            nks = min(sp.ps, nk - k0);
            part = a.ws + kWsHeaderFloats + static_cast<int64_t>(q) * kPartFloats;
        }
        const TileInfo ti = decode_tile(a, s_cum, L, kTile);
        if (part && k0 == 0 && threadIdx.x == 0) {
            int *d = hdr + 64 + (L - sp.full) * 8;
            d[0] = ti.seg;
            d[1] = ti.m0;
            d[2] = ti.n_tile;
            d[3] = ti.M;
            d[4] = ti.row0;
            d[5] = ti.shared ? 1 : 0;
        }
        if (ti.M - ti.m0 > kTile / 2) gemm_tile<MODE, ODD, false>(a, ti, LB0, LB1, k0, nks, part);
        else gemm_tile<MODE, ODD, true>(a, ti, LB0, LB1, k0, nks, part);
    }
}

// Token subtile J of wave `wave` of a split tile: sum of the pieces (piece
// order), then that subtile's epilogue.
template <int MODE, bool HALF, int J>
__device__ __forceinline__ void reduce_subtile(const GGArgs &a, const TileInfo &ti, const float4 *P4, int s,
                                               int wave, int lane) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int tid = wave * 64 + lane;
    floatx16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][J][q] = 0.0f;
    for (int p = 0; p < s; ++p) {
        const float4 *Pp = P4 + static_cast<int64_t>(p) * (kPartFloats / 4);
        float4 v[NI][4];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[i][q] = Pp[((i * NJ + J) * 4 + q) * 256 + tid];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[i][J][4 * q] += v[i][q].x;
                acc[i][J][4 * q + 1] += v[i][q].y;
                acc[i][J][4 * q + 2] += v[i][q].z;
                acc[i][J][4 * q + 3] += v[i][q].w;
            }
    }
    store_tile<MODE, HALF, J>(a, ti, acc, wave, lane);
}

// Sum of every split tile's pieces, in piece order, into piece 0 (one
// float4 per thread, all tiles' positions spread over the grid).
__global__ __launch_bounds__(256) void split_sum_kernel(GGArgs a) {
    const int *hdr = reinterpret_cast<const int *>(a.ws);
    const int rem = hdr[0], s = hdr[1];
    if (s < 2) return;
    constexpr int kQ = kPartFloats / 4;
    const int64_t n = static_cast<int64_t>(rem) * kQ;
    float4 *P4 = reinterpret_cast<float4 *>(a.ws + kWsHeaderFloats);
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t t = i / kQ, f = i - t * kQ;
        float4 *base = P4 + t * s * kQ + f;
        float4 acc = base[0];
        for (int p = 1; p < s; ++p) {
            const float4 v = base[static_cast<int64_t>(p) * kQ];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        base[0] = acc;
    }
}

// Block b: split tile b / 16, wave (b / 4) % 4, token subtile b % 4 (the
// pieces already summed into piece 0 by split_sum_kernel).
template <int MODE>
__global__ __launch_bounds__(64) void split_reduce(GGArgs a) {
    const int *hdr = reinterpret_cast<const int *>(a.ws);
    const int rem = hdr[0], s = hdr[1];
    const int t = blockIdx.x >> 4, wave = (blockIdx.x >> 2) & 3, J = blockIdx.x & 3;
    if (s == 0 || t >= rem) return;
    const int *d = hdr + 64 + t * 8;
    TileInfo ti;
    ti.seg = d[0];
    ti.m0 = d[1];
    ti.n_tile = d[2];
    ti.M = d[3];
    ti.row0 = d[4];
    ti.shared = d[5] != 0;
    const float4 *P4 = reinterpret_cast<const float4 *>(a.ws + kWsHeaderFloats) +
                       static_cast<int64_t>(t) * s * (kPartFloats / 4);
    const bool half = ti.M - ti.m0 <= kTile / 2;
    const int s1 = 1;   // summed into piece 0
    const int lane = threadIdx.x;
    switch (J) {
    case 0:
        if (half) reduce_subtile<MODE, true, 0>(a, ti, P4, s1, wave, lane);
        else reduce_subtile<MODE, false, 0>(a, ti, P4, s1, wave, lane);
        break;
    case 1:
        if (half) reduce_subtile<MODE, true, 1>(a, ti, P4, s1, wave, lane);
        else reduce_subtile<MODE, false, 1>(a, ti, P4, s1, wave, lane);
        break;
    case 2:
        if (half) reduce_subtile<MODE, true, 2>(a, ti, P4, s1, wave, lane);
        else reduce_subtile<MODE, false, 2>(a, ti, P4, s1, wave, lane);
        break;
    default:
        if (half) reduce_subtile<MODE, true, 3>(a, ti, P4, s1, wave, lane);
        else reduce_subtile<MODE, false, 3>(a, ti, P4, s1, wave, lane);
        break;
    }
}

// fp32 grouped GEMM (the fp32 layer): v_mfma_f32_16x16x4_f32, 64 x 64 tiles,
// 16 deep, single-buffered LDS with padded rows.
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GGArgs a) {
    constexpr int BM = 64, BN = 64, BK = 16, LD = BK + 1;
    constexpr int NT = 2, MT = 2;   // wave tile 32 x 32
    __shared__ float sw[BN * LD];
    __shared__ float sx[BM * LD];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int total = build_tile_prefix(a, BM, s_cum, s_tmp);
    const int nb_rows = (MODE & 7) == kModeSwiGLU ? 2 * a.N_out : a.N_out;
    const int BN_out = (MODE & 7) == kModeSwiGLU ? BN / 2 : BN;
    const int K = a.K;
    const int r = tid >> 2, c4 = (tid & 3) * 4;

    for (int L = xcd_block_index(blockIdx.x, a.grid); L < total; L += a.grid) {
        const TileInfo ti = decode_tile(a, s_cum, L, BM);
        const float *Aseg = ti.shared ? static_cast<const float *>(a.A_sh)
                                      : static_cast<const float *>(a.A) + static_cast<int64_t>(ti.row0) * K;
        const float *Bseg = ti.shared ? static_cast<const float *>(a.B_sh)
                                      : static_cast<const float *>(a.B) + static_cast<int64_t>(ti.seg) * nb_rows * K;
        int wrow;
        if ((MODE & 7) == kModeSwiGLU) {
            const int blk = r >> 4;
            const int f = ti.n_tile * (BN / 2) + (blk >> 1) * 16 + (r & 15);
            wrow = (blk & 1) ? a.N_out + f : f;
            if (f >= a.N_out) wrow = 0;
        } else {
            wrow = ti.n_tile * BN + r;
            if (wrow >= nb_rows) wrow = 0;
        }
        int m = ti.m0 + r;
        if (m >= ti.M) m = ti.M - 1;
        const float *gw = Bseg + static_cast<int64_t>(wrow) * K + c4;
        const float *gx = Aseg + static_cast<int64_t>(m) * K + c4;
        if (a.gather && !ti.shared) {
            // gathered token row (indices checked on the device: out of range reads row 0)
            int src = a.gather[ti.row0 + m];
            if (src < 0 || src >= a.a_rows) src = 0;
            gx = static_cast<const float *>(a.A) + static_cast<int64_t>(src) * K + c4;
        }

        floatx4 acc[NT][MT];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < MT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < K; k0 += BK) {
            const float4 vw = *reinterpret_cast<const float4 *>(gw + k0);
            const float4 vx = *reinterpret_cast<const float4 *>(gx + k0);
            __syncthreads();
            sw[r * LD + c4 + 0] = vw.x; sw[r * LD + c4 + 1] = vw.y;
            sw[r * LD + c4 + 2] = vw.z; sw[r * LD + c4 + 3] = vw.w;
            sx[r * LD + c4 + 0] = vx.x; sx[r * LD + c4 + 1] = vx.y;
            sx[r * LD + c4 + 2] = vx.z; sx[r * LD + c4 + 3] = vx.w;
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BK; kk += 4) {
                float af[NT], bfv[MT];
#pragma unroll
                for (int i = 0; i < NT; ++i) af[i] = sw[(wn * 32 + i * 16 + (lane & 15)) * LD + kk + (lane >> 4)];
#pragma unroll
                for (int j = 0; j < MT; ++j) bfv[j] = sx[(wm * 32 + j * 16 + (lane & 15)) * LD + kk + (lane >> 4)];
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int j = 0; j < MT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfv[j], acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();

        float *Cseg = ti.shared ? static_cast<float *>(a.C_sh)
                                : static_cast<float *>(a.C) + static_cast<int64_t>(ti.row0) * a.N_out;
        float *GUseg = nullptr;
        if ((MODE & 7) == kModeSwiGLU || (MODE & 7) == kModeGELU) {
            const int gw = (MODE & 7) == kModeSwiGLU ? 2 * a.N_out : a.N_out;
            GUseg = ti.shared ? static_cast<float *>(a.GU_sh)
                              : (a.GU ? static_cast<float *>(a.GU) + static_cast<int64_t>(ti.row0) * gw : nullptr);
        }
        const float *bias = (a.bias && !ti.shared)
                                ? static_cast<const float *>(a.bias) + static_cast<int64_t>(ti.seg) * nb_rows
                                : nullptr;
        const float *roww = (MODE & kRowW) && !ti.shared ? a.row_w + ti.row0 : nullptr;
        const int ng = lane >> 4;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int mm = ti.m0 + wm * 32 + j * 16 + (lane & 15);
            if (mm >= ti.M) continue;
            const float rw = roww ? roww[mm] : 1.0f;
            if ((MODE & 7) == kModeSwiGLU) {
                const int f = ti.n_tile * BN_out + wn * 16 + 4 * ng;
                if (f >= a.N_out) continue;
                float4 hv, gv, uv;
                float *hp = &hv.x, *gp = &gv.x, *up = &uv.x;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float g = acc[0][j][i], u = acc[1][j][i];
                    if (bias) {
                        g += bias[f + i];
                        u += bias[a.N_out + f + i];
                    }
                    gp[i] = g;
                    up[i] = u;
                    hp[i] = silu_f(g) * u * rw;
                }
                *reinterpret_cast<float4 *>(Cseg + static_cast<int64_t>(mm) * a.N_out + f) = hv;
                if (GUseg) {
                    float *gr = GUseg + static_cast<int64_t>(mm) * 2 * a.N_out;
                    *reinterpret_cast<float4 *>(gr + f) = gv;
                    *reinterpret_cast<float4 *>(gr + a.N_out + f) = uv;
                }
            } else {
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const int n = ti.n_tile * BN + wn * 32 + i * 16 + 4 * ng;
                    if (n >= a.N_out) continue;
                    float4 o, pre;
                    float *op = &o.x, *pp = &pre.x;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = acc[i][j][q];
                        if (bias) v += bias[n + q];
                        pp[q] = v;
                        if ((MODE & 7) == kModeGELU) v = gelu_erf_f(v) * rw;
                        op[q] = v;
                    }
                    *reinterpret_cast<float4 *>(Cseg + static_cast<int64_t>(mm) * a.N_out + n) = o;
                    if ((MODE & 7) == kModeGELU && GUseg)
                        *reinterpret_cast<float4 *>(GUseg + static_cast<int64_t>(mm) * a.N_out + n) = pre;
                }
            }
        }
    }
}

template <int MODE>
int launch_gemm(GGArgs a, int dtype, int64_t P, hipStream_t s, const char *what) {
    const int S = a.E + (a.M_sh > 0 ? 1 : 0);
    int64_t upper;
    if (dtype == MOE_DTYPE_BF16) {
        const int BNo = (MODE & 7) == kModeSwiGLU ? 128 : 256;
        a.n_tiles = (a.N_out + BNo - 1) / BNo;
        upper = ((P + a.M_sh) / 256 + S) * static_cast<int64_t>(a.n_tiles);
    } else {
        const int BNo = (MODE & 7) == kModeSwiGLU ? 32 : 64;
        a.n_tiles = (a.N_out + BNo - 1) / BNo;
        upper = ((P + a.M_sh) / 64 + S) * static_cast<int64_t>(a.n_tiles);
    }
    int64_t grid = static_cast<int64_t>(num_cus()) * (dtype == MOE_DTYPE_BF16 ? 1 : 2);
    // with a split workspace every CU gets a block: a GEMM of few tiles is
    // then cut along k over the whole GPU (blocks without work exit)
    const bool splits = dtype == MOE_DTYPE_BF16 && a.ws && ((a.K / kBK) & 1) == 0;
    if (grid > upper && !splits) grid = upper;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    if (dtype == MOE_DTYPE_BF16) {
        if ((a.K / kBK) & 1) {
            a.ws = nullptr;
            hipLaunchKernelGGL((grouped_gemm_bf16<MODE, true>), dim3(a.grid), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((grouped_gemm_bf16<MODE, false>), dim3(a.grid), dim3(256), 0, s, a);
            if (a.ws) {
                const int st = check_launch(what);
                if (st != MOE_OK) return st;
                hipLaunchKernelGGL(split_sum_kernel, dim3(2048), dim3(256), 0, s, a);
                // at most grid / 2 split tiles, 16 blocks each
                hipLaunchKernelGGL((split_reduce<MODE>), dim3(16 * (a.grid / 2 > 0 ? a.grid / 2 : 1)), dim3(64),
                                   0, s, a);
            }
        }
    } else
        hipLaunchKernelGGL((grouped_gemm_f32<MODE>), dim3(a.grid), dim3(256), 0, s, a);
    return check_launch(what);
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {

size_t gemm_split_workspace_bytes() {
    return sizeof(float) * (static_cast<size_t>(kWsHeaderFloats) + static_cast<size_t>(num_cus()) * kPartFloats);
}

int gemm_bf16_f32out(const void *A, const void *B, int T, int K, int N, float *C, int32_t *offsets, void *ws,
                     size_t ws_bytes, hipStream_t s) {
    launch_fill<int32_t>(offsets, 1, 0, s);
    launch_fill<int32_t>(offsets + 1, 1, T, s);
    GGArgs g{};
    g.A = A;
    g.B = B;
    g.C = C;
    g.offsets = offsets;
    g.E = 1;
    g.N_out = N;
    g.K = K;
    const size_t hdr_bytes = sizeof(float) * kWsHeaderFloats, part_bytes = sizeof(float) * kPartFloats;
    if (ws && ws_bytes >= hdr_bytes + 2 * part_bytes) {
        g.ws = static_cast<float *>(ws);
        const size_t n = (ws_bytes - hdr_bytes) / part_bytes;
        g.ws_tiles = n > (size_t(1) << 20) ? (1 << 20) : static_cast<int>(n);
    }
    return launch_gemm<kModeF32Out>(g, MOE_DTYPE_BF16, T, s, "moe_route logits GEMM");
}

}  // namespace moe

extern "C" size_t moe_grouped_ffn_workspace_size(int dtype) {
    if (dtype != MOE_DTYPE_BF16) return 0;
    return sizeof(float) * (static_cast<size_t>(kWsHeaderFloats) +
                            static_cast<size_t>(num_cus()) * kPartFloats);
}

namespace {

int grouped_ffn(const void *x_perm, const int32_t *gather_rows, int64_t x_rows, int dtype, int64_t P, int64_t h,
                int64_t F, int E, const int32_t *offsets, int act_kind, const void *w1, const void *b1,
                const void *w2, const void *b2, const void *x_sh, int64_t T_sh, const void *w1_sh,
                const void *w2_sh, const float *row_w, void *act, void *gu, void *y, void *y_sh, void *workspace,
                size_t workspace_bytes, void *stream) {
    MOE_CHECK_ARG(offsets && w1 && w2 && (P == 0 || (act && y)), MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: null required pointer");
    MOE_CHECK_ARG(P == 0 || x_perm, MOE_ERR_INVALID_ARG, "moe_grouped_ffn: null x_perm");
    MOE_CHECK_ARG(gather_rows == nullptr || (x_rows > 0 && x_rows * h * 4 < (int64_t(1) << 31)),
                  gather_rows == nullptr || x_rows > 0 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: gathering needs 0 < x_rows and x_rows * h * 4 < 2^31");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: bad dtype %d", dtype);
    MOE_CHECK_ARG(act_kind == MOE_ACT_GELU || act_kind == MOE_ACT_SWIGLU, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: bad activation %d", act_kind);
    MOE_CHECK_ARG(P >= 0 && h > 0 && F > 0 && E > 0 && T_sh >= 0, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: bad sizes");
    MOE_CHECK_ARG(h % 64 == 0 && F % 64 == 0 && E <= 256, MOE_ERR_UNSUPPORTED,
                  "moe_grouped_ffn: need h %% 64 == 0, F %% 64 == 0, E <= 256");
    MOE_CHECK_ARG(P + T_sh < (int64_t(1) << 31) && h < (int64_t(1) << 20) && F < (int64_t(1) << 20),
                  MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: sizes too large");
    const bool has_sh = T_sh > 0;
    MOE_CHECK_ARG(!has_sh || (x_sh && w1_sh && w2_sh && y_sh), MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: shared expert needs x_sh, w1_sh, w2_sh and y_sh");
    MOE_CHECK_ARG(workspace_bytes == 0 || workspace, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: workspace_bytes > 0 with a null workspace");
    const void *ptrs[] = {x_perm, w1, b1, w2, b2, x_sh, w1_sh, w2_sh, act, gu, y, y_sh, workspace};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(p == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
    const int n1 = act_kind == MOE_ACT_SWIGLU ? 2 : 1;
    // split workspace: header plus at least two partial tiles, else unused
    const size_t hdr_bytes = sizeof(float) * kWsHeaderFloats, part_bytes = sizeof(float) * kPartFloats;
    float *ws = nullptr;
    int ws_tiles = 0;
    if (dtype == MOE_DTYPE_BF16 && workspace && workspace_bytes >= hdr_bytes + 2 * part_bytes) {
        ws = static_cast<float *>(workspace);
        const size_t n = (workspace_bytes - hdr_bytes) / part_bytes;
        ws_tiles = n > (size_t(1) << 20) ? (1 << 20) : static_cast<int>(n);
    }

    // first projection + activation
    GGArgs g1{};
    g1.A = x_perm;
    g1.gather = gather_rows;
    g1.a_rows = static_cast<int>(gather_rows ? x_rows : 0);
    g1.B = w1;
    g1.bias = b1;
    g1.C = act;
    g1.GU = gu;
    g1.M_sh = static_cast<int>(T_sh);
    g1.A_sh = x_sh;
    g1.B_sh = w1_sh;
    g1.C_sh = has_sh ? static_cast<char *>(act) + static_cast<size_t>(P) * F * es : nullptr;
    g1.GU_sh = (has_sh && gu) ? static_cast<char *>(gu) + static_cast<size_t>(P) * n1 * F * es : nullptr;
    g1.offsets = offsets;
    g1.row_w = row_w;
    g1.E = E;
    g1.N_out = static_cast<int>(F);
    g1.K = static_cast<int>(h);
    g1.ws = ws;
    g1.ws_tiles = ws_tiles;
    int st;
    if (row_w)
        st = act_kind == MOE_ACT_SWIGLU ? launch_gemm<kModeSwiGLU | kRowW>(g1, dtype, P, s, "moe_grouped_ffn gemm1")
                                        : launch_gemm<kModeGELU | kRowW>(g1, dtype, P, s, "moe_grouped_ffn gemm1");
    else
        st = act_kind == MOE_ACT_SWIGLU ? launch_gemm<kModeSwiGLU>(g1, dtype, P, s, "moe_grouped_ffn gemm1")
                                        : launch_gemm<kModeGELU>(g1, dtype, P, s, "moe_grouped_ffn gemm1");
    if (st != MOE_OK) return st;

    // second projection
    GGArgs g2{};
    g2.A = act;
    g2.B = w2;
    g2.bias = b2;
    g2.C = y;
    g2.M_sh = static_cast<int>(T_sh);
    g2.A_sh = g1.C_sh;
    g2.B_sh = w2_sh;
    g2.C_sh = y_sh;
    g2.offsets = offsets;
    g2.E = E;
    g2.N_out = static_cast<int>(h);
    g2.K = static_cast<int>(F);
    g2.ws = ws;
    g2.ws_tiles = ws_tiles;
    return launch_gemm<kModePlain>(g2, dtype, P, s, "moe_grouped_ffn gemm2");
}

}  // namespace

extern "C" int moe_grouped_ffn(const void *x_perm, const int32_t *gather_rows, int64_t x_rows, int dtype,
                               int64_t P, int64_t h, int64_t F,
                               int E, const int32_t *offsets, int act_kind, const void *w1,
                               const void *b1, const void *w2, const void *b2, const void *x_sh,
                               int64_t T_sh, const void *w1_sh, const void *w2_sh, void *act,
                               void *gu, void *y, void *y_sh, void *workspace,
                               size_t workspace_bytes, void *stream) {
    clear_error();
    return grouped_ffn(x_perm, gather_rows, x_rows, dtype, P, h, F, E, offsets, act_kind, w1, b1, w2, b2, x_sh,
                       T_sh, w1_sh, w2_sh, nullptr, act, gu, y, y_sh, workspace, workspace_bytes, stream);
}

extern "C" int moe_grouped_ffn_weighted(const void *x_perm, const int32_t *gather_rows, int64_t x_rows,
                                        int dtype, int64_t P, int64_t h, int64_t F, int E,
                                        const int32_t *offsets, int act_kind, const void *w1, const void *b1,
                                        const void *w2, const void *x_sh, int64_t T_sh, const void *w1_sh,
                                        const void *w2_sh, const float *row_w, void *act, void *gu, void *y,
                                        void *y_sh, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(P == 0 || row_w, MOE_ERR_INVALID_ARG, "moe_grouped_ffn_weighted: null row_w");
    return grouped_ffn(x_perm, gather_rows, x_rows, dtype, P, h, F, E, offsets, act_kind, w1, b1, w2, nullptr,
                       x_sh, T_sh, w1_sh, w2_sh, row_w, act, gu, y, y_sh, workspace, workspace_bytes, stream);
}
