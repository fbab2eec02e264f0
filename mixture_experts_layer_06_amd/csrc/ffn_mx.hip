// Expert computation in MXFP8 ("Scalable Training of Mixture-of-Experts
// Models with Megatron Core", section 5.3.3: activations and weights
// quantised in 1 x 32 blocks with E8M0 scales; E4M3 elements), on CDNA4's
// scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, which applies a
// block's E8M0 scale inside the product.
//
// * moe_mx_quantize: rows of K values (bf16 or fp32) to E4M3 codes and one
//   E8M0 scale per 32 consecutive values. Shared exponent of a block:
//   floor(log2 max|v|) - 8 (the largest element lands in [256, 512)),
//   clamped to [-127, 127]; elements v * 2^-exp rounded to nearest-even on
//   the E4M3 grid, saturated at 448. One thread per block of 32, in integer
//   and exact float operations only, so the codes are those of any correct
//   implementation of the same rule.
// * grouped_gemm_mx: the bf16 grouped kernel's design with fp8 operands:
//   a k-step is 128 fp8 values, i.e. the same 128-byte rows, 16-byte chunks,
//   LDS swizzle and global -> VGPR -> LDS staging; each k-step runs two
//   halves of 16 scaled MFMAs (k = 64 each). Operand layout of the
//   instruction (checked on the device): lane l supplies row l % 32; bytes
//   0-15 of lanes l and l + 32 hold the row's first block of 32 k values (k
//   0..15 and 16..31), bytes 16-31 its second block (32..47, 48..63), and the
//   scale of block b of row r comes from lane r + 32 b. So lane half g reads
//   chunks 4s + g and 4s + 2 + g of k-sub s and supplies the scale of block
//   2s + g. The four block scales of a row and k-step (one 4-byte word) are
//   staged through LDS with the k-step's data (both stages' scale blocks
//   ahead of their operand data), one word of weight rows and one of token
//   rows per thread; a lane reads its row's word, shifted right by 8 g bits,
//   so that k-sub s takes byte 2s (opsel 2s). Accumulators as in the bf16
//   kernel.
// * moe_grouped_ffn_mx: first projection with SwiGLU, whose epilogue
//   quantises the fp32 activation along F (and optionally also stores it in
//   bf16), then the second projection on those codes (bf16 expert outputs).
//   Tokens enter quantised along h, optionally gathered.
// * mx_gemm_rows / mx_gemm_kseg (for the backward in ffn_mx_bwd.hip): the
//   same tile body by token segments with an fp32 or bf16 epilogue, and by
//   per-expert k-ranges of shared operands (weight gradients, fp32).
#include <type_traits>

#include "mx_common.hpp"

namespace moe {
namespace {


// --------------------------------------------------------------- GEMM

constexpr int kMxBK = 128;                   // fp8 values (bytes) per k-step
constexpr int kMxTile = 256;
constexpr int kMxRegion = kMxTile * kMxBK;   // bytes of one operand region of a stage
constexpr int kMxStage = 2 * kMxRegion;
constexpr int kMxScaleBytes = 2 * kMxTile * 4;   // per stage: a scale word per weight row and per token row
constexpr int kModeF32T = 4;   // fp32 out, stored transposed (the k-segment products)

static_assert(kMxBK == 128, "mswz assumes 128-byte rows");

struct MXArgs {
    GGArgs g;              // A: weight codes [E][nb_rows][K]; tokens: g.A (codes, rows of the
                           // segments or, with g.gather, rows of the unpermuted tokens)
    const uint8_t *ws;     // weight scales [E][nb_rows][K/32]
    const uint8_t *xs;     // token scales, rows as g.A
};

// Weight row (within the expert) of LDS row r of tile n_tile.
template <int MODE>
__device__ __forceinline__ int weight_row(int n_tile, int r, int N_out) {
    if (MODE == kModeSwiGLU) {
        const int jb = r >> 5;
        const int f = n_tile * (kMxTile / 2) + (jb >> 1) * 32 + (r & 31);
        return f < N_out ? ((jb & 1) ? N_out + f : f) : 0;
    }
    const int n = n_tile * kMxTile + r;
    return n < N_out ? n : 0;
}

// Even spread of NRD fragment reads, NWR LDS writes and NLD global loads
// over the NMF MFMAs of a half k-step.
template <int NMF, int NRD, int NWR, int NLD, int Q = 0>
__device__ __forceinline__ void mx_sched() {
    if constexpr (Q < NMF) {
        MOE_SGB(kSgMfma, 1);
        constexpr int r = (Q + 1) * NRD / NMF - Q * NRD / NMF;
        if constexpr (r > 0) MOE_SGB(kSgDsRead, r);
        constexpr int w = (Q + 1) * NWR / NMF - Q * NWR / NMF;
        if constexpr (w > 0) MOE_SGB(kSgDsWrite, w);
        constexpr int l = (Q + 1) * NLD / NMF - Q * NLD / NMF;
        if constexpr (l > 0) MOE_SGB(kSgVmemRead, l);
        mx_sched<NMF, NRD, NWR, NLD, Q + 1>();
    }
}

// Epilogue of a SwiGLU tile (the first projection): the activation
// silu(g) * u of every output element in fp32, quantised at once, a
// 32-column block at a time, into the codes a.GU [rows][N_out] and the
// scales a.GU_sh [rows][N_out / 32] (GGArgs fields the fp8 kernels do not
// otherwise use; the argument block of the second projection's launch is
// then the same as without this epilogue). A lane
// holds 16 of a block's values for one token row (columns 8 gq + 4 lhi + q)
// and lane l ^ 32 the other 16, so the block maximum takes one exchange;
// each lane then stores 16 bytes of codes (after one more exchange, so that
// lane half 0 holds columns 0..15 and half 1 columns 16..31) and half 0 the
// scale byte. The bf16 activation is stored too when a.C is set.
template <bool HALF>
__device__ __forceinline__ void store_tile_mx_swiglu(const GGArgs &a, const TileInfo &ti,
                                                     floatx16 (&acc)[HALF ? 2 : 4][4], int wave, int lane,
                                                     int64_t crow0) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    const int rows = min(kMxTile, ti.M - ti.m0);
    bf16_t *Cseg = a.C ? static_cast<bf16_t *>(a.C) + crow0 * a.N_out : nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int m = tok0 + j * 32 + l32;
        if (m >= rows) continue;   // lanes l and l ^ 32 share m: both skip or neither
#pragma unroll
        for (int p = 0; p < NI / 2; ++p) {
            // first column of the 32-column block (N_out % 128 == 0: whole blocks)
            const int fb = ti.n_tile * (kMxTile / 2) + wrow0 / 2 + p * 32;
            float hv[16];
            float amax = 0.0f;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float v = silu_fast(acc[2 * p][j][4 * gq + q]) * acc[2 * p + 1][j][4 * gq + q];
                    hv[4 * gq + q] = v;
                    amax = fmaxf(amax, fabsf(v));
                }
            if (Cseg) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    uint2 o;
                    o.x = pack_bf16x2(hv[4 * gq], hv[4 * gq + 1]);
                    o.y = pack_bf16x2(hv[4 * gq + 2], hv[4 * gq + 3]);
                    *reinterpret_cast<uint2 *>(Cseg + static_cast<int64_t>(m) * a.N_out + fb + 8 * gq + 4 * lhi) = o;
                }
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int ex = mx_block_exponent(amax);
            uint32_t c[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                c[gq] = e4m3_word(ldexpf(hv[4 * gq], -ex), ldexpf(hv[4 * gq + 1], -ex), ldexpf(hv[4 * gq + 2], -ex),
                                  ldexpf(hv[4 * gq + 3], -ex));
            // half 0 keeps columns 0..15 (its gq 0, 1 and the partner's), half 1
            // columns 16..31 (gq 2, 3)
            const uint32_t r0 = __shfl_xor(lhi ? c[0] : c[2], 32);
            const uint32_t r1 = __shfl_xor(lhi ? c[1] : c[3], 32);
            u32x4 w;
            if (lhi) {
                w[0] = r0; w[1] = c[2]; w[2] = r1; w[3] = c[3];
            } else {
                w[0] = c[0]; w[1] = r0; w[2] = c[1]; w[3] = r1;
            }
            const int64_t row = crow0 + m;
            *reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(a.GU) + row * a.N_out + fb + 16 * lhi) = w;
            if (!lhi) static_cast<uint8_t *>(a.GU_sh)[row * (a.N_out / 32) + fb / 32] = static_cast<uint8_t>(ex + 127);
        }
    }
}

// Epilogue of a plain tile: the outputs in bf16 (the second projection), or
// in fp32 (kModeF32Out), at rows crow0 + m of C [.][N_out]. In fp32 the four
// stores that fill a row's 128-byte line (columns 8 gq + 4 lhi of one
// 32-column subtile) are issued back to back, so that L2 holds no partly
// written lines that it might write back twice.
template <int MODE, bool HALF>
__device__ __forceinline__ void store_tile_mx_plain(const GGArgs &a, const TileInfo &ti,
                                                    floatx16 (&acc)[HALF ? 2 : 4][4], int wave, int lane,
                                                    int64_t crow0) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    const int rows = min(kMxTile, ti.M - ti.m0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int m = tok0 + j * 32 + l32;
        if (m >= rows) continue;
        const int64_t e0 = (crow0 + m) * a.N_out;
        if constexpr (MODE == kModeF32Out) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int n0 = ti.n_tile * kMxTile + wrow0 + i * 32;
                if (n0 >= a.N_out) continue;   // N_out % 32 == 0: whole subtiles
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.C) + e0 + n0 + 8 * gq + 4 * lhi) =
                        make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                                    acc[i][j][4 * gq + 3]);
            }
        } else {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int nl = 8 * gq + 4 * lhi;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int n = ti.n_tile * kMxTile + wrow0 + i * 32 + nl;
                    if (n >= a.N_out) continue;
                    uint2 o;
                    o.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
                    o.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    *reinterpret_cast<uint2 *>(static_cast<bf16_t *>(a.C) + e0 + n) = o;
                }
            }
        }
    }
}

// Epilogue of a k-segment tile, stored transposed in fp32: the weight-slot
// row is the row of C (rows crow0 + n_tile * 256 + ...) and the token-slot
// row its column (pitch ti.M). A lane's accumulators run down one column, so
// each dword store writes two whole 128-byte lines (32 consecutive columns of
// rows r and r + 4), and the four stores of a row's 512 bytes follow each
// other. (Stored untransposed, each 16-byte store touched 32 rows.) The
// stores are non-temporal: nothing reads the gradients back in this pass.
template <bool HALF>
__device__ __forceinline__ void store_tile_mx_t(const GGArgs &a, const TileInfo &ti,
                                                floatx16 (&acc)[HALF ? 2 : 4][4], int wave, int lane,
                                                int64_t crow0) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    const int cols = min(kMxTile, ti.M - ti.m0);
    float *C = static_cast<float *>(a.C);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r0 = ti.n_tile * kMxTile + wrow0 + i * 32;
        if (r0 >= a.N_out) continue;   // N_out % 32 == 0: whole subtiles
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float *dst = C + (crow0 + r0 + 8 * gq + 4 * lhi + q) * ti.M + ti.m0 + tok0 + l32;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    if (tok0 + j * 32 + l32 < cols) __builtin_nontemporal_store(acc[i][j][4 * gq + q], dst + j * 32);
            }
    }
}

// The staging registers of one k-step: 8 weight chunks, XJ token chunks and
// the two scale words of this thread.
template <int XJ>
struct MxStage {
    u32x4 W[8], X[XJ];
    uint32_t S[2];
};

// A tile's operand sources: buffer resources over its weight rows, token
// rows and scale words (bounded to its valid rows, so rows past them read as
// zeros), this thread's offsets, and the k-step map (k-steps k0 + t for t <
// nreal, the zero k-step kzero after them). load_item issues staging item q
// of k-step kt: q < 8 the weight chunk q, then the token chunks, then the
// two scale words.
template <int MODE, bool HALF, bool GATHER>
struct MxTileSrc {
    static constexpr int XJ = HALF ? 4 : 8;
    static constexpr int NIT = 8 + XJ + 2;
    __amdgpu_buffer_rsrc_t rwg, rwu, rx, rws, rxs;
    int K, k0, nreal, kzero, wlane, wsr, xsr;
    int xv[GATHER ? XJ : 1];

    __device__ __forceinline__ MxTileSrc(const MXArgs &x, const TileInfo &ti, int k0_, int nreal_, int kzero_) {
        const GGArgs &a = x.g;
        const int tid = threadIdx.x;
        K = a.K;
        const int KS = K / 32;
        k0 = __builtin_amdgcn_readfirstlane(k0_);
        nreal = __builtin_amdgcn_readfirstlane(nreal_);
        kzero = __builtin_amdgcn_readfirstlane(kzero_);
        const int chunk = tid & 7, rb = tid >> 3;
        const int rows = min(kMxTile, ti.M - ti.m0);
        const int nb_rows = MODE == kModeSwiGLU ? 2 * a.N_out : a.N_out;
        const uint8_t *wseg = static_cast<const uint8_t *>(a.B) + static_cast<int64_t>(ti.seg) * nb_rows * K;
        const uint8_t *wsseg = x.ws + static_cast<int64_t>(ti.seg) * nb_rows * KS;
        // weight rows of the tile: SwiGLU j even -> gate rows wfirst + (j/2)*32 + rb,
        // j odd -> the up rows N_out + the same; plain: wfirst + 32 j + rb
        const int wfirst = MODE == kModeSwiGLU ? ti.n_tile * (kMxTile / 2) : ti.n_tile * kMxTile;
        const int wvalid = min(MODE == kModeSwiGLU ? kMxTile / 2 : kMxTile, a.N_out - wfirst);
        const uint32_t wbytes = static_cast<uint32_t>(wvalid) * static_cast<uint32_t>(K);
        rwg = make_rsrc(wseg + static_cast<int64_t>(wfirst) * K, wbytes);
        rwu = make_rsrc(wseg + static_cast<int64_t>(MODE == kModeSwiGLU ? a.N_out + wfirst : wfirst) * K, wbytes);
        wlane = rb * K + chunk * 16;
        const uint8_t *xbase = GATHER ? static_cast<const uint8_t *>(a.A)
                                      : static_cast<const uint8_t *>(a.A) + (static_cast<int64_t>(ti.row0) + ti.m0) * K;
        const uint8_t *xsbase = GATHER ? x.xs : x.xs + (static_cast<int64_t>(ti.row0) + ti.m0) * KS;
        rx = make_rsrc(xbase, static_cast<uint32_t>(GATHER ? a.a_rows : rows) * static_cast<uint32_t>(K));
        rws = make_rsrc(wsseg);
        rxs = make_rsrc(xsbase, static_cast<uint32_t>(GATHER ? a.a_rows : rows) * static_cast<uint32_t>(KS));
        if constexpr (GATHER) {
#pragma unroll
            for (int j = 0; j < XJ; ++j) {
                const int r = rb + 32 * j;
                xv[j] = a.gather[ti.row0 + ti.m0 + (r < rows ? r : rows - 1)] * K + chunk * 16;
            }
        } else {
            xv[0] = rb * K + chunk * 16;
        }
        // the scale words this thread stages: weight row and token row tid of the tile
        wsr = weight_row<MODE>(ti.n_tile, tid, a.N_out) * KS;
        xsr = (GATHER ? a.gather[ti.row0 + ti.m0 + min(tid, rows - 1)] : min(tid, rows - 1)) * KS;
    }

    template <int q>
    __device__ __forceinline__ void load_item(int kt, MxStage<XJ> &R) const {
        const int ka = kt < nreal ? k0 + kt : kzero;
        if constexpr (q < 8) {
            const int soff = (MODE == kModeSwiGLU ? (q >> 1) : q) * 32 * K + ka * kMxBK;
            R.W[q] = __builtin_amdgcn_raw_buffer_load_b128((MODE == kModeSwiGLU && (q & 1)) ? rwu : rwg, wlane, soff, 0);
        } else if constexpr (q < 8 + XJ) {
            if constexpr (GATHER)
                R.X[q - 8] = __builtin_amdgcn_raw_buffer_load_b128(rx, xv[q - 8], ka * kMxBK, 0);
            else
                R.X[q - 8] = __builtin_amdgcn_raw_buffer_load_b128(rx, xv[0], (q - 8) * 32 * K + ka * kMxBK, 0);
        } else if constexpr (q == 8 + XJ) {
            R.S[0] = __builtin_amdgcn_raw_buffer_load_b32(rws, wsr, ka * 4, 0);
        } else {
            R.S[1] = __builtin_amdgcn_raw_buffer_load_b32(rxs, xsr, ka * 4, 0);
        }
    }
    __device__ __forceinline__ void load_step(int kt, MxStage<XJ> &R) const {
        constexpr_for<NIT>([&](auto q_tag) { load_item<decltype(q_tag)::value>(kt, R); });
    }
};

// One tile over all k-steps. Each k-step t runs two halves (k-subs s = 0,
// 1) of NI x NJ scaled MFMAs, weight-subtile-major. Fragments stream one
// weight subtile ahead: during the MFMAs of weight subtile i the next weight
// fragment is read, and one (half tile: two) of the token fragments of the
// next k-sub, so a half ends with the next k-sub's token fragments and its
// first weight fragment in registers (80 fragment VGPRs instead of 128 for
// two full sets). Half 0 also writes k-step t+1 (held in VGPRs) to the
// other stage and loads k-step t+2 and the scales of k-step t+1, one
// staging item after each MFMA slot in a fixed order; then this wave's LDS
// traffic is waited for and the block synchronises; half 1 reads the next
// k-sub from the other stage. Half 1 still reads the current stage (its
// weight fragments), so each k-step starts with a second block
// synchronisation before that stage is written again. Weight rows and
// (without gathering) token rows are addressed as one per-lane offset plus
// a per-row-group scalar offset, through buffer resources bounded to the
// tile's valid rows (rows past them read as zeros and are never stored).
// k-steps k0 + t for t < nreal, then (t >= nreal, when nks > nreal) the
// k-step kzero, which holds zero codes and scales: a product of zeros adds
// exactly nothing, so a tile may run an even number of steps.
template <int MODE, bool ODD, bool HALF, bool GATHER>
__device__ __forceinline__ void gemm_tile_mx(const MXArgs &x, const TileInfo &ti, uint8_t *LDSM, int k0, int nks,
                                             float *part, int64_t crow0, int nreal, int kzero) {
    const GGArgs &a = x.g;
    constexpr int NI = HALF ? 2 : 4;
    constexpr int NJ = 4;
    constexpr int NBR = NJ / NI;          // token fragments read per weight subtile
    constexpr int XJ = HALF ? 4 : 8;      // token chunks per thread per k-step
    constexpr int NMF = NI * NJ;          // MFMAs per half
    constexpr int NRD = NI * 2 * (1 + NBR);   // 16-byte fragment reads per half
    constexpr int NWR = 8 + XJ;           // chunk writes (and loads) per k-step
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wrow0 = HALF ? wave * 64 : (wave & 1) * 128;
    const int tok0 = HALF ? 0 : (wave >> 1) * 128;
    // k-steps [k0, k0 + nks) of the tile (all of them unless a split piece)
    const MxTileSrc<MODE, HALF, GATHER> src(x, ti, k0, nreal, kzero);
    const int nk = __builtin_amdgcn_readfirstlane(nks);
    const int chunk = tid & 7, rb = tid >> 3;
    const int so = mswz(rb, chunk);
    (void)a;
    // LDS: the two stages' scale blocks first, then their operand data, so
    // that every scale word sits at a 16-bit immediate offset from one
    // per-lane base (behind a stage's 64 KB of data each word needed an
    // address register of its own, which the loop spilled and reloaded)
    uint8_t *const SC0 = LDSM, *const SC1 = LDSM + kMxScaleBytes;
    uint8_t *const LB0 = LDSM + 2 * kMxScaleBytes, *const LB1 = LB0 + kMxStage;

    floatx16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    MxStage<XJ> R;   // the next k-step's staging registers
    // the scale words of the lane's rows, shifted to its blocks; one set for
    // even and one for odd k-steps
    uint32_t SA0[NI], SB0[NJ], SA1[NI], SB1[NJ];
    v8i fx, fy, fb0[NJ], fb1[NJ];

    auto frag = [&](const uint8_t *LB, int row, int sub) -> v8i {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(LB + mswz(row, 4 * sub + lhi));
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(LB + mswz(row, 4 * sub + 2 + lhi));
        v8i f;
        f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
        f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
        return f;
    };
    auto read_scales = [&](const uint8_t *SC, uint32_t (&SA)[NI], uint32_t (&SB)[NJ]) {
        const uint32_t *LS = reinterpret_cast<const uint32_t *>(SC);
#pragma unroll
        for (int i = 0; i < NI; ++i) SA[i] = LS[wrow0 + i * 32 + l32] >> (8 * lhi);
#pragma unroll
        for (int j = 0; j < NJ; ++j) SB[j] = LS[kMxTile + tok0 + j * 32 + l32] >> (8 * lhi);
    };
    auto write_step = [&](uint8_t *LB, uint8_t *SC) {
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(LB + so + j * 32 * kMxBK) = R.W[j];
#pragma unroll
        for (int j = 0; j < XJ; ++j) *reinterpret_cast<u32x4 *>(LB + kMxRegion + so + j * 32 * kMxBK) = R.X[j];
        reinterpret_cast<uint32_t *>(SC)[tid] = R.S[0];
        reinterpret_cast<uint32_t *>(SC)[kMxTile + tid] = R.S[1];
    };
    // One half: MFMAs of k-sub S of stage LBc (weight fragment 0 in fx,
    // token fragments in FBc), streaming in weight fragments of the same
    // k-sub and the next k-sub (stage LBn, k-sub SN) into FBn and fx.
    auto half = [&](auto s_tag, auto sn_tag, const uint8_t *LBc, const uint8_t *LBn, v8i (&FBc)[NJ],
                    v8i (&FBn)[NJ], const uint32_t (&SA)[NI], const uint32_t (&SB)[NJ]) {
        constexpr int S = decltype(s_tag)::value, SN = decltype(sn_tag)::value;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            v8i &fa = (i & 1) ? fy : fx;
            v8i &fo = (i & 1) ? fx : fy;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, FBc[j], acc[i][j], 0, 0, 2 * S, SA[i],
                                                                            2 * S, SB[j]);
            fo = (i + 1 < NI) ? frag(LBc, wrow0 + (i + 1) * 32 + l32, S) : frag(LBn, wrow0 + l32, SN);
#pragma unroll
            for (int r = 0; r < NBR; ++r) FBn[i * NBR + r] = frag(LBn + kMxRegion, tok0 + (i * NBR + r) * 32 + l32, SN);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Staging item q of a k-step (R.W[q] for q < 8, then the token chunks,
    // then the two scale words) to its place in stage LB (scale words: SC).
    constexpr int NIT = NWR + 2;
    auto write_item = [&](uint8_t *LB, uint8_t *SC, auto q_tag) {
        constexpr int q = decltype(q_tag)::value;
        if constexpr (q < 8) *reinterpret_cast<u32x4 *>(LB + so + q * 32 * kMxBK) = R.W[q];
        else if constexpr (q < NWR) *reinterpret_cast<u32x4 *>(LB + kMxRegion + so + (q - 8) * 32 * kMxBK) = R.X[q - 8];
        else reinterpret_cast<uint32_t *>(SC)[(q - NWR) * kMxTile + tid] = R.S[q - NWR];
    };
    // Half 0 with the staging pinned: MFMA slot q (weight subtile i = q / NJ,
    // token subtile j) is followed by its fragment reads (the next weight
    // fragment at j = 0, the next k-sub's token fragments at j = 1 ..), then
    // the LDS write of item q of k-step t+1 and the load of item q of k-step
    // t+2 (items spread evenly over the slots). Items keep one order in
    // every step, so each write waits for the load issued one k-step before
    // it and no earlier one.
    auto half0 = [&](const uint8_t *LBc, uint8_t *NXT, uint8_t *SNXT, int kk, const uint32_t (&SA)[NI],
                     const uint32_t (&SB)[NJ]) {
        constexpr_for<NMF>([&](auto q_tag) {
            constexpr int q = decltype(q_tag)::value;
            constexpr int i = q / NJ, j = q % NJ;
            v8i &fa = (i & 1) ? fy : fx;
            v8i &fo = (i & 1) ? fx : fy;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb0[j], acc[i][j], 0, 0, 0, SA[i], 0,
                                                                        SB[j]);
            if constexpr (j == 0) fo = i + 1 < NI ? frag(LBc, wrow0 + (i + 1) * 32 + l32, 0) : frag(LBc, wrow0 + l32, 1);
            if constexpr (j >= 1 && j <= NBR) fb1[i * NBR + j - 1] = frag(LBc + kMxRegion, tok0 + (i * NBR + j - 1) * 32 + l32, 1);
            constexpr int lo = q * NIT / NMF, hi = (q + 1) * NIT / NMF;
            constexpr_for<hi - lo>([&](auto r_tag) {
                constexpr int it = lo + decltype(r_tag)::value;
                write_item(NXT, SNXT, std::integral_constant<int, it>{});
                src.template load_item<it>(kk, R);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto step = [&](const uint8_t *CUR, uint8_t *NXT, uint8_t *SNXT, int t, const uint32_t (&SAc)[NI],
                    const uint32_t (&SBc)[NJ], uint32_t (&SAn)[NI], uint32_t (&SBn)[NJ]) {
        const int kk = t + 2 < nk ? t + 2 : nk - 1;
        // NXT held k-step t-1, whose second k-sub every wave read during the
        // second half of the previous step: all of them are past it before
        // anyone overwrites it
        MOE_LDS_BARRIER();
        half0(CUR, NXT, SNXT, kk, SAc, SBc);
        MOE_LDS_BARRIER();
        read_scales(SNXT, SAn, SBn);
        half(I1{}, I0{}, CUR, NXT, fb1, fb0, SAc, SBc);
        mx_sched<NMF, NRD + NI + NJ, 0, 0>();
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: k-step 0 into stage 0 with its scales, k-step 1 into VGPRs
    src.load_step(0, R);
    MOE_LDS_BARRIER();   // every wave is done reading the previous tile's stages
    write_step(LB0, SC0);
    src.load_step(nk > 1 ? 1 : 0, R);
    MOE_LDS_BARRIER();
    read_scales(SC0, SA0, SB0);
    fx = frag(LB0, wrow0 + l32, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb0[j] = frag(LB0 + kMxRegion, tok0 + j * 32 + l32, 0);
    if (ODD) {
        for (int t = 0; t + 1 < nk; t += 2) {
            step(LB0, LB1, SC1, t, SA0, SB0, SA1, SB1);
            step(LB1, LB0, SC0, t + 1, SA1, SB1, SA0, SB0);
        }
        step(LB0, LB1, SC1, nk - 1, SA0, SB0, SA1, SB1);
    } else {
        for (int t = 0; t < nk; t += 2) {
            step(LB0, LB1, SC1, t, SA0, SB0, SA1, SB1);
            step(LB1, LB0, SC0, t + 1, SA1, SB1, SA0, SB0);
        }
    }
    if (part) {
        // a split piece: the raw accumulators, element e = 16 (i*4 + j) + q of
        // thread tid at float4 index (e/4) * 256 + tid
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
    if constexpr (MODE == kModeSwiGLU) store_tile_mx_swiglu<HALF>(a, ti, acc, wave, lane, crow0);
    else if constexpr (MODE == kModeF32T) store_tile_mx_t<HALF>(a, ti, acc, wave, lane, crow0);
    else store_tile_mx_plain<MODE, HALF>(a, ti, acc, wave, lane, crow0);
}

// Split workspace (second projection only): an int header of 64 KB ([0..2]:
// split tiles, pieces per tile, k-steps per piece; from int 64, 8 ints per
// split tile: seg, m0, n_tile, M, row0), then fp32 partial tiles of
// kMxPartFloats each, piece p of split tile t at index t * s + p.
constexpr int kMxWsHeaderInts = 16384;
constexpr int kMxWsMaxSplitTiles = (kMxWsHeaderInts - 64) / 8;
constexpr int kMxPartFloats = kMxTile * kMxTile;

// When the last round of tiles would leave more than half of the blocks
// idle, its tiles are split along K into s pieces of ps k-steps (ps even)
// so that it keeps up to G blocks busy; split_reduce_mx sums each tile's
// pieces in piece order (deterministic) and runs the epilogue. Every block
// derives the same plan from the segment offsets.
struct MxSplitPlan {
    int full, s, ps, items;   // whole tiles, pieces per split tile, k-steps per piece, work items
};

__device__ __forceinline__ MxSplitPlan mx_split_plan(const GGArgs &a, int total, int nk, bool odd) {
    MxSplitPlan p{total, 0, 0, total};
    const int G = a.grid, rem = total % G;
    if (odd || a.ws == nullptr || rem == 0 || 2 * rem > G || nk < 4) return p;
    int s = min(G / rem, nk / 2);
    const int ps = 2 * ((nk + 2 * s - 1) / (2 * s));
    s = (nk + ps - 1) / ps;
    if (s < 2 || rem * s > a.ws_tiles || rem > kMxWsMaxSplitTiles) return p;
    p.full = total - rem;
    p.s = s;
    p.ps = ps;
    p.items = p.full + rem * s;
    return p;
}

template <int MODE, bool ODD, bool GATHER>
__global__ __launch_bounds__(256, 1) void grouped_gemm_mx(MXArgs x) {
    __shared__ __attribute__((aligned(16))) uint8_t LDSM[2 * (kMxScaleBytes + kMxStage)];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    const int total = __builtin_amdgcn_readfirstlane(build_tile_prefix(x.g, kMxTile, s_cum, s_tmp));
    const int nk = x.g.K / kMxBK;
    // split pieces only in the plain (second) projection
    const MxSplitPlan sp = mx_split_plan(x.g, total, nk, ODD || MODE != kModePlain || GATHER);
    int *hdr = reinterpret_cast<int *>(x.g.ws);
    if (MODE == kModePlain && hdr && blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[0] = sp.s ? total - sp.full : 0;
        hdr[1] = sp.s;
        hdr[2] = sp.ps;
    }
    for (int w = xcd_block_index(blockIdx.x, x.g.grid); w < sp.items; w += x.g.grid) {
        int L = w, k0 = 0, nks = nk;
        float *part = nullptr;
        if (sp.s && w >= sp.full) {
            const int q = w - sp.full;
            L = sp.full + q / sp.s;
            k0 = (q % sp.s) * sp.ps;
            nks = min(sp.ps, nk - k0);
            part = x.g.ws + kMxWsHeaderInts + static_cast<int64_t>(q) * kMxPartFloats;
        }
        const TileInfo ti = decode_tile(x.g, s_cum, L, kMxTile);
        if (part && k0 == 0 && threadIdx.x == 0) {
            int *d = hdr + 64 + (L - sp.full) * 8;
            d[0] = ti.seg;
            d[1] = ti.m0;
            d[2] = ti.n_tile;
            d[3] = ti.M;
            d[4] = ti.row0;
        }
        const int64_t crow0 = static_cast<int64_t>(ti.row0) + ti.m0;
        if (ti.M - ti.m0 > kMxTile / 2)
            gemm_tile_mx<MODE, ODD, false, GATHER>(x, ti, LDSM, k0, nks, part, crow0, nks, 0);
        else
            gemm_tile_mx<MODE, ODD, true, GATHER>(x, ti, LDSM, k0, nks, part, crow0, nks, 0);
    }
}

// Weight gradients by k-segments: the token-slot operand A [M][K] and the
// weight-slot operand B [N_out][K] are shared by all experts (K: the row
// stride, the padded token count); expert e reduces over its k-steps
// [poffs[e], poffs[e+1]) / 128 into C[e] = B A^T, [N_out][M] in fp32 (zeros
// for an expert without tokens), stored by the transposed epilogue. Tile
// order: the experts by decreasing k-range, then groups of 4 weight-slot
// tiles (rows of C), then the token-slot tile (columns of C), then the
// weight-slot tile within the group; the tile body is the rows mode's, with
// the expert's k-range. An odd number of k-steps is completed by one step on
// the zero k-step kzero (the last 128 columns of A and B), so the kernel
// holds the even tile body only; half tiles (128 rows of A) only when
// M % 256 != 0 (HALF_TAIL).
template <bool HALF_TAIL>
__global__ __launch_bounds__(256, 1) void grouped_gemm_mx_kseg(MXArgs x, const int32_t *poffs, int M, int kzero) {
    __shared__ __attribute__((aligned(16))) uint8_t LDSM[2 * (kMxScaleBytes + kMxStage)];
    __shared__ int s_order[256], s_len[256];
    const int tid = threadIdx.x;
    // experts by decreasing k-range (ties: lower index first)
    s_len[tid] = tid < x.g.E ? poffs[tid + 1] - poffs[tid] : -1;
    __syncthreads();
    if (tid < x.g.E) {
        const int m = s_len[tid];
        int rank = 0;
        for (int e = 0; e < x.g.E; ++e) rank += (s_len[e] > m) || (s_len[e] == m && e < tid);
        s_order[rank] = tid;
    }
    __syncthreads();
    const int m_tiles = (M + kMxTile - 1) / kMxTile;
    const int per = m_tiles * x.g.n_tiles;
    const int total = x.g.E * per;
    const int G = x.g.grid, slot = xcd_block_index(blockIdx.x, G);
    for (int w0 = 0; w0 < total; w0 += G) {
        // every other round of tiles in reverse block order, so that a block
        // that took a heavy expert's tile takes a light one next
        const int w = ((w0 / G) & 1) ? w0 + G - 1 - slot : w0 + slot;
        if (w >= total) continue;
        // groups of 4 weight-slot tiles by every token-slot tile, column by
        // column: the 32 tiles an XCD runs at a time (consecutive w) form a
        // 4 x 8 block and share 12 operand panels per k-step
        const int eo = w / per, r = w - eo * per;
        const int e = s_order[eo];
        const int g = r / (4 * m_tiles), rg = r - g * (4 * m_tiles);
        const int gn = min(x.g.n_tiles - 4 * g, 4);
        const int mt = rg / gn;
        TileInfo ti;
        ti.seg = 0;
        ti.m0 = mt * kMxTile;
        ti.n_tile = 4 * g + (rg - mt * gn);
        ti.M = M;
        ti.row0 = 0;
        ti.shared = false;
        const int k0 = poffs[e] / kMxBK, nks = (poffs[e + 1] - poffs[e]) / kMxBK;
        const int64_t crow0 = static_cast<int64_t>(e) * x.g.N_out;
        const int nrun = nks + (nks & 1);
        if (HALF_TAIL && M - ti.m0 <= kMxTile / 2)
            gemm_tile_mx<kModeF32T, false, true, false>(x, ti, LDSM, k0, nrun, nullptr, crow0, nks, kzero);
        else
            gemm_tile_mx<kModeF32T, false, false, false>(x, ti, LDSM, k0, nrun, nullptr, crow0, nks, kzero);
    }
}

// A split tile's partial sums (s pieces, piece order), then the plain epilogue.
template <bool HALF>
__device__ __forceinline__ void mx_reduce_tile(const GGArgs &a, const TileInfo &ti, const float4 *P4, int s) {
    constexpr int NI = HALF ? 2 : 4, NJ = 4;
    const int tid = threadIdx.x;
    floatx16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    for (int p = 0; p < s; ++p) {
        const float4 *Pp = P4 + static_cast<int64_t>(p) * (kMxPartFloats / 4);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = Pp[((i * NJ + j) * 4 + q) * 256 + tid];
                    acc[i][j][4 * q] += v.x;
                    acc[i][j][4 * q + 1] += v.y;
                    acc[i][j][4 * q + 2] += v.z;
                    acc[i][j][4 * q + 3] += v.w;
                }
    }
    store_tile_mx_plain<kModePlain, HALF>(a, ti, acc, tid >> 6, tid & 63, static_cast<int64_t>(ti.row0) + ti.m0);
}

// Sum of every split tile's pieces, in piece order, into piece 0 (one
// float4 per thread, all tiles' positions spread over the grid).
__global__ __launch_bounds__(256) void split_sum_mx(GGArgs a) {
    const int *hdr = reinterpret_cast<const int *>(a.ws);
    const int rem = hdr[0], s = hdr[1];
    if (s < 2) return;
    constexpr int kQ = kMxPartFloats / 4;
    const int64_t n = static_cast<int64_t>(rem) * kQ;
    float4 *P4 = reinterpret_cast<float4 *>(a.ws + kMxWsHeaderInts);
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

// One block per split tile: its summed piece 0, then the plain epilogue.
__global__ __launch_bounds__(256, 1) void split_reduce_mx(GGArgs a) {
    const int *hdr = reinterpret_cast<const int *>(a.ws);
    const int rem = hdr[0], s = hdr[1] > 0 ? 1 : 0;   // the pieces are summed into piece 0
    const int t = blockIdx.x;
    if (s == 0 || t >= rem) return;
    const int *d = hdr + 64 + t * 8;
    TileInfo ti;
    ti.seg = d[0];
    ti.m0 = d[1];
    ti.n_tile = d[2];
    ti.M = d[3];
    ti.row0 = d[4];
    ti.shared = false;
    const float4 *P4 = reinterpret_cast<const float4 *>(a.ws + kMxWsHeaderInts) +
                       static_cast<int64_t>(t) * hdr[1] * (kMxPartFloats / 4);
    if (ti.M - ti.m0 <= kMxTile / 2) mx_reduce_tile<true>(a, ti, P4, s);
    else mx_reduce_tile<false>(a, ti, P4, s);
}

template <int MODE>
int launch_mx(MXArgs x, int64_t P, hipStream_t s, const char *what) {
    const int BNo = MODE == kModeSwiGLU ? 128 : 256;
    x.g.n_tiles = (x.g.N_out + BNo - 1) / BNo;
    const int64_t upper = (P / 256 + x.g.E) * static_cast<int64_t>(x.g.n_tiles);
    int64_t grid = num_cus();
    if (grid > upper) grid = upper;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    x.g.grid = static_cast<int>(grid);
    const bool odd = (x.g.K / kMxBK) & 1;
    if (x.g.gather) {
        if (odd) hipLaunchKernelGGL((grouped_gemm_mx<MODE, true, true>), dim3(x.g.grid), dim3(256), 0, s, x);
        else hipLaunchKernelGGL((grouped_gemm_mx<MODE, false, true>), dim3(x.g.grid), dim3(256), 0, s, x);
    } else {
        if (odd) hipLaunchKernelGGL((grouped_gemm_mx<MODE, true, false>), dim3(x.g.grid), dim3(256), 0, s, x);
        else hipLaunchKernelGGL((grouped_gemm_mx<MODE, false, false>), dim3(x.g.grid), dim3(256), 0, s, x);
    }
    // split tiles: at most half the grid (the plan's condition)
    if (MODE == kModePlain && x.g.ws != nullptr && !odd && !x.g.gather) {
        hipLaunchKernelGGL(split_sum_mx, dim3(1024), dim3(256), 0, s, x.g);
        hipLaunchKernelGGL(split_reduce_mx, dim3(static_cast<unsigned>(x.g.grid / 2 > 0 ? x.g.grid / 2 : 1)), dim3(256), 0,
                           s, x.g);
    }
    return check_launch(what);
}

}  // namespace

int mx_gemm_rows(const uint8_t *a_codes, const uint8_t *a_scales, const int32_t *gather, int a_rows,
                 const int32_t *offsets, int E, int64_t P, const uint8_t *b_codes, const uint8_t *b_scales, int N_out,
                 int K, void *C, bool f32_out, hipStream_t s, const char *what) {
    MXArgs g{};
    g.g.A = a_codes;
    g.g.gather = gather;
    g.g.a_rows = gather ? a_rows : 0;
    g.g.B = b_codes;
    g.g.C = C;
    g.g.offsets = offsets;
    g.g.E = E;
    g.g.N_out = N_out;
    g.g.K = K;
    g.ws = b_scales;
    g.xs = a_scales;
    return f32_out ? launch_mx<kModeF32Out>(g, P, s, what) : launch_mx<kModePlain>(g, P, s, what);
}

int mx_gemm_kseg(const uint8_t *a_codes, const uint8_t *a_scales, int M, const uint8_t *b_codes,
                 const uint8_t *b_scales, int N, int64_t ld, const int32_t *poffs, int E, float *C, hipStream_t s,
                 const char *what) {
    // A in the kernel's weight slot and B in its token slot, so that a lane's
    // accumulators run along a row of C (the transposed epilogue): the
    // kernel's tiles are 256 rows of A (n_tile) by 256 rows of B (m0)
    MXArgs g{};
    g.g.A = b_codes;
    g.g.B = a_codes;
    g.g.C = C;
    g.g.E = E;
    g.g.N_out = M;
    g.g.K = static_cast<int>(ld);
    g.ws = a_scales;
    g.xs = b_scales;
    g.g.n_tiles = (M + kMxTile - 1) / kMxTile;
    const int64_t tiles = static_cast<int64_t>(E) * ((N + kMxTile - 1) / kMxTile) * g.g.n_tiles;
    int64_t grid = num_cus();
    if (grid > tiles) grid = tiles;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    g.g.grid = static_cast<int>(grid);
    const int kzero = static_cast<int>(ld / kMxBK) - 1;
    if (N % kMxTile)
        hipLaunchKernelGGL(grouped_gemm_mx_kseg<true>, dim3(g.g.grid), dim3(256), 0, s, g, poffs, N, kzero);
    else
        hipLaunchKernelGGL(grouped_gemm_mx_kseg<false>, dim3(g.g.grid), dim3(256), 0, s, g, poffs, N, kzero);
    return check_launch(what);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_mx_quantize(const void *src, int dtype, int64_t rows, int64_t K, uint8_t *codes,
                               uint8_t *scales, void *stream) {
    clear_error();
    MOE_CHECK_ARG(rows >= 0 && K > 0, MOE_ERR_INVALID_ARG, "moe_mx_quantize: bad sizes");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_mx_quantize: bad dtype %d", dtype);
    MOE_CHECK_ARG(rows == 0 || (src && codes && scales), MOE_ERR_INVALID_ARG, "moe_mx_quantize: null pointer");
    MOE_CHECK_ARG(K % 32 == 0, MOE_ERR_UNSUPPORTED, "moe_mx_quantize: K must be a multiple of 32");
    MOE_CHECK_ARG(rows == 0 || (aligned16(src) && aligned16(codes)), MOE_ERR_INVALID_ARG,
                  "moe_mx_quantize: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    if (dtype == MOE_DTYPE_BF16)
        launch_quantize(static_cast<const bf16_t *>(src), rows, K, codes, scales, s);
    else
        launch_quantize(static_cast<const float *>(src), rows, K, codes, scales, s);
    return check_launch("moe_mx_quantize");
}

extern "C" size_t moe_grouped_ffn_mx_workspace_size(int64_t P, int64_t h, int64_t F, int E) {
    if (P <= 0 || h <= 0 || F <= 0 || E <= 0) return 0;
    // the header and 256 partial tiles (one per compute unit of the MI355X;
    // a grid of more blocks would split fewer tiles)
    return static_cast<size_t>(kMxWsHeaderInts) * 4 + static_cast<size_t>(256) * kMxPartFloats * 4;
}

extern "C" int moe_grouped_ffn_mx(const uint8_t *x_codes, const uint8_t *x_scales, const int32_t *gather_rows,
                                  int64_t x_rows, int64_t P, int64_t h, int64_t F, int E, const int32_t *offsets,
                                  int act_kind, const uint8_t *w1_codes, const uint8_t *w1_scales,
                                  const uint8_t *w2_codes, const uint8_t *w2_scales, void *act, uint8_t *act_codes,
                                  uint8_t *act_scales, void *y, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    clear_error();
    MOE_CHECK_ARG(offsets && w1_codes && w1_scales && w2_codes && w2_scales &&
                      (P == 0 || (x_codes && x_scales && act_codes && act_scales && y)),
                  MOE_ERR_INVALID_ARG, "moe_grouped_ffn_mx: null required pointer");
    MOE_CHECK_ARG(P >= 0 && h > 0 && F > 0 && E > 0, MOE_ERR_INVALID_ARG, "moe_grouped_ffn_mx: bad sizes");
    MOE_CHECK_ARG(act_kind == MOE_ACT_SWIGLU, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_mx: SwiGLU experts only");
    MOE_CHECK_ARG(h % 128 == 0 && F % 128 == 0 && E <= 256, MOE_ERR_UNSUPPORTED,
                  "moe_grouped_ffn_mx: need h %% 128 == 0, F %% 128 == 0, E <= 256");
    MOE_CHECK_ARG(gather_rows == nullptr || x_rows > 0, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_mx: gathering needs x_rows > 0");
    const int64_t xr = gather_rows ? x_rows : P;
    MOE_CHECK_ARG(P < (int64_t(1) << 31) && xr * h < (int64_t(1) << 31) && P * F < (int64_t(1) << 31) &&
                      2 * F * h < (int64_t(1) << 31),
                  MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_mx: sizes too large");
    const void *ptrs[] = {x_codes, w1_codes, w2_codes, act, act_codes, y, workspace};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(p == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn_mx: code, output and workspace pointers must be 16-byte aligned");
    const void *sp[] = {x_scales, w1_scales, w2_scales, act_scales};
    for (const void *p : sp)
        MOE_CHECK_ARG((reinterpret_cast<uintptr_t>(p) & 3u) == 0, MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn_mx: scale pointers must be 4-byte aligned");
    hipStream_t s = as_stream(stream);

    MXArgs g1{};
    g1.g.A = x_codes;
    g1.g.gather = gather_rows;
    g1.g.a_rows = static_cast<int>(gather_rows ? x_rows : 0);
    g1.g.B = w1_codes;
    g1.g.C = act;
    g1.g.offsets = offsets;
    g1.g.E = E;
    g1.g.N_out = static_cast<int>(F);
    g1.g.K = static_cast<int>(h);
    g1.ws = w1_scales;
    g1.xs = x_scales;
    g1.g.GU = act_codes;
    g1.g.GU_sh = act_scales;
    const int st = launch_mx<kModeSwiGLU>(g1, P, s, "moe_grouped_ffn_mx gemm1");
    if (st != MOE_OK) return st;

    MXArgs g2{};
    g2.g.A = act_codes;
    g2.g.B = w2_codes;
    g2.g.C = y;
    g2.g.offsets = offsets;
    g2.g.E = E;
    g2.g.N_out = static_cast<int>(h);
    g2.g.K = static_cast<int>(F);
    g2.ws = w2_scales;
    g2.xs = act_scales;
    // split pieces of the last round of tiles, when a workspace is given
    const size_t hdr = static_cast<size_t>(kMxWsHeaderInts) * 4;
    if (workspace && workspace_bytes >= hdr + static_cast<size_t>(kMxPartFloats) * 4) {
        g2.g.ws = static_cast<float *>(workspace);
        const size_t nt = (workspace_bytes - hdr) / (static_cast<size_t>(kMxPartFloats) * 4);
        g2.g.ws_tiles = static_cast<int>(nt < (1u << 20) ? nt : (1u << 20));
    }
    return launch_mx<kModePlain>(g2, P, s, "moe_grouped_ffn_mx gemm2");
}
