// Expert computation: one grouped GEMM launch per projection over all
// experts' ragged segments ("Scalable Training of Mixture-of-Experts Models
// with Megatron Core", section 2.1 stage 3: all local experts in a single
// grouped GEMM call). SwiGLU experts without bias ("Mixture-of-Experts from
// Architecture to Large-Scale Training", section 2.5: gate, up and down
// matrices) or GELU(erf) experts with biases ("emerging-techniques-moe-
// training", Quick Start).
//
// bf16 kernel, CDNA4 (gfx950), one persistent launch per projection:
// - every expert segment (and the shared expert's rows) is cut into balanced
//   tiles of at most 256 token rows; tiles are 256 weight rows wide; the tile
//   list is built on the device from the segment offsets, numbered m-fastest
//   (consecutive tiles share a weight panel) and mapped so that the blocks of
//   one XCD take consecutive tiles (their shared panels stay in that XCD's L2);
// - 8 waves per block, v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the
//   weight tile is the MFMA "A" operand, so a lane's accumulators are runs of
//   4 consecutive output columns of one token row;
// - operands reach LDS through global_load_lds_dwordx4 in a 4-stage ring
//   (details at the kernel);
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

// Tile: 256 weight rows (n) x up to 256 token rows (m), 8 waves. Wave w owns
// weight rows [64 (w%4), +64) of the tile (two 32-row MFMA subtiles) and
// token rows [128 (w/4), +128) (four 32-row subtiles). Waves w and w+4 share a
// SIMD, so a tile with few rows leaves half of each SIMD's work undone rather
// than idling whole SIMDs; subtiles past the tile's row count are skipped.
//
// MFMA v_mfma_f32_32x32x16_bf16: lane l supplies row l%32, k = 8(l/32)..+7
// of each operand; accumulator element i of lane l is row
// 8(i/4) + 4(l/32) + i%4 (weight row) and column l%32 (token row).
//
// Operand staging: a ring of kStages LDS stages, each 256 weight rows and 256
// token rows of kBK = 32 bf16 (64-byte rows, four 16-byte chunks; chunk c of
// row r sits at chunk c ^ ((r >> 2) & 3), so the 16 rows one read phase
// touches cover all 64 banks). Global -> LDS moves use global_load_lds_dwordx4:
// one instruction fills 1 KB of LDS (16 rows) with lane l's 16 bytes at byte
// 16 l, so each lane fetches the global chunk that the swizzle puts there. No
// VGPR staging, no ds_write. Loads run kStages - 1 k-steps ahead; a k-step
// waits only for its own stage (s_waitcnt vmcnt on the wave's later loads,
// then s_barrier).
constexpr int kBK = 32;
constexpr int kStages = 4;

#define MOE_AS3(p) ((__attribute__((address_space(3))) void *)(p))

__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ ((r >> 2) & 3)) << 3); }

// s_waitcnt with only vmcnt constrained (expcnt 7, lgkmcnt 15 = no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bf16(GGArgs a) {
    constexpr int TILE = 256;
    constexpr int NS = 2, MS = 4;
    constexpr int STAGE = 2 * TILE * kBK;       // elements per LDS stage (weights + tokens)
    // one array per stage: the compiler then sees which stage a pending
    // global->LDS load writes and does not wait for all of them before a read
    __shared__ __attribute__((aligned(16))) bf16_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) bf16_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) bf16_t st2[STAGE];
    __shared__ __attribute__((aligned(16))) bf16_t st3[STAGE];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 3, wm = wave >> 2;
    const int l32 = lane & 31, lhi = lane >> 5;

    const int total = build_tile_prefix_bal(a, s_cum, s_tmp);
    const int nb_rows = MODE == kModeSwiGLU ? 2 * a.N_out : a.N_out;
    const int K = a.K;
    const int nk = K / kBK;
    // this wave fills LDS regions 4w..4w+3 of each stage (16 rows each):
    // waves 0..3 the weight rows, waves 4..7 the token rows
    const bool fills_w = wave < 4;
    const int prow0 = (wave & 3) * 64 + (lane >> 2);   // tile row of load i: prow0 + 16 i
    const int pchunk = lane & 3;

    for (int L = xcd_block_index(blockIdx.x, a.grid); L < total; L += a.grid) {
        const BalTile ti = decode_tile_bal(a, s_cum, L);
        const int nact = (ti.rows + 31) >> 5;   // active 32-row token subtiles of the tile
        int nw = nact - wm * MS;                // ... of this wave
        nw = nw < 0 ? 0 : (nw > MS ? MS : nw);

        // global source of each of this lane's 4 chunks per stage
        const bf16_t *src[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = prow0 + 16 * i;                       // tile row
            const int c = pchunk ^ ((r >> 2) & 3);              // logical 16-byte chunk
            if (fills_w) {
                int wrow;
                if (MODE == kModeSwiGLU) {
                    const int f = ti.n_tile * (TILE / 2) + (r >> 6) * 32 + (r & 31);
                    wrow = ((r >> 5) & 1) ? a.N_out + f : f;
                    if (f >= a.N_out) wrow = 0;
                } else {
                    wrow = ti.n_tile * TILE + r;
                    if (wrow >= nb_rows) wrow = 0;
                }
                const bf16_t *Bseg = ti.shared ? static_cast<const bf16_t *>(a.B_sh)
                                               : static_cast<const bf16_t *>(a.B) +
                                                     static_cast<int64_t>(ti.seg) * nb_rows * K;
                src[i] = Bseg + static_cast<int64_t>(wrow) * K + c * 8;
            } else {
                const bf16_t *Aseg = ti.shared ? static_cast<const bf16_t *>(a.A_sh)
                                               : static_cast<const bf16_t *>(a.A) + static_cast<int64_t>(ti.row0) * K;
                const int m = r < ti.rows ? r : ti.rows - 1;   // clamped: in bounds, never stored
                src[i] = Aseg + (static_cast<int64_t>(ti.row_lo) + m) * K + c * 8;
            }
        }
        const int dsto = (fills_w ? 0 : TILE * kBK) + (wave & 3) * 64 * kBK;   // region of load 0

        floatx16 acc[NS][MS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int j = 0; j < MS; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

#define MOE_FILL(ARR, KT)                                                                       \
    do {                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                         \
            __builtin_amdgcn_global_load_lds(src[i] + (KT) * kBK, MOE_AS3(ARR + dsto + 16 * i * kBK), 16, 0, 0); \
    } while (0)

        // prologue: stages 0 .. kStages-2
        if (0 < nk) MOE_FILL(st0, 0);
        if (1 < nk) MOE_FILL(st1, 1);
        if (2 < nk) MOE_FILL(st2, 2);

// One k-step on stage CUR; refills NXT (the stage read one step earlier)
// with k-step KT + kStages - 1. UNIFORM: every step issues its loads (the
// tail re-fetches the last k-step into a stage nobody reads again), so the
// wave always waits for exactly the 8 later loads and the compiler can prove
// that the stage being read has landed.
#define MOE_KSTEP(CUR, NXT, KT, UNIFORM)                                                        \
    do {                                                                                      \
        const int kt_ = (KT);                                                                 \
        if (UNIFORM) {                                                                        \
            wait_vmcnt<8>();                                                                  \
        } else {                                                                              \
            const int later_ = nk - 1 - kt_;                                                  \
            if (later_ >= 2) wait_vmcnt<8>();                                                 \
            else if (later_ == 1) wait_vmcnt<4>();                                            \
            else wait_vmcnt<0>();                                                             \
        }                                                                                     \
        __builtin_amdgcn_s_barrier();                                                         \
        if (UNIFORM) MOE_FILL(NXT, min(kt_ + kStages - 1, nk - 1));                           \
        else if (kt_ + kStages - 1 < nk) MOE_FILL(NXT, kt_ + kStages - 1);                    \
        if (nw > 0) {                                                                         \
            const bf16_t *sw_ = CUR;                                                          \
            const bf16_t *sx_ = CUR + TILE * kBK;                                             \
            _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                \
                const int ch = ks * 2 + lhi;                                                  \
                bf16x8_t af[NS], bfr[MS];                                                     \
                _Pragma("unroll") for (int i = 0; i < NS; ++i)                                \
                    af[i] = *reinterpret_cast<const bf16x8_t *>(sw_ + lds_off(wn * 64 + i * 32 + l32, ch)); \
                _Pragma("unroll") for (int j = 0; j < MS; ++j)                                \
                    bfr[j] = *reinterpret_cast<const bf16x8_t *>(sx_ + lds_off(wm * 128 + j * 32 + l32, ch)); \
                if (nw == MS) {                                                               \
                    _Pragma("unroll") for (int j = 0; j < MS; ++j)                            \
                        _Pragma("unroll") for (int i = 0; i < NS; ++i)                        \
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0); \
                } else {                                                                      \
                    _Pragma("unroll") for (int j = 0; j < MS; ++j)                            \
                        if (j < nw)                                                           \
                            _Pragma("unroll") for (int i = 0; i < NS; ++i)                    \
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0); \
                }                                                                             \
            }                                                                                 \
        }                                                                                     \
    } while (0)

        if (nk % kStages == 0) {
            for (int kt = 0; kt < nk; kt += kStages) {
                MOE_KSTEP(st0, st3, kt, true);
                MOE_KSTEP(st1, st0, kt + 1, true);
                MOE_KSTEP(st2, st1, kt + 2, true);
                MOE_KSTEP(st3, st2, kt + 3, true);
            }
        } else {
            for (int kt = 0; kt < nk; kt += kStages) {
                MOE_KSTEP(st0, st3, kt, false);
                if (kt + 1 < nk) MOE_KSTEP(st1, st0, kt + 1, false);
                if (kt + 2 < nk) MOE_KSTEP(st2, st1, kt + 2, false);
                if (kt + 3 < nk) MOE_KSTEP(st3, st2, kt + 3, false);
            }
        }
#undef MOE_KSTEP
#undef MOE_FILL
        // drain the tail loads and make sure every wave is past its last read
        // of the ring before the next tile starts refilling it
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        // ------------------------------------------------------- epilogue
        const int64_t crow0 = static_cast<int64_t>(ti.row0) + ti.row_lo;
        bf16_t *Cseg = ti.shared ? static_cast<bf16_t *>(a.C_sh) + static_cast<int64_t>(ti.row_lo) * a.N_out
                                 : static_cast<bf16_t *>(a.C) + crow0 * a.N_out;
        bf16_t *GUseg = nullptr;
        if (MODE == kModeSwiGLU) {
            if (ti.shared)
                GUseg = a.GU_sh ? static_cast<bf16_t *>(a.GU_sh) + static_cast<int64_t>(ti.row_lo) * 2 * a.N_out
                                : nullptr;
            else
                GUseg = a.GU ? static_cast<bf16_t *>(a.GU) + crow0 * 2 * a.N_out : nullptr;
        }
        const bf16_t *bias = (a.bias && !ti.shared)
                                 ? static_cast<const bf16_t *>(a.bias) + static_cast<int64_t>(ti.seg) * nb_rows
                                 : nullptr;
#pragma unroll
        for (int j = 0; j < MS; ++j) {
            const int m = wm * 128 + j * 32 + l32;
            if (j >= nw || m >= ti.rows) continue;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int nl = 8 * gq + 4 * lhi;   // row offset inside a 32-row subtile
                if (MODE == kModeSwiGLU) {
                    const int f = ti.n_tile * (TILE / 2) + wn * 32 + nl;
                    if (f >= a.N_out) continue;
                    float g[4], u[4], hv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        g[q] = acc[0][j][4 * gq + q];
                        u[q] = acc[1][j][4 * gq + q];
                        if (bias) {
                            g[q] += bf16_to_f32(bias[f + q]);
                            u[q] += bf16_to_f32(bias[a.N_out + f + q]);
                        }
                        hv[q] = silu_f(g[q]) * u[q];
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
                } else {
#pragma unroll
                    for (int i = 0; i < NS; ++i) {
                        const int n = ti.n_tile * TILE + wn * 64 + i * 32 + nl;
                        if (n >= a.N_out) continue;
                        float v[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[q] = acc[i][j][4 * gq + q];
                            if (bias) v[q] += bf16_to_f32(bias[n + q]);
                            if (MODE == kModeGELU) v[q] = gelu_erf_f(v[q]);
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
    const int nb_rows = MODE == kModeSwiGLU ? 2 * a.N_out : a.N_out;
    const int BN_out = MODE == kModeSwiGLU ? BN / 2 : BN;
    const int K = a.K;
    const int r = tid >> 2, c4 = (tid & 3) * 4;

    for (int L = xcd_block_index(blockIdx.x, a.grid); L < total; L += a.grid) {
        const TileInfo ti = decode_tile(a, s_cum, L, BM);
        const float *Aseg = ti.shared ? static_cast<const float *>(a.A_sh)
                                      : static_cast<const float *>(a.A) + static_cast<int64_t>(ti.row0) * K;
        const float *Bseg = ti.shared ? static_cast<const float *>(a.B_sh)
                                      : static_cast<const float *>(a.B) + static_cast<int64_t>(ti.seg) * nb_rows * K;
        int wrow;
        if (MODE == kModeSwiGLU) {
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
        if (MODE == kModeSwiGLU)
            GUseg = ti.shared ? static_cast<float *>(a.GU_sh)
                              : (a.GU ? static_cast<float *>(a.GU) + static_cast<int64_t>(ti.row0) * 2 * a.N_out
                                      : nullptr);
        const float *bias = (a.bias && !ti.shared)
                                ? static_cast<const float *>(a.bias) + static_cast<int64_t>(ti.seg) * nb_rows
                                : nullptr;
        const int ng = lane >> 4;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int mm = ti.m0 + wm * 32 + j * 16 + (lane & 15);
            if (mm >= ti.M) continue;
            if (MODE == kModeSwiGLU) {
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
                    hp[i] = silu_f(g) * u;
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
                    float4 o;
                    float *op = &o.x;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = acc[i][j][q];
                        if (bias) v += bias[n + q];
                        if (MODE == kModeGELU) v = gelu_erf_f(v);
                        op[q] = v;
                    }
                    *reinterpret_cast<float4 *>(Cseg + static_cast<int64_t>(mm) * a.N_out + n) = o;
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
        const int BNo = MODE == kModeSwiGLU ? 128 : 256;
        a.n_tiles = (a.N_out + BNo - 1) / BNo;
        upper = ((P + a.M_sh) / 256 + S) * static_cast<int64_t>(a.n_tiles);
    } else {
        const int BNo = MODE == kModeSwiGLU ? 32 : 64;
        a.n_tiles = (a.N_out + BNo - 1) / BNo;
        upper = ((P + a.M_sh) / 64 + S) * static_cast<int64_t>(a.n_tiles);
    }
    int64_t grid = static_cast<int64_t>(num_cus()) * (dtype == MOE_DTYPE_BF16 ? 1 : 2);
    if (grid > upper) grid = upper;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    if (dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL((grouped_gemm_bf16<MODE>), dim3(a.grid), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL((grouped_gemm_f32<MODE>), dim3(a.grid), dim3(256), 0, s, a);
    return check_launch(what);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_ffn(const void *x_perm, int dtype, int64_t P, int64_t h, int64_t F,
                               int E, const int32_t *offsets, int act_kind, const void *w1,
                               const void *b1, const void *w2, const void *b2, const void *x_sh,
                               int64_t T_sh, const void *w1_sh, const void *w2_sh, void *act,
                               void *gu, void *y, void *y_sh, void *stream) {
    clear_error();
    MOE_CHECK_ARG(offsets && w1 && w2 && act && y, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: null required pointer");
    MOE_CHECK_ARG(P == 0 || x_perm, MOE_ERR_INVALID_ARG, "moe_grouped_ffn: null x_perm");
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
    MOE_CHECK_ARG(gu == nullptr || act_kind == MOE_ACT_SWIGLU, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn: gu is kept for SwiGLU only");
    const void *ptrs[] = {x_perm, w1, b1, w2, b2, x_sh, w1_sh, w2_sh, act, gu, y, y_sh};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(p == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,
                      "moe_grouped_ffn: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
    const int n1 = act_kind == MOE_ACT_SWIGLU ? 2 : 1;

    // first projection + activation
    GGArgs g1{};
    g1.A = x_perm;
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
    g1.E = E;
    g1.N_out = static_cast<int>(F);
    g1.K = static_cast<int>(h);
    int st = act_kind == MOE_ACT_SWIGLU ? launch_gemm<kModeSwiGLU>(g1, dtype, P, s, "moe_grouped_ffn gemm1")
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
    return launch_gemm<kModePlain>(g2, dtype, P, s, "moe_grouped_ffn gemm2");
}
