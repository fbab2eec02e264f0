// Expert computation: one grouped GEMM launch per projection over all
// experts' ragged segments ("Scalable Training of Mixture-of-Experts Models
// with Megatron Core", section 2.1 stage 3: all local experts in a single
// grouped GEMM call). SwiGLU experts without bias ("Mixture-of-Experts from
// Architecture to Large-Scale Training", section 2.5: gate, up and down
// matrices) or GELU(erf) experts with biases ("emerging-techniques-moe-
// training", Quick Start).
//
// bf16 kernel, CDNA4 (gfx950):
// - MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulators. The weight tile is the
//   MFMA "A" operand and the token tile the "B" operand, so a lane's four
//   accumulators are four consecutive output columns of one token row and the
//   epilogue writes 8-byte row pieces.
// - Tiles BM tokens x BN weight rows x 64 deep; 4 waves in a 2 x 2 grid.
//   Operands are staged global -> registers -> LDS (double-buffered, one
//   barrier per k-step) with 16-byte accesses; LDS rows are 128 bytes and
//   16-byte chunk c of row r is stored at chunk c ^ (r % 8), so the 16 rows a
//   fragment read touches fall in distinct bank groups.
// - SwiGLU: the weight tile interleaves 16-row blocks of gate rows and up rows
//   of the same 16 output columns, so each lane holds the gate and up values
//   of the same output element and applies silu(g) * u in registers.
// - Persistent blocks walk a device-built tile list (segments x m-tiles x
//   n-tiles, m fastest) with XCD-aware numbering.
#include "gemm_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Tile: 256 weight rows (n) x up to 256 token rows (m) x 64 deep, 8 waves.
// Wave w owns weight rows [64 (w%4), +64) (two 32-row MFMA subtiles) and
// token rows [128 (w/4), +128) (four 32-row subtiles). Waves w and w+4 share a
// SIMD, so a tile with few rows leaves half of each SIMD's work undone rather
// than idling whole SIMDs; subtiles past the tile's row count are skipped.
// MFMA v_mfma_f32_32x32x16_bf16: lane l supplies row l%32, k = 8(l/32)..+7
// of each operand; accumulator element i of lane l is row
// 8(i/4) + 4(l/32) + i%4 (weight row) and column l%32 (token row).
template <int MODE>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bf16(GGArgs a) {
    constexpr int BK = 64;
    constexpr int TILE = 256;
    constexpr int NS = 2, MS = 4;
    constexpr int STAGE = 2 * TILE * BK;        // elements per LDS stage (weights + tokens)
    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];
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
    const int nk = K / BK;
    const int chunk = tid & 7;
    const int rbase = tid >> 3;                 // rows rbase and rbase + 64 of each operand

    for (int L = xcd_block_index(blockIdx.x, a.grid); L < total; L += a.grid) {
        const BalTile ti = decode_tile_bal(a, s_cum, L);
        const int nact = (ti.rows + 31) >> 5;   // active 32-row token subtiles of the tile
        int nw = nact - wm * MS;                // ... of this wave
        nw = nw < 0 ? 0 : (nw > MS ? MS : nw);
        const bf16_t *Aseg = ti.shared ? static_cast<const bf16_t *>(a.A_sh)
                                       : static_cast<const bf16_t *>(a.A) + static_cast<int64_t>(ti.row0) * K;
        const bf16_t *xb = Aseg + static_cast<int64_t>(ti.row_lo) * K + chunk * 8;
        const bf16_t *wb = (ti.shared ? static_cast<const bf16_t *>(a.B_sh)
                                      : static_cast<const bf16_t *>(a.B) + static_cast<int64_t>(ti.seg) * nb_rows * K) +
                           chunk * 8;
        int woff[4], xoff[4], soff[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rbase + 64 * j;
            int wrow;
            if (MODE == kModeSwiGLU) {
                const int f = ti.n_tile * (TILE / 2) + (r >> 6) * 32 + (r & 31);
                wrow = ((r >> 5) & 1) ? a.N_out + f : f;
                if (f >= a.N_out) wrow = 0;
            } else {
                wrow = ti.n_tile * TILE + r;
                if (wrow >= nb_rows) wrow = 0;
            }
            woff[j] = wrow * K;
            xoff[j] = (r < ti.rows ? r : ti.rows - 1) * K;
            soff[j] = r * BK + ((chunk ^ (r & 7)) << 3);
        }

        floatx16 acc[NS][MS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int j = 0; j < MS; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        // rows past the tile were clamped to its last row above: every load is
        // in bounds and unconditional (their products land in skipped subtiles
        // or in rows the epilogue does not store)
        u32x4 rw[4], rx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rw[j] = *reinterpret_cast<const u32x4 *>(wb + woff[j]);
            rx[j] = *reinterpret_cast<const u32x4 *>(xb + xoff[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<u32x4 *>(smem + soff[j]) = rw[j];
            *reinterpret_cast<u32x4 *>(smem + TILE * BK + soff[j]) = rx[j];
        }
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = (kt & 1) * STAGE;
            if (kt + 1 < nk) {
                const int ko = (kt + 1) * BK;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    rw[j] = *reinterpret_cast<const u32x4 *>(wb + woff[j] + ko);
                    rx[j] = *reinterpret_cast<const u32x4 *>(xb + xoff[j] + ko);
                }
            }
            const bf16_t *sw = smem + cur;
            const bf16_t *sx = smem + cur + TILE * BK;
            if (nw > 0) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int ch = ks * 2 + lhi;
                    bf16x8_t af[NS], bfr[MS];
#pragma unroll
                    for (int i = 0; i < NS; ++i) {
                        const int r = wn * 64 + i * 32 + l32;
                        af[i] = *reinterpret_cast<const bf16x8_t *>(sw + r * BK + ((ch ^ (r & 7)) << 3));
                    }
#pragma unroll
                    for (int j = 0; j < MS; ++j) {
                        const int r = wm * 128 + j * 32 + l32;
                        bfr[j] = *reinterpret_cast<const bf16x8_t *>(sx + r * BK + ((ch ^ (r & 7)) << 3));
                    }
                    if (nw == MS) {
#pragma unroll
                        for (int j = 0; j < MS; ++j)
#pragma unroll
                            for (int i = 0; i < NS; ++i)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    } else {
#pragma unroll
                        for (int j = 0; j < MS; ++j)
                            if (j < nw)
#pragma unroll
                                for (int i = 0; i < NS; ++i)
                                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    }
                }
            }
            if (kt + 1 < nk) {
                const int nxt = ((kt + 1) & 1) * STAGE;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    *reinterpret_cast<u32x4 *>(smem + nxt + soff[j]) = rw[j];
                    *reinterpret_cast<u32x4 *>(smem + nxt + TILE * BK + soff[j]) = rx[j];
                }
            }
            __syncthreads();
        }

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
