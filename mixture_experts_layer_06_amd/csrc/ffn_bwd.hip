// Backward of the grouped SwiGLU FFN: four grouped GEMMs per step.
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
// One kernel template serves all four. The MFMA (v_mfma_f32_32x32x16_bf16)
// reads both operands K-contiguous from LDS. Operands stored with K as the
// slow index (weights [K][cols] in the two data-gradient GEMMs, activations
// [tokens][cols] in the weight-gradient GEMMs) are transposed on the way to
// LDS: a thread loads an 8 x 8 block (eight 16-byte rows), transposes it in
// registers with byte permutes and writes eight K-contiguous 16-byte rows.
// Weight-gradient tiles cover the whole K range of their expert (no split-K,
// so results are deterministic), are ordered heaviest expert first, and
// experts without tokens get zero gradients.
#include "gemm_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

enum BwdKind { kDgradSwiGLU = 0, kDgradPlain = 1, kWgrad = 2 };

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
};

constexpr int TILE = 256, BK = 64, STAGE = 2 * TILE * BK;

// Column c of an 8 x 8 bf16 block whose row j is in[j] (8 elements in 4
// dwords): element j of the result is in[j][c]. Built from byte permutes.
__device__ __forceinline__ u32x4 column8(const u32x4 *in, int c) {
    const int p = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = __builtin_amdgcn_perm(in[2 * t + 1][p], in[2 * t][p], sel);
    return o;
}

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }

template <int KIND>
__global__ __launch_bounds__(512, 1) void bwd_gemm(BGArgs a) {
    constexpr int NS = 2, MS = 4;
    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    __shared__ int s_order[256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 3, wm = wave >> 2;
    const int l32 = lane & 31, lhi = lane >> 5;
    const bool loads_a = wave < 4;       // waves 0..3 stage A, waves 4..7 stage B
    const int lt = tid & 255;

    // ---------------------------------------------------------- schedule
    int total;
    if (KIND == kWgrad) {
        // experts by decreasing token count (ties: lower index first)
        if (tid < 256) {
            const int m = tid < a.E ? a.offsets[tid + 1] - a.offsets[tid] : -1;
            s_tmp[tid] = m;
        }
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
        total = build_tile_prefix_bal(g, s_cum, s_tmp);
    }

    for (int L = xcd_block_index(blockIdx.x, a.grid); L < total; L += a.grid) {
        int e, a_tile, row0, K, nact, rows = 0, b0 = 0, row_lo = 0;
        if (KIND == kWgrad) {
            const int per = a.n_tiles_a * a.n_tiles_b;
            e = s_order[L / per];
            const int local = L % per;
            a_tile = local % a.n_tiles_a;
            b0 = (local / a.n_tiles_a) * TILE;
            row0 = a.offsets[e];
            K = a.offsets[e + 1] - row0;
            nact = MS * 2;
        } else {
            GGArgs g{};
            g.offsets = a.offsets;
            g.E = a.E;
            g.n_tiles = a.n_tiles_a;
            const BalTile ti = decode_tile_bal(g, s_cum, L);
            e = ti.seg;
            a_tile = ti.n_tile;
            row0 = ti.row0;
            row_lo = ti.row_lo;
            rows = ti.rows;
            K = a.K;
            nact = (rows + 31) >> 5;
        }
        int nw = nact - wm * MS;
        nw = nw < 0 ? 0 : (nw > MS ? MS : nw);
        nw = __builtin_amdgcn_readfirstlane(nw);   // wave-uniform
        const int a0 = a_tile * TILE;
        const int nk = (K + BK - 1) / BK;

        // ---- per-thread staging geometry: waves 0..3 stage A, waves 4..7 B.
        // K-major operand: block (cb = lt & 31, kb = lt >> 5) covers storage
        // rows k0 + 8 kb + j (j < 8) and columns c0 + 8 cb .. +7, transposed
        // into LDS rows 8 cb + c. Row-major operand (B of the data-gradient
        // GEMMs): 16-byte chunk lt & 7 of tile rows (lt >> 3) + 32 j.
        const bool ks_loader = loads_a || KIND == kWgrad;
        const int cb = lt & 31, kb = lt >> 5;
        const int ks_ld = loads_a ? a.lda : a.ldb;
        const bool col_ok = loads_a ? (a0 + 8 * cb < a.a_dim) : (KIND != kWgrad || b0 + 8 * cb < a.b_dim);
        const bf16_t *base;
        if (loads_a)
            base = (KIND == kWgrad ? a.A + static_cast<int64_t>(row0) * a.lda
                                   : a.A + static_cast<int64_t>(e) * a.a_expert_stride) + a0 + 8 * cb;
        else if (KIND == kWgrad)
            base = a.B + static_cast<int64_t>(row0) * a.ldb + b0 + 8 * cb;
        else
            base = a.B + (static_cast<int64_t>(row0) + row_lo) * a.ldb + (lt & 7) * 8;
        const int ks_off = loads_a ? 0 : TILE * BK;

        floatx16 acc[NS][MS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int j = 0; j < MS; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        u32x4 v[8];

#define MOE_BWD_LOAD(kt_)                                                                     \
    do {                                                                                    \
        const int k0_ = (kt_) * BK;                                                         \
        if (ks_loader) {                                                                    \
            _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                 \
                const int k = k0_ + 8 * kb + j;                                             \
                u32x4 z = {0u, 0u, 0u, 0u};                                                 \
                if (col_ok && k < K)                                                        \
                    z = *reinterpret_cast<const u32x4 *>(base + static_cast<int64_t>(k) * ks_ld); \
                v[j] = z;                                                                   \
            }                                                                               \
        } else {                                                                            \
            _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                 \
                const int r = (lt >> 3) + 32 * j;                                           \
                v[j] = *reinterpret_cast<const u32x4 *>(base + (r < rows ? r : rows - 1) * ks_ld + k0_); \
            }                                                                               \
        }                                                                                   \
    } while (0)

#define MOE_BWD_STORE(buf_)                                                                   \
    do {                                                                                    \
        bf16_t *s_ = smem + (buf_) * STAGE + ks_off;                                        \
        if (ks_loader) {                                                                    \
            _Pragma("unroll") for (int c = 0; c < 8; ++c)                                   \
                *reinterpret_cast<u32x4 *>(s_ + swz(8 * cb + c, kb)) = column8(v, c);       \
        } else {                                                                            \
            _Pragma("unroll") for (int j = 0; j < 8; ++j)                                   \
                *reinterpret_cast<u32x4 *>(s_ + swz((lt >> 3) + 32 * j, lt & 7)) = v[j];    \
        }                                                                                   \
    } while (0)

        if (nk > 0) {
            MOE_BWD_LOAD(0);
            MOE_BWD_STORE(0);
        }
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) MOE_BWD_LOAD(kt + 1);
            const bf16_t *sa = smem + (kt & 1) * STAGE;
            const bf16_t *sb = sa + TILE * BK;
            if (nw > 0) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int ch = ks * 2 + lhi;
                    bf16x8_t af[NS], bfr[MS];
#pragma unroll
                    for (int i = 0; i < NS; ++i)
                        af[i] = *reinterpret_cast<const bf16x8_t *>(sa + swz(wn * 64 + i * 32 + l32, ch));
#pragma unroll
                    for (int j = 0; j < MS; ++j)
                        bfr[j] = *reinterpret_cast<const bf16x8_t *>(sb + swz(wm * 128 + j * 32 + l32, ch));
#pragma unroll
                    for (int j = 0; j < MS; ++j)
                        if (j < nw)
#pragma unroll
                            for (int i = 0; i < NS; ++i)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                }
            }
            if (kt + 1 < nk) MOE_BWD_STORE((kt + 1) & 1);
            __syncthreads();
        }
#undef MOE_BWD_LOAD
#undef MOE_BWD_STORE

        // ---------------------------------------------------------- epilogue
#pragma unroll
        for (int j = 0; j < MS; ++j) {
            const int bl = wm * 128 + j * 32 + l32;   // row of C within the tile
            if (j >= nw) continue;
            if (KIND != kWgrad && bl >= rows) continue;
            if (KIND == kWgrad && b0 + bl >= a.b_dim) continue;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int col = a0 + wn * 64 + i * 32 + 8 * gq + 4 * lhi;
                    if (col >= a.a_dim) continue;
                    if (KIND == kWgrad) {
                        float4 o = make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                                               acc[i][j][4 * gq + 3]);
                        float *C = static_cast<float *>(a.C) +
                                   (static_cast<int64_t>(e) * a.b_dim + b0 + bl) * a.a_dim + col;
                        *reinterpret_cast<float4 *>(C) = o;
                    } else if (KIND == kDgradPlain) {
                        uint2 o;
                        o.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
                        o.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                        bf16_t *C = static_cast<bf16_t *>(a.C) +
                                    (static_cast<int64_t>(row0) + row_lo + bl) * a.a_dim + col;
                        *reinterpret_cast<uint2 *>(C) = o;
                    } else {
                        const int64_t r = static_cast<int64_t>(row0) + row_lo + bl;
                        const bf16_t *gr = a.GU + r * 2 * a.a_dim;
                        const uint2 gv = *reinterpret_cast<const uint2 *>(gr + col);
                        const uint2 uv = *reinterpret_cast<const uint2 *>(gr + a.a_dim + col);
                        const float g[4] = {bf16lo(gv.x), bf16hi(gv.x), bf16lo(gv.y), bf16hi(gv.y)};
                        const float u[4] = {bf16lo(uv.x), bf16hi(uv.x), bf16lo(uv.y), bf16hi(uv.y)};
                        float dg[4], du[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float d = acc[i][j][4 * gq + q];
                            const float s = 1.0f / (1.0f + expf(-g[q]));
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
    }
}

template <int KIND>
int launch_bwd(BGArgs a, int64_t P, hipStream_t s, const char *what) {
    a.n_tiles_a = (a.a_dim + TILE - 1) / TILE;
    int64_t upper;
    if (KIND == kWgrad) {
        a.n_tiles_b = (a.b_dim + TILE - 1) / TILE;
        upper = static_cast<int64_t>(a.E) * a.n_tiles_a * a.n_tiles_b;
    } else {
        a.n_tiles_b = 1;
        upper = (P / 256 + a.E) * static_cast<int64_t>(a.n_tiles_a);
    }
    int64_t grid = num_cus();
    if (grid > upper) grid = upper;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    hipLaunchKernelGGL((bwd_gemm<KIND>), dim3(a.grid), dim3(512), 0, s, a);
    return check_launch(what);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_ffn_bwd(const void *grad_y, const void *x_perm, const void *act,
                                   const void *gu, int dtype, int64_t P, int64_t h, int64_t F, int E,
                                   const int32_t *offsets, int act_kind, const void *w1,
                                   const void *w2, void *grad_gu, void *grad_x_perm, float *grad_w1,
                                   float *grad_w2, void *stream) {
    clear_error();
    MOE_CHECK_ARG(grad_y && x_perm && act && gu && offsets && w1 && w2 && grad_gu && grad_x_perm &&
                      grad_w1 && grad_w2,
                  MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd: null required pointer");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_bwd: bad dtype %d", dtype);
    MOE_CHECK_ARG(act_kind == MOE_ACT_GELU || act_kind == MOE_ACT_SWIGLU, MOE_ERR_INVALID_ARG,
                  "moe_grouped_ffn_bwd: bad activation %d", act_kind);
    MOE_CHECK_ARG(P >= 0 && h > 0 && F > 0 && E > 0, MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd: bad sizes");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_BF16 && act_kind == MOE_ACT_SWIGLU, MOE_ERR_UNSUPPORTED,
                  "moe_grouped_ffn_bwd: bf16 SwiGLU experts only");
    MOE_CHECK_ARG(h % 64 == 0 && F % 64 == 0 && E <= 256, MOE_ERR_UNSUPPORTED,
                  "moe_grouped_ffn_bwd: need h %% 64 == 0, F %% 64 == 0, E <= 256");
    MOE_CHECK_ARG(P < (int64_t(1) << 31) && h < (int64_t(1) << 20) && F < (int64_t(1) << 20) &&
                      P * (2 * F > h ? 2 * F : h) < (int64_t(1) << 31),
                  MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_bwd: sizes too large");
    const void *ptrs[] = {grad_y, x_perm, act, gu, w1, w2, grad_gu, grad_x_perm, grad_w1, grad_w2};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(aligned16(p), MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    const bf16_t *dY = static_cast<const bf16_t *>(grad_y);
    const bf16_t *X = static_cast<const bf16_t *>(x_perm);
    const bf16_t *H = static_cast<const bf16_t *>(act);
    bf16_t *dGU = static_cast<bf16_t *>(grad_gu);
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
    int st = launch_bwd<kDgradSwiGLU>(d2, P, s, "moe_grouped_ffn_bwd dact");
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
