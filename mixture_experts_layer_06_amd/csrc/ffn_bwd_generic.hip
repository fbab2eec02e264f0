// Backward of the grouped FFN for the experts the bf16 SwiGLU kernels of
// ffn_bwd.hip do not cover: Linear + GELU(erf) + Linear with biases (the
// expert of "emerging-techniques-moe-training", Quick Start) in bf16 or fp32,
// and SwiGLU in fp32; plus the bias gradients of every expert kind.
//
// Per segment e (rows of expert e), with dY = grad_y and the pre-activations
// kept by the forward (GELU: a = X W1[e]^T + b1[e]; SwiGLU: g, u):
//   dact      = dY W2[e]
//   GELU:     da = dact * gelu'(a),  gelu'(a) = Phi(a) + a phi(a)
//   SwiGLU:   dg = dact * u * silu'(g),  du = dact * silu(g)
//   dX        = da W1[e]
//   dW2[e]    = dY_e^T act_e,   dW1[e] = da_e^T X_e
//   db2[e]    = column sums of dY_e,  db1[e] = column sums of da_e
//
// One segmented GEMM kernel does all four products: C[i][j] = sum_k L(i, k)
// R(k, j) with strided operands, 64 x 64 output tiles, 16-deep k-steps
// staged in LDS, 4 x 4 outputs per thread, fp32 FMA in ascending k (so the
// results are deterministic). These layers are small (the largest such
// workload is the 256-token fp32 layer), so the kernel favours plainness
// over speed; the large SwiGLU layers keep the matrix-core kernels.
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kGT = 64;   // output tile edge
constexpr int kGK = 16;   // k-step

enum GenEpi { kEpiStore = 0, kEpiStoreF32 = 1, kEpiGeluBwd = 2, kEpiSwigluBwd = 3 };

// Data-gradient form: rows of C are the segments' rows (expert e = segment
// of the row block), C [P][N] = B [P][K] (row stride ldb) times W[e] stored
// [K][N] (row stride N, expert stride w_stride).
// Weight-gradient form: per expert e, C[e] [M][N] = sum over the segment's
// rows r of L[r][i] R[r][j] (row strides ldl, ldr), fp32 out.
template <typename TE>
struct GenArgs {
    const TE *L;            // dgrad: B [P][K]; wgrad: the left rows [P][M]
    const TE *R;            // dgrad: W [E][K][N]; wgrad: the right rows [P][N]
    void *C;                // dgrad: [P][N] (TE; epilogue outputs below); wgrad: [E][M][N] fp32
    const TE *pre;          // GELU: a [P][N]; SwiGLU: g, u [P][2N]
    TE *dpre;               // GELU: da [P][N]; SwiGLU: dg, du [P][2N]
    const int32_t *offsets; // [E+1]
    int E, M, N, K;         // wgrad: M rows of C per expert; dgrad: K reduction length
    int ldl, ldr;
    int64_t w_stride;
    int n_tiles;            // dgrad: N tiles; wgrad: M tiles * N tiles
    int grid;
};

__device__ __forceinline__ float gelu_grad(float a) {
    const float phi = 0.3989422804014327f * expf(-0.5f * a * a);
    return 0.5f * (1.0f + erff(a * 0.70710678118654752f)) + a * phi;
}

// One 64 x 64 tile: rows [r0, r0 + nr) of the left operand (dgrad: of the
// segment; wgrad: indices into the expert's M rows), columns [c0, c0 + 64),
// k over [k0, k1) (wgrad: the segment's row range).
template <typename TE, bool WG, int EPI>
__device__ void gen_tile(const GenArgs<TE> &a, int e, int r0, int nr, int c0, int k0, int k1, float (*sl)[kGT + 1],
                         float (*sr)[kGT + 1]) {
    const int tid = threadIdx.x;
    const int tr = tid >> 4, tc = tid & 15;   // this thread: rows 4 tr .., columns 4 tc ..
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    const int ncol = WG ? a.N : a.N;
    const TE *Rbase = WG ? a.R : a.R + static_cast<int64_t>(e) * a.w_stride;
    for (int kb = k0; kb < k1; kb += kGK) {
        // stage L (64 rows x 16 k) and R (16 k x 64 columns); 4 elements of each per thread
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u;           // 0 .. 1023
            const int kk = idx >> 6, ii = idx & 63;  // k within the step, row/column within the tile
            const int k = kb + kk;
            float lv = 0.0f, rv = 0.0f;
            if (k < k1) {
                if (ii < nr) {
                    // dgrad: L(i, k) = B[r0 + i][k]; wgrad: L(i, k) = Lrows[k][r0 + i]
                    lv = WG ? Elem<TE>::load(a.L, static_cast<int64_t>(k) * a.ldl + r0 + ii)
                            : Elem<TE>::load(a.L, static_cast<int64_t>(r0 + ii) * a.ldl + k);
                }
                if (c0 + ii < ncol) {
                    // dgrad: R(k, j) = W[e][k][j]; wgrad: R(k, j) = Rrows[k][j]
                    rv = WG ? Elem<TE>::load(Rbase, static_cast<int64_t>(k) * a.ldr + c0 + ii)
                            : Elem<TE>::load(Rbase, static_cast<int64_t>(k) * a.N + c0 + ii);
                }
            }
            sl[kk][ii] = lv;
            sr[kk][ii] = rv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGK; ++kk) {
            float lv[4], rv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) lv[i] = sl[kk][4 * tr + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) rv[j] = sr[kk][4 * tc + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(lv[i], rv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ri = 4 * tr + i;
        if (ri >= nr) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 + 4 * tc + j;
            if (c >= ncol) continue;
            const float v = acc[i][j];
            if (WG) {
                float *C = static_cast<float *>(a.C) + static_cast<int64_t>(e) * a.M * a.N;
                C[static_cast<int64_t>(r0 + ri) * a.N + c] = v;
            } else {
                const int64_t r = r0 + ri;
                if (EPI == kEpiStore) {
                    Elem<TE>::store(static_cast<TE *>(a.C), r * a.N + c, v);
                } else if (EPI == kEpiGeluBwd) {
                    const float pa = Elem<TE>::load(a.pre, r * a.N + c);
                    Elem<TE>::store(a.dpre, r * a.N + c, v * gelu_grad(pa));
                } else if (EPI == kEpiSwigluBwd) {
                    const float g = Elem<TE>::load(a.pre, r * 2 * a.N + c);
                    const float u = Elem<TE>::load(a.pre, r * 2 * a.N + a.N + c);
                    const float s = 1.0f / (1.0f + expf(-g));
                    Elem<TE>::store(a.dpre, r * 2 * a.N + c, v * u * (s * (1.0f + g * (1.0f - s))));
                    Elem<TE>::store(a.dpre, r * 2 * a.N + a.N + c, v * (g * s));
                }
            }
        }
    }
}

// Data-gradient form over the segments: tiles of 64 segment rows by 64
// columns, listed on the device from the offsets (persistent blocks).
template <typename TE, int EPI>
__global__ __launch_bounds__(256) void gen_dgrad_kernel(GenArgs<TE> a) {
    __shared__ float sl[kGK][kGT + 1];
    __shared__ float sr[kGK][kGT + 1];
    __shared__ int s_cum[kMaxSeg];
    __shared__ int s_tmp[256];
    GGArgs g{};
    g.offsets = a.offsets;
    g.E = a.E;
    g.n_tiles = a.n_tiles;
    const int total = build_tile_prefix(g, kGT, s_cum, s_tmp);
    for (int L = blockIdx.x; L < total; L += a.grid) {
        const TileInfo ti = decode_tile(g, s_cum, L, kGT);
        const int nr = min(kGT, ti.M - ti.m0);
        gen_tile<TE, false, EPI>(a, ti.seg, ti.row0 + ti.m0, nr, ti.n_tile * kGT, 0, a.K, sl, sr);
    }
}

// Weight-gradient form: block b takes tiles b, b + grid, ... of the E x
// (M tiles x N tiles) list; an expert without rows gets zeros.
template <typename TE>
__global__ __launch_bounds__(256) void gen_wgrad_kernel(GenArgs<TE> a) {
    __shared__ float sl[kGK][kGT + 1];
    __shared__ float sr[kGK][kGT + 1];
    const int ntm = (a.M + kGT - 1) / kGT;
    const int total = a.E * a.n_tiles;
    for (int L = blockIdx.x; L < total; L += a.grid) {
        const int e = L / a.n_tiles, t = L % a.n_tiles;
        const int mt = t % ntm, nt = t / ntm;
        const int k0 = a.offsets[e], k1 = a.offsets[e + 1];
        gen_tile<TE, true, kEpiStoreF32>(a, e, mt * kGT, min(kGT, a.M - mt * kGT), nt * kGT, k0, k1, sl, sr);
    }
}

// db[e][c] = sum over the rows of segment e (ascending) of M[r][c], fp32; one
// thread per (expert, column).
template <typename TE>
__global__ __launch_bounds__(256) void seg_colsum_kernel(const TE *__restrict__ M, int N, const int32_t *offsets,
                                                         int E, float *__restrict__ db) {
    const int e = blockIdx.y;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E || c >= N) return;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    float s = 0.0f;
    for (int r = r0; r < r1; ++r) s += Elem<TE>::load(M, static_cast<int64_t>(r) * N + c);
    db[static_cast<int64_t>(e) * N + c] = s;
}

template <typename TE, int EPI>
int launch_dgrad(GenArgs<TE> a, int64_t P, hipStream_t s, const char *what) {
    a.n_tiles = (a.N + kGT - 1) / kGT;
    const int64_t upper = (P / kGT + a.E) * static_cast<int64_t>(a.n_tiles);
    int64_t grid = static_cast<int64_t>(num_cus()) * 4;
    if (grid > upper) grid = upper;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    hipLaunchKernelGGL((gen_dgrad_kernel<TE, EPI>), dim3(a.grid), dim3(256), 0, s, a);
    return check_launch(what);
}

template <typename TE>
int launch_wgrad(GenArgs<TE> a, hipStream_t s, const char *what) {
    a.n_tiles = ((a.M + kGT - 1) / kGT) * ((a.N + kGT - 1) / kGT);
    int64_t grid = static_cast<int64_t>(num_cus()) * 4;
    const int64_t upper = static_cast<int64_t>(a.E) * a.n_tiles;
    if (grid > upper) grid = upper;
    if (grid < 1) grid = 1;
    a.grid = static_cast<int>(grid);
    hipLaunchKernelGGL(gen_wgrad_kernel<TE>, dim3(a.grid), dim3(256), 0, s, a);
    return check_launch(what);
}

template <typename TE>
int launch_colsum(const TE *M, int N, const int32_t *offsets, int E, float *db, hipStream_t s, const char *what) {
    hipLaunchKernelGGL(seg_colsum_kernel<TE>, dim3((N + 255) / 256, E), dim3(256), 0, s, M, N, offsets, E, db);
    return check_launch(what);
}

template <typename TE>
int ffn_bwd_generic_t(const void *grad_y, const void *x_perm, const void *act, const void *gu, int64_t P, int64_t h,
                      int64_t F, int E, const int32_t *offsets, bool swiglu, const void *w1, const void *w2,
                      void *grad_gu, void *grad_x_perm, float *grad_w1, float *grad_w2, float *grad_b1,
                      float *grad_b2, hipStream_t s) {
    const int hi = static_cast<int>(h), Fi = static_cast<int>(F), n1 = swiglu ? 2 : 1;
    const TE *dY = static_cast<const TE *>(grad_y);
    TE *dA = static_cast<TE *>(grad_gu);
    int st;
    // dact = dY W2[e] (W2[e] stored [h][F]: k = h rows of F), activation backward fused
    GenArgs<TE> d2{};
    d2.L = dY;
    d2.R = static_cast<const TE *>(w2);
    d2.pre = static_cast<const TE *>(gu);
    d2.dpre = dA;
    d2.offsets = offsets;
    d2.E = E;
    d2.N = Fi;
    d2.K = hi;
    d2.ldl = hi;
    d2.w_stride = static_cast<int64_t>(h) * F;
    st = swiglu ? launch_dgrad<TE, kEpiSwigluBwd>(d2, P, s, "moe_grouped_ffn_bwd dact")
                : launch_dgrad<TE, kEpiGeluBwd>(d2, P, s, "moe_grouped_ffn_bwd dact");
    if (st != MOE_OK) return st;
    // dX = dA W1[e] (W1[e] stored [n1 F][h])
    GenArgs<TE> d1{};
    d1.L = dA;
    d1.R = static_cast<const TE *>(w1);
    d1.C = grad_x_perm;
    d1.offsets = offsets;
    d1.E = E;
    d1.N = hi;
    d1.K = n1 * Fi;
    d1.ldl = n1 * Fi;
    d1.w_stride = static_cast<int64_t>(n1) * F * h;
    st = launch_dgrad<TE, kEpiStore>(d1, P, s, "moe_grouped_ffn_bwd dx");
    if (st != MOE_OK) return st;
    // dW2[e] [h][F] = dY_e^T act_e
    GenArgs<TE> w2g{};
    w2g.L = dY;
    w2g.R = static_cast<const TE *>(act);
    w2g.C = grad_w2;
    w2g.offsets = offsets;
    w2g.E = E;
    w2g.M = hi;
    w2g.N = Fi;
    w2g.ldl = hi;
    w2g.ldr = Fi;
    st = launch_wgrad<TE>(w2g, s, "moe_grouped_ffn_bwd dW2");
    if (st != MOE_OK) return st;
    // dW1[e] [n1 F][h] = dA_e^T X_e
    GenArgs<TE> w1g{};
    w1g.L = dA;
    w1g.R = static_cast<const TE *>(x_perm);
    w1g.C = grad_w1;
    w1g.offsets = offsets;
    w1g.E = E;
    w1g.M = n1 * Fi;
    w1g.N = hi;
    w1g.ldl = n1 * Fi;
    w1g.ldr = hi;
    st = launch_wgrad<TE>(w1g, s, "moe_grouped_ffn_bwd dW1");
    if (st != MOE_OK) return st;
    if (grad_b2) {
        st = launch_colsum<TE>(dY, hi, offsets, E, grad_b2, s, "moe_grouped_ffn_bwd db2");
        if (st != MOE_OK) return st;
    }
    if (grad_b1) st = launch_colsum<TE>(dA, n1 * Fi, offsets, E, grad_b1, s, "moe_grouped_ffn_bwd db1");
    return st;
}

}  // namespace

// The whole backward of GELU experts (bf16 or fp32) and fp32 SwiGLU experts;
// grad_b1 / grad_b2 may be NULL.
int ffn_bwd_generic(const void *grad_y, const void *x_perm, const void *act, const void *gu, int dtype, int64_t P,
                    int64_t h, int64_t F, int E, const int32_t *offsets, int act_kind, const void *w1, const void *w2,
                    void *grad_gu, void *grad_x_perm, float *grad_w1, float *grad_w2, float *grad_b1,
                    float *grad_b2, hipStream_t s) {
    const bool swiglu = act_kind == MOE_ACT_SWIGLU;
    if (dtype == MOE_DTYPE_BF16)
        return ffn_bwd_generic_t<bf16_t>(grad_y, x_perm, act, gu, P, h, F, E, offsets, swiglu, w1, w2, grad_gu,
                                         grad_x_perm, grad_w1, grad_w2, grad_b1, grad_b2, s);
    return ffn_bwd_generic_t<float>(grad_y, x_perm, act, gu, P, h, F, E, offsets, swiglu, w1, w2, grad_gu,
                                    grad_x_perm, grad_w1, grad_w2, grad_b1, grad_b2, s);
}

// Bias gradients alone (the bf16 SwiGLU path): db[e] = column sums of M over
// segment e, M bf16 [P][N].
int segment_colsums_bf16(const void *M, int N, const int32_t *offsets, int E, float *db, hipStream_t s,
                         const char *what) {
    return launch_colsum<bf16_t>(static_cast<const bf16_t *>(M), N, offsets, E, db, s, what);
}

}  // namespace moe
