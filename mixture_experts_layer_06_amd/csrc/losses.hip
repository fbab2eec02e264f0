// Auxiliary router losses and the router backward of a dense logit gradient.
//
// "emerging-techniques-moe-training", section 3 (Load Balancing):
//   load-balancing loss  aux = E * sum_e f_e P_e,
//     f_e = share of the T*k routing slots that chose expert e (from counts),
//     P_e = mean over tokens of softmax(l_t)_e (softmax over all E logits);
//   router z-loss        z = mean over tokens of logsumexp(l_t)^2.
// Both read the router's logits (gate bias included, selection bias not),
// whatever the scoring function. f_e is piecewise constant in the logits and
// carries no gradient, so
//   d aux / d l_{t,j} = (E/T) p_{t,j} (f_j - sum_e f_e p_{t,e}),
//   d z   / d l_{t,j} = (2/T) lse_t p_{t,j}.
// That gradient is dense over the experts; moe_router_dense_bwd turns any
// dense logit gradient D [T,E] into the router's weight, bias and input
// gradients: grad_w_gate += D^T x, grad_b_gate += column sums of D,
// grad_x += D w_gate.
//
// Every reduction has a fixed order (no floating-point atomics): per-token
// quantities over the experts by a wave-wide shuffle tree, sums over tokens
// in token-chunk order. With bf16 operands and a multiple of 32 experts the
// two dense products of the router backward run on MFMA (see below), else on
// the vector ALU.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kLossMaxE = 256;
constexpr int kLossChunk = 32;      // tokens per partial sum of the forward (8 per wave)
constexpr int kDenseChunk = 256;    // tokens per partial weight-gradient sum
constexpr int kDenseCols = 512;     // columns per weight-gradient block (64 threads x 8)
constexpr int kDenseExp = 8;        // experts per weight-gradient block

// Softmax statistics of one token's logits, held by a wave: lane l has
// experts l + 64 m. Returns the row maximum and the sum of exp(l - max) in
// every lane (shuffle tree, fixed order).
__device__ __forceinline__ void row_softmax_stats(const float *lrow, int E, int lane, float (&v)[4], float &mx,
                                                  float &sum) {
    mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        v[m] = e < E ? lrow[e] : -INFINITY;
        mx = fmaxf(mx, v[m]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    sum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        v[m] = e < E ? expf(v[m] - mx) : 0.0f;
        sum += v[m];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
}

// Pass 1: block b sums, over its chunk of kLossChunk tokens, p_{t,e} for every
// expert and lse_t^2. Wave w takes tokens w, w+4, ... of the chunk; the four
// waves' sums are then added in wave order. partial[b][0..E) and [E].
// Each wave's tokens are independent: the loop is unrolled so that their
// loads and shuffle trees overlap.
__global__ __launch_bounds__(256) void losses_partial_kernel(const float *__restrict__ logits, int T, int E,
                                                             float *__restrict__ partial) {
    __shared__ float s_p[4][kLossMaxE + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kLossChunk;
    float pacc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, zacc = 0.0f;
#pragma unroll 2
    for (int tt = wave; tt < kLossChunk; tt += 4) {
        const int t = t0 + tt;
        if (t >= T) break;
        float v[4], mx, sum;
        row_softmax_stats(logits + static_cast<int64_t>(t) * E, E, lane, v, mx, sum);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int m = 0; m < 4; ++m) pacc[m] += v[m] * inv;
        const float lse = mx + logf(sum);
        zacc = fmaf(lse, lse, zacc);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        if (e < E) s_p[wave][e] = pacc[m];
    }
    if (lane == 0) s_p[wave][kLossMaxE] = zacc;
    __syncthreads();
    float *out = partial + static_cast<int64_t>(blockIdx.x) * (E + 1);
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        const int src = e == E ? kLossMaxE : e;
        out[e] = ((s_p[0][src] + s_p[1][src]) + s_p[2][src]) + s_p[3][src];
    }
}

// Pass 2 (one block of 1024 threads, E <= 256): P_e and z from the chunk
// sums, thread group g (of 4) summing chunks g, g + 4, ... in ascending order
// and the four group sums added in group order; then aux = E sum_e f_e P_e
// (a fixed tree over the experts).
__global__ __launch_bounds__(1024) void losses_final_kernel(const float *__restrict__ partial, int nb, int T, int E,
                                                            int k, const int32_t *__restrict__ counts,
                                                            float *__restrict__ losses, float *__restrict__ pmean) {
    __shared__ float s_sum[4][kLossMaxE + 1];
    __shared__ float s_fp[256];
    const int e = threadIdx.x & 255, g = threadIdx.x >> 8;
    const int64_t stride = E + 1;
    if (e < E) {
        float s = 0.0f;
#pragma unroll 16
        for (int b = g; b < nb; b += 4) s += partial[b * stride + e];
        s_sum[g][e] = s;
    }
    if (e == 0) {
        float s = 0.0f;
#pragma unroll 16
        for (int b = g; b < nb; b += 4) s += partial[b * stride + E];
        s_sum[g][kLossMaxE] = s;
    }
    __syncthreads();
    if (g == 0) {
        float term = 0.0f;
        if (e < E) {
            const float mean = (((s_sum[0][e] + s_sum[1][e]) + s_sum[2][e]) + s_sum[3][e]) / static_cast<float>(T);
            if (pmean) pmean[e] = mean;
            const float f = static_cast<float>(counts[e]) / (static_cast<float>(T) * static_cast<float>(k));
            term = f * mean;
        }
        if (e == 0)
            losses[1] = (((s_sum[0][kLossMaxE] + s_sum[1][kLossMaxE]) + s_sum[2][kLossMaxE]) + s_sum[3][kLossMaxE]) /
                        static_cast<float>(T);   // z
        s_fp[e] = term;
    }
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (static_cast<int>(threadIdx.x) < st) s_fp[threadIdx.x] += s_fp[threadIdx.x + st];
        __syncthreads();
    }
    if (threadIdx.x == 0) losses[0] = static_cast<float>(E) * s_fp[0];
}

// Dense logit gradient of coef_aux * aux + coef_z * z: one wave per token.
__global__ __launch_bounds__(256) void losses_bwd_kernel(const float *__restrict__ logits,
                                                         const int32_t *__restrict__ counts, int T, int E, int k,
                                                         float coef_aux, float coef_z, float *__restrict__ dl) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[4], mx, sum;
    row_softmax_stats(logits + static_cast<int64_t>(t) * E, E, lane, v, mx, sum);
    const float inv = 1.0f / sum, lse = mx + logf(sum);
    const float fden = static_cast<float>(T) * static_cast<float>(k);
    float f[4], a = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        v[m] *= inv;   // p_{t,e}
        f[m] = e < E ? static_cast<float>(counts[e]) / fden : 0.0f;
        a = fmaf(f[m], v[m], a);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
    const float ca = coef_aux * static_cast<float>(E) / static_cast<float>(T);
    const float cz = coef_z * 2.0f * lse / static_cast<float>(T);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        if (e < E) dl[static_cast<int64_t>(t) * E + e] = ca * v[m] * (f[m] - a) + cz * v[m];
    }
}

// grad_w_gate pass 1: block (column block cb, expert group eg, token chunk c)
// sums D[t,e] x[t, cols] over the chunk's tokens (ascending) for kDenseExp
// experts and kDenseCols columns (64 threads x 8 columns).
template <typename TE>
__global__ __launch_bounds__(64) void dense_wgrad_partial_kernel(const TE *__restrict__ x,
                                                                 const float *__restrict__ D, int T, int h, int E,
                                                                 float *__restrict__ partial) {
    const int cb = blockIdx.x, eg = blockIdx.y, c = blockIdx.z;
    const int col = cb * kDenseCols + 8 * threadIdx.x;
    const int e0 = eg * kDenseExp;
    float acc[kDenseExp][8];
#pragma unroll
    for (int j = 0; j < kDenseExp; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    const int tlo = c * kDenseChunk, thi = min(T, tlo + kDenseChunk);
    if (col < h) {
        for (int t = tlo; t < thi; ++t) {
            float xv[8];
            load8(x + static_cast<int64_t>(t) * h + col, xv);
            const float *drow = D + static_cast<int64_t>(t) * E + e0;
#pragma unroll
            for (int j = 0; j < kDenseExp; ++j) {
                const float d = e0 + j < E ? drow[j] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(d, xv[i], acc[j][i]);
            }
        }
#pragma unroll
        for (int j = 0; j < kDenseExp; ++j) {
            if (e0 + j >= E) continue;
            float *out = partial + (static_cast<int64_t>(c) * E + e0 + j) * h + col;
            *reinterpret_cast<float4 *>(out) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
            *reinterpret_cast<float4 *>(out + 4) = make_float4(acc[j][4], acc[j][5], acc[j][6], acc[j][7]);
        }
    }
}

// grad_w_gate pass 2: grad_w_gate[e][i] += sum over chunks (in order).
__global__ __launch_bounds__(256) void dense_wgrad_reduce_kernel(const float *__restrict__ partial, int nchunk,
                                                                 int64_t n, float *__restrict__ gw) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.0f;
#pragma unroll 8
    for (int c = 0; c < nchunk; ++c) s += partial[static_cast<int64_t>(c) * n + i];
    gw[i] += s;
}

// grad_b_gate[e] += sum_t D[t,e]: one block per expert, thread i sums tokens
// i, i + 256, ... (ascending), then a fixed tree over the threads.
__global__ __launch_bounds__(256) void dense_bgrad_kernel(const float *__restrict__ D, int T, int E,
                                                          float *__restrict__ gb) {
    __shared__ float s[256];
    const int e = blockIdx.x;
    float a = 0.0f;
#pragma unroll 8
    for (int t = threadIdx.x; t < T; t += 256) a += D[static_cast<int64_t>(t) * E + e];
    s[threadIdx.x] = a;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (static_cast<int>(threadIdx.x) < st) s[threadIdx.x] += s[threadIdx.x + st];
        __syncthreads();
    }
    if (threadIdx.x == 0) gb[e] += s[0];
}

// grad_x[t] += sum_e D[t,e] w_gate[e] (experts ascending, fp32, one rounding
// of the sum to the output type): block = 8 tokens x 512 columns (64 threads
// x 8 columns).
template <typename TE>
__global__ __launch_bounds__(64) void dense_xgrad_kernel(const TE *__restrict__ wg, const float *__restrict__ D,
                                                         int T, int h, int E, TE *__restrict__ gx) {
    const int col = blockIdx.x * kDenseCols + 8 * threadIdx.x;
    const int t0 = blockIdx.y * 8;
    if (col >= h) return;
    float acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] = 0.0f;
    for (int e = 0; e < E; ++e) {
        float wv[8];
        load8(wg + static_cast<int64_t>(e) * h + col, wv);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int t = t0 + r;
            const float d = t < T ? D[static_cast<int64_t>(t) * E + e] : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[r][i] = fmaf(d, wv[i], acc[r][i]);
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int t = t0 + r;
        if (t >= T) continue;
        TE *p = gx + static_cast<int64_t>(t) * h + col;
        float cur[8];
        load8(p, cur);
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] += acc[r][i];
        store8(p, cur);
    }
}

// ------------------------------------------------ dense backward on MFMA
//
// With bf16 token rows and router weights, D^T x and D w_gate run as bf16
// matrix products on the backward's GEMM kernel: D is split into a bf16
// high part and a bf16 low part (D = hi + lo to about 2^-16 relative), the
// two side by side as D2 [T][2E], so that each product is exact in fp32 and
// the sums keep fp32 accuracy:
//   D^T x   = rows 0..E-1 + rows E..2E-1 of D2^T x  (weight-gradient GEMM
//             over token chunks, partial sums added in chunk order)
//   D w_gate = D2 [w_gate; w_gate]                  (data-gradient GEMM)

// D2[t][e] = hi, D2[t][E + e] = lo.
__global__ __launch_bounds__(256) void split_hilo_kernel(const float *__restrict__ D, int64_t n, int E,
                                                         bf16_t *__restrict__ D2) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t t = i / E;
    const int e = static_cast<int>(i - t * E);
    const float d = D[i];
    const bf16_t hi = f32_to_bf16(d);
    const bf16_t lo = f32_to_bf16(d - bf16_to_f32(hi));
    D2[t * 2 * E + e] = hi;
    D2[t * 2 * E + E + e] = lo;
}

// W2 = [w; w]: 8 elements per thread.
__global__ __launch_bounds__(256) void stack_twice_kernel(const bf16_t *__restrict__ w, int64_t npieces,
                                                          bf16_t *__restrict__ w2) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= npieces) return;
    const uint4 q = reinterpret_cast<const uint4 *>(w)[i];
    reinterpret_cast<uint4 *>(w2)[i] = q;
    reinterpret_cast<uint4 *>(w2)[npieces + i] = q;
}

// offs[i] = min(i * chunk, T) for i <= nchunk; then {0, T}.
__global__ void chunk_offsets_kernel(int32_t *offs, int nchunk, int chunk, int T) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i <= nchunk) offs[i] = min(i * chunk, T);
    if (i == 0) {
        offs[nchunk + 1] = 0;
        offs[nchunk + 2] = T;
    }
}

// gw[e][c] += sum over chunks (in order) of P[ch][e][c] + P[ch][E + e][c].
__global__ __launch_bounds__(256) void hilo_reduce_kernel(const float *__restrict__ P, int nchunk, int E, int h,
                                                          float *__restrict__ gw) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n = static_cast<int64_t>(E) * h;
    if (i >= n) return;
    const int64_t stride = 2 * n;
    float s = 0.0f;
#pragma unroll 4
    for (int c = 0; c < nchunk; ++c) s += P[c * stride + i] + P[c * stride + n + i];
    gw[i] += s;
}

// gx += xo (bf16, fp32 add, one rounding): 8 elements per thread.
__global__ __launch_bounds__(256) void add_rows_kernel(const bf16_t *__restrict__ xo, int64_t npieces,
                                                       bf16_t *__restrict__ gx) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= npieces) return;
    float a[8], b[8];
    load8(gx + 8 * i, a);
    load8(xo + 8 * i, b);
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] += b[q];
    store8(gx + 8 * i, a);
}

struct DenseMfmaPlan {
    int nchunk, chunk;
    size_t off_w2, off_offs, off_part, off_xo, total;
};

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Token chunks so that the weight-gradient GEMM has about one tile per
// compute unit (tiles per chunk: ceil(h/256) * ceil(2E/256)), chunks of at
// least 256 tokens, a multiple of 64.
DenseMfmaPlan dense_mfma_plan(int64_t T, int64_t h, int E) {
    DenseMfmaPlan p{};
    const int64_t tiles = ((h + 255) / 256) * ((2 * E + 255) / 256);
    int64_t nchunk = (256 + tiles - 1) / tiles;
    const int64_t maxchunks = (T + 255) / 256;
    if (nchunk > maxchunks) nchunk = maxchunks;
    if (nchunk < 1) nchunk = 1;
    int64_t chunk = (T + nchunk - 1) / nchunk;
    chunk = (chunk + 63) & ~int64_t(63);
    nchunk = (T + chunk - 1) / chunk;
    p.nchunk = static_cast<int>(nchunk);
    p.chunk = static_cast<int>(chunk);
    p.off_w2 = align256(static_cast<size_t>(T) * 2 * E * sizeof(bf16_t));
    p.off_offs = p.off_w2 + align256(static_cast<size_t>(2 * E) * h * sizeof(bf16_t));
    p.off_part = p.off_offs + align256((nchunk + 3) * sizeof(int32_t));
    p.off_xo = p.off_part + align256(static_cast<size_t>(nchunk) * 2 * E * h * sizeof(float));
    p.total = p.off_xo + align256(static_cast<size_t>(T) * h * sizeof(bf16_t));
    return p;
}

// The GEMM kernel indexes a whole operand with 32-bit offsets.
bool dense_mfma_ok(int dtype, int64_t T, int64_t h, int E) {
    return dtype == MOE_DTYPE_BF16 && E >= 32 && E % 32 == 0 && h < (int64_t(1) << 20) &&
           T * (h > 2 * E ? h : 2 * E) < (int64_t(1) << 31);
}

}  // namespace

int bwd_wgrad_segments(const bf16_t *A, int lda, int a_dim, const bf16_t *B, int ldb, int b_dim,
                       const int32_t *offsets, int nseg, int64_t rows, float *C, hipStream_t s);
int bwd_dgrad_plain(const bf16_t *B, int ldb, const bf16_t *A, int lda, int a_dim, int K, const int32_t *offsets,
                    int nseg, int64_t P, bf16_t *C, hipStream_t s);

}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_losses_workspace_size(int64_t T, int E) {
    if (T <= 0 || E <= 0) return 0;
    const int64_t nb = (T + kLossChunk - 1) / kLossChunk;
    return static_cast<size_t>(nb) * static_cast<size_t>(E + 1) * sizeof(float);
}

extern "C" int moe_router_losses(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                                 float *losses, float *probs_mean, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    clear_error();
    MOE_CHECK_ARG(losses && counts && (T == 0 || logits), MOE_ERR_INVALID_ARG,
                  "moe_router_losses: null required pointer");
    MOE_CHECK_ARG(T >= 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG, "moe_router_losses: bad sizes");
    MOE_CHECK_ARG(E <= kLossMaxE && k <= E && T < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_router_losses: need k <= E <= 256, T < 2^31");
    hipStream_t s = as_stream(stream);
    if (T == 0) {
        launch_fill<float>(losses, 2, 0.0f, s);
        if (probs_mean) launch_fill<float>(probs_mean, E, 0.0f, s);
        return check_launch("moe_router_losses");
    }
    const size_t need = moe_router_losses_workspace_size(T, E);
    MOE_CHECK_ARG(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                  "moe_router_losses: workspace of %zu bytes needed", need);
    const int nb = static_cast<int>((T + kLossChunk - 1) / kLossChunk);
    float *partial = static_cast<float *>(workspace);
    hipLaunchKernelGGL(losses_partial_kernel, dim3(nb), dim3(256), 0, s, logits, static_cast<int>(T), E, partial);
    hipLaunchKernelGGL(losses_final_kernel, dim3(1), dim3(1024), 0, s, partial, nb, static_cast<int>(T), E, k,
                       counts, losses, probs_mean);
    return check_launch("moe_router_losses");
}

extern "C" int moe_router_losses_bwd(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                                     float coef_aux, float coef_z, float *grad_logits, void *stream) {
    clear_error();
    MOE_CHECK_ARG(counts && (T == 0 || (logits && grad_logits)), MOE_ERR_INVALID_ARG,
                  "moe_router_losses_bwd: null required pointer");
    MOE_CHECK_ARG(T >= 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG, "moe_router_losses_bwd: bad sizes");
    MOE_CHECK_ARG(E <= kLossMaxE && k <= E && T < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_router_losses_bwd: need k <= E <= 256, T < 2^31");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(losses_bwd_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s, logits, counts,
                       static_cast<int>(T), E, k, coef_aux, coef_z, grad_logits);
    return check_launch("moe_router_losses_bwd");
}

extern "C" size_t moe_router_dense_bwd_workspace_size(int64_t T, int64_t h, int E) {
    if (T <= 0 || h <= 0 || E <= 0) return 0;
    const int64_t nchunk = (T + kDenseChunk - 1) / kDenseChunk;
    const size_t valu = static_cast<size_t>(nchunk) * static_cast<size_t>(E) * static_cast<size_t>(h) * sizeof(float);
    const size_t mfma = E >= 32 && E % 32 == 0 ? dense_mfma_plan(T, h, E).total : 0;
    return valu > mfma ? valu : mfma;
}

extern "C" int moe_router_dense_bwd(const void *x, const void *w_gate, int dtype, int64_t T, int64_t h, int E,
                                    const float *grad_logits, float *grad_w_gate, float *grad_b_gate,
                                    void *grad_x, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_router_dense_bwd: bad dtype %d", dtype);
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0, MOE_ERR_INVALID_ARG, "moe_router_dense_bwd: bad sizes");
    MOE_CHECK_ARG(T == 0 || (grad_logits && (grad_w_gate == nullptr || x) && (grad_x == nullptr || w_gate)),
                  MOE_ERR_INVALID_ARG, "moe_router_dense_bwd: null required pointer");
    MOE_CHECK_ARG(h % 64 == 0 && E <= kLossMaxE && T < (int64_t(1) << 31) && h < (int64_t(1) << 31),
                  MOE_ERR_UNSUPPORTED, "moe_router_dense_bwd: need h %% 64 == 0, E <= 256");
    const void *ptrs[] = {x, w_gate, grad_w_gate, grad_x, workspace};
    for (const void *p : ptrs)
        MOE_CHECK_ARG(p == nullptr || aligned16(p), MOE_ERR_INVALID_ARG,
                      "moe_router_dense_bwd: pointers must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    const int TT = static_cast<int>(T), hh = static_cast<int>(h);
    const unsigned ncb = static_cast<unsigned>((h + kDenseCols - 1) / kDenseCols);
    if (dense_mfma_ok(dtype, T, h, E) && (grad_w_gate || grad_x)) {
        const DenseMfmaPlan pl = dense_mfma_plan(T, h, E);
        MOE_CHECK_ARG(workspace && workspace_bytes >= pl.total, MOE_ERR_WORKSPACE,
                      "moe_router_dense_bwd: workspace of %zu bytes needed", pl.total);
        char *ws = static_cast<char *>(workspace);
        bf16_t *D2 = reinterpret_cast<bf16_t *>(ws);
        int32_t *offs = reinterpret_cast<int32_t *>(ws + pl.off_offs);
        const int64_t nd = T * E;
        hipLaunchKernelGGL(split_hilo_kernel, dim3(static_cast<unsigned>((nd + 255) / 256)), dim3(256), 0, s,
                           grad_logits, nd, E, D2);
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(static_cast<unsigned>((pl.nchunk + 256) / 256)), dim3(256), 0,
                           s, offs, pl.nchunk, pl.chunk, TT);
        int st = check_launch("moe_router_dense_bwd split");
        if (st != MOE_OK) return st;
        if (grad_w_gate) {
            float *part = reinterpret_cast<float *>(ws + pl.off_part);
            st = bwd_wgrad_segments(static_cast<const bf16_t *>(x), hh, hh, D2, 2 * E, 2 * E, offs, pl.nchunk, T,
                                    part, s);
            if (st != MOE_OK) return st;
            const int64_t n = static_cast<int64_t>(E) * h;
            hipLaunchKernelGGL(hilo_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                               part, pl.nchunk, E, hh, grad_w_gate);
        }
        if (grad_x) {
            bf16_t *W2 = reinterpret_cast<bf16_t *>(ws + pl.off_w2);
            bf16_t *xo = reinterpret_cast<bf16_t *>(ws + pl.off_xo);
            const int64_t nw = static_cast<int64_t>(E) * h / 8;
            hipLaunchKernelGGL(stack_twice_kernel, dim3(static_cast<unsigned>((nw + 255) / 256)), dim3(256), 0, s,
                               static_cast<const bf16_t *>(w_gate), nw, W2);
            st = bwd_dgrad_plain(D2, 2 * E, W2, hh, hh, 2 * E, offs + pl.nchunk + 1, 1, T, xo, s);
            if (st != MOE_OK) return st;
            const int64_t np = T * h / 8;
            hipLaunchKernelGGL(add_rows_kernel, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0, s, xo,
                               np, static_cast<bf16_t *>(grad_x));
        }
        if (grad_b_gate)
            hipLaunchKernelGGL(dense_bgrad_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, s, grad_logits, TT, E,
                               grad_b_gate);
        return check_launch("moe_router_dense_bwd");
    }
    if (grad_w_gate) {
        const size_t need = moe_router_dense_bwd_workspace_size(T, h, E);
        MOE_CHECK_ARG(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                      "moe_router_dense_bwd: workspace of %zu bytes needed", need);
        const unsigned nchunk = static_cast<unsigned>((T + kDenseChunk - 1) / kDenseChunk);
        const dim3 g1(ncb, static_cast<unsigned>((E + kDenseExp - 1) / kDenseExp), nchunk);
        float *partial = static_cast<float *>(workspace);
        if (dtype == MOE_DTYPE_BF16)
            hipLaunchKernelGGL(dense_wgrad_partial_kernel<bf16_t>, g1, dim3(64), 0, s,
                               static_cast<const bf16_t *>(x), grad_logits, TT, hh, E, partial);
        else
            hipLaunchKernelGGL(dense_wgrad_partial_kernel<float>, g1, dim3(64), 0, s,
                               static_cast<const float *>(x), grad_logits, TT, hh, E, partial);
        const int64_t n = static_cast<int64_t>(E) * h;
        hipLaunchKernelGGL(dense_wgrad_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                           partial, static_cast<int>(nchunk), n, grad_w_gate);
    }
    if (grad_b_gate)
        hipLaunchKernelGGL(dense_bgrad_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, s, grad_logits, TT, E,
                           grad_b_gate);
    if (grad_x) {
        const dim3 g3(ncb, static_cast<unsigned>((T + 7) / 8));
        if (dtype == MOE_DTYPE_BF16)
            hipLaunchKernelGGL(dense_xgrad_kernel<bf16_t>, g3, dim3(64), 0, s, static_cast<const bf16_t *>(w_gate),
                               grad_logits, TT, hh, E, static_cast<bf16_t *>(grad_x));
        else
            hipLaunchKernelGGL(dense_xgrad_kernel<float>, g3, dim3(64), 0, s, static_cast<const float *>(w_gate),
                               grad_logits, TT, hh, E, static_cast<float *>(grad_x));
    }
    return check_launch("moe_router_dense_bwd");
}
