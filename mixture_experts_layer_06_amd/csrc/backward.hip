// Router backward.
//
// Routing weights are the softmax of the selected logits (renormalised top-k,
// "emerging-techniques-moe-training", Quick Start and Mixtral block) or the
// selected sigmoid scores over their sum (DeepSeek-V3 style, "Scalable
// Training of Mixture-of-Experts Models with Megatron Core", section 2.2).
// With g = dL/dw:
//   softmax:  dL/dl_j = w_j (g_j - sum_i w_i g_i)
//   sigmoid:  dL/dl_j = s_j (1 - s_j) / S (g_j - sum_i w_i g_i)
// and unselected logits get no gradient. With one expert or top-1 the weight
// is the constant 1 and the router gradient is exactly zero, as the handbook
// page reports ("Mixture-of-Experts from Architecture to Large-Scale
// Training", section 2.5).
//
// Weight gradient: grad_w_gate[e] = sum over the rows r of expert e's
// permuted segment (ascending) of dl(r) x[sorted_token[r]]. To spread a hot
// expert over many workgroups without floating-point atomics, each segment is
// cut into chunks of kRC rows; pass 1 writes one partial sum per chunk, pass 2
// adds an expert's chunks in chunk order. Both orders are fixed, so the
// result is deterministic. The logit gradient of each permuted row is looked
// up once beforehand (one thread per row), so that pass 1 only streams rows
// of x, four rows per thread in flight.
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kRC = 256;      // rows per chunk
constexpr int kCB = 512;      // columns per pass-1 block (64 threads x 8)

__global__ __launch_bounds__(256) void route_bwd_dl_kernel(int T, int k, int E, int sigmoid,
                                                           const float *__restrict__ logits,
                                                           const int32_t *__restrict__ topk_idx,
                                                           const float *__restrict__ w,
                                                           const float *__restrict__ gw,
                                                           float *__restrict__ dl) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const int64_t base = static_cast<int64_t>(t) * k;
    float c = 0.0f;
    for (int j = 0; j < k; ++j) c = fmaf(w[base + j], gw[base + j], c);
    if (!sigmoid) {
        for (int j = 0; j < k; ++j) dl[base + j] = w[base + j] * (gw[base + j] - c);
    } else {
        // the selected sigmoids: their sum, then each again (the same value)
        auto sig_of = [&](int j) {
            int e = topk_idx[base + j];
            e = (e >= 0 && e < E) ? e : 0;
            return 1.0f / (1.0f + expf(-logits[static_cast<int64_t>(t) * E + e]));
        };
        float S = 0.0f;
        for (int j = 0; j < k; ++j) S += sig_of(j);
        for (int j = 0; j < k; ++j) {
            const float sj = sig_of(j);
            dl[base + j] = sj * (1.0f - sj) / S * (gw[base + j] - c);
        }
    }
}

// dl_row[r] = dl of permuted row r: the token t = sorted_token[r] of expert
// e's segment (the largest e with offsets[e] <= r) at the slot j where
// topk_idx[t][j] == e.
__global__ __launch_bounds__(256) void route_bwd_rowdl_kernel(int P, int E, int k, const int32_t *__restrict__ offsets,
                                                              const int32_t *__restrict__ sorted_token,
                                                              const int32_t *__restrict__ topk_idx,
                                                              const float *__restrict__ dl, float *__restrict__ dl_row) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= P) return;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int64_t t = sorted_token[r];
    float d = 0.0f;
    for (int j = 0; j < k; ++j)
        if (topk_idx[t * k + j] == lo) d = dl[t * k + j];
    dl_row[r] = d;
}

// Chunk prefix over experts in LDS: s_ck[e] = chunks of experts < e.
__device__ int build_chunk_prefix(const int32_t *offsets, int E, int *s_ck, int *s_tmp) {
    const int t = threadIdx.x;
    const int m = t < E ? offsets[t + 1] - offsets[t] : 0;
    const int v = m > 0 ? (m + kRC - 1) / kRC : 0;
    s_tmp[t] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int add = t >= d ? s_tmp[t - d] : 0;
        __syncthreads();
        s_tmp[t] += add;
        __syncthreads();
    }
    s_ck[t] = s_tmp[t] - v;
    __syncthreads();
    return s_tmp[255];
}

template <typename TE>
__global__ __launch_bounds__(256) void route_bwd_partial_kernel(
    const TE *__restrict__ x, int h, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_token, const float *__restrict__ dl_row, float *__restrict__ partial,
    float *__restrict__ partial_b) {
    __shared__ int s_ck[256];
    __shared__ int s_tmp[256];
    __shared__ float s_acc[4][kCB];
    __shared__ float s_b[4];
    const int nchunks = build_chunk_prefix(offsets, E, s_ck, s_tmp);
    const int q = blockIdx.x;
    if (q >= nchunks) return;
    int lo = 0, hi = E - 1;   // expert e: largest with s_ck[e] <= q and a chunk
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_ck[mid] <= q) lo = mid;
        else hi = mid - 1;
    }
    const int e = lo;
    const int r0 = offsets[e] + (q - s_ck[e]) * kRC;
    int r1 = r0 + kRC;
    if (r1 > offsets[e + 1]) r1 = offsets[e + 1];
    const int grp = threadIdx.x >> 6;          // rows r0 + grp, r0 + grp + 4, ...
    const int col = blockIdx.y * kCB + (threadIdx.x & 63) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float bsum = 0.0f;
    // rows r0 + grp + 4 i, ascending; four of them loaded before use
    const int cc = col < h ? col : 0;   // out-of-range columns load column 0, never stored
    for (int rb = r0 + grp; rb < r1; rb += 16) {
        float d[4], xv[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = rb + 4 * u;
            d[u] = 0.0f;
            if (r < r1) {
                d[u] = dl_row[r];
                load8(x + static_cast<int64_t>(sorted_token[r]) * h + cc, xv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (rb + 4 * u < r1) {
                bsum += d[u];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(d[u], xv[u][i], acc[i]);
            }
        }
    }
    const int c0 = (threadIdx.x & 63) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) s_acc[grp][c0 + i] = acc[i];
    if ((threadIdx.x & 63) == 0) s_b[grp] = bsum;
    __syncthreads();
    if (threadIdx.x < 64 && col < h) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = ((s_acc[0][c0 + i] + s_acc[1][c0 + i]) + s_acc[2][c0 + i]) + s_acc[3][c0 + i];
        store8(partial + static_cast<int64_t>(q) * h + col, o);
    }
    if (threadIdx.x == 0 && blockIdx.y == 0) partial_b[q] = ((s_b[0] + s_b[1]) + s_b[2]) + s_b[3];
}

__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(
    int h, int E, const int32_t *__restrict__ offsets, const float *__restrict__ partial,
    const float *__restrict__ partial_b, float *__restrict__ gwg, float *__restrict__ gbg) {
    __shared__ int s_ck[256];
    __shared__ int s_tmp[256];
    build_chunk_prefix(offsets, E, s_ck, s_tmp);
    const int e = blockIdx.x;
    const int m = offsets[e + 1] - offsets[e];
    const int nq = m > 0 ? (m + kRC - 1) / kRC : 0;
    const int q0 = s_ck[e];
    for (int c = blockIdx.y * 256 * 8 + threadIdx.x * 8; c < h; c += gridDim.y * 256 * 8) {
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int q = q0; q < q0 + nq; ++q) {
            float p[8];
            load8(partial + static_cast<int64_t>(q) * h + c, p);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] += p[i];
        }
        store8(gwg + static_cast<int64_t>(e) * h + c, o);
    }
    if (gbg && blockIdx.y == 0 && threadIdx.x == 0) {
        float b = 0.0f;
        for (int q = q0; q < q0 + nq; ++q) b += partial_b[q];
        gbg[e] = b;
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_bwd_workspace_size(int64_t T, int64_t h, int E, int k) {
    if (T < 0 || h <= 0 || E <= 0 || k <= 0) return 0;
    const int64_t nq = (T * k) / kRC + E + 1;
    return static_cast<size_t>(nq * h + nq + T * k) * sizeof(float) + 256;
}

extern "C" int moe_route_bwd(const void *x, int dtype, int64_t T, int64_t h, int E, int k,
                             int score, const float *logits, const int32_t *topk_idx,
                             const float *topk_w, const float *grad_topk_w,
                             const int32_t *offsets, const int32_t *sorted_token,
                             float *grad_logits_sel, float *grad_w_gate, float *grad_b_gate,
                             void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(offsets && grad_w_gate &&
                      (T == 0 || (x && topk_idx && topk_w && grad_topk_w && sorted_token && grad_logits_sel)),
                  MOE_ERR_INVALID_ARG, "moe_route_bwd: null required pointer");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_route_bwd: bad dtype %d", dtype);
    MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID, MOE_ERR_INVALID_ARG,
                  "moe_route_bwd: bad score %d", score);
    MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || logits, MOE_ERR_INVALID_ARG,
                  "moe_route_bwd: sigmoid scoring needs the logits");
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG, "moe_route_bwd: bad sizes");
    MOE_CHECK_ARG(k <= E && E <= 256 && h % 64 == 0, MOE_ERR_UNSUPPORTED,
                  "moe_route_bwd: need k <= E <= 256, h %% 64 == 0");
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31) && h < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_route_bwd: T*k must be < 2^31");
    const size_t need = moe_route_bwd_workspace_size(T, h, E, k);
    MOE_CHECK_ARG(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                  "moe_route_bwd: workspace of %zu bytes needed", need);
    MOE_CHECK_ARG(aligned16(x) && aligned16(grad_w_gate) && aligned16(workspace), MOE_ERR_INVALID_ARG,
                  "moe_route_bwd: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    const int64_t nq = (T * k) / kRC + E + 1;
    float *partial = static_cast<float *>(workspace);
    float *partial_b = partial + nq * h;
    float *dl_row = partial_b + nq;
    const int P = static_cast<int>(T * k);
    if (T > 0)
        hipLaunchKernelGGL(route_bwd_dl_kernel, dim3(static_cast<unsigned>((T + 255) / 256)), dim3(256), 0,
                           s, static_cast<int>(T), k, E, score == MOE_SCORE_SIGMOID, logits, topk_idx,
                           topk_w, grad_topk_w, grad_logits_sel);
    if (P > 0)
        hipLaunchKernelGGL(route_bwd_rowdl_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0, s, P,
                           E, k, offsets, sorted_token, topk_idx, grad_logits_sel, dl_row);
    const dim3 g1(static_cast<unsigned>(nq), static_cast<unsigned>((h + kCB - 1) / kCB));
    if (dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL(route_bwd_partial_kernel<bf16_t>, g1, dim3(256), 0, s,
                           static_cast<const bf16_t *>(x), static_cast<int>(h), E, offsets, sorted_token, dl_row,
                           partial, partial_b);
    else
        hipLaunchKernelGGL(route_bwd_partial_kernel<float>, g1, dim3(256), 0, s,
                           static_cast<const float *>(x), static_cast<int>(h), E, offsets, sorted_token, dl_row,
                           partial, partial_b);
    unsigned gy = static_cast<unsigned>((h + 2047) / 2048);
    hipLaunchKernelGGL(route_bwd_reduce_kernel, dim3(E, gy), dim3(256), 0, s, static_cast<int>(h), E,
                       offsets, partial, partial_b, grad_w_gate, grad_b_gate);
    return check_launch("moe_route_bwd");
}

