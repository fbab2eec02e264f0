// Routing variants of "emerging-techniques-moe-training":
//
// * Capacity-factor token dropping (Capacity Factor Tuning; the DeepSpeed
//   MoE config's drop_tokens): every expert takes at most `capacity` of its
//   (token, expert) pairs, the first ones in ascending token order; the
//   others are dropped (they reach no expert and add nothing to the output;
//   the kept pairs keep their routing weights). Built on the stable
//   permutation of moe_permute, whose segments already list each expert's
//   pairs in ascending token order, so dropping keeps a prefix of each
//   segment and compacts the kept rows.
// * Expert-choice routing (Routing Mechanisms, Expert Choice Routing): the
//   router's logits transposed to [experts, tokens], each expert takes its
//   `capacity` largest (ties: lower token index). A chosen pair is weighted
//   by the token's softmax gate probability over all experts. The chosen
//   tokens of expert e form segment e (rows e*C .. e*C+C-1, ascending token
//   order), which the grouped FFN consumes with gather_rows; a per-token
//   list of its rows (ascending expert) drives the combine.
//
// Every selection and compaction here is integer work with one defined
// result (no atomics whose order could matter).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kVarMaxE = 256;

// ------------------------------------------------------------- dropping

// offsets_kept[e] = sum over e' < e of min(count_e', C); one block.
__global__ __launch_bounds__(256) void cap_offsets_kernel(const int32_t *__restrict__ offsets, int E, int C,
                                                          int32_t *__restrict__ offsets_kept) {
    __shared__ int s[256];
    const int t = threadIdx.x;
    int v = 0;
    if (t < E) {
        const int m = offsets[t + 1] - offsets[t];
        v = m < C ? (m < 0 ? 0 : m) : C;
    }
    s[t] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int add = t >= d ? s[t - d] : 0;
        __syncthreads();
        s[t] += add;
        __syncthreads();
    }
    if (t < E) offsets_kept[t] = s[t] - v;
    if (t == 255) offsets_kept[E] = s[255];
}

// Per pair: rank of its row inside its expert's segment; kept when rank < C.
__global__ __launch_bounds__(256) void cap_rows_kernel(const int32_t *__restrict__ topk_idx,
                                                       const int32_t *__restrict__ offsets,
                                                       const int32_t *__restrict__ row_of,
                                                       const int32_t *__restrict__ offsets_kept, int64_t P, int k,
                                                       int E, int C, int32_t *__restrict__ row_of_kept,
                                                       int32_t *__restrict__ sorted_token_kept) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= P) return;
    const int e = topk_idx[i];
    const int r = row_of[i];
    int out = -1;
    if (e >= 0 && e < E && r >= offsets[e] && r < offsets[e + 1]) {
        const int rank = r - offsets[e];
        if (rank < C) {
            out = offsets_kept[e] + rank;
            sorted_token_kept[out] = static_cast<int32_t>(i / k);
        }
    }
    row_of_kept[i] = out;
}

// x_perm_kept[row_of_kept[t,j]] = x[t] for kept pairs: one 16-byte piece of
// a token row per thread, stored to each kept row.
template <typename TE>
__global__ __launch_bounds__(256) void cap_copy_kernel(const TE *__restrict__ x, int h, int k,
                                                       const int32_t *__restrict__ row_of_kept,
                                                       TE *__restrict__ xk, int64_t npieces, int64_t P) {
    constexpr int kVec = 16 / sizeof(TE);
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h / kVec;
    const int64_t t = idx / nv;
    const int v = static_cast<int>(idx - t * nv);
    const u32x4 q = *reinterpret_cast<const u32x4 *>(x + t * h + kVec * v);
    for (int j = 0; j < k; ++j) {
        const int r = row_of_kept[t * k + j];
        if (r >= 0 && r < P) *reinterpret_cast<u32x4 *>(xk + static_cast<int64_t>(r) * h + kVec * v) = q;
    }
}

// --------------------------------------------------------- expert choice

// Monotone map of a float to uint32 (larger float, larger key); -0 = +0.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (v == 0.0f) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// lT[e][t] = logits[t][e] through 32 x 32 LDS tiles; lse[t] on the side by
// a separate kernel.
__global__ __launch_bounds__(256) void transpose_kernel(const float *__restrict__ l, int T, int E,
                                                        float *__restrict__ lT) {
    __shared__ float tile[32][33];
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 8 rows per pass
    for (int r = ty; r < 32; r += 8) {
        const int t = t0 + r, e = e0 + tx;
        tile[r][tx] = (t < T && e < E) ? l[static_cast<int64_t>(t) * E + e] : 0.0f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int e = e0 + r, t = t0 + tx;
        if (e < E && t < T) lT[static_cast<int64_t>(e) * T + t] = tile[tx][r];
    }
}

// lse[t] = logsumexp of token t's logits: one wave per token, shuffle trees.
__global__ __launch_bounds__(256) void lse_kernel(const float *__restrict__ l, int T, int E,
                                                  float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *row = l + static_cast<int64_t>(t) * E;
    float mx = -INFINITY;
    for (int e = lane; e < E; e += 64) mx = fmaxf(mx, row[e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float s = 0.0f;
    for (int e = lane; e < E; e += 64) s += expf(row[e] - mx);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) lse[t] = mx + logf(s);
}

// Exclusive prefix of a 0/1 flag over the 1024 threads of a block, plus the
// block total. s_w: 16 ints of LDS.
__device__ __forceinline__ int block_flag_scan(bool f, int *s_w, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t b = __ballot(f);
    const int below = __popcll(b & ((uint64_t(1) << lane) - 1));
    if (lane == 0) s_w[wave] = __popcll(b);
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
        const int c = s_w[w];
        base += w < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return base + below;
}

// One block of 1024 threads per expert e: the C-th largest key of row e of
// lT by four 8-bit radix passes (LDS histograms), then the chosen tokens in
// ascending order: every key above it, and the lowest-indexed tokens of the
// keys equal to it until C are taken.
__global__ __launch_bounds__(1024) void ec_select_kernel(const float *__restrict__ lT, const float *__restrict__ lse,
                                                         int T, int C, int32_t *__restrict__ sorted_token,
                                                         float *__restrict__ row_w) {
    __shared__ int hist[256];
    __shared__ int s_w[16];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remain;
    const int e = blockIdx.x, tid = threadIdx.x;
    const float *row = lT + static_cast<int64_t>(e) * T;
    uint32_t prefix = 0, mask = 0;
    int remain = C;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += 1024) {
            const uint32_t key = order_key(row[t]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid == 0) {
            int above = 0, b = 255;
            for (; b > 0; --b) {
                if (above + hist[b] >= remain) break;
                above += hist[b];
            }
            s_prefix = prefix | (static_cast<uint32_t>(b) << shift);
            s_remain = remain - above;
        }
        __syncthreads();
        prefix = s_prefix;
        remain = s_remain;
        mask |= 0xffu << shift;
    }
    // prefix = the C-th largest key; remain = how many of the keys equal to
    // it are taken (>= 1)
    int carry_eq = 0, carry_pos = 0;
    int32_t *st = sorted_token + static_cast<int64_t>(e) * C;
    float *rw = row_w + static_cast<int64_t>(e) * C;
    for (int t0 = 0; t0 < T; t0 += 1024) {
        const int t = t0 + tid;
        const float v = t < T ? row[t] : 0.0f;
        const uint32_t key = t < T ? order_key(v) : 0u;
        const bool eq = t < T && key == prefix;
        int n_eq;
        const int r_eq = block_flag_scan(eq, s_w, n_eq);
        const bool take = t < T && (key > prefix || (eq && carry_eq + r_eq < remain));
        int n_take;
        const int pos = block_flag_scan(take, s_w, n_take);
        if (take) {
            st[carry_pos + pos] = t;
            rw[carry_pos + pos] = expf(v - lse[t]);
        }
        carry_eq += n_eq;
        carry_pos += n_take;
    }
}

// Rows of token t in ascending expert order: one wave per token, lane l
// searching segments l, l+64, ... (ascending tokens) for t.
__global__ __launch_bounds__(256) void ec_token_rows_kernel(const int32_t *__restrict__ sorted_token, int T, int E,
                                                            int C, int32_t *__restrict__ token_rows,
                                                            int32_t *__restrict__ token_nrows) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        int found = -1;
        if (e < E) {
            const int32_t *seg = sorted_token + static_cast<int64_t>(e) * C;
            int lo = 0, hi = C;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (seg[mid] < t) lo = mid + 1;
                else hi = mid;
            }
            if (lo < C && seg[lo] == t) found = e * C + lo;
        }
        const uint64_t b = __ballot(found >= 0);
        if (found >= 0)
            token_rows[static_cast<int64_t>(t) * E + base + __popcll(b & ((uint64_t(1) << lane) - 1))] = found;
        base += __popcll(b);
    }
    if (lane == 0) token_nrows[t] = base;
}

// out[t] = sum over token t's rows (ascending expert) of y[row] (+ y_sh[t]),
// fp32, one rounding: one 8-element piece per thread.
template <typename TE>
__global__ __launch_bounds__(256) void combine_rows_kernel(const TE *__restrict__ y, int h, int E,
                                                           const int32_t *__restrict__ token_rows,
                                                           const int32_t *__restrict__ token_nrows,
                                                           const TE *__restrict__ y_sh, TE *__restrict__ out,
                                                           int64_t npieces, int64_t P) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h >> 3;
    const int64_t t = idx / nv;
    const int v = static_cast<int>(idx - t * nv);
    int n = token_nrows[t];
    n = n < 0 ? 0 : (n > E ? E : n);
    const int32_t *rows = token_rows + t * E;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int i = 0; i < n; ++i) {
        const int r = rows[i];
        if (r < 0 || r >= P) continue;
        float yv[8];
        load8(y + static_cast<int64_t>(r) * h + 8 * v, yv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += yv[q];
    }
    if (y_sh) {
        float sv[8];
        load8(y_sh + t * h + 8 * v, sv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += sv[q];
    }
    store8(out + t * h + 8 * v, acc);
}

__global__ void ec_offsets_kernel(int32_t *offsets, int E, int C) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i <= E) offsets[i] = i * C;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_capacity_drop(const int32_t *topk_idx, const int32_t *offsets, const int32_t *row_of,
                                 const void *x, int dtype, int64_t T, int64_t h, int E, int k, int capacity,
                                 int32_t *offsets_kept, int32_t *row_of_kept, int32_t *sorted_token_kept,
                                 void *x_perm_kept, void *stream) {
    clear_error();
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && k > 0 && capacity >= 0, MOE_ERR_INVALID_ARG,
                  "moe_capacity_drop: bad sizes");
    MOE_CHECK_ARG(offsets && offsets_kept && (T == 0 || (topk_idx && row_of && row_of_kept && sorted_token_kept)),
                  MOE_ERR_INVALID_ARG, "moe_capacity_drop: null required pointer");
    MOE_CHECK_ARG(x_perm_kept == nullptr || x != nullptr, MOE_ERR_INVALID_ARG,
                  "moe_capacity_drop: x_perm_kept requested without x");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_capacity_drop: bad dtype %d", dtype);
    MOE_CHECK_ARG(k <= E && E <= kVarMaxE && h % 64 == 0 && T * k < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_capacity_drop: need k <= E <= 256, h %% 64 == 0, T*k < 2^31");
    MOE_CHECK_ARG(x_perm_kept == nullptr || (aligned16(x) && aligned16(x_perm_kept)), MOE_ERR_INVALID_ARG,
                  "moe_capacity_drop: pointers must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(cap_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, E, capacity, offsets_kept);
    if (T == 0) return check_launch("moe_capacity_drop");
    const int64_t P = T * k;
    hipLaunchKernelGGL(cap_rows_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0, s, topk_idx,
                       offsets, row_of, offsets_kept, P, k, E, capacity, row_of_kept, sorted_token_kept);
    if (x_perm_kept) {
        if (dtype == MOE_DTYPE_BF16) {
            const int64_t np = T * (h / 8);
            hipLaunchKernelGGL(cap_copy_kernel<bf16_t>, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0,
                               s, static_cast<const bf16_t *>(x), static_cast<int>(h), k, row_of_kept,
                               static_cast<bf16_t *>(x_perm_kept), np, P);
        } else {
            const int64_t np = T * (h / 4);
            hipLaunchKernelGGL(cap_copy_kernel<float>, dim3(static_cast<unsigned>((np + 255) / 256)), dim3(256), 0,
                               s, static_cast<const float *>(x), static_cast<int>(h), k, row_of_kept,
                               static_cast<float *>(x_perm_kept), np, P);
        }
    }
    return check_launch("moe_capacity_drop");
}

extern "C" size_t moe_expert_choice_workspace_size(int64_t T, int E) {
    if (T <= 0 || E <= 0) return 0;
    return (static_cast<size_t>(T) * static_cast<size_t>(E) + static_cast<size_t>(T) + 64) * sizeof(float);
}

extern "C" int moe_expert_choice(const float *logits, int64_t T, int E, int capacity, int32_t *offsets,
                                 int32_t *sorted_token, float *row_w, int32_t *token_rows, int32_t *token_nrows,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(T > 0 && E > 0 && capacity > 0, MOE_ERR_INVALID_ARG, "moe_expert_choice: bad sizes");
    MOE_CHECK_ARG(logits && offsets && sorted_token && row_w && token_rows && token_nrows, MOE_ERR_INVALID_ARG,
                  "moe_expert_choice: null required pointer");
    MOE_CHECK_ARG(capacity <= T && E <= kVarMaxE && T * E < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_expert_choice: need capacity <= T, E <= 256, T*E < 2^31");
    const size_t need = moe_expert_choice_workspace_size(T, E);
    MOE_CHECK_ARG(workspace && workspace_bytes >= need && aligned16(workspace), MOE_ERR_WORKSPACE,
                  "moe_expert_choice: a 16-byte aligned workspace of %zu bytes is needed", need);
    hipStream_t s = as_stream(stream);
    const int TT = static_cast<int>(T);
    float *lT = static_cast<float *>(workspace);
    float *lse = lT + T * E;
    hipLaunchKernelGGL(transpose_kernel, dim3(static_cast<unsigned>((T + 31) / 32), static_cast<unsigned>((E + 31) / 32)),
                       dim3(256), 0, s, logits, TT, E, lT);
    hipLaunchKernelGGL(lse_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s, logits, TT, E, lse);
    hipLaunchKernelGGL(ec_offsets_kernel, dim3(static_cast<unsigned>((E + 256) / 256)), dim3(256), 0, s, offsets, E,
                       capacity);
    hipLaunchKernelGGL(ec_select_kernel, dim3(static_cast<unsigned>(E)), dim3(1024), 0, s, lT, lse, TT, capacity,
                       sorted_token, row_w);
    hipLaunchKernelGGL(ec_token_rows_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s, sorted_token,
                       TT, E, capacity, token_rows, token_nrows);
    return check_launch("moe_expert_choice");
}

extern "C" int moe_combine_rows(const void *y, int dtype, int64_t T, int64_t h, int E, int64_t P,
                                const int32_t *token_rows, const int32_t *token_nrows, const void *y_sh, void *out,
                                void *stream) {
    clear_error();
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && P >= 0, MOE_ERR_INVALID_ARG, "moe_combine_rows: bad sizes");
    MOE_CHECK_ARG(T == 0 || (y && token_rows && token_nrows && out), MOE_ERR_INVALID_ARG,
                  "moe_combine_rows: null required pointer");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_combine_rows: bad dtype %d", dtype);
    MOE_CHECK_ARG(h % 64 == 0 && E <= kVarMaxE && P < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_combine_rows: need h %% 64 == 0, E <= 256");
    MOE_CHECK_ARG(T == 0 || (aligned16(y) && aligned16(out) && (!y_sh || aligned16(y_sh))), MOE_ERR_INVALID_ARG,
                  "moe_combine_rows: pointers must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    const int64_t np = T * (h / 8);
    const dim3 grid(static_cast<unsigned>((np + 255) / 256)), block(256);
    if (dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL(combine_rows_kernel<bf16_t>, grid, block, 0, s, static_cast<const bf16_t *>(y),
                           static_cast<int>(h), E, token_rows, token_nrows, static_cast<const bf16_t *>(y_sh),
                           static_cast<bf16_t *>(out), np, P);
    else
        hipLaunchKernelGGL(combine_rows_kernel<float>, grid, block, 0, s, static_cast<const float *>(y),
                           static_cast<int>(h), E, token_rows, token_nrows, static_cast<const float *>(y_sh),
                           static_cast<float *>(out), np, P);
    return check_launch("moe_combine_rows");
}
