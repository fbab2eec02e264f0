// Dispatch stage: regroup the (token, expert) pairs into expert-contiguous
// order and copy token rows there ("Scalable Training of Mixture-of-Experts
// Models with Megatron Core", section 2.1 stage 2; every expert is local, so
// there is no all-to-all).
//
// Row of pair (t, e) = offsets[e] + #{t' < t : t' selected e}, i.e. stable
// ascending token order inside each expert segment. Four launches, all
// integer work except the copy:
//   1. block_hist: per block of 256 tokens, tokens per expert (LDS integer
//      atomics; order cannot change an integer count).
//   2. scan: one workgroup; offsets = exclusive prefix over experts, and the
//      base row of each (block, expert).
//   3. ranks: per block, a 256-bit mask per expert in LDS; the rank of token
//      t among the block's tokens of expert e is a popcount of the mask bits
//      below t. Writes row_of and sorted_token.
//   4. copy: each token row is read once from HBM and written to its k
//      permuted rows with 16-byte accesses.
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kBlockTok = 256;
constexpr int kMaxE = 256;

__global__ __launch_bounds__(256) void block_hist_kernel(const int32_t *__restrict__ topk_idx,
                                                         int T, int E, int k,
                                                         int32_t *__restrict__ blockcounts) {
    __shared__ int cnt[kMaxE];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * kBlockTok + threadIdx.x;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[static_cast<int64_t>(t) * k + j];
            if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        blockcounts[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// One workgroup of 256 threads; thread e owns expert e.
__global__ __launch_bounds__(256) void scan_kernel(const int32_t *__restrict__ blockcounts,
                                                   int nb, int E, int32_t *__restrict__ blockbase,
                                                   int32_t *__restrict__ offsets) {
    __shared__ int tot[kMaxE];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E)
        for (int b = 0; b < nb; ++b) run += blockcounts[static_cast<int64_t>(b) * E + e];
    tot[e] = e < E ? run : 0;
    __syncthreads();
    // inclusive Hillis-Steele scan over 256 entries
    for (int d = 1; d < kMaxE; d <<= 1) {
        const int v = e >= d ? tot[e - d] : 0;
        __syncthreads();
        tot[e] += v;
        __syncthreads();
    }
    if (e < E) {
        const int start = tot[e] - run;   // exclusive prefix
        offsets[e] = start;
        if (e == E - 1) offsets[E] = tot[e];
        int base = start;
        for (int b = 0; b < nb; ++b) {
            blockbase[static_cast<int64_t>(b) * E + e] = base;
            base += blockcounts[static_cast<int64_t>(b) * E + e];
        }
    }
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t *__restrict__ topk_idx, int T,
                                                   int E, int k,
                                                   const int32_t *__restrict__ blockbase,
                                                   int P, int32_t *__restrict__ row_of,
                                                   int32_t *__restrict__ sorted_token) {
    __shared__ unsigned long long mask[kMaxE][kBlockTok / 64];
    for (int i = threadIdx.x; i < E * (kBlockTok / 64); i += blockDim.x)
        (&mask[0][0])[i] = 0ull;
    __syncthreads();
    const int lt = threadIdx.x;
    const int t = blockIdx.x * kBlockTok + lt;
    const int word = lt >> 6;
    const unsigned long long bit = 1ull << (lt & 63);
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[static_cast<int64_t>(t) * k + j];
            if (e >= 0 && e < E) atomicOr(&mask[e][word], bit);
        }
    }
    __syncthreads();
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[static_cast<int64_t>(t) * k + j];
            int row = -1;
            if (e >= 0 && e < E) {
                int rank = __popcll(mask[e][word] & (bit - 1ull));
                for (int w = 0; w < word; ++w) rank += __popcll(mask[e][w]);
                row = blockbase[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
                if (row < 0 || row >= P) row = -1;
            }
            row_of[static_cast<int64_t>(t) * k + j] = row;
            if (row >= 0) sorted_token[row] = t;
        }
    }
}

// Block of 256 threads per token row; each thread moves 16-byte pieces.
// One thread per 16-byte piece of a token row (a flat grid over T x pieces):
// the piece is read once and stored to the token's k rows of x_perm (rows
// outside [0, T k) are skipped).
template <typename TE, int KM, bool WT>
__global__ __launch_bounds__(256) void copy_rows_kernel(const TE *__restrict__ x, int h, int k,
                                                        const int32_t *__restrict__ row_of,
                                                        TE *__restrict__ x_perm, int64_t npieces) {
    constexpr int kVec = 16 / sizeof(TE);
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h / kVec;
    int t = static_cast<int>(idx / nv);
    const int v = static_cast<int>(idx - static_cast<int64_t>(t) * nv);
    if constexpr (WT) t = __builtin_amdgcn_readfirstlane(t);   // one token per wave: scalar index loads
    // the piece and the row indices of the KM top-k slots in flight together
    // (KM = k rounded up to 1, 2, 4 or 8; slots past k re-read slot k - 1
    // and store nothing; for k > 8 further chunks of 8 follow)
    int rows[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) rows[j] = row_of[static_cast<int64_t>(t) * k + (j < k ? j : k - 1)];
    const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(t) * h) + v);
    // the piece is waited for here, once: a wait inside the conditional
    // stores below would, with the in-order memory counter, also wait for
    // the stores issued before it
    __asm__ volatile("" ::"v"(d));
    for (int j0 = 0; j0 < k; j0 += KM) {
        const int kc = min(KM, k - j0);
        if (j0 > 0) {
#pragma unroll
            for (int j = 0; j < KM; ++j) rows[j] = row_of[static_cast<int64_t>(t) * k + j0 + (j < kc ? j : kc - 1)];
        }
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc && rows[j] >= 0 && static_cast<int64_t>(rows[j]) < npieces / nv * k)
                __builtin_nontemporal_store(d, reinterpret_cast<u32x4 *>(x_perm + static_cast<int64_t>(rows[j]) * h) + v);
    }
}

// Routing weights in permuted-row order and back:
//   row_w[row_of[t,j]] = topk_w[t,j];   grad_topk_w[t,j] = grad_row_w[row_of[t,j]]
// (one (t, j) pair per thread; rows outside [0, T k) are skipped, or read as 0).
__global__ __launch_bounds__(256) void permute_weights_kernel(const float *__restrict__ topk_w,
                                                              const int32_t *__restrict__ row_of, int64_t P,
                                                              float *__restrict__ row_w) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= P) return;
    const int r = row_of[i];
    if (r >= 0 && r < P) row_w[r] = topk_w[i];
}

__global__ __launch_bounds__(256) void permute_weights_bwd_kernel(const float *__restrict__ grad_row_w,
                                                                  const int32_t *__restrict__ row_of, int64_t P,
                                                                  float *__restrict__ grad_topk_w) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= P) return;
    const int r = row_of[i];
    grad_topk_w[i] = (r >= 0 && r < P) ? grad_row_w[r] : 0.0f;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {

// Checks shared by moe_permute and moe_permute_noalloc (everything but the
// workspace).
int permute_check(const void *x, int dtype, int64_t T, int64_t h, int E, int k, const int32_t *topk_idx,
                  const int32_t *offsets, const int32_t *sorted_token, const int32_t *row_of, const void *x_perm,
                  const char *name) {
    MOE_CHECK_ARG(offsets && (T == 0 || (topk_idx && sorted_token && row_of)), MOE_ERR_INVALID_ARG,
                  "%s: null required pointer", name);
    MOE_CHECK_ARG(x_perm == nullptr || x != nullptr, MOE_ERR_INVALID_ARG, "%s: x_perm requested without x", name);
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG, "%s: bad dtype %d", name,
                  dtype);
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG, "%s: bad sizes", name);
    MOE_CHECK_ARG(k <= E && E <= kMaxE && h % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: need k <= E <= 256, h %% 64 == 0",
                  name);
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31) && h < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "%s: T*k must be < 2^31", name);
    MOE_CHECK_ARG(x_perm == nullptr || (aligned16(x) && aligned16(x_perm)), MOE_ERR_INVALID_ARG,
                  "%s: pointers must be 16-byte aligned", name);
    return MOE_OK;
}

// The four launches of the dispatch; ws: 2 nb E ints (block counts, then
// block bases), every entry written by block_hist and scan before it is read.
int permute_launch(const void *x, int dtype, int64_t T, int64_t h, int E, int k, const int32_t *topk_idx,
                   int32_t *offsets, int32_t *sorted_token, int32_t *row_of, void *x_perm, int32_t *ws,
                   hipStream_t s, const char *name) {
    const int nb = static_cast<int>((T + kBlockTok - 1) / kBlockTok);
    int32_t *blockcounts = ws;
    int32_t *blockbase = blockcounts + static_cast<int64_t>(nb) * E;
    const int P = static_cast<int>(T * k);
    if (nb > 0)
        hipLaunchKernelGGL(block_hist_kernel, dim3(nb), dim3(256), 0, s, topk_idx,
                           static_cast<int>(T), E, k, blockcounts);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, blockcounts, nb, E, blockbase, offsets);
    if (nb > 0)
        hipLaunchKernelGGL(rank_kernel, dim3(nb), dim3(256), 0, s, topk_idx, static_cast<int>(T), E,
                           k, blockbase, P, row_of, sorted_token);
    if (x_perm && T > 0) {
        const int64_t nv = dtype == MOE_DTYPE_BF16 ? h / 8 : h / 4;   // 16-byte pieces per row
        auto go = [&](auto km) {
            constexpr int KM = decltype(km)::value;
            const dim3 grid(static_cast<unsigned>((T * nv + 255) / 256));
            const bool wt = nv % 64 == 0;   // each wave's pieces in one token
            if (dtype == MOE_DTYPE_BF16) {
                auto kfn = wt ? copy_rows_kernel<bf16_t, KM, true> : copy_rows_kernel<bf16_t, KM, false>;
                hipLaunchKernelGGL(kfn, grid, dim3(256), 0, s, static_cast<const bf16_t *>(x), static_cast<int>(h), k,
                                   row_of, static_cast<bf16_t *>(x_perm), T * nv);
            } else {
                auto kfn = wt ? copy_rows_kernel<float, KM, true> : copy_rows_kernel<float, KM, false>;
                hipLaunchKernelGGL(kfn, grid, dim3(256), 0, s, static_cast<const float *>(x), static_cast<int>(h), k,
                                   row_of, static_cast<float *>(x_perm), T * nv);
            }
        };
        if (k <= 1) go(std::integral_constant<int, 1>{});
        else if (k <= 2) go(std::integral_constant<int, 2>{});
        else if (k <= 4) go(std::integral_constant<int, 4>{});
        else go(std::integral_constant<int, 8>{});
    }
    return check_launch(name);
}

// Scratch of moe_permute_noalloc: one copy per GPU, in the library's device
// image, held until the process ends. Its name is a host-side stand-in: host
// code uses only the device address that hipGetSymbolAddress returns for the
// current device, cached per device below.
constexpr int64_t kNoAllocScratchInts = 262144;   // 1 MiB: 2 nb E <= 262144
static __device__ __align__(256) int32_t scratch[kNoAllocScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per
// device, with that device current); null with the error set on failure.
int32_t *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        set_error("moe_permute_noalloc: no current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            set_error(std::string("moe_permute_noalloc: hipGetSymbolAddress failed: ") + hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t moe_permute_workspace_size(int64_t T, int E, int k) {
    (void)k;
    if (T < 0 || E <= 0) return 0;
    const int64_t nb = (T + kBlockTok - 1) / kBlockTok;
    return static_cast<size_t>(2 * nb * E) * sizeof(int32_t) + 256;
}

extern "C" int moe_permute(const void *x, int dtype, int64_t T, int64_t h, int E, int k,
                           const int32_t *topk_idx, int32_t *offsets, int32_t *sorted_token,
                           int32_t *row_of, void *x_perm, void *workspace, size_t workspace_bytes,
                           void *stream) {
    clear_error();
    const int st = permute_check(x, dtype, T, h, E, k, topk_idx, offsets, sorted_token, row_of, x_perm,
                                 "moe_permute");
    if (st != MOE_OK) return st;
    const size_t need = moe_permute_workspace_size(T, E, k);
    MOE_CHECK_ARG(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                  "moe_permute: workspace of %zu bytes needed", need);
    MOE_CHECK_ARG(aligned16(workspace), MOE_ERR_INVALID_ARG, "moe_permute: pointers must be 16-byte aligned");
    return permute_launch(x, dtype, T, h, E, k, topk_idx, offsets, sorted_token, row_of, x_perm,
                          static_cast<int32_t *>(workspace), as_stream(stream), "moe_permute");
}

extern "C" int moe_permute_noalloc(const void *x, int dtype, int64_t T, int64_t h, int E, int k,
                                   const int32_t *topk_idx, int32_t *offsets, int32_t *sorted_token,
                                   int32_t *row_of, void *x_perm, void *stream) {
    clear_error();
    const int st = permute_check(x, dtype, T, h, E, k, topk_idx, offsets, sorted_token, row_of, x_perm,
                                 "moe_permute_noalloc");
    if (st != MOE_OK) return st;
    const int64_t nb = (T + kBlockTok - 1) / kBlockTok;
    MOE_CHECK_ARG(2 * nb * E <= kNoAllocScratchInts, MOE_ERR_UNSUPPORTED,
                  "moe_permute_noalloc: ceil(T/256) * E = %lld exceeds the static scratch's %lld",
                  static_cast<long long>(nb * E), static_cast<long long>(kNoAllocScratchInts / 2));
    int32_t *ws = scratch_on_current_device();
    if (ws == nullptr) return MOE_ERR_HIP;
    return permute_launch(x, dtype, T, h, E, k, topk_idx, offsets, sorted_token, row_of, x_perm, ws,
                          as_stream(stream), "moe_permute_noalloc");
}

extern "C" int moe_permute_weights(const float *topk_w, int64_t T, int k, const int32_t *row_of, float *row_w,
                                   void *stream) {
    clear_error();
    MOE_CHECK_ARG(T >= 0 && k > 0, MOE_ERR_INVALID_ARG, "moe_permute_weights: bad sizes");
    MOE_CHECK_ARG(T == 0 || (topk_w && row_of && row_w), MOE_ERR_INVALID_ARG,
                  "moe_permute_weights: null required pointer");
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED, "moe_permute_weights: T*k must be < 2^31");
    if (T == 0) return MOE_OK;
    const int64_t P = T * k;
    hipLaunchKernelGGL(permute_weights_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0,
                       as_stream(stream), topk_w, row_of, P, row_w);
    return check_launch("moe_permute_weights");
}

extern "C" int moe_permute_weights_bwd(const float *grad_row_w, int64_t T, int k, const int32_t *row_of,
                                       float *grad_topk_w, void *stream) {
    clear_error();
    MOE_CHECK_ARG(T >= 0 && k > 0, MOE_ERR_INVALID_ARG, "moe_permute_weights_bwd: bad sizes");
    MOE_CHECK_ARG(T == 0 || (grad_row_w && row_of && grad_topk_w), MOE_ERR_INVALID_ARG,
                  "moe_permute_weights_bwd: null required pointer");
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED, "moe_permute_weights_bwd: T*k must be < 2^31");
    if (T == 0) return MOE_OK;
    const int64_t P = T * k;
    hipLaunchKernelGGL(permute_weights_bwd_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0,
                       as_stream(stream), grad_row_w, row_of, P, grad_topk_w);
    return check_launch("moe_permute_weights_bwd");
}
