// Combine stage and the two row-wise backward passes around the experts.
//
//   unpermute:      out[t] = sum_j w[t,j] y[row_of[t,j]] (+ y_sh[t])
//   unpermute_bwd:  grad_y[row_of[t,j]] = w[t,j] grad_out[t];
//                   grad_w[t,j] = <grad_out[t], y[row_of[t,j]]>
//   permute_bwd:    grad_x[t] = sum_j grad_x_perm[row_of[t,j]]
//                             + sum_j grad_l[t,j] w_gate[topk_idx[t,j]]
//
// Combine: "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2.1 stage 4 (inverse of the dispatch, restoring token order)
// and section 1.1 (MoE(x) = sum over the top-k of p_i E_i(x)). The shared
// expert's output is added with weight 1.
//
// All three are HBM-bound row streams (one thread per 8-element piece;
// unpermute_bwd: one workgroup per token for its dot products), 16-byte
// accesses, fp32 accumulation in a fixed order (j ascending), one rounding to
// the output type. Reductions use a fixed shuffle tree, so results are
// deterministic.
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

// Streaming loads and stores of 8 elements (rows read or written once):
// non-temporal, so they do not displace reusable lines from the caches.
__device__ __forceinline__ void load8_nt(const bf16_t *p, float *v) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        v[2 * c] = bf16lo(q[c]);
        v[2 * c + 1] = bf16hi(q[c]);
    }
}
__device__ __forceinline__ void load8_nt(const float *p, float *v) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        v[c] = __uint_as_float(a[c]);
        v[4 + c] = __uint_as_float(b[c]);
    }
}
// Raw 8-element pieces: the load only (converted to fp32 where used), so a
// load under a condition does not make the wave wait for it right there.
template <typename TE> struct Raw8 {
    u32x4 q[sizeof(TE) / 2];   // bf16: one 16-byte piece, fp32: two
};
template <typename TE> __device__ __forceinline__ void raw8_load_nt(const TE *p, Raw8<TE> &r) {
#pragma unroll
    for (int c = 0; c < static_cast<int>(sizeof(TE) / 2); ++c)
        r.q[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + c);
}
template <typename TE> __device__ __forceinline__ void raw8_load(const TE *p, Raw8<TE> &r) {
#pragma unroll
    for (int c = 0; c < static_cast<int>(sizeof(TE) / 2); ++c) r.q[c] = reinterpret_cast<const u32x4 *>(p)[c];
}
__device__ __forceinline__ void raw8_f32(const Raw8<bf16_t> &r, float *v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        v[2 * c] = bf16lo(r.q[0][c]);
        v[2 * c + 1] = bf16hi(r.q[0][c]);
    }
}
__device__ __forceinline__ void raw8_f32(const Raw8<float> &r, float *v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        v[c] = __uint_as_float(r.q[0][c]);
        v[4 + c] = __uint_as_float(r.q[1][c]);
    }
}

__device__ __forceinline__ void store8_nt(bf16_t *p, const float *v) {
    u32x4 q;
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = pack_bf16x2(v[2 * c], v[2 * c + 1]);
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store8_nt(float *p, const float *v) {
    __builtin_nontemporal_store(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                      __float_as_uint(v[3])},
                                reinterpret_cast<u32x4 *>(p));
    __builtin_nontemporal_store(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                      __float_as_uint(v[7])},
                                reinterpret_cast<u32x4 *>(p + 4));
}

// One thread per 8-element piece of an output row (a flat grid over
// T x h/8 pieces): the k source pieces are all loaded before the fixed-order
// weighted sum, so each thread keeps k loads in flight.
template <typename TE, int KM, bool WT>
__global__ __launch_bounds__(256) void unpermute_kernel(const TE *__restrict__ y, int h, int k,
                                                        const int32_t *__restrict__ row_of,
                                                        const float *__restrict__ topk_w,
                                                        const TE *__restrict__ y_sh,
                                                        TE *__restrict__ out, int64_t npieces) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h >> 3;
    int t = static_cast<int>(idx / nv);
    const int v = static_cast<int>(idx - static_cast<int64_t>(t) * nv);
    if constexpr (WT) t = __builtin_amdgcn_readfirstlane(t);   // one token per wave: scalar index loads
    const int64_t P = npieces / nv * k;   // rows of y
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // the slots in chunks of KM (one chunk unless k > 8): indices without
    // branches (slots past the chunk re-read its last slot), then every row
    // piece loaded raw before any is used: one round trip per phase
    for (int j0 = 0; j0 < k; j0 += KM) {
        const int kc = min(KM, k - j0);
        const int64_t base = static_cast<int64_t>(t) * k + j0;
        int rows[KM];
        float w[KM];
        bool ok[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            rows[j] = row_of[base + (j < kc ? j : kc - 1)];
            w[j] = topk_w ? topk_w[base + (j < kc ? j : kc - 1)] : 1.0f;
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            ok[j] = j < kc && rows[j] >= 0 && rows[j] < P;
            rows[j] = ok[j] ? rows[j] : 0;
        }
        Raw8<TE> yr[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc) raw8_load_nt(y + static_cast<int64_t>(rows[j]) * h + 8 * v, yr[j]);
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc) {
                float yv[8];
                raw8_f32(yr[j], yv);
                // a dropped pair (row -1) loaded row 0 only to keep the loads
                // uniform: its value is masked, not just its weight, so that a
                // non-finite row 0 cannot reach this token (0 * inf = NaN)
#pragma unroll
                for (int i = 0; i < 8; ++i) yv[i] = ok[j] ? yv[i] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], yv[i], acc[i]);
            }
    }
    if (y_sh) {
        float sv[8];
        load8_nt(y_sh + static_cast<int64_t>(t) * h + 8 * v, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sv[i];
    }
    store8_nt(out + static_cast<int64_t>(t) * h + 8 * v, acc);
}

// One block per token with one thread per 8-element piece (blockDim =
// h/8 rounded up to a wave, at most 1024; a thread takes pieces v, v +
// blockDim, ...): the piece of grad_out and the k pieces of y are loaded
// before use. The dot products are reduced in a fixed order: a shuffle tree
// in each wave, then the waves in order.
template <typename TE>
__global__ __launch_bounds__(1024) void unpermute_bwd_kernel(
    const TE *__restrict__ gout, const TE *__restrict__ y, int h, int k,
    const int32_t *__restrict__ row_of, const float *__restrict__ topk_w, TE *__restrict__ gy,
    float *__restrict__ gw) {
    __shared__ float red[8][16];
    const int t = blockIdx.x;
    const int nv = h / 8;
    // the slots in chunks of 8 (one chunk unless k > 8)
    for (int j0 = 0; j0 < k; j0 += 8) {
        const int kc = min(8, k - j0);
        const int64_t base = static_cast<int64_t>(t) * k + j0;
        int rows[8];
        float w[8], dot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            rows[j] = j < kc ? row_of[base + j] : -1;
            if (rows[j] >= static_cast<int64_t>(gridDim.x) * k) rows[j] = -1;   // rows of y: T k
            w[j] = j < kc ? topk_w[base + j] : 0.0f;
            dot[j] = 0.0f;
        }
        for (int v = threadIdx.x; v < nv; v += blockDim.x) {
            // every piece loaded raw before any is used (one round trip)
            Raw8<TE> gr, yr[8];
            raw8_load_nt(gout + static_cast<int64_t>(t) * h + 8 * v, gr);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < kc) raw8_load_nt(y + static_cast<int64_t>(rows[j] >= 0 ? rows[j] : 0) * h + 8 * v, yr[j]);
            float g[8];
            raw8_f32(gr, g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < kc && rows[j] >= 0) {
                    float yv[8], d[8];
                    raw8_f32(yr[j], yv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        dot[j] = fmaf(g[i], yv[i], dot[j]);
                        d[i] = w[j] * g[i];
                    }
                    store8_nt(gy + static_cast<int64_t>(rows[j]) * h + 8 * v, d);
                }
            }
        }
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float sdot = dot[j];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) sdot += __shfl_down(sdot, off);
            if (lane == 0) red[j][wave] = sdot;
        }
        __syncthreads();
        if (threadIdx.x < kc) {
            const int j = threadIdx.x;
            float sdot = red[j][0];
            for (int wv = 1; wv < nw; ++wv) sdot += red[j][wv];
            gw[base + j] = sdot;
        }
        __syncthreads();   // red is rewritten by the next chunk
    }
}

// One thread per 8-element piece (flat grid over T x h/8): the k pieces of
// grad_x_perm and the router term's gate pieces are loaded before use.
template <typename TE, int KM, bool WT>
__global__ __launch_bounds__(256) void permute_bwd_kernel(
    const TE *__restrict__ gxp, int h, int k, const int32_t *__restrict__ row_of,
    const float *__restrict__ gl, const int32_t *__restrict__ topk_idx,
    const TE *__restrict__ wg, int E, TE *__restrict__ gx, int64_t npieces) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h >> 3;
    int t = static_cast<int>(idx / nv);
    const int v = static_cast<int>(idx - static_cast<int64_t>(t) * nv);
    if constexpr (WT) t = __builtin_amdgcn_readfirstlane(t);   // one token per wave: scalar index loads
    const int64_t P = npieces / nv * k;   // rows of grad_x_perm
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // the slots in chunks of KM (one chunk unless k > 8); every load of a
    // phase is issued before any of its values is used (k is uniform, so
    // `j < kc` is a scalar branch; out-of-range indices are clamped to a
    // valid address and their terms dropped by a select), so the phases cost
    // one memory round trip each
    for (int j0 = 0; j0 < k; j0 += KM) {
        const int kc = min(KM, k - j0);
        const int64_t base = static_cast<int64_t>(t) * k + j0;
        // index loads without branches: slots past the chunk re-read its last slot
        int rows[KM], ex[KM];
        float dl[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) rows[j] = row_of[base + (j < kc ? j : kc - 1)];
        if (gl) {
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                ex[j] = topk_idx[base + (j < kc ? j : kc - 1)];
                dl[j] = gl[base + (j < kc ? j : kc - 1)];
            }
        } else {
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                ex[j] = -1;
                dl[j] = 0.0f;
            }
        }
        bool rok[KM], eok[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            rok[j] = j < kc && rows[j] >= 0 && rows[j] < P;
            eok[j] = j < kc && ex[j] >= 0 && ex[j] < E;
            rows[j] = rok[j] ? rows[j] : 0;
            ex[j] = eok[j] ? ex[j] : 0;
        }
        Raw8<TE> d[KM], wr[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc) raw8_load_nt(gxp + static_cast<int64_t>(rows[j]) * h + 8 * v, d[j]);
        if (gl) {
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (j < kc) raw8_load(wg + static_cast<int64_t>(ex[j]) * h + 8 * v, wr[j]);
        }
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc) {
                float dv[8];
                raw8_f32(d[j], dv);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += rok[j] ? dv[i] : 0.0f;
            }
        if (gl) {
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (j < kc) {
                    float wv[8];
                    raw8_f32(wr[j], wv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(dl[j], eok[j] ? wv[i] : 0.0f, acc[i]);
                }
        }
    }
    store8_nt(gx + static_cast<int64_t>(t) * h + 8 * v, acc);
}

// Unweighted combine backward: grad_y[row_of[t,j]] = grad_out[t] for every
// j, one 8-element piece of grad_out per thread (loaded once, stored k times).
template <typename TE, int KM, bool WT>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const TE *__restrict__ gout, int h, int k,
                                                           const int32_t *__restrict__ row_of, TE *__restrict__ gy,
                                                           int64_t npieces) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= npieces) return;
    const int nv = h >> 3;
    int t = static_cast<int>(idx / nv);
    const int v = static_cast<int>(idx - static_cast<int64_t>(t) * nv);
    if constexpr (WT) t = __builtin_amdgcn_readfirstlane(t);   // one token per wave: scalar index loads
    const int64_t P = npieces / nv * k;
    // the piece and a chunk's KM row indices in flight together (slots past
    // the chunk re-read its last slot and store nothing; one chunk unless
    // k > 8)
    float g[8];
    for (int j0 = 0; j0 < k; j0 += KM) {
        const int kc = min(KM, k - j0);
        const int64_t base = static_cast<int64_t>(t) * k + j0;
        int rows[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) rows[j] = row_of[base + (j < kc ? j : kc - 1)];
        if (j0 == 0) load8_nt(gout + static_cast<int64_t>(t) * h + 8 * v, g);
#pragma unroll
        for (int j = 0; j < KM; ++j)
            if (j < kc && rows[j] >= 0 && rows[j] < P) store8_nt(gy + static_cast<int64_t>(rows[j]) * h + 8 * v, g);
    }
}

// f(KM, WT) with KM the top-k slots a thread walks at a time (k rounded up
// to 1, 2, 4 or 8, and 8 at a time for k > 8; slots past k re-read slot
// k - 1 and add nothing) and WT whether each
// wave's 64 pieces belong to one token (h / 8 a multiple of 64), so that the
// token's indices and weights are wave-uniform and read by scalar loads.
template <typename Fn>
void with_slots(int k, int64_t h, Fn &&f) {
    auto go = [&](auto km) {
        if ((h / 8) % 64 == 0) f(km, std::true_type{});
        else f(km, std::false_type{});
    };
    if (k <= 1) go(std::integral_constant<int, 1>{});
    else if (k <= 2) go(std::integral_constant<int, 2>{});
    else if (k <= 4) go(std::integral_constant<int, 4>{});
    else go(std::integral_constant<int, 8>{});
}

int check_common(const char *fn, int dtype, int64_t T, int64_t h, int k) {
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "%s: bad dtype %d", fn, dtype);
    MOE_CHECK_ARG(T >= 0 && h > 0 && k > 0, MOE_ERR_INVALID_ARG, "%s: bad sizes", fn);
    MOE_CHECK_ARG(k <= 256 && h % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: need k <= 256, h %% 64 == 0", fn);
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31) && T < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "%s: T*k must be < 2^31", fn);
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_unpermute(const void *y, int dtype, int64_t T, int64_t h, int k,
                             const int32_t *row_of, const float *topk_w, const void *y_sh,
                             void *out, void *stream) {
    clear_error();
    MOE_CHECK_ARG(T == 0 || (y && row_of && out), MOE_ERR_INVALID_ARG, "moe_unpermute: null required pointer");
    int st = check_common("moe_unpermute", dtype, T, h, k);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(aligned16(y) && aligned16(out) && (!y_sh || aligned16(y_sh)), MOE_ERR_INVALID_ARG,
                  "moe_unpermute: pointers must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    const int64_t npieces = T * (h / 8);
    const dim3 grid(static_cast<unsigned>((npieces + 255) / 256)), block(256);
    with_slots(k, h, [&](auto km, auto wt) {
        constexpr int KM = decltype(km)::value;
        constexpr bool WT = decltype(wt)::value;
        if (dtype == MOE_DTYPE_BF16)
            hipLaunchKernelGGL((unpermute_kernel<bf16_t, KM, WT>), grid, block, 0, s, static_cast<const bf16_t *>(y),
                               static_cast<int>(h), k, row_of, topk_w, static_cast<const bf16_t *>(y_sh),
                               static_cast<bf16_t *>(out), npieces);
        else
            hipLaunchKernelGGL((unpermute_kernel<float, KM, WT>), grid, block, 0, s, static_cast<const float *>(y),
                               static_cast<int>(h), k, row_of, topk_w, static_cast<const float *>(y_sh),
                               static_cast<float *>(out), npieces);
    });
    return check_launch("moe_unpermute");
}

extern "C" int moe_unpermute_bwd(const void *grad_out, const void *y, int dtype, int64_t T,
                                 int64_t h, int k, const int32_t *row_of, const float *topk_w,
                                 void *grad_y, float *grad_topk_w, void *stream) {
    clear_error();
    MOE_CHECK_ARG(T == 0 || (grad_out && row_of && grad_y && (topk_w == nullptr || (y && grad_topk_w))),
                  MOE_ERR_INVALID_ARG, "moe_unpermute_bwd: null required pointer");
    int st = check_common("moe_unpermute_bwd", dtype, T, h, k);
    if (st != MOE_OK) return st;
    if (topk_w == nullptr) {
        MOE_CHECK_ARG(aligned16(grad_out) && aligned16(grad_y), MOE_ERR_INVALID_ARG,
                      "moe_unpermute_bwd: pointers must be 16-byte aligned");
        if (T == 0) return MOE_OK;
        hipStream_t s = as_stream(stream);
        const int64_t npieces = T * (h / 8);
        const dim3 grid(static_cast<unsigned>((npieces + 255) / 256)), block(256);
        with_slots(k, h, [&](auto km, auto wt) {
            constexpr int KM = decltype(km)::value;
            constexpr bool WT = decltype(wt)::value;
            if (dtype == MOE_DTYPE_BF16)
                hipLaunchKernelGGL((scatter_rows_kernel<bf16_t, KM, WT>), grid, block, 0, s,
                                   static_cast<const bf16_t *>(grad_out), static_cast<int>(h), k, row_of,
                                   static_cast<bf16_t *>(grad_y), npieces);
            else
                hipLaunchKernelGGL((scatter_rows_kernel<float, KM, WT>), grid, block, 0, s,
                                   static_cast<const float *>(grad_out), static_cast<int>(h), k, row_of,
                                   static_cast<float *>(grad_y), npieces);
        });
        return check_launch("moe_unpermute_bwd");
    }
    MOE_CHECK_ARG(aligned16(grad_out) && aligned16(y) && aligned16(grad_y), MOE_ERR_INVALID_ARG,
                  "moe_unpermute_bwd: pointers must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    int bs = static_cast<int>(((h / 8 + 63) / 64) * 64);
    if (bs > 1024) bs = 1024;
    const dim3 grid(static_cast<unsigned>(T)), block(static_cast<unsigned>(bs));
    if (dtype == MOE_DTYPE_BF16)
        hipLaunchKernelGGL(unpermute_bwd_kernel<bf16_t>, grid, block, 0, s,
                           static_cast<const bf16_t *>(grad_out), static_cast<const bf16_t *>(y),
                           static_cast<int>(h), k, row_of, topk_w, static_cast<bf16_t *>(grad_y),
                           grad_topk_w);
    else
        hipLaunchKernelGGL(unpermute_bwd_kernel<float>, grid, block, 0, s,
                           static_cast<const float *>(grad_out), static_cast<const float *>(y),
                           static_cast<int>(h), k, row_of, topk_w, static_cast<float *>(grad_y),
                           grad_topk_w);
    return check_launch("moe_unpermute_bwd");
}

extern "C" int moe_permute_bwd(const void *grad_x_perm, int dtype, int64_t T, int64_t h, int k,
                               const int32_t *row_of, const float *grad_logits_sel,
                               const int32_t *topk_idx, const void *w_gate, int E, void *grad_x,
                               void *stream) {
    clear_error();
    MOE_CHECK_ARG(T == 0 || (grad_x_perm && row_of && grad_x), MOE_ERR_INVALID_ARG,
                  "moe_permute_bwd: null required pointer");
    MOE_CHECK_ARG(grad_logits_sel == nullptr || (topk_idx && w_gate && E > 0), MOE_ERR_INVALID_ARG,
                  "moe_permute_bwd: the router term needs topk_idx, w_gate and E");
    int st = check_common("moe_permute_bwd", dtype, T, h, k);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(aligned16(grad_x_perm) && aligned16(grad_x) && (!w_gate || aligned16(w_gate)),
                  MOE_ERR_INVALID_ARG, "moe_permute_bwd: pointers must be 16-byte aligned");
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    const int64_t npieces = T * (h / 8);
    const dim3 grid(static_cast<unsigned>((npieces + 255) / 256)), block(256);
    with_slots(k, h, [&](auto km, auto wt) {
        constexpr int KM = decltype(km)::value;
        constexpr bool WT = decltype(wt)::value;
        if (dtype == MOE_DTYPE_BF16)
            hipLaunchKernelGGL((permute_bwd_kernel<bf16_t, KM, WT>), grid, block, 0, s,
                               static_cast<const bf16_t *>(grad_x_perm), static_cast<int>(h), k, row_of,
                               grad_logits_sel, topk_idx, static_cast<const bf16_t *>(w_gate), E,
                               static_cast<bf16_t *>(grad_x), npieces);
        else
            hipLaunchKernelGGL((permute_bwd_kernel<float, KM, WT>), grid, block, 0, s,
                               static_cast<const float *>(grad_x_perm), static_cast<int>(h), k, row_of,
                               grad_logits_sel, topk_idx, static_cast<const float *>(w_gate), E,
                               static_cast<float *>(grad_x), npieces);
    });
    return check_launch("moe_permute_bwd");
}
