// Route stage: fp32 gate logits in a fixed summation order, selection key,
// wave-level top-k with lowest-index ties, renormalised routing weights,
// routing map and per-expert counts.
//
// Router maths: "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2.2 (gating l = W_r^T x, softmax or sigmoid scores, top-k;
// the aux-loss-free selection bias of DeepSeek-V3) and section 5.1 (router in
// fp32); top-k renormalisation: "emerging-techniques-moe-training", Quick
// Start and Mixtral block.
//
// Work layout. A block of 4 waves holds 8 tokens. Its work items are
// (token, group of EPG experts): EPG = 8 when E is large (each loaded x piece
// feeds 8 experts), EPG = 1 when E <= 16 (more items, hence more waves in
// flight, for a pass that is then bound by HBM latency rather than ALU). The
// 8 lanes of a lane group serve one item; lane q owns residues 8q..8q+7 of
// every 64-wide chunk of h, so the 64 partial sums of the fixed order are
// spread 8 per lane over 8 lanes, and each lane reads 16 contiguous bytes of
// x and of each gate row per chunk. The halving tree of the order maps to:
// s=32 -> lane q+4, s=16 -> lane q+2, s=8 -> lane q+1, then s=4,2,1 inside
// lane 0's registers.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kTokPerBlock = 8;
constexpr int kMaxE = 256;

// sigma_c: clamp to [-80,80]; in fp64, d = 1 + exp(-l) with exp evaluated as
// Cody-Waite reduction (n = rint(y log2 e); r = y - n ln2 with ln2 split into
// a high part with 32 trailing zero bits and a low part) and the degree-13
// Taylor polynomial of e^r in Horner form with coefficients 1/m! rounded to
// nearest; s = 1/d correctly rounded; round s to fp32. All IEEE-exact or
// correctly rounded steps, so the bits are fixed by the definition.
__device__ __forceinline__ float sigmoid_canonical(float l) {
    if (l != l) return l;
    if (l > 80.0f) l = 80.0f;
    if (l < -80.0f) l = -80.0f;
    const double y = -static_cast<double>(l);
    const double n = rint(__dmul_rn(y, 1.4426950408889634));
    double r = __fma_rn(-n, 6.93147180369123816490e-01, y);
    r = __fma_rn(-n, 1.90821492927058770002e-10, r);
    double p = 1.0 / 6227020800.0;                 // 1/13!
    p = __fma_rn(p, r, 1.0 / 479001600.0);         // 1/12!
    p = __fma_rn(p, r, 1.0 / 39916800.0);          // 1/11!
    p = __fma_rn(p, r, 1.0 / 3628800.0);           // 1/10!
    p = __fma_rn(p, r, 1.0 / 362880.0);            // 1/9!
    p = __fma_rn(p, r, 1.0 / 40320.0);             // 1/8!
    p = __fma_rn(p, r, 1.0 / 5040.0);              // 1/7!
    p = __fma_rn(p, r, 1.0 / 720.0);               // 1/6!
    p = __fma_rn(p, r, 1.0 / 120.0);               // 1/5!
    p = __fma_rn(p, r, 1.0 / 24.0);                // 1/4!
    p = __fma_rn(p, r, 1.0 / 6.0);                 // 1/3!
    p = __fma_rn(p, r, 0.5);                       // 1/2!
    p = __fma_rn(p, r, 1.0);                       // 1/1!
    p = __fma_rn(p, r, 1.0);                       // 1/0!
    const double e = ldexp(p, static_cast<int>(n));
    const double d = __dadd_rn(1.0, e);
    return static_cast<float>(__ddiv_rn(1.0, d));
}

// Total order of the selection: a before b iff key_a > key_b, or equal keys
// and a lower expert index.
__device__ __forceinline__ bool precedes(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Raw 16-byte piece of 8 elements (bf16) or half of one (fp32 needs two).
template <typename TIn> struct Piece;
template <> struct Piece<bf16_t> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const u32x4 *>(p); }
    __device__ __forceinline__ float at(int s) const {
        const uint32_t w = v[s >> 1];
        return (s & 1) ? bf16hi(w) : bf16lo(w);
    }
};
template <> struct Piece<float> {
    u32x4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const u32x4 *>(p);
        b = *reinterpret_cast<const u32x4 *>(p + 4);
    }
    __device__ __forceinline__ float at(int s) const {
        return __uint_as_float(s < 4 ? a[s] : b[s - 4]);
    }
};

// Halving tree of the fixed order over the 64 partial sums held 8 per lane
// by the 8 lanes of a lane group; the result lands in lane q = 0, slot 0.
__device__ __forceinline__ float gate_tree(float *p) {
#pragma unroll
    for (int s = 0; s < 8; ++s) p[s] = p[s] + __shfl_down(p[s], 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) p[s] = p[s] + __shfl_down(p[s], 2);
#pragma unroll
    for (int s = 0; s < 8; ++s) p[s] = p[s] + __shfl_down(p[s], 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) p[s] = p[s] + p[s + 4];
#pragma unroll
    for (int s = 0; s < 2; ++s) p[s] = p[s] + p[s + 2];
    return p[0] + p[1];
}

// Logits of one work item: token tt of the block against EPG consecutive
// experts starting at e0. U chunks are loaded before they are used so that
// several loads per lane are in flight.
template <typename TIn, int EPG, int U>
__device__ __forceinline__ void gate_item(const TIn *__restrict__ xrow, const TIn *__restrict__ wg,
                                          int h, int E, int e0, int q, float (*acc)[8]) {
#pragma unroll
    for (int ee = 0; ee < EPG; ++ee)
#pragma unroll
        for (int s = 0; s < 8; ++s) acc[ee][s] = 0.0f;
    int64_t woff[EPG];
#pragma unroll
    for (int ee = 0; ee < EPG; ++ee) {
        const int e = e0 + ee < E ? e0 + ee : E - 1;
        woff[ee] = static_cast<int64_t>(e) * h + 8 * q;
    }
    const int nchunk = h >> 6;
    int c = 0;
    for (; c + U <= nchunk; c += U) {
        Piece<TIn> xp[U], wp[U][EPG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xp[u].load(xrow + 64 * (c + u));
#pragma unroll
            for (int ee = 0; ee < EPG; ++ee) wp[u][ee].load(wg + woff[ee] + 64 * (c + u));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int ee = 0; ee < EPG; ++ee)
#pragma unroll
                for (int s = 0; s < 8; ++s) acc[ee][s] = fmaf(xp[u].at(s), wp[u][ee].at(s), acc[ee][s]);
    }
    for (; c < nchunk; ++c) {
        Piece<TIn> xp, wp;
        xp.load(xrow + 64 * c);
#pragma unroll
        for (int ee = 0; ee < EPG; ++ee) {
            wp.load(wg + woff[ee] + 64 * c);
#pragma unroll
            for (int s = 0; s < 8; ++s) acc[ee][s] = fmaf(xp.at(s), wp.at(s), acc[ee][s]);
        }
    }
}

// Work items of a block: (token tt in [0,8), expert group eg); lane group lg
// of the block (32 per block, 8 per wave) takes items lg, lg + 32, ...
template <typename TIn, int EPG, int U>
__global__ __launch_bounds__(256) void route_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ wg, const float *__restrict__ bg,
    const float *__restrict__ sel_bias, int T, int h, int E, int k, int sigmoid,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    uint8_t *__restrict__ rmap, int32_t *__restrict__ counts) {
    __shared__ float s_logit[kTokPerBlock][kMaxE];
    __shared__ float s_key[kTokPerBlock][kMaxE];
    __shared__ int s_cnt[kMaxE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;   // lane group within the wave
    const int q = lane & 7;    // residues 8q..8q+7 of each 64-chunk
    const int lg = wave * 8 + g;
    const int t0 = blockIdx.x * kTokPerBlock;

    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;

    const int ngroups = (E + EPG - 1) / EPG;
    const int nitems = kTokPerBlock * ngroups;
    for (int item = lg; item < nitems; item += 32) {
        const int tt = item % kTokPerBlock;
        const int e0 = (item / kTokPerBlock) * EPG;
        int t = t0 + tt;
        t = t < T ? t : T - 1;   // rows past T are read, never stored
        float acc[EPG][8];
        gate_item<TIn, EPG, U>(x + static_cast<int64_t>(t) * h + 8 * q, wg, h, E, e0, q, acc);
#pragma unroll
        for (int ee = 0; ee < EPG; ++ee) {
            const float l = gate_tree(acc[ee]);
            const int e = e0 + ee;
            if (q == 0 && e < E) s_logit[tt][e] = bg ? l + bg[e] : l;
        }
    }
    __syncthreads();

    // Selection keys (and the optional logits output, coalesced rows).
    for (int i = threadIdx.x; i < kTokPerBlock * E; i += blockDim.x) {
        const int tt = i / E, e = i - tt * E;
        const float l = s_logit[tt][e];
        if (logits_out && t0 + tt < T) logits_out[static_cast<int64_t>(t0 + tt) * E + e] = l;
        float key = l;
        if (sigmoid) {
            key = sigmoid_canonical(l);
            if (sel_bias) key = key + sel_bias[e];
        }
        if (key != key) key = -INFINITY;
        s_key[tt][e] = key + 0.0f;   // -0 -> +0
    }
    __syncthreads();

    // Top-k: wave 0, lane group g handles token g. Lane q owns experts
    // e = q + 8m; its removed experts are bits m of `removed`.
    const int t = t0 + g;
    if (wave == 0 && t < T) {
        const int nm = (E + 7) >> 3;
        uint32_t removed = 0;
        float sel_l[8];
        int sel_e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) { sel_l[j] = 0.0f; sel_e[j] = 0; }
        for (int j = 0; j < k; ++j) {
            float bk = 0.0f;
            int bi = 0x7fffffff;
            bool have = false;
            for (int m = 0; m < nm; ++m) {
                const int e = q + 8 * m;
                if (e >= E || ((removed >> m) & 1u)) continue;
                const float key = s_key[g][e];
                if (!have || precedes(key, e, bk, bi)) { bk = key; bi = e; have = true; }
            }
            if (!have) { bk = -INFINITY; bi = 0x7fffffff; }
            // reduce over the 8 lanes of the group
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) {
                const float ok = __shfl_xor(bk, off);
                const int oi = __shfl_xor(bi, off);
                if (precedes(ok, oi, bk, bi)) { bk = ok; bi = oi; }
            }
            if ((bi & 7) == q && bi < E) removed |= 1u << (bi >> 3);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                if (jj == j) { sel_e[jj] = bi; sel_l[jj] = s_logit[g][bi < E ? bi : 0]; }
        }
        if (q == 0) {
            float wsum = 0.0f, wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                wv[j] = 0.0f;
                if (j < k) {
                    if (sigmoid) wv[j] = 1.0f / (1.0f + expf(-sel_l[j]));
                    else wv[j] = expf(sel_l[j] - sel_l[0]);
                    wsum += wv[j];
                }
            }
            const float inv = 1.0f / wsum;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < k) {
                    topk_idx[static_cast<int64_t>(t) * k + j] = sel_e[j];
                    topk_w[static_cast<int64_t>(t) * k + j] = wv[j] * inv;
                    if (sel_e[j] >= 0 && sel_e[j] < E) atomicAdd(&s_cnt[sel_e[j]], 1);
                }
            }
        }
        if (rmap) {
            uint8_t *row = rmap + static_cast<int64_t>(t) * E;
            for (int e = q; e < E; e += 8) {
                bool on = false;
#pragma unroll
                for (int j = 0; j < 8; ++j) on |= (j < k) && (sel_e[j] == e);
                row[e] = on ? 1 : 0;
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (s_cnt[e]) atomicAdd(&counts[e], s_cnt[e]);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_route(const void *x, int dtype, int64_t T, int64_t h, const void *w_gate,
                         const float *b_gate, int E, int k, int score, const float *sel_bias,
                         float *logits, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
                         int32_t *counts, void *stream) {
    clear_error();
    MOE_CHECK_ARG(x && w_gate && topk_idx && topk_w && counts, MOE_ERR_INVALID_ARG,
                  "moe_route: null required pointer");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_route: bad dtype %d", dtype);
    MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID, MOE_ERR_INVALID_ARG,
                  "moe_route: bad score %d", score);
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG,
                  "moe_route: bad sizes T=%lld h=%lld E=%d k=%d", (long long)T, (long long)h, E, k);
    MOE_CHECK_ARG(h % 64 == 0, MOE_ERR_UNSUPPORTED, "moe_route: h=%lld not a multiple of 64",
                  (long long)h);
    MOE_CHECK_ARG(k <= E && E <= kMaxE && k <= 8, MOE_ERR_UNSUPPORTED,
                  "moe_route: need k <= E <= 256 and k <= 8 (E=%d k=%d)", E, k);
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31) && h < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_route: T*k must be < 2^31");
    MOE_CHECK_ARG(sel_bias == nullptr || score == MOE_SCORE_SIGMOID, MOE_ERR_INVALID_ARG,
                  "moe_route: sel_bias applies to sigmoid scoring only");
    MOE_CHECK_ARG(aligned16(x) && aligned16(w_gate), MOE_ERR_INVALID_ARG,
                  "moe_route: x and w_gate must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    launch_fill<int32_t>(counts, E, 0, s);
    if (T == 0) return check_launch("moe_route fill");
    const dim3 grid(static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock));
    const dim3 block(256);
    const int sig = score == MOE_SCORE_SIGMOID;
    const int hh = static_cast<int>(h), TT = static_cast<int>(T);
    if (dtype == MOE_DTYPE_BF16) {
        const bf16_t *xp = static_cast<const bf16_t *>(x), *wp = static_cast<const bf16_t *>(w_gate);
        if (E <= 16)
            hipLaunchKernelGGL((route_kernel<bf16_t, 1, 8>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map, counts);
        else
            hipLaunchKernelGGL((route_kernel<bf16_t, 8, 2>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map, counts);
    } else {
        const float *xp = static_cast<const float *>(x), *wp = static_cast<const float *>(w_gate);
        if (E <= 16)
            hipLaunchKernelGGL((route_kernel<float, 1, 4>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map, counts);
        else
            hipLaunchKernelGGL((route_kernel<float, 8, 1>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map, counts);
    }
    return check_launch("moe_route");
}
