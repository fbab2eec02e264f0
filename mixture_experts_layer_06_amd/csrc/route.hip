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
#include "gemm_common.hpp"

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

// Routing weights of the k selected experts (logits sel_l, best first):
// softmax renormalised over them, or sigma(l_j) / sum of the selected sigmas.
__device__ __forceinline__ void route_weights(const float *sel_l, int k, int sigmoid, float *wv) {
    float wsum = 0.0f;
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
    for (int j = 0; j < 8; ++j) wv[j] = wv[j] * inv;
}

// Raw 16-byte piece of 8 elements (bf16) or half of one (fp32 needs two).
template <typename TIn> struct Piece;
template <> struct Piece<bf16_t> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const u32x4 *>(p); }
    // through a buffer resource: per-lane byte offset, uniform byte offset
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
        v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    }
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
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
        a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        b = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16, 0);
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
// BIGK (k > 8): each round's choice is recorded in LDS instead of the
// registers of the lane group, the weights are formed from there in the same
// order, and the routing map is read from the groups' removed-expert bits.
template <typename TIn, int EPG, int U, bool BIGK>
__global__ __launch_bounds__(256) void route_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ wg, const float *__restrict__ bg,
    const float *__restrict__ sel_bias, int T, int h, int E, int k, int sigmoid,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    uint8_t *__restrict__ rmap) {
    __shared__ float s_logit[kTokPerBlock][kMaxE];
    __shared__ float s_key[kTokPerBlock][kMaxE];
    __shared__ float s_sel_l[BIGK ? kTokPerBlock : 1][BIGK ? kMaxE : 1];
    __shared__ int s_sel_e[BIGK ? kTokPerBlock : 1][BIGK ? kMaxE : 1];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;   // lane group within the wave
    const int q = lane & 7;    // residues 8q..8q+7 of each 64-chunk
    const int lg = wave * 8 + g;
    const int t0 = blockIdx.x * kTokPerBlock;


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
            if constexpr (BIGK) {
                if (q == 0) {
                    s_sel_e[g][j] = bi;
                    s_sel_l[g][j] = s_logit[g][bi < E ? bi : 0];
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    if (jj == j) { sel_e[jj] = bi; sel_l[jj] = s_logit[g][bi < E ? bi : 0]; }
            }
        }
        if constexpr (BIGK) {
            // lane 0 of the group wrote the lists: the weights as in
            // route_weights, over k entries
            if (q == 0) {
                float wsum = 0.0f;
                for (int j = 0; j < k; ++j) {
                    const float l = s_sel_l[g][j];
                    wsum += sigmoid ? 1.0f / (1.0f + expf(-l)) : expf(l - s_sel_l[g][0]);
                }
                const float inv = 1.0f / wsum;
                for (int j = 0; j < k; ++j) {
                    const float l = s_sel_l[g][j];
                    const float wj = sigmoid ? 1.0f / (1.0f + expf(-l)) : expf(l - s_sel_l[g][0]);
                    topk_idx[static_cast<int64_t>(t) * k + j] = s_sel_e[g][j];
                    topk_w[static_cast<int64_t>(t) * k + j] = wj * inv;
                }
            }
            if (rmap) {
                uint8_t *row = rmap + static_cast<int64_t>(t) * E;
                for (int m = 0; q + 8 * m < E; ++m) row[q + 8 * m] = (removed >> m) & 1u;
            }
        } else {
            if (q == 0) {
                float wv[8];
                route_weights(sel_l, k, sigmoid, wv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (j < k) {
                        topk_idx[static_cast<int64_t>(t) * k + j] = sel_e[j];
                        topk_w[static_cast<int64_t>(t) * k + j] = wv[j];
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
    }
}


// Few experts (E <= 16, gate matrix <= 64 KB): one persistent block of 8
// waves per compute unit.
// - The block stages the gate matrix in LDS once, widened to fp32 (at most
//   128 KB; rows padded by 16 bytes), so the inner loop converts only the
//   token's values; blocks start
//   their staging at different offsets, so that the compute units of an XCD
//   do not all ask its L2 for the same lines at once.
// - It takes a contiguous run of tokens in rounds of R = 64 / ngroups tokens:
//   lane group lg (8 lanes) computes token lg / ngroups of the round against
//   EPG experts (lg % ngroups + m ngroups), in the fixed order of gate_item (lane q: residues 8q..8q+7
//   of every 64-chunk, fma chains over ascending chunks, then gate_tree).
// - x is streamed in batches of kFewU chunks, one batch ahead (the first
//   before the staging), with loads that take no branch, so that the
//   compiler waits for each chunk as it is used rather than for every load
//   in flight.
// - After each round one thread per token takes its keys, top-k (insertion
//   into a list kept in key order, experts in ascending order, so equal keys
//   keep the lower index first), weights and outputs: no shuffles or
//   barriers on that path; it adds the token's experts to the block's LDS
//   histogram, which is added into `counts` (zeroed by the caller) with one
//   atomic per expert when the block ends.
constexpr int kFewU = 8;
constexpr int kFewMaxR = 64;

template <typename TIn, int EPG>
__global__ __launch_bounds__(512) void route_few_kernel(
    const TIn *__restrict__ x, const TIn *__restrict__ wg, const float *__restrict__ bg,
    const float *__restrict__ sel_bias, int T, int h, int E, int k, int sigmoid, int tpb,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    uint8_t *__restrict__ rmap, int32_t *__restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_wdyn[];   // fp32 [E][h]
    __shared__ float s_logit[kFewMaxR][17];
    __shared__ float s_bg[16], s_sel[16];   // gate bias, selection bias (0 when absent)
    __shared__ int s_cnt[16];               // the block's selections per expert
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 3, q = lane & 7;
    const int lg = wave * 8 + g;              // lane group 0..63
    const int ngroups = (E + EPG - 1) / EPG;
    const int R = kFewMaxR / ngroups;         // tokens per round
    // lane group lg: token tt of the round, experts eg, eg + ngroups, ...
    // (the two lane groups of a 16-lane quarter then read neighbouring
    // experts, whose padded LDS rows start 16 bytes apart in the banks)
    const int tt = lg / ngroups, eg = lg % ngroups;
    const bool item = tt < R;                 // lane groups past R * ngroups idle in the gate phase
    const int t_begin = blockIdx.x * tpb;
    const int t_end = min(T, t_begin + tpb);
    const int nrounds = (t_end - t_begin + R - 1) / R;
    const int nchunk = h >> 6;
    // batches per token, rounded up to even (an extra batch past the row
    // loads but computes nothing), so that the two register buffers keep
    // fixed roles: even batches in xa, odd ones in xb
    const int nb = ((nchunk + kFewU - 1) / kFewU + 1) & ~1;
    const int total = nrounds * nb;

    // batch i: kFewU chunks of a token row, without branches (chunks past
    // the row re-read its last chunk; rows past the block's range re-read a
    // valid row), through a buffer resource over x: one per-lane offset (the
    // row and the lane's residues) and a uniform offset per chunk, so no
    // 64-bit address registers are built per load
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(static_cast<int64_t>(T) * h * sizeof(TIn)));
    auto load_batch = [&](Piece<TIn> (&xp)[kFewU], int i) {
        int t = t_begin + (i / nb) * R + (item ? tt : 0);
        t = min(t, T - 1);
        const int c0 = __builtin_amdgcn_readfirstlane((i % nb) * kFewU);
        const int voff = (t * h + 8 * q) * static_cast<int>(sizeof(TIn));
#pragma unroll
        for (int u = 0; u < kFewU; ++u)
            xp[u].load_buf(rx, voff, 64 * min(c0 + u, nchunk - 1) * static_cast<int>(sizeof(TIn)));
    };

    Piece<TIn> xa[kFewU], xb[kFewU];
    load_batch(xa, 0);

    // the biases into LDS too: a global load in the round's epilogue would
    // make the wave wait for every token batch loaded ahead of it
    if (tid < E) {
        s_bg[tid] = bg ? bg[tid] : 0.0f;
        s_sel[tid] = sel_bias ? sel_bias[tid] : 0.0f;
        s_cnt[tid] = 0;
    }
    // the gate matrix, widened to fp32, into LDS: 8 elements per thread and
    // step, the block's starting piece rotated by its index
    float *wl = reinterpret_cast<float *>(s_wdyn);
    const int hp = h + 4;   // LDS row stride of the gate matrix (floats)
    {
        // all of a thread's pieces loaded before any is stored (one round
        // trip; E h / 8 <= 4096 pieces, so at most 8 per thread)
        const int n8 = E * h / 8;
        const int rot = static_cast<int>((static_cast<int64_t>(blockIdx.x) * 97) % n8);
        Piece<TIn> w[8];
        int jj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int j = min(tid + 512 * u, n8 - 1) + rot;
            jj[u] = j >= n8 ? j - n8 : j;
            w[u].load(wg + 8 * static_cast<int64_t>(jj[u]));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (tid + 512 * u < n8) {
                float4 lo, hi;
                lo.x = w[u].at(0); lo.y = w[u].at(1); lo.z = w[u].at(2); lo.w = w[u].at(3);
                hi.x = w[u].at(4); hi.y = w[u].at(5); hi.z = w[u].at(6); hi.w = w[u].at(7);
                const int e = (8 * jj[u]) / h, c = 8 * jj[u] - e * h;
                *reinterpret_cast<float4 *>(wl + e * hp + c) = lo;
                *reinterpret_cast<float4 *>(wl + e * hp + c + 4) = hi;
            }
        }
    }
    __syncthreads();
    int woff[EPG];
#pragma unroll
    for (int ee = 0; ee < EPG; ++ee) woff[ee] = min(eg + ee * ngroups, E - 1) * hp + 8 * q;

    float acc[EPG][8];
    auto zero = [&]() {
#pragma unroll
        for (int ee = 0; ee < EPG; ++ee)
#pragma unroll
            for (int s = 0; s < 8; ++s) acc[ee][s] = 0.0f;
    };
    // fma chains over the batch's chunks, ascending (the fixed order)
    auto compute = [&](const Piece<TIn> (&xp)[kFewU], int i) {
        const int c0 = (i % nb) * kFewU;
#pragma unroll
        for (int u = 0; u < kFewU; ++u) {
            if (c0 + u < nchunk) {
                float xv[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) xv[s] = xp[u].at(s);
#pragma unroll
                for (int ee = 0; ee < EPG; ++ee) {
                    const float *wp = wl + woff[ee] + 64 * (c0 + u);
                    const float4 lo = *reinterpret_cast<const float4 *>(wp);
                    const float4 hi = *reinterpret_cast<const float4 *>(wp + 4);
                    const float wv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int s = 0; s < 8; ++s) acc[ee][s] = fmaf(xv[s], wv[s], acc[ee][s]);
                }
            }
        }
    };
    // end of a round: logits to LDS, then one thread per token selects
    auto finish_round = [&](int r) {
#pragma unroll
        for (int ee = 0; ee < EPG; ++ee) {
            const float l = gate_tree(acc[ee]);
            const int e = eg + ee * ngroups;
            if (item && q == 0 && e < E) s_logit[tt][e] = bg ? l + s_bg[e] : l;
        }
        __syncthreads();
        const int t = t_begin + r * R + tid;
        if (tid < R && t < t_end) {
            // the k best (key, expert) so far, in selection order
            float sk[8], sl[8];
            int se[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) { sk[j] = -INFINITY; sl[j] = 0.0f; se[j] = 0x7fffffff; }
            for (int e = 0; e < E; ++e) {
                const float l = s_logit[tid][e];
                if (logits_out) logits_out[static_cast<int64_t>(t) * E + e] = l;
                float key = l;
                if (sigmoid) {
                    key = sigmoid_canonical(l);
                    if (sel_bias) key = key + s_sel[e];
                }
                if (key != key) key = -INFINITY;
                key = key + 0.0f;   // -0 -> +0
                // insert (key, e) before the first entry it precedes; experts
                // arrive in ascending order, so it never precedes an equal key
#pragma unroll
                for (int j = 7; j >= 0; --j) {
                    if (j >= k) continue;
                    const bool here = precedes(key, e, sk[j], se[j]) && (j == 0 || !precedes(key, e, sk[j - 1], se[j - 1]));
                    const bool shift = j > 0 && precedes(key, e, sk[j - 1], se[j - 1]);
                    if (shift) { sk[j] = sk[j - 1]; sl[j] = sl[j - 1]; se[j] = se[j - 1]; }
                    else if (here) { sk[j] = key; sl[j] = l; se[j] = e; }
                }
            }
            float wv[8];
            route_weights(sl, k, sigmoid, wv);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < k) {
                    topk_idx[static_cast<int64_t>(t) * k + j] = se[j];
                    topk_w[static_cast<int64_t>(t) * k + j] = wv[j];
                    atomicAdd(&s_cnt[se[j]], 1);
                }
            }
            if (rmap) {
                uint8_t *row = rmap + static_cast<int64_t>(t) * E;
                for (int e = 0; e < E; ++e) {
                    bool on = false;
#pragma unroll
                    for (int j = 0; j < 8; ++j) on |= (j < k) && (se[j] == e);
                    row[e] = on ? 1 : 0;
                }
            }
        }
        __syncthreads();   // s_logit is rewritten by the next round
    };

    // Two buffers, one batch ahead. Every prefetch is issued, clamped to the
    // last batch at the end, so that every path keeps the same loads in
    // flight and the compiler waits for each batch only when it is used.
    for (int r = 0; r < nrounds; ++r) {
        zero();
        for (int b = 0; b < nb; b += 2) {
            const int i = r * nb + b;
            load_batch(xb, min(i + 1, total - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(xa, i);
            load_batch(xa, min(i + 2, total - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(xb, i + 1);
        }
        finish_round(r);
    }
    // finish_round ends with a barrier, so the histogram is complete
    if (tid < E && s_cnt[tid]) atomicAdd(&counts[tid], s_cnt[tid]);
}

// Tokens per expert from topk_idx: a histogram in LDS per block of
// kCountChunk entries, then (one block) the bins written directly or (more
// blocks) added into counts, which the caller has zeroed. Per-token global
// atomics into E adjacent counters would serialise in a few L2 lines.
constexpr int kCountChunk = 65536;
__global__ __launch_bounds__(1024) void count_kernel(const int32_t *__restrict__ topk_idx, int64_t n, int E,
                                                     int32_t *__restrict__ counts) {
    __shared__ int s_hist[16][kMaxE];   // one sub-histogram per wave: fewer colliding LDS atomics
    const int wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 16 * kMaxE; i += blockDim.x) s_hist[i / kMaxE][i % kMaxE] = 0;
    __syncthreads();
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * kCountChunk;
    const int64_t hi = lo + kCountChunk < n ? lo + kCountChunk : n;
    // 16 loads of 4 entries per thread, all in flight (kCountChunk = 1024 *
    // 64); the chunk start is a multiple of 4 entries, so 16-byte loads are
    // aligned when topk_idx is
    int v[16][4];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int64_t i = lo + 4 * (static_cast<int64_t>(u) * blockDim.x + threadIdx.x);
        if (i + 4 <= hi) {
            const int4 q = *reinterpret_cast<const int4 *>(topk_idx + i);
            v[u][0] = q.x; v[u][1] = q.y; v[u][2] = q.z; v[u][3] = q.w;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[u][r] = i + r < hi ? topk_idx[i + r] : -1;
        }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (v[u][r] >= 0 && v[u][r] < E) atomicAdd(&s_hist[wave][v[u][r]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) c += s_hist[w][e];
        if (gridDim.x == 1) counts[e] = c;
        else if (c) atomicAdd(&counts[e], c);
    }
}

// ---------------------------------------------------------------------------
// Fast path with the same results (many experts, bf16, no logits output).
//
// 1. l'(t,e) by bf16 MFMA with fp32 accumulation: the grouped GEMM kernel
//    (v_mfma_f32_32x32x16_bf16, one accumulator chain along h per piece, at
//    most 8 pieces summed in fp32 when the few tiles are split along h),
//    and |x_t|_2, |w_e|_2.
// 2. Both l' and the fixed-order logit l differ from the exact dot product
//    by at most a multiple of u * S, S = sum_i |x_i w_i| <= |x_t| |w_e|,
//    plus an absolute term for results below fp32's normal range: every
//    fp32 addition or fma rounds once, with an error of at most u times its
//    result or, for a subnormal result, half the subnormal spacing (2^-150);
//    the matrix instruction may also flush to zero a product of bf16 values
//    below 2^-126 (each losing less than 2^-126) or a subnormal partial sum.
//    Relative terms: the MFMA chain (h/16 + 16) u S (h/16 accumulations into
//    C, up to 16 roundings inside one instruction, the final sum of pieces
//    included), the fixed order (h/64 + 6) u S (chains of h/64 fmas, a
//    6-level tree); both doubled, the sum doubled again. Absolute term:
//    2 (h + h/16 + 70) 2^-126 (every product and every accumulation of the
//    MFMA flushed, which also covers the fixed order's h + 64 roundings of at
//    most 2^-150 each). The norms are computed in fp32, where the squares of
//    elements below 2^-63 underflow: each norm is raised by sqrt(h) 2^-63,
//    more than that loss can take away.
// 3. Keys of the interval ends (the sigmoid key is monotone in l, and so is
//    adding the selection bias), L_k = the k-th largest lower end; the
//    experts whose upper end reaches L_k contain the top-k (every other
//    expert is beaten by k experts for certain).
// 4. Those candidates get their logits in the fixed order (the same code as
//    route_kernel), and the top-k and the weights are taken from them
//    exactly as route_kernel does: identical results, bit for bit.

__global__ __launch_bounds__(64) void row_norm_kernel(const bf16_t *__restrict__ w, int h, float *__restrict__ out) {
    const bf16_t *row = w + static_cast<int64_t>(blockIdx.x) * h;
    float s = 0.0f;
    for (int i = 8 * threadIdx.x; i < h; i += 8 * 64) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(row + i);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = bf16lo(v[c]), b = bf16hi(v[c]);
            s = fmaf(a, a, s);
            s = fmaf(b, b, s);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    // squares below 2^-126 are lost: sqrt(h) 2^-63 bounds what they add
    if (threadIdx.x == 0) out[blockIdx.x] = sqrtf(s) + sqrtf(static_cast<float>(h)) * 0x1p-63f;
}

// One wave per token (4 per block). Lane l holds experts l + 64 m.
template <int SIGMOID>
__global__ __launch_bounds__(256) void route_select_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ wg, const float *__restrict__ bg,
    const float *__restrict__ sel_bias, const float *__restrict__ lp, const float *__restrict__ wnorm, int T,
    int h, int E, int k, float cb, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    uint8_t *__restrict__ rmap, int32_t *__restrict__ counts) {
    __shared__ int s_cand[4][kMaxE];
    __shared__ float s_cl[4][kMaxE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // no block-wide barrier below
    const bf16_t *xrow = x + static_cast<int64_t>(t) * h;

    // |x_t|_2 (fp32; its rounding is far inside the factor-2 margins, its
    // underflow is covered by the added term)
    float xs = 0.0f;
#pragma unroll 4
    for (int i = 8 * lane; i < h; i += 8 * 64) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xrow + i);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float a = bf16lo(v[c]), b = bf16hi(v[c]);
            xs = fmaf(a, a, xs);
            xs = fmaf(b, b, xs);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xs += __shfl_xor(xs, off);
    const float xn = sqrtf(xs) + sqrtf(static_cast<float>(h)) * 0x1p-63f;   // see row_norm_kernel
    // absolute part of the half-width (results below the normal range)
    const float dabs = 2.0f * static_cast<float>(h + h / 16 + 70) * 0x1p-126f;

    // key intervals
    constexpr int M = kMaxE / 64;
    float klo[M], khi[M];
    bool bad = false;
    // this lane's experts' inputs, all loaded before use (experts past E read
    // expert E - 1 and are dropped below)
    float lv[M], bv[M], nv[M], sv[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int ec = min(lane + 64 * m, E - 1);
        lv[m] = lp[static_cast<int64_t>(t) * E + ec];
        bv[m] = bg ? bg[ec] : 0.0f;
        nv[m] = wnorm[ec];
        sv[m] = (SIGMOID && sel_bias) ? sel_bias[ec] : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int e = lane + 64 * m;
        klo[m] = -INFINITY;
        khi[m] = -INFINITY;
        if (e < E) {
            float l = lv[m];
            if (bg) l = l + bv[m];
            const float d = cb * xn * nv[m] + 4.0f * 0x1p-24f * (fabsf(l) + (bg ? fabsf(bv[m]) : 0.0f)) + dabs;
            float lo = l - d, hi = l + d;
            if (!(lo == lo) || !(hi == hi) || isinf(lo) || isinf(hi)) bad = true;
            if (SIGMOID) {
                lo = sigmoid_canonical(lo);
                hi = sigmoid_canonical(hi);
                if (sel_bias) {
                    lo = lo + sv[m];
                    hi = hi + sv[m];
                }
            }
            klo[m] = lo;
            khi[m] = hi;
        }
    }
    bad = __any(bad);

    // L_k: the k-th largest lower end
    float Lk = -INFINITY;
    {
        uint32_t removed = 0;
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int e = lane + 64 * m;
                if (e < E && !((removed >> m) & 1u) && precedes(klo[m], e, bv, bi)) {
                    bv = klo[m];
                    bi = e;
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                if (precedes(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            if (bi < E && (bi & 63) == lane) removed |= 1u << (bi >> 6);
            Lk = bv;
        }
    }

    // candidates: upper end reaching L_k (all of them if a bound is not finite)
    int nc = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int e = lane + 64 * m;
        const bool c = e < E && (bad || !(khi[m] < Lk));
        const uint64_t mask = __ballot(c);
        if (c) s_cand[wave][nc + __popcll(mask & ((uint64_t(1) << lane) - 1))] = e;
        nc += __popcll(mask);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // exact logits of the candidates, eight at a time: lane group g (8
    // lanes) takes candidate c0 + g with route_kernel's fixed-order dot
    // product (lane q: residues 8q..8q+7 of each 64-chunk, 16-byte pieces),
    // so the same bits as the fixed-order pass
    {
        const int g = lane >> 3, q = lane & 7;
        for (int c0 = 0; c0 < nc; c0 += 8) {
            const int ci = c0 + g;
            const int e = s_cand[wave][ci < nc ? ci : nc - 1];
            float acc[1][8];
            gate_item<bf16_t, 1, 8>(xrow + 8 * q, wg, h, E, e, q, acc);
            const float l = gate_tree(acc[0]);
            if (q == 0 && ci < nc) s_cl[wave][ci] = bg ? l + bg[e] : l;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

    // exact top-k among the candidates (lane-strided), as route_kernel; the
    // winner's logit travels with its key and index through the reduction
    float sel_l[8];
    int sel_e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { sel_l[j] = 0.0f; sel_e[j] = 0; }
    // the keys of this lane's candidate slots, computed once (their
    // selection biases loaded together)
    int ce[M];
    float cl[M], ck[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int ci = lane + 64 * m;
        ce[m] = ci < nc ? s_cand[wave][ci] : 0;
        cl[m] = ci < nc ? s_cl[wave][ci] : 0.0f;
    }
    float cb_sel[M];
#pragma unroll
    for (int m = 0; m < M; ++m) cb_sel[m] = (SIGMOID && sel_bias) ? sel_bias[ce[m]] : 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float key = cl[m];
        if (SIGMOID) {
            key = sigmoid_canonical(cl[m]);
            if (sel_bias) key = key + cb_sel[m];
        }
        if (key != key) key = -INFINITY;
        ck[m] = key + 0.0f;
    }
    uint32_t removed = 0;   // bit m: candidate lane + 64 m taken
    for (int j = 0; j < k; ++j) {
        float bk = -INFINITY, bl = 0.0f;
        int bi = 0x7fffffff, bm = -1;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int ci = lane + 64 * m;
            if (ci >= nc || ((removed >> m) & 1u)) continue;
            if (bm < 0 || precedes(ck[m], ce[m], bk, bi)) { bk = ck[m]; bi = ce[m]; bl = cl[m]; bm = m; }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ok = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            const float ol = __shfl_xor(bl, off);
            if (precedes(ok, oi, bk, bi)) { bk = ok; bi = oi; bl = ol; }
        }
        // the lane that held the winner marks its slot
        if (bm >= 0 && s_cand[wave][lane + 64 * bm] == bi) removed |= 1u << bm;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            if (jj == j) { sel_e[jj] = bi; sel_l[jj] = bl; }
    }
    if (lane == 0) {
        float wv[8];
        route_weights(sel_l, k, SIGMOID, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < k) {
                topk_idx[static_cast<int64_t>(t) * k + j] = sel_e[j];
                topk_w[static_cast<int64_t>(t) * k + j] = wv[j];
            }
        }
    }
    if (rmap) {
        uint8_t *row = rmap + static_cast<int64_t>(t) * E;
        for (int e = lane; e < E; e += 64) {
            bool on = false;
#pragma unroll
            for (int j = 0; j < 8; ++j) on |= (j < k) && (sel_e[j] == e);
            row[e] = on ? 1 : 0;
        }
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

// Workspace: l' [T][E] fp32, |w_e| [E] fp32, 2 ints of GEMM offsets, then
// the GEMM's split workspace (256-byte aligned).
static size_t route_ws_head(int64_t T, int E) {
    const size_t b = sizeof(float) * (static_cast<size_t>(T) * E + E) + 2 * sizeof(int32_t);
    return (b + 255) & ~static_cast<size_t>(255);
}

extern "C" size_t moe_route_workspace_size(int64_t T, int E) {
    if (T <= 0 || E <= 0) return 0;
    return route_ws_head(T, E) + gemm_split_workspace_bytes();
}

extern "C" int moe_route(const void *x, int dtype, int64_t T, int64_t h, const void *w_gate,
                         const float *b_gate, int E, int k, int score, const float *sel_bias,
                         float *logits, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
                         int32_t *counts, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    MOE_CHECK_ARG(w_gate && counts && (T == 0 || (x && topk_idx && topk_w)), MOE_ERR_INVALID_ARG,
                  "moe_route: null required pointer");
    MOE_CHECK_ARG(dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16, MOE_ERR_INVALID_ARG,
                  "moe_route: bad dtype %d", dtype);
    MOE_CHECK_ARG(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID, MOE_ERR_INVALID_ARG,
                  "moe_route: bad score %d", score);
    MOE_CHECK_ARG(T >= 0 && h > 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG,
                  "moe_route: bad sizes T=%lld h=%lld E=%d k=%d", (long long)T, (long long)h, E, k);
    MOE_CHECK_ARG(h % 64 == 0, MOE_ERR_UNSUPPORTED, "moe_route: h=%lld not a multiple of 64",
                  (long long)h);
    MOE_CHECK_ARG(k <= E && E <= kMaxE, MOE_ERR_UNSUPPORTED, "moe_route: need k <= E <= 256 (E=%d k=%d)", E, k);
    MOE_CHECK_ARG(T * k < (int64_t(1) << 31) && h < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
                  "moe_route: T*k must be < 2^31");
    MOE_CHECK_ARG(sel_bias == nullptr || score == MOE_SCORE_SIGMOID, MOE_ERR_INVALID_ARG,
                  "moe_route: sel_bias applies to sigmoid scoring only");
    MOE_CHECK_ARG(aligned16(x) && aligned16(w_gate) && aligned16(topk_idx), MOE_ERR_INVALID_ARG,
                  "moe_route: x, w_gate and topk_idx must be 16-byte aligned");
    MOE_CHECK_ARG(workspace_bytes == 0 || workspace, MOE_ERR_INVALID_ARG,
                  "moe_route: workspace_bytes > 0 with a null workspace");
    hipStream_t s = as_stream(stream);
    const int64_t npairs = T * k;
    const unsigned count_blocks = static_cast<unsigned>((npairs + kCountChunk - 1) / kCountChunk);
    const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
    const size_t wbytes = static_cast<size_t>(E) * static_cast<size_t>(h) * es;
    // route_few_kernel: the gate in LDS, x through a buffer resource (32-bit offsets)
    const bool few = E <= 16 && wbytes <= 65536 && T * h * static_cast<int64_t>(es) < (int64_t(1) << 31);
    if (T == 0 || count_blocks > 1 || few) launch_fill<int32_t>(counts, E, 0, s);
    if (T == 0) return check_launch("moe_route fill");
    // the histogram of the selections, after whichever routing kernel ran
    auto count = [&](const char *what) {
        const int st = check_launch(what);
        if (st != MOE_OK) return st;
        hipLaunchKernelGGL(count_kernel, dim3(count_blocks), dim3(1024), 0, s, topk_idx, npairs, E, counts);
        return check_launch("moe_route counts");
    };
    const int sig = score == MOE_SCORE_SIGMOID;
    const int hh = static_cast<int>(h), TT = static_cast<int>(T);
    if (k > 8) {
        // more than 8 selections per token: the fixed-order kernel with its
        // selections kept in LDS (no workload on the pages selects more than 8)
        const dim3 grid(static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock));
        if (dtype == MOE_DTYPE_BF16) {
            const bf16_t *xp = static_cast<const bf16_t *>(x), *wp = static_cast<const bf16_t *>(w_gate);
            if (E <= 16)
                hipLaunchKernelGGL((route_kernel<bf16_t, 1, 8, true>), grid, dim3(256), 0, s, xp, wp, b_gate, sel_bias,
                                   TT, hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
            else
                hipLaunchKernelGGL((route_kernel<bf16_t, 8, 2, true>), grid, dim3(256), 0, s, xp, wp, b_gate, sel_bias,
                                   TT, hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
        } else {
            const float *xp = static_cast<const float *>(x), *wp = static_cast<const float *>(w_gate);
            if (E <= 16)
                hipLaunchKernelGGL((route_kernel<float, 1, 4, true>), grid, dim3(256), 0, s, xp, wp, b_gate, sel_bias,
                                   TT, hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
            else
                hipLaunchKernelGGL((route_kernel<float, 8, 1, true>), grid, dim3(256), 0, s, xp, wp, b_gate, sel_bias,
                                   TT, hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
        }
        return count("moe_route (k > 8)");
    }
    if (dtype == MOE_DTYPE_BF16 && logits == nullptr && E >= 32 && workspace && h <= 8192 &&
        workspace_bytes >= moe_route_workspace_size(T, E) && T * E < (int64_t(1) << 31)) {
        const bf16_t *xp = static_cast<const bf16_t *>(x), *wp = static_cast<const bf16_t *>(w_gate);
        float *lp = static_cast<float *>(workspace);
        float *wn = lp + static_cast<size_t>(T) * E;
        int32_t *offs = reinterpret_cast<int32_t *>(wn + E);
        char *gws = static_cast<char *>(workspace) + route_ws_head(T, E);
        hipLaunchKernelGGL(row_norm_kernel, dim3(E), dim3(64), 0, s, wp, hh, wn);
        const int st = gemm_bf16_f32out(xp, wp, TT, hh, E, lp, offs, gws, gemm_split_workspace_bytes(), s);
        if (st != MOE_OK) return st;
        // interval half-width per unit |x||w|: 2 * (2 (h/16 + 16) + 2 (h/64 + 6)) u
        const float cb = static_cast<float>(2.0 * (2.0 * (h / 16 + 16) + 2.0 * (h / 64 + 6)) * 0x1p-24 * 1.001);
        const dim3 g2(static_cast<unsigned>((T + 3) / 4));
        if (sig)
            hipLaunchKernelGGL((route_select_kernel<1>), g2, dim3(256), 0, s, xp, wp, b_gate, sel_bias, lp, wn, TT,
                               hh, E, k, cb, topk_idx, topk_w, routing_map, counts);
        else
            hipLaunchKernelGGL((route_select_kernel<0>), g2, dim3(256), 0, s, xp, wp, b_gate, sel_bias, lp, wn, TT,
                               hh, E, k, cb, topk_idx, topk_w, routing_map, counts);
        return count("moe_route (MFMA filter)");
    }
    const dim3 grid(static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock));
    const dim3 block(256);
    if (few) {
        // few experts: persistent blocks, the gate matrix staged in LDS once
        // per block (fp32); each lane group takes EPG = 2 experts of a token;
        // the blocks add their histograms into the zeroed counts
        const int ngroups = (E + 1) / 2;
        const int R = kFewMaxR / ngroups;
        int64_t G = (T + R - 1) / R;
        if (G > num_cus()) G = num_cus();
        const int tpb = static_cast<int>((T + G - 1) / G);
        G = (T + tpb - 1) / tpb;
        const size_t lds = static_cast<size_t>(E) * static_cast<size_t>(h + 4) * sizeof(float);
#define MOE_ROUTE_FEW(TIN)                                                                              \
    do {                                                                                              \
        auto kfn = &route_few_kernel<TIN, 2>;                                                         \
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kfn),                                 \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));   \
        hipLaunchKernelGGL(kfn, dim3(static_cast<unsigned>(G)), dim3(512), lds, s,                    \
                           static_cast<const TIN *>(x), static_cast<const TIN *>(w_gate), b_gate, sel_bias, \
                           TT, hh, E, k, sig, tpb, logits, topk_idx, topk_w, routing_map, counts);    \
    } while (0)
        if (dtype == MOE_DTYPE_BF16) MOE_ROUTE_FEW(bf16_t);
        else MOE_ROUTE_FEW(float);
#undef MOE_ROUTE_FEW
        return check_launch("moe_route");
    }
    if (dtype == MOE_DTYPE_BF16) {
        const bf16_t *xp = static_cast<const bf16_t *>(x), *wp = static_cast<const bf16_t *>(w_gate);
        if (E <= 16)
            hipLaunchKernelGGL((route_kernel<bf16_t, 1, 8, false>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
        else
            hipLaunchKernelGGL((route_kernel<bf16_t, 8, 2, false>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
    } else {
        const float *xp = static_cast<const float *>(x), *wp = static_cast<const float *>(w_gate);
        if (E <= 16)
            hipLaunchKernelGGL((route_kernel<float, 1, 4, false>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
        else
            hipLaunchKernelGGL((route_kernel<float, 8, 1, false>), grid, block, 0, s, xp, wp, b_gate, sel_bias, TT,
                               hh, E, k, sig, logits, topk_idx, topk_w, routing_map);
    }
    return count("moe_route");
}
