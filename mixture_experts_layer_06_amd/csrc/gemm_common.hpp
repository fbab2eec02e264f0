// Shared pieces of the grouped GEMM kernels: segment/tile scheduling on the
// device and the fused epilogues.
//
// A grouped GEMM here computes, for every segment s (one expert's rows of the
// permuted activations, plus optionally the shared expert's rows),
//   C_s[m, n] = epilogue( sum_k A_s[m, k] * B_s[n, k] )
// with A_s row-major [M_s, K] and B_s row-major [N, K] (both K-contiguous).
// Segment sizes are read from `offsets` on the device, so the host never
// waits for the routing result.
#pragma once

#include "common.hpp"

namespace moe {

enum GemmMode { kModePlain = 0, kModeSwiGLU = 1, kModeGELU = 2, kModeF32Out = 3 };
// Added to kModeSwiGLU / kModeGELU: the activation of segment row r is scaled
// by GGArgs::row_w[r]. A separate instantiation, so the unscaled kernels are
// unchanged.
constexpr int kRowW = 8;

// fp32 C = A B^T for one segment of T rows (bf16 A [T][K], B [N][K]) on the
// grouped GEMM kernel, split along K when few tiles; ws: the grouped FFN's
// split workspace layout, offsets: 2 device ints set here. Used for the
// router's MFMA logits.
int gemm_bf16_f32out(const void *A, const void *B, int T, int K, int N, float *C, int32_t *offsets, void *ws,
                     size_t ws_bytes, hipStream_t s);
size_t gemm_split_workspace_bytes();

// Backward of the expert kinds the bf16 SwiGLU kernels do not cover (GELU in
// bf16 or fp32, SwiGLU in fp32), bias gradients included (NULL: skipped);
// and the per-segment column sums that give bias gradients (bf16 rows).
int ffn_bwd_generic(const void *grad_y, const void *x_perm, const void *act, const void *gu, int dtype, int64_t P,
                    int64_t h, int64_t F, int E, const int32_t *offsets, int act_kind, const void *w1, const void *w2,
                    void *grad_gu, void *grad_x_perm, float *grad_w1, float *grad_w2, float *grad_b1,
                    float *grad_b2, hipStream_t s);
int segment_colsums_bf16(const void *M, int N, const int32_t *offsets, int E, float *db, hipStream_t s,
                         const char *what);

struct GGArgs {
    const void *A;          // activations; segment s starts at row offsets[s]
    const void *B;          // weights, [E][nb_rows][K]
    const void *bias;       // [E][nb_rows] or null
    void *C;                // output, rows as A, N_out columns
    void *GU;               // SwiGLU only: pre-activations [rows][2*N_out] or null
    const void *A_sh;       // shared-expert segment (M_sh = 0: none)
    const void *B_sh;
    void *C_sh;
    void *GU_sh;
    int M_sh;
    const int32_t *offsets; // [E+1]
    int E;
    int N_out;              // output columns
    int K;                  // reduction length
    int n_tiles;            // ceil(N_out / tile width)
    int grid;               // blocks launched (persistent)
    float *ws;              // split workspace or null (bf16 forward kernel)
    int ws_tiles;           // fp32 partial tiles the workspace holds
    const int32_t *gather;  // null, or: row r of the segments is row gather[r] of A
    int a_rows;             // rows of A when gathering
    const float *row_w;     // null, or: the activation of segment row r is scaled by row_w[r]
                            // (shared-expert rows are not scaled)
};

constexpr int kMaxSeg = 260;

// Builds, in LDS, s_cum[s] = number of tiles of segments < s and returns the
// total. 256 threads; each thread covers two segments.
__device__ __forceinline__ int build_tile_prefix(const GGArgs &a, int BM, int *s_cum, int *s_tmp) {
    const int S = a.E + (a.M_sh > 0 ? 1 : 0);
    const int t = threadIdx.x;
    int v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = 2 * t + i;
        int m = 0;
        if (s < a.E) m = a.offsets[s + 1] - a.offsets[s];
        else if (s < S) m = a.M_sh;
        if (m < 0) m = 0;
        v[i] = s < S ? ((m + BM - 1) / BM) * a.n_tiles : 0;
    }
    s_tmp[t] = v[0] + v[1];
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int add = t >= d ? s_tmp[t - d] : 0;
        __syncthreads();
        s_tmp[t] += add;
        __syncthreads();
    }
    const int incl = s_tmp[t];
    const int excl = incl - v[0] - v[1];
    if (2 * t < kMaxSeg) s_cum[2 * t] = excl;
    if (2 * t + 1 < kMaxSeg) s_cum[2 * t + 1] = excl + v[0];
    __syncthreads();
    return s_tmp[255];
}

// Segment containing tile L: the largest s with s_cum[s] <= L.
__device__ __forceinline__ int find_segment(const int *s_cum, int S, int L) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= L) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b on XCD b % 8).
// Renumber so that the blocks of one XCD take consecutive tile indices:
// consecutive tiles share a weight panel, which then stays in that XCD's L2.
__device__ __forceinline__ int xcd_block_index(int b, int G) {
    if (G % 8 != 0) return b;
    return (b % 8) * (G / 8) + b / 8;
}

struct TileInfo {
    int seg, m0, n_tile, M, row0;   // row0: first row of the segment in A/C
    bool shared;
};

__device__ __forceinline__ TileInfo decode_tile(const GGArgs &a, const int *s_cum, int L, int BM) {
    const int S = a.E + (a.M_sh > 0 ? 1 : 0);
    TileInfo ti;
    ti.seg = find_segment(s_cum, S, L);
    ti.shared = ti.seg >= a.E;
    if (ti.shared) {
        ti.M = a.M_sh;
        ti.row0 = 0;
    } else {
        ti.row0 = a.offsets[ti.seg];
        ti.M = a.offsets[ti.seg + 1] - ti.row0;
    }
    const int mt = (ti.M + BM - 1) / BM;
    const int local = L - s_cum[ti.seg];
    // m fastest: consecutive tiles reuse the same weight panel
    ti.m0 = (local % mt) * BM;
    ti.n_tile = local / mt;
    return ti;
}

// Raw buffer resource over [p, p + bytes): reads past the end return zero,
// writes past it are dropped; the bound applies to voffset + soffset. p and
// bytes must be uniform across the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes = 0x7fffffffu) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    // the size too must be provably uniform, or every buffer access gets a
    // loop over the lanes' distinct descriptors
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo),
                                             static_cast<short>(0), static_cast<int>(n), 0x00020000);
}

#define MOE_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100, kSgDsWrite = 0x200, kSgVmemRead = 0x020;
// all LDS traffic of this wave done, then the workgroup barrier; the memory
// clobber keeps the compiler from moving LDS accesses across it
#define MOE_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }
// g * sigmoid(g) with the hardware exp2 and reciprocal (about 2 ulp; the
// result is rounded to bf16): six VALU operations instead of a library exp
// and an IEEE divide in the GEMM epilogue. Saturates correctly: g -> -inf
// gives exp2 -> inf, rcp -> 0, product -0; g -> +inf gives g.
__device__ __forceinline__ float silu_fast(float g) {
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_erf_f(float a) {
    return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
}

}  // namespace moe
