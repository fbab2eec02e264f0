// MXFP8 pieces shared by the forward and backward expert kernels: the
// quantisation rule ("Scalable Training of Mixture-of-Experts Models with
// Megatron Core", section 5.3.3: 1 x 32 blocks, E8M0 scales, E4M3
// elements) and the LDS layout of the scaled-MFMA operand tiles.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// E4M3 codes of four values y (fp32, the exact scaled values, |y| < 2^9),
// packed little-endian into a word: the hardware's round-to-nearest-even
// conversion (v_cvt_pk_fp8_f32, two values per instruction), with each
// value clamped to +-448 first, so that (464, 512) saturates to 448 like
// the rest of [448, 512) (alone, the conversion rounds it to 480, which
// E4M3 has no code for, and returns the NaN code). Checked on the device
// against a bitwise reference rounding for every fp32 in [0, 512) and its
// negative: equal everywhere (subnormals and signed zeros included).
// Finite inputs only.
__device__ __forceinline__ float e4m3_clamp(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }
__device__ __forceinline__ uint32_t e4m3_word(float y0, float y1, float y2, float y3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(y0), e4m3_clamp(y1), 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(y2), e4m3_clamp(y3), lo, true));
}

// Shared exponent of a block whose largest magnitude is amax (>= 0):
// floor(log2 amax) - 8 clamped to [-127, 127]; -127 for a zero block (fp32
// subnormal maxima also land on -127, as floor(log2) - 8 < -127 for them).
__device__ __forceinline__ int mx_block_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    const int eb = static_cast<int>(__float_as_uint(amax) >> 23);
    const int ex = eb == 0 ? -127 : eb - 127 - 8;
    return ex < -127 ? -127 : ex;
}

// One thread per block of 32 values of a row.
template <typename TE>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const TE *__restrict__ src, int64_t nblocks,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) load8(src + b * 32 + 8 * c, v + 8 * c);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int ex = mx_block_exponent(amax);
    u32x4 out[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t word = e4m3_word(ldexpf(v[4 * w], -ex), ldexpf(v[4 * w + 1], -ex),
                                        ldexpf(v[4 * w + 2], -ex), ldexpf(v[4 * w + 3], -ex));
        out[w >> 2][w & 3] = word;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(codes + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    scales[b] = static_cast<uint8_t>(ex + 127);
}

template <typename TE>
void launch_quantize(const TE *src, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t nb = rows * (K / 32);
    if (nb == 0) return;
    hipLaunchKernelGGL(mx_quantize_kernel<TE>, dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256), 0, s, src,
                       nb, codes, scales);
}

// fn(integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time.
template <int N, int I = 0, typename Fn>
__device__ __forceinline__ void constexpr_for(Fn &&fn) {
    if constexpr (I < N) {
        fn(std::integral_constant<int, I>{});
        constexpr_for<N, I + 1>(fn);
    }
}

// byte offset of 16-byte chunk c of row r in an operand region with
// 128-byte rows (a k-step of 128 fp8 values): the chunk index is XOR-ed with
// bits 1..3 of the row, which keeps both the row-chunk writes and the
// fragment reads free of LDS bank conflicts
__device__ __forceinline__ int mswz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

}  // namespace

// The MXFP8 grouped GEMM (256 x 256 tiles of scaled MFMAs, persistent grid)
// for the backward's products:
// * rows mode: C [P][N_out] = A B_e^T per token segment e (offsets), A the
//   codes [.][K] of the segment rows (row r is A row gather[r] when gather
//   is set; a_rows rows then), B_e = b_codes + e N_out K, both with their
//   block scales along K; C in fp32 (f32_out) or bf16.
// * k-segment mode: C[e] [M][N] (fp32) = A_e B_e^T with A [M][ld] and
//   B [N][ld] shared by the experts, expert e reducing over its columns
//   [poffs[e], poffs[e+1]) (multiples of 128); the last 128 columns of A and
//   B (and their scale bytes) must be zeros; M % 32 == 0.
int mx_gemm_rows(const uint8_t *a_codes, const uint8_t *a_scales, const int32_t *gather, int a_rows,
                 const int32_t *offsets, int E, int64_t P, const uint8_t *b_codes, const uint8_t *b_scales, int N_out,
                 int K, void *C, bool f32_out, hipStream_t s, const char *what);
int mx_gemm_kseg(const uint8_t *a_codes, const uint8_t *a_scales, int M, const uint8_t *b_codes,
                 const uint8_t *b_scales, int N, int64_t ld, const int32_t *poffs, int E, float *C, hipStream_t s,
                 const char *what);

}  // namespace moe
