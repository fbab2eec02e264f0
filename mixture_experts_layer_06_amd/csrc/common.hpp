// Internal helpers shared by the HIP sources of libmoe.so: status reporting,
// argument checks, device properties and bf16/fp32 element access.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- status

void set_error(const std::string &msg);
void clear_error();

#define MOE_CHECK_ARG(cond, code, ...)                                    \
    do {                                                                  \
        if (!(cond)) {                                                    \
            char _b[512];                                                 \
            snprintf(_b, sizeof(_b), __VA_ARGS__);                        \
            ::moe::set_error(_b);                                         \
            return (code);                                                \
        }                                                                 \
    } while (0)

// Checks the launch that was just enqueued.
int check_launch(const char *what);

// Number of compute units of the current device (cached per device).
int num_cus();

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------- elements

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16-byte vector
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));  // 8-byte vector

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

// Low and high bf16 halves of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two values rounded to nearest even in one v_cvt_pk_bf16_f32 (lo in the
// low half); NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 8 consecutive elements as fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16_t *p, float *v) {
    uint4 q = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16lo(q.x); v[1] = bf16hi(q.x);
    v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
    v[4] = bf16lo(q.z); v[5] = bf16hi(q.z);
    v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
}
__device__ __forceinline__ void load8(const float *p, float *v) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t *p, const float *v) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = q;
}
__device__ __forceinline__ void store8(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Fill kernel used instead of hipMemsetAsync so that the entry points stay
// safe to record in a HIP graph.
template <typename T>
__global__ void fill_kernel(T *p, int64_t n, T v) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

template <typename T>
inline void launch_fill(T *p, int64_t n, T v, hipStream_t s) {
    if (n <= 0) return;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n, v);
}

}  // namespace moe
