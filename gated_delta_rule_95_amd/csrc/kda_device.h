// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;

// bf16 <-> fp32.  The fp32 -> bf16 direction rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }
__device__ __forceinline__ float u16_to_f(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Register exchanges across 16-lane rows and across half waves (gfx950).
// v_permlane16_swap a, b trades the odd rows of a with the even rows of b;
// v_permlane32_swap a, b trades the upper half of a with the lower half of
// b.  Starting from a = b = x, afterwards a holds, in every lane, the value
// of the even row of its row pair (upper: of the lower half) and b the value
// of the odd row (upper half).  They are written as inline assembly: with the
// same value in both operands, the compiler's handling of the swap builtins
// was seen to merge the two results (a + b compiled as 2a).  The s_nop pairs
// cover the two wait states between a vector write and the swap.
__device__ __forceinline__ void row_pair(float x, float &even, float &odd)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    even = __builtin_bit_cast(float, a);
    odd = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ void half_pair(float x, float &lower, float &upper)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    lower = __builtin_bit_cast(float, a);
    upper = __builtin_bit_cast(float, b);
}

// Element loads/stores that convert between the storage type and fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p) { return *p; }
    static __device__ __forceinline__ void st(float *p, float x) { *p = x; }
    // four consecutive elements (16-byte aligned for float, 8 for bf16)
    static __device__ __forceinline__ f32x4 ld4(const float *p) {
        return *reinterpret_cast<const f32x4 *>(p);
    }
    static __device__ __forceinline__ void st4(float *p, f32x4 x) {
        *reinterpret_cast<f32x4 *>(p) = x;
    }
};
template <> struct Elem<bf16> {
    static __device__ __forceinline__ float ld(const bf16 *p) { return bf2f(*p); }
    static __device__ __forceinline__ void st(bf16 *p, float x) { *p = f2bf(x); }
    static __device__ __forceinline__ f32x4 ld4(const bf16 *p) {
        bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
        return f32x4{bf2f(v[0]), bf2f(v[1]), bf2f(v[2]), bf2f(v[3])};
    }
    static __device__ __forceinline__ void st4(bf16 *p, f32x4 x) {
        bf16x4 v = {f2bf(x[0]), f2bf(x[1]), f2bf(x[2]), f2bf(x[3])};
        *reinterpret_cast<bf16x4 *>(p) = v;
    }
};

}  // namespace kda
