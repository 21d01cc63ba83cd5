// common.hpp -- device-side helpers shared by the gfx950 kernels of libdiffattn.
//
// Matrix-core layouts used throughout (wave64, gfx950):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l supplies row m = l % 32 and eight k-slots (l / 32, e), e = 0..7
//     B: lane l supplies column n = l % 32 and the same eight k-slots
//     D: lane l, register r holds D[m][n], n = l % 32,
//        m = 8 * (r / 4) + 4 * (l / 32) + (r % 4)
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: row m = l % 16, eight k-slots (l / 16, e); B: column n = l % 16, same slots
//     D: lane l, register r holds D[m][n], n = l % 16, m = 4 * (l / 16) + r
// Whatever order the hardware gives the k-slots, A and B share it, so a
// contraction is correct as long as both operands put the same k index in
// the same (lane group, element) slot -- which every kernel here does.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Lambdas inside the kernels capture the kernel's state by reference; one
// left out of line would move that state (parameters, accumulator arrays) to
// scratch memory, so every such lambda is marked always-inline.
#define DA_INLINE __attribute__((always_inline))

namespace da {

// Index of the calling wave in its work-group, as a wave-uniform (scalar)
// value. Derived from threadIdx.x alone the compiler treats it as per-lane:
// a kernel-argument pointer chosen by wave index is then fetched with a
// vector load, whose vmcnt wait also waits for every global -> LDS tile copy
// the wave has in flight.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Load of a wave-uniform value that no kernel writes while this one runs,
// through the constant address space: a scalar load, counted by lgkmcnt. As a
// vector load inside a tile loop its vmcnt wait would also wait for the tile
// copies issued before it.
__device__ __forceinline__ float ld_uniform(const float *p) {
    return *(const __attribute__((address_space(4))) float *)(uintptr_t)p;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32). Inputs here are <= 0 or -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack two fp32 values to bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 pack2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
    bf16x2 p0 = pack2(a0, a1), p1 = pack2(a2, a3), p2 = pack2(a4, a5), p3 = pack2(a6, a7);
    bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Combine a value with the one held by lane l ^ 32 (the other half of the
// wave) using v_permlane32_swap (a VALU lane swap, no LDS round trip): with
// both operands = x, the two results hold x[l % 32] and x[32 + l % 32].
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace da
