// Device helpers shared by the gfx950 kernels of liblora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace lora {

// Global-memory pointer. Loads through it are global loads; a generic
// pointer the compiler cannot place (one picked by a select, or read from a
// struct) gives flat loads, which also count against the LDS wait counter.
template <class T>
using gptr = const __attribute__((address_space(1))) T*;

template <class T>
__device__ __forceinline__ gptr<T> as_global(const void* p) {
    return (gptr<T>)p;
}

// 16 zero bytes in device memory: a masked-off 16-byte load reads from here
// (the address is selected, not the loaded value, so no load is waited on
// early and no branch is needed).
static __device__ const u32x4 kZeros16[1] = {{0, 0, 0, 0}};

__device__ __forceinline__ gptr<u32x4> or_zero(bool ok, const void* p) {
    return ok ? as_global<u32x4>(p) : as_global<u32x4>(kZeros16);
}

// Keeps the loads issued above this point above it: neither the optimiser
// nor the instruction scheduler moves memory operations across it, and it
// does not wait for them (it uses no loaded value).
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bit pattern, round to nearest, ties to even; NaN stays a
// (quiet) NaN. gfx950 converts in hardware (v_cvt_pk_bf16_f32, two values
// per instruction).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 16x16x32 bf16 matrix-core product: lane l supplies row (l % 16) of the
// left operand and column (l % 16) of the right one, 8 consecutive k each
// (k = 8 * (l / 16) + e); lane l receives rows 4 * (l / 16) + i, column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// 16x16x16 bf16 product, 4 consecutive k per lane (k = 4 * (l / 16) + e).
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}

}  // namespace lora
