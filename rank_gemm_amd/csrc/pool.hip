// Slot-pool kernels: the finite check that precedes any write, and the
// zero-padded copy of one adapter into its slot ("43. Beyond text ...",
// inference.shantanugoel.com, section "Slots are storage; identities are
// content": validate all, then zero the slot and copy A into its first r
// rows and B into its first r columns).
#include "common.h"
#include "kernels.h"

namespace lora {

template <typename E>
__device__ __forceinline__ bool finite_elem(E v);
template <>
__device__ __forceinline__ bool finite_elem<uint16_t>(uint16_t v) {
    return (v & 0x7f80u) != 0x7f80u;
}
template <>
__device__ __forceinline__ bool finite_elem<float>(float v) {
    return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u;
}

template <typename E>
__global__ __launch_bounds__(256) void finite_kernel(const E* __restrict__ p, int64_t n, int* __restrict__ flag) {
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        bad |= !finite_elem<E>(p[i]);
    if (bad) *flag = 1;  // every writer stores the same value
}

template <typename E>
__global__ __launch_bounds__(256) void write_slot_kernel(E* __restrict__ A_pool, E* __restrict__ B_pool,
                                                         int32_t* __restrict__ rank, float* __restrict__ scale,
                                                         int slot, const E* __restrict__ A, const E* __restrict__ B,
                                                         int r, float sc, int r_max, int d_in, int d_out) {
    const int64_t na = (int64_t)r_max * d_in, nb = (int64_t)d_out * r_max;
    E* ad = A_pool + (int64_t)slot * na;
    E* bd = B_pool + (int64_t)slot * nb;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < na + nb; i += (int64_t)gridDim.x * 256) {
        if (i < na) {
            const int64_t q = i / d_in, k = i - q * d_in;
            ad[i] = (A && q < r) ? A[q * d_in + k] : E(0);
        } else {
            const int64_t ib = i - na, j = ib / r_max, q = ib - j * r_max;
            bd[ib] = (B && q < r) ? B[j * r + q] : E(0);
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        rank[slot] = r;
        scale[slot] = sc;
    }
}

hipError_t pool_check_finite(int dtype, const void* p, int64_t n, int* flag, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (dtype == 1)
        finite_kernel<uint16_t><<<(unsigned)blocks, 256, 0, st>>>((const uint16_t*)p, n, flag);
    else
        finite_kernel<float><<<(unsigned)blocks, 256, 0, st>>>((const float*)p, n, flag);
    return hipGetLastError();
}

hipError_t pool_write_slot(int dtype, void* A_pool, void* B_pool, int32_t* rank, float* scale, int slot, const void* A,
                           const void* B, int r, float sc, int r_max, int d_in, int d_out, hipStream_t st) {
    const int64_t n = (int64_t)r_max * d_in + (int64_t)d_out * r_max;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (dtype == 1)
        write_slot_kernel<uint16_t><<<(unsigned)blocks, 256, 0, st>>>((uint16_t*)A_pool, (uint16_t*)B_pool, rank,
                                                                      scale, slot, (const uint16_t*)A,
                                                                      (const uint16_t*)B, r, sc, r_max, d_in, d_out);
    else
        write_slot_kernel<float><<<(unsigned)blocks, 256, 0, st>>>((float*)A_pool, (float*)B_pool, rank, scale, slot,
                                                                   (const float*)A, (const float*)B, r, sc, r_max,
                                                                   d_in, d_out);
    return hipGetLastError();
}

}  // namespace lora
