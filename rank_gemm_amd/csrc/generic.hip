// Element-generic path of the layer: fp32 pools (true fp32 FMA, no
// reduced-precision splitting) and bf16 pools whose d_in is not a multiple of
// 8, where rows of x, W and A_s do not start on 16-byte boundaries and the
// vector kernels' 16-byte loads do not apply. Every load here is a scalar
// load, so any width works and K tails are masked element by element (the
// page's kernels "accumulate in FP32, mask odd widths": "43. Beyond text:
// images, embeddings, reranking and many LoRAs", section "Many adapters, one
// base-model batch").
//
// Two kernels:
//  1. shrink_generic_kernel: per work item (<= 16 rows of one slot's
//     segment), h[p][q] = sum_k x[t_p, k] A_s[q, k] in fp32, q < r_s.
//  2. gemm_generic_kernel: 64 x 64 tiles over (sorted positions, columns),
//     acc = sum_k x[t_p, k] W[n, k] in fp32, then the expand fused into the
//     epilogue: y[t_p][n] = acc + scale_s * sum_q h[p][q] B_s[n][q], rounded
//     once to the element type. The k order of acc does not depend on the
//     plan, so rows on slot 0 equal a base-only call bit for bit.
#include "common.h"
#include "kernels.h"
#include "shrink.h"

namespace lora {

template <typename E>
__device__ __forceinline__ float ld_elem(const E* p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, int64_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

template <typename E>
__device__ __forceinline__ E st_elem(float v);
template <>
__device__ __forceinline__ float st_elem<float>(float v) {
    return v;
}
template <>
__device__ __forceinline__ uint16_t st_elem<uint16_t>(float v) {
    return f32_to_bf16(v);
}

// grid n_items, 256 threads: thread (m0 = tid / 16, q0 = tid % 16) computes
// rows m0, m0 + 16, ... of the item and ranks q0, q0 + 16, ... below r_s.
template <typename E>
__global__ __launch_bounds__(256) void shrink_generic_kernel(const E* __restrict__ X, const E* __restrict__ A_pool,
                                                             const int32_t* __restrict__ rank,
                                                             const int32_t* __restrict__ token_order,
                                                             const Item* __restrict__ work, float* __restrict__ h,
                                                             int K, int r_max) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    for (int m = threadIdx.x >> 4; m < it.count; m += 16) {
        const int64_t xrow = (int64_t)token_order[it.begin + m] * K;
        float* hp = h + (int64_t)(it.begin + m) * r_max;
        for (int q = threadIdx.x & 15; q < r; q += 16) {
            const int64_t arow = ((int64_t)it.slot * r_max + q) * K;
            float s = 0.f;
            for (int k = 0; k < K; ++k) s = __builtin_fmaf(ld_elem(X, xrow + k), ld_elem(A_pool, arow + k), s);
            hp[q] = s;
        }
    }
}

// y[t_p][n] = round(y[t_p][n] + scale_s * sum_q h[p][q] B_s[n][q]) in place,
// one thread per output column, the item's rows in turn (items of any row
// count). grid (n_items, ceil(N / 256)).
template <typename E>
__global__ __launch_bounds__(256) void expand_generic_kernel(const float* __restrict__ h, const E* __restrict__ B_pool,
                                                             const int32_t* __restrict__ rank,
                                                             const float* __restrict__ scale,
                                                             const int32_t* __restrict__ token_order,
                                                             const Item* __restrict__ work, E* __restrict__ Y, int N,
                                                             int r_max) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int n = blockIdx.y * 256 + threadIdx.x;
    if (n >= N) return;
    const float sc = scale[it.slot];
    const E* bp = B_pool + ((int64_t)it.slot * N + n) * r_max;
    for (int m = 0; m < it.count; ++m) {
        const float* hp = h + (int64_t)(it.begin + m) * r_max;
        float e = 0.f;
        for (int q = 0; q < r; ++q) e = __builtin_fmaf(ld_elem(bp, q), hp[q], e);
        E* yp = Y + (int64_t)token_order[it.begin + m] * N + n;
        *yp = st_elem<E>(__builtin_fmaf(sc, e, ld_elem(yp, 0)));
    }
}

// Slot of sorted position p: the last s with slot_indptr[s] <= p.
__device__ __forceinline__ int slot_of(const int32_t* __restrict__ slot_indptr, int S, int p) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_indptr[mid] <= p) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// grid (ceil(M / 64), ceil(N / 64)), 256 threads; thread (ty, tx) owns rows
// m0 + 4 ty .. + 3 and columns n0 + 4 tx .. + 3 of the tile, K staged 16 at a
// time through LDS. Rows are sorted positions: x row and y row token_order[p].
template <typename E>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const E* __restrict__ X, const E* __restrict__ W,
                                                           E* __restrict__ Y, const int32_t* __restrict__ token_order,
                                                           const int32_t* __restrict__ slot_indptr, int S,
                                                           const int32_t* __restrict__ rank,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ h,
                                                           const E* __restrict__ B_pool, int adapters, int M, int N,
                                                           int K, int r_max) {
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    __shared__ int tok[64];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
    if (tid < 64) tok[tid] = m0 + tid < M ? token_order[m0 + tid] : 0;
    __syncthreads();
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int i = tid; i < 64 * 16; i += 256) {
            const int r = i >> 4, c = i & 15;
            const int m = m0 + r, n = n0 + r, k = k0 + c;
            As[c][r] = (m < M && k < K) ? ld_elem(X, (int64_t)tok[r] * K + k) : 0.f;
            Bs[c][r] = (n < N && k < K) ? ld_elem(W, (int64_t)n * K + k) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[c][ty * 4 + i];
                b[i] = Bs[c][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = m0 + ty * 4 + i;
        if (p >= M) continue;
        int s = 0, r = 0;
        if (adapters) {
            s = slot_of(slot_indptr, S, p);
            r = s != 0 ? rank[s] : 0;
        }
        const float sc = r > 0 ? scale[s] : 0.f;
        const float* hp = h + (int64_t)p * r_max;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float v = acc[i][j];
            if (r > 0) {
                const E* bp = B_pool + ((int64_t)s * N + n) * r_max;
                float e = 0.f;
                for (int q = 0; q < r; ++q) e = __builtin_fmaf(ld_elem(bp, q), hp[q], e);
                v = __builtin_fmaf(sc, e, v);
            }
            Y[(int64_t)tok[ty * 4 + i] * N + n] = st_elem<E>(v);
        }
    }
}

hipError_t generic_shrink(int dtype, const void* X, const void* A_pool, const int32_t* rank,
                          const int32_t* token_order, const int32_t* work, int n_items, float* h, int K, int r_max,
                          hipStream_t st, StageTimer* tm) {
    if (n_items == 0) return hipSuccess;
    if (dtype == 1)
        return launch(tm, "sgmv_shrink", shrink_generic_kernel<uint16_t>, dim3(n_items), dim3(256), st,
                      (const uint16_t*)X, (const uint16_t*)A_pool, rank, token_order, (const Item*)work, h, K, r_max);
    return launch(tm, "sgmv_shrink", shrink_generic_kernel<float>, dim3(n_items), dim3(256), st, (const float*)X,
                  (const float*)A_pool, rank, token_order, (const Item*)work, h, K, r_max);
}

hipError_t generic_expand(int dtype, const float* h, const void* B_pool, const int32_t* rank, const float* scale,
                          const int32_t* token_order, const int32_t* work, int n_items, void* Y, int N, int r_max,
                          hipStream_t st, StageTimer* tm) {
    if (n_items == 0 || N == 0) return hipSuccess;
    const dim3 grid(n_items, (N + 255) / 256);
    if (dtype == 1)
        return launch(tm, "delta_expand", expand_generic_kernel<uint16_t>, grid, dim3(256), st, h,
                      (const uint16_t*)B_pool, rank, scale, token_order, (const Item*)work, (uint16_t*)Y, N, r_max);
    return launch(tm, "delta_expand", expand_generic_kernel<float>, grid, dim3(256), st, h, (const float*)B_pool, rank,
                  scale, token_order, (const Item*)work, (float*)Y, N, r_max);
}

hipError_t generic_linear(int dtype, const void* X, const void* W, void* Y, const int32_t* token_order,
                          const int32_t* slot_indptr, const int32_t* work, int n_items, int S, const void* A_pool,
                          const void* B_pool, const int32_t* rank, const float* scale, float* h, int adapters, int M,
                          int N, int K, int r_max, hipStream_t st, StageTimer* tm) {
    if (M == 0 || N == 0) return hipSuccess;
    if (adapters) {
        const hipError_t e = generic_shrink(dtype, X, A_pool, rank, token_order, work, n_items, h, K, r_max, st, tm);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((M + 63) / 64, (N + 63) / 64);
    if (dtype == 1)
        return launch(tm, "gemm_generic", gemm_generic_kernel<uint16_t>, grid, dim3(256), st, (const uint16_t*)X,
                      (const uint16_t*)W, (uint16_t*)Y, token_order, slot_indptr, S, rank, scale, (const float*)h,
                      (const uint16_t*)B_pool, adapters, M, N, K, r_max);
    return launch(tm, "gemm_generic", gemm_generic_kernel<float>, grid, dim3(256), st, (const float*)X,
                  (const float*)W, (float*)Y, token_order, slot_indptr, S, rank, scale, (const float*)h,
                  (const float*)B_pool, adapters, M, N, K, r_max);
}

}  // namespace lora
