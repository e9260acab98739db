// Element-generic path of the layer: fp32 pools (true fp32 FMA, no
// reduced-precision splitting) and bf16 pools whose d_in is not a multiple of
// 8, where rows of x, W and A_s do not start on 16-byte boundaries and the
// vector kernels' 16-byte loads do not apply. Every load here is a scalar
// load, so any width works and K tails are masked element by element, with
// fp32 accumulation, as the kernels of "43. Beyond text: images, embeddings,
// reranking and many LoRAs", section "Many adapters, one base-model batch",
// also do.
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

// Loads of one K stage are issued together and kept in registers while the
// previous stage is multiplied out of LDS, so a call costs about one memory
// round trip per stage. Every address is clamped into the operands (rows past
// the tile's end read row 0 of the tile, k past K reads k = 0) and the
// k-tail values are zeroed afterwards, so no load sits under a branch.
constexpr int kGenKs = 64;  // k per stage

// grid n_items, 256 threads. Per 16-row block of the item and 16-rank block
// (r_s masked): thread (i, q) = (tid / 16, tid % 16) owns h[row i][rank q],
// summed over k in order; X rows (through token_order) and A_s rows are staged
// through LDS kGenKs columns at a time.
template <typename E>
__global__ __launch_bounds__(256) void shrink_generic_kernel(const E* __restrict__ X, const E* __restrict__ A_pool,
                                                             const int32_t* __restrict__ rank,
                                                             const int32_t* __restrict__ token_order,
                                                             const Item* __restrict__ work, float* __restrict__ h,
                                                             int K, int r_max) {
    __shared__ float Xs[16][kGenKs + 1];
    __shared__ float As[16][kGenKs + 1];
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int tid = threadIdx.x, c = tid & 63, lr = tid >> 6;  // loader: column c, rows lr + 4 j
    const int oi = tid >> 4, oq = tid & 15;                     // owner: row oi, rank oq
    for (int b0 = 0; b0 < it.count; b0 += 16) {
        int64_t xrow[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = b0 + lr + 4 * j;
            xrow[j] = (int64_t)token_order[it.begin + (m < it.count ? m : b0)] * K;
        }
        for (int q0 = 0; q0 < r; q0 += 16) {
            int64_t arow[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = q0 + lr + 4 * j;
                arow[j] = ((int64_t)it.slot * r_max + (q < r ? q : 0)) * K;
            }
            float vx[4], va[4];
            auto fetch = [&](int k0) {
                const int k = k0 + c;
                const int kc = k < K ? k : 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vx[j] = ld_elem(X, xrow[j] + kc);
                    va[j] = ld_elem(A_pool, arow[j] + kc);
                }
                if (k >= K) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) vx[j] = va[j] = 0.f;
                }
            };
            fetch(0);
            float acc = 0.f;
            for (int k0 = 0; k0 < K; k0 += kGenKs) {
                __syncthreads();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Xs[lr + 4 * j][c] = vx[j];
                    As[lr + 4 * j][c] = va[j];
                }
                __syncthreads();
                if (k0 + kGenKs < K) fetch(k0 + kGenKs);
#pragma unroll 16
                for (int cc = 0; cc < kGenKs; ++cc) acc = __builtin_fmaf(Xs[oi][cc], As[oq][cc], acc);
            }
            const int m = b0 + oi, q = q0 + oq;
            if (m < it.count && q < r) h[(int64_t)(it.begin + m) * r_max + q] = acc;
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

typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int R>
struct FragOf;
template <>
struct FragOf<4> {
    using type = f32x4;
};
template <>
struct FragOf<2> {
    using type = f32x2;
};

// grid (ceil(M / TM), ceil(N / TM)), 256 threads; thread (ty, tx) owns rows
// m0 + R ty .. + R - 1 and columns n0 + R tx .. + R - 1 of the tile
// (R = TM / 16), summed over k in order; x rows (through token_order) and W
// rows are staged through LDS kGenKs columns at a time. Rows are sorted
// positions: x row and y row token_order[p]. Rows past M and columns past N
// read row m0 / row n0 and are not stored; they touch no other output.
// TM = 32 gives four times the workgroups of TM = 64 for grids that would
// leave most of the chip idle.
template <typename E, int TM>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const E* __restrict__ X, const E* __restrict__ W,
                                                           E* __restrict__ Y, const int32_t* __restrict__ token_order,
                                                           const int32_t* __restrict__ slot_indptr, int S,
                                                           const int32_t* __restrict__ rank,
                                                           const float* __restrict__ scale,
                                                           const float* __restrict__ h,
                                                           const E* __restrict__ B_pool, int adapters, int M, int N,
                                                           int K, int r_max) {
    constexpr int R = TM / 16;              // outputs per thread along each side
    constexpr int PER = TM * kGenKs / 256;  // elements of each operand per thread and stage
    using Frag = typename FragOf<R>::type;
    // rows of TM + 4 floats: a thread's R consecutive values are one aligned read
    __shared__ __align__(16) float As[kGenKs][TM + 4];
    __shared__ __align__(16) float Bs[kGenKs][TM + 4];
    __shared__ int tok[TM], slot_row[TM], rank_row[TM];
    __shared__ float scale_row[TM];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int c = tid & 63, lr = tid >> 6;  // loader: column c, tile rows lr + 4 j
    const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TM;
    if (tid < TM) tok[tid] = token_order[m0 + tid < M ? m0 + tid : m0];
    __syncthreads();
    int64_t xrow[PER], wrow[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int rr = lr + 4 * j;
        xrow[j] = (int64_t)tok[rr] * K;
        wrow[j] = (int64_t)(n0 + rr < N ? n0 + rr : n0) * K;
    }
    float va[PER], vb[PER];
    auto fetch = [&](int k0) {
        const int k = k0 + c;
        const int kc = k < K ? k : 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            va[j] = ld_elem(X, xrow[j] + kc);
            vb[j] = ld_elem(W, wrow[j] + kc);
        }
        if (k >= K) {
#pragma unroll
            for (int j = 0; j < PER; ++j) va[j] = vb[j] = 0.f;
        }
    };
    fetch(0);
    // slot, rank and scale of each tile row, found while the first stage loads
    if (tid < TM) {
        const int p = m0 + tid;
        int sl = 0, rk = 0;
        if (adapters && p < M) {
            sl = slot_of(slot_indptr, S, p);
            rk = sl != 0 ? rank[sl] : 0;
        }
        slot_row[tid] = sl;
        rank_row[tid] = rk;
        scale_row[tid] = rk > 0 ? scale[sl] : 0.f;
    }
    float acc[R][R] = {};
    for (int k0 = 0; k0 < K; k0 += kGenKs) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            As[c][lr + 4 * j] = va[j];
            Bs[c][lr + 4 * j] = vb[j];
        }
        __syncthreads();
        if (k0 + kGenKs < K) fetch(k0 + kGenKs);
        // 4 k at a time; the next 4 k's reads are issued before this block's
        // products, so LDS latency hides behind them
        Frag a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = *reinterpret_cast<const Frag*>(&As[u][ty * R]);
            b[u] = *reinterpret_cast<const Frag*>(&Bs[u][tx * R]);
        }
#pragma unroll
        for (int cc = 0; cc < kGenKs; cc += 4) {
            Frag an[4], bn[4];
            if (cc + 4 < kGenKs) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    an[u] = *reinterpret_cast<const Frag*>(&As[cc + 4 + u][ty * R]);
                    bn[u] = *reinterpret_cast<const Frag*>(&Bs[cc + 4 + u][tx * R]);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < R; ++i)
#pragma unroll
                    for (int j = 0; j < R; ++j) acc[i][j] = __builtin_fmaf(a[u][i], b[u][j], acc[i][j]);
            if (cc + 4 < kGenKs) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a[u] = an[u];
                    b[u] = bn[u];
                }
            }
        }
    }
    // Epilogue: the expand of the thread's R rows over their slots' ranks in
    // batches of 4, each batch's h and B loads (all R rows) issued together.
    int rs[R], rmax = 0;
    const float* hp[R];
    const E* bp[R][R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = ty * R + i;
        rs[i] = rank_row[row];
        rmax = max(rmax, rs[i]);
        hp[i] = h + (int64_t)(m0 + row) * r_max;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int n = n0 + tx * R + j;
            bp[i][j] = B_pool + ((int64_t)slot_row[row] * N + (n < N ? n : n0)) * r_max;
        }
    }
    float e[R][R] = {};
    for (int q0 = 0; q0 < rmax; q0 += 4) {
        float hv[R][4], bv[R][R][4];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = q0 + u < rs[i] ? q0 + u : 0;
                hv[i][u] = rs[i] > 0 ? hp[i][q] : 0.f;
#pragma unroll
                for (int j = 0; j < R; ++j) bv[i][j][u] = rs[i] > 0 ? ld_elem(bp[i][j], q) : 0.f;
            }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (q0 + u < rs[i]) {
#pragma unroll
                    for (int j = 0; j < R; ++j) e[i][j] = __builtin_fmaf(bv[i][j][u], hv[i][u], e[i][j]);
                }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = ty * R + i;
        if (m0 + row >= M) continue;
        const float sc = scale_row[row];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int n = n0 + tx * R + j;
            if (n >= N) continue;
            const float v = rs[i] > 0 ? __builtin_fmaf(sc, e[i][j], acc[i][j]) : acc[i][j];
            Y[(int64_t)tok[row] * N + n] = st_elem<E>(v);
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
    // 64 x 64 tiles when they make enough workgroups to fill the chip, else 32 x 32
    const bool big = (int64_t)((M + 63) / 64) * ((N + 63) / 64) >= 256;
    const int tile = big ? 64 : 32;
    const dim3 grid((M + tile - 1) / tile, (N + tile - 1) / tile);
    auto go = [&](auto kern, auto elem) {
        using T = decltype(elem);
        return launch(tm, "gemm_generic", kern, grid, dim3(256), st, (const T*)X, (const T*)W, (T*)Y, token_order,
                      slot_indptr, S, rank, scale, (const float*)h, (const T*)B_pool, adapters, M, N, K, r_max);
    };
    if (dtype == 1)
        return big ? go(gemm_generic_kernel<uint16_t, 64>, uint16_t{}) : go(gemm_generic_kernel<uint16_t, 32>, uint16_t{});
    return big ? go(gemm_generic_kernel<float, 64>, float{}) : go(gemm_generic_kernel<float, 32>, float{});
}

}  // namespace lora
