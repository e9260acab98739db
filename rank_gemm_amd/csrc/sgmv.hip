// Segmented gather shrink / expand (SGMV) of the LoRA correction on gfx950.
//
// The plan groups tokens by slot ("LoRA serving, embeddings, rerankers,
// pooling", mlinterviewnotes.com, section "vLLM: preallocated stacked
// buffers ...": sorted token indices and per-slot start offsets); its work
// list cuts every non-zero segment into items of at most 16 rows, one
// matrix-core tile. Each item gathers its rows of x through token_order and
// multiplies them by its own slot's factors:
//   shrink: part[z][p][q] = sum_{k in split z} x[t_p, k] * A_s[q, k]    (fp32)
//   expand: y[t_p, j]    += scale_s * sum_q h[p][q] * B_s[j, q],
//           h[p][q]       = sum_z part[z][p][q]   (split order, fp32)
// Rank masking ("SGLang: chunked SGMV, and a rank-aware kernel"): rows q >=
// r_s of A and columns q >= r_s of B are never loaded, and a rank-0 slot's
// items exit at once.
#include "common.h"
#include "kernels.h"

namespace lora {

struct Item {
    int slot, begin, count, pad;
};

// ---------------------------------------------------------------- shrink --
// grid (n_items, ks), one wave per block: the item's <= 16 rows x up to 64
// ranks over one K split. Lane l carries row l % 16 and k-group l / 16.
__global__ __launch_bounds__(64) void shrink_bf16_kernel(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ A_pool,
                                                         const int32_t* __restrict__ rank,
                                                         const int32_t* __restrict__ token_order,
                                                         const Item* __restrict__ work, float* __restrict__ part,
                                                         int T, int K, int r_max, int k_chunk) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int lane = threadIdx.x, row = lane & 15, kg = lane >> 4;
    const bool valid = row < it.count;
    const int t = token_order[it.begin + (valid ? row : 0)];
    const uint16_t* xp = X + (int64_t)t * K;
    const uint16_t* ap = A_pool + (int64_t)it.slot * r_max * K;
    const int kz = blockIdx.y;
    const int kbeg = kz * k_chunk, kend = min(K, kbeg + k_chunk);
    const int nq = (r + 15) >> 4;

    float* pp = part + (int64_t)kz * T * r_max;
    for (int g0 = 0; g0 < nq; g0 += 4) {  // groups of 64 ranks
        f32x4 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k = kbeg; k < kend; k += 32) {
            const int kk = k + kg * 8;
            const bool kin = kk < kend;
            const u32x4 a = (valid && kin) ? *(const u32x4*)(xp + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                if (g0 + qb < nq) {
                    const int q = (g0 + qb) * 16 + row;
                    const u32x4 b =
                        (kin && q < r) ? *(const u32x4*)(ap + (int64_t)q * K + kk) : u32x4{0, 0, 0, 0};
                    acc[qb] = mfma16x16x32(a, b, acc[qb]);
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
            if (g0 + qb < nq) {
                const int q = (g0 + qb) * 16 + row;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = kg * 4 + e;
                    if (m < it.count && q < r_max) pp[(int64_t)(it.begin + m) * r_max + q] = acc[qb][e];
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void shrink_f32_kernel(const float* __restrict__ X, const float* __restrict__ A_pool,
                                                         const int32_t* __restrict__ rank,
                                                         const int32_t* __restrict__ token_order,
                                                         const Item* __restrict__ work, float* __restrict__ part,
                                                         int T, int K, int r_max, int k_chunk) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int m = threadIdx.x >> 4;
    if (m >= it.count) return;
    const int t = token_order[it.begin + m];
    const int kz = blockIdx.y;
    const int kbeg = kz * k_chunk, kend = min(K, kbeg + k_chunk);
    const float* xp = X + (int64_t)t * K;
    float* pp = part + (int64_t)kz * T * r_max + (int64_t)(it.begin + m) * r_max;
    for (int q = threadIdx.x & 15; q < r_max; q += 16) {
        float s = 0.f;
        if (q < r) {
            const float* ap = A_pool + ((int64_t)it.slot * r_max + q) * K;
            for (int k = kbeg; k < kend; ++k) s += xp[k] * ap[k];
        }
        pp[q] = s;
    }
}

// h[p][q] of an item row: its split partials summed in split order.
__device__ __forceinline__ float gather_h(const float* __restrict__ part, int ks, int64_t plane, int64_t off) {
    float s = 0.f;
    for (int z = 0; z < ks; ++z) s += part[z * plane + off];
    return s;
}

// ---------------------------------------------------------------- expand --
// grid (n_items, ceil(N / 256)), 4 waves per block, 64 output columns per
// wave. The product is taken transposed, D[j][t] = sum_q B_s[j][q] h[t][q],
// so each lane ends with 4 consecutive columns of one token row. h is fed
// to the bf16 matrix cores as hi + lo halves (scale folded in first), which
// keeps the fp32 intermediate's precision.
template <bool VEC>
__global__ __launch_bounds__(256) void expand_bf16_kernel(const float* __restrict__ part, int ks,
                                                          const uint16_t* __restrict__ B_pool,
                                                          const int32_t* __restrict__ rank,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ token_order,
                                                          const Item* __restrict__ work, uint16_t* __restrict__ Y,
                                                          int T, int N, int r_max) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const float sc = scale[it.slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j0 = blockIdx.y * 256 + wave * 64;
    if (j0 >= N) return;
    const int trow = lane & 15, qg = lane >> 4;
    const bool valid = trow < it.count;
    const int nq = (r + 15) >> 4;
    const int64_t plane = (int64_t)T * r_max;
    const int64_t hoff = (int64_t)(it.begin + trow) * r_max;

    const uint16_t* bp = B_pool + (int64_t)it.slot * N * r_max;
    const int t = token_order[it.begin + (valid ? trow : 0)];
    uint16_t* yrow = Y + (int64_t)t * N;
    f32x4 acc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < nq; g0 += 4) {  // groups of 64 ranks
        u32x2 hhi[4], hlo[4];
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
            float hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = (g0 + qs) * 16 + qg * 4 + e;
                const float v = (valid && q < r) ? gather_h(part, ks, plane, hoff + q) * sc : 0.f;
                hi[e] = bf16_to_f32(f32_to_bf16(v));
                lo[e] = v - hi[e];
            }
            hhi[qs] = u32x2{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
            hlo[qs] = u32x2{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
        }
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const int j = j0 + jb * 16 + (lane & 15);
#pragma unroll
            for (int qs = 0; qs < 4; ++qs) {
                if (g0 + qs < nq) {
                    const int q = (g0 + qs) * 16 + qg * 4;
                    u32x2 b = u32x2{0, 0};
                    if (j < N) {
                        const uint16_t* src = bp + (int64_t)j * r_max + q;
                        if (VEC) {
                            if (q < r) b = *(const u32x2*)src;  // r_max % 4 == 0; B is zero past r
                        } else {
                            uint16_t e4[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) e4[e] = (q + e < r) ? src[e] : uint16_t(0);
                            b = u32x2{uint32_t(e4[0]) | (uint32_t(e4[1]) << 16),
                                      uint32_t(e4[2]) | (uint32_t(e4[3]) << 16)};
                        }
                    }
                    acc[jb] = mfma16x16x16(b, hhi[qs], acc[jb]);
                    acc[jb] = mfma16x16x16(b, hlo[qs], acc[jb]);
                }
            }
        }
    }
    if (valid) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = j0 + jb * 16 + qg * 4 + e;
                if (jj < N) yrow[jj] = f32_to_bf16(bf16_to_f32(yrow[jj]) + acc[jb][e]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void expand_f32_kernel(const float* __restrict__ part, int ks,
                                                         const float* __restrict__ B_pool,
                                                         const int32_t* __restrict__ rank,
                                                         const float* __restrict__ scale,
                                                         const int32_t* __restrict__ token_order,
                                                         const Item* __restrict__ work, float* __restrict__ Y, int T,
                                                         int N, int r_max) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int j = blockIdx.y * 256 + threadIdx.x;
    if (j >= N) return;
    const float sc = scale[it.slot];
    const int64_t plane = (int64_t)T * r_max;
    const float* bp = B_pool + ((int64_t)it.slot * N + j) * r_max;
    for (int m = 0; m < it.count; ++m) {
        const int64_t hoff = (int64_t)(it.begin + m) * r_max;
        float e = 0.f;
        for (int q = 0; q < r; ++q) e += bp[q] * (gather_h(part, ks, plane, hoff + q) * sc);
        float* yp = Y + (int64_t)token_order[it.begin + m] * N + j;
        *yp = *yp + e;
    }
}

// h[t][q] for every token (zeros for slot 0, rank-0 slots and q >= r_s).
__global__ __launch_bounds__(256) void shrink_to_h_kernel(const float* __restrict__ part, int ks,
                                                          const int32_t* __restrict__ rank,
                                                          const int32_t* __restrict__ token_order,
                                                          const int32_t* __restrict__ slot_indptr, int S,
                                                          float* __restrict__ h, int T, int r_max) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * r_max) return;
    const int p = (int)(idx / r_max), q = (int)(idx % r_max);
    int lo = 0, hi = S - 1;  // last slot s with slot_indptr[s] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_indptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int s = lo, r = rank[s];
    float v = 0.f;
    if (s != 0 && q < r) v = gather_h(part, ks, (int64_t)T * r_max, (int64_t)p * r_max + q);
    h[(int64_t)token_order[p] * r_max + q] = v;
}

int shrink_splits(int n_items, int K) {
    // aim for ~2048 waves in flight; each split spans >= 128 of K
    int ks = n_items > 0 ? (2048 + n_items - 1) / n_items : 1;
    const int max_ks = K / 128 > 0 ? K / 128 : 1;
    if (ks > max_ks) ks = max_ks;
    if (ks > kMaxShrinkSplits) ks = kMaxShrinkSplits;
    return ks < 1 ? 1 : ks;
}

static int chunk_for(int K, int ks) {
    int c = (K + ks - 1) / ks;
    return (c + 31) / 32 * 32;
}

hipError_t sgmv_shrink(int dtype, const void* X, const void* A_pool, const int32_t* rank, const int32_t* token_order,
                       const int32_t* work, int n_items, float* part, int ks, int T, int K, int r_max,
                       hipStream_t st, StageTimer* tm) {
    if (n_items == 0) return hipSuccess;
    dim3 grid(n_items, ks);
    TimedScope ts(tm, "sgmv_shrink", st);
    const int kc = chunk_for(K, ks);
    if (dtype == 1)
        shrink_bf16_kernel<<<grid, 64, 0, st>>>((const uint16_t*)X, (const uint16_t*)A_pool, rank, token_order,
                                                (const Item*)work, part, T, K, r_max, kc);
    else
        shrink_f32_kernel<<<grid, 256, 0, st>>>((const float*)X, (const float*)A_pool, rank, token_order,
                                                (const Item*)work, part, T, K, r_max, kc);
    return hipGetLastError();
}

hipError_t sgmv_expand(int dtype, const float* part, int ks, const void* B_pool, const int32_t* rank,
                       const float* scale, const int32_t* token_order, const int32_t* work, int n_items, void* Y,
                       int T, int N, int r_max, hipStream_t st, StageTimer* tm) {
    if (n_items == 0) return hipSuccess;
    dim3 grid(n_items, (N + 255) / 256);
    TimedScope ts(tm, "sgmv_expand", st);
    if (dtype == 1) {
        if (r_max % 4 == 0)
            expand_bf16_kernel<true><<<grid, 256, 0, st>>>(part, ks, (const uint16_t*)B_pool, rank, scale, token_order,
                                                           (const Item*)work, (uint16_t*)Y, T, N, r_max);
        else
            expand_bf16_kernel<false><<<grid, 256, 0, st>>>(part, ks, (const uint16_t*)B_pool, rank, scale,
                                                            token_order, (const Item*)work, (uint16_t*)Y, T, N, r_max);
    } else {
        expand_f32_kernel<<<grid, 256, 0, st>>>(part, ks, (const float*)B_pool, rank, scale, token_order,
                                                (const Item*)work, (float*)Y, T, N, r_max);
    }
    return hipGetLastError();
}

hipError_t shrink_to_h(const float* part, int ks, const int32_t* rank, const int32_t* token_order,
                       const int32_t* slot_indptr, int S, float* h, int T, int r_max, hipStream_t st,
                       StageTimer* tm) {
    const int64_t n = (int64_t)T * r_max;
    if (n == 0) return hipSuccess;
    TimedScope ts(tm, "shrink_to_h", st);
    shrink_to_h_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, ks, rank, token_order, slot_indptr, S, h, T,
                                                                     r_max);
    return hipGetLastError();
}

}  // namespace lora
