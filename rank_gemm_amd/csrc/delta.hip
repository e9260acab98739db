// The correction alone, y += delta(x), for callers that compute the base
// product themselves: the LoraLayerDelta contract of
// "mstar.engine.resources.lora.pool" (mstar.stanford.edu), where the layer
// output receives a per-row delta and rows on slot 0 are left as they are.
//   y[t][n] = round(y[t][n] + scale_s * sum_q h[t][q] B_s[n][q]),
//   h[t][q] = sum_k x[t][k] A_s[q][k],   q < r_s, s = slot of token t
// Two forms, set against each other in "LoRA serving, embeddings, rerankers,
// pooling" (mlinterviewnotes.com), section "SGLang: chunked SGMV, and a
// rank-aware kernel", and in "43. Beyond text: ...", section "Many adapters,
// one base-model batch":
//  * SGMV over a chunked plan: the tokens grouped by slot and cut into items
//    of at most `chunk` rows (16, 32, 64 or 128). A work item reads A_s and
//    B_s once for all its rows; smaller chunks give more, shorter items, so a
//    popular adapter's segment spreads over more workgroups.
//  * BGMV, token by token from the raw slot map, with no plan: every token
//    reads its own slot's A_s and B_s.
// Both are two kernels: a shrink into fp32 planes (K split across
// workgroups when there are few of them), then an expand that adds the planes
// in split order and updates y in place with one rounding per element. The
// chunk sets how many rows one workgroup of either SGMV kernel takes.
#include "common.h"
#include "kernels.h"
#include "shrink.h"

namespace lora {

// ---------------------------------------------------------------- SGMV shrink --
// grid (n_items, hs), 64 WAVES threads: the workgroup takes its item's 16-row
// blocks in turn; for each, its waves split K range kz and add their partial
// sums in wave order through LDS (shrink_item), into plane kz:
//   part[kz][p][q] = sum_{k in range} x[t_p, k] A_s[q, k],   q < r_s
// A_s is read from memory once per item; the item's later blocks find it in
// the caches.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void delta_shrink_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ A_pool,
                                                                  const int32_t* __restrict__ rank,
                                                                  const int32_t* __restrict__ token_order,
                                                                  const Item* __restrict__ work,
                                                                  float* __restrict__ part, int T, int hkc, int K,
                                                                  int r_max) {
    __shared__ f32x4 red[WAVES * 4 * 64];
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int kz = blockIdx.y;
    const int kbeg = kz * hkc, kend = min(K, kbeg + hkc);
    const ShrinkOut out{part + (int64_t)kz * T * r_max, nullptr, 0, 0.f};
    for (int b0 = 0; b0 < it.count; b0 += 16) {
        const Item sub{it.slot, it.begin + b0, min(16, it.count - b0), 0};
        shrink_item<WAVES>(X, A_pool, r, token_order, sub, out, K, kbeg, kend, r_max, red);
    }
}

// ---------------------------------------------------------------- expand --------
// Rows of h staged in LDS per batch: at most kDeltaLds floats.
constexpr int kDeltaLds = 8192;
constexpr int kDeltaRegRanks = 64;  // ranks whose B values a thread keeps in registers

// y[t][n] += scale * sum_q h[q] * b(q) for one row, b from registers when the
// rank fits, else from memory.
__device__ __forceinline__ float delta_dot(const float* __restrict__ hrow, const float* b,
                                           const uint16_t* __restrict__ bp, int r) {
    float e = 0.f;
    if (r <= kDeltaRegRanks) {
#pragma unroll
        for (int q = 0; q < kDeltaRegRanks; ++q)
            if (q < r) e = __builtin_fmaf(hrow[q], b[q], e);
    } else {
        for (int q = 0; q < r; ++q) e = __builtin_fmaf(hrow[q], bf16_to_f32(bp[q]), e);
    }
    return e;
}

// SGMV expand: grid (n_items, ceil(N / 64)), 256 threads; thread (g, c) =
// (tid / 64, tid % 64) owns column n0 + c and rows g, g + 4, ... of the item.
// B_s[n][0..r) is read once per item and thread, the item's h rows (planes
// added in kz order) are staged in LDS in batches, and the rows of y are
// updated in groups of 8: their loads are issued before any store, so they
// are in flight together.
__global__ __launch_bounds__(256) void delta_expand_kernel(const float* __restrict__ part, int hs,
                                                           const uint16_t* __restrict__ B_pool,
                                                           const int32_t* __restrict__ rank,
                                                           const float* __restrict__ scale,
                                                           const int32_t* __restrict__ token_order,
                                                           const Item* __restrict__ work, uint16_t* __restrict__ Y,
                                                           int T, int N, int r_max) {
    __shared__ float hl[kDeltaLds];
    __shared__ int tok[kDeltaLds / 16];
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const float sc = scale[it.slot];
    const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int n = blockIdx.y * 64 + c;
    const bool nok = n < N;
    const uint16_t* bp = B_pool + ((int64_t)it.slot * N + (nok ? n : 0)) * r_max;
    float b[kDeltaRegRanks];
    if (r <= kDeltaRegRanks) {
#pragma unroll
        for (int q = 0; q < kDeltaRegRanks; ++q) b[q] = q < r ? bf16_to_f32(bp[q < r ? q : 0]) : 0.f;
    }
    const int batch = min(kDeltaLds / 16, max(1, kDeltaLds / r));
    constexpr int U = 8;
    for (int m0 = 0; m0 < it.count; m0 += batch) {
        const int mb = min(batch, it.count - m0);
        __syncthreads();
        for (int i = threadIdx.x; i < mb * r; i += 256) {
            const int m = i / r, q = i - m * r;
            const int64_t row = it.begin + m0 + m;
            float v = 0.f;
            for (int kz = 0; kz < hs; ++kz) v += part[((int64_t)kz * T + row) * r_max + q];
            hl[i] = v;
        }
        for (int i = threadIdx.x; i < mb; i += 256) tok[i] = token_order[it.begin + m0 + i];
        __syncthreads();
        if (!nok) continue;
        for (int mg = g; mg < mb; mg += 4 * U) {
            uint16_t yv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int m = mg + 4 * u;
                yv[u] = m < mb ? Y[(int64_t)tok[m] * N + n] : uint16_t(0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int m = mg + 4 * u;
                if (m >= mb) continue;
                const float e = delta_dot(hl + m * r, b, bp, r);
                Y[(int64_t)tok[m] * N + n] = f32_to_bf16(__builtin_fmaf(sc, e, bf16_to_f32(yv[u])));
            }
        }
    }
}

// BGMV expand: grid (T, ceil(N / 256)), 256 threads; token t's h (planes of
// bgmv_shrink_kernel added in kz order) in LDS, its slot's B_s read for it
// alone; ids outside [1, S) and rank-0 slots leave the row unchanged.
__global__ __launch_bounds__(256) void bgmv_expand_kernel(const float* __restrict__ part, int hs,
                                                          const uint16_t* __restrict__ B_pool,
                                                          const int32_t* __restrict__ rank,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ slot_ids, int S,
                                                          uint16_t* __restrict__ Y, int T, int N, int r_max) {
    __shared__ float hl[kMaxRank];
    const int t = blockIdx.x;
    const int s = slot_ids[t];
    const int r = (s <= 0 || s >= S) ? 0 : rank[s];
    if (r == 0) return;
    for (int q = threadIdx.x; q < r; q += 256) {
        float v = 0.f;
        for (int kz = 0; kz < hs; ++kz) v += part[((int64_t)kz * T + t) * r_max + q];
        hl[q] = v;
    }
    __syncthreads();
    const int n = blockIdx.y * 256 + threadIdx.x;
    if (n >= N) return;
    const uint16_t* bp = B_pool + ((int64_t)s * N + n) * r_max;
    float e = 0.f;
    for (int q = 0; q < r; ++q) e = __builtin_fmaf(hl[q], bf16_to_f32(bp[q]), e);
    uint16_t* yp = Y + (int64_t)t * N + n;
    *yp = f32_to_bf16(__builtin_fmaf(scale[s], e, bf16_to_f32(*yp)));
}

hipError_t delta_sgmv(const uint16_t* X, const uint16_t* A_pool, const uint16_t* B_pool, const int32_t* rank,
                      const float* scale, const int32_t* token_order, const int32_t* work, int n_items, int chunk,
                      int hs, int hkc, float* part, uint16_t* Y, int T, int N, int K, int r_max, hipStream_t st,
                      StageTimer* tm) {
    if (n_items == 0) return hipSuccess;
    // few workgroups: 16 waves per item over the K range, else 4
    hipError_t e = n_items * hs >= 256
                       ? launch(tm, "delta_shrink", delta_shrink_kernel<4>, dim3(n_items, hs), dim3(256), st, X,
                                A_pool, rank, token_order, (const Item*)work, part, T, hkc, K, r_max)
                       : launch(tm, "delta_shrink", delta_shrink_kernel<16>, dim3(n_items, hs), dim3(1024), st, X,
                                A_pool, rank, token_order, (const Item*)work, part, T, hkc, K, r_max);
    if (e != hipSuccess) return e;
    return launch(tm, "delta_expand", delta_expand_kernel, dim3(n_items, (N + 63) / 64), dim3(256), st,
                  (const float*)part, hs, B_pool, rank, scale, token_order, (const Item*)work, Y, T, N, r_max);
}

hipError_t delta_bgmv(const uint16_t* X, const uint16_t* A_pool, const uint16_t* B_pool, const int32_t* rank,
                      const float* scale, const int32_t* slot_ids, int S, int hs, int hkc, float* part, uint16_t* Y,
                      int T, int N, int K, int r_max, hipStream_t st, StageTimer* tm) {
    if (T == 0) return hipSuccess;
    hipError_t e = bgmv_shrink_planes(X, A_pool, rank, slot_ids, S, T, hs, hkc, part, K, r_max, st, tm);
    if (e != hipSuccess) return e;
    return launch(tm, "bgmv_expand", bgmv_expand_kernel, dim3(T, (N + 255) / 256), dim3(256), st, (const float*)part,
                  hs, B_pool, rank, scale, slot_ids, S, Y, T, N, r_max);
}

}  // namespace lora
