// Segmented gather shrink (SGMV) of the LoRA correction on gfx950 (bf16
// pools with 16-byte aligned rows), its BGMV counterpart and the scatter of h
// to token order.
//
// The plan groups tokens by slot ("LoRA serving, embeddings, rerankers,
// pooling", mlinterviewnotes.com, section "vLLM: preallocated stacked
// buffers ...": token indices sorted by slot plus per-slot start offsets);
// its work list cuts every non-zero segment into items of at most 16 rows,
// one matrix-core tile. Each item gathers its rows of x through token_order
// and multiplies them by its own slot's A:
//   h[p][q] = sum_k x[t_p, k] * A_s[q, k]     (fp32, p = sorted position)
// the narrow T x r intermediate of the same page. The waves of a
// workgroup split K and their partial sums are added in wave order through
// LDS, so h is deterministic. Rank masking ("SGLang: chunked SGMV, and a
// rank-aware kernel"): rows q >= r_s of A are never loaded and a rank-0
// slot's items exit at once.
#include "common.h"
#include "kernels.h"
#include "shrink.h"

namespace lora {

// ---------------------------------------------------------------- shrink --
// grid n_items, WAVES waves per block, the full K range: h is final.
// With ext set, writes the expand operand (scaled, bf16 hi / lo) instead of h.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void shrink_bf16_kernel(const uint16_t* __restrict__ X,
                                                                 const uint16_t* __restrict__ A_pool,
                                                                 const int32_t* __restrict__ rank,
                                                                 const float* __restrict__ scale,
                                                                 const int32_t* __restrict__ token_order,
                                                                 const Item* __restrict__ work,
                                                                 float* __restrict__ h, uint16_t* __restrict__ ext,
                                                                 int K, int r_max) {
    __shared__ f32x4 red[WAVES * 4 * 64];
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const ShrinkOut out{h, ext, (r_max + 7) & ~7, ext ? scale[it.slot] : 0.f};
    shrink_item<WAVES>(X, A_pool, r, token_order, it, out, K, 0, K, r_max, red);
}

// Several slices reading the same x: grid n_items, WAVES waves, the full K
// range, each slice's expand operand written to its own ext.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void shrink_slices_kernel(const uint16_t* __restrict__ X, ShrinkSlices ss,
                                                                   const int32_t* __restrict__ token_order,
                                                                   const Item* __restrict__ work, int K, int r_max) {
    __shared__ f32x4 red[WAVES * 4 * 64];
    const Item it = work[blockIdx.x];
    shrink_item_slices<WAVES>(X, ss, token_order, it, K, r_max, red);
}

// Few items: grid n_items * hs, block b = kz * n_items + item computes its
// item over K range kz (hkc k, 4 waves) into its own 16-row plane of part
// ([n_items * hs][16][r_max] fp32); shrink_finish_kernel adds the planes in
// kz order.
__global__ __launch_bounds__(256) void shrink_split_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ A_pool,
                                                           const int32_t* __restrict__ rank,
                                                           const int32_t* __restrict__ token_order,
                                                           const Item* __restrict__ work, float* __restrict__ part,
                                                           int n_items, int hkc, int K, int r_max) {
    __shared__ f32x4 red[4 * 4 * 64];
    const int item = blockIdx.x % n_items, kz = blockIdx.x / n_items;
    const Item it = work[item];
    const int r = rank[it.slot];
    if (r == 0) return;
    ShrinkOut out{part + (int64_t)blockIdx.x * 16 * r_max, nullptr, 0, 0.f};
    out.row0 = it.begin;
    const int kbeg = kz * hkc, kend = min(K, kbeg + hkc);
    shrink_item<4>(X, A_pool, r, token_order, it, out, K, kbeg, kend, r_max, red);
}

// h (fp32, or with ext the scaled bf16 hi / lo operand) of an item's rows:
// its hs planes added in kz order; ranks past the slot's are zero.
__global__ __launch_bounds__(256) void shrink_finish_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ rank,
                                                            const float* __restrict__ scale,
                                                            const Item* __restrict__ work, float* __restrict__ h,
                                                            uint16_t* __restrict__ ext, int n_items, int hs,
                                                            int r_max) {
    const Item it = work[blockIdx.x];
    const int r = rank[it.slot];
    if (r == 0) return;
    const int rp = (r_max + 7) & ~7;
    const int width = ext ? rp : r_max;
    const float sc = ext ? scale[it.slot] : 0.f;
    for (int i = threadIdx.x; i < 16 * width; i += blockDim.x) {
        const int m = i / width, q = i - m * width;
        if (m >= it.count) continue;
        float v = 0.f;
        if (q < r)
            for (int kz = 0; kz < hs; ++kz) v += part[((int64_t)(kz * n_items + blockIdx.x) * 16 + m) * r_max + q];
        const int64_t p = it.begin + m;
        if (ext) {
            v *= sc;
            const uint16_t hi = f32_to_bf16(v);
            ext[(p * 2) * rp + q] = hi;
            ext[(p * 2 + 1) * rp + q] = f32_to_bf16(v - bf16_to_f32(hi));
        } else {
            h[p * r_max + q] = v;
        }
    }
}

// BGMV shrink: one token at a time, no grouping (the batched gather
// matrix-vector form that "LoRA serving, embeddings, rerankers, pooling"
// contrasts with the segmented SGMV). grid (T, hs): block (t, kz) computes
// x[t] . A_s[q] over K range kz for every q < r_s, s = slot_ids[t]; thread
// (qi = tid / 16, ki = tid % 16) takes rank q0 + qi and every 16th 8-wide k
// chunk, then 16-lane sums. Planes part[kz][t][q] (q < r_s only).
__global__ __launch_bounds__(256) void bgmv_shrink_kernel(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ A_pool,
                                                          const int32_t* __restrict__ rank,
                                                          const int32_t* __restrict__ slot_ids, int S,
                                                          float* __restrict__ part, int T, int hkc, int K,
                                                          int r_max) {
    const int t = blockIdx.x, kz = blockIdx.y;
    const int s = slot_ids[t];
    const int r = (s <= 0 || s >= S) ? 0 : rank[s];
    if (r == 0) return;
    const int qi = threadIdx.x >> 4, ki = threadIdx.x & 15;
    const int kbeg = kz * hkc, kend = min(K, kbeg + hkc);
    const uint16_t* xp = X + (int64_t)t * K;
    for (int q0 = 0; q0 < r; q0 += 16) {
        const int q = q0 + qi;
        const uint16_t* ap = A_pool + ((int64_t)s * r_max + min(q, r - 1)) * K;
        float acc = 0.f;
        for (int k = kbeg + ki * 8; k < kend; k += 128) {
            const u32x4 xv = *as_global<u32x4>(xp + k);
            const u32x4 av = *as_global<u32x4>(ap + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = __builtin_fmaf(__uint_as_float(xv[e] << 16), __uint_as_float(av[e] << 16), acc);
                acc = __builtin_fmaf(__uint_as_float(xv[e] & 0xffff0000u), __uint_as_float(av[e] & 0xffff0000u), acc);
            }
        }
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
        if (ki == 0 && q < r) part[((int64_t)kz * T + t) * r_max + q] = acc;
    }
}

// h[t][q] (token order) = the planes of bgmv_shrink_kernel added in kz order
// for q < r_s; zero past the rank and on slot 0 or a rank-0 slot.
__global__ __launch_bounds__(256) void bgmv_finish_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ rank,
                                                          const int32_t* __restrict__ slot_ids, int S,
                                                          float* __restrict__ h, int T, int hs, int r_max) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * r_max) return;
    const int t = (int)(i / r_max), q = (int)(i - (int64_t)t * r_max);
    const int s = slot_ids[t];
    const int r = (s <= 0 || s >= S) ? 0 : rank[s];
    float v = 0.f;
    if (q < r)
        for (int kz = 0; kz < hs; ++kz) v += part[((int64_t)kz * T + t) * r_max + q];
    h[i] = v;
}

// h_out[t][q] (token order) from h[p][q] (sorted order); zeros for slot 0,
// rank-0 slots and q >= r_s.
__global__ __launch_bounds__(256) void scatter_h_kernel(const float* __restrict__ h, const int32_t* __restrict__ rank,
                                                        const int32_t* __restrict__ token_order,
                                                        const int32_t* __restrict__ slot_indptr, int S,
                                                        float* __restrict__ h_out, int T, int r_max) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * r_max) return;
    const int p = (int)(idx / r_max), q = (int)(idx % r_max);
    int lo = 0, hi = S - 1;  // last slot s with slot_indptr[s] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_indptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const float v = (s != 0 && q < rank[s]) ? h[idx] : 0.f;
    h_out[(int64_t)token_order[p] * r_max + q] = v;
}

hipError_t sgmv_shrink(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const int32_t* token_order,
                       const int32_t* work, int n_items, float* h, int K, int r_max, hipStream_t st,
                       StageTimer* tm, const float* scale, uint16_t* ext) {
    if (n_items == 0) return hipSuccess;
    if (n_items >= 256)
        return launch(tm, "sgmv_shrink", shrink_bf16_kernel<4>, dim3(n_items), dim3(256), st, X, A_pool, rank, scale,
                      token_order, (const Item*)work, h, ext, K, r_max);
    return launch(tm, "sgmv_shrink", shrink_bf16_kernel<16>, dim3(n_items), dim3(1024), st, X, A_pool, rank, scale,
                  token_order, (const Item*)work, h, ext, K, r_max);
}

hipError_t sgmv_shrink_slices(const uint16_t* X, const ShrinkSlices& ss, const int32_t* token_order,
                              const int32_t* work, int n_items, int K, int r_max, hipStream_t st, StageTimer* tm) {
    static_assert(kShrinkMaxSlices == kMaxSlices, "slice tables");
    if (n_items == 0) return hipSuccess;
    if (n_items >= 256)
        return launch(tm, "sgmv_shrink", shrink_slices_kernel<4>, dim3(n_items), dim3(256), st, X, ss, token_order,
                      (const Item*)work, K, r_max);
    return launch(tm, "sgmv_shrink", shrink_slices_kernel<16>, dim3(n_items), dim3(1024), st, X, ss, token_order,
                  (const Item*)work, K, r_max);
}

hipError_t sgmv_shrink_split(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const float* scale,
                             const int32_t* token_order, const int32_t* work, int n_items, int hs, int hkc,
                             float* part, float* h, uint16_t* ext, int K, int r_max, hipStream_t st,
                             StageTimer* tm) {
    if (n_items == 0) return hipSuccess;
    hipError_t e = launch(tm, "sgmv_shrink", shrink_split_kernel, dim3(n_items * hs), dim3(256), st, X, A_pool,
                          rank, token_order, (const Item*)work, part, n_items, hkc, K, r_max);
    if (e != hipSuccess) return e;
    return launch(tm, "sgmv_shrink_finish", shrink_finish_kernel, dim3(n_items), dim3(256), st, (const float*)part,
                  rank, scale, (const Item*)work, h, ext, n_items, hs, r_max);
}

hipError_t bgmv_shrink_planes(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const int32_t* slot_ids,
                              int S, int T, int hs, int hkc, float* part, int K, int r_max, hipStream_t st,
                              StageTimer* tm) {
    if (T == 0) return hipSuccess;
    return launch(tm, "bgmv_shrink", bgmv_shrink_kernel, dim3(T, hs), dim3(256), st, X, A_pool, rank, slot_ids, S,
                  part, T, hkc, K, r_max);
}

hipError_t bgmv_shrink(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const int32_t* slot_ids,
                       int S, int T, int hs, int hkc, float* part, float* h, int K, int r_max, hipStream_t st,
                       StageTimer* tm) {
    if (T == 0) return hipSuccess;
    hipError_t e = bgmv_shrink_planes(X, A_pool, rank, slot_ids, S, T, hs, hkc, part, K, r_max, st, tm);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)T * r_max;
    return launch(tm, "bgmv_finish", bgmv_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st,
                  (const float*)part, rank, slot_ids, S, h, T, hs, r_max);
}

hipError_t scatter_h(const float* h, const int32_t* rank, const int32_t* token_order, const int32_t* slot_indptr,
                     int S, float* h_out, int T, int r_max, hipStream_t st, StageTimer* tm) {
    const int64_t n = (int64_t)T * r_max;
    if (n == 0) return hipSuccess;
    return launch(tm, "scatter_h", scatter_h_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, h, rank,
                  token_order, slot_indptr, S, h_out, T, r_max);
}

}  // namespace lora
