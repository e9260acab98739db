// Segment planner on the device: the same stable counting sort as the host
// planner (plan.cpp), so that a step's plan can be built from device-resident
// slot ids inside a captured HIP graph, with no host work and no copy.
//
// "LoRA serving, embeddings, rerankers, pooling" (mlinterviewnotes.com),
// section "vLLM: preallocated stacked buffers ...": the kernels' metadata is a
// stable sort of the token -> slot map plus per-slot counts, rebuilt every
// forward pass. One workgroup: an LDS histogram (atomic adds), exclusive
// scans by one wave, then a stable scatter by one wave that walks the tokens
// in index order, 64 at a time, ranking equal slots within a group of 64 by
// ballots. The work list is padded to its capacity with empty items on slot
// 0 (rank 0), which every kernel skips, so launches sized for the capacity
// need no host knowledge of the plan.
#include <algorithm>

#include "../../include/lora.h"
#include "common.h"
#include "kernels.h"

namespace lora {

namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d));
    return v;
}

// plan: [work 4 * cap][token_order T][slot_indptr S + 1][info 8]
__global__ __launch_bounds__(kPlanThreads) void plan_device_kernel(const int32_t* __restrict__ ids, int T, int S,
                                                                   int cap, int32_t* __restrict__ plan) {
    __shared__ int cnt[kDevPlanMaxSlots];
    __shared__ int ptr[kDevPlanMaxSlots + 1];
    __shared__ int aux[kDevPlanMaxSlots + 1];  // item offsets, then the scatter cursors
    __shared__ int totals[4];                  // n_items, k, max_seg, any invalid id
    int32_t* work = plan;
    int32_t* order = plan + 4 * (int64_t)cap;
    int32_t* indptr = order + T;
    int32_t* info = indptr + S + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int s = tid; s < S; s += kPlanThreads) cnt[s] = 0;
    if (tid == 0) totals[3] = 0;
    __syncthreads();
    // histogram; an id outside [0, S) counts as slot 0 and is reported
    for (int t = tid; t < T; t += kPlanThreads) {
        int s = ids[t];
        if (s < 0 || s >= S) {
            s = 0;
            totals[3] = 1;
        }
        atomicAdd(&cnt[s], 1);
    }
    __syncthreads();

    if (wave == 0) {
        // exclusive scans of the counts (-> ptr) and of the item counts of
        // slots >= 1 (-> aux); lane l owns slots [l * ch, (l + 1) * ch)
        const int ch = (S + 63) / 64;
        const int s0 = min(S, lane * ch), s1 = min(S, s0 + ch);
        int c = 0, it = 0, k = 0, mx = 0;
        for (int s = s0; s < s1; ++s) {
            c += cnt[s];
            if (s >= 1 && cnt[s] > 0) {
                it += (cnt[s] + LORA_PLAN_ROWS - 1) / LORA_PLAN_ROWS;
                ++k;
                mx = max(mx, cnt[s]);
            }
        }
        int pc = wave_incl_scan(c, lane) - c;
        int pi = wave_incl_scan(it, lane) - it;
        for (int s = s0; s < s1; ++s) {
            ptr[s] = pc;
            aux[s] = pi;
            pc += cnt[s];
            if (s >= 1) pi += (cnt[s] + LORA_PLAN_ROWS - 1) / LORA_PLAN_ROWS;
        }
        const int n_items = wave_sum(it), kk = wave_sum(k), mseg = wave_max(mx);
        if (lane == 0) {
            ptr[S] = T;
            totals[0] = n_items;
            totals[1] = kk;
            totals[2] = mseg;
        }
    }
    __syncthreads();

    // slot_indptr and the work list (items of at most 16 rows per segment of
    // a slot >= 1, in ascending slot order), padded with empty items
    for (int s = tid; s <= S; s += kPlanThreads) indptr[s] = ptr[s];
    for (int s = 1 + tid; s < S; s += kPlanThreads) {
        const int n = cnt[s];
        for (int j = 0; j * LORA_PLAN_ROWS < n; ++j) {
            int32_t* w = work + 4 * (int64_t)(aux[s] + j);
            w[0] = s;
            w[1] = ptr[s] + j * LORA_PLAN_ROWS;
            w[2] = min(LORA_PLAN_ROWS, n - j * LORA_PLAN_ROWS);
            w[3] = 0;
        }
    }
    for (int i = totals[0] + tid; i < cap; i += kPlanThreads) {
        int32_t* w = work + 4 * (int64_t)i;
        w[0] = 0;
        w[1] = 0;
        w[2] = 0;
        w[3] = 0;
    }
    __syncthreads();
    for (int s = tid; s < S; s += kPlanThreads) aux[s] = ptr[s];
    __syncthreads();

    if (wave == 0) {
        // stable scatter: groups of 64 tokens in index order; within a group,
        // the lanes of one slot take consecutive positions in lane order
        for (int t0 = 0; t0 < T; t0 += 64) {
            const int t = t0 + lane;
            const bool valid = t < T;
            int s = valid ? ids[t] : 0;
            if (s < 0 || s >= S) s = 0;
            uint64_t todo = __ballot(valid);
            while (todo) {
                const int leader = __ffsll((unsigned long long)todo) - 1;
                const int v = __shfl(s, leader);
                const uint64_t m = __ballot(valid && s == v);
                if (valid && s == v) {
                    const int below = __popcll(m & ((1ull << lane) - 1));
                    order[aux[v] + below] = t;
                }
                if (lane == leader) aux[v] += __popcll(m);
                todo &= ~m;
            }
        }
    }
    if (tid == 0) {
        info[0] = T;
        info[1] = S;
        info[2] = T - cnt[0];
        info[3] = totals[1];
        info[4] = totals[0];
        info[5] = totals[2];
        info[6] = totals[3] ? LORA_ESLOT : LORA_OK;
        info[7] = 0;
    }
}

// Copy of a pinned host buffer: 16-byte pieces when both ends allow, then
// the tail words.
__global__ __launch_bounds__(256) void plan_upload_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst,
                                                          size_t words, int vec) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t n4 = vec ? words / 4 : 0;
    if (i < n4) reinterpret_cast<int4*>(dst)[i] = reinterpret_cast<const int4*>(src)[i];
    const size_t t = 4 * n4 + i;
    if (t < words && i < (vec ? 4 : words)) dst[t] = src[t];
}

}  // namespace

hipError_t plan_upload(const int32_t* src, int32_t* dst, size_t words, hipStream_t st) {
    if (words == 0) return hipSuccess;
    const int vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    const size_t n = vec ? std::max<size_t>(words / 4, 4) : words;
    return launch(nullptr, "plan_upload", plan_upload_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, src, dst,
                  words, vec);
}

hipError_t plan_device(const int32_t* ids, int T, int S, int cap, int32_t* plan, hipStream_t st) {
    return launch(nullptr, "plan_device", plan_device_kernel, dim3(1), dim3(kPlanThreads), st, ids, T, S, cap, plan);
}

}  // namespace lora
