// Host-side launchers of the liblora gfx950 kernels (internal interface).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lora {

// Optional per-kernel timing. When a timer is given, a kernel is launched with
// hipExtLaunchKernel and a pair of events that the runtime stamps with the
// kernel's own start and end on its stream (no marker packets around it).
struct StageTimer {
    // events to attach to the next launch of `kernel`; false: launch untimed
    virtual bool pair(const char* kernel, hipEvent_t* start, hipEvent_t* stop) = 0;
    virtual ~StageTimer() = default;
};

template <typename... Params, typename... Args>
inline hipError_t launch_shm(StageTimer* tm, const char* name, void (*kernel)(Params...), dim3 grid, dim3 block,
                             uint32_t shmem, hipStream_t st, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (tm && tm->pair(name, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0, static_cast<Params>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, static_cast<Params>(args)...);
    return hipGetLastError();
}

template <typename... Params, typename... Args>
inline hipError_t launch(StageTimer* tm, const char* name, void (*kernel)(Params...), dim3 grid, dim3 block,
                         hipStream_t st, Args... args) {
    return launch_shm(tm, name, kernel, grid, block, 0, st, args...);
}

// ---- bf16 forward: shrink + base GEMM with the expand in its epilogue ------
// y[token_order[p]] = bf16(x[token_order[p]] W^T + scale_s h[p] B_s^T), rows
// visited in plan order; with adapters == 0 the correction is skipped.
// Several slices (projections reading the same x, each with its own W, y and
// pool) can be computed in one pass.
struct GemmPlan {
    int bm, bn;          // macro tile of the tiled path
    int nsub;            // split-K path: 128-wide K sub-chunks per split (0 = tiled path)
    int ks, n_mt, n_nt;  // split-K path: splits and 64 x 64 tile grid
    int tks, tkc;        // tiled path split over K: tks ranges of tkc k (tkc % 64 == 0); tks < 2: none
};
GemmPlan gemm_bf16_plan(int M, int N, int K);

constexpr int kMaxSlices = 4;
struct SliceArgs {
    const uint16_t* W;       // [N][K]
    uint16_t* Y;             // [M][N]
    int N;
    const uint16_t* A_pool;  // [S][r_max][K]
    const uint16_t* B_pool;  // [S][N][r_max]
    const int32_t* rank;     // [S]
    const float* scale;      // [S]
};

struct LinearArgs {
    const uint16_t* X;  // [M][K]
    int M, K;
    const int32_t* token_order;
    const int32_t* slot_indptr;
    const int32_t* work;
    int n_items;
    int S, r_max;
    int adapters;
    void* workspace;
    int n_slices;
    SliceArgs slice[kMaxSlices];
};
// workspace of a forward over slices of N[0..n_slices) columns
size_t gemm_bf16_workspace(int M, const int* N, int n_slices, int K, int r_max);
hipError_t lora_forward_bf16(const LinearArgs& L, hipStream_t st, StageTimer* tm);

// ---- element-generic path (fp32 pools; bf16 pools with d_in % 8 != 0) --------
// dtype 0 = fp32, 1 = bf16. Shrink into h [T][r_max] fp32 (sorted positions),
// then the base GEMM over sorted positions with the expand in its epilogue and
// one rounding; with adapters == 0 neither h nor the pool is read.
hipError_t generic_shrink(int dtype, const void* X, const void* A_pool, const int32_t* rank,
                          const int32_t* token_order, const int32_t* work, int n_items, float* h, int K, int r_max,
                          hipStream_t st, StageTimer* tm);
hipError_t generic_linear(int dtype, const void* X, const void* W, void* Y, const int32_t* token_order,
                          const int32_t* slot_indptr, const int32_t* work, int n_items, int S, const void* A_pool,
                          const void* B_pool, const int32_t* rank, const float* scale, float* h, int adapters, int M,
                          int N, int K, int r_max, hipStream_t st, StageTimer* tm);

// ---- device planner -----------------------------------------------------------
// plan: [work 4 * cap][token_order T][slot_indptr S + 1][info 8], work padded
// to cap with empty items on slot 0; one workgroup.
constexpr int kDevPlanMaxSlots = 4096;
hipError_t plan_device(const int32_t* ids, int T, int S, int cap, int32_t* plan, hipStream_t st);
hipError_t plan_upload(const int32_t* src, int32_t* dst, size_t words, hipStream_t st);

// ---- SGMV shrink (bf16, K % 8 == 0) --------------------------------------------
// h: fp32 [T][r_max] indexed by sorted position (rows of adapter items only).
// With ext, writes the expand operand of the tiled GEMM's extra K steps,
// scale_s * h as bf16 hi / lo: [T][2][round_up(r_max, 8)].
hipError_t sgmv_shrink(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank,
                       const int32_t* token_order, const int32_t* work, int n_items, float* h, int K, int r_max,
                       hipStream_t st, StageTimer* tm, const float* scale = nullptr, uint16_t* ext = nullptr);
// The expand operands of up to kMaxSlices projections over the same x in one
// pass (x rows read once): slice i's A_pool, rank, scale and ext in ss.
struct ShrinkSlices;
hipError_t sgmv_shrink_slices(const uint16_t* X, const ShrinkSlices& ss, const int32_t* token_order,
                              const int32_t* work, int n_items, int K, int r_max, hipStream_t st, StageTimer* tm);
// The same over hs K ranges of hkc k each (few items, long K): fp32 planes in
// part ([n_items * hs][16][r_max]), then h or ext as above.
constexpr int kShrinkSplitMaxBlocks = 256;
hipError_t sgmv_shrink_split(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const float* scale,
                             const int32_t* token_order, const int32_t* work, int n_items, int hs, int hkc,
                             float* part, float* h, uint16_t* ext, int K, int r_max, hipStream_t st,
                             StageTimer* tm);
// BGMV shrink (token by token, no plan): planes part [hs][T][r_max] (q < r_s
// of tokens on an installed slot only), then h [T][r_max] in token order.
hipError_t bgmv_shrink_planes(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const int32_t* slot_ids,
                              int S, int T, int hs, int hkc, float* part, int K, int r_max, hipStream_t st,
                              StageTimer* tm);
hipError_t bgmv_shrink(const uint16_t* X, const uint16_t* A_pool, const int32_t* rank, const int32_t* slot_ids,
                       int S, int T, int hs, int hkc, float* part, float* h, int K, int r_max, hipStream_t st,
                       StageTimer* tm);
hipError_t scatter_h(const float* h, const int32_t* rank, const int32_t* token_order, const int32_t* slot_indptr,
                     int S, float* h_out, int T, int r_max, hipStream_t st, StageTimer* tm);

// ---- the correction alone, y += delta (bf16, K % 8 == 0) --------------------------
// SGMV over a plan of `chunk`-row items (16, 32, 64, 128): shrink into planes
// part [hs][T][r_max] by sorted position over hs K ranges of hkc k, then the
// expand adds the planes and updates y in place. BGMV: the same token by token
// from device slot ids, planes by token index.
constexpr int kMaxRank = 1024;
hipError_t delta_sgmv(const uint16_t* X, const uint16_t* A_pool, const uint16_t* B_pool, const int32_t* rank,
                      const float* scale, const int32_t* token_order, const int32_t* work, int n_items, int chunk,
                      int hs, int hkc, float* part, uint16_t* Y, int T, int N, int K, int r_max, hipStream_t st,
                      StageTimer* tm);
hipError_t delta_bgmv(const uint16_t* X, const uint16_t* A_pool, const uint16_t* B_pool, const int32_t* rank,
                      const float* scale, const int32_t* slot_ids, int S, int hs, int hkc, float* part, uint16_t* Y,
                      int T, int N, int K, int r_max, hipStream_t st, StageTimer* tm);
// element-generic pools: h from generic_shrink (items of any row count), then
// y[t_p][n] = round(y + scale_s * h[p] . B_s[n]) in place
hipError_t generic_expand(int dtype, const float* h, const void* B_pool, const int32_t* rank, const float* scale,
                          const int32_t* token_order, const int32_t* work, int n_items, void* Y, int N, int r_max,
                          hipStream_t st, StageTimer* tm);

// ---- slot pool ------------------------------------------------------------
hipError_t pool_check_finite(int dtype, const void* p, int64_t n, int* flag, hipStream_t st);
hipError_t pool_write_slot(int dtype, void* A_pool, void* B_pool, int32_t* rank, float* scale, int slot,
                           const void* A, const void* B, int r, float sc, int r_max, int d_in, int d_out,
                           hipStream_t st);

}  // namespace lora
