// Host-side launchers of the liblora gfx950 kernels (internal interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lora {

// Optional per-kernel timing: when a timer is passed, each launcher records a
// HIP event pair around every kernel it launches, on the launch stream.
struct StageTimer {
    virtual void begin(const char* kernel, hipStream_t st) = 0;
    virtual void end(hipStream_t st) = 0;
    virtual ~StageTimer() = default;
};

struct TimedScope {
    StageTimer* t;
    hipStream_t st;
    TimedScope(StageTimer* t_, const char* name, hipStream_t s) : t(t_), st(s) {
        if (t) t->begin(name, st);
    }
    ~TimedScope() {
        if (t) t->end(st);
    }
};

// ---- base GEMM: Y[M][N] = X[M][K] * W[N][K]^T --------------------------
struct GemmShape {
    int bm, bn;   // macro tile
    int ks;       // K splits (1 = no split, result written directly)
    int k_chunk;  // K elements per split (multiple of 64)
};
GemmShape gemm_bf16_shape(int M, int N, int K);
size_t gemm_bf16_workspace(int M, int N, int K);  // fp32 split-K partials
hipError_t gemm_bf16(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K, float* ws,
                     hipStream_t st, StageTimer* tm);
hipError_t gemm_f32(const float* X, const float* W, float* Y, int M, int N, int K, hipStream_t st, StageTimer* tm);

// ---- SGMV shrink / expand ------------------------------------------------
// Shrink partials: part[ks][T][r_max] fp32, indexed by sorted position.
int shrink_splits(int n_items, int K);
constexpr int kMaxShrinkSplits = 32;
hipError_t sgmv_shrink(int dtype, const void* X, const void* A_pool, const int32_t* rank,
                       const int32_t* token_order, const int32_t* work, int n_items, float* part, int ks, int T,
                       int K, int r_max, hipStream_t st, StageTimer* tm);
hipError_t sgmv_expand(int dtype, const float* part, int ks, const void* B_pool, const int32_t* rank,
                       const float* scale, const int32_t* token_order, const int32_t* work, int n_items, void* Y,
                       int T, int N, int r_max, hipStream_t st, StageTimer* tm);
hipError_t shrink_to_h(const float* part, int ks, const int32_t* rank, const int32_t* token_order,
                       const int32_t* slot_indptr, int S, float* h, int T, int r_max, hipStream_t st,
                       StageTimer* tm);

// ---- slot pool ------------------------------------------------------------
hipError_t pool_check_finite(int dtype, const void* p, int64_t n, int* flag, hipStream_t st);
hipError_t pool_write_slot(int dtype, void* A_pool, void* B_pool, int32_t* rank, float* scale, int slot,
                           const void* A, const void* B, int r, float sc, int r_max, int d_in, int d_out,
                           hipStream_t st);

}  // namespace lora
