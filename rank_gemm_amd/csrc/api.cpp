// C ABI of liblora: argument validation, the pool handle and launch order.
// Declarations and contracts: include/lora.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/lora.h"
#include "kernels.h"

struct lora_pool {
    int S, r_max, d_in, d_out, dtype;
    void* A;
    void* B;
    int32_t* rank_dev;
    float* scale_dev;
    int* flag_dev;  // finite-check result of the last install
    std::vector<int> rank;
    std::vector<float> scale;
};

namespace {

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline size_t es_of(int dtype) { return dtype == LORA_BF16 ? 2 : 4; }

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// The vector kernels read rows of x, W and A_s in 16-byte pieces: bf16 pools
// whose d_in is a multiple of 8. Every other pool (fp32, or rows that do not
// start on 16-byte boundaries) takes the element-generic kernels.
inline bool vector_path(const lora_pool* p) { return p->dtype == LORA_BF16 && p->d_in % 8 == 0; }

// K splits of the stand-alone shrinks: SGMV over few items (at most
// kShrinkSplitMaxBlocks workgroups) and BGMV (one workgroup per token and split)
inline void sgmv_split(int n_items, int K, int* hs, int* hkc) {
    *hs = 1;
    *hkc = K;
    if (n_items >= lora::kShrinkSplitMaxBlocks / 2) return;
    const int h = std::min(8, lora::kShrinkSplitMaxBlocks / std::max(n_items, 1));
    *hkc = std::max(256, ((K + h - 1) / h + 31) / 32 * 32);
    *hs = (K + *hkc - 1) / *hkc;
}
inline void bgmv_split(int T, int K, int* hs, int* hkc) {
    const int h = std::max(1, std::min(8, 2048 / std::max(T, 1)));
    *hkc = std::max(256, ((K + h - 1) / h + 31) / 32 * 32);
    *hs = (K + *hkc - 1) / *hkc;
}

// workspace: the bf16 path's partial products and h, and the stand-alone
// shrinks' h plus split planes; the fp32 path's h
inline size_t h_bytes(const lora_pool* p, int T) {
    const size_t h = align256((size_t)T * p->r_max * sizeof(float));
    if (!vector_path(p)) return h;
    const size_t g = lora::gemm_bf16_workspace(T, &p->d_out, 1, p->d_in, p->r_max);
    const size_t rows = std::max<size_t>({(size_t)lora::kShrinkSplitMaxBlocks * 16, 2048, (size_t)T});
    const size_t s = h + align256(rows * p->r_max * sizeof(float));
    return std::max(g, s);
}

static_assert(LORA_MAX_SLICES == lora::kMaxSlices, "slice limit of the interface and the kernels");
static_assert(LORA_MAX_RANK == lora::kMaxRank, "rank limit of the interface and the kernels");

// Every slice's pool must agree with the first on S, r_max, d_in and element
// type; with buffers, no output may alias x, a weight or another output.
int check_slices(const lora_slice* sl, int n, const void* x, bool buffers) {
    if (!sl || n < 1 || n > LORA_MAX_SLICES) return LORA_EINVAL;
    const lora_pool* p0 = sl[0].pool;
    for (int i = 0; i < n; ++i) {
        const lora_pool* p = sl[i].pool;
        if (!p) return LORA_EINVAL;
        if (p->S != p0->S || p->r_max != p0->r_max || p->d_in != p0->d_in || p->dtype != p0->dtype)
            return LORA_EINVAL;
        if (!buffers) continue;
        if (!sl[i].W || !sl[i].y || sl[i].y == x) return LORA_EINVAL;
        for (int j = 0; j < n; ++j) {
            if (sl[i].y == sl[j].W) return LORA_EINVAL;
            if (j != i && sl[i].y == sl[j].y) return LORA_EINVAL;
        }
    }
    return LORA_OK;
}

size_t multi_bytes(const lora_slice* sl, int n, int T) {
    const lora_pool* p0 = sl[0].pool;
    const size_t h = align256((size_t)T * p0->r_max * sizeof(float));
    if (!vector_path(p0)) return h;
    int N[LORA_MAX_SLICES];
    for (int i = 0; i < n; ++i) N[i] = sl[i].pool->d_out;
    const size_t g = lora::gemm_bf16_workspace(T, N, n, p0->d_in, p0->r_max);
    return g > h ? g : h;
}

// Per-kernel timing for diagnostics: HIP event pairs around each kernel on
// its launch stream, aggregated by kernel name at lora_profile_end.
struct Profiler final : lora::StageTimer {
    std::mutex mu;
    bool on = false;
    int max_records = 0;
    struct Rec {
        const char* name;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> spare;

    hipEvent_t take() {
        if (!spare.empty()) {
            hipEvent_t e = spare.back();
            spare.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    bool pair(const char* kernel, hipEvent_t* start, hipEvent_t* stop) override {
        if ((int)recs.size() >= max_records) return false;
        hipEvent_t a = take(), b = take();
        if (!a || !b) return false;
        recs.push_back({kernel, a, b});
        *start = a;
        *stop = b;
        return true;
    }
};

Profiler& profiler() {
    static Profiler p;
    return p;
}

// Timer for a call on `st`, or nullptr when profiling is off, full, or the
// stream is being captured into a graph.
lora::StageTimer* timer_for(hipStream_t st) {
    Profiler& p = profiler();
    if (!p.on || (int)p.recs.size() >= p.max_records) return nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    return &p;
}

inline bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

// A plan for this pool; `any_chunk` admits plans of chunked items (lora_delta),
// every other caller needs LORA_PLAN_ROWS-row items.
int check_plan(const lora_pool* p, const int32_t* token_order, const int32_t* slot_indptr, const int32_t* work,
               const lora_plan_info* info, bool any_chunk = false) {
    if (!p || !info) return LORA_EINVAL;
    if (info->S != p->S || info->T < 0 || info->T_a < 0 || info->T_a > info->T || info->n_items < 0)
        return LORA_EINVAL;
    if (any_chunk ? !valid_chunk(info->chunk) : info->chunk != LORA_PLAN_ROWS) return LORA_EINVAL;
    if (info->T > 0 && (!token_order || !slot_indptr)) return LORA_EINVAL;
    if (info->n_items > 0 && !work) return LORA_EINVAL;
    return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_status_string(int status) {
    switch (status) {
        case LORA_OK: return "ok";
        case LORA_EINVAL: return "invalid argument";
        case LORA_ESLOT: return "slot id out of range";
        case LORA_ERANK: return "rank out of range";
        case LORA_ENONFINITE: return "non-finite adapter weights or alpha";
        case LORA_EHIP: return "HIP runtime error";
        case LORA_ESPACE: return "buffer too small";
        default: return "unknown status";
    }
}

int lora_pool_create(lora_pool** out, int S, int r_max, int d_in, int d_out, int dtype, void* A_pool, void* B_pool,
                     int32_t* rank_dev, float* scale_dev, void* stream) {
    if (!out) return LORA_EINVAL;
    *out = nullptr;
    if (S < 2 || r_max < 1 || r_max > LORA_MAX_RANK || d_in < 1 || d_out < 1) return LORA_EINVAL;
    if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_EINVAL;
    if (!A_pool || !B_pool || !rank_dev || !scale_dev) return LORA_EINVAL;
    lora_pool* p = new (std::nothrow) lora_pool();
    if (!p) return LORA_EINVAL;
    p->S = S;
    p->r_max = r_max;
    p->d_in = d_in;
    p->d_out = d_out;
    p->dtype = dtype;
    p->A = A_pool;
    p->B = B_pool;
    p->rank_dev = rank_dev;
    p->scale_dev = scale_dev;
    p->rank.assign(S, 0);
    p->scale.assign(S, 0.f);
    hipStream_t st = as_stream(stream);
    const size_t es = es_of(dtype);
    bool ok = hipMalloc(&p->flag_dev, sizeof(int)) == hipSuccess;
    ok = ok && hipMemsetAsync(A_pool, 0, (size_t)S * r_max * d_in * es, st) == hipSuccess;
    ok = ok && hipMemsetAsync(B_pool, 0, (size_t)S * d_out * r_max * es, st) == hipSuccess;
    ok = ok && hipMemsetAsync(rank_dev, 0, (size_t)S * sizeof(int32_t), st) == hipSuccess;
    ok = ok && hipMemsetAsync(scale_dev, 0, (size_t)S * sizeof(float), st) == hipSuccess;
    ok = ok && hipStreamSynchronize(st) == hipSuccess;
    if (!ok) {
        if (p->flag_dev) (void)hipFree(p->flag_dev);
        delete p;
        return LORA_EHIP;
    }
    *out = p;
    return LORA_OK;
}

void lora_pool_destroy(lora_pool* pool) {
    if (!pool) return;
    if (pool->flag_dev) (void)hipFree(pool->flag_dev);
    delete pool;
}

int lora_pool_rank(const lora_pool* pool, int slot) {
    if (!pool || slot < 0 || slot >= pool->S) return -1;
    return pool->rank[slot];
}

int lora_pool_install(lora_pool* p, int slot, const void* A, const void* B, int r, float alpha, void* stream) {
    if (!p || !A || !B) return LORA_EINVAL;
    if (slot < 1 || slot >= p->S) return LORA_ESLOT;
    if (r < 1 || r > p->r_max) return LORA_ERANK;
    if (!std::isfinite(alpha)) return LORA_ENONFINITE;
    const float sc = alpha / (float)r;
    if (!std::isfinite(sc)) return LORA_ENONFINITE;
    hipStream_t st = as_stream(stream);
    int flag = 0;
    if (hipMemsetAsync(p->flag_dev, 0, sizeof(int), st) != hipSuccess) return LORA_EHIP;
    if (lora::pool_check_finite(p->dtype, A, (int64_t)r * p->d_in, p->flag_dev, st) != hipSuccess) return LORA_EHIP;
    if (lora::pool_check_finite(p->dtype, B, (int64_t)p->d_out * r, p->flag_dev, st) != hipSuccess) return LORA_EHIP;
    if (hipMemcpyAsync(&flag, p->flag_dev, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return LORA_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_EHIP;
    if (flag) return LORA_ENONFINITE;
    if (lora::pool_write_slot(p->dtype, p->A, p->B, p->rank_dev, p->scale_dev, slot, A, B, r, sc, p->r_max, p->d_in,
                              p->d_out, st) != hipSuccess)
        return LORA_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_EHIP;
    p->rank[slot] = r;
    p->scale[slot] = sc;
    return LORA_OK;
}

int lora_pool_clear(lora_pool* p, int slot, void* stream) {
    if (!p) return LORA_EINVAL;
    if (slot < 1 || slot >= p->S) return LORA_ESLOT;
    hipStream_t st = as_stream(stream);
    if (lora::pool_write_slot(p->dtype, p->A, p->B, p->rank_dev, p->scale_dev, slot, nullptr, nullptr, 0, 0.f,
                              p->r_max, p->d_in, p->d_out, st) != hipSuccess)
        return LORA_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LORA_EHIP;
    p->rank[slot] = 0;
    p->scale[slot] = 0.f;
    return LORA_OK;
}

size_t lora_workspace_bytes(const lora_pool* pool, int T) {
    if (!pool || T < 0) return 0;
    return h_bytes(pool, T);
}

int lora_linear(const lora_pool* p, const void* x, const void* W, const int32_t* token_order,
                const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info, void* y,
                void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_plan(p, token_order, slot_indptr, work, info);
    if (rc != LORA_OK) return rc;
    const int T = info->T;
    if (T == 0) return LORA_OK;
    if (!x || !W || !y) return LORA_EINVAL;
    if (y == x || y == W) return LORA_EINVAL;
    const bool adapters = info->T_a > 0 && info->n_items > 0;
    if (adapters && (!workspace || workspace_bytes < lora_workspace_bytes(p, T))) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    float* h = static_cast<float*>(workspace);

    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);

    if (vector_path(p)) {
        if (!workspace || workspace_bytes < lora_workspace_bytes(p, T)) return LORA_ESPACE;
        lora::LinearArgs la{};
        la.X = (const uint16_t*)x;
        la.M = T;
        la.K = p->d_in;
        la.token_order = token_order;
        la.slot_indptr = slot_indptr;
        la.work = work;
        la.n_items = info->n_items;
        la.S = p->S;
        la.r_max = p->r_max;
        la.adapters = adapters ? 1 : 0;
        la.workspace = workspace;
        la.n_slices = 1;
        la.slice[0] = {(const uint16_t*)W, (uint16_t*)y, p->d_out, (const uint16_t*)p->A, (const uint16_t*)p->B,
                       p->rank_dev, p->scale_dev};
        return lora::lora_forward_bf16(la, st, tm) == hipSuccess ? LORA_OK : LORA_EHIP;
    }
    // element-generic kernels: the shrink (adapter rows only), then the base
    // GEMM with the expand in its epilogue
    return lora::generic_linear(p->dtype, x, W, y, token_order, slot_indptr, work, info->n_items, p->S, p->A, p->B,
                                p->rank_dev, p->scale_dev, h, adapters ? 1 : 0, T, p->d_out, p->d_in, p->r_max, st,
                                tm) == hipSuccess
               ? LORA_OK
               : LORA_EHIP;
}

size_t lora_plan_device_words(int T, int S) {
    if (T < 0 || S < 1 || S > LORA_DEVICE_PLAN_MAX_SLOTS) return 0;
    const int cap = std::max(lora_plan_max_items(T, S), 1);
    return 4 * (size_t)cap + (size_t)T + (size_t)S + 1 + 8;
}

int lora_plan_upload(const int32_t* host_plan, int32_t* dev_plan, size_t words, void* stream) {
    if (words == 0) return LORA_OK;
    if (!host_plan || !dev_plan) return LORA_EINVAL;
    // the device's address of the pinned buffer (fails for pageable memory)
    void* src = nullptr;
    if (hipHostGetDevicePointer(&src, const_cast<int32_t*>(host_plan), 0) != hipSuccess || !src) {
        (void)hipGetLastError();
        return LORA_EINVAL;
    }
    return lora::plan_upload(static_cast<const int32_t*>(src), dev_plan, words, as_stream(stream)) == hipSuccess
               ? LORA_OK
               : LORA_EHIP;
}

int lora_plan_device(int S, const int32_t* slot_ids, int T, int32_t* plan, void* stream) {
    if (S < 1 || S > LORA_DEVICE_PLAN_MAX_SLOTS || T < 0 || !plan || (T > 0 && !slot_ids)) return LORA_EINVAL;
    const int cap = std::max(lora_plan_max_items(T, S), 1);
    return lora::plan_device(slot_ids, T, S, cap, plan, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_EHIP;
}

int lora_linear_device_plan(const lora_pool* p, const void* x, const void* W, const int32_t* plan, int T, void* y,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (!p || !plan || T < 0 || p->S > LORA_DEVICE_PLAN_MAX_SLOTS) return LORA_EINVAL;
    const int cap = std::max(lora_plan_max_items(T, p->S), 1);
    const int32_t* work = plan;
    const int32_t* token_order = plan + 4 * (size_t)cap;
    const int32_t* slot_indptr = token_order + T;
    // the host knows only the shapes: every row may carry an adapter, and the
    // work list is launched at its capacity (padding items are on slot 0)
    lora_plan_info info{T, p->S, T, 0, lora_plan_max_items(T, p->S), 0, LORA_PLAN_ROWS};
    return lora_linear(p, x, W, token_order, slot_indptr, work, &info, y, workspace, workspace_bytes, stream);
}

int lora_linear_multi_device_plan(const lora_slice* slices, int n, const void* x, const int32_t* plan, int T,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_slices(slices, n, x, false);  // buffers: checked by lora_linear_multi when T > 0
    if (rc != LORA_OK) return rc;
    const lora_pool* p0 = slices[0].pool;
    if (!plan || T < 0 || p0->S > LORA_DEVICE_PLAN_MAX_SLOTS) return LORA_EINVAL;
    const int cap = std::max(lora_plan_max_items(T, p0->S), 1);
    const int32_t* work = plan;
    const int32_t* token_order = plan + 4 * (size_t)cap;
    const int32_t* slot_indptr = token_order + T;
    lora_plan_info info{T, p0->S, T, 0, lora_plan_max_items(T, p0->S), 0, LORA_PLAN_ROWS};
    return lora_linear_multi(slices, n, x, token_order, slot_indptr, work, &info, workspace, workspace_bytes, stream);
}

size_t lora_workspace_bytes_multi(const lora_slice* slices, int n, int T) {
    if (T < 0 || check_slices(slices, n, nullptr, false) != LORA_OK) return 0;
    return multi_bytes(slices, n, T);
}

int lora_linear_multi(const lora_slice* slices, int n, const void* x, const int32_t* token_order,
                      const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info,
                      void* workspace, size_t workspace_bytes, void* stream) {
    // the pools first; the buffers only when there are rows (an empty batch
    // may pass null or coinciding pointers for its empty outputs)
    int rc = check_slices(slices, n, x, false);
    if (rc != LORA_OK) return rc;
    const lora_pool* p0 = slices[0].pool;
    rc = check_plan(p0, token_order, slot_indptr, work, info);
    if (rc != LORA_OK) return rc;
    const int T = info->T;
    if (T == 0) return LORA_OK;
    rc = check_slices(slices, n, x, true);
    if (rc != LORA_OK) return rc;
    if (!x) return LORA_EINVAL;
    if (!vector_path(p0)) {
        // element-generic pools: the slices one after another on the same
        // stream (the workspace is reused in stream order)
        for (int i = 0; i < n; ++i) {
            rc = lora_linear(slices[i].pool, x, slices[i].W, token_order, slot_indptr, work, info, slices[i].y,
                             workspace, workspace_bytes, stream);
            if (rc != LORA_OK) return rc;
        }
        return LORA_OK;
    }
    if (!workspace || workspace_bytes < multi_bytes(slices, n, T)) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);
    lora::LinearArgs la{};
    la.X = (const uint16_t*)x;
    la.M = T;
    la.K = p0->d_in;
    la.token_order = token_order;
    la.slot_indptr = slot_indptr;
    la.work = work;
    la.n_items = info->n_items;
    la.S = p0->S;
    la.r_max = p0->r_max;
    la.adapters = info->T_a > 0 && info->n_items > 0 ? 1 : 0;
    la.workspace = workspace;
    la.n_slices = n;
    for (int i = 0; i < n; ++i) {
        const lora_pool* p = slices[i].pool;
        la.slice[i] = {(const uint16_t*)slices[i].W, (uint16_t*)slices[i].y, p->d_out, (const uint16_t*)p->A,
                       (const uint16_t*)p->B, p->rank_dev, p->scale_dev};
    }
    return lora::lora_forward_bf16(la, st, tm) == hipSuccess ? LORA_OK : LORA_EHIP;
}

int lora_shrink(const lora_pool* p, const void* x, const int32_t* token_order, const int32_t* slot_indptr,
                const int32_t* work, const lora_plan_info* info, float* h, void* workspace, size_t workspace_bytes,
                void* stream) {
    int rc = check_plan(p, token_order, slot_indptr, work, info);
    if (rc != LORA_OK) return rc;
    const int T = info->T;
    if (T == 0) return LORA_OK;
    if (!x || !h) return LORA_EINVAL;
    if (!workspace || workspace_bytes < lora_workspace_bytes(p, T)) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    float* hs = static_cast<float*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)T * p->r_max * 4));
    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);
    int ks = 1, kc = p->d_in;
    if (vector_path(p)) sgmv_split(info->n_items, p->d_in, &ks, &kc);
    if (info->n_items > 0) {
        hipError_t e;
        if (!vector_path(p))
            e = lora::generic_shrink(p->dtype, x, p->A, p->rank_dev, token_order, work, info->n_items, hs, p->d_in,
                                     p->r_max, st, tm);
        else if (ks > 1)
            e = lora::sgmv_shrink_split((const uint16_t*)x, (const uint16_t*)p->A, p->rank_dev, p->scale_dev,
                                        token_order, work, info->n_items, ks, kc, part, hs, nullptr, p->d_in,
                                        p->r_max, st, tm);
        else
            e = lora::sgmv_shrink((const uint16_t*)x, (const uint16_t*)p->A, p->rank_dev, token_order, work,
                                  info->n_items, hs, p->d_in, p->r_max, st, tm);
        if (e != hipSuccess) return LORA_EHIP;
    }
    if (lora::scatter_h(hs, p->rank_dev, token_order, slot_indptr, p->S, h, T, p->r_max, st, tm) != hipSuccess)
        return LORA_EHIP;
    return LORA_OK;
}

int lora_shrink_bgmv(const lora_pool* p, const void* x, const int32_t* slot_ids, int T, float* h, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (!p || T < 0) return LORA_EINVAL;
    if (!vector_path(p)) return LORA_EINVAL;
    if (T == 0) return LORA_OK;
    if (!x || !slot_ids || !h) return LORA_EINVAL;
    if (!workspace || workspace_bytes < lora_workspace_bytes(p, T)) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)T * p->r_max * 4));
    int ks = 1, kc = p->d_in;
    bgmv_split(T, p->d_in, &ks, &kc);
    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);
    return lora::bgmv_shrink((const uint16_t*)x, (const uint16_t*)p->A, p->rank_dev, slot_ids, p->S, T, ks, kc, part,
                             h, p->d_in, p->r_max, st, tm) == hipSuccess
               ? LORA_OK
               : LORA_EHIP;
}

int lora_delta(const lora_pool* p, const void* x, const int32_t* token_order, const int32_t* slot_indptr,
               const int32_t* work, const lora_plan_info* info, void* y, void* workspace, size_t workspace_bytes,
               void* stream) {
    int rc = check_plan(p, token_order, slot_indptr, work, info, true);
    if (rc != LORA_OK) return rc;
    const int T = info->T;
    if (T == 0) return LORA_OK;
    if (!x || !y || y == x) return LORA_EINVAL;
    if (info->T_a == 0 || info->n_items == 0) return LORA_OK;
    if (!workspace || workspace_bytes < lora_workspace_bytes(p, T)) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);
    float* part = static_cast<float*>(workspace);
    hipError_t e;
    if (vector_path(p)) {
        // split K over workgroups when the items are few; the planes
        // [hs][T][r_max] fit the workspace while hs <= 1 + max(4096, T) / T
        int hs = 1, hkc = p->d_in;
        sgmv_split(info->n_items, p->d_in, &hs, &hkc);
        const int cap = 1 + std::max(4096, T) / T;
        if (hs > cap) {
            hkc = std::max(256, ((p->d_in + cap - 1) / cap + 31) / 32 * 32);
            hs = (p->d_in + hkc - 1) / hkc;
        }
        e = lora::delta_sgmv((const uint16_t*)x, (const uint16_t*)p->A, (const uint16_t*)p->B, p->rank_dev,
                             p->scale_dev, token_order, work, info->n_items, info->chunk, hs, hkc, part, (uint16_t*)y,
                             T, p->d_out, p->d_in, p->r_max, st, tm);
    } else {
        e = lora::generic_shrink(p->dtype, x, p->A, p->rank_dev, token_order, work, info->n_items, part, p->d_in,
                                 p->r_max, st, tm);
        if (e == hipSuccess)
            e = lora::generic_expand(p->dtype, part, p->B, p->rank_dev, p->scale_dev, token_order, work,
                                     info->n_items, y, p->d_out, p->r_max, st, tm);
    }
    return e == hipSuccess ? LORA_OK : LORA_EHIP;
}

int lora_delta_bgmv(const lora_pool* p, const void* x, const int32_t* slot_ids, int T, void* y, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!p || T < 0) return LORA_EINVAL;
    if (!vector_path(p)) return LORA_EINVAL;
    if (T == 0) return LORA_OK;
    if (!x || !slot_ids || !y || y == x) return LORA_EINVAL;
    if (!workspace || workspace_bytes < lora_workspace_bytes(p, T)) return LORA_ESPACE;
    hipStream_t st = as_stream(stream);
    int hs = 1, hkc = p->d_in;
    bgmv_split(T, p->d_in, &hs, &hkc);
    std::unique_lock<std::mutex> lk(profiler().mu, std::defer_lock);
    if (profiler().on) lk.lock();
    lora::StageTimer* tm = timer_for(st);
    return lora::delta_bgmv((const uint16_t*)x, (const uint16_t*)p->A, (const uint16_t*)p->B, p->rank_dev,
                            p->scale_dev, slot_ids, p->S, hs, hkc, static_cast<float*>(workspace), (uint16_t*)y, T,
                            p->d_out, p->d_in, p->r_max, st, tm) == hipSuccess
               ? LORA_OK
               : LORA_EHIP;
}

int lora_profile_begin(int max_records) {
    if (max_records < 8) return LORA_EINVAL;
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.on) return LORA_EINVAL;
    for (auto& r : p.recs) {
        p.spare.push_back(r.a);
        p.spare.push_back(r.b);
    }
    p.recs.clear();
    p.recs.reserve(max_records);
    p.max_records = max_records;
    p.on = true;
    return LORA_OK;
}

int lora_profile_end(lora_kernel_stat* out, int cap, int* n_out) {
    Profiler& p = profiler();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on) return LORA_EINVAL;
    p.on = false;
    struct Acc {
        int n = 0;
        double sum = 0, mn = 1e30, mx = 0;
        std::vector<float> all;
    };
    std::map<std::string, Acc> acc;
    std::vector<std::string> order;
    int rc = LORA_OK;
    for (auto& r : p.recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            rc = LORA_EHIP;
            continue;
        }
        auto it = acc.find(r.name);
        if (it == acc.end()) {
            order.push_back(r.name);
            it = acc.emplace(r.name, Acc{}).first;
        }
        Acc& a = it->second;
        ++a.n;
        a.sum += ms;
        a.mn = ms < a.mn ? ms : a.mn;
        a.mx = ms > a.mx ? ms : a.mx;
        a.all.push_back(ms);
    }
    for (auto& r : p.recs) {
        p.spare.push_back(r.a);
        p.spare.push_back(r.b);
    }
    p.recs.clear();
    int n = 0;
    for (const auto& name : order) {
        if (out && n < cap) {
            Acc& a = acc[name];
            std::memset(&out[n], 0, sizeof(out[n]));
            std::strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
            out[n].count = a.n;
            out[n].mean_ms = a.sum / a.n;
            out[n].min_ms = a.mn;
            out[n].max_ms = a.mx;
            // median: the middle element, or the mean of the two middle ones
            const size_t h = a.all.size() / 2;
            std::nth_element(a.all.begin(), a.all.begin() + h, a.all.end());
            double med = a.all[h];
            if (a.all.size() % 2 == 0) med = 0.5 * (med + *std::max_element(a.all.begin(), a.all.begin() + h));
            out[n].median_ms = med;
        }
        ++n;
    }
    if (n_out) *n_out = n;
    if (rc == LORA_OK && out && n > cap) rc = LORA_ESPACE;
    return rc;
}

}  // extern "C"
