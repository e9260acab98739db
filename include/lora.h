/*
 * liblora: mixed-adapter LoRA linear layer for AMD Instinct MI355X (gfx950).
 *
 *   y_i = x_i W^T + (alpha_s / r_s) (x_i A_s^T) B_s^T,   s = slot_ids[i]
 *
 * The base GEMM runs once over every row; each row's slot selects a resident
 * adapter in a fixed device slot pool, and the low-rank correction is
 * applied as a segmented gather shrink (x -> [T, r] fp32) and expand
 * ([T, r] -> y). Row formula: "43. Beyond text: images, embeddings,
 * reranking and many LoRAs" (inference.shantanugoel.com), section "Many
 * adapters, one base-model batch". Slot 0 is the zero adapter (rank 0,
 * scaling 0) that every base-only row addresses and that the kernels skip:
 * "mstar.engine.resources.lora.pool" (mstar.stanford.edu), module text.
 *
 * Conventions for every call:
 *  - Every function returns LORA_OK (0) or a negative LORA_E* status; no C++
 *    exception crosses this interface. lora_status_string() names a status.
 *  - "dev" pointers are HIP device memory, "host" pointers are CPU memory.
 *    The caller owns every buffer passed in; the library keeps only the
 *    small host-side pool handle (plus a 4-byte device status word).
 *  - `stream` is a hipStream_t (NULL = the default stream). Device work is
 *    asynchronous on it unless a call says it synchronises.
 *  - Matrices are row-major and contiguous. Element offsets are computed in
 *    64-bit, so T*d may exceed 2^31 ("Silent: int32 overflow at long
 *    context", "LoRA serving, embeddings, rerankers, pooling",
 *    mlinterviewnotes.com).
 *  - Element type is the pool's: LORA_BF16 (uint16 bf16 bit patterns,
 *    fp32 accumulation, y rounded to nearest even) or LORA_F32.
 *  - A call over T = 0 tokens returns LORA_OK at once, after checking the
 *    pool and plan arguments; its x, W, y and workspace pointers may then be
 *    null.
 *  - Widths are free: T, d_in, d_out and S take any value in range, and
 *    ragged tails are masked (the kernels of "43. Beyond text", section
 *    "Many adapters, one base-model batch", mask them too). bf16 pools whose d_in is a
 *    multiple of 8 run the matrix-core kernels, whose rows are read in
 *    16-byte pieces; fp32 pools and bf16 pools of any other d_in run the
 *    element-generic kernels (scalar loads, fp32 FMA, the expand fused into
 *    the base GEMM's epilogue, one rounding of y).
 */
#ifndef RANK_GEMM_AMD_LORA_H
#define RANK_GEMM_AMD_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LORA_OK 0
#define LORA_EINVAL (-1)     /* null pointer, bad size, plan/pool mismatch */
#define LORA_ESLOT (-2)      /* slot id out of range */
#define LORA_ERANK (-3)      /* rank outside [1, r_max] */
#define LORA_ENONFINITE (-4) /* adapter weights or alpha not finite */
#define LORA_EHIP (-5)       /* a HIP runtime call or kernel launch failed */
#define LORA_ESPACE (-6)     /* a caller buffer is too small */

/* element types */
#define LORA_F32 0
#define LORA_BF16 1

/* rows per work item of the plan (one 16-row matrix-core tile) */
#define LORA_PLAN_ROWS 16

/* largest r_max a pool may have */
#define LORA_MAX_RANK 1024

typedef struct lora_pool lora_pool;

/* Summary of one plan; filled by lora_plan, read by lora_linear. */
typedef struct lora_plan_info {
    int32_t T;       /* tokens in the step */
    int32_t S;       /* slot count the plan was built for */
    int32_t T_a;     /* tokens whose slot is not 0 */
    int32_t k;       /* distinct non-zero slots that have tokens */
    int32_t n_items; /* entries in the work list */
    int32_t max_seg; /* longest non-zero segment, in tokens */
    int32_t chunk;   /* rows per work item at most: LORA_PLAN_ROWS, or the
                        chunk of lora_plan_chunked */
} lora_plan_info;

/*
 * Create a pool handle over caller-owned device buffers and zero every slot.
 * Layout ("stacked" slot buffers padded to a common maximum rank, unused rows
 * of A and columns of B zero: shantanugoel page, "Many adapters, one
 * base-model batch"; mlinterviewnotes page, "vLLM: preallocated stacked
 * buffers ..."):
 *   A_pool    dev [S][r_max][d_in]   pool element type
 *   B_pool    dev [S][d_out][r_max]  pool element type
 *   rank_dev  dev int32 [S]          true rank per slot, 0 = empty
 *   scale_dev dev float [S]          alpha_s / r_s per slot, 0 for empty
 * Slot 0 stays rank 0, scale 0 for the pool's lifetime.
 * Synchronises `stream`. Errors: LORA_EINVAL (S < 2, r_max outside
 * [1, LORA_MAX_RANK], d_in < 1, d_out < 1, unknown dtype, null pointer),
 * LORA_EHIP.
 */
int lora_pool_create(lora_pool** out, int S, int r_max, int d_in, int d_out, int dtype,
                     void* A_pool, void* B_pool, int32_t* rank_dev, float* scale_dev, void* stream);

/* Release the host handle and its status word (not the caller's buffers). */
void lora_pool_destroy(lora_pool* pool);

/*
 * Install an adapter into `slot`:
 *   A dev [r][d_in], B dev [d_out][r] (pool element type), scaling alpha / r
 *   with r the adapter's true rank ("LoRA adapter application at serve
 *   time", voxlang.org, conventions table: "alpha / rank").
 * Validates everything before writing anything (shantanugoel page,
 * AdapterBank.load): slot in [1, S) (slot 0 is never handed out), 1 <= r <=
 * r_max, non-null pointers, alpha and every weight finite. Then copies A into
 * rows 0..r-1 of the slot, zeroes rows r..r_max-1, copies B into columns
 * 0..r-1, zeroes the rest, and sets rank[slot] = r, scale[slot] = alpha / r
 * (computed in fp32). Reinstalling an occupied slot is allowed: work queued
 * earlier on `stream` sees the old weights, later work the new ones; the
 * caller must not let work on another stream read the slot meanwhile.
 * Synchronises `stream` (cold path). Errors: LORA_EINVAL, LORA_ESLOT,
 * LORA_ERANK, LORA_ENONFINITE (pool unchanged), LORA_EHIP.
 */
int lora_pool_install(lora_pool* pool, int slot, const void* A, const void* B, int r, float alpha,
                      void* stream);

/* Reset `slot` (1..S-1) to rank 0, scale 0 and zero weights. Synchronises. */
int lora_pool_clear(lora_pool* pool, int slot, void* stream);

/* Host mirror of a slot's rank (-1 if slot is out of range). */
int lora_pool_rank(const lora_pool* pool, int slot);

/*
 * Per-step segment plan, a pure host function (integer work, bit-exact).
 * It is built once per step and shared by every adapted linear of every
 * layer ("mstar.engine.resources.lora.pool", LoraAddressing and
 * LoraLayerDelta); it holds no weights, so reinstalling a slot does not
 * invalidate it.
 *   slot_ids     host int32 [T], each in [0, S)
 *   token_order  host int32 [T]   out: token indices sorted by (slot, index)
 *   slot_indptr  host int32 [S+1] out: slot_indptr[s] = #tokens with slot < s
 *   work         host int32 [work_cap][4] out: {slot, first sorted position,
 *                row count <= LORA_PLAN_ROWS, 0}, covering every segment of a
 *                slot >= 1 in ascending slot order
 *   info         out
 * Stable counting sort: ascending slot, ascending token index within a slot
 * (the stable sort plus sorted unique of "LoRA serving, embeddings,
 * rerankers, pooling", section "vLLM: preallocated stacked buffers ...").
 * Validates every id before writing any output. Errors: LORA_EINVAL (S < 1,
 * T < 0, null pointer), LORA_ESLOT, LORA_ESPACE (work_cap too small).
 */
int lora_plan(int S, const int32_t* slot_ids, int T, int32_t* token_order, int32_t* slot_indptr,
              int32_t* work, int work_cap, lora_plan_info* info);

/* Upper bound on the work list length of any plan over T tokens, S slots
 * (of any chunk: larger chunks give fewer items). */
int lora_plan_max_items(int T, int S);

/*
 * lora_plan with work items of up to `chunk` rows, chunk in {16, 32, 64,
 * 128}: the chunked SGMV of "LoRA serving, embeddings, rerankers, pooling"
 * (mlinterviewnotes.com), section "SGLang: chunked SGMV, and a rank-aware
 * kernel", where the chunk size trades parallelism on skewed adapter
 * popularity (more, shorter items for a hot adapter) against re-reading the
 * adapter's weights once per item. token_order and slot_indptr do not depend
 * on the chunk; info->chunk records it. lora_plan is this call with
 * chunk = LORA_PLAN_ROWS. lora_linear, lora_linear_multi and lora_shrink
 * take plans of LORA_PLAN_ROWS rows only (their kernels are built on 16-row
 * items); lora_delta takes any chunk. Errors as lora_plan, plus LORA_EINVAL
 * for another chunk.
 */
int lora_plan_chunked(int S, const int32_t* slot_ids, int T, int chunk, int32_t* token_order,
                      int32_t* slot_indptr, int32_t* work, int work_cap, lora_plan_info* info);

/*
 * Copy a plan (or any int32 buffer) from pinned host memory to the device
 * with one kernel on `stream` that reads the host buffer in place over the
 * bus. The plan is rebuilt on the host every step and read by every layer
 * ("LoRA serving, embeddings, rerankers, pooling", mlinterviewnotes.com,
 * worked example in section "LoRA and speculative decoding"); copied this
 * way its upload is ordered on the compute stream like any kernel, instead
 * of waiting for a copy engine between two kernels.
 *   host_plan  host int32 [words], pinned (hipHostMalloc, or torch's
 *              pin_memory); caller-owned; read when the stream reaches this
 *              call, so it must not be rewritten before then (record an
 *              event after the call and wait on it)
 *   dev_plan   dev int32 [words], caller-owned
 * Errors: LORA_EINVAL (null pointers; a host buffer the GPU cannot read,
 * i.e. not pinned), LORA_EHIP. words == 0 launches nothing.
 */
int lora_plan_upload(const int32_t* host_plan, int32_t* dev_plan, size_t words, void* stream);

/*
 * The same plan built on the device, for steps captured in a HIP graph (no
 * host work, no host-to-device copy, no allocation, one kernel). Launch
 * overhead is what drives engines to fixed-size buffers and graph capture
 * ("LoRA serving, embeddings, rerankers, pooling", mlinterviewnotes.com,
 * worked example in section "LoRA and speculative decoding"); the plan's
 * content is that of lora_plan ("mstar.engine.resources.lora.pool",
 * LoraAddressing).
 *   slot_ids  dev int32 [T]
 *   plan      dev int32 [lora_plan_device_words(T, S)], caller-owned, laid out
 *             [work 4 * W][token_order T][slot_indptr S + 1][info 8] with
 *             W = max(lora_plan_max_items(T, S), 1); work, token_order and
 *             slot_indptr are bit-identical to lora_plan's for the same ids,
 *             the work list is padded to W with empty items {0, 0, 0, 0}, and
 *             info holds {T, S, T_a, k, n_items, max_seg, status, 0}
 * 1 <= S <= LORA_DEVICE_PLAN_MAX_SLOTS. An id outside [0, S) cannot be
 * reported at call time: it is planned as slot 0 (base output) and the
 * status word becomes LORA_ESLOT. Asynchronous on `stream`.
 * Errors: LORA_EINVAL (sizes, null pointers), LORA_EHIP.
 */
#define LORA_DEVICE_PLAN_MAX_SLOTS 4096
size_t lora_plan_device_words(int T, int S);
int lora_plan_device(int S, const int32_t* slot_ids, int T, int32_t* plan, void* stream);

/* Device workspace lora_linear and lora_shrink need for T tokens. */
size_t lora_workspace_bytes(const lora_pool* pool, int T);

/*
 * y = x W^T + per-row adapter correction, on `stream`, without host sync.
 *   x            dev [T][d_in]    pool element type
 *   W            dev [d_out][d_in]
 *   token_order, slot_indptr, work: dev copies of lora_plan's outputs
 *   info         host, from the same lora_plan call (info->S == pool S)
 *   y            dev [T][d_out]   out; overwritten completely, so its prior
 *                contents never leak into the result (the uninitialised-output
 *                hazard of "Silent: the wrong adapter, applied correctly",
 *                mlinterviewnotes page)
 *   workspace    dev, at least lora_workspace_bytes(pool, T) bytes (bf16 pools
 *                always need it; fp32 pools only when info->T_a > 0); holds
 *                partial products and the shrink output between kernels, so
 *                calls that may overlap need separate workspaces
 * Then y += delta for adapter rows only (LoraLayerDelta semantics); rows on
 * slot 0 and on rank-0 slots are the base output bit for bit. When
 * info->T_a == 0 no correction kernel is launched. y must not alias x or W.
 * Errors: LORA_EINVAL, LORA_ESPACE, LORA_EHIP (launch failure). A device
 * fault surfaces at the caller's next synchronisation.
 */
int lora_linear(const lora_pool* pool, const void* x, const void* W, const int32_t* token_order,
                const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info, void* y,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_linear over a device plan from lora_plan_device (T tokens, the pool's
 * S): the same kernels, launched for the plan's capacity W, with empty items
 * exiting at once, so the host needs nothing from the plan and a captured
 * graph stays valid for any token-to-slot assignment of T tokens. Rows on
 * slot 0 equal the base output bit for bit, as with lora_linear.
 * Workspace and errors as lora_linear.
 */
int lora_linear_device_plan(const lora_pool* pool, const void* x, const void* W, const int32_t* plan, int T,
                            void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several adapted projections that read the same x (a merged q/k/v or
 * gate/up wrapper), in one call: the "output slices" that one shrink and one
 * expand launch cover in "LoRA serving, embeddings, rerankers, pooling"
 * (mlinterviewnotes.com), section "vLLM: preallocated stacked buffers plus a
 * Punica-style Triton kernel". Each slice has its own base weight, output
 * and adapter pool; all slices share x and the plan, so slot s means the
 * same adapter identity in every slice's pool (each pool may hold its own
 * rank for it).
 *   slices       host [n], 1 <= n <= LORA_MAX_SLICES; every pool has the same
 *                S, r_max, d_in and element type; slice i writes
 *                y_i = x W_i^T + per-row correction from slices[i].pool,
 *                exactly what lora_linear(slices[i].pool, x, W_i, ..., y_i)
 *                defines (to fp32 rounding order for bf16 pools: split points
 *                of K may differ)
 *   x, token_order, slot_indptr, work, info, stream: as lora_linear
 *   workspace    dev, at least lora_workspace_bytes_multi(slices, n, T) bytes
 * With bf16 pools, slices whose concatenated columns fall on the decode
 * (split-K) path are computed by one GEMM launch and one epilogue launch
 * between them, x being read once per K split for all slices; otherwise each
 * slice has its own GEMM launch, and when every slice takes the unsplit tiled
 * path with the expand as extra K steps and the plan has at least 128 work
 * items, one shrink launch serves all slices (x rows read once; each slice's
 * output then equals its own lora_linear call bit for bit). No y may alias
 * x, any W or another y.
 * Errors: LORA_EINVAL (n out of range, pools that differ, null pointer,
 * aliasing), LORA_ESPACE, LORA_EHIP.
 */
#define LORA_MAX_SLICES 4

typedef struct lora_slice {
    const lora_pool* pool; /* adapters of this projection, d_out columns */
    const void* W;         /* dev [pool d_out][d_in] */
    void* y;               /* dev [T][pool d_out] out */
} lora_slice;

/* Device workspace of lora_linear_multi over these pools (slices[i].W and
 * .y are not read); 0 when the pools cannot share a call. */
size_t lora_workspace_bytes_multi(const lora_slice* slices, int n, int T);

/* lora_linear_multi over a device plan from lora_plan_device (T tokens, the
 * pools' S), as lora_linear_device_plan is to lora_linear. */
int lora_linear_multi_device_plan(const lora_slice* slices, int n, const void* x, const int32_t* plan, int T,
                                  void* workspace, size_t workspace_bytes, void* stream);

int lora_linear_multi(const lora_slice* slices, int n, const void* x, const int32_t* token_order,
                      const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The shrink alone, for inspection: h dev fp32 [T][r_max] receives
 * h[t][q] = sum_k x[t,k] A_s[q,k] for q < r_s, and 0 for q >= r_s and for
 * rows on slot 0 or a rank-0 slot (the T x r intermediate of the rank
 * bottleneck, mlinterviewnotes page, opening section). It uses the same per-item
 * shrink code as lora_linear over the whole K range (lora_linear may split K
 * and add the splits, so the two agree to fp32 rounding, not bit for bit).
 * Errors as lora_linear.
 */
int lora_shrink(const lora_pool* pool, const void* x, const int32_t* token_order, const int32_t* slot_indptr,
                const int32_t* work, const lora_plan_info* info, float* h, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * The shrink in BGMV form, for the SGMV / BGMV comparison: the same h as
 * lora_shrink (token order, fp32 [T][r_max], zeros past each row's rank and
 * on slot 0 or rank-0 slots), computed one token at a time from the raw slot
 * map with no grouping and no plan: the batched gather matrix-vector kernel
 * that "LoRA serving, embeddings, rerankers, pooling" (mlinterviewnotes.com)
 * sets against the segmented SGMV, section "SGLang: chunked SGMV, and a
 * rank-aware kernel". Each token reads its slot's A_s; SGMV reads A_s once
 * per item of up to 16 tokens.
 *   slot_ids  dev int32 [T]; ids outside [1, S) give zero rows
 *   workspace dev, at least lora_workspace_bytes(pool, T) bytes
 * bf16 pools whose d_in is a multiple of 8 only. Errors: LORA_EINVAL (fp32
 * pool, d_in % 8 != 0, null pointer), LORA_ESPACE, LORA_EHIP.
 */
int lora_shrink_bgmv(const lora_pool* pool, const void* x, const int32_t* slot_ids, int T, float* h,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The correction alone, for callers that compute the base product
 * themselves: y += delta(x), the LoraLayerDelta contract of
 * "mstar.engine.resources.lora.pool" (mstar.stanford.edu):
 *   y[t][n] = round(y[t][n] + (alpha_s / r_s) sum_q h[t][q] B_s[n][q]),
 *   h[t][q] = sum_k x[t][k] A_s[q][k]
 * for every token t whose slot s is >= 1 with r_s > 0; other rows of y are
 * not touched. fp32 accumulation, one rounding of each updated element (so a
 * bf16 y that already held a rounded base output is rounded twice in all).
 *   x            dev [T][d_in], y dev [T][d_out] (in place; must not alias x)
 *   token_order, slot_indptr, work, info: a plan of any chunk (lora_plan or
 *                lora_plan_chunked), on the device as for lora_linear
 *   workspace    dev, at least lora_workspace_bytes(pool, T) bytes
 * SGMV form: per work item, its rows of x are shrunk against A_s (read once
 * per item), then B_s is read once per item and column block and applied to
 * every row of the item. Asynchronous on `stream`. Errors: LORA_EINVAL
 * (null pointer, plan/pool mismatch, a chunk outside {16, 32, 64, 128}),
 * LORA_ESPACE, LORA_EHIP.
 */
int lora_delta(const lora_pool* pool, const void* x, const int32_t* token_order, const int32_t* slot_indptr,
               const int32_t* work, const lora_plan_info* info, void* y, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * The same correction in BGMV form: token by token from the raw slot map,
 * with no grouping and no plan; each token reads its own slot's A_s and B_s
 * (the batched gather matrix-vector kernel that "43. Beyond text: images,
 * embeddings, reranking and many LoRAs" (inference.shantanugoel.com), section
 * "Many adapters, one base-model batch", uses for both the shrink and the
 * expand).
 *   slot_ids  dev int32 [T]; ids outside [1, S) and rank-0 slots leave their
 *             row of y unchanged
 * bf16 pools whose d_in is a multiple of 8 only. Errors: LORA_EINVAL (other
 * pools, null pointer, y aliasing x), LORA_ESPACE, LORA_EHIP.
 */
int lora_delta_bgmv(const lora_pool* pool, const void* x, const int32_t* slot_ids, int T, void* y, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * lora_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of lora_linear, without the
 * workspace: the kernels use a device array inside the library instead, of
 * LORA_NOALLOC_MAX_WORKSPACE bytes, one per GPU, held from the first call on
 * that GPU until the process ends. The call allocates and frees nothing. It
 * runs on the current device (`stream` must belong to it). A call whose
 * lora_workspace_bytes(pool, info->T) exceeds LORA_NOALLOC_MAX_WORKSPACE
 * returns LORA_ESPACE and launches nothing. All calls on one GPU share that
 * GPU's array: calls that may overlap on one GPU (two streams, two threads)
 * race on it, so overlapping callers must use lora_linear with separate
 * workspaces. The array keeps the last call's contents; no kernel depends on
 * it starting at zero.
 */
#define LORA_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
int lora_linear_noalloc(const lora_pool* pool, const void* x, const void* W, const int32_t* token_order,
                        const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info, void* y,
                        void* stream);

/*
 * Per-kernel timing, for diagnostics and the benchmark's roofline figures.
 * Between lora_profile_begin and lora_profile_end, lora_linear,
 * lora_linear_multi and lora_shrink record a HIP event pair around every
 * kernel they launch, on the stream it is launched on (not while that stream
 * is being captured into a graph, and at most max_records kernels).
 * lora_profile_end waits for the recorded events and writes one entry per
 * kernel name, in first-launch order, into out[0..cap): count, mean, min,
 * max and median duration; *n_out receives the number of names. Profiling
 * serialises the calls across threads while it is on.
 * Errors: LORA_EINVAL (begin while on, end while off, max_records < 8),
 * LORA_ESPACE (more names than cap), LORA_EHIP.
 */
typedef struct lora_kernel_stat {
    char name[48];
    int32_t count;
    double mean_ms, min_ms, max_ms, median_ms;
} lora_kernel_stat;

int lora_profile_begin(int max_records);
int lora_profile_end(lora_kernel_stat* out, int cap, int* n_out);

/* Human-readable name of a status code (static storage). */
const char* lora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RANK_GEMM_AMD_LORA_H */
