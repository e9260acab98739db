// Host segment planner: stable counting sort of the per-token slot map.
//
// "LoRA serving, embeddings, rerankers, pooling" (mlinterviewnotes.com),
// section "vLLM: preallocated stacked buffers ...": the kernel metadata is a
// stable sort of the token -> slot map plus a sorted unique with counts,
// rebuilt every forward pass. Here it is one O(T + S) counting sort:
// histogram, exclusive scan, stable scatter. Slot 0 (the zero adapter of
// "mstar.engine.resources.lora.pool") replaces the page's -1 base marker,
// and slot_indptr covers every slot in CSR form (LoraAddressing).
#include <vector>

#include "../../include/lora.h"

extern "C" int lora_plan_max_items(int T, int S) {
    if (T <= 0 || S <= 1) return 0;
    // sum_s ceil(n_s / R) <= T / R + (number of non-empty segments)
    const int segs = T < S - 1 ? T : S - 1;
    return T / LORA_PLAN_ROWS + segs;
}

extern "C" int lora_plan_chunked(int S, const int32_t* slot_ids, int T, int chunk, int32_t* token_order,
                                 int32_t* slot_indptr, int32_t* work, int work_cap, lora_plan_info* info) {
    if (S < 1 || T < 0 || !slot_indptr || !info || (T > 0 && (!slot_ids || !token_order))) return LORA_EINVAL;
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return LORA_EINVAL;
    for (int t = 0; t < T; ++t)
        if (slot_ids[t] < 0 || slot_ids[t] >= S) return LORA_ESLOT;

    std::vector<int32_t> count(S, 0);
    for (int t = 0; t < T; ++t) ++count[slot_ids[t]];
    int n_items = 0, k = 0, max_seg = 0;
    for (int s = 1; s < S; ++s) {
        if (count[s] == 0) continue;
        ++k;
        n_items += (count[s] + chunk - 1) / chunk;
        if (count[s] > max_seg) max_seg = count[s];
    }
    if (n_items > 0 && (!work || work_cap < n_items)) return LORA_ESPACE;

    // exclusive scan -> CSR offsets
    slot_indptr[0] = 0;
    for (int s = 0; s < S; ++s) slot_indptr[s + 1] = slot_indptr[s] + count[s];
    // stable scatter: tokens visited in index order
    std::vector<int32_t> next(slot_indptr, slot_indptr + S);
    for (int t = 0; t < T; ++t) token_order[next[slot_ids[t]]++] = t;

    int i = 0;
    for (int s = 1; s < S; ++s)
        for (int p = slot_indptr[s]; p < slot_indptr[s + 1]; p += chunk) {
            const int left = slot_indptr[s + 1] - p;
            work[4 * i + 0] = s;
            work[4 * i + 1] = p;
            work[4 * i + 2] = left < chunk ? left : chunk;
            work[4 * i + 3] = 0;
            ++i;
        }
    info->T = T;
    info->S = S;
    info->T_a = T - count[0];
    info->k = k;
    info->n_items = n_items;
    info->max_seg = max_seg;
    info->chunk = chunk;
    return LORA_OK;
}

extern "C" int lora_plan(int S, const int32_t* slot_ids, int T, int32_t* token_order, int32_t* slot_indptr,
                         int32_t* work, int work_cap, lora_plan_info* info) {
    return lora_plan_chunked(S, slot_ids, T, LORA_PLAN_ROWS, token_order, slot_indptr, work, work_cap, info);
}
