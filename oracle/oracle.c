/*
 * CPU oracle for the mixed-adapter LoRA linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header or constant with the HIP
 * library it checks.
 *
 * Everything is computed in IEEE double from the exact input values (fp32
 * inputs widen exactly; bf16 inputs are decoded here as bits << 16). Loops
 * are plain and in the order the formulas are written; the only parallelism
 * is OpenMP over independent output rows, which does not change any sum.
 *
 * Sources:
 *  - Row formula: "43. Beyond text: images, embeddings, reranking and many
 *    LoRAs" (inference.shantanugoel.com), section "Many adapters, one
 *    base-model batch", displayed equation
 *        y_i = W x_i + (alpha_{s_i} / r_{s_i}) B_{s_i} (A_{s_i} x_i),
 *    with W [d_out, d_in], A_s [r_s, d_in], B_s [d_out, r_s] as stored in
 *    "LoRA serving, embeddings, rerankers, pooling" (mlinterviewnotes.com),
 *    opening section, and scaling alpha / rank as in the conventions table of
 *    "LoRA adapter application at serve time" (voxlang.org).
 *  - Slot 0 is the zero adapter (rank 0, scaling 0): the class description of
 *    "mstar.engine.resources.lora.pool" (mstar.stanford.edu). Rows on it get
 *    exactly the base output.
 *  - Merged form W' = W + (alpha/r) B A: the opening section of the
 *    mlinterviewnotes page and the "Delta" row of the voxlang table.
 *  - Grouped form (group rows by slot, shrink, expand, scatter): the
 *    grouped_lora reference of the same section of the shantanugoel page.
 *
 * Adapter storage used by this oracle (not the GPU pool's layout): A_cat is
 * the concatenation over s = 0..S-1 of A_s [rank[s]][d_in] (row-major),
 * B_cat the concatenation of B_s [d_out][rank[s]] (row-major).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };

static double decode_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void* p, int dtype, int64_t i) {
    if (dtype == OR_BF16) return decode_bf16(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16(in[i]);
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* element offsets of slot s's A and B inside A_cat / B_cat */
static void slot_offsets(int S, const int32_t* rank, int d_in, int d_out, int64_t* a_off, int64_t* b_off) {
    int64_t a = 0, b = 0;
    for (int s = 0; s < S; ++s) {
        a_off[s] = a;
        b_off[s] = b;
        a += (int64_t)rank[s] * d_in;
        b += (int64_t)d_out * rank[s];
    }
}

/*
 * Per-row unmerged formula. Computes the requested rows (rows == NULL: all
 * T rows in order) into y_out[n][d_out]. If h_out is not NULL it also
 * receives h_i[q] = sum_k x[i,k] A_s[q,k] for q < rank[s] (zeros elsewhere
 * and for rows on slot 0), with row stride h_stride. If base_out is not
 * NULL it also receives the base term sum_k W[j,k] x[i,k] of every element,
 * the same value y_out starts from, so a caller that needs both the layer
 * and the base output pays for one pass over W.
 * Returns 0, or -1 for a slot id outside [0, S).
 */
int oracle_lora_rows(int dtype, int T, int d_in, int d_out, int S,
                     const void* x, const void* W,
                     const int32_t* rank, const double* alpha,
                     const void* A_cat, const void* B_cat,
                     const int32_t* slot_ids,
                     int n_rows, const int32_t* rows,
                     double* y_out, double* h_out, int h_stride, double* base_out) {
    int64_t* a_off = (int64_t*)malloc(sizeof(int64_t) * S);
    int64_t* b_off = (int64_t*)malloc(sizeof(int64_t) * S);
    slot_offsets(S, rank, d_in, d_out, a_off, b_off);
    int n = rows ? n_rows : T;
    int bad = 0;
    for (int n_i = 0; n_i < n; ++n_i) {
        int i = rows ? rows[n_i] : n_i;
        if (i < 0 || i >= T || slot_ids[i] < 0 || slot_ids[i] >= S) bad = 1;
    }
    if (bad) {
        free(a_off);
        free(b_off);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int n_i = 0; n_i < n; ++n_i) {
        int i = rows ? rows[n_i] : n_i;
        int s = slot_ids[i];
        int r = rank[s];
        double* xi = (double*)malloc(sizeof(double) * d_in);
        double* h = (double*)malloc(sizeof(double) * (r > 0 ? r : 1));
        for (int k = 0; k < d_in; ++k) xi[k] = elem(x, dtype, (int64_t)i * d_in + k);
        /* shrink: h = A_s x_i */
        int adapted = (s != 0 && r > 0);
        if (adapted) {
            for (int q = 0; q < r; ++q) {
                double acc = 0.0;
                for (int k = 0; k < d_in; ++k) acc += elem(A_cat, dtype, a_off[s] + (int64_t)q * d_in + k) * xi[k];
                h[q] = acc;
            }
        }
        double scale = adapted ? alpha[s] / (double)r : 0.0;
        for (int j = 0; j < d_out; ++j) {
            double base = 0.0;
            for (int k = 0; k < d_in; ++k) base += elem(W, dtype, (int64_t)j * d_in + k) * xi[k];
            double y = base;
            if (adapted) {
                double e = 0.0;
                for (int q = 0; q < r; ++q) e += elem(B_cat, dtype, b_off[s] + (int64_t)j * r + q) * h[q];
                y = base + scale * e;
            }
            y_out[(int64_t)n_i * d_out + j] = y;
            if (base_out) base_out[(int64_t)n_i * d_out + j] = base;
        }
        if (h_out) {
            double* hr = h_out + (int64_t)n_i * h_stride;
            for (int q = 0; q < h_stride; ++q) hr[q] = (adapted && q < r) ? h[q] : 0.0;
        }
        free(xi);
        free(h);
    }
    free(a_off);
    free(b_off);
    return 0;
}

/*
 * Merged form: for each row, W' = W + (alpha_s / r_s) B_s A_s is formed
 * element by element and y_i = W' x_i. Meant for tiny shapes only (it
 * rebuilds W' for every row).
 */
int oracle_lora_merged(int dtype, int T, int d_in, int d_out, int S,
                       const void* x, const void* W,
                       const int32_t* rank, const double* alpha,
                       const void* A_cat, const void* B_cat,
                       const int32_t* slot_ids, double* y_out) {
    int64_t* a_off = (int64_t*)malloc(sizeof(int64_t) * S);
    int64_t* b_off = (int64_t*)malloc(sizeof(int64_t) * S);
    slot_offsets(S, rank, d_in, d_out, a_off, b_off);
    double* wp = (double*)malloc(sizeof(double) * (size_t)d_out * d_in);
    for (int i = 0; i < T; ++i) {
        int s = slot_ids[i];
        if (s < 0 || s >= S) {
            free(wp);
            free(a_off);
            free(b_off);
            return -1;
        }
        int r = rank[s];
        double scale = (s != 0 && r > 0) ? alpha[s] / (double)r : 0.0;
        for (int j = 0; j < d_out; ++j)
            for (int k = 0; k < d_in; ++k) {
                double ba = 0.0;
                if (s != 0)
                    for (int q = 0; q < r; ++q)
                        ba += elem(B_cat, dtype, b_off[s] + (int64_t)j * r + q) *
                              elem(A_cat, dtype, a_off[s] + (int64_t)q * d_in + k);
                wp[(int64_t)j * d_in + k] = elem(W, dtype, (int64_t)j * d_in + k) + scale * ba;
            }
        for (int j = 0; j < d_out; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d_in; ++k) acc += wp[(int64_t)j * d_in + k] * elem(x, dtype, (int64_t)i * d_in + k);
            y_out[(int64_t)i * d_out + j] = acc;
        }
    }
    free(wp);
    free(a_off);
    free(b_off);
    return 0;
}

/*
 * Grouped form: the base projection over all rows once, then for each slot
 * the rows that select it are gathered, shrunk to [n, r_s], expanded to
 * [n, d_out], scaled and added back in place.
 */
int oracle_lora_grouped(int dtype, int T, int d_in, int d_out, int S,
                        const void* x, const void* W,
                        const int32_t* rank, const double* alpha,
                        const void* A_cat, const void* B_cat,
                        const int32_t* slot_ids, double* y_out) {
    for (int i = 0; i < T; ++i)
        if (slot_ids[i] < 0 || slot_ids[i] >= S) return -1;
    int64_t* a_off = (int64_t*)malloc(sizeof(int64_t) * S);
    int64_t* b_off = (int64_t*)malloc(sizeof(int64_t) * S);
    slot_offsets(S, rank, d_in, d_out, a_off, b_off);
    /* base, all rows */
    for (int i = 0; i < T; ++i)
        for (int j = 0; j < d_out; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d_in; ++k)
                acc += elem(x, dtype, (int64_t)i * d_in + k) * elem(W, dtype, (int64_t)j * d_in + k);
            y_out[(int64_t)i * d_out + j] = acc;
        }
    int* grp = (int*)malloc(sizeof(int) * (T > 0 ? T : 1));
    for (int s = 1; s < S; ++s) {
        int r = rank[s];
        if (r == 0) continue;
        int n = 0;
        for (int i = 0; i < T; ++i)
            if (slot_ids[i] == s) grp[n++] = i;
        if (n == 0) continue;
        double* hh = (double*)malloc(sizeof(double) * (size_t)n * r);
        for (int g = 0; g < n; ++g)
            for (int q = 0; q < r; ++q) {
                double acc = 0.0;
                for (int k = 0; k < d_in; ++k)
                    acc += elem(x, dtype, (int64_t)grp[g] * d_in + k) * elem(A_cat, dtype, a_off[s] + (int64_t)q * d_in + k);
                hh[(int64_t)g * r + q] = acc;
            }
        double scale = alpha[s] / (double)r;
        for (int g = 0; g < n; ++g)
            for (int j = 0; j < d_out; ++j) {
                double acc = 0.0;
                for (int q = 0; q < r; ++q) acc += hh[(int64_t)g * r + q] * elem(B_cat, dtype, b_off[s] + (int64_t)j * r + q);
                y_out[(int64_t)grp[g] * d_out + j] += scale * acc;
            }
        free(hh);
    }
    free(grp);
    free(a_off);
    free(b_off);
    return 0;
}
