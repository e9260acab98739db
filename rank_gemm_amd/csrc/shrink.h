// The SGMV shrink of one work item over one K range, shared by the standalone
// shrink kernel and the shrink workgroups of the split-K decode kernel.
//
// An item is <= 16 rows of one slot's segment (sorted positions begin ..
// begin + count); its rows of x are gathered through token_order and
// multiplied by the slot's A, giving the narrow T x r intermediate of the
// rank bottleneck (opening section of "LoRA serving, embeddings, rerankers,
// pooling", mlinterviewnotes.com):
//   out[p][q] = sum_{k in [kbeg, kend)} x[t_p, k] A_s[q, k],   q < r_s
// Rows q >= r_s of A are never loaded (rank masking, "SGLang: chunked SGMV,
// and a rank-aware kernel"). The WAVES waves split the K range; their
// partial sums are added in wave order through LDS (deterministic).
#pragma once

#include <type_traits>

#include "common.h"

namespace lora {

struct Item {
    int slot, begin, count, pad;
};

// Output of the shrink: fp32 h, or the operand of the expand as the GEMM's
// extra K steps: scale_s * h split into bf16 hi and lo halves,
// ext[p][0][q] = hi, ext[p][1][q] = lo, rows of 2 * rp elements.
struct ShrinkOut {
    float* h;          // [T][r_max] fp32 (when ext is null), row p - row0
    uint16_t* ext;     // [T][2][rp] bf16 bits
    int rp;            // r_max rounded up to 8
    float scale;       // scale_s of the item's slot (ext only)
    int row0 = 0;      // sorted position of h's first row
};

// red: LDS scratch of WAVES * 4 * 64 f32x4. Must be called by every thread of
// the workgroup (it synchronises).
template <int WAVES>
__device__ __forceinline__ void shrink_item(const uint16_t* __restrict__ X, const uint16_t* __restrict__ A_pool,
                                            int r, const int32_t* __restrict__ token_order, const Item& it,
                                            const ShrinkOut& out, int K, int kbeg, int kend, int r_max,
                                            f32x4* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, kg = lane >> 4;
    const bool valid = row < it.count;
    const uint16_t* xp = X + (int64_t)token_order[it.begin + (valid ? row : 0)] * K;
    const uint16_t* ap = A_pool + (int64_t)it.slot * r_max * K;
    const int steps = (kend - kbeg + 31) >> 5;
    const int per = (steps + WAVES - 1) / WAVES;
    const int s_beg = wave * per, s_end = min(steps, s_beg + per);
    const int nq = (r + 15) >> 4;

    // Every load is issued (masked-off ones read zeros: or_zero), so a round
    // of loads is in flight together; a load under a branch is waited on
    // inside it. The number of 16-rank blocks in a group is a compile-time
    // constant (NB).
    for (int g0 = 0; g0 < nq; g0 += 4) {  // groups of 64 ranks
        f32x4 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto run = [&](auto nb_tag) {
            constexpr int NB = decltype(nb_tag)::value;
            const uint16_t* aq[NB];
            bool qok[NB];
#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
                const int q = (g0 + qb) * 16 + row;
                qok[qb] = q < r;
                aq[qb] = ap + (int64_t)q * K;
            }
            constexpr int U = 4;
            for (int s0 = s_beg; s0 < s_end; s0 += U) {
                u32x4 a[U], b[U][NB];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int kk = kbeg + (s0 + u) * 32 + kg * 8;
                    const bool kin = (s0 + u) < s_end && kk < kend;
                    a[u] = *or_zero(valid && kin, xp + kk);
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) b[u][qb] = *or_zero(kin && qok[qb], aq[qb] + kk);
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) acc[qb] = mfma16x16x32(a[u], b[u][qb], acc[qb]);
            }
        };
        switch (min(nq - g0, 4)) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
        __syncthreads();  // red is reused across rank groups
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) red[(wave * 4 + qb) * 64 + lane] = acc[qb];
        __syncthreads();
        // wave w finishes rank block g0 + w; lane holds rows 4 kg + e, column row
        if (wave < 4 && g0 + wave < nq) {
            f32x4 s = red[wave * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) s += red[(w * 4 + wave) * 64 + lane];
            const int q = (g0 + wave) * 16 + row;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = kg * 4 + e;
                if (m >= it.count) continue;
                const int64_t p = it.begin + m;
                if (out.ext) {
                    if (q < out.rp) {
                        const float v = s[e] * out.scale;
                        const uint16_t hi = f32_to_bf16(v);
                        out.ext[(p * 2) * out.rp + q] = hi;
                        out.ext[(p * 2 + 1) * out.rp + q] = f32_to_bf16(v - bf16_to_f32(hi));
                    }
                } else if (q < r_max) {
                    out.h[(p - out.row0) * r_max + q] = s[e];
                }
            }
        }
    }
}

// The expand operands of several projections that read the same x (the
// output slices of a merged gate/up or q/k/v, section "vLLM: preallocated
// stacked buffers plus a Punica-style Triton kernel" of the page above): one
// pass over the item's x rows feeds every slice's A rows. The 16-rank blocks
// of all slices are taken in slice order, four at a time, each with its own
// slice's A, rank mask, scale and output; a block's arithmetic is that of
// shrink_item's, so each slice's operand is the same bit for bit.
constexpr int kShrinkMaxSlices = 4;
struct ShrinkSlices {
    int n;
    const uint16_t* A_pool[kShrinkMaxSlices];
    const int32_t* rank[kShrinkMaxSlices];
    const float* scale[kShrinkMaxSlices];
    uint16_t* ext[kShrinkMaxSlices];  // [T][2][rp] each
};

template <int WAVES>
__device__ __forceinline__ void shrink_item_slices(const uint16_t* __restrict__ X, const ShrinkSlices& ss,
                                                   const int32_t* __restrict__ token_order, const Item& it, int K,
                                                   int r_max, f32x4* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, kg = lane >> 4;
    const bool valid = row < it.count;
    const uint16_t* xp = X + (int64_t)token_order[it.begin + (valid ? row : 0)] * K;
    const int rp = (r_max + 7) & ~7;
    const int steps = (K + 31) >> 5;
    const int per = (steps + WAVES - 1) / WAVES;
    const int s_beg = wave * per, s_end = min(steps, s_beg + per);
    // rank blocks per slice (uniform) and their running total
    int nq[kShrinkMaxSlices], rs[kShrinkMaxSlices], total = 0;
#pragma unroll
    for (int i = 0; i < kShrinkMaxSlices; ++i) {
        rs[i] = i < ss.n ? ss.rank[i][it.slot] : 0;
        nq[i] = (rs[i] + 15) >> 4;
        total += nq[i];
    }
    // global block b -> (slice, first rank of the block)
    auto block_of = [&](int b, int& sl, int& q0) {
        sl = 0;
        q0 = 0;
        int first = 0;
#pragma unroll
        for (int i = 0; i < kShrinkMaxSlices; ++i) {
            if (b >= first && b < first + nq[i]) {
                sl = i;
                q0 = (b - first) * 16;
            }
            first += nq[i];
        }
    };
    for (int g0 = 0; g0 < total; g0 += 4) {
        f32x4 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto run = [&](auto nb_tag) {
            constexpr int NB = decltype(nb_tag)::value;
            const uint16_t* aq[NB];
            bool qok[NB];
#pragma unroll
            for (int qb = 0; qb < NB; ++qb) {
                int sl, q0;
                block_of(g0 + qb, sl, q0);
                const int q = q0 + row;
                qok[qb] = q < rs[sl];
                aq[qb] = ss.A_pool[sl] + ((int64_t)it.slot * r_max + (qok[qb] ? q : 0)) * K;
            }
            // 8 rounds of 32 k in flight per wave (shrink_item keeps 4: it
            // also runs beside the decode GEMM blocks, which more loads in
            // flight slow down); the k order of every sum is the same
            constexpr int U = 8;
            for (int s0 = s_beg; s0 < s_end; s0 += U) {
                u32x4 a[U], b[U][NB];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int kk = (s0 + u) * 32 + kg * 8;
                    const bool kin = (s0 + u) < s_end && kk < K;
                    a[u] = *or_zero(valid && kin, xp + kk);
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) b[u][qb] = *or_zero(kin && qok[qb], aq[qb] + kk);
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) acc[qb] = mfma16x16x32(a[u], b[u][qb], acc[qb]);
            }
        };
        switch (min(total - g0, 4)) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
        }
        __syncthreads();  // red is reused across block groups
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) red[(wave * 4 + qb) * 64 + lane] = acc[qb];
        __syncthreads();
        // wave w finishes block g0 + w; lane holds rows 4 kg + e, column row
        if (wave < 4 && g0 + wave < total) {
            f32x4 v4 = red[wave * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) v4 += red[(w * 4 + wave) * 64 + lane];
            int sl, q0;
            block_of(g0 + wave, sl, q0);
            const int q = q0 + row;
            const float sc = ss.scale[sl][it.slot];
            uint16_t* ext = ss.ext[sl];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = kg * 4 + e;
                if (m >= it.count || q >= rp) continue;
                const int64_t p = it.begin + m;
                const float v = v4[e] * sc;
                const uint16_t hi = f32_to_bf16(v);
                ext[(p * 2) * rp + q] = hi;
                ext[(p * 2 + 1) * rp + q] = f32_to_bf16(v - bf16_to_f32(hi));
            }
        }
    }
}

}  // namespace lora
