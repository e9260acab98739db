// Base GEMM of the LoRA linear on gfx950 matrix cores, with the SGMV expand
// fused into its epilogue:
//   y[t_p] = bf16( x[t_p] W^T + scale_s * h[p] B_s^T )   for sorted position p
// where t_p = token_order[p] and s is the slot whose segment holds p. The base
// product is the plain GEMM of "LoRA serving, embeddings, rerankers, pooling"
// (mlinterviewnotes.com, opening section: base GEMM once over the batch, then
// the per-row indexed low-rank correction); doing the correction in the
// epilogue writes y once instead of re-reading it.
//
// Rows are visited in plan (segment) order, so a 16-row block meets few
// slots: each slot met adds one more rank-deep product per block, with h
// (fp32, from the shrink) fed to the matrix cores as bf16 hi + lo halves.
// Rows on slot 0, or on a rank-0 slot, get no product at all, so their bits
// equal those of a run with no adapter row.
//
// Two paths:
//  * tiled (prefill-sized T): 256 x 256 macro tiles over 8 waves with K in
//    stages of 32 through a 3-deep LDS ring filled by direct-to-LDS loads
//    (128 x 128 and 64 x 128 tiles with 4 waves and register-staged loads for
//    smaller T); the shrink runs before it as its own kernel.
//  * split-K (decode-sized T): kernel 1 computes 64 x 64 output tiles over K
//    splits, streaming the split's gathered x rows and W rows through a
//    5-deep LDS ring of 64-k stages by direct-to-LDS loads; extra workgroups
//    of the same launch compute the shrink over the same K splits. Kernel 2
//    adds the partial products in split order, applies the expand and rounds
//    once. No workgroup waits on another.
#include "common.h"
#include "kernels.h"
#include "shrink.h"

#include <type_traits>

namespace lora {

constexpr int kBK = 64;
constexpr int kThreads = 256;

struct Fuse {
    const int32_t* token_order;  // sorted position -> token row
    const int32_t* slot_indptr;  // [S+1]
    const float* h;              // h_splits planes of [T][r_max], sorted positions, unscaled
    const uint16_t* B_pool;      // [S][N][r_max]
    const int32_t* rank;
    const float* scale;
    int S, r_max;
    int h_splits;     // planes of h to add (1 when the shrink produced final h)
    int64_t h_plane;  // elements per plane
    int adapters;     // 0: no adapter row in the batch, skip the correction
    const uint16_t* ext;  // tiled path: scaled h as bf16 hi / lo rows [T][2][rp], or null
    int rp;               // r_max rounded up to 8
};

// Slot metadata (segment offsets, ranks, scales) staged in LDS at kernel
// start, so the epilogue's slot walk does not chain global-memory latencies.
// Pools with more than kMetaSlots slots read it from global memory instead.
constexpr int kMetaSlots = 1024;
struct SlotMeta {
    int indptr[kMetaSlots + 1];
    int rank[kMetaSlots];
    float scale[kMetaSlots];
};

struct MetaView {
    const int* indptr;
    const int* rank;
    const float* scale;
};

// Cooperative copy by every thread of the block; call before a barrier.
__device__ __forceinline__ MetaView stage_meta(const Fuse& f, SlotMeta* sm) {
    if (!f.adapters || f.S > kMetaSlots) return MetaView{f.slot_indptr, f.rank, f.scale};
    for (int i = threadIdx.x; i <= f.S; i += blockDim.x) {
        sm->indptr[i] = f.slot_indptr[i];
        if (i < f.S) {
            sm->rank[i] = f.rank[i];
            sm->scale[i] = f.scale[i];
        }
    }
    return MetaView{sm->indptr, sm->rank, sm->scale};
}

// 16-byte LDS chunk of (row, logical chunk c in 0..7). The XOR spreads the
// 16 rows one MFMA operand read touches over distinct banks.
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

// Last slot s with slot_indptr[s] <= p (the slot whose segment holds p).
__device__ __forceinline__ int slot_of(const int* indptr, int S, int p) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (indptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// acc[i][j] covers sorted rows p0 + 16 i + (4 (lane/16) + e) and columns
// n0 + 16 j + lane % 16. Adds scale_s * h[p] . B_s[n] for every adapter row.
template <int FM, int FN>
__device__ __forceinline__ void fused_expand(f32x4 (&acc)[FM][FN], const Fuse& f, const MetaView& mv, int p0,
                                             int n0, int M, int N, int lane) {
    const int pend = min(M, p0 + FM * 16);
    if (!f.adapters || p0 >= pend) return;
    const int col = lane & 15, qg = lane >> 4;
    const bool vec = (f.r_max & 3) == 0;
    for (int s = slot_of(mv.indptr, f.S, p0); s < f.S; ++s) {
        const int sb = mv.indptr[s], se = mv.indptr[s + 1];
        if (sb >= pend) break;
        const int r = mv.rank[s];
        if (s == 0 || r == 0 || se <= p0 || se <= sb) continue;
        const float sc = mv.scale[s];
        const uint16_t* bs = f.B_pool + (int64_t)s * N * f.r_max;
        const int nq = (r + 15) >> 4;
        for (int qs = 0; qs < nq; ++qs) {
            const int q = qs * 16 + qg * 4;
            u32x2 bfr[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + j * 16 + col;
                const uint16_t* src = bs + (int64_t)n * f.r_max + q;
                if (vec) {  // B is zero past r inside the padded row
                    bfr[j] = (n < N && q < r) ? *(const u32x2*)src : u32x2{0, 0};
                } else {
                    uint16_t e4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) e4[e] = (n < N && q + e < r) ? src[e] : uint16_t(0);
                    bfr[j] = u32x2{uint32_t(e4[0]) | (uint32_t(e4[1]) << 16),
                                   uint32_t(e4[2]) | (uint32_t(e4[3]) << 16)};
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int bb = p0 + i * 16;
                if (bb >= se || bb + 16 <= sb) continue;  // block outside the segment (uniform)
                const int p = bb + col;                   // this lane's row of the A operand
                const bool in = p >= sb && p < se;
                float hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = 0.f;
                    if (in && q + e < r) {
                        const float* hp = f.h + (int64_t)p * f.r_max + q + e;
                        for (int z = 0; z < f.h_splits; ++z) v += hp[z * f.h_plane];
                        v *= sc;
                    }
                    hi[e] = bf16_to_f32(f32_to_bf16(v));
                    lo[e] = v - hi[e];
                }
                const u32x2 ahi{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
                const u32x2 alo{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    acc[i][j] = mfma16x16x16(ahi, bfr[j], acc[i][j]);
                    acc[i][j] = mfma16x16x16(alo, bfr[j], acc[i][j]);
                }
            }
        }
    }
}

// Round and store: y[token_order[p]][n] for the rows and columns of acc.
template <int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[FM][FN], uint16_t* __restrict__ Y,
                                           const int32_t* __restrict__ token_order, int p0, int n0, int M, int N,
                                           int lane) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = p0 + i * 16 + (lane >> 4) * 4 + e;
            if (p >= M) continue;
            uint16_t* yr = Y + (int64_t)token_order[p] * N;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + j * 16 + (lane & 15);
                if (n < N) yr[n] = f32_to_bf16(acc[i][j][e]);
            }
        }
}

// Map a linear block id to (tile_m, tile_n). Consecutive ids go round-robin
// over the 8 XCDs, so ids are first regrouped so that each XCD owns one
// contiguous run of tiles; inside a run tiles are ordered in groups of 8
// tile-rows so that concurrently running tiles share x rows and W rows in
// that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int nt = tiles_m * tiles_n;
    int t = bid;
    if ((nt & 7) == 0) t = (bid & 7) * (nt >> 3) + (bid >> 3);
    constexpr int G = 8;
    const int per_group = G * tiles_n;
    const int g = t / per_group;
    const int first = g * G;
    const int gsize = min(tiles_m - first, G);
    const int in = t - g * per_group;
    tm = first + in % gsize;
    tn = in / gsize;
}

// The expand as extra K steps of the tiled GEMM. For each slot s whose
// segment meets the tile's rows [m0, mend) the K dimension is extended by
// 2 rp (rp = r_max rounded up to 8): the A operand of row p is its ext row
// [bf16 hi of scale_s h | lo remainder] (zero for rows of other segments),
// the B operand of column n is [B_s[n] | B_s[n]], so the products add
// scale_s h . B_s. The extension is walked in steps of 64 (or 32).
struct ExtraStep {
    int s, sb, se, r, t;
};

// Number of extra steps of `step` k (e < 0) or the decoding of step e.
__device__ __forceinline__ int extra_steps(const MetaView& mv, const Fuse& f, int m0, int mend, int e,
                                           ExtraStep* out, int step = 64) {
    int n = 0;
    for (int s = slot_of(mv.indptr, f.S, m0); s < f.S; ++s) {
        const int sb = mv.indptr[s], se = mv.indptr[s + 1];
        if (sb >= mend) break;
        const int r = mv.rank[s];
        if (s == 0 || r == 0 || se <= m0 || se <= sb) continue;
        const int k = (2 * f.rp + step - 1) / step;
        if (e >= 0 && e < n + k) {
            *out = ExtraStep{s, sb, se, r, e - n};
            return e;
        }
        n += k;
    }
    return n;
}

// ------------------------------------------------------------------ tiled --
template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(const uint16_t* __restrict__ X,
                                                                 const uint16_t* __restrict__ W,
                                                                 uint16_t* __restrict__ Y, int M, int N, int K,
                                                                 int tiles_m, int tiles_n, Fuse f) {
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int AC = BM * 8 / kThreads;  // 16-byte chunks per thread per stage
    constexpr int BC = BN * 8 / kThreads;
    __shared__ u32x4 lds[2 * (BM + BN) * 8];
    __shared__ SlotMeta meta;
    u32x4* As = lds;
    u32x4* Bs = lds + 2 * BM * 8;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const MetaView mv = stage_meta(f, &meta);  // ordered by the main loop's barriers
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (K + kBK - 1) / kBK;

    const int lc = tid & 7, lr = tid >> 3;
    const uint16_t* xrow[AC];  // gathered x rows of this thread's chunks (clamped; xok masks)
    bool xok[AC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int p = m0 + lr + 32 * i;
        xok[i] = p < M;
        xrow[i] = X + (int64_t)f.token_order[min(p, M - 1)] * K;
    }
    const int mend = min(M, m0 + BM);
    // interior tiles (the uniform common case) load without masks; elsewhere
    // a masked-off chunk reads zeros (or_zero selects the address)
    const bool interior = m0 + BM <= M && n0 + BN <= N && (K % kBK) == 0;
    const uint16_t* wtile = W + (int64_t)n0 * K;
    u32x4 ra[AC], rb[BC];
    auto gload = [&](int it) {
        if (it < nk) {
            const int kk = it * kBK + lc * 8;
            if (interior) {
#pragma unroll
                for (int i = 0; i < AC; ++i) ra[i] = *(const u32x4*)(xrow[i] + kk);
#pragma unroll
                for (int i = 0; i < BC; ++i) rb[i] = *(const u32x4*)(wtile + (int64_t)(lr + 32 * i) * K + kk);
                return;
            }
            const bool kin = kk < K;  // K % 8 == 0: a chunk is fully in or out
#pragma unroll
            for (int i = 0; i < AC; ++i) ra[i] = *or_zero(kin && xok[i], xrow[i] + kk);
#pragma unroll
            for (int i = 0; i < BC; ++i) {
                const int r = n0 + lr + 32 * i;
                rb[i] = *or_zero(kin && r < N, W + (int64_t)r * K + kk);
            }
            return;
        }
        ExtraStep x{};
        extra_steps(mv, f, m0, mend, it - nk, &x);
        const int k0 = x.t * 64 + lc * 8;       // position in the 2 rp extension
        const int q0 = k0 < f.rp ? k0 : k0 - f.rp;  // rank of the chunk (rp % 8 == 0)
        const bool qin = k0 < 2 * f.rp && q0 < x.r;
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int p = m0 + lr + 32 * i;
            ra[i] = *or_zero(qin && p >= x.sb && p < x.se, f.ext + (int64_t)p * 2 * f.rp + k0);
        }
#pragma unroll
        for (int i = 0; i < BC; ++i) {
            const int n = n0 + lr + 32 * i;
            rb[i] = *or_zero(qin && n < N, f.B_pool + ((int64_t)x.s * N + n) * f.r_max + q0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AC; ++i) As[buf * BM * 8 + swz(lr + 32 * i, lc)] = ra[i];
#pragma unroll
        for (int i = 0; i < BC; ++i) Bs[buf * BN * 8 + swz(lr + 32 * i, lc)] = rb[i];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    sstore(0);
    __syncthreads();
    // the slot metadata is in LDS now: count the expand's extra K steps
    const int nt = nk + ((f.adapters && f.ext) ? extra_steps(mv, f, m0, mend, -1, nullptr) : 0);
    for (int kt = 0; kt < nt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nt) gload(kt + 1);
        const u32x4* Ab = As + buf * BM * 8;
        const u32x4* Bb = Bs + buf * BN * 8;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = kk * 4 + (lane >> 4);
            u32x4 af[FM], bfg[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = Ab[swz(wm * WTM + i * 16 + (lane & 15), c)];
#pragma unroll
            for (int j = 0; j < FN; ++j) bfg[j] = Bb[swz(wn * WTN + j * 16 + (lane & 15), c)];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(af[i], bfg[j], acc[i][j]);
        }
        if (kt + 1 < nt) sstore(buf ^ 1);
        __syncthreads();
    }

    const int p0 = m0 + wm * WTM, nb = n0 + wn * WTN;
    if (!f.ext) fused_expand<FM, FN>(acc, f, mv, p0, nb, M, N, lane);
    store_tile<FM, FN>(acc, Y, f.token_order, p0, nb, M, N, lane);
}

// ------------------------------------------------------- tiled, 256 x 256 --
// 8 waves (2 per SIMD) as 2 x 4, wave tile 128 x 64 (8 x 4 MFMA tiles); K in
// stages of 32 through kDmaStages LDS buffers, filled by direct-to-LDS loads
// (global_load_lds_dwordx4: 16 B per lane, written at the wave's LDS base +
// 16 * lane). A stage's A and B operands are 16 blocks each of 16 rows x 32 k
// (1 KB). Lane i of a block load fetches row i / 4, k chunk (i % 4) ^
// dma_swz(row): the bank swizzle is applied by choosing the source, so the
// MFMA fragment reads (row l % 16, chunk l / 16) are free of bank conflicts.
// Stage kt + kDmaStages - 1 is loaded once every wave is past stage kt's
// barrier. The fragment reads are issued and waited on by hand: with LDS
// loads in flight the compiler would wait for all of them at the first use.
constexpr int kDmaStages = 3;
constexpr int kDmaStageChunks = (256 + 256) * 32 * 2 / 16;  // 16-byte chunks

__device__ __forceinline__ int dma_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) u32x4* lds_u32x4_ptr;

__device__ __forceinline__ void dma16(gptr<u32x4> src, u32x4* lds_dst) {
    __builtin_amdgcn_global_load_lds((gptr<void>)src, (lds_void_ptr)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ uint32_t lds_offset(const u32x4* p) { return (uint32_t)(uintptr_t)(lds_u32x4_ptr)p; }

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}
// at most N LDS reads of this wave still outstanding; ties the wait to the
// fragment registers so that no use of them moves above it
template <int N>
__device__ __forceinline__ void lds_landed(u32x4& a) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_landed(u32x4& a, u32x4& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
// at most N vector-memory ops of this wave outstanding, no LDS op
template <int N>
__device__ __forceinline__ void vm_landed() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// EPI: the expand runs in the epilogue from fp32 h (r_max % 8 != 0);
// otherwise it runs as extra K steps (or there is no adapter row).
// KTAIL: K % 32 != 0, the last base stage masks the chunks past K.
template <bool EPI, bool KTAIL>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_dma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int N, int K,
    int tiles_m, int tiles_n, Fuse f) {
    constexpr int BM = 256, BN = 256, BK = 32, NS = kDmaStages, STAGE = kDmaStageChunks;
    __shared__ u32x4 lds[NS * STAGE];
    __shared__ SlotMeta meta;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const MetaView mv = stage_meta(f, &meta);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int mend = min(M, m0 + BM);
    const int nk = (K + BK - 1) / BK;
    // this lane's rows of the two A and two B blocks it loads (rows past M or
    // N are clamped: their products land in outputs that are not stored)
    const int rl = lane >> 2;
    const int cl = (lane & 3) ^ dma_swz(rl);
    int prow[2], ncol[2];
    const uint16_t* ap[2];
    const uint16_t* bp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        prow[b] = m0 + (wave * 2 + b) * 16 + rl;
        ncol[b] = n0 + (wave * 2 + b) * 16 + rl;
        ap[b] = X + (int64_t)f.token_order[min(prow[b], M - 1)] * K + cl * 8;
        bp[b] = W + (int64_t)min(ncol[b], N - 1) * K + cl * 8;
    }
    __syncthreads();  // slot metadata staged
    // the same for every lane; read from LDS it would be a per-lane value, and
    // the loop would be compiled as divergent control flow
    const int nt = __builtin_amdgcn_readfirstlane(
        nk + ((f.adapters && f.ext) ? extra_steps(mv, f, m0, mend, -1, nullptr, BK) : 0));

    auto issue = [&](int kt) {
        u32x4* st = lds + (kt % NS) * STAGE;
        gptr<u32x4> asrc[2], bsrc[2];
        if (kt < nk) {
            const int k = kt * BK;
            const bool kin = !KTAIL || k + cl * 8 < K;  // K % 8 == 0: a chunk is fully in or out
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                asrc[b] = KTAIL ? or_zero(kin, ap[b] + k) : as_global<u32x4>(ap[b] + k);
                bsrc[b] = KTAIL ? or_zero(kin, bp[b] + k) : as_global<u32x4>(bp[b] + k);
            }
        } else {
            ExtraStep x{};
            extra_steps(mv, f, m0, mend, kt - nk, &x, BK);
            const int k = x.t * BK + cl * 8;            // position in the 2 rp extension
            const int q = k < f.rp ? k : k - f.rp;      // rank of the chunk (rp % 8 == 0)
            const bool qin = k < 2 * f.rp && q < x.r;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                asrc[b] = or_zero(qin && prow[b] >= x.sb && prow[b] < x.se, f.ext + (int64_t)prow[b] * 2 * f.rp + k);
                bsrc[b] = or_zero(qin && ncol[b] < N, f.B_pool + ((int64_t)x.s * N + ncol[b]) * f.r_max + q);
            }
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) dma16(asrc[b], st + (wave * 2 + b) * 64);
#pragma unroll
        for (int b = 0; b < 2; ++b) dma16(bsrc[b], st + 16 * 64 + (wave * 2 + b) * 64);
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fc = lane >> 4;
    const int foff = fr * 4 + (fc ^ dma_swz(fr));
    const uint32_t abase = lds_offset(lds + wm * 8 * 64 + foff);
    const uint32_t bbase = lds_offset(lds + 16 * 64 + wn * 4 * 64 + foff);

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nt) issue(s);
    for (int kt = 0; kt < nt; ++kt) {
        // stage kt landed for this wave (the one issued after it may be in flight)
        static_assert(NS == 3, "wait counts assume 3 stages");
        if (kt + 1 < nt) vm_landed<4>();
        else vm_landed<0>();
        stage_barrier();
        if (kt + NS - 1 < nt) issue(kt + NS - 1);  // into stage kt - 1's buffer
        const uint32_t so = (kt % NS) * STAGE * 16;
        u32x4 bf[4], af[8];
        bf[0] = lds_read16<0>(bbase + so);
        bf[1] = lds_read16<1024>(bbase + so);
        bf[2] = lds_read16<2048>(bbase + so);
        bf[3] = lds_read16<3072>(bbase + so);
        af[0] = lds_read16<0>(abase + so);
        af[1] = lds_read16<1024>(abase + so);
        af[2] = lds_read16<2048>(abase + so);
        af[3] = lds_read16<3072>(abase + so);
        af[4] = lds_read16<4096>(abase + so);
        af[5] = lds_read16<5120>(abase + so);
        af[6] = lds_read16<6144>(abase + so);
        af[7] = lds_read16<7168>(abase + so);
        lds_landed<7>(bf[0], af[0]);
        lds_landed<7>(bf[1], bf[2]);
        lds_landed<7>(bf[3]);
        auto row = [&](auto i_) {
            constexpr int i = decltype(i_)::value;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        };
        row(std::integral_constant<int, 0>{});
        lds_landed<6>(af[1]);
        row(std::integral_constant<int, 1>{});
        lds_landed<5>(af[2]);
        row(std::integral_constant<int, 2>{});
        lds_landed<4>(af[3]);
        row(std::integral_constant<int, 3>{});
        lds_landed<3>(af[4]);
        row(std::integral_constant<int, 4>{});
        lds_landed<2>(af[5]);
        row(std::integral_constant<int, 5>{});
        lds_landed<1>(af[6]);
        row(std::integral_constant<int, 6>{});
        lds_landed<0>(af[7]);
        row(std::integral_constant<int, 7>{});
    }
    const int p0 = m0 + wm * 128, nb = n0 + wn * 64;
    if constexpr (EPI) fused_expand<8, 4>(acc, f, mv, p0, nb, M, N, lane);
    store_tile<8, 4>(acc, Y, f.token_order, p0, nb, M, N, lane);
}

// -------------------------------------------------------------- split-K --
struct SplitArgs {
    const uint16_t* X;
    const uint16_t* W;
    float* part_y;  // [ks][n_mt][n_nt][16 fragments][64 lanes] f32x4
    int M, N, K, n_mt, n_nt, ks;
    // shrink workgroups (the first n_items * hs blocks), hkc k each
    const uint16_t* A_pool;
    const int32_t* rank;
    const int32_t* token_order;
    const Item* work;
    int n_items, r_max;
    float* part_h;  // [hs][M][r_max]
    int hs, hkc;
};

// grid: n_items * hs shrink blocks, then n_mt * n_nt * ks GEMM blocks. The
// shrink splits are finer than the GEMM's, so that they finish early.
// Wave w of a GEMM block owns columns n0 + 16 w .. + 15 of a 64 x 64 tile.
// The split's x rows (gathered through token_order) and W rows stream
// through kSplitStages LDS buffers of 64 k by direct-to-LDS loads: a stage is
// 8 blocks each of x and of W, a block being 8 rows x 128 B; lane i of a
// block load fetches row i / 8, chunk (i % 8) ^ (row % 8), so that each load
// instruction reads whole 128-byte lines and the MFMA fragment reads (row
// l % 16, chunk l / 16) are free of bank conflicts. Rows past M or N are
// clamped (their partials are not stored); chunks past K read zeros.
constexpr int kSplitStages = 5;
constexpr int kSplitStageChunks = 1024;  // 16-byte chunks: x 512, W 512

template <int NSUB>
__global__ __launch_bounds__(kThreads) void splitk_gemm_kernel(SplitArgs a) {
    __shared__ u32x4 lds[kSplitStages * kSplitStageChunks];  // 80 KB
    constexpr int KC = NSUB * 128, NST = NSUB * 2, NS = kSplitStages, SC = kSplitStageChunks;
    const int n_shrink = a.n_items * a.hs;
    if ((int)blockIdx.x < n_shrink) {
        const int item = blockIdx.x % a.n_items, kz = blockIdx.x / a.n_items;
        const Item it = a.work[item];
        const int r = a.rank[it.slot];
        if (r == 0) return;
        const int kbeg = kz * a.hkc, kend = min(a.K, kbeg + a.hkc);
        const ShrinkOut out{a.part_h + (int64_t)kz * a.M * a.r_max, nullptr, 0, 0.f};
        shrink_item<4>(a.X, a.A_pool, r, a.token_order, it, out, a.K, kbeg, kend, a.r_max,
                       reinterpret_cast<f32x4*>(lds));
        return;
    }
    const int g = blockIdx.x - n_shrink;
    const int tiles = a.n_mt * a.n_nt;
    const int kz = g / tiles, t = g - kz * tiles;
    const int mt = t / a.n_nt, nt = t - mt * a.n_nt;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = mt * 64, n0 = nt * 64;
    const int kbeg = kz * KC;
    const int K = a.K;
    // this lane's rows and chunk in its two x and two W block loads
    const int dr = lane >> 3, dc = lane & 7;
    const uint16_t* xs[2];
    const uint16_t* ws[2];
    int kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 16 * wave + 8 * j + dr;  // tile row / column 0..63
        kc[j] = kbeg + (dc ^ (r & 7)) * 8;     // this lane's k within a stage
        xs[j] = a.X + (int64_t)a.token_order[min(m0 + r, a.M - 1)] * K + kc[j];
        ws[j] = a.W + (int64_t)min(n0 + r, a.N - 1) * K + kc[j];
    }
    auto issue = [&](int s) {
        u32x4* st = lds + (s % NS) * SC;
        const int k = s * 64;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(or_zero(kc[j] + k < K, xs[j] + k), st + (2 * wave + j) * 64);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(or_zero(kc[j] + k < K, ws[j] + k), st + 512 + (2 * wave + j) * 64);
    };
    // fragment reads: row r = lane % 16 of a 16-row tile, chunk 4 u + lane / 16
    const int fr = lane & 15, fq = lane >> 4;
    int fo[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) fo[u] = fr * 8 + ((4 * u + fq) ^ (fr & 7));
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < NST) issue(s);
#pragma unroll
    for (int s = 0; s < NST; ++s) {
        // stage s landed for this wave; the stages issued after it may be in flight
        const int later = (s + NS - 2 < NST ? NS - 2 : NST - 1 - s);
        static_assert(kSplitStages == 5, "wait counts assume 5 stages");
        if (later >= 3) vm_landed<12>();
        else if (later == 2) vm_landed<8>();
        else if (later == 1) vm_landed<4>();
        else vm_landed<0>();
        stage_barrier();
        if (s + NS - 1 < NST) issue(s + NS - 1);  // into stage s - 1's buffer
        const u32x4* st = lds + (s % NS) * SC;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const u32x4 wf = st[512 + wave * 128 + fo[u]];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = mfma16x16x32(st[i * 128 + fo[u]], wf, acc[i]);
        }
    }
    f32x4* out = reinterpret_cast<f32x4*>(a.part_y) + ((int64_t)(kz * a.n_mt + mt) * a.n_nt + nt) * 16 * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(i * 4 + wave) * 64 + lane] = acc[i];
}

// grid (n_nt, 4 * n_mt): block (nt, 4 mt + rb) finishes row block rb (16
// rows) of tile (mt, nt); wave w takes its 16 columns n0 + 16 w. Lane l holds
// rows p0 + 4 (l / 16) + e, e < 4, of column n0 + 16 w + l % 16.
//
// Two rounds of global loads. Round 1: the split partials, the output rows'
// token indices, the slot metadata (lane s keeps segment start, rank and scale
// of slot s when S <= 64) and the block's h rows (split planes, added in
// split order, then kept in LDS). Round 2, addressed by the rows' slots: each
// lane's B_s rows. Then every lane adds, in fp32, scale_s * h[p] . B_s[n]
// to its rows, and the tile is rounded once.
//
// ADAPT false: no adapter row in the batch (partials only). VEC: r_max % 8
// == 0 (16-byte h and B loads); otherwise element loads, waited in turn.
// LANE_META: S <= 64, metadata held one slot per lane; otherwise staged in
// LDS (one more round). Dynamic LDS: 16 * r_max + 32 floats (the tail keeps
// the last row's 32-rank reads in bounds; what they read there is not used).
constexpr int kLaneMetaSlots = 64;

template <bool ADAPT, bool VEC, bool LANE_META>
__global__ __launch_bounds__(kThreads) void splitk_epilogue_kernel(const float* __restrict__ part_y, int ks, int n_mt,
                                                                   int n_nt, uint16_t* __restrict__ Y, int M, int N,
                                                                   Fuse f) {
    const int nt = blockIdx.x, mt = blockIdx.y >> 2, rb = blockIdx.y & 3;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int p0 = mt * 64 + rb * 16;
    if (p0 >= M) return;  // uniform for the block
    const f32x4* in = reinterpret_cast<const f32x4*>(part_y);
    const int64_t zstride = (int64_t)n_mt * n_nt * 16 * 64;
    const int64_t o = (((int64_t)mt * n_nt + nt) * 16 + rb * 4 + w) * 64 + lane;
    const int n = nt * 64 + w * 16 + (lane & 15);
    // splits are added in split order; loads are issued unconditionally from
    // clamped addresses (a load under a branch is waited on inside it) and
    // the extra ones are not added
    f32x4 part[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) part[z] = in[min(z, ks - 1) * zstride + o];
    int tok[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) tok[e] = f.token_order[min(p0 + (lane >> 4) * 4 + e, M - 1)];

    float d[4] = {0.f, 0.f, 0.f, 0.f};
    int rr[4] = {0, 0, 0, 0};
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ADAPT) {
        __shared__ SlotMeta meta;
        extern __shared__ __align__(16) float hs[];  // [16][r_max]
        const int S = f.S, r_max = f.r_max;
        int ip = 0, rk = 0;
        float sv = 0.f;
        if constexpr (LANE_META) {
            ip = f.slot_indptr[min(lane, S)];
            rk = f.rank[min(lane, S - 1)];
            sv = f.scale[min(lane, S - 1)];
        }
        // h: 16 rows x r_max, h_splits planes; 16-byte pieces when VEC
        constexpr int HU = 2;  // pieces per thread in round 1
        const int rq = VEC ? r_max >> 2 : r_max;
        const int npc = 16 * rq;
        f32x4 hv[HU][8];
        if constexpr (VEC) {
#pragma unroll
            for (int u = 0; u < HU; ++u) {
                const int i = tid + u * kThreads;
                const int row = i / rq, c = i - row * rq;
                const float* hp = f.h + (int64_t)min(p0 + row, M - 1) * r_max + c * 4;
#pragma unroll
                for (int z = 0; z < 8; ++z)
                    hv[u][z] = __builtin_bit_cast(f32x4, *or_zero(i < npc && z < f.h_splits, hp + (int64_t)z * f.h_plane));
            }
        }
        issue_fence();  // round 1 is in flight
        if constexpr (!LANE_META) {  // large pools: metadata staged in LDS
            for (int i = tid; i <= S; i += kThreads) {
                meta.indptr[i] = f.slot_indptr[i];
                if (i < S) {
                    meta.rank[i] = f.rank[i];
                    meta.scale[i] = f.scale[i];
                }
            }
            __syncthreads();
        }
        // slots of this lane's rows
        int sl[4] = {0, 0, 0, 0};
        if constexpr (LANE_META) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // slot of row p = number of slots s in 1..S-1 starting at or before p
                const uint64_t m = __ballot(lane >= 1 && lane < S && ip <= p0 + j);
                const int sj = p0 + j < M ? __popcll(m) : 0;
                if ((lane >> 4) == (j >> 2)) sl[j & 3] = sj;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = __shfl(rk, sl[e]);
                rr[e] = sl[e] == 0 ? 0 : r;
                sc[e] = __shfl(sv, sl[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = p0 + (lane >> 4) * 4 + e;
                sl[e] = p < M ? slot_of(meta.indptr, S, p) : 0;
                rr[e] = sl[e] == 0 ? 0 : meta.rank[sl[e]];
                sc[e] = meta.scale[sl[e]];
            }
        }
        const uint16_t* bp[4];
        int rmax = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bp[e] = f.B_pool + ((int64_t)sl[e] * N + min(n, N - 1)) * r_max;
            rmax = max(rmax, rr[e]);
        }
        // round 2 (first 32 ranks), issued before h is written to LDS
        constexpr int NC = 4;  // 8-rank chunks per row per round
        u32x4 b[4][NC];
        auto bload = [&](int q0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c = 0; c < NC; ++c) b[e][c] = *or_zero(q0 + 8 * c < rr[e], bp[e] + q0 + 8 * c);
        };
        if constexpr (VEC) bload(0);
        issue_fence();  // round 2 is in flight
        // h planes added in split order, into LDS
        if constexpr (VEC) {
#pragma unroll
            for (int u = 0; u < HU; ++u) {
                const int i = tid + u * kThreads;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int z = 0; z < 8; ++z)
                    if (z < f.h_splits) v += hv[u][z];
                for (int z0 = 8; z0 < f.h_splits; z0 += 8) {
                    const int row = i / rq, c = i - row * rq;
                    const float* hp = f.h + (int64_t)min(p0 + row, M - 1) * r_max + c * 4;
#pragma unroll
                    for (int z = 0; z < 8; ++z)
                        hv[u][z] = __builtin_bit_cast(
                            f32x4, *or_zero(i < npc && z0 + z < f.h_splits, hp + (int64_t)(z0 + z) * f.h_plane));
#pragma unroll
                    for (int z = 0; z < 8; ++z)
                        if (z0 + z < f.h_splits) v += hv[u][z];
                }
                if (i < npc) reinterpret_cast<f32x4*>(hs)[i] = v;
            }
            for (int i = tid + HU * kThreads; i < npc; i += kThreads) {  // r_max > 128
                const int row = i / rq, c = i - row * rq;
                const float* hp = f.h + (int64_t)min(p0 + row, M - 1) * r_max + c * 4;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                for (int z = 0; z < f.h_splits; ++z) v += *as_global<f32x4>(hp + (int64_t)z * f.h_plane);
                reinterpret_cast<f32x4*>(hs)[i] = v;
            }
        } else {
            for (int i = tid; i < npc; i += kThreads) {
                const int row = i / r_max;
                const float* hp = f.h + (int64_t)min(p0 + row, M - 1) * r_max + (i - row * r_max);
                float v = 0.f;
                for (int z = 0; z < f.h_splits; ++z) v += hp[(int64_t)z * f.h_plane];
                hs[i] = v;
            }
        }
        __syncthreads();
        // fp32 dot products, ranks in order; terms past the row's rank are
        // computed and dropped by a select (no branch)
        auto fma_round = [&](int q0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* hr = hs + ((lane >> 4) * 4 + e) * r_max + q0;
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int q = q0 + 8 * c + 2 * t;
                        const uint32_t wv = b[e][c][t];
                        const float t0 = __builtin_fmaf(hr[8 * c + 2 * t], __uint_as_float(wv << 16), d[e]);
                        d[e] = q < rr[e] ? t0 : d[e];
                        const float t1 = __builtin_fmaf(hr[8 * c + 2 * t + 1], __uint_as_float(wv & 0xffff0000u), d[e]);
                        d[e] = q + 1 < rr[e] ? t1 : d[e];
                    }
            }
        };
        if constexpr (VEC) {
            fma_round(0);
            for (int q0 = 8 * NC; q0 < rmax; q0 += 8 * NC) {
                bload(q0);
                fma_round(q0);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* hr = hs + ((lane >> 4) * 4 + e) * r_max;
                for (int q = 0; q < rr[e]; ++q) d[e] = __builtin_fmaf(hr[q], bf16_to_f32(bp[e][q]), d[e]);
            }
        }
    }
    f32x4 acc = part[0];
#pragma unroll
    for (int z = 1; z < 8; ++z)
        if (z < ks) acc += part[z];
    for (int z0 = 8; z0 < ks; z0 += 8) {
#pragma unroll
        for (int z = 0; z < 8; ++z) part[z] = in[min(z0 + z, ks - 1) * zstride + o];
#pragma unroll
        for (int z = 0; z < 8; ++z)
            if (z0 + z < ks) acc += part[z];
    }
    if (n >= N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (p0 + (lane >> 4) * 4 + e >= M) continue;
        float v = acc[e];
        if (rr[e] > 0) v = __builtin_fmaf(sc[e], d[e], v);
        Y[(int64_t)tok[e] * N + n] = f32_to_bf16(v);
    }
}

// ------------------------------------------------------------------ plan --
static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

GemmPlan gemm_bf16_plan(int M, int N, int K) {
    GemmPlan g{};
    if (M <= 0 || N <= 0 || K <= 0) return g;  // nothing to launch
    const int64_t t256 = (int64_t)cdiv(M, 256) * cdiv(N, 256);
    const int64_t t128 = (int64_t)cdiv(M, 128) * cdiv(N, 128);
    const int64_t t64 = (int64_t)cdiv(M, 64) * cdiv(N, 128);
    if (t256 >= 256) { g.bm = 256; g.bn = 256; return g; }
    if (t128 >= 256) { g.bm = 128; g.bn = 128; return g; }
    if (M > 256 && t64 >= 128) { g.bm = 64; g.bn = 128; return g; }
    // split-K: 64 x 64 tiles, enough K splits for ~256 workgroups
    g.bm = 64; g.bn = 64;
    g.n_mt = cdiv(M, 64);
    g.n_nt = cdiv(N, 64);
    const int tiles = g.n_mt * g.n_nt;
    const int want = tiles >= 256 ? 1 : cdiv(256, tiles);
    const int need = cdiv(cdiv(K, want), 128);  // sub-chunks per split
    int nsub = 1;
    while (nsub < need && nsub < 16) nsub *= 2;
    g.nsub = nsub;
    g.ks = cdiv(K, nsub * 128);
    // shrink splits of at least 256 k, at most 8 of them (kernel 2 adds the
    // h planes in one round of loads)
    g.hkc = max(256, (cdiv(K, 8) + 31) / 32 * 32);
    g.hs = cdiv(K, g.hkc);
    return g;
}

size_t gemm_bf16_workspace(int M, int N, int K, int r_max) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const GemmPlan g = gemm_bf16_plan(M, N, K);
    // fp32 h [M][r_max], or bf16 hi / lo [M][2][round_up(r_max, 8)]
    const size_t h_final = (size_t)M * ((r_max + 7) & ~7) * sizeof(float);
    if (g.nsub == 0) return (h_final + 255) & ~size_t(255);
    const size_t py = (size_t)g.ks * g.n_mt * g.n_nt * 16 * 64 * 16;
    const size_t ph = (size_t)g.hs * M * r_max * sizeof(float);
    return ((py + 255) & ~size_t(255)) + ((ph + 255) & ~size_t(255));
}

template <int BM, int BN>
static hipError_t launch_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K,
                               const Fuse& f, hipStream_t st, StageTimer* tm) {
    const int tiles_m = cdiv(M, BM), tiles_n = cdiv(N, BN);
    return launch(tm, "gemm_bf16", gemm_tiled_kernel<BM, BN>, dim3(tiles_m * tiles_n), dim3(kThreads), st, X, W, Y,
                  M, N, K, tiles_m, tiles_n, f);
}

template <int NSUB>
static hipError_t launch_split(const SplitArgs& a, int n_blocks, hipStream_t st, StageTimer* tm) {
    return launch(tm, "gemm_splitk", splitk_gemm_kernel<NSUB>, dim3(n_blocks), dim3(kThreads), st, a);
}

hipError_t lora_forward_bf16(const LinearArgs& L, hipStream_t st, StageTimer* tm) {
    const int M = L.M, N = L.N, K = L.K;
    if (M == 0 || N == 0) return hipSuccess;
    const GemmPlan g = gemm_bf16_plan(M, N, K);
    Fuse f{L.token_order, L.slot_indptr, nullptr, L.B_pool, L.rank, L.scale, L.S, L.r_max, 1, 0, L.adapters,
           nullptr, (L.r_max + 7) & ~7};
    char* ws = static_cast<char*>(L.workspace);
    if (g.nsub == 0) {
        // shrink to final h, then the tiled GEMM with the expand in its epilogue
        // r_max % 8 == 0: the expand runs as extra K steps (operand: scaled
        // h as bf16 hi / lo); otherwise in the epilogue from fp32 h
        float* hbuf = reinterpret_cast<float*>(ws);
        uint16_t* ext = (L.r_max % 8 == 0) ? reinterpret_cast<uint16_t*>(ws) : nullptr;
        f.h = ext ? nullptr : hbuf;
        f.ext = ext;
        if (L.adapters) {
            const hipError_t e = sgmv_shrink(1, L.X, L.A_pool, L.rank, L.token_order, L.work, L.n_items,
                                             ext ? nullptr : hbuf, K, L.r_max, st, tm, L.scale, ext);
            if (e != hipSuccess) return e;
        }
        if (g.bm == 256) {
            const int tiles_m = cdiv(M, 256), tiles_n = cdiv(N, 256);
            const bool epi = L.adapters && !f.ext, ktail = K % 32 != 0;
            auto ker = epi ? (ktail ? gemm_dma_kernel<true, true> : gemm_dma_kernel<true, false>)
                           : (ktail ? gemm_dma_kernel<false, true> : gemm_dma_kernel<false, false>);
            return launch(tm, "gemm_bf16", ker, dim3(tiles_m * tiles_n), dim3(512), st, L.X, L.W, L.Y, M, N, K, tiles_m,
                          tiles_n, f);
        }
        if (g.bm == 128) return launch_tiled<128, 128>(L.X, L.W, L.Y, M, N, K, f, st, tm);
        return launch_tiled<64, 128>(L.X, L.W, L.Y, M, N, K, f, st, tm);
    }
    const size_t py = ((size_t)g.ks * g.n_mt * g.n_nt * 16 * 64 * 16 + 255) & ~size_t(255);
    SplitArgs a{L.X, L.W, reinterpret_cast<float*>(ws), M, N, K, g.n_mt, g.n_nt, g.ks,
                L.A_pool, L.rank, L.token_order, reinterpret_cast<const Item*>(L.work),
                L.adapters ? L.n_items : 0, L.r_max, reinterpret_cast<float*>(ws + py), g.hs, g.hkc};
    const int n_blocks = a.n_items * g.hs + g.n_mt * g.n_nt * g.ks;
    hipError_t e;
    switch (g.nsub) {
        case 1: e = launch_split<1>(a, n_blocks, st, tm); break;
        case 2: e = launch_split<2>(a, n_blocks, st, tm); break;
        case 4: e = launch_split<4>(a, n_blocks, st, tm); break;
        case 8: e = launch_split<8>(a, n_blocks, st, tm); break;
        default: e = launch_split<16>(a, n_blocks, st, tm); break;
    }
    if (e != hipSuccess) return e;
    f.h = a.part_h;
    f.h_splits = g.hs;
    f.h_plane = (int64_t)M * L.r_max;
    const dim3 eg(g.n_nt, 4 * g.n_mt);
    auto epi = splitk_epilogue_kernel<false, false, false>;
    if (L.adapters) {
        if (L.r_max % 8 != 0) epi = splitk_epilogue_kernel<true, false, false>;
        else if (L.S <= kLaneMetaSlots) epi = splitk_epilogue_kernel<true, true, true>;
        else epi = splitk_epilogue_kernel<true, true, false>;
    }
    const uint32_t shm = L.adapters ? (uint32_t)((16 * L.r_max + 32) * sizeof(float)) : 0u;
    return launch_shm(tm, "gemm_splitk_epilogue", epi, eg, dim3(kThreads), shm, st, (const float*)a.part_y, g.ks,
                      g.n_mt, g.n_nt, L.Y, M, N, f);
}

}  // namespace lora
