// Device pieces shared by the bf16 GEMM kernels of liblora: the fused
// correction's arguments and slot metadata, the row scatter of the output,
// the XCD-aware tile order, and the direct-to-LDS load helpers.
//
// The correction follows "LoRA serving, embeddings, rerankers, pooling"
// (mlinterviewnotes.com, opening section): base GEMM once over the batch,
// then the per-row indexed low-rank correction scale_s * (x A_s^T) B_s^T.
#pragma once

#include "common.h"
#include "kernels.h"

namespace lora {

static inline __host__ __device__ int cdiv(int a, int b) { return (a + b - 1) / b; }

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

// Last slot s with slot_indptr[s] <= p (the slot whose segment holds p).
__device__ __forceinline__ int slot_of(const int* indptr, int S, int p) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (indptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// acc[i][j][e] is sorted row p0 + 16 i + lane % 16, column n0 + 16 j +
// 4 (lane / 16) + e (the products are taken as (W x^T) blocks, so that a lane
// holds 4 consecutive columns of one row). Adds scale_s * h[p] . B_s[n] for
// every adapter row.
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
                    acc[i][j] = mfma16x16x16(bfr[j], ahi, acc[i][j]);
                    acc[i][j] = mfma16x16x16(bfr[j], alo, acc[i][j]);
                }
            }
        }
    }
}

// Round and store through LDS (acc laid out as for fused_expand). The wave's
// block is written to its staging area `stg` as bf16 rows of FN * 32 bytes in
// 8-byte units (unit index XOR an even function of the row, against bank
// conflicts), then read back as 16-byte row pieces, so that each store
// instruction writes whole row segments y[token_order[p]][n .. n + 8). The
// staging area is private to the wave: no barrier between the two halves.
template <int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[FM][FN], char* stg, uint16_t* __restrict__ Y,
                                           const int32_t* __restrict__ token_order, int p0, int n0, int M, int N,
                                           int lane) {
    constexpr int RB = FN * 32, U = FN * 4;      // row bytes, 8-byte units per row
    constexpr int LPR = FN * 2, RPI = 64 / LPR;  // lanes per row, rows per read
    static_assert(64 % LPR == 0 && (FM * 16) % RPI == 0, "staging layout");
    constexpr int NR = FM * 16 / RPI;  // rows (read instructions) per lane
    auto swz = [](int r) { return (2 * (r >> 1)) & (U - 2); };
    // the output rows' token indices are loaded first: fetched between the
    // stores, each would wait behind the store traffic of every CU
    int tok[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) tok[t] = token_order[min(p0 + t * RPI + lane / LPR, M - 1)];
    const int c = lane & 15, q = lane >> 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = 16 * i + c;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x2 v{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
            *reinterpret_cast<u32x2*>(stg + r * RB + ((4 * j + q) ^ swz(r)) * 8) = v;
        }
    }
    const bool vec = (N & 7) == 0;  // rows of y are 16-byte aligned
    const int u2 = lane % LPR;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        const int r = t * RPI + lane / LPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * RB + ((2 * u2) ^ swz(r)) * 8);
        const int p = p0 + r, n = n0 + u2 * 8;
        if (p < M && n < N) {
            uint16_t* yp = Y + (int64_t)tok[t] * N + n;
            if (vec) {  // non-temporal: the output is written once and not read back here
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(yp));
            } else {
                const int ne = min(8, N - n);
                for (int e = 0; e < ne; ++e) yp[e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
            }
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

// The expand as extra K steps of the tiled GEMM. The tile's live slots are
// the slots s >= 1 of nonzero rank whose segment [indptr[s], indptr[s + 1])
// is non-empty and meets the tile's rows [m0, mend); taken in slot order,
// each extends K by 2 rp (rp = r_max rounded up to 8): the A operand of row
// p is its ext row [bf16 hi of scale_s h | lo remainder] (zero for rows of
// other segments), the B operand of column n is [B_s[n] | B_s[n]], so the
// products add scale_s h . B_s. When 2 rp divides 64 (rp = 8, 16, 32) the
// extensions of P = 64 / (2 rp) consecutive live slots share one 64-wide
// step: every row belongs to one slot, so a row's products outside its own
// slot's part are exact zeros. Otherwise each slot takes ceil(2 rp / 64)
// steps of its own.
//
// The slot metadata is read from its LDS copy (the host takes the
// extra-step form only for pools of at most kMetaSlots slots): a flat or
// global load here would also wait for every direct-to-LDS load in flight.
typedef const __attribute__((address_space(3))) SlotMeta* lds_meta_ptr;

typedef __attribute__((address_space(3))) uint16_t* lds_u16_ptr;  // slot ids (S <= kMetaSlots)

// Live slots among slots 64 c .. 64 c + 63, as a wave-uniform bit mask.
__device__ __forceinline__ uint64_t live_slots(lds_meta_ptr meta, int S, int m0, int mend, int c) {
    const int s = 64 * c + (int)(threadIdx.x & 63);
    bool live = false;
    if (s >= 1 && s < S) {
        const int sb = meta->indptr[s], se = meta->indptr[s + 1];
        live = se > sb && sb < mend && se > m0 && meta->rank[s] != 0;
    }
    return __ballot(live);
}

// The tile's extra steps: its live slots, listed in slot order in an LDS
// list, and how they map to steps. Every wave computes the same schedule;
// only the `writer` wave fills the list, so the workgroup passes a barrier
// before any wave reads it (when n > 0, which is uniform over the workgroup).
struct ExtraSched {
    int n;    // live slots
    int P;    // live slots per step (P > 1: 2 rp divides 64)
    int spk;  // steps per slot (P == 1)
    int lw;   // log2 of the 8-element chunks of one slot's part in a step
    __device__ __forceinline__ int steps() const { return P > 1 ? (n + P - 1) / P : n * spk; }
};

// on: the batch has adapter rows and the expand takes this form (the
// metadata is staged in LDS); otherwise the tile has no extra step. `list`
// holds at least min(S, mend - m0) entries (a live slot has a row in the tile).
__device__ __forceinline__ ExtraSched extra_schedule(bool on, lds_meta_ptr meta, int S, int m0, int mend, int rp,
                                                     lds_u16_ptr list, bool writer) {
    ExtraSched x;
    const int r2 = on ? 2 * rp : 16;
    x.P = (64 % r2 == 0) ? 64 / r2 : 1;
    x.spk = x.P > 1 ? 1 : (r2 + 63) / 64;
    x.lw = x.P == 4 ? 1 : x.P == 2 ? 2 : 3;
    // chunks of 64 slots whose segments meet the tile: a chunk's segments
    // span indptr[64 c] .. indptr[min(64 c + 64, S)]
    int c_lo = 0, c_hi = on ? (S - 1) >> 6 : -1;
    const int lane = (int)(threadIdx.x & 63);
    if (c_hi > 0) {
        bool meets = false;
        if (lane <= c_hi) meets = meta->indptr[64 * lane] < mend && meta->indptr[min(64 * lane + 64, S)] > m0;
        const uint64_t mm = __ballot(meets);
        c_lo = mm ? __builtin_ctzll(mm) : 1;
        c_hi = mm ? 63 - __builtin_clzll(mm) : 0;
    }
    int n = 0;
    for (int c = c_lo; c <= c_hi; ++c) {
        const uint64_t mask = live_slots(meta, S, m0, mend, c);
        if (writer && ((mask >> lane) & 1)) list[n + __popcll(mask & ((1ull << lane) - 1))] = (uint16_t)(64 * c + lane);
        n += __popcll(mask);
    }
    x.n = n;
    return x;
}

// Operands of one load instruction's chunk in an extra step: chunk ch (0..7)
// of the 64-wide step belongs to the step's slot e = ch >> lw; `k` is its
// position in that slot's [hi | lo] part, `q` its rank, `ok` whether it
// holds ranks below the slot's rank, [sb, se) the slot's segment.
struct ExtraChunk {
    int s, sb, se, k, q;
    bool ok;
};
struct ExtraSlot {
    int s, sb, se, r;
};
struct ExtraStepMeta {
    ExtraSlot e0, e1, e2, e3;
    int t;
};
// slot j of the list (none past the end: rank 0)
__device__ __forceinline__ ExtraSlot extra_slot(lds_meta_ptr meta, lds_u16_ptr list, int n, int j) {
    const bool has = j < n;
    const int s = has ? list[has ? j : 0] : 0;
    return ExtraSlot{s, meta->indptr[s], meta->indptr[s + 1], has ? meta->rank[s] : 0};
}
// extra step kt of the tile
__device__ __forceinline__ ExtraStepMeta extra_step(const ExtraSched& x, lds_meta_ptr meta, lds_u16_ptr list,
                                                    int kt) {
    ExtraStepMeta m;
    const int j0 = x.P > 1 ? kt * x.P : (x.spk == 1 ? kt : kt / x.spk);
    m.t = x.P > 1 ? 0 : kt - j0 * x.spk;
    const int n1 = x.P > 1 ? x.n : min(x.n, j0 + 1);  // P == 1: one slot per step
    m.e0 = extra_slot(meta, list, n1, j0);
    m.e1 = extra_slot(meta, list, n1, j0 + 1);
    m.e2 = extra_slot(meta, list, x.P > 2 ? n1 : 0, j0 + 2);
    m.e3 = extra_slot(meta, list, x.P > 2 ? n1 : 0, j0 + 3);
    return m;
}
__device__ __forceinline__ ExtraChunk extra_chunk(const ExtraSched& x, const ExtraStepMeta& m, int ch, int rp) {
    const int e = ch >> x.lw;
    // field by field: a select between the structs themselves would take
    // their addresses and put them in scratch memory
    auto pick = [e](int v0, int v1, int v2, int v3) { return e == 0 ? v0 : e == 1 ? v1 : e == 2 ? v2 : v3; };
    ExtraChunk c;
    c.s = pick(m.e0.s, m.e1.s, m.e2.s, m.e3.s);
    c.sb = pick(m.e0.sb, m.e1.sb, m.e2.sb, m.e3.sb);
    c.se = pick(m.e0.se, m.e1.se, m.e2.se, m.e3.se);
    const int r = pick(m.e0.r, m.e1.r, m.e2.r, m.e3.r);
    c.k = m.t * 64 + ((ch & ((1 << x.lw) - 1)) << 3);
    c.q = c.k < rp ? c.k : c.k - rp;
    c.ok = c.k < 2 * rp && c.q < r;
    return c;
}

// ------------------------------------------------- direct-to-LDS loads --
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) u32x4* lds_u32x4_ptr;

__device__ __forceinline__ void dma16(gptr<u32x4> src, u32x4* lds_dst) {
    __builtin_amdgcn_global_load_lds((gptr<void>)src, (lds_void_ptr)lds_dst, 16, 0, 0);
}
// the same with the non-temporal hint (data read once: kept out of the way of
// what the caches should hold)
__device__ __forceinline__ void dma16_nt(gptr<u32x4> src, u32x4* lds_dst) {
    __builtin_amdgcn_global_load_lds((gptr<void>)src, (lds_void_ptr)lds_dst, 16, 0, 2);
}
// A raw buffer resource over [p, p + bytes) (bytes < 2^31): a load whose
// per-lane offset is at or past its end returns zeros without touching
// memory. The same direct-to-LDS load through it takes a 32-bit per-lane byte
// offset and a uniform one (soff, not range-checked), so a tile's row offsets
// are set once and each step only moves soff: no per-step address arithmetic
// per lane, and half the address registers of 64-bit pointers.
typedef __amdgpu_buffer_rsrc_t brsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a per-lane offset past every resource
__device__ __forceinline__ brsrc make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bdma16(brsrc r, uint32_t voff, uint32_t soff, u32x4* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds_dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ uint32_t lds_offset(const u32x4* p) { return (uint32_t)(uintptr_t)(lds_u32x4_ptr)p; }

template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
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

// The split-K decode path (kernel 1 + kernel 2) over every slice of L
// together, defined in splitk.hip. `g` is the plan of the slices'
// concatenated columns (its n_nt is recomputed per slice).
hipError_t splitk_forward_bf16(const LinearArgs& L, const GemmPlan& g, hipStream_t st, StageTimer* tm);

// Kernel 2 of the split-K path for one slice whose fp32 partials (ks splits,
// the 64 x 64 tile layout of kernel 1) were written by another kernel: adds
// the splits, applies the expand from fp32 h (h_splits planes of [M][r_max],
// unscaled) and stores y.
hipError_t splitk_finish_bf16(const LinearArgs& L, const SliceArgs& s, const float* part, int ks, int n_mt,
                              const float* h, int h_splits, hipStream_t st, StageTimer* tm);

}  // namespace lora
