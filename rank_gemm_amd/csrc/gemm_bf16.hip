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
// Two paths, chosen by (T, d_out) only:
//  * tiled (T above decode sizes, this file): one kernel template with K in
//    stages of 64 through an LDS ring filled by direct-to-LDS loads; the
//    macro tile is the one of 256 x 256 (4 waves), 256 x 128, 128 x 128 and
//    64 x 128 (8 waves) that takes the fewest rounds of 256 tiles times the
//    tile's time. The shrink runs before it as its own kernel.
//  * split-K (decode-sized T, splitk.hip): a K-split GEMM with the shrink in
//    extra workgroups of the same launch, then a kernel that adds the splits
//    and applies the expand.
#include "fuse.h"
#include "shrink.h"

#include <type_traits>
#include <utility>

namespace lora {

// --------------------------------------------- tiled, direct-to-LDS loads --
// BM x BN macro tiles over WM x WN waves, wave tile (BM / WM) x (BN / WN) of
// 16 x 16 MFMA tiles; K in stages of 64 through NS LDS buffers, filled by
// direct-to-LDS loads (global_load_lds_dwordx4: 16 B per lane, written at the
// instruction's LDS base + 16 * lane). A row of a stage is one 128-byte line
// (8 chunks of 16 B). Rows go in groups of 64; load instruction q (0..7) of a
// group fetches rows q, q + 8, ..., q + 56, the 8 lanes 8 i .. 8 i + 7 one
// whole line of row q + 8 i, so the instruction's 1 KB lands at q * 1024 in
// the group. Lane 8 i + j takes chunk j ^ q of its row (the XOR swizzle of
// the chunk by the row's index within its 8-row stripe): the MFMA fragment
// read of chunk c over 16 consecutive rows then finds their pieces at 16
// distinct 16-byte slots of one aligned 256-byte window modulo 1 KB, which
// this LDS serves in the minimum 4 cycles per ds_read_b128. (Rows merely
// padded apart by 16 bytes spread those pieces over two windows for chunks
// past the first: 8 cycles per read.)
// The fragment reads are issued and waited on by hand: with LDS loads in
// flight the compiler would wait for all of them at the first use.
constexpr int kInstrBytes = 1024;              // 1 KB of 8 rows
constexpr int kGroupBytes = 8 * kInstrBytes;   // 64 rows

// byte offset of the 16-row block starting at row r0 (r0 % 16 == 0)
__host__ __device__ constexpr int block_off(int r0) { return (r0 / 64) * kGroupBytes + (r0 % 64) / 8 * 128; }

// ------------------------------------------------- the pipelined tile --
// Each wave owns a (BM / WM) x (BN / WN) block of 16 x 16 MFMA tiles (fp32
// accumulators in AGPRs) and keeps its matrix core busy by interleaving all
// other work between its MFMAs. A 64-wide step has two 32-wide halves:
//   phase A of step kt: the MFMAs of the first half (fragments F0), one
//     fragment read of the second half (F1) per group of MFMAs;
//   the wave's loads of step kt + 1 landed; barrier;
//   phase B: the MFMAs of F1, one fragment read of step kt + 1's first half
//     per group, and the 1 KB loads of a later step.
// 256 x 256 runs on 4 waves, one per SIMD, with 128 x 128 wave tiles: a step
// reads 2/3 of the LDS bytes of an 8-wave 128 x 64 tiling. The smaller tiles
// run on 8 waves, two per SIMD: with so few MFMAs per phase one wave per SIMD
// hides too little of the fragment reads and barriers (a 4-wave 128 x 128
// took 57.7 us against 47.3 us at T = 1024, 4096 -> 4096).
// The accumulators are tied to AGPRs by issuing these MFMAs as inline asm
// (left to itself the register allocator shuffles accumulators through
// VGPRs at every loop back edge, ~400 copies per stage). The compiler then
// cannot see that those MFMAs read their fragment registers after issue:
// every phase ends by keeping its fragments alive through two s_nop 7, so no
// later instruction writes them while an MFMA may still read them, and 96
// wait states separate the last MFMA from the first read of the accumulators.
__device__ __forceinline__ void mfma_agpr(f32x4& acc, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int G>
struct Idx {
    static constexpr int v = G;
};
template <class F, int... Gs>
__device__ __forceinline__ void static_for(std::integer_sequence<int, Gs...>, F&& fn) {
    (fn(Idx<Gs>{}), ...);
}
template <int I, int N>
__device__ __forceinline__ void frags_tie(u32x4 (&a)[N]) {
    if constexpr (I < N) {
        asm volatile("" : "+v"(a[I]));
        frags_tie<I + 1, N>(a);
    }
}
template <int I, int N>
__device__ __forceinline__ void frags_use(const u32x4 (&a)[N]) {
    if constexpr (I < N) {
        asm volatile("" ::"v"(a[I]));
        frags_use<I + 1, N>(a);
    }
}
// every LDS read of this wave landed; ties the wait to the fragment
// registers so that no use of them moves above it
template <int N>
__device__ __forceinline__ void frags_landed(u32x4 (&a)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]));
    frags_tie<1, N>(a);
}
// 16 wait states during which the fragment registers stay live: the MFMAs
// issued above may still read them
template <int NA, int NB>
__device__ __forceinline__ void frags_retire(const u32x4 (&a)[NA], const u32x4 (&b)[NB]) {
    asm volatile("s_nop 7\n\ts_nop 7");
    frags_use<0, NA>(a);
    frags_use<0, NB>(b);
}

// Split over K (mid-sized T): block b takes tile b % n_tiles over the k
// range [kz kc, (kz + 1) kc), kz = b / n_tiles, and writes fp32 partials in
// the layout of the split-K path ([split][64-row tile][64-column tile][16
// blocks of 16 x 16][64 lanes] f32x4, lane l holding rows 4 (l / 16) + e of
// column l % 16). Split 0 also runs the expand's extra K steps, so the
// split-K path's kernel 2 only adds the partials and rounds.
struct SplitOut {
    float* part;     // null: no split
    int kc;          // k per split, a multiple of 64
    int n_mt, n_nt;  // 64 x 64 tile grid of the partials
};

// BM x BN tiles over WM x WN waves with NS stage buffers. With 2 stages, step
// kt + 2 is loaded during step kt into step kt's own buffer, free only in
// phase B. With NS >= 3, step kt + NS - 1 is loaded during step kt into the
// buffer of step kt - 1 (every wave finished reading it before step kt - 1's
// barrier), so its loads are spread over both phases.
// BUF: loads through buffer resources (x, the tile's W rows, ext, B_pool; the
// host takes this form when each is under 2 GiB): per-lane row offsets set
// once per tile, the base step's k in the uniform offset. Otherwise 64-bit
// addresses, moved by k every step (8192 x 4096 -> 14336: 737-747 us against
// 750-757 us, interleaved on one box, identical outputs).
template <int BM, int BN, int WM, int WN, int NS, bool EPI, bool KTAIL, bool SPLIT, bool BUF>
__global__ __launch_bounds__(64 * WM * WN, 1) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_tile_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Y, int M, int N, int K,
    int tiles_m, int tiles_n, Fuse f, SplitOut so) {
    static_assert(!(SPLIT && EPI), "a split runs no expand");
    static_assert(!(SPLIT && BUF), "splits take 64-bit addresses");
    constexpr int BK = 64, NW = WM * WN;
    constexpr int FI = BM / WM / 16, FJ = BN / WN / 16;    // MFMA blocks of a wave
    constexpr int DA = BM / 8 / NW, DB = BN / 8 / NW, ND = DA + DB;  // load instructions of a wave per step
    constexpr int NM = FI * FJ, NR = FI + FJ;              // MFMAs and fragment reads per half step
    constexpr int ABYTES = BM / 64 * kGroupBytes, STAGE = (BM + BN) / 64 * kGroupBytes / 16;  // 16-byte units
    static_assert(BM % 64 == 0 && BN % 64 == 0 && DA * NW * 8 == BM && DB * NW * 8 == BN && NW % 4 == 0, "tile shape");
    constexpr int L = NS >= 3 ? NS - 1 : 2;                // step kt + L is loaded during step kt
    constexpr int NDA = NS >= 3 ? ND / 2 : 0;              // its loads issued in phase A
    constexpr int NDB = ND - NDA;                          // ... and in phase B
    constexpr int VM_MID = (L - 2) * ND + NDA;             // loads younger than step kt + 1's at mid-step
    static_assert(NS >= 2 && VM_MID < 64 && (L - 1) * ND < 64 && NR <= 16, "wait counters");
    __shared__ u32x4 lds[NS * STAGE];
    __shared__ SlotMeta meta;
    __shared__ uint16_t xlist[BM];  // the tile's live slots
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const MetaView mv = stage_meta(f, &meta);
    const int n_tiles = tiles_m * tiles_n;
    const int kz = SPLIT ? (int)blockIdx.x / n_tiles : 0;
    int tm, tn;
    tile_coords(SPLIT ? (int)blockIdx.x - kz * n_tiles : (int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int mend = min(M, m0 + BM);
    const int kb = SPLIT ? kz * so.kc : 0;             // this block's k range [kb, kb + Kr)
    const int Kr = SPLIT ? min(K - kb, so.kc) : K;
    const int nk = (Kr + BK - 1) / BK;
    // load instruction u of the tile fetches rows (u / 8) * 64 + u % 8 + 8 i
    // (rows past M or N are clamped; their outputs are not stored)
    const int rl = lane >> 3, cl = lane & 7;
    int prow[DA], ncol[DB];
    const uint16_t* ap[DA];
    const uint16_t* bp[DB];
#pragma unroll
    for (int b = 0; b < DA; ++b) {
        const int u = wave * DA + b;
        prow[b] = m0 + (u >> 3) * 64 + (u & 7) + 8 * rl;
        ap[b] = X + (int64_t)f.token_order[min(prow[b], M - 1)] * K + kb + (cl ^ (u & 7)) * 8;
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        const int u = wave * DB + b;
        ncol[b] = n0 + (u >> 3) * 64 + (u & 7) + 8 * rl;
        bp[b] = W + (int64_t)min(ncol[b], N - 1) * K + kb + (cl ^ (u & 7)) * 8;
    }
    // the buffer form's resources and this lane's byte offsets of its rows
    const brsrc rX = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
    const brsrc rW = make_rsrc(W + (int64_t)n0 * K, (uint32_t)(min(N, n0 + BN) - n0) * (uint32_t)K * 2u);
    const brsrc rE = make_rsrc(f.ext, (uint32_t)M * (uint32_t)f.rp * 4u);
    const brsrc rB = make_rsrc(f.B_pool, (uint32_t)f.S * (uint32_t)N * (uint32_t)f.r_max * 2u);
    uint32_t aoff[DA], boff[DB];
    if constexpr (BUF) {
#pragma unroll
        for (int b = 0; b < DA; ++b)
            aoff[b] = (uint32_t)(f.token_order[min(prow[b], M - 1)] * K + (cl ^ ((wave * DA + b) & 7)) * 8) * 2u;
#pragma unroll
        for (int b = 0; b < DB; ++b)
            boff[b] = (uint32_t)((min(ncol[b], N - 1) - n0) * K + (cl ^ ((wave * DB + b) & 7)) * 8) * 2u;
    }
    uint32_t vsrc[ND];  // buffer form: per-lane offsets of an extra step, or of a K-tail base step
    uint32_t soff = 0;  // buffer form: the base step's k, in bytes
    __syncthreads();  // slot metadata staged
    // the expand's extra steps; in a split, split kz takes extra steps kz,
    // kz + ks, kz + 2 ks, ... of the tile (the partials carry the correction)
    const int ks = SPLIT ? (int)gridDim.x / n_tiles : 1;
    const lds_meta_ptr lmeta = (lds_meta_ptr)&meta;
    const lds_u16_ptr wlist = (lds_u16_ptr)xlist;
    const ExtraSched xs = extra_schedule(f.adapters && f.ext, lmeta, f.S, m0, mend, f.rp, wlist, wave == 0);
    if (xs.n > 0) __syncthreads();  // the slot list written
    const int ne_all = xs.steps();
    const int ne = __builtin_amdgcn_readfirstlane(SPLIT ? (ne_all > kz ? (ne_all - kz + ks - 1) / ks : 0) : ne_all);
    const int nt = nk + ne;
    // sources of step kt's load instructions (A 0..DA-1, then B), set once
    // per step
    gptr<u32x4> src[ND];
    // lane cl fetches chunk cl ^ (u % 8) with load instruction u
    auto sources_base = [&](int kt) {
        const int k = (kt - ne) * BK;
        if constexpr (BUF) {
            soff = (uint32_t)k * 2u;
            if constexpr (KTAIL) {
#pragma unroll
                for (int b = 0; b < DA; ++b)
                    vsrc[b] = k + (cl ^ ((wave * DA + b) & 7)) * 8 < Kr ? aoff[b] : kOutOfRange;
#pragma unroll
                for (int b = 0; b < DB; ++b)
                    vsrc[DA + b] = k + (cl ^ ((wave * DB + b) & 7)) * 8 < Kr ? boff[b] : kOutOfRange;
            }
            return;
        }
#pragma unroll
        for (int b = 0; b < DA; ++b) {
            const bool kin = !KTAIL || k + (cl ^ ((wave * DA + b) & 7)) * 8 < Kr;
            src[b] = KTAIL ? or_zero(kin, ap[b] + k) : as_global<u32x4>(ap[b] + k);
        }
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const bool kin = !KTAIL || k + (cl ^ ((wave * DB + b) & 7)) * 8 < Kr;
            src[DA + b] = KTAIL ? or_zero(kin, bp[b] + k) : as_global<u32x4>(bp[b] + k);
        }
    };
    // W is the left operand (acc holds blocks of W x^T, a lane 4 consecutive
    // columns of one row) except in a split, whose partials take the split-K
    // path's orientation (a lane 4 consecutive rows of one column)
    auto mfma = [&](f32x4& c, const u32x4& a, const u32x4& w) {
        if constexpr (SPLIT) mfma_agpr(c, a, w);
        else mfma_agpr(c, w, a);
    };
    auto sources_extra = [&](int kt) {
        const ExtraStepMeta xm = extra_step(xs, lmeta, wlist, kz + ks * kt);  // the tile's step of this split
        if constexpr (BUF) {
#pragma unroll
            for (int b = 0; b < DA; ++b) {
                const ExtraChunk c = extra_chunk(xs, xm, cl ^ ((wave * DA + b) & 7), f.rp);
                vsrc[b] = c.ok && prow[b] >= c.sb && prow[b] < c.se ? (uint32_t)(prow[b] * 2 * f.rp + c.k) * 2u
                                                                    : kOutOfRange;
            }
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const ExtraChunk c = extra_chunk(xs, xm, cl ^ ((wave * DB + b) & 7), f.rp);
                vsrc[DA + b] =
                    c.ok && ncol[b] < N ? (uint32_t)((c.s * N + ncol[b]) * f.r_max + c.q) * 2u : kOutOfRange;
            }
            return;
        }
#pragma unroll
        for (int b = 0; b < DA; ++b) {
            const ExtraChunk c = extra_chunk(xs, xm, cl ^ ((wave * DA + b) & 7), f.rp);
            src[b] = or_zero(c.ok && prow[b] >= c.sb && prow[b] < c.se, f.ext + (int64_t)prow[b] * 2 * f.rp + c.k);
        }
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const ExtraChunk c = extra_chunk(xs, xm, cl ^ ((wave * DB + b) & 7), f.rp);
            src[DA + b] = or_zero(c.ok && ncol[b] < N, f.B_pool + ((int64_t)c.s * N + ncol[b]) * f.r_max + c.q);
        }
    };
    // XN: the loads are of an extra step (in the buffer form: ext and B_pool
    // with per-lane offsets; else x and W)
    auto load_piece = [&](int g, int buf, auto xn_tag) {
        constexpr bool XN = decltype(xn_tag)::value;
        const int u = g < DA ? wave * DA + g : wave * DB + (g - DA);
        u32x4* dst = lds + buf * STAGE + ((g < DA ? 0 : ABYTES) + (u >> 3) * kGroupBytes + (u & 7) * kInstrBytes) / 16;
        if constexpr (BUF) {
            if constexpr (XN) bdma16(g < DA ? rE : rB, vsrc[g], 0u, dst);
            else bdma16(g < DA ? rX : rW, KTAIL ? vsrc[g] : (g < DA ? aoff[g] : boff[g - DA]), soff, dst);
        } else {
            dma16(src[g], dst);
        }
    };
    using XT = std::true_type;
    using XF = std::false_type;
    const int fr = lane & 15, fc = lane >> 4;
    const uint32_t lane_off = lds_offset(lds) + (fr & 7) * kInstrBytes + (fr >> 3) * 128;
    uint32_t abase[2], bbase[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // chunk h * 4 + fc of row fr sits at slot (h * 4 + fc) ^ (fr % 8)
        abase[h] = lane_off + block_off(wm * FI * 16) + ((h * 4 + fc) ^ (fr & 7)) * 16;
        bbase[h] = lane_off + ABYTES + block_off(wn * FJ * 16) + ((h * 4 + fc) ^ (fr & 7)) * 16;
    }
    u32x4 A0[FI], B0[FJ], A1[FI], B1[FJ];
    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // steps 0 .. L - 1 in flight, step 0 landed, its first half read
#pragma unroll
    for (int s0 = 0; s0 < L; ++s0) {
        if (s0 < ne) {
            sources_extra(s0);
#pragma unroll
            for (int g = 0; g < ND; ++g) load_piece(g, s0, XT{});
        } else {
            sources_base(min(s0, nt - 1));
#pragma unroll
            for (int g = 0; g < ND; ++g) load_piece(g, s0, XF{});
        }
    }
    vm_landed<(L - 1) * ND>();
    stage_barrier();
    static_for(std::make_integer_sequence<int, (FI > FJ ? FI : FJ)>{}, [&](auto ic) {
        constexpr int i = decltype(ic)::v;
        if constexpr (i < FJ) B0[i] = lds_read16<block_off(16 * i)>(bbase[0]);
        if constexpr (i < FI) A0[i] = lds_read16<block_off(16 * i)>(abase[0]);
    });
    // fragment read r of a half: B blocks first (the first MFMAs need all of them)
    auto read_half = [&](auto rc, u32x4 (&A)[FI], u32x4 (&B)[FJ], uint32_t ab, uint32_t bb) {
        constexpr int r = decltype(rc)::v;
        if constexpr (r < FJ) B[r] = lds_read16<block_off(16 * r)>(bb);
        else A[r - FJ] = lds_read16<block_off(16 * (r - FJ))>(ab);
    };
    // one step; `next` sets the sources of step kt + L, loaded into buffer bn
    // (step kt's own buffer with 2 stages: only after every wave has read it)
    // bcv: the buffer of step kt (kt % NS), a run-time int or a constant
    auto step = [&](int kt, auto&& next, auto xn_tag, auto bcv) {
        int bc;
        if constexpr (std::is_integral_v<decltype(bcv)>) bc = bcv;
        else bc = decltype(bcv)::v;
        const int bn = bc + L >= 2 * NS ? bc + L - 2 * NS : bc + L >= NS ? bc + L - NS : bc + L;  // step kt + L's
        const uint32_t so = bc * STAGE * 16, sn = (bc + 1 == NS ? 0 : bc + 1) * STAGE * 16;
        next(kt + L);
        frags_landed(A0);
        frags_landed(B0);
        // phase A: MFMAs of the first half, reads of the second half. In a
        // group, the fragment read follows the group's first MFMA and its
        // loads the second, so that each waits in an MFMA's shadow.
        static_for(std::make_integer_sequence<int, NR>{}, [&](auto gc) {
            constexpr int g = decltype(gc)::v;
            constexpr int t0 = (g * NM + NR - 1) / NR, t1 = ((g + 1) * NM + NR - 1) / NR;  // this group's MFMAs
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (t0 < t1) mfma(acc[t0 / FJ][t0 % FJ], A0[t0 / FJ], B0[t0 % FJ]);
            __builtin_amdgcn_sched_barrier(0);
            read_half(gc, A1, B1, abase[1] + so, bbase[1] + so);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (t0 + 1 < t1) mfma(acc[(t0 + 1) / FJ][(t0 + 1) % FJ], A0[(t0 + 1) / FJ], B0[(t0 + 1) % FJ]);
            __builtin_amdgcn_sched_barrier(0);
            static_for(std::make_integer_sequence<int, ND>{}, [&](auto pc) {  // loads of this group
                constexpr int pi = decltype(pc)::v;
                if constexpr (pi < NDA && pi * NR / NDA == g) load_piece(pi, bn, xn_tag);
            });
            __builtin_amdgcn_sched_barrier(0);
            static_for(std::make_integer_sequence<int, NM>{}, [&](auto tc) {  // the group's other MFMAs
                constexpr int t = decltype(tc)::v;
                if constexpr (t >= t0 + 2 && t < t1) mfma(acc[t / FJ][t % FJ], A0[t / FJ], B0[t % FJ]);
            });
        });
        __builtin_amdgcn_sched_barrier(0);
        frags_retire(A0, B0);
        frags_landed(A1);
        frags_landed(B1);
        vm_landed<VM_MID>();  // step kt + 1 landed (this wave's loads; those of later steps may not)
        stage_barrier();
        // phase B: MFMAs of the second half, reads of step kt + 1's first half, the other loads
        static_for(std::make_integer_sequence<int, NR>{}, [&](auto gc) {
            constexpr int g = decltype(gc)::v;
            constexpr int t0 = (g * NM + NR - 1) / NR, t1 = ((g + 1) * NM + NR - 1) / NR;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (t0 < t1) mfma(acc[t0 / FJ][t0 % FJ], A1[t0 / FJ], B1[t0 % FJ]);
            __builtin_amdgcn_sched_barrier(0);
            read_half(gc, A0, B0, abase[0] + sn, bbase[0] + sn);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (t0 + 1 < t1) mfma(acc[(t0 + 1) / FJ][(t0 + 1) % FJ], A1[(t0 + 1) / FJ], B1[(t0 + 1) % FJ]);
            __builtin_amdgcn_sched_barrier(0);
            static_for(std::make_integer_sequence<int, ND>{}, [&](auto pc) {
                constexpr int pi = decltype(pc)::v;
                if constexpr (pi >= NDA && (pi - NDA) * NR / NDB == g) load_piece(pi, bn, xn_tag);
            });
            __builtin_amdgcn_sched_barrier(0);
            static_for(std::make_integer_sequence<int, NM>{}, [&](auto tc) {
                constexpr int t = decltype(tc)::v;
                if constexpr (t >= t0 + 2 && t < t1) mfma(acc[t / FJ][t % FJ], A1[t / FJ], B1[t % FJ]);
            });
        });
        __builtin_amdgcn_sched_barrier(0);
        frags_retire(A1, B1);
    };
    // steps whose step kt + L is an extra step, then the rest (the last L
    // steps reload the last step: the load count per step stays fixed). The
    // base steps run NS to an iteration, so that their buffers, and with them
    // every LDS address of the step, are constants.
    int kt = 0, bcr = 0;  // bcr = kt % NS
    auto adv = [&] { bcr = bcr + 1 == NS ? 0 : bcr + 1; };
    auto base_next = [&](int s) { sources_base(min(s, nt - 1)); };
    for (; kt + L < ne; ++kt, adv()) step(kt, sources_extra, XT{}, bcr);
    for (; kt < nt && bcr != 0; ++kt, adv()) step(kt, base_next, XF{}, bcr);
    for (; kt + NS <= nt; kt += NS)
        static_for(std::make_integer_sequence<int, NS>{}, [&](auto sc) { step(kt + decltype(sc)::v, base_next, XF{}, sc); });
    for (; kt < nt; ++kt, adv()) step(kt, base_next, XF{}, bcr);
    frags_landed(A0);
    frags_landed(B0);
    vm_landed<0>();
#pragma unroll
    for (int i = 0; i < 12; ++i) asm volatile("s_nop 7");  // last MFMA results written
    const int p0 = m0 + wm * FI * 16, nb = n0 + wn * FJ * 16;
    if constexpr (SPLIT) {
        f32x4* out = reinterpret_cast<f32x4*>(so.part) + (int64_t)kz * so.n_mt * so.n_nt * 1024;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int rb = p0 / 16 + i;  // 16-row block
            if ((rb >> 2) >= so.n_mt) continue;
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int cb = nb / 16 + j;
                if ((cb >> 2) >= so.n_nt) continue;
                out[((int64_t)(rb >> 2) * so.n_nt + (cb >> 2)) * 1024 + ((rb & 3) * 4 + (cb & 3)) * 64 + lane] = acc[i][j];
            }
        }
        return;
    }
    if constexpr (EPI) fused_expand<FI, FJ>(acc, f, mv, p0, nb, M, N, lane);
    static_assert(NW * FI * FJ * 16 * 16 * 2 <= NS * STAGE * 16, "output staging");
    __syncthreads();
    store_tile<FI, FJ>(acc, reinterpret_cast<char*>(lds) + wave * (FI * 16) * (FJ * 32), Y, f.token_order, p0, nb, M,
                       N, lane);
}

// ------------------------------------------------------------------ plan --
GemmPlan gemm_bf16_plan(int M, int N, int K) {
    GemmPlan g{};
    if (M <= 0 || N <= 0 || K <= 0) return g;  // nothing to launch
    // tiled path: the macro tile with the least (rounds of 256 tiles) x (time
    // of one tile); the relative tile times are measured ones (K = 4096:
    // 256 x 256 96.5 us, 256 x 128 55 us, 128 x 128 39.5 us, 64 x 128 30 us)
    auto n_tiles = [&](int bm, int bn) { return (int64_t)cdiv(M, bm) * cdiv(N, bn); };
    if (n_tiles(256, 256) >= 200 || (M > 256 && n_tiles(64, 128) >= 128)) {
        struct Cand {
            int bm, bn;
            double t;
        };
        constexpr Cand cands[] = {{256, 256, 96.5}, {256, 128, 55.0}, {128, 128, 39.5}, {64, 128, 30.0}};
        double best = 0.0;
        for (const Cand& c : cands) {
            const double cost = (double)((n_tiles(c.bm, c.bn) + 255) / 256) * c.t;
            if (g.bm == 0 || cost < best) {
                best = cost;
                g.bm = c.bm;
                g.bn = c.bn;
            }
        }
        // or 256 x 128 tiles split over K (few tiles, long K): each split's
        // tile time scales with its k range, plus its fp32 partial writes (at
        // 5 TB/s) and ~7 us of fill and drain; then the reduction reads the
        // partials and writes y (at 4.4 TB/s, + 1 us). Measured at T = 512:
        // 14336 -> 4096 split 4 ways 63 + 7 us against ~105 us unsplit;
        // 4096 -> 4096 stays unsplit (33 us).
        const double plain = best * K / 4096.0;
        double best_split = 0.9 * plain;  // taken only when clearly cheaper
        for (int ks = 2; ks <= 8; ks *= 2) {
            const int kc = cdiv(cdiv(K, ks), 64) * 64;
            const int kse = cdiv(K, kc);
            if (kc < 512 || kse < 2) break;
            const double part_bytes = kse * (double)M * N * 4.0;
            const double cost = (double)((n_tiles(256, 128) * kse + 255) / 256) * 55.0 * kc / 4096.0 +
                                part_bytes / 5.0e6 + 7.0 + (part_bytes + (double)M * N * 2.0) / 4.4e6 + 1.0;
            if (cost < best_split) {
                best_split = cost;
                g.tks = kse;
                g.tkc = kc;
            }
        }
        if (g.tks > 1) {
            g.bm = 256;
            g.bn = 128;
        }
        return g;
    }
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
    return g;
}

// Workspace of the split-K pass over all slices together.
static size_t split_workspace(int M, int n_nt_total, const GemmPlan& g, int n_slices, int r_max) {
    const size_t py = (size_t)g.ks * g.n_mt * n_nt_total * 16 * 64 * 16;
    // h planes: the GEMM's ks splits (shrink tiles) or up to 8 shrink splits
    const size_t ph = (size_t)n_slices * max(g.ks, 8) * M * r_max * sizeof(float);
    return ((py + 255) & ~size_t(255)) + ((ph + 255) & ~size_t(255));
}

// tiled path: fp32 h [M][r_max] or bf16 hi / lo [M][2][round_up(r_max, 8)],
// then the K-split shrink's planes (at most kShrinkSplitMaxBlocks x 16 rows)
static size_t tiled_workspace(int M, int r_max) {
    const size_t h_final = (size_t)M * ((r_max + 7) & ~7) * sizeof(float);
    const size_t planes = (size_t)kShrinkSplitMaxBlocks * 16 * r_max * sizeof(float);
    return ((h_final + 255) & ~size_t(255)) + planes;
}

// one slice's expand operand (bf16 hi / lo, [M][2][rp]) in the workspace
static size_t ext_stride(int M, int r_max) {
    return ((size_t)M * ((r_max + 7) & ~7) * sizeof(float) + 255) & ~size_t(255);
}

static int total_tiles_n(const int* N, int n_slices) {
    int t = 0;
    for (int i = 0; i < n_slices; ++i) t += cdiv(N[i], 64);
    return t;
}

// Slices share one pass when their concatenated columns take the split-K
// path; otherwise each slice runs on its own (tiled or split-K).
static bool joint_split(int M, const int* N, int n_slices, int K, GemmPlan* out) {
    int n_total = 0;
    for (int i = 0; i < n_slices; ++i) n_total += N[i];
    const GemmPlan g = gemm_bf16_plan(M, n_total, K);
    if (out) *out = g;
    return g.nsub != 0;
}

// tiled path split over K: the partials, then the tiled path's h area
static size_t split_tiled_workspace(int M, int N, const GemmPlan& g, int r_max) {
    const size_t py = ((size_t)g.tks * cdiv(M, 64) * cdiv(N, 64) * 16 * 64 * 16 + 255) & ~size_t(255);
    return py + tiled_workspace(M, r_max);
}

size_t gemm_bf16_workspace(int M, const int* N, int n_slices, int K, int r_max) {
    if (M <= 0 || K <= 0 || n_slices < 1) return 0;
    GemmPlan gj;
    if (n_slices > 1 && joint_split(M, N, n_slices, K, &gj)) {
        // the joint plan's tiles are those of the concatenated columns;
        // count whole 64-column tiles per slice
        GemmPlan g = gj;
        g.n_nt = total_tiles_n(N, n_slices);
        return split_workspace(M, g.n_nt, g, n_slices, r_max);
    }
    // several slices may share one shrink: an expand operand area per slice
    size_t need = n_slices > 1 ? n_slices * ext_stride(M, r_max) : 0;
    for (int i = 0; i < n_slices; ++i) {
        if (N[i] <= 0) continue;
        const GemmPlan g = gemm_bf16_plan(M, N[i], K);
        const size_t b = g.nsub != 0 ? split_workspace(M, g.n_nt, g, 1, r_max)
                         : g.tks > 1 ? split_tiled_workspace(M, N[i], g, r_max)
                                     : tiled_workspace(M, r_max);
        need = b > need ? b : need;
    }
    return need;
}

// Whether every buffer the tile kernel's buffer form reads fits a buffer
// resource (under 2 GiB, so per-lane byte offsets and the out-of-range offset
// stay apart): x, one tile's W rows, ext, B_pool.
static bool buffers_fit(int M, int N, int K, int BN, const Fuse& f) {
    const int64_t lim = int64_t(1) << 31;
    return (int64_t)M * K * 2 < lim && (int64_t)BN * K * 2 < lim && (int64_t)M * f.rp * 4 < lim &&
           (int64_t)f.S * N * f.r_max * 2 < lim;
}

template <int BM, int BN, int WM, int WN, int NS, bool SPLIT_OK, bool BUF_OK = false>
static hipError_t launch_tile(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K, const Fuse& f,
                            bool epi, hipStream_t st, StageTimer* tm, const SplitOut& so = SplitOut{}, int ks = 1) {
    const int tiles_m = cdiv(M, BM), tiles_n = cdiv(N, BN);
    const bool ktail = K % 64 != 0;
    const dim3 block(64 * WM * WN);
    decltype(&gemm_tile_kernel<BM, BN, WM, WN, NS, false, false, false, false>) ker;
    if constexpr (SPLIT_OK) {
        if (so.part) {
            ker = ktail ? gemm_tile_kernel<BM, BN, WM, WN, NS, false, true, true, false>
                        : gemm_tile_kernel<BM, BN, WM, WN, NS, false, false, true, false>;
            return launch(tm, "gemm_bf16", ker, dim3(tiles_m * tiles_n * ks), block, st, X, W, Y, M, N, K, tiles_m,
                          tiles_n, f, so);
        }
    }
    bool buf = false;
    if constexpr (BUF_OK) buf = buffers_fit(M, N, K, BN, f);
    if (buf) {
        if constexpr (BUF_OK)
            ker = epi ? (ktail ? gemm_tile_kernel<BM, BN, WM, WN, NS, true, true, false, true>
                               : gemm_tile_kernel<BM, BN, WM, WN, NS, true, false, false, true>)
                      : (ktail ? gemm_tile_kernel<BM, BN, WM, WN, NS, false, true, false, true>
                               : gemm_tile_kernel<BM, BN, WM, WN, NS, false, false, false, true>);
    } else {
        ker = epi ? (ktail ? gemm_tile_kernel<BM, BN, WM, WN, NS, true, true, false, false>
                           : gemm_tile_kernel<BM, BN, WM, WN, NS, true, false, false, false>)
                  : (ktail ? gemm_tile_kernel<BM, BN, WM, WN, NS, false, true, false, false>
                           : gemm_tile_kernel<BM, BN, WM, WN, NS, false, false, false, false>);
    }
    return launch(tm, "gemm_bf16", ker, dim3(tiles_m * tiles_n), block, st, X, W, Y, M, N, K, tiles_m, tiles_n, f,
                  SplitOut{});
}

// The shrink of the tiled path, into fp32 h [M][r_max] or, with ext, the
// expand operand of the extra K steps; ws: h_final bytes for h or ext, then
// the K-split shrink's planes.
static hipError_t tiled_shrink(const LinearArgs& L, const SliceArgs& sl, char* ws, float* h, uint16_t* ext,
                               hipStream_t st, StageTimer* tm) {
    const int M = L.M, K = L.K;
    // few items over a long K: split K over more workgroups, then add the splits
    int hs = 1, hkc = K;
    if (L.n_items < kShrinkSplitMaxBlocks / 2) {
        hs = min(8, kShrinkSplitMaxBlocks / max(L.n_items, 1));
        hkc = max(256, (cdiv(K, hs) + 31) / 32 * 32);
        hs = cdiv(K, hkc);
    }
    const size_t h_final = (size_t)M * ((L.r_max + 7) & ~7) * sizeof(float);
    float* part = reinterpret_cast<float*>(ws + ((h_final + 255) & ~size_t(255)));
    return hs > 1 ? sgmv_shrink_split(L.X, sl.A_pool, sl.rank, sl.scale, L.token_order, L.work, L.n_items, hs, hkc,
                                      part, h, ext, K, L.r_max, st, tm)
                  : sgmv_shrink(L.X, sl.A_pool, sl.rank, L.token_order, L.work, L.n_items, h, K, L.r_max, st, tm,
                                sl.scale, ext);
}

// One slice on the tiled path split over K: the shrink to the expand operand,
// the 256 x 128 kernel writing partials (the extra K steps dealt round the
// splits), then the split-K path's kernel 2 without adapters (adds the
// partials, rounds).
// Without the extra-step form of the expand (r_max % 8 != 0, or pools of more
// than kMetaSlots slots), or when the extra steps would add more than a fifth
// to a split, the slice runs unsplit.
static hipError_t tiled_forward(const LinearArgs& L, const SliceArgs& sl, const GemmPlan& g, hipStream_t st,
                                StageTimer* tm, uint16_t* ext_ready = nullptr);
static hipError_t split_tiled_forward(const LinearArgs& L, const SliceArgs& sl, const GemmPlan& g, hipStream_t st,
                                      StageTimer* tm) {
    const bool ext_ok = L.r_max % 8 == 0 && L.S <= kMetaSlots;
    // extra steps per 256-row tile, from the live slots of 256 rows bounded
    // by the work items (16 rows of one slot each) that fall in them (64 /
    // (2 rp) slots share a step when 2 rp divides 64); spread over the splits
    // they should stay small next to a split's base steps
    const int64_t items_per_tile = ((int64_t)L.n_items * 256 + L.M - 1) / L.M;
    const int64_t slots_per_tile = items_per_tile < L.S ? items_per_tile : (int64_t)L.S;
    const int r2 = 2 * ((L.r_max + 7) & ~7);
    const int64_t est_extra = 64 % r2 == 0 ? (slots_per_tile * r2 + 63) / 64 : slots_per_tile * cdiv(r2, 64);
    if (L.adapters && (!ext_ok || est_extra * 5 > (int64_t)g.tks * (g.tkc / 64))) {
        GemmPlan gu = g;
        gu.tks = 0;
        return tiled_forward(L, sl, gu, st, tm);
    }
    const int M = L.M, N = sl.N, K = L.K;
    const int n_mt = cdiv(M, 64), n_nt = cdiv(N, 64);
    char* ws = static_cast<char*>(L.workspace);
    const size_t py = ((size_t)g.tks * n_mt * n_nt * 16 * 64 * 16 + 255) & ~size_t(255);
    float* part = reinterpret_cast<float*>(ws);
    uint16_t* ext = reinterpret_cast<uint16_t*>(ws + py);
    if (L.adapters) {
        const hipError_t e = tiled_shrink(L, sl, ws + py, nullptr, ext, st, tm);
        if (e != hipSuccess) return e;
    }
    const Fuse f{L.token_order, L.slot_indptr, nullptr, sl.B_pool, sl.rank, sl.scale, L.S, L.r_max, 1, 0, L.adapters,
                 ext, (L.r_max + 7) & ~7};
    const hipError_t e =
        launch_tile<256, 128, 4, 2, 3, true>(L.X, sl.W, nullptr, M, N, K, f, false, st, tm, SplitOut{part, g.tkc, n_mt, n_nt},
                                     g.tks);
    if (e != hipSuccess) return e;
    LinearArgs base = L;
    base.adapters = 0;
    return splitk_finish_bf16(base, sl, part, g.tks, n_mt, nullptr, 1, st, tm);
}

// One slice on the tiled path: the shrink to final h, then the tiled GEMM
// with the expand fused (r_max % 8 == 0: as extra K steps from scaled h as
// bf16 hi / lo; otherwise in the epilogue from fp32 h). With ext_ready the
// expand operand was already written there (several slices, one shrink).
static hipError_t tiled_forward(const LinearArgs& L, const SliceArgs& sl, const GemmPlan& g, hipStream_t st,
                                StageTimer* tm, uint16_t* ext_ready) {
    if (g.tks > 1) return split_tiled_forward(L, sl, g, st, tm);
    const int M = L.M, N = sl.N, K = L.K;
    Fuse f{L.token_order, L.slot_indptr, nullptr, sl.B_pool, sl.rank, sl.scale, L.S, L.r_max, 1, 0, L.adapters,
           nullptr, (L.r_max + 7) & ~7};
    char* ws = static_cast<char*>(L.workspace);
    float* hbuf = reinterpret_cast<float*>(ws);
    // the expand as extra K steps needs r_max % 8 == 0 and the slot metadata in LDS
    uint16_t* ext = (L.r_max % 8 == 0 && L.S <= kMetaSlots) ? reinterpret_cast<uint16_t*>(ws) : nullptr;
    if (ext_ready) ext = ext_ready;
    f.h = ext ? nullptr : hbuf;
    f.ext = ext;
    if (L.adapters && !ext_ready) {
        const hipError_t e = tiled_shrink(L, sl, ws, ext ? nullptr : hbuf, ext, st, tm);
        if (e != hipSuccess) return e;
    }
    const bool epi = L.adapters && !f.ext;
    if (g.bm == 256 && g.bn == 256) return launch_tile<256, 256, 2, 2, 2, false, true>(L.X, sl.W, sl.Y, M, N, K, f, epi, st, tm);
    if (g.bm == 256) return launch_tile<256, 128, 4, 2, 3, false>(L.X, sl.W, sl.Y, M, N, K, f, epi, st, tm);
    if (g.bm == 128) return launch_tile<128, 128, 2, 4, 3, false>(L.X, sl.W, sl.Y, M, N, K, f, epi, st, tm);
    return launch_tile<64, 128, 2, 4, 4, false>(L.X, sl.W, sl.Y, M, N, K, f, epi, st, tm);
}

// Several slices that all take the unsplit tiled path with the expand as
// extra K steps share one shrink (x rows read once), each slice's operand in
// its own workspace area; enough items that the single-slice shrink would not
// split K either, so each operand equals that slice's own bit for bit.
static bool slices_share_shrink(const LinearArgs& L, const int* N, GemmPlan* gs) {
    if (L.n_slices < 2 || !L.adapters || L.r_max % 8 != 0 || L.S > kMetaSlots ||
        L.n_items < kShrinkSplitMaxBlocks / 2)
        return false;
    for (int i = 0; i < L.n_slices; ++i) {
        if (N[i] <= 0) return false;
        gs[i] = gemm_bf16_plan(L.M, N[i], L.K);
        if (gs[i].nsub != 0 || gs[i].tks > 1) return false;
    }
    return true;
}

hipError_t lora_forward_bf16(const LinearArgs& L, hipStream_t st, StageTimer* tm) {
    const int M = L.M, K = L.K, n = L.n_slices;
    if (M == 0 || n < 1) return hipSuccess;
    int N[kMaxSlices];
    for (int i = 0; i < n; ++i) N[i] = L.slice[i].N;
    GemmPlan gj;
    if (n > 1 && joint_split(M, N, n, K, &gj)) return splitk_forward_bf16(L, gj, st, tm);
    GemmPlan gs[kMaxSlices];
    if (slices_share_shrink(L, N, gs)) {
        ShrinkSlices ss{};
        ss.n = n;
        char* ws = static_cast<char*>(L.workspace);
        for (int i = 0; i < n; ++i) {
            ss.A_pool[i] = L.slice[i].A_pool;
            ss.rank[i] = L.slice[i].rank;
            ss.scale[i] = L.slice[i].scale;
            ss.ext[i] = reinterpret_cast<uint16_t*>(ws + i * ext_stride(M, L.r_max));
        }
        hipError_t e = sgmv_shrink_slices(L.X, ss, L.token_order, L.work, L.n_items, K, L.r_max, st, tm);
        for (int i = 0; i < n && e == hipSuccess; ++i) e = tiled_forward(L, L.slice[i], gs[i], st, tm, ss.ext[i]);
        return e;
    }
    for (int i = 0; i < n; ++i) {
        if (N[i] == 0) continue;
        const GemmPlan g = gemm_bf16_plan(M, N[i], K);
        hipError_t e;
        if (g.nsub == 0) {
            e = tiled_forward(L, L.slice[i], g, st, tm);
        } else {
            LinearArgs one = L;
            one.n_slices = 1;
            one.slice[0] = L.slice[i];
            e = splitk_forward_bf16(one, g, st, tm);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lora
