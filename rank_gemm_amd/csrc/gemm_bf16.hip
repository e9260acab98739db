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
//  * tiled (prefill-sized T, this file): 256 x 256 macro tiles over 8 waves
//    with K in stages of 32 through a 3-deep LDS ring filled by direct-to-LDS
//    loads (128 x 128 and 64 x 128 tiles with 4 waves and register-staged
//    loads for smaller T); the shrink runs before it as its own kernel.
//  * split-K (decode-sized T, splitk.hip): a K-split GEMM with the shrink in
//    extra workgroups of the same launch, then a kernel that adds the splits
//    and applies the expand.
#include "fuse.h"

#include <type_traits>

namespace lora {

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

// ------------------------------------------------------------------ plan --
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

// Workspace of the split-K pass over all slices together.
static size_t split_workspace(int M, int n_nt_total, const GemmPlan& g, int n_slices, int r_max) {
    const size_t py = (size_t)g.ks * g.n_mt * n_nt_total * 16 * 64 * 16;
    const size_t ph = (size_t)n_slices * g.hs * M * r_max * sizeof(float);
    return ((py + 255) & ~size_t(255)) + ((ph + 255) & ~size_t(255));
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
    size_t need = 0;
    for (int i = 0; i < n_slices; ++i) {
        if (N[i] <= 0) continue;
        const GemmPlan g = gemm_bf16_plan(M, N[i], K);
        // fp32 h [M][r_max], or bf16 hi / lo [M][2][round_up(r_max, 8)]
        const size_t h_final = (size_t)M * ((r_max + 7) & ~7) * sizeof(float);
        const size_t b = g.nsub == 0 ? ((h_final + 255) & ~size_t(255)) : split_workspace(M, g.n_nt, g, 1, r_max);
        need = b > need ? b : need;
    }
    return need;
}

template <int BM, int BN>
static hipError_t launch_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K,
                               const Fuse& f, hipStream_t st, StageTimer* tm) {
    const int tiles_m = cdiv(M, BM), tiles_n = cdiv(N, BN);
    return launch(tm, "gemm_bf16", gemm_tiled_kernel<BM, BN>, dim3(tiles_m * tiles_n), dim3(kThreads), st, X, W, Y,
                  M, N, K, tiles_m, tiles_n, f);
}

// One slice on the tiled path: the shrink to final h, then the tiled GEMM
// with the expand fused (r_max % 8 == 0: as extra K steps from scaled h as
// bf16 hi / lo; otherwise in the epilogue from fp32 h).
static hipError_t tiled_forward(const LinearArgs& L, const SliceArgs& sl, const GemmPlan& g, hipStream_t st,
                                StageTimer* tm) {
    const int M = L.M, N = sl.N, K = L.K;
    Fuse f{L.token_order, L.slot_indptr, nullptr, sl.B_pool, sl.rank, sl.scale, L.S, L.r_max, 1, 0, L.adapters,
           nullptr, (L.r_max + 7) & ~7};
    char* ws = static_cast<char*>(L.workspace);
    float* hbuf = reinterpret_cast<float*>(ws);
    uint16_t* ext = (L.r_max % 8 == 0) ? reinterpret_cast<uint16_t*>(ws) : nullptr;
    f.h = ext ? nullptr : hbuf;
    f.ext = ext;
    if (L.adapters) {
        const hipError_t e = sgmv_shrink(1, L.X, sl.A_pool, sl.rank, L.token_order, L.work, L.n_items,
                                         ext ? nullptr : hbuf, K, L.r_max, st, tm, sl.scale, ext);
        if (e != hipSuccess) return e;
    }
    if (g.bm == 256) {
        const int tiles_m = cdiv(M, 256), tiles_n = cdiv(N, 256);
        const bool epi = L.adapters && !f.ext, ktail = K % 32 != 0;
        auto ker = epi ? (ktail ? gemm_dma_kernel<true, true> : gemm_dma_kernel<true, false>)
                       : (ktail ? gemm_dma_kernel<false, true> : gemm_dma_kernel<false, false>);
        return launch(tm, "gemm_bf16", ker, dim3(tiles_m * tiles_n), dim3(512), st, L.X, sl.W, sl.Y, M, N, K,
                      tiles_m, tiles_n, f);
    }
    if (g.bm == 128) return launch_tiled<128, 128>(L.X, sl.W, sl.Y, M, N, K, f, st, tm);
    return launch_tiled<64, 128>(L.X, sl.W, sl.Y, M, N, K, f, st, tm);
}

hipError_t lora_forward_bf16(const LinearArgs& L, hipStream_t st, StageTimer* tm) {
    const int M = L.M, K = L.K, n = L.n_slices;
    if (M == 0 || n < 1) return hipSuccess;
    int N[kMaxSlices];
    for (int i = 0; i < n; ++i) N[i] = L.slice[i].N;
    GemmPlan gj;
    if (n > 1 && joint_split(M, N, n, K, &gj)) return splitk_forward_bf16(L, gj, st, tm);
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
