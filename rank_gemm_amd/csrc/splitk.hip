// Decode-sized T: the bf16 LoRA linear as a K-split GEMM plus a finishing
// kernel (the correction of "LoRA serving, embeddings, rerankers, pooling",
// mlinterviewnotes.com, opening section: base GEMM once over the batch, then
// the per-row indexed low-rank correction).
//
// Kernel 1 computes 64 x 64 output tiles over K splits, streaming the split's
// gathered x rows and W rows through a 5-deep LDS ring of 64-k stages by
// direct-to-LDS loads; extra tiles of the same launch compute the SGMV shrink
// over the same K splits, with the rows of a few work items in place of the
// batch rows and their slots' A rows in place of W rows. Kernel 2 adds the
// partial products in split order, applies the expand scale_s * h[p] B_s^T in
// fp32 and rounds once. No workgroup waits on another.
//
// Projections that read the same x (the output slices of a merged q/k/v or
// gate/up wrapper, section "vLLM: preallocated stacked buffers plus a
// Punica-style Triton kernel" of the same page) can share both launches:
// their 64-column tiles are numbered one after the other, and each tile takes
// the weight, output and adapter pool of the slice it falls in; the shrink
// workgroups cover every slice's A over the same K splits. The MULTI template
// flag keeps the one-slice kernels free of the slice lookup.
#include <cstddef>
#include <cstring>

#include "fuse.h"
#include "shrink.h"

namespace lora {

// -------------------------------------------------------------- split-K --
// The slices of one pass (projections reading the same x), their 64-column
// tiles numbered one after the other: slice i owns tiles nt0[i] .. nt0[i+1).
// One-slice kernels take a table of one entry: the kernel arguments stay
// small, and their layout measurably moves the kernels' start (a table of
// four entries made both decode kernels slower even with one slice).
template <int NSL>
struct SliceTable {
    int n;
    int nt0[NSL + 1];
    int N[NSL];
    const uint16_t* W[NSL];
    const uint16_t* A_pool[NSL];
    const uint16_t* B_pool[NSL];
    const int32_t* rank[NSL];
    const float* scale[NSL];
    uint16_t* Y[NSL];
};
using SliceTableAll = SliceTable<kMaxSlices>;
template <bool MULTI>
using SliceTableFor = SliceTable<MULTI ? kMaxSlices : 1>;

template <int NSL>
static SliceTable<NSL> table_of(const SliceTableAll& t) {
    SliceTable<NSL> r{};
    r.n = t.n;
    for (int i = 0; i < NSL; ++i) {
        r.nt0[i] = t.nt0[i];
        r.N[i] = t.N[i];
        r.W[i] = t.W[i];
        r.A_pool[i] = t.A_pool[i];
        r.B_pool[i] = t.B_pool[i];
        r.rank[i] = t.rank[i];
        r.scale[i] = t.scale[i];
        r.Y[i] = t.Y[i];
    }
    r.nt0[NSL] = t.nt0[NSL];
    return r;
}

// Entry i of a slice array, by selects (a dynamically indexed kernel
// argument would be copied to scratch memory).
template <class T, int NSL>
__device__ __forceinline__ T pick(const T (&v)[NSL], int i) {
    T r = v[0];
#pragma unroll
    for (int j = 1; j < NSL; ++j) r = i == j ? v[j] : r;
    return r;
}

template <int NSL>
__device__ __forceinline__ int nt_first(const SliceTable<NSL>& t, int i) {
    int r = t.nt0[0];
#pragma unroll
    for (int j = 1; j < NSL; ++j) r = i == j ? t.nt0[j] : r;
    return r;
}

template <int NSL>
__device__ __forceinline__ int slice_of(const SliceTable<NSL>& t, int nt) {
    int i = 0;
#pragma unroll
    for (int j = 1; j < NSL; ++j) i += (j < t.n && nt >= t.nt0[j]) ? 1 : 0;
    return i;
}

template <int NSL>
struct SplitArgs {
    const uint16_t* X;
    float* part_y;  // [ks][n_mt][n_nt][16 fragments][64 lanes] f32x4, n_nt over all slices
    int M, K, n_mt, n_nt, ks;
    // shrink tiles: groups of G work items, rc columns per item (r_max rounded
    // up to 16), E 64-column tiles per group
    const int32_t* token_order;
    const Item* work;
    int n_items, r_max;
    float* part_h;  // [n][planes][M][r_max], rows by sorted position
    // shrink workgroups (light shrinks): n_items * hs * n of them, hkc k
    // each, hs planes; hs == 0 when the shrink runs as tiles (ks planes)
    int hs, hkc;
    int n_groups, G, rc, E;
    SliceTable<NSL> sl;
};

// grid: n_items * hs * n shrink workgroups (light shrinks only), then
// n_mt * n_nt * ks GEMM blocks, then ks * n * n_groups * E shrink tiles (heavy
// shrinks only). The shrink workgroups run shrink_item over K ranges finer
// than the GEMM's splits, so that they finish early; a shrink tile has the
// shape of work of a GEMM block (a 64 x 64 tile over one K split). A CU's
// direct-to-LDS feed is the bound of this kernel: a GEMM block alone on a
// CU streams its 256 KB in ~6.3 us, two blocks on one CU take ~10.4 us each,
// so a few shrink tiles beside 256 GEMM blocks would set the kernel's time,
// while many shrink tiles move fewer bytes than per-item workgroups.
// Wave w of a block owns columns 16 w .. 16 w + 15 of its tile. The split's
// x rows (gathered through token_order) and W rows stream through
// kSplitStages LDS buffers of 64 k by direct-to-LDS loads: a stage is 8
// blocks each of x and of W, a block being 8 rows x 128 B; lane i of a block
// load fetches row i / 8, chunk (i % 8) ^ (row % 8), so that each load
// instruction reads whole 128-byte lines and the MFMA fragment reads (row
// l % 16, chunk l / 16) are free of bank conflicts. GEMM tiles clamp rows past
// M or N (their partials are not stored); chunks past K read zeros.
//
// A shrink tile of group g takes, as its row block i < G, the rows of work
// item g G + i, and as its column c the rank q = c' % rc of item c' / rc's
// slot (c' = 64 e + c), i.e. row q of that slot's A (the T x r bottleneck
// of the opening section of "LoRA serving, embeddings, rerankers,
// pooling", mlinterviewnotes.com). Only the blocks pairing an item's rows
// with its own slot's ranks are kept: they are h over the split's K range,
// written to the split's h plane. Ranks at or past r_s are never loaded
// (rank masking, "SGLang: chunked SGMV, and a rank-aware kernel"), a row
// block with no item issues no x loads, and a tile with no live item exits
// before loading anything.
constexpr int kSplitStages = 5;
constexpr int kSplitStageChunks = 1024;  // 16-byte chunks: x 512, W 512

template <int NSUB, bool MULTI, bool TILES>
__global__ __launch_bounds__(kThreads) void splitk_gemm_kernel(SplitArgs<MULTI ? kMaxSlices : 1> a) {
    __shared__ u32x4 lds[kSplitStages * kSplitStageChunks];  // 80 KB
    constexpr int KC = NSUB * 128, NST = NSUB * 2, NS = kSplitStages, SC = kSplitStageChunks;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = a.K;
    const int n_shrink = TILES ? 0 : a.n_items * a.hs * (MULTI ? a.sl.n : 1);
    if (!TILES && (int)blockIdx.x < n_shrink) {
        const int item = blockIdx.x % a.n_items, rest = blockIdx.x / a.n_items;
        const int hz = MULTI ? rest % a.hs : rest, hi = MULTI ? rest / a.hs : 0;
        const Item it = a.work[item];
        const int r = pick(a.sl.rank, hi)[it.slot];
        if (r == 0) return;
        const int kbeg = hz * a.hkc, kend = min(K, kbeg + a.hkc);
        const ShrinkOut out{a.part_h + ((int64_t)hi * a.hs + hz) * a.M * a.r_max, nullptr, 0, 0.f};
        shrink_item<4>(a.X, pick(a.sl.A_pool, hi), r, a.token_order, it, out, K, kbeg, kend, a.r_max,
                       reinterpret_cast<f32x4*>(lds));
        return;
    }
    const int b = blockIdx.x - n_shrink;
    const int n_gemm = a.n_mt * a.n_nt * a.ks;
    const bool gemm = !TILES || b < n_gemm;
    // this lane's rows and chunk in its two x and two W block loads
    const int dr = lane >> 3, dc = lane & 7;
    const uint16_t* xs[2];
    const uint16_t* ws[2];
    int kc[2];
    bool xv[2], wv[2];
    int kz, mt = 0, nt = 0, si = 0, g = 0, ex = 0;
    bool xl = true;  // wave-uniform: this wave loads x rows
    if (gemm) {
        const int tiles = a.n_mt * a.n_nt;
        kz = b / tiles;
        const int t = b - kz * tiles;
        mt = t / a.n_nt;
        nt = t - mt * a.n_nt;
        si = MULTI ? slice_of(a.sl, nt) : 0;
        const uint16_t* __restrict__ W = pick(a.sl.W, si);
        const int N = pick(a.sl.N, si);
        const int m0 = mt * 64, n0 = (nt - nt_first(a.sl, si)) * 64;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * wave + 8 * j + dr;  // tile row / column 0..63
            kc[j] = kz * KC + (dc ^ (r & 7)) * 8;  // this lane's k within a stage
            xs[j] = a.X + (int64_t)a.token_order[min(m0 + r, a.M - 1)] * K + kc[j];
            ws[j] = W + (int64_t)min(n0 + r, N - 1) * K + kc[j];
            xv[j] = wv[j] = true;
        }
    } else if constexpr (TILES) {
        int e = b - n_gemm;
        const int ge = a.n_groups * a.E;
        const int per_z = ge * (MULTI ? a.sl.n : 1);
        kz = e / per_z;
        e -= kz * per_z;
        si = MULTI ? e / ge : 0;
        e -= si * ge;
        g = e / a.E;
        ex = e - g * a.E;
        const int32_t* rank = pick(a.sl.rank, si);
        const uint16_t* A = pick(a.sl.A_pool, si);
        // uniform: does a live item own columns of this tile?
        const int j0 = 64 * ex / a.rc, j1 = min(a.G - 1, (64 * ex + 63) / a.rc);
        bool live = false;
        for (int j = j0; j <= j1; ++j) {
            const int i = g * a.G + j;
            if (i < a.n_items) {
                const Item it = a.work[i];
                live |= it.count > 0 && rank[it.slot] > 0;
            }
        }
        if (!live) return;
        // x rows of row block `wave`: item g G + wave
        const int ix = g * a.G + wave;
        const bool xin = wave < a.G && ix < a.n_items;
        xl = xin;
        const Item itx = a.work[xin ? ix : 0];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * wave + 8 * j + dr;
            kc[j] = kz * KC + (dc ^ (r & 7)) * 8;
            const int rr = 8 * j + dr;
            xv[j] = xin && rr < itx.count;
            xs[j] = a.X + (int64_t)a.token_order[xv[j] ? itx.begin + rr : 0] * K + kc[j];
            // column r: rank q of item jj's slot
            const int c = 64 * ex + r, jj = c / a.rc, q = c - jj * a.rc;
            const int iw = g * a.G + jj;
            const bool win = jj < a.G && iw < a.n_items;
            const Item itw = a.work[win ? iw : 0];
            wv[j] = win && itw.count > 0 && q < rank[itw.slot];
            ws[j] = A + ((int64_t)(wv[j] ? itw.slot : 0) * a.r_max + (wv[j] ? q : 0)) * K + kc[j];
        }
    }
    // fragment reads: row r = lane % 16 of a 16-row tile, chunk 4 u + lane / 16
    const int fr = lane & 15, fq = lane >> 4;
    int fo[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) fo[u] = fr * 8 + ((4 * u + fq) ^ (fr & 7));
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // XL: this wave loads x rows (4 loads per stage, else 2); CHK: the loads
    // carry the shrink tile's row and rank masks. Instantiated per case, so
    // that the GEMM blocks' loop has no branch.
    auto run = [&](auto xl_tag, auto chk_tag) {
        constexpr bool XL = decltype(xl_tag)::value, CHK = decltype(chk_tag)::value;
        auto issue = [&](int s) {
            u32x4* st = lds + (s % NS) * SC;
            const int k = s * 64;
            if constexpr (XL)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(or_zero((!CHK || xv[j]) && kc[j] + k < K, xs[j] + k), st + (2 * wave + j) * 64);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                dma16_nt(or_zero((!CHK || wv[j]) && kc[j] + k < K, ws[j] + k), st + 512 + (2 * wave + j) * 64);
        };
        constexpr int PER = XL ? 4 : 2;
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < NST) issue(s);
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            // stage s landed for this wave; the stages issued after it may be in flight
            const int later = (s + NS - 2 < NST ? NS - 2 : NST - 1 - s);
            static_assert(kSplitStages == 5, "wait counts assume 5 stages");
            if (later >= 3) vm_landed<3 * PER>();
            else if (later == 2) vm_landed<2 * PER>();
            else if (later == 1) vm_landed<PER>();
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
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (!TILES || gemm) run(T_{}, F_{});
    else if (xl) run(T_{}, T_{});
    else run(F_{}, T_{});
    if (!TILES || gemm) {
        f32x4* out = reinterpret_cast<f32x4*>(a.part_y) + ((int64_t)(kz * a.n_mt + mt) * a.n_nt + nt) * 16 * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(i * 4 + wave) * 64 + lane] = acc[i];
        return;
    }
    // lane holds rows 4 (lane / 16) + e of every row block, column 16 wave +
    // lane % 16; the wave's 16 columns belong to one item jj (rc % 16 == 0)
    const int c = 64 * ex + 16 * wave + (lane & 15), jj = c / a.rc, q = c - jj * a.rc;
    const int i = g * a.G + jj;
    if (jj >= a.G || i >= a.n_items) return;
    const Item it = a.work[i];
    if (q >= pick(a.sl.rank, si)[it.slot]) return;
    f32x4 v = acc[0];
#pragma unroll
    for (int b = 1; b < 4; ++b) v = jj == b ? acc[b] : v;
    float* hp = a.part_h + ((int64_t)si * a.ks + kz) * a.M * a.r_max + (int64_t)it.begin * a.r_max + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = 4 * (lane >> 4) + e;
        if (rr < it.count) hp[(int64_t)rr * a.r_max] = v[e];
    }
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
// distinct slots of a 16-row block whose expand kernel 2 runs on the matrix
// cores: 4 for ranks up to 32 (one fragment per slot), 8 for ranks up to 64
// (each of the 8 loads per slot pair costs a round-2 load in every block, so
// the smaller count stays where it suffices)
template <int MQ>
constexpr int kMfmaSlots = MQ == 2 ? 8 : 4;

template <bool ADAPT, bool VEC, bool LANE_META, bool MULTI, int MQ = 0>
__global__ __launch_bounds__(kThreads) void splitk_epilogue_kernel(const float* __restrict__ part_y, int ks, int n_mt,
                                                                   int n_nt, int M, Fuse f, SliceTableFor<MULTI> tab) {
    const int nt = blockIdx.x, mt = blockIdx.y >> 2, rb = blockIdx.y & 3;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int p0 = mt * 64 + rb * 16;
    if (p0 >= M) return;  // uniform for the block
    // this tile's slice: its columns, output and pool
    const int si = MULTI ? slice_of(tab, nt) : 0;
    const int N = pick(tab.N, si);
    uint16_t* __restrict__ Y = pick(tab.Y, si);
    f.B_pool = pick(tab.B_pool, si);
    f.rank = pick(tab.rank, si);
    f.scale = pick(tab.scale, si);
    if (ADAPT) f.h += (int64_t)si * f.h_splits * f.h_plane;
    const f32x4* in = reinterpret_cast<const f32x4*>(part_y);
    const int64_t zstride = (int64_t)n_mt * n_nt * 16 * 64;
    const int64_t o = (((int64_t)mt * n_nt + nt) * 16 + rb * 4 + w) * 64 + lane;
    const int n = (nt - nt_first(tab, si)) * 64 + w * 16 + (lane & 15);
    // splits are added in split order; loads are issued unconditionally from
    // clamped addresses (a load under a branch is waited on inside it) and
    // the extra ones are not added
    f32x4 part[8] = {};
#pragma unroll
    for (int z = 0; z < 4; ++z) part[z] = in[min(z, ks - 1) * zstride + o];
    if (ks > 4) {  // uniform
#pragma unroll
        for (int z = 4; z < 8; ++z) part[z] = in[min(z, ks - 1) * zstride + o];
    }
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
        constexpr int HU = MQ > 0 ? 1 : 2;  // pieces per thread in round 1 (r_max <= 64: 16 r_max / 4 <= 256)
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
        // large pools: metadata staged in LDS, or read in place past kMetaSlots
        const int* m_indptr = meta.indptr;
        const int* m_rank = meta.rank;
        const float* m_scale = meta.scale;
        if constexpr (!LANE_META) {
            if (S <= kMetaSlots) {  // uniform
                for (int i = tid; i <= S; i += kThreads) {
                    meta.indptr[i] = f.slot_indptr[i];
                    if (i < S) {
                        meta.rank[i] = f.rank[i];
                        meta.scale[i] = f.scale[i];
                    }
                }
                __syncthreads();
            } else {
                m_indptr = f.slot_indptr;
                m_rank = f.rank;
                m_scale = f.scale;
            }
        }
        // slots of this lane's rows, of block row lane % 16 (row_slot) and of
        // the block's first and last rows (its rows hold slots s_lo .. s_hi);
        // for MQ == 2 also smask, the set of non-zero slots of the block's
        // rows (S <= 64)
        int sl[4] = {0, 0, 0, 0};
        int row_slot = 0, s_lo = 0, s_hi = 0;
        uint64_t smask = 0;
        if constexpr (LANE_META) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // slot of row p = number of slots s in 1..S-1 starting at or before p
                const uint64_t m = __ballot(lane >= 1 && lane < S && ip <= p0 + j);
                const int sj = p0 + j < M ? __popcll(m) : 0;
                if ((lane >> 4) == (j >> 2)) sl[j & 3] = sj;
                if ((lane & 15) == j) row_slot = sj;
                if (j == 0) s_lo = sj;
                if (p0 + j < M) s_hi = sj;
                if constexpr (MQ == 2) smask |= sj != 0 ? 1ull << sj : 0ull;
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
                sl[e] = p < M ? slot_of(m_indptr, S, p) : 0;
                rr[e] = sl[e] == 0 ? 0 : m_rank[sl[e]];
                sc[e] = m_scale[sl[e]];
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
        // MQ > 0 (r_max <= 32 MQ) and at most NSL slots in the block
        // (uniform): the expand runs on the matrix cores, one pass per slot,
        // D[row][col] = sum_q (scale_s h[row][q]) B_s[col][q] over the rows
        // of slot s, the scaled h split into bf16 hi + lo (as the tiled
        // path's extra K steps). Round 2 then loads each slot's B fragments:
        // lane l takes column l % 16 of the wave, ranks 32 c + 8 (l / 16) ..,
        // so a load instruction reads 64 consecutive bytes of each of 16
        // columns. Slot k of the block: MQ == 1, s_lo + k up to s_hi (slot
        // ids in between without rows included); MQ == 2, the k-th distinct
        // slot (the k-th set bit of smask). S: none.
        constexpr int NQ = MQ > 0 ? MQ : 1;
        constexpr int NSL = kMfmaSlots<MQ>;
        const bool mx = MQ == 2 ? __popcll(smask) <= NSL : MQ > 0 && s_hi - s_lo < NSL;
        auto distinct_slot = [&](int k) {  // MQ == 2: the k-th set bit of smask, S past the last
            uint64_t m = smask;
#pragma unroll
            for (int i = 0; i < NSL; ++i)
                if (i < k) m &= m - 1;
            return m ? (int)__builtin_ctzll(m) : S;
        };
        u32x4 bf[NSL][NQ];
        if (mx) {
            if constexpr (MQ == 2) {
#pragma unroll
                for (int k = 0; k < NSL; ++k) {
                    const int s_k = distinct_slot(k);
                    const int sk = min(s_k, S - 1);
                    const int rk_s = __shfl(rk, sk);
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        const int q0 = 32 * c + 8 * (lane >> 4);
                        const bool ok = s_k < S && q0 < rk_s && n < N;
                        bf[k][c] = *or_zero(ok, f.B_pool + ((int64_t)sk * N + min(n, N - 1)) * r_max + q0);
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < NSL; ++k) {
                    const int sk = min(s_lo + k, S - 1);
                    const int rk_s = __shfl(rk, sk);
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        const int q0 = 32 * c + 8 * (lane >> 4);
                        const bool ok = s_lo + k <= s_hi && sk != 0 && q0 < rk_s && n < N;
                        bf[k][c] = *or_zero(ok, f.B_pool + ((int64_t)sk * N + min(n, N - 1)) * r_max + q0);
                    }
                }
            }
        } else if constexpr (VEC) {
            bload(0);
        }
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
        if (mx) {
            // h past the row's rank is not written by the shrink (stale
            // workspace): it is dropped by a select, never multiplied
            const float sc_row = __shfl(sv, row_slot);
            const int rk_row = __shfl(rk, row_slot);  // every lane takes part in the shuffle
            const int r_row = row_slot == 0 ? 0 : rk_row;
            f32x4 dm = {0.f, 0.f, 0.f, 0.f};
            // one slot's pass: rows of slot s (mine) times its B fragments
            auto pass = [&](int k, bool mine) {
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const int q0 = 32 * c + 8 * (lane >> 4);
                    const float* hr = hs + (lane & 15) * r_max + (q0 < r_max ? q0 : 0);
                    const f32x4 h0 = reinterpret_cast<const f32x4*>(hr)[0];
                    const f32x4 h1 = reinterpret_cast<const f32x4*>(hr)[1];
                    float v[8], lo[8];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v[t] = mine && q0 + t < r_row ? sc_row * h0[t] : 0.f;
                        v[4 + t] = mine && q0 + 4 + t < r_row ? sc_row * h1[t] : 0.f;
                    }
#pragma unroll
                    for (int t = 0; t < 8; ++t) lo[t] = v[t] - bf16_to_f32(f32_to_bf16(v[t]));
                    const u32x4 ahi{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                    pack_bf16x2(v[6], v[7])};
                    const u32x4 alo{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(lo[4], lo[5]),
                                    pack_bf16x2(lo[6], lo[7])};
                    dm = mfma16x16x32(ahi, bf[k][c], dm);
                    dm = mfma16x16x32(alo, bf[k][c], dm);
                }
            };
            if constexpr (MQ == 2) {
#pragma unroll
                for (int k = 0; k < NSL; ++k) {
                    const int s_k = distinct_slot(k);
                    if (s_k >= S) break;  // uniform
                    pass(k, row_slot == s_k);
                }
            } else {
#pragma unroll
                for (int k = 0; k < NSL; ++k) {
                    if (s_lo + k > s_hi) break;  // uniform
                    pass(k, row_slot == s_lo + k && row_slot != 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d[e] = dm[e];
                sc[e] = 1.f;  // scale_s already applied
            }
        } else if constexpr (VEC) {
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

template <int NSUB, bool TILES>
static hipError_t launch_split(const SplitArgs<kMaxSlices>& a, int n_blocks, hipStream_t st, StageTimer* tm) {
    if (a.sl.n > 1)
        return launch(tm, "gemm_splitk", splitk_gemm_kernel<NSUB, true, TILES>, dim3(n_blocks), dim3(kThreads), st, a);
    static_assert(offsetof(SplitArgs<1>, sl) == offsetof(SplitArgs<kMaxSlices>, sl), "common head");
    SplitArgs<1> a1;
    std::memcpy(&a1, &a, offsetof(SplitArgs<1>, sl));
    a1.sl = table_of<1>(a.sl);
    return launch(tm, "gemm_splitk", splitk_gemm_kernel<NSUB, false, TILES>, dim3(n_blocks), dim3(kThreads), st, a1);
}

template <bool TILES>
static hipError_t launch_split_n(const SplitArgs<kMaxSlices>& a, int nsub, int n_blocks, hipStream_t st,
                                 StageTimer* tm) {
    switch (nsub) {
        case 1: return launch_split<1, TILES>(a, n_blocks, st, tm);
        case 2: return launch_split<2, TILES>(a, n_blocks, st, tm);
        case 4: return launch_split<4, TILES>(a, n_blocks, st, tm);
        case 8: return launch_split<8, TILES>(a, n_blocks, st, tm);
        default: return launch_split<16, TILES>(a, n_blocks, st, tm);
    }
}

template <bool MULTI>
static auto epilogue_for(const LinearArgs& L) {
    if (!L.adapters) return splitk_epilogue_kernel<false, false, false, MULTI>;
    if (L.r_max % 8 != 0) return splitk_epilogue_kernel<true, false, false, MULTI>;
    if (L.S <= kLaneMetaSlots) {
        // the matrix-core expand for ranks up to 64, the per-lane one past
        // that (and for blocks of more distinct slots than kMfmaSlots<MQ>)
        if (L.r_max <= 32) return splitk_epilogue_kernel<true, true, true, MULTI, 1>;
        if (L.r_max <= 64) return splitk_epilogue_kernel<true, true, true, MULTI, 2>;
        return splitk_epilogue_kernel<true, true, true, MULTI>;
    }
    return splitk_epilogue_kernel<true, true, false, MULTI>;
}

hipError_t splitk_forward_bf16(const LinearArgs& L, const GemmPlan& g, hipStream_t st, StageTimer* tm) {
    const int M = L.M, K = L.K, n = L.n_slices;
    SliceTableAll sl{};
    sl.n = n;
    int nt = 0;
    for (int i = 0; i < kMaxSlices; ++i) {
        sl.nt0[i] = nt;
        if (i >= n) continue;
        const SliceArgs& s = L.slice[i];
        sl.N[i] = s.N;
        sl.W[i] = s.W;
        sl.A_pool[i] = s.A_pool;
        sl.B_pool[i] = s.B_pool;
        sl.rank[i] = s.rank;
        sl.scale[i] = s.scale;
        sl.Y[i] = s.Y;
        nt += cdiv(s.N, 64);
    }
    sl.nt0[kMaxSlices] = nt;
    char* ws = static_cast<char*>(L.workspace);
    const size_t py = ((size_t)g.ks * g.n_mt * nt * 16 * 64 * 16 + 255) & ~size_t(255);
    // The shrink runs as tiles when it is heavy against the GEMM (its item
    // rows x + A_s exceed 1/8 of the GEMM tiles' x + W rows), else as
    // workgroups over K ranges of at least 256 k, at most 8 of them. Tiles:
    // as many items per tile as 64 columns hold whole (16-column rounded)
    // ranks, at least one.
    const int rc = (L.r_max + 15) & ~15, G = max(1, 64 / rc), E = cdiv(G * rc, 64);
    const int n_items = L.adapters ? L.n_items : 0;
    const bool tiles = (int64_t)n_items * n * (16 + rc) * 8 > (int64_t)g.n_mt * nt * 128;
    const int hkc = max(256, (cdiv(K, 8) + 31) / 32 * 32), hs = tiles ? 0 : cdiv(K, hkc);
    const int n_groups = tiles ? cdiv(n_items, G) : 0;
    SplitArgs<kMaxSlices> a{L.X, reinterpret_cast<float*>(ws), M, K, g.n_mt, nt, g.ks, L.token_order,
                reinterpret_cast<const Item*>(L.work), n_items, L.r_max,
                reinterpret_cast<float*>(ws + py), hs, hkc, n_groups, G, rc, E, sl};
    const int n_blocks = n_items * hs * n + g.n_mt * nt * g.ks + g.ks * n * n_groups * E;
    const hipError_t e = tiles ? launch_split_n<true>(a, g.nsub, n_blocks, st, tm)
                               : launch_split_n<false>(a, g.nsub, n_blocks, st, tm);
    if (e != hipSuccess) return e;
    // per-slice pool pointers and h planes are set by each kernel-2 block
    const Fuse f{L.token_order, L.slot_indptr, a.part_h, nullptr, nullptr, nullptr, L.S, L.r_max, tiles ? g.ks : hs,
                 (int64_t)M * L.r_max, L.adapters, nullptr, (L.r_max + 7) & ~7};
    const dim3 eg(nt, 4 * g.n_mt);
    const uint32_t shm = L.adapters ? (uint32_t)((16 * L.r_max + 32) * sizeof(float)) : 0u;
    if (n > 1)
        return launch_shm(tm, "gemm_splitk_epilogue", epilogue_for<true>(L), eg, dim3(kThreads), shm, st,
                          (const float*)a.part_y, g.ks, g.n_mt, nt, M, f, sl);
    return launch_shm(tm, "gemm_splitk_epilogue", epilogue_for<false>(L), eg, dim3(kThreads), shm, st,
                      (const float*)a.part_y, g.ks, g.n_mt, nt, M, f, table_of<1>(sl));
}

hipError_t splitk_finish_bf16(const LinearArgs& L, const SliceArgs& s, const float* part, int ks, int n_mt,
                              const float* h, int h_splits, hipStream_t st, StageTimer* tm) {
    SliceTable<1> sl{};
    sl.n = 1;
    sl.N[0] = s.N;
    sl.W[0] = s.W;
    sl.A_pool[0] = s.A_pool;
    sl.B_pool[0] = s.B_pool;
    sl.rank[0] = s.rank;
    sl.scale[0] = s.scale;
    sl.Y[0] = s.Y;
    const int nt = cdiv(s.N, 64);
    sl.nt0[1] = nt;
    const Fuse f{L.token_order, L.slot_indptr, h, nullptr, nullptr, nullptr, L.S, L.r_max, h_splits,
                 (int64_t)L.M * L.r_max, L.adapters, nullptr, (L.r_max + 7) & ~7};
    const dim3 eg(nt, 4 * n_mt);
    const uint32_t shm = L.adapters ? (uint32_t)((16 * L.r_max + 32) * sizeof(float)) : 0u;
    return launch_shm(tm, "gemm_splitk_epilogue", epilogue_for<false>(L), eg, dim3(kThreads), shm, st, part, ks,
                      n_mt, nt, L.M, f, sl);
}

}  // namespace lora
