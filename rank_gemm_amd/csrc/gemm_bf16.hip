// Base GEMM of the LoRA linear on gfx950 matrix cores:
//   Y[M][N] = bf16( X[M][K] * W[N][K]^T ), fp32 accumulation.
// Both operands are K-contiguous (x rows, nn.Linear weight rows), so the
// same LDS path serves both. Macro tiles of BM x BN are computed by 4 waves
// in a 2 x 2 grid with v_mfma_f32_16x16x32_bf16; K advances 64 at a time
// through a double-buffered, XOR-swizzled LDS stage.
#include "common.h"
#include "kernels.h"

namespace lora {

constexpr int kBK = 64;
constexpr int kThreads = 256;

// 16-byte LDS chunk of (row, logical chunk c in 0..7). The XOR spreads the
// 16 rows one MFMA operand read touches over distinct banks.
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

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

template <int BM, int BN, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ X,
                                                                const uint16_t* __restrict__ W,
                                                                void* __restrict__ out, int M, int N, int K,
                                                                int k_chunk, int tiles_m, int tiles_n) {
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int AC = BM * 8 / kThreads;  // 16-byte chunks per thread per stage
    constexpr int BC = BN * 8 / kThreads;
    __shared__ u32x4 lds[2 * (BM + BN) * 8];
    u32x4* As = lds;
    u32x4* Bs = lds + 2 * BM * 8;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kz = blockIdx.y;
    const int kbeg = kz * k_chunk;
    const int kend = min(K, kbeg + k_chunk);
    const int nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

    const int lc = tid & 7, lr = tid >> 3;
    u32x4 ra[AC], rb[BC];
    auto gload = [&](int k0) {
        const int kk = k0 + lc * 8;
        const bool kin = kk < kend;  // K % 8 == 0: a chunk is fully in or out
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int r = m0 + lr + 32 * i;
            ra[i] = (kin && r < M) ? *(const u32x4*)(X + (int64_t)r * K + kk) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < BC; ++i) {
            const int r = n0 + lr + 32 * i;
            rb[i] = (kin && r < N) ? *(const u32x4*)(W + (int64_t)r * K + kk) : u32x4{0, 0, 0, 0};
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

    if (nk > 0) {
        gload(kbeg);
        sstore(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kbeg + (kt + 1) * kBK);
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
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // lane holds rows 4*(lane/16)+e, column lane%16 of every 16x16 block
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * WTM + i * 16 + (lane >> 4) * 4 + e;
                if (row < M && col < N) {
                    if constexpr (SPLIT)
                        ((float*)out)[((int64_t)kz * M + row) * N + col] = acc[i][j][e];
                    else
                        ((uint16_t*)out)[(int64_t)row * N + col] = f32_to_bf16(acc[i][j][e]);
                }
            }
        }
}

// Sum the K-split partials in split order and round once.
__global__ __launch_bounds__(256) void splitk_reduce_bf16(const float* __restrict__ part, uint16_t* __restrict__ Y,
                                                          int64_t MN, int ks) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float s = 0.f;
    for (int z = 0; z < ks; ++z) s += part[(int64_t)z * MN + i];
    Y[i] = f32_to_bf16(s);
}

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

GemmShape gemm_bf16_shape(int M, int N, int K) {
    GemmShape g{256, 256, 1, 0};
    const int kt = cdiv(K, kBK);
    if ((int64_t)cdiv(M, 256) * cdiv(N, 256) >= 256) {
        g = {256, 256, 1, kt * kBK};
    } else if ((int64_t)cdiv(M, 128) * cdiv(N, 128) >= 256) {
        g = {128, 128, 1, kt * kBK};
    } else {
        const int bm = M > 64 ? 128 : 64;
        const int bn = bm;
        const int tiles = cdiv(M, bm) * cdiv(N, bn);
        int ks = 256 / (tiles > 0 ? tiles : 1);
        ks = ks < 1 ? 1 : ks;
        const int max_ks = kt / 8 > 0 ? kt / 8 : 1;  // at least 512 K per split
        ks = ks > max_ks ? max_ks : ks;
        const int chunk_t = cdiv(kt, ks);
        ks = cdiv(kt, chunk_t);
        g = {bm, bn, ks, chunk_t * kBK};
    }
    return g;
}

size_t gemm_bf16_workspace(int M, int N, int K) {
    GemmShape g = gemm_bf16_shape(M, N, K);
    return g.ks > 1 ? (size_t)g.ks * M * N * sizeof(float) : 0;
}

template <int BM, int BN>
static hipError_t launch(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K, float* ws,
                         const GemmShape& g, hipStream_t st, StageTimer* tm) {
    const int tiles_m = cdiv(M, BM), tiles_n = cdiv(N, BN);
    dim3 grid(tiles_m * tiles_n, g.ks);
    if (g.ks > 1) {
        {
            TimedScope ts(tm, "gemm_bf16", st);
            gemm_bf16_kernel<BM, BN, true>
                <<<grid, kThreads, 0, st>>>(X, W, ws, M, N, K, g.k_chunk, tiles_m, tiles_n);
        }
        const int64_t MN = (int64_t)M * N;
        TimedScope ts(tm, "gemm_splitk_reduce", st);
        splitk_reduce_bf16<<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(ws, Y, MN, g.ks);
    } else {
        TimedScope ts(tm, "gemm_bf16", st);
        gemm_bf16_kernel<BM, BN, false><<<grid, kThreads, 0, st>>>(X, W, Y, M, N, K, g.k_chunk, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

hipError_t gemm_bf16(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K, float* ws,
                     hipStream_t st, StageTimer* tm) {
    if (M == 0 || N == 0) return hipSuccess;
    const GemmShape g = gemm_bf16_shape(M, N, K);
    if (g.bm == 256) return launch<256, 256>(X, W, Y, M, N, K, ws, g, st, tm);
    if (g.bm == 128) return launch<128, 128>(X, W, Y, M, N, K, ws, g, st, tm);
    return launch<64, 64>(X, W, Y, M, N, K, ws, g, st, tm);
}

}  // namespace lora
