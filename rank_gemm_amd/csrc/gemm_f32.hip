// fp32 base GEMM, Y[M][N] = X[M][K] * W[N][K]^T, in true fp32 FMA (no
// reduced-precision splitting). Used for pools of element type fp32; 64 x 64
// tiles, each of the 256 threads owns a 4 x 4 block, K staged 16 at a time.
#include "common.h"
#include "kernels.h"

namespace lora {

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                       float* __restrict__ Y, int M, int N, int K) {
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int i = tid; i < 64 * 16; i += 256) {
            const int r = i >> 4, c = i & 15;
            const int m = m0 + r, n = n0 + r, k = k0 + c;
            As[c][r] = (m < M && k < K) ? X[(int64_t)m * K + k] : 0.f;
            Bs[c][r] = (n < N && k < K) ? W[(int64_t)n * K + k] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[c][ty * 4 + i];
                b[i] = Bs[c][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < M && n < N) Y[(int64_t)m * N + n] = acc[i][j];
        }
}

hipError_t gemm_f32(const float* X, const float* W, float* Y, int M, int N, int K, hipStream_t st, StageTimer* tm) {
    if (M == 0 || N == 0) return hipSuccess;
    return launch(tm, "gemm_f32", gemm_f32_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), st, X, W, Y, M, N,
                  K);
}

}  // namespace lora
