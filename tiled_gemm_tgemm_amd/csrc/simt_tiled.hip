// Ablation 3: the tiled kernel with more work per thread, on the vector ALUs.
//
// Page 1 ("[Multi-Core & GPU Programming] CUDA - Matrix Multiplication"),
// end of section [Shared Memory], "Tile Size 결정": with one output per
// thread the tile size is capped by the thread count of a block, so the way
// to use more on-chip memory is to let each thread compute several outputs.
// Here a 256-thread work-group owns a 128×128 tile of C and each thread an
// 8×8 micro-tile in registers: rows 4·ty .. 4·ty+3 and 64+4·ty .. 64+4·ty+3,
// columns 4·tx .. 4·tx+3 and 64+4·tx .. 64+4·tx+3 (ty, tx in 0..15), so that
// every operand read from LDS is one 16-byte read of four consecutive values.
//
// Per phase of 8 values of k the work-group copies the 128×8 slice of A and
// the 8×128 slice of B into LDS (page 1, "Work Flow - Compute Block(0, 0)").
// A is read along its rows (coalesced, page 1 section [Coalescing]) and
// written into LDS transposed, As[k][m], so that the k loop reads it along m:
// the "Corner Turning" of page 1 section [Coalescing].  Two LDS stages, the
// next phase's elements held in registers while the current one computes,
// one barrier per phase.  Out-of-range elements load as zero.
//
// Each output is one fused multiply-add chain in ascending k from +0, so the
// result equals the naive and LDS-tiled kernels (and the sequential float32
// model) bit for bit.  The arithmetic is plain v_fma_f32 (packed fp32 is off
// for all of this library), whose rate bounds the kernel.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 8, kThreads = 256;
constexpr int kAS = kBM + 4;  // As[k][m] row stride (words)
constexpr int kBS = kBN + 4;  // Bs[k][n] row stride (words)
constexpr int kStage = kBK * kAS + kBK * kBS;

__global__ __launch_bounds__(kThreads) void simt_tiled_kernel(int M, int N, int K,
                                                              const float *__restrict__ A, int64_t lda,
                                                              const float *__restrict__ B, int64_t ldb,
                                                              float *__restrict__ C, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) float lds[2 * kStage];

    const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
    const int t = threadIdx.x;
    const int tx = t % 16, ty = t / 16;

    // copy slots: A element (m0 + t/2, k0 + 4(t%2) + q), B element
    // (k0 + t/32, n0 + 4(t%32) + q), q = 0..3
    const int a_m = t / 2, a_k = 4 * (t % 2);
    const int b_k = t / 32, b_n = 4 * (t % 32);
    const bool a_row_in = m0 + a_m < M;
    const float *a_row = A + (int64_t)(a_row_in ? m0 + a_m : 0) * lda;
    float a_reg[4], b_reg[4];

    auto load_phase = [&] __device__(int k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = k0 + a_k + q;
            a_reg[q] = (a_row_in && k < K) ? a_row[k] : 0.0f;
        }
        const int kb = k0 + b_k;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + b_n + q;
            b_reg[q] = (kb < K && n < N) ? B[(int64_t)kb * ldb + n] : 0.0f;
        }
    };
    auto store_phase = [&] __device__(int stage) {
        float *as = lds + stage * kStage;
        float *bs = as + kBK * kAS;
#pragma unroll
        for (int q = 0; q < 4; ++q) as[(a_k + q) * kAS + a_m] = a_reg[q];
        *reinterpret_cast<f32x4 *>(bs + b_k * kBS + b_n) = f32x4{b_reg[0], b_reg[1], b_reg[2], b_reg[3]};
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const int phases = (K + kBK - 1) / kBK;
    load_phase(0);
    store_phase(0);
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        const bool more = p + 1 < phases;
        if (more) load_phase((p + 1) * kBK);
        const float *as = lds + (p & 1) * kStage;
        const float *bs = as + kBK * kAS;
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(as + k * kAS + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(as + k * kAS + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bs + k * kBS + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bs + k * kBS + 64 + 4 * tx);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (more) store_phase((p + 1) & 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + (j < 4 ? 4 * tx + j : 64 + 4 * tx + j - 4);
            if (col < N) C[(int64_t)row * ldc + col] = acc[i][j];
        }
    }
}

}  // namespace

hipError_t launch_simt_tiled(const GemmArgs &g, hipStream_t stream)
{
    const dim3 grid((g.N + kBN - 1) / kBN, (g.M + kBM - 1) / kBM);
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&simt_tiled_kernel), grid, dim3(kThreads), args,
                           0, stream);
}

}  // namespace tgemm
