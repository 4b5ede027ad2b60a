// Ablation 1: one thread per output element.
//
// Page 1 ("[Multi-Core & GPU Programming] CUDA - Matrix Multiplication"),
// section [Matrix Multiplication]: each thread owns one output, derives its
// row and column from the block and thread indices (col from the x
// dimension, row from the y dimension, "Work Flow"), accumulates the k-sum in
// a register and writes the output once.  Page 2 ("Lec 29 · GPU Architecture
// (2)") §1.2 names its cost: every thread streams a full row of A and column
// of B from device memory, 2·M·N·K element reads in total.
//
// On a 64-wide wavefront a 16×16 block covers four output rows: the B reads of
// a wave are 16 consecutive words (coalesced), its A reads are four words, one
// per row, each shared by 16 lanes (page 1, section [Coalescing]).
// Each step is one fused multiply-add in ascending k, rounded once.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

constexpr int kBlock = 16;

// Row `a` of A against column `b` of B (stride ldb): one fused multiply-add
// per k in ascending order, rounded once each.
__device__ __forceinline__ float row_dot_column(const float *__restrict__ a, const float *__restrict__ b,
                                                int64_t ldb, int K)
{
    float acc = 0.0f;
    for (int k = 0; k < K; ++k, b += ldb) acc = __builtin_fmaf(a[k], *b, acc);
    return acc;
}

__global__ __launch_bounds__(kBlock *kBlock) void naive_kernel(int M, int N, int K,
                                                               const float *__restrict__ A,
                                                               int64_t lda,
                                                               const float *__restrict__ B,
                                                               int64_t ldb,
                                                               float *__restrict__ C,
                                                               int64_t ldc)
{
    // this thread's output: x along C's columns, y along its rows
    const int i = blockIdx.y * kBlock + threadIdx.y;
    const int j = blockIdx.x * kBlock + threadIdx.x;
    if (i < M && j < N) C[(int64_t)i * ldc + j] = row_dot_column(A + (int64_t)i * lda, B + j, ldb, K);
}

}  // namespace

hipError_t launch_naive(const GemmArgs &g, hipStream_t stream)
{
    const dim3 block(kBlock, kBlock);
    const dim3 grid((g.N + kBlock - 1) / kBlock, (g.M + kBlock - 1) / kBlock);
    if (grid.y > 65535u) return hipErrorInvalidConfiguration;
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&naive_kernel), grid, block, args, 0,
                           stream);
}

}  // namespace tgemm
