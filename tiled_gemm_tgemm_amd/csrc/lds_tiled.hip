// Ablation 2: the shared-memory (LDS) tiled kernel, one output per thread.
//
// Page 1 ("[Multi-Core & GPU Programming] CUDA - Matrix Multiplication"),
// section [Shared Memory] ("Work Flow - Compute Block(0, 0)", "Tiled Matrix
// Multiplication Kernel", "__syncthreads( )"), and page 2 ("Lec 29 · GPU
// Architecture (2)") §1.2: a T×T thread block owns a T×T output tile and walks
// K in phases of T.  In each phase every thread copies one element of A and
// one of B into two T×T on-chip tiles, the block waits until both tiles are
// complete, every thread adds the T products of its row and column to its
// register sum, and the block waits again so that no thread refills a tile
// another thread is still reading.  Each element read from device memory is
// reused T times, so device reads drop from 2·N^3 to 2·N^3/T.
//
// Both tile copies are coalesced: consecutive lanes (lx) read consecutive addresses of
// one A row and one B row (page 1, section [Coalescing], the tiled kernel's
// two loads).  With PAD = 1 every tile row is one word longer, the
// tile[32][33] idea of page 2 §1.4: on a 64-wide wavefront one wave spans
// 64/T tile rows, so its A reads (row ly, column k of the A slice) from
// different rows land T words apart; the padding moves them to different
// banks.
//
// Edges: the pages assume Width is a multiple of the tile.  Here rows, columns
// and k beyond the matrix load as zero and are never stored, so any M, N, K
// works; a zero-padded product adds +0 and leaves every sum unchanged.
// Each step is one fused multiply-add in ascending k, rounded once.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

// One operand's T×T slice of a phase in LDS (rows padded by PAD words), and
// the thread's place in it.  fill_a / fill_b copy the thread's one element from
// device memory, zero where it lies outside the operand.  Aligned to 16 bytes,
// so that without padding a row's consecutive words can be read 16 bytes at a
// time.
template <int T, int PAD>
struct alignas(16) Stage {
    float cell[T][T + PAD];

    // A slice: the element (row, k0 + lane) of A, kept at [lane_y][lane_x]
    __device__ __forceinline__ void fill_a(const float *a_row, bool row_ok, int k, int K, int ly, int lx)
    {
        cell[ly][lx] = (row_ok && k < K) ? a_row[k] : 0.0f;
    }
    // B slice: the element (k0 + lane_y, col) of B, kept at [lane_y][lane_x]
    __device__ __forceinline__ void fill_b(const float *b_col, int64_t ldb, bool col_ok, int k, int K, int ly,
                                           int lx)
    {
        cell[ly][lx] = (col_ok && k < K) ? b_col[(int64_t)k * ldb] : 0.0f;
    }
};

// The thread's output summed over one phase: row ly of the A slice against
// column lx of the B slice, one fused multiply-add per k in ascending order.
template <int T, int PAD>
__device__ __forceinline__ float dot_phase(const Stage<T, PAD> &a, const Stage<T, PAD> &b, int ly, int lx,
                                           float acc)
{
#pragma unroll
    for (int k = 0; k < T; ++k) acc = __builtin_fmaf(a.cell[ly][k], b.cell[k][lx], acc);
    return acc;
}

template <int T, int PAD>
__global__ __launch_bounds__(T *T) void lds_tiled_kernel(int M, int N, int K,
                                                         const float *__restrict__ A, int64_t lda,
                                                         const float *__restrict__ B, int64_t ldb,
                                                         float *__restrict__ C, int64_t ldc)
{
    __shared__ Stage<T, PAD> a_stage, b_stage;

    // the block's output tile and this thread's output in it (x along columns)
    const int lx = threadIdx.x, ly = threadIdx.y;
    const int out_row = blockIdx.y * T + ly, out_col = blockIdx.x * T + lx;
    const bool row_ok = out_row < M, col_ok = out_col < N;
    const float *a_row = A + (int64_t)(row_ok ? out_row : 0) * lda;
    const float *b_col = B + (col_ok ? out_col : 0);

    float acc = 0.0f;
    for (int k0 = 0; k0 < K; k0 += T) {
        a_stage.fill_a(a_row, row_ok, k0 + lx, K, ly, lx);
        b_stage.fill_b(b_col, ldb, col_ok, k0 + ly, K, ly, lx);
        __syncthreads();  // both slices complete before any thread reads them
        acc = dot_phase(a_stage, b_stage, ly, lx, acc);
        __syncthreads();  // no thread still reads a slice when the next phase refills it
    }
    if (row_ok && col_ok) C[(int64_t)out_row * ldc + out_col] = acc;
}

template <int T, int PAD>
hipError_t launch_t(const GemmArgs &g, hipStream_t stream)
{
    const dim3 block(T, T);
    const dim3 grid((g.N + T - 1) / T, (g.M + T - 1) / T);
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&lds_tiled_kernel<T, PAD>), grid, block,
                           args, 0, stream);
}

}  // namespace

hipError_t launch_lds_tiled(const GemmArgs &g, int tile, int pad, hipStream_t stream)
{
    switch (tile * 2 + pad) {
        case 2 * 2 + 0: return launch_t<2, 0>(g, stream);
        case 2 * 2 + 1: return launch_t<2, 1>(g, stream);
        case 8 * 2 + 0: return launch_t<8, 0>(g, stream);
        case 8 * 2 + 1: return launch_t<8, 1>(g, stream);
        case 16 * 2 + 0: return launch_t<16, 0>(g, stream);
        case 16 * 2 + 1: return launch_t<16, 1>(g, stream);
        case 32 * 2 + 0: return launch_t<32, 0>(g, stream);
        case 32 * 2 + 1: return launch_t<32, 1>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

__global__ void fill_zero_kernel(int M, int N, float *__restrict__ C, int64_t ldc)
{
    for (int64_t i = blockIdx.y; i < M; i += gridDim.y)
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < N;
             j += (int64_t)gridDim.x * blockDim.x)
            C[i * ldc + j] = 0.0f;
}

hipError_t launch_fill_zero(int M, int N, float *C, int64_t ldc, hipStream_t stream)
{
    const dim3 block(256);
    const unsigned gx = (unsigned)((N + 255) / 256 < 64 ? (N + 255) / 256 : 64);
    const unsigned gy = (unsigned)(M < 4096 ? M : 4096);
    void *args[] = {&M, &N, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&fill_zero_kernel), dim3(gx, gy), block,
                           args, 0, stream);
}

}  // namespace tgemm
