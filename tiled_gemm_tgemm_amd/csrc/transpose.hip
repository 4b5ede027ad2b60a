// Matrix transpose, B = Aᵀ (page 2, "Lec 29 · GPU Architecture (2)", §1.4).
//
// A is M×N with leading dimension lda, B is N×M with leading dimension ldb,
// both row-major float32; B(j, i) = A(i, j).  Words are moved, never
// computed on, so every bit pattern arrives unchanged.  Work-groups are
// numbered in one dimension, column tiles fastest, so no grid dimension
// limits M or N.
//
// Three kernels follow the page's progression for its hardware, on gfx950:
//
// * naive: 32×32 tiles, 32×8 threads, each thread four elements in a loop
//   over rows (the page amortises index arithmetic this way).  Reads run
//   along A's rows (coalesced); writes run down B's columns, one element per
//   row of B — the page's uncoalesced store.
// * tiled<PAD>: the same tile read along A's rows into LDS, a barrier, then,
//   with the block offsets swapped, each thread writes along a row of B from
//   a column of the LDS tile — both global directions coalesced.  PAD = 1 is
//   the page's tile[32][33], which moves each row of the tile by one bank.
//
// and one is this library's design for CDNA4:
//
// * blocked: no LDS at all.  Each thread moves 4×4 blocks: four 16-byte
//   reads of consecutive A rows, and four 16-byte writes of consecutive B
//   rows, each write holding one column of the block (the corner turn is a
//   register permutation).  Lanes sit on an 8×8 grid of blocks per
//   wavefront, so every read and every write instruction of a wavefront is 8
//   runs of 128 contiguous bytes — whole cache lines in both directions,
//   with no barrier and no bank conflicts.  Tiles that reach past M or N, and
//   operands that are not 16-byte aligned with leading dimensions multiples
//   of four, take the same mapping with single-word, masked accesses.  The
//   output is written with non-temporal stores (B is not read back by the
//   kernel): measured on MI355X, 16384² 5.33 → 5.39 TB/s, 8192² 4.44 → 6.31
//   TB/s (B no longer displaces A from the 256 MB Infinity Cache), 4096²
//   5.80 → 6.10 TB/s.  Non-temporal loads as well gain 1.7% more at 16384²
//   but lose 30% at 8192² and 15% at 4096², so loads stay ordinary.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32, kRows = 8;

__device__ __forceinline__ void tile_origin(int tiles_n, int tile, int &y0, int &x0)
{
    y0 = (blockIdx.x / tiles_n) * tile;
    x0 = (blockIdx.x % tiles_n) * tile;
}

__global__ __launch_bounds__(kTile *kRows) void transpose_naive_kernel(int M, int N, const float *__restrict__ A,
                                                                        int64_t lda, float *__restrict__ B,
                                                                        int64_t ldb, int tiles_n)
{
    int y0, x0;
    tile_origin(tiles_n, kTile, y0, x0);
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
    const int x = x0 + tx;
    if (x >= N) return;
#pragma unroll
    for (int j = 0; j < kTile; j += kRows) {
        const int y = y0 + ty + j;
        if (y < M) B[(int64_t)x * ldb + y] = A[(int64_t)y * lda + x];
    }
}

template <int PAD>
__global__ __launch_bounds__(kTile *kRows) void transpose_tiled_kernel(int M, int N, const float *__restrict__ A,
                                                                        int64_t lda, float *__restrict__ B,
                                                                        int64_t ldb, int tiles_n)
{
    __shared__ float tile[kTile][kTile + PAD];
    int y0, x0;
    tile_origin(tiles_n, kTile, y0, x0);
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
#pragma unroll
    for (int j = 0; j < kTile; j += kRows) {
        const int y = y0 + ty + j, x = x0 + tx;
        if (y < M && x < N) tile[ty + j][tx] = A[(int64_t)y * lda + x];
    }
    __syncthreads();  // the whole tile is in LDS before any column of it is read
#pragma unroll
    for (int j = 0; j < kTile; j += kRows) {
        const int r = x0 + ty + j, c = y0 + tx;  // B(r, c) = A(c, r)
        if (r < N && c < M) B[(int64_t)r * ldb + c] = tile[tx][ty + j];
    }
}

// blocked: a work-group of 4 wavefronts (2×2) owns a 64×(64·PC) tile of A;
// lane l of a wavefront owns, in each of the PC 64×64 sub-tiles, the 4×4
// block at block row l / 8, block column l % 8 of the wavefront's 32×32
// quarter.  All reads are issued before the first write.
constexpr int kBlkRows = 64, kBlkThreads = 256;

template <int PC, bool VEC4>
__global__ __launch_bounds__(kBlkThreads) void transpose_blocked_kernel(int M, int N, const float *__restrict__ A,
                                                                         int64_t lda, float *__restrict__ B,
                                                                         int64_t ldb, int tiles_n)
{
    constexpr int kCols = 64 * PC;
    const int y0 = (blockIdx.x / tiles_n) * kBlkRows, x0 = (blockIdx.x % tiles_n) * kCols;
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    const int i0 = y0 + 32 * (w / 2) + 4 * (lane / 8);  // first A row of the blocks
    const int jb = x0 + 32 * (w % 2) + 4 * (lane % 8);  // first A column of the first block

    if (VEC4 && y0 + kBlkRows <= M && x0 + kCols <= N) {
        f32x4 r[PC][4];
#pragma unroll
        for (int p = 0; p < PC; ++p)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                r[p][s] = *reinterpret_cast<const f32x4 *>(A + (int64_t)(i0 + s) * lda + jb + 64 * p);
#pragma unroll
        for (int p = 0; p < PC; ++p)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                __builtin_nontemporal_store(f32x4{r[p][0][s], r[p][1][s], r[p][2][s], r[p][3][s]},
                                            reinterpret_cast<f32x4 *>(B + (int64_t)(jb + 64 * p + s) * ldb + i0));
        return;
    }
#pragma unroll
    for (int p = 0; p < PC; ++p) {
        const int j0 = jb + 64 * p;
        float r[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = i0 + s, j = j0 + q;
                r[s][q] = (i < M && j < N) ? A[(int64_t)i * lda + j] : 0.0f;
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = i0 + s, j = j0 + q;
                if (i < M && j < N) __builtin_nontemporal_store(r[s][q], B + (int64_t)j * ldb + i);
            }
    }
}

template <class Kernel>
hipError_t launch_1d(Kernel *kernel, int tile_rows, int tile_cols, int threads, const TransposeArgs &t,
                     hipStream_t stream)
{
    const int64_t tiles_m = (t.M + tile_rows - 1) / tile_rows, tiles_n = (t.N + tile_cols - 1) / tile_cols;
    if (tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidConfiguration;
    int M = t.M, N = t.N, tn = (int)tiles_n;
    const float *A = t.A;
    float *B = t.B;
    int64_t lda = t.lda, ldb = t.ldb;
    void *args[] = {&M, &N, &A, &lda, &B, &ldb, &tn};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(threads), args, 0, stream);
}

// Wide tiles (64×256, four sub-tiles per thread) keep more reads in flight
// and read 1 KB of each A row per work-group; they pay off once there are
// enough of them to fill the GPU many times over (measured: 16384×16384 at
// 5.4 TB/s against 4.5 TB/s for 64×64 tiles); smaller matrices keep 64×64
// tiles so that every CU has work.
constexpr int64_t kWideMinElements = (int64_t)1 << 24;

}  // namespace

hipError_t launch_transpose(TransposeKind kind, const TransposeArgs &t, hipStream_t stream)
{
    constexpr int kT = kTile * kRows;
    switch (kind) {
        case TransposeKind::kNaive: return launch_1d(&transpose_naive_kernel, kTile, kTile, kT, t, stream);
        case TransposeKind::kTiled: return launch_1d(&transpose_tiled_kernel<0>, kTile, kTile, kT, t, stream);
        case TransposeKind::kTiledPadded:
            return launch_1d(&transpose_tiled_kernel<1>, kTile, kTile, kT, t, stream);
        case TransposeKind::kBlocked:
            if ((int64_t)t.M * t.N >= kWideMinElements)
                return t.vec4 ? launch_1d(&transpose_blocked_kernel<4, true>, kBlkRows, 256, kBlkThreads, t, stream)
                              : launch_1d(&transpose_blocked_kernel<4, false>, kBlkRows, 256, kBlkThreads, t, stream);
            return t.vec4 ? launch_1d(&transpose_blocked_kernel<1, true>, kBlkRows, 64, kBlkThreads, t, stream)
                          : launch_1d(&transpose_blocked_kernel<1, false>, kBlkRows, 64, kBlkThreads, t, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace tgemm
