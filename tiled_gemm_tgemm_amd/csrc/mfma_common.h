// Pieces shared by the two matrix-core kernels (mfma_sgemm.hip, mfma_sgemm_flat.hip):
// the work-group → C-tile map, the k-group fragment reads and MFMA steps, and
// the masked epilogue.  See mfma_sgemm.hip for the design and its citations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {
namespace mfma {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kXcds = 8;

// Map the hardware work-group id to a C tile (tm, tn).  The hardware deals
// ids round-robin to the eight XCDs (each with its own L2): XCD x holds ids
// x, x+8, x+16, ...  Each XCD is given the contiguous run of logical ids
// that starts after the runs of XCDs 0..x-1, and logical ids walk groups of
// group_m tile rows column by column, so the work-groups resident on one XCD
// cover a compact block of C tiles and share A rows and B columns in its L2.
// Both steps are bijections on [0, tiles_m * tiles_n).
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int q = nwg / kXcds, r = nwg % kXcds;
    const int x = wg % kXcds;
    const int logical = wg / kXcds + x * q + (x < r ? x : r);
    const int per_group = group_m * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// One wavefront's view of a phase held in LDS: As holds the BM×BK slice of A
// (row-major, layout chosen by the kernel), Bs[k][n] the BK×BN slice of B
// with row stride BS words.  In step s of k-group g the lanes of half h feed
// k = 8g + 4h + s to both operands, so a lane's four A values of a group are
// adjacent and come in one 16-byte read.
template <int FM, int FN, int BS>
struct Fragments {
    f32x4 a[FM];
    float b[FN][4];

    // a_off[i]: word offset in As of (row wm*TM + 32i + l32, columns 8g+4h ..
    // 8g+4h+3) for this group g; b_frag: offset of (row 4h, column
    // wn*TN + l32) in Bs.
    __device__ __forceinline__ void read(const float *as, const float *bs, const int (&a_off)[FM],
                                         int b_frag, int g)
    {
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const f32x4 *>(as + a_off[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s) b[j][s] = bs[b_frag + (8 * g + s) * BS + j * 32];
    }
};

// The four steps of one k-group on every 32×32 block of the wavefront.
template <int FM, int FN, class Frag>
__device__ __forceinline__ void mfma_group(f32x16 (&acc)[FM][FN], const Frag &f)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[j][s], acc[i][j], 0, 0, 0);
}

// A whole phase of BK values of k from one LDS stage; the reads of group
// g+1 are issued before the matrix-core steps of group g.
template <int FM, int FN, int BS, int BK>
__device__ __forceinline__ void mfma_phase(f32x16 (&acc)[FM][FN], const float *as, const float *bs,
                                           const int (&a_off)[BK / 8][FM], int b_frag)
{
    Fragments<FM, FN, BS> f[2];
    f[0].read(as, bs, a_off[0], b_frag, 0);
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
        if (g + 1 < BK / 8) f[(g + 1) & 1].read(as, bs, a_off[g + 1], b_frag, g + 1);
        mfma_group<FM, FN>(acc, f[g & 1]);
    }
}

// Accumulator register r of lane (l32, half) in block (i, j) is C row
// 8*(r/4) + 4*half + r%4 and column l32 of that block.  Rows >= M and columns
// >= N are not written.
template <int FM, int FN>
__device__ __forceinline__ void store_c(const f32x16 (&acc)[FM][FN], float *__restrict__ C, int64_t ldc,
                                        int M, int N, int row0, int col0, int half, int l32)
{
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 32 + l32;
        if (col >= N) continue;
        float *c = C + col;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (row < M) c[(int64_t)row * ldc] = acc[i][j][r];
            }
    }
}

}  // namespace mfma
}  // namespace tgemm
