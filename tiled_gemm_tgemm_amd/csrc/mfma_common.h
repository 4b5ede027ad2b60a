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

// Map tile id wg of nwg = tiles_m * tiles_n (the hardware work-group id when
// the grid has one work-group per tile) to a C tile (tm, tn).  The hardware
// deals work-group ids round-robin to the eight XCDs (each with its own L2):
// XCD x holds ids x, x+8, x+16, ...; a persistent grid whose size is a
// multiple of 8 keeps tile id ≡ work-group id (mod 8).  Each XCD is given the
// contiguous run of logical ids that starts after the runs of XCDs 0..x-1,
// and logical ids walk groups of group_m tile rows column by column, so the
// work-groups resident on one XCD cover a compact block of C tiles and share
// A rows and B columns in its L2.  Both steps are bijections on [0, nwg).
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int group_m, int &tm, int &tn,
                                        int wg = blockIdx.x, int nwg = gridDim.x)
{
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

// Reading one operand's fragments for a k-group from an LDS stage.  In step
// s of k-group g the lanes of half h feed k = 8g + 4h + s to both operands,
// so each lane needs four consecutive values of k per 32-row (or 32-column)
// block.  A slice kept k-contiguous ([mn][k], KC) gives them in one 16-byte
// read at `off`; a slice kept mn-contiguous ([k][mn], row stride S words)
// gives them in four 4-byte reads at off, off + S, off + 2S, off + 3S.
template <bool KC, int S>
__device__ __forceinline__ f32x4 read_frag(const float *base, int off)
{
    if constexpr (KC) {
        return *reinterpret_cast<const f32x4 *>(base + off);
    } else {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = base[off + q * S];
        return v;
    }
}

// Word distance from a lane's fragment of k-group 0 to its fragment of k-group
// g in the same slice: 8g values of k further along a KC row, or 8g rows
// further down an MC slice (row stride S).
template <bool KC, int S>
__device__ __forceinline__ constexpr int group_step(int g)
{
    return KC ? 8 * g : 8 * g * S;
}

// One wavefront's fragments of one k-group: a[i] for its FM row blocks of A,
// b[j] for its FN column blocks of B.
template <int FM, int FN, bool A_KC, int AS, bool B_KC, int BS>
struct Fragments {
    f32x4 a[FM];
    f32x4 b[FN];

    // a_off / b_off: the offsets of k-group 0 (frag_offset with g = 0); the
    // step to group g is a compile-time constant once the caller's loop over
    // groups is unrolled, so it folds into the LDS reads' immediate offsets
    // and only group 0's offsets occupy registers.
    __device__ __forceinline__ void read(const float *as, const float *bs, const int (&a_off)[FM],
                                         const int (&b_off)[FN], int g)
    {
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = read_frag<A_KC, AS>(as, a_off[i] + group_step<A_KC, AS>(g));
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = read_frag<B_KC, BS>(bs, b_off[j] + group_step<B_KC, BS>(g));
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

// The same steps with the operands exchanged: the matrix core then forms
// the transpose of each 32×32 block, so that a lane holds four consecutive
// columns of one row of C (store_c_t) instead of four rows of one column.
// The products and the order in which they are added are the same.
template <int FM, int FN, class Frag>
__device__ __forceinline__ void mfma_group_t(f32x16 (&acc)[FM][FN], const Frag &f)
{
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.b[j][s], f.a[i][s], acc[i][j], 0, 0, 0);
}

// Word offset of this lane's fragment of block `blk` (32 rows of A or 32
// columns of B, counted from the wavefront's first) for k-group g, in a
// slice kept KC ([mn][k], row stride S) or MC ([k][mn], row stride S).
template <bool KC, int S>
__device__ __forceinline__ int frag_offset(int mn, int g, int half)
{
    return KC ? mn * S + 8 * g + 4 * half : (8 * g + 4 * half) * S + mn;
}

// A whole phase of BK values of k from one LDS stage; the reads of group
// g+1 are issued before the matrix-core steps of group g.  a_off[i] and
// b_off[j] are the k-group 0 offsets from frag_offset.
template <int FM, int FN, int BK, bool A_KC, int AS, bool B_KC, int BS>
__device__ __forceinline__ void mfma_phase(f32x16 (&acc)[FM][FN], const float *as, const float *bs,
                                           const int (&a_off)[FM], const int (&b_off)[FN])
{
    Fragments<FM, FN, A_KC, AS, B_KC, BS> f[2];
    f[0].read(as, bs, a_off, b_off, 0);
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
        if (g + 1 < BK / 8) f[(g + 1) & 1].read(as, bs, a_off, b_off, g + 1);
        mfma_group<FM, FN>(acc, f[g & 1]);
    }
}

// Scheduling hints for one k-group's MFMA block: NX instructions of class MX
// and then NY of class MY are spread evenly among its NM matrix-core
// instructions (classes as for __builtin_amdgcn_sched_group_barrier: 0x008
// MFMA, 0x020 VMEM read, 0x100 DS read, 0x200 DS write).
template <int NM, int NX, int MX, int NY, int MY, int ID>
__device__ __forceinline__ void interleave()
{
    constexpr int n = NX + NY;
    constexpr int per = n == 0 ? NM : (NM / n > 0 ? NM / n : 1);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, per, ID);
        __builtin_amdgcn_sched_group_barrier(MX, 1, ID);
    }
#pragma unroll
    for (int i = 0; i < NY; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, per, ID);
        __builtin_amdgcn_sched_group_barrier(MY, 1, ID);
    }
    if constexpr (NM > per * n) __builtin_amdgcn_sched_group_barrier(0x008, NM - per * n, ID);
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

// The epilogue for blocks formed by mfma_group_t: accumulator r of lane (l32,
// half) in block (i, j) is C row i*32 + l32, column j*32 + 8*(r/4) + 4*half +
// r%4.  With `vec` (C and its leading dimension 16-byte aligned) each group
// of four columns inside C is one 16-byte store; otherwise, and at the last
// columns, one store per element.  Rows >= M and columns >= N are not written.
template <int FM, int FN>
__device__ __forceinline__ void store_c_t(const f32x16 (&acc)[FM][FN], float *__restrict__ C, int64_t ldc,
                                          int M, int N, int row0, int col0, int half, int l32, bool vec)
{
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = row0 + i * 32 + l32;
        if (row >= M) continue;
        float *c = C + (int64_t)row * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = col0 + j * 32 + 8 * q + 4 * half;
                if (vec && col + 3 < N) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                    *reinterpret_cast<f32x4 *>(c + col) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N) c[col + e] = acc[i][j][4 * q + e];
                }
            }
    }
}

}  // namespace mfma
}  // namespace tgemm
