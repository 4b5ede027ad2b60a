// Matrix-core kernel for small products (a few hundred to ~1000 on a side).
//
// Same product (page 1, "[Multi-Core & GPU Programming] CUDA - Matrix
// Multiplication", section [Matrix Multiplication]).  On small shapes the
// tiled kernels have too few tiles to give every SIMD a wavefront, and a
// phase holds fewer matrix-core steps than one trip to memory takes, so time
// goes to latency.  Here work is cut finer, the way page 1 ("Tile Size 결정")
// trades tile size against the number of blocks:
//
// * One work-group owns a 32×32 tile of C; its KS wavefronts split K into KS
//   contiguous ranges (a multiple of 8 long) and each accumulates its range
//   in one 32×32 block of v_mfma_f32_32x32x2_f32 accumulators.
// * Each wavefront reads its fragments straight from device memory, with the
//   k order of the tiled kernels (lane half h feeds k = 8g + 4h + s in step
//   s of group g): one 16-byte A read and four 4-byte B reads per lane per
//   group, coalesced along A rows and B rows (page 1, section [Coalescing]).
//   D groups are kept in flight in a ring of registers.  Buffer descriptors
//   rebased on every group return zero outside the matrix and outside the
//   wavefront's own K range, so edges need no branches.
// * The KS partial tiles are added in LDS in a fixed order (wavefront 0 first)
//   after one barrier — the only synchronisation — so results do not depend
//   on timing; C is written once, 32 consecutive columns per 32 lanes.
// * Transposed operands are read along the dimension they are contiguous in:
//   a k-contiguous operand (A as stored, B transposed) gives a lane its four
//   k values in one read; an mn-contiguous one (B as stored, A transposed) in
//   four reads, each coalesced across the 32 lanes of a half-wavefront.
#include "mfma_common.h"
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

using mfma::f32x16;
using mfma::f32x4;
using mfma::kWave;

constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t small_buffer(const float *base, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n, 0x00020000);
}

// One lane's fragment reads for one group of 8 values of k (k0 .. k0+7):
// the four values k0 + 4h .. k0 + 4h + 3 of row (A) or column (B) l32 of
// the tile.  `tile` points at the operand's element (mn0, 0) in its own
// storage order; reads outside rows/columns [0, mn_valid) or past ke give 0.
template <bool KC, int VEC>
struct SmallOperand {
    uint32_t lane_off[4];  // byte offsets of the lane's four values from (mn0, k0)

    __device__ __forceinline__ void init(int64_t ld, int mn_valid, int l32, int half)
    {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t o = KC ? l32 * ld + 4 * half + s : (4 * half + s) * ld + l32;
            lane_off[s] = l32 < mn_valid ? (uint32_t)(o * 4) : kOutside;
        }
    }

    __device__ __forceinline__ f32x4 load(const float *tile, int64_t ld, int k0, int ke, int K,
                                          int mn_valid, int half) const
    {
        f32x4 v;
        if constexpr (KC) {
            // k runs along the row: only this wavefront's range may be read
            const __amdgpu_buffer_rsrc_t r =
                small_buffer(tile + k0, ((int64_t)(mn_valid - 1) * ld + (K - k0)) * 4);
            if constexpr (VEC == 4) {
                const uint32_t o = k0 + 4 * half < ke ? lane_off[0] : kOutside;
                v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint32_t o = k0 + 4 * half + s < ke ? lane_off[s] : kOutside;
                    v[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0));
                }
            }
        } else {
            // k runs down the rows: rows >= ke lie past the extent
            const __amdgpu_buffer_rsrc_t r =
                small_buffer(tile + (int64_t)k0 * ld, ((int64_t)(ke - k0 - 1) * ld + mn_valid) * 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t o = lane_off[s];
                v[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0));
            }
        }
        return v;
    }
};

template <int KS_, int D_, int VEC_, int OCC_, bool TA_, bool TB_>
struct SmallCfg {
    static constexpr int KS = KS_, D = D_, VEC = VEC_, OCC = OCC_;
    static constexpr bool TA = TA_, TB = TB_;
    static constexpr int NT = kWave * KS;
};

template <class G>
__global__ __launch_bounds__(G::NT) __attribute__((amdgpu_waves_per_eu(G::OCC)))
void mfma_sgemm_small_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
                             const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                             int64_t ldc)
{
    constexpr int KS = G::KS, D = G::D, VEC = G::VEC;
    constexpr bool A_KC = !G::TA, B_KC = G::TB;
    __shared__ float part[KS][16 * kWave];

    const int tiles_m = (M + 31) / 32, tiles_n = (N + 31) / 32;
    int tm, tn;
    mfma::tile_of(tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * 32, n0 = tn * 32;
    const int rows_valid = min(32, M - m0), cols_valid = min(32, N - n0);

    const int t = threadIdx.x;
    const int lane = t % kWave, w = t / kWave;
    const int l32 = lane % 32, half = lane / 32;

    // this wavefront's K range [kb, ke), in whole groups of 8 except at K
    const int chunk = ((K + KS - 1) / KS + 7) / 8 * 8;
    const int kb = min(K, w * chunk), ke = min(K, kb + chunk);
    const int groups = (ke - kb + 7) / 8;

    SmallOperand<A_KC, VEC> oa;
    SmallOperand<B_KC, VEC> ob;
    oa.init(lda, rows_valid, l32, half);
    ob.init(ldb, cols_valid, l32, half);
    const float *a_tile = A + (A_KC ? (int64_t)m0 * lda : (int64_t)m0);
    const float *b_tile = B + (B_KC ? (int64_t)n0 * ldb : (int64_t)n0);

    f32x4 a_ring[D], b_ring[D];
    // Issue the reads of group g (k0 = kb + 8g) into ring slot `slot`; past
    // the wavefront's range they read zero.
    auto issue = [&] __device__(int g, int slot) {
        const int k0 = kb + 8 * g;
        a_ring[slot] = oa.load(a_tile, lda, k0, ke, K, rows_valid, half);
        b_ring[slot] = ob.load(b_tile, ldb, k0, ke, K, cols_valid, half);
    };

    f32x16 acc = f32x16(0.0f);
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j, j);
    for (int g0 = 0; g0 < groups; g0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a_ring[j][s], b_ring[j][s], acc, 0, 0, 0);
            issue(g0 + j + D, j);  // past the range: reads zero, never used for a sum
        }
    }

    // fixed-order sum of the KS partial tiles
#pragma unroll
    for (int r = 0; r < 16; ++r) part[w][r * kWave + lane] = acc[r];
    __syncthreads();
#pragma unroll
    for (int o = t; o < 16 * kWave; o += G::NT) {
        float v = part[0][o];
#pragma unroll
        for (int q = 1; q < KS; ++q) v += part[q][o];
        const int ln = o % kWave, r = o / kWave;
        const int row = m0 + 8 * (r / 4) + 4 * (ln / 32) + r % 4;
        const int col = n0 + ln % 32;
        if (row < M && col < N) C[(int64_t)row * ldc + col] = v;
    }
}

template <class G>
hipError_t launch_small(const GemmArgs &g, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((g.M + 31) / 32) * ((g.N + 31) / 32);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sgemm_small_kernel<G>),
                           dim3((unsigned)tiles), dim3(G::NT), args, 0, stream);
}

// One split in its four operand orders (NN, TN, NT, TT).
template <int KS, int D, int VEC, int OCC>
struct Split {
    template <bool TA, bool TB>
    using C = SmallCfg<KS, D, VEC, OCC, TA, TB>;
    static hipError_t launch(const GemmArgs &g, hipStream_t stream)
    {
        switch ((g.trans_a ? 1 : 0) + (g.trans_b ? 2 : 0)) {
            case 0: return launch_small<C<false, false>>(g, stream);
            case 1: return launch_small<C<true, false>>(g, stream);
            case 2: return launch_small<C<false, true>>(g, stream);
            default: return launch_small<C<true, true>>(g, stream);
        }
    }
};

//            KS  D VEC OCC
typedef Split<4, 4, 4, 4> S4D4v4;
typedef Split<8, 8, 4, 4> S8D8v4;
typedef Split<4, 4, 1, 4> S4D4v1;
typedef Split<8, 8, 1, 4> S8D8v1;

// Offsets span 32 rows of a k-contiguous operand and 8 rows of an
// mn-contiguous one.
constexpr int64_t kMaxLdKc = ((((int64_t)1 << 31) - 16) / 4 - 8) / 32;
constexpr int64_t kMaxLdMc = ((((int64_t)1 << 31) - 16) / 4 - 32) / 8;

// bk = 8·KS: the K granularity of a work-group.  Efficiencies and the fixed
// cost per round measured on MI355X over 27 small, ragged, skinny and long-K
// shapes with both load widths (one work-group per CU: 256 tiles with
// K = 16384; CU full: 512 or 1024 tiles; the fixed cost from 64³).  On every
// one of them a 32×32 tile of the LDS-staged kernel with K split over its
// wavefronts (mfma_sgemm.hip) is as fast or faster, so the selection model
// does not pick these; they stay available through tgemm_sgemm_mfma.
const MfmaVariant kSmallVariants[] = {
    {"m32n32k8_s4d4_vec4", 32, 32, 32, 4, 4, kMaxLdKc, kMaxLdMc, kMaxLdMc, kMaxLdKc, true, 0.24, 0.39, 10000.0,
     &S4D4v4::launch},
    {"m32n32k8_s8d8_vec4", 32, 32, 64, 4, 2, kMaxLdKc, kMaxLdMc, kMaxLdMc, kMaxLdKc, true, 0.365, 0.43, 22000.0,
     &S8D8v4::launch},
    {"m32n32k8_s4d4_vec1", 32, 32, 32, 1, 4, kMaxLdKc, kMaxLdMc, kMaxLdMc, kMaxLdKc, true, 0.18, 0.20, 10000.0,
     &S4D4v1::launch},
    {"m32n32k8_s8d8_vec1", 32, 32, 64, 1, 2, kMaxLdKc, kMaxLdMc, kMaxLdMc, kMaxLdKc, true, 0.215, 0.21, 22000.0,
     &S8D8v1::launch},
};

}  // namespace

int mfma_small_variant_count() { return (int)(sizeof(kSmallVariants) / sizeof(kSmallVariants[0])); }

const MfmaVariant *mfma_small_variant(int index)
{
    if (index < 0 || index >= mfma_small_variant_count()) return nullptr;
    return &kSmallVariants[index];
}

}  // namespace tgemm
