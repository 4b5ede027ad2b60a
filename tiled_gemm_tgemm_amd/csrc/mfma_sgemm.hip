// The product kernel: tiled fp32 GEMM on the gfx950 matrix cores.
//
// What it computes is page 1's product ("[Multi-Core & GPU Programming] CUDA -
// Matrix Multiplication", section [Matrix Multiplication]); how it is staged
// follows the tiling plan of page 1's section [Shared Memory] and page 2
// ("Lec 29 · GPU Architecture (2)") §1.1-1.2, redone for CDNA4:
//
// * One work-group owns a BM×BN tile of C and walks K in phases of BK
//   (page 1, "Work Flow - Compute Block(0, 0)": tile phases).
// * Per phase the work-group copies a BM×BK slice of A and a BK×BN slice of B
//   from device memory into LDS.  Consecutive lanes read consecutive
//   addresses of one row (page 1, section [Coalescing]; page 2 §1.4, bursts):
//   4 lanes × 16 bytes cover a 64-byte A row segment, 32 lanes a 512-byte B
//   row.
// * The copies are buffer loads: each phase rebases a buffer descriptor on the
//   slice's first element with the exact byte extent of what remains of the
//   operand, and every lane keeps a fixed 32-bit offset.  Reads past the
//   extent return zero in hardware, and lanes whose row (A) or column (B)
//   lies outside the matrix carry an offset beyond any extent, so edge tiles
//   need no per-element tests and no load leaves the operand.  Only the last,
//   partial phase of K masks A's columns explicitly; B's rows past K fall
//   outside its extent on their own.
// * LDS holds two stages.  Phase p reads stage p%2 while the loads for phase
//   p+1 are in flight in registers; they are written to the other stage after
//   the matrix-core work of phase p.  One barrier per phase covers both of the
//   pages' reasons to synchronise (page 1, "__syncthreads( )"): the stage
//   about to be read is complete, and the stage about to be refilled was last
//   read before the previous barrier.  The main loop has no branches (the
//   partial K phase is peeled off after it), so the compiler schedules loads,
//   LDS traffic and matrix-core instructions of a phase as one block.
// * "More work per thread" (page 1, end of "Tile Size 결정"): each 64-lane
//   wavefront owns a (BM/WM)×(BN/WN) sub-tile held in accumulator registers
//   for the whole K loop, built from 32×32 blocks of v_mfma_f32_32x32x2_f32.
//   C is written once at the end.
// * Tile size (page 1, "Tile Size 결정", redone for gfx950's 160 KB of LDS and
//   512 registers per lane and SIMD): the 256×128×16 tile takes 57 KB of LDS
//   and at most 256 registers per lane, so two work-groups share a compute
//   unit and each one's barrier and load waits are covered by the other's
//   matrix-core work.
// * LDS layout against bank conflicts (page 2 §1.3-1.4, tile[32][33]): A is
//   kept row-major, As[m][k], rows padded from BK to BK+4 words (16-byte
//   reads of 32 rows hit distinct banks); B is kept as it arrives, Bs[k][n],
//   rows padded from BN to BN+8 words.
// * Corner turning (page 1, section [Coalescing]) by the choice of k: see
//   mfma_common.h.  The summation order is not part of the product's
//   definition; rounding stays within the accepted bound and integer inputs
//   whose partial sums stay below 2^24 come out exact.
#include "mfma_common.h"
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

using mfma::f32x16;
using mfma::f32x4;
using mfma::kWave;

constexpr uint32_t kOutside = 0x80000000u;  // an offset beyond every extent (all are < 2^31)

template <int BM_, int BN_, int BK_, int WM_, int WN_, int VEC_, int GROUP_M_, int OCC_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, VEC = VEC_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int OCC = OCC_;                   // wavefronts per SIMD to budget registers for
    static constexpr int NT = kWave * WM * WN;         // threads per work-group
    static constexpr int TM = BM / WM, TN = BN / WN;   // wavefront sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;   // 32×32 blocks per wavefront
    static constexpr int AS = BK + 4;                  // As row stride (words)
    static constexpr int BS = BN + 8;                  // Bs row stride (words)
    static constexpr int A_STAGE = BM * AS;
    static constexpr int STAGE = A_STAGE + BK * BS;
    static constexpr int LDS_WORDS = 2 * STAGE;
    static constexpr int LA = BM * BK / (VEC * NT);    // A loads per thread per phase
    static constexpr int LB = BK * BN / (VEC * NT);    // B loads per thread per phase
    static constexpr int RA = NT * VEC / BK;           // rows between a thread's A slots
    static constexpr int RB = NT * VEC / BN;           // rows between a thread's B slots
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront sub-tile must be 32-aligned");
    static_assert(BK % 8 == 0, "phase depth must be a multiple of 8");
    static_assert((NT * VEC) % BK == 0 && (NT * VEC) % BN == 0 && LA >= 1 && LB >= 1 &&
                      LA * RA == BM && LB * RB == BK,
                  "slices must split into whole rows per load step");
    static_assert(LDS_WORDS * 4 <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <int VEC>
struct Vec;
template <>
struct Vec<4> {
    typedef f32x4 type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
template <>
struct Vec<1> {
    typedef float type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
};

// Raw buffer over [base, base + bytes); bytes is clamped to 2^31 - 1, which
// only ever shortens an extent that reaches beyond every offset in use.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const float *base, int64_t bytes)
{
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n, 0x00020000);
}

template <class G>
__global__ __launch_bounds__(G::NT) __attribute__((amdgpu_waves_per_eu(G::OCC, G::OCC)))
void mfma_sgemm_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
                       const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                       int64_t ldc)
{
    typedef typename Vec<G::VEC>::type vec_t;
    constexpr int VEC = G::VEC;

    __shared__ __attribute__((aligned(16))) float lds[G::LDS_WORDS];

    const int tiles_m = (M + G::BM - 1) / G::BM;
    const int tiles_n = (N + G::BN - 1) / G::BN;
    int tm, tn;
    mfma::tile_of(tiles_m, tiles_n, G::GROUP_M, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int rows_valid = min(G::BM, M - m0), cols_valid = min(G::BN, N - n0);

    const int t = threadIdx.x;
    const int lane = t % kWave, wave = t / kWave;
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int l32 = lane % 32, half = lane / 32;

    // Load slots.  A slot i: row a_r0 + i*RA, columns a_c .. a_c+VEC-1 of the
    // BM×BK slice; B slot i: row b_r0 + i*RB, columns b_c .. b_c+VEC-1 of the
    // BK×BN slice.  Offsets are in bytes from the slice's first element.
    const int a_r0 = t * VEC / G::BK, a_c = t * VEC % G::BK;
    const int b_r0 = t * VEC / G::BN, b_c = t * VEC % G::BN;
    uint32_t a_off[G::LA], b_off[G::LB];
#pragma unroll
    for (int i = 0; i < G::LA; ++i) {
        const int r = a_r0 + i * G::RA;
        a_off[i] = r < rows_valid ? (uint32_t)((r * lda + a_c) * 4) : kOutside;
    }
#pragma unroll
    for (int i = 0; i < G::LB; ++i) {
        const int r = b_r0 + i * G::RB;
        b_off[i] = b_c < cols_valid ? (uint32_t)((r * ldb + b_c) * 4) : kOutside;
    }
    const float *a_panel = A + (int64_t)m0 * lda;
    const float *b_panel = B + n0;

    vec_t a_reg[G::LA], b_reg[G::LB];
    // Issue the loads of the phase starting at k0.  `partial` marks the last
    // phase when K is not a multiple of BK: A columns >= K are then read as
    // zero explicitly (B's rows >= K lie past its extent anyway).
    auto load_phase = [&] __device__(int k0, bool partial) {
        const __amdgpu_buffer_rsrc_t ra =
            buffer(a_panel + k0, ((int64_t)(rows_valid - 1) * lda + (K - k0)) * 4);
        const __amdgpu_buffer_rsrc_t rb =
            buffer(b_panel + (int64_t)k0 * ldb, ((int64_t)(K - k0 - 1) * ldb + cols_valid) * 4);
        const bool a_cut = partial && k0 + a_c >= K;
#pragma unroll
        for (int i = 0; i < G::LA; ++i) {
            const uint32_t off = a_cut ? kOutside : a_off[i];
            a_reg[i] = Vec<VEC>::load(ra, off);
        }
#pragma unroll
        for (int i = 0; i < G::LB; ++i) {
            const uint32_t off = b_off[i];
            b_reg[i] = Vec<VEC>::load(rb, off);
        }
    };
    // LDS word offset of each A slot in a stage
    int a_st[G::LA];
#pragma unroll
    for (int i = 0; i < G::LA; ++i) a_st[i] = (a_r0 + i * G::RA) * G::AS + a_c;
    float *b_st = lds + G::A_STAGE + b_r0 * G::BS + b_c;
    auto store_phase = [&] __device__(int stage) {
#pragma unroll
        for (int i = 0; i < G::LA; ++i)
            *reinterpret_cast<vec_t *>(lds + stage * G::STAGE + a_st[i]) = a_reg[i];
#pragma unroll
        for (int i = 0; i < G::LB; ++i)
            *reinterpret_cast<vec_t *>(b_st + stage * G::STAGE + i * G::RB * G::BS) = b_reg[i];
    };

    f32x16 acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x16(0.0f);

    int a_frag[G::BK / 8][G::FM];
#pragma unroll
    for (int g = 0; g < G::BK / 8; ++g)
#pragma unroll
        for (int i = 0; i < G::FM; ++i) a_frag[g][i] = (wm * G::TM + i * 32 + l32) * G::AS + 8 * g + 4 * half;
    const int b_frag = (4 * half) * G::BS + wn * G::TN + l32;
    auto compute = [&] __device__(int stage) {
        const float *as = lds + stage * G::STAGE;
        mfma::mfma_phase<G::FM, G::FN, G::BS, G::BK>(acc, as, as + G::A_STAGE, a_frag, b_frag);
    };

    const int full = K / G::BK;            // phases with all BK values of k
    const bool partial = K % G::BK != 0;   // one more, shorter phase
    load_phase(0, full == 0);
    store_phase(0);
    __syncthreads();
    int p = 0;
    for (; p + 1 < full; ++p) {            // the next phase is a full one
        load_phase((p + 1) * G::BK, false);
        compute(p & 1);
        store_phase((p + 1) & 1);
        __syncthreads();
    }
    if (partial && full > 0) {
        load_phase(full * G::BK, true);
        compute(p & 1);
        store_phase((p + 1) & 1);
        __syncthreads();
        ++p;
    }
    compute(p & 1);

    mfma::store_c<G::FM, G::FN>(acc, C, ldc, M, N, m0 + wm * G::TM, n0 + wn * G::TN, half, l32);
}

template <class G>
hipError_t launch_cfg(const GemmArgs &g, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((g.M + G::BM - 1) / G::BM) * ((g.N + G::BN - 1) / G::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sgemm_kernel<G>),
                           dim3((unsigned)tiles), dim3(G::NT), args, 0, stream);
}

//           BM   BN  BK WM WN VEC GROUP_M OCC
typedef Cfg<256, 128, 16, 2, 2, 4, 4, 2> Large4;
typedef Cfg<128, 128, 32, 2, 2, 4, 8, 2> Mid4;
typedef Cfg<64, 64, 32, 2, 2, 4, 8, 4> Small4;
typedef Cfg<256, 128, 16, 2, 2, 1, 4, 2> Large1;
typedef Cfg<128, 128, 32, 2, 2, 1, 8, 2> Mid1;
typedef Cfg<64, 64, 32, 2, 2, 1, 8, 4> Small1;

template <class G>
constexpr int wg_per_cu()
{
    return (160 * 1024) / (G::LDS_WORDS * 4) < G::OCC ? (160 * 1024) / (G::LDS_WORDS * 4) : G::OCC;
}

// Buffer offsets are 32-bit and kept below 2^31: a slot's offset spans at
// most BM rows of A or BK rows of B, which bounds the leading dimensions
// these configurations take.
template <class G>
constexpr int64_t max_lda()
{
    return ((((int64_t)1 << 31) - 16) / 4) / G::BM;
}
template <class G>
constexpr int64_t max_ldb()
{
    return ((((int64_t)1 << 31) - 16) / 4 - G::BN) / G::BK;
}

#define TGEMM_VARIANT(name, G, alone, full)                                                    \
    {                                                                                           \
        name, G::BM, G::BN, G::BK, G::VEC, wg_per_cu<G>(), max_lda<G>(), max_ldb<G>(), alone, \
            full, 7000.0, &launch_cfg<G>                                                        \
    }

// Efficiencies measured on MI355X (square and ragged shapes from 512 to 8192).
const MfmaVariant kVariants[] = {
    TGEMM_VARIANT("m256n128k16_w2x2_vec4", Large4, 0.70, 0.91),
    TGEMM_VARIANT("m128n128k32_w2x2_vec4", Mid4, 0.68, 0.88),
    TGEMM_VARIANT("m64n64k32_w2x2_vec4", Small4, 0.49, 0.77),
    TGEMM_VARIANT("m256n128k16_w2x2_vec1", Large1, 0.66, 0.86),
    TGEMM_VARIANT("m128n128k32_w2x2_vec1", Mid1, 0.64, 0.84),
    TGEMM_VARIANT("m64n64k32_w2x2_vec1", Small1, 0.47, 0.74),
};

}  // namespace

int mfma_buffer_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }

const MfmaVariant *mfma_buffer_variant(int index)
{
    if (index < 0 || index >= mfma_buffer_variant_count()) return nullptr;
    return &kVariants[index];
}

}  // namespace tgemm
