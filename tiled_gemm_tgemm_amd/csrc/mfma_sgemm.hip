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
//   from device memory into LDS with 16-byte loads in which consecutive lanes
//   read consecutive addresses of one row (page 1, section [Coalescing];
//   page 2 §1.4, bursts).  Elements outside the matrix load as zero.
// * LDS holds two stages.  Phase p reads stage p%2 while the loads for phase
//   p+1 are in flight in registers; they are written to the other stage after
//   the matrix-core work of phase p.  One barrier per phase then covers both
//   of the pages' reasons to synchronise (page 1, "__syncthreads( )"): the
//   stage about to be read is complete, and the stage about to be refilled
//   was last read before the previous barrier.
// * "More work per thread" (page 1, end of "Tile Size 결정"): each 64-lane
//   wavefront owns a (BM/WM)×(BN/WN) sub-tile held in matrix-core accumulator
//   registers for the whole K loop, built from 32×32 blocks of
//   v_mfma_f32_32x32x2_f32.  C is written once at the end.
// * LDS layout against bank conflicts (page 2 §1.3-1.4, tile[32][33]):
//   A is kept row-major, As[m][k], rows padded from BK to BK+4 words; B is
//   kept as it arrives, Bs[k][n], rows padded from BN to BN+8 words.
// * The k order inside a phase is permuted so that A needs no transpose
//   ("corner turning", page 1 section [Coalescing], is done by the choice of
//   k instead): in step s of k-group g, the lanes of half h of the wavefront
//   feed k = 8g + 4h + s to both operands.  A lane's four A values for the
//   four steps of a group are then adjacent in As and come in one 16-byte LDS
//   read.  Summation order is not specified by the product's definition;
//   rounding stays within the accepted bound and integer inputs stay exact.
// * Work-group order: the hardware deals work-groups round-robin to the eight
//   XCDs, each with its own L2.  Ids are renumbered so that each XCD receives
//   a contiguous run, and runs are laid over groups of tile rows so that the
//   work-groups resident on one XCD share A rows and B columns in its L2.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kXcds = 8;

template <int BM_, int BN_, int BK_, int WM_, int WN_, int VEC_, int GROUP_M_, int OCC_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, VEC = VEC_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int OCC = OCC_;                    // wavefronts per SIMD to budget registers for
    static constexpr int NT = kWave * WM * WN;         // threads per work-group
    static constexpr int TM = BM / WM, TN = BN / WN;   // wavefront sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;   // 32×32 blocks per wavefront
    static constexpr int AS = BK + 4;                  // As row stride (words)
    static constexpr int BS = BN + 8;                  // Bs row stride (words)
    static constexpr int A_STAGE = BM * AS;
    static constexpr int B_STAGE = BK * BS;
    static constexpr int LDS_WORDS = 2 * (A_STAGE + B_STAGE);
    static constexpr int LA = BM * BK / (VEC * NT);    // A loads per thread per phase
    static constexpr int LB = BK * BN / (VEC * NT);    // B loads per thread per phase
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront sub-tile must be 32-aligned");
    static_assert(BK % 8 == 0, "phase depth must be a multiple of 8");
    static_assert((BM * BK) % (VEC * NT) == 0 && (BK * BN) % (VEC * NT) == 0,
                  "tile slices must split evenly over the threads");
    static_assert(BK % VEC == 0 && BN % VEC == 0, "vector loads must stay inside a row");
    static_assert(LDS_WORDS * 4 <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <int VEC>
struct VecT;
template <>
struct VecT<4> {
    typedef f32x4 type;
};
template <>
struct VecT<1> {
    typedef float type;
};

// Map the hardware work-group id to a C tile (tile_m, tile_n).
template <class G>
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    // XCD x holds ids x, x+8, x+16, ...; give it the contiguous run of
    // logical ids that starts after the runs of XCDs 0..x-1.
    const int q = nwg / kXcds, r = nwg % kXcds;
    const int x = wg % kXcds;
    const int logical = wg / kXcds + x * q + (x < r ? x : r);
    // Groups of GROUP_M tile rows; inside a group, consecutive ids walk down
    // the rows first, so a run of ids covers a compact block of tiles.
    const int per_group = G::GROUP_M * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * G::GROUP_M;
    const int rows = min(tiles_m - first_m, G::GROUP_M);
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

template <class G>
__global__ __launch_bounds__(G::NT) __attribute__((amdgpu_waves_per_eu(G::OCC, G::OCC)))
void mfma_sgemm_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
                       const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                       int64_t ldc)
{
    typedef typename VecT<G::VEC>::type vec_t;
    constexpr int VEC = G::VEC;

    __shared__ __attribute__((aligned(16))) float lds[G::LDS_WORDS];

    const int tiles_m = (M + G::BM - 1) / G::BM;
    const int tiles_n = (N + G::BN - 1) / G::BN;
    int tm, tn;
    tile_of<G>(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * G::BM;
    const int n0 = tn * G::BN;

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = t / kWave;
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int l32 = lane % 32, half = lane / 32;

    // ---- per-thread load slots (fixed rows/columns; k advances per phase)
    // A slot i covers elements (i*NT + t)*VEC .. +VEC-1 of the BM×BK slice.
    int a_r[G::LA], a_c[G::LA];
    const float *a_ptr[G::LA];
    bool a_row_ok[G::LA];
#pragma unroll
    for (int i = 0; i < G::LA; ++i) {
        const int e = (i * G::NT + t) * VEC;
        a_r[i] = e / G::BK;
        a_c[i] = e % G::BK;
        const int row = m0 + a_r[i];
        a_row_ok[i] = row < M;
        a_ptr[i] = A + (int64_t)(a_row_ok[i] ? row : 0) * lda + a_c[i];
    }
    // B slot i covers elements (i*NT + t)*VEC .. +VEC-1 of the BK×BN slice.
    int b_r[G::LB], b_c[G::LB];
    const float *b_ptr[G::LB];
    bool b_col_ok[G::LB];
#pragma unroll
    for (int i = 0; i < G::LB; ++i) {
        const int e = (i * G::NT + t) * VEC;
        b_r[i] = e / G::BN;
        b_c[i] = e % G::BN;
        const int col = n0 + b_c[i];
        b_col_ok[i] = col < N;
        b_ptr[i] = B + (int64_t)b_r[i] * ldb + (b_col_ok[i] ? col : 0);
    }

    vec_t a_reg[G::LA], b_reg[G::LB];
    const vec_t zero = vec_t(0.0f);

    // Global -> registers for the phase starting at k0.  A slot whose
    // elements lie outside the matrix reads the operand's first element
    // instead (a valid address) and is replaced by zero only when it is
    // written to LDS, so nothing waits on these loads before the phase's
    // matrix-core work.
    auto load_phase = [&](int k0) {
#pragma unroll
        for (int i = 0; i < G::LA; ++i) {
            const bool ok = a_row_ok[i] && (k0 + a_c[i] < K);
            a_reg[i] = *reinterpret_cast<const vec_t *>(ok ? a_ptr[i] + k0 : A);
        }
#pragma unroll
        for (int i = 0; i < G::LB; ++i) {
            const bool ok = b_col_ok[i] && (k0 + b_r[i] < K);
            b_reg[i] = *reinterpret_cast<const vec_t *>(ok ? b_ptr[i] + (int64_t)k0 * ldb : B);
        }
    };
    // Registers -> LDS stage, zeroing what lies outside the matrix.
    auto store_phase = [&](int stage, int k0) {
        float *as = lds + stage * (G::A_STAGE + G::B_STAGE);
        float *bs = as + G::A_STAGE;
#pragma unroll
        for (int i = 0; i < G::LA; ++i) {
            const bool ok = a_row_ok[i] && (k0 + a_c[i] < K);
            *reinterpret_cast<vec_t *>(as + a_r[i] * G::AS + a_c[i]) = ok ? a_reg[i] : zero;
        }
#pragma unroll
        for (int i = 0; i < G::LB; ++i) {
            const bool ok = b_col_ok[i] && (k0 + b_r[i] < K);
            *reinterpret_cast<vec_t *>(bs + b_r[i] * G::BS + b_c[i]) = ok ? b_reg[i] : zero;
        }
    };

    f32x16 acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x16(0.0f);

    // Offsets of this lane's fragments inside a stage.
    const int a_frag = (wm * G::TM + l32) * G::AS + 4 * half;       // + i*32*AS + 8g
    const int b_frag = (4 * half) * G::BS + wn * G::TN + l32;       // + (8g+s)*BS + j*32

    // Fragments of one k-group (8 values of k): af[i][s] and bf[j][s] feed
    // step s of 32×32 block (i, j).  Two sets, so that the LDS reads of
    // group g+1 are in flight while group g's matrix-core work issues.
    f32x4 af[2][G::FM];
    float bf[2][G::FN][4];
    auto read_group = [&](const float *as, const float *bs, int g, int set) {
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
            af[set][i] = *reinterpret_cast<const f32x4 *>(as + a_frag + i * 32 * G::AS + 8 * g);
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s) bf[set][j][s] = bs[b_frag + (8 * g + s) * G::BS + j * 32];
    };

    constexpr int GROUPS = G::BK / 8;
    const int phases = (K + G::BK - 1) / G::BK;
    load_phase(0);
    store_phase(0, 0);
    __syncthreads();

    for (int p = 0; p < phases; ++p) {
        const bool more = p + 1 < phases;
        if (more) load_phase((p + 1) * G::BK);

        const float *as = lds + (p & 1) * (G::A_STAGE + G::B_STAGE);
        const float *bs = as + G::A_STAGE;
        read_group(as, bs, 0, 0);
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) {
            if (g + 1 < GROUPS) read_group(as, bs, g + 1, (g + 1) & 1);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < G::FM; ++i)
#pragma unroll
                    for (int j = 0; j < G::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            af[g & 1][i][s], bf[g & 1][j][s], acc[i][j], 0, 0, 0);
        }

        if (more) store_phase((p + 1) & 1, (p + 1) * G::BK);
        __syncthreads();
    }

    // ---- epilogue: accumulator register r of lane (l32, half) in block
    // (i, j) is C row 8*(r/4) + 4*half + r%4 and column l32 of that block.
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {
            const int col = n0 + wn * G::TN + j * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * G::TM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                if (row < M) C[(int64_t)row * ldc + col] = acc[i][j][r];
            }
        }
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
typedef Cfg<256, 256, 32, 2, 2, 4, 4, 1> Big4;
typedef Cfg<128, 128, 32, 2, 2, 4, 8, 2> Mid4;
typedef Cfg<64, 64, 32, 2, 2, 4, 8, 4> Small4;
typedef Cfg<256, 256, 32, 2, 2, 1, 4, 1> Big1;
typedef Cfg<128, 128, 32, 2, 2, 1, 8, 2> Mid1;
typedef Cfg<64, 64, 32, 2, 2, 1, 8, 4> Small1;

template <class G>
constexpr int wg_per_cu()
{
    return (160 * 1024) / (G::LDS_WORDS * 4);
}

const MfmaVariant kVariants[] = {
    {"m256n256k32_w2x2_vec4", 256, 256, 32, 4, wg_per_cu<Big4>(), &launch_cfg<Big4>},
    {"m128n128k32_w2x2_vec4", 128, 128, 32, 4, wg_per_cu<Mid4>(), &launch_cfg<Mid4>},
    {"m64n64k32_w2x2_vec4", 64, 64, 32, 4, wg_per_cu<Small4>(), &launch_cfg<Small4>},
    {"m256n256k32_w2x2_vec1", 256, 256, 32, 1, wg_per_cu<Big1>(), &launch_cfg<Big1>},
    {"m128n128k32_w2x2_vec1", 128, 128, 32, 1, wg_per_cu<Mid1>(), &launch_cfg<Mid1>},
    {"m64n64k32_w2x2_vec1", 64, 64, 32, 1, wg_per_cu<Small1>(), &launch_cfg<Small1>},
};

}  // namespace

int mfma_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }

const MfmaVariant *mfma_variant(int index)
{
    if (index < 0 || index >= mfma_variant_count()) return nullptr;
    return &kVariants[index];
}

}  // namespace tgemm
