// Matrix-core kernel for operands whose leading dimensions are too large for
// the 32-bit buffer offsets of mfma_sgemm.hip (operands as stored only).  Same product, same tiling
// plan (page 1, "[Multi-Core & GPU Programming] CUDA - Matrix
// Multiplication", section [Shared Memory]; page 2, "Lec 29 · GPU
// Architecture (2)", §1.2): 128×128 tiles, phases of 32 values of k, two LDS
// stages and one barrier per phase, register-blocked v_mfma_f32_32x32x2_f32
// accumulation.  The copies use 64-bit pointers; a slot whose element lies
// outside the matrix reads the operand's first element instead (a valid
// address) and is replaced by zero when it is written to LDS.
#include "mfma_common.h"
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

using mfma::f32x16;
using mfma::f32x4;
using mfma::kWave;

template <int BM_, int BN_, int BK_, int WM_, int WN_, int VEC_, int GROUP_M_, int OCC_>
struct FlatCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, VEC = VEC_;
    static constexpr int GROUP_M = GROUP_M_, OCC = OCC_;
    static constexpr int NT = kWave * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int AS = BK + 4, BS = BN + 8;
    static constexpr int A_STAGE = BM * AS;
    static constexpr int STAGE = A_STAGE + BK * BS;
    static constexpr int LDS_WORDS = 2 * STAGE;
    static constexpr int LA = BM * BK / (VEC * NT), LB = BK * BN / (VEC * NT);
    static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 8 == 0, "tile shape");
    static_assert((BM * BK) % (VEC * NT) == 0 && (BK * BN) % (VEC * NT) == 0, "even split");
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

template <class G>
__global__ __launch_bounds__(G::NT) __attribute__((amdgpu_waves_per_eu(G::OCC, G::OCC)))
void mfma_sgemm_flat_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
                            const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                            int64_t ldc)
{
    typedef typename VecT<G::VEC>::type vec_t;
    constexpr int VEC = G::VEC;

    __shared__ __attribute__((aligned(16))) float lds[G::LDS_WORDS];

    const int tiles_m = (M + G::BM - 1) / G::BM;
    const int tiles_n = (N + G::BN - 1) / G::BN;
    int tm, tn;
    mfma::tile_of(tiles_m, tiles_n, G::GROUP_M, tm, tn);
    const int m0 = tm * G::BM, n0 = tn * G::BN;

    const int t = threadIdx.x;
    const int lane = t % kWave, wave = t / kWave;
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int l32 = lane % 32, half = lane / 32;

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
    auto load_phase = [&] __device__(int k0) {
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
    auto store_phase = [&] __device__(int stage, int k0) {
        float *as = lds + stage * G::STAGE;
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

    int a_frag[G::FM], b_frag[G::FN];  // k-group 0; later groups add a constant step
#pragma unroll
    for (int i = 0; i < G::FM; ++i) a_frag[i] = mfma::frag_offset<true, G::AS>(wm * G::TM + i * 32 + l32, 0, half);
#pragma unroll
    for (int j = 0; j < G::FN; ++j) b_frag[j] = mfma::frag_offset<false, G::BS>(wn * G::TN + j * 32 + l32, 0, half);
    const int phases = (K + G::BK - 1) / G::BK;
    load_phase(0);
    store_phase(0, 0);
    __syncthreads();
    for (int p = 0; p < phases; ++p) {
        const bool more = p + 1 < phases;
        if (more) load_phase((p + 1) * G::BK);
        const float *as = lds + (p & 1) * G::STAGE;
        mfma::mfma_phase<G::FM, G::FN, G::BK, true, G::AS, false, G::BS>(acc, as, as + G::A_STAGE, a_frag,
                                                                         b_frag);
        if (more) store_phase((p + 1) & 1, (p + 1) * G::BK);
        __syncthreads();
    }

    mfma::store_c<G::FM, G::FN>(acc, C, ldc, M, N, m0 + wm * G::TM, n0 + wn * G::TN, half, l32);
}

template <class G>
hipError_t launch_flat(const GemmArgs &g, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((g.M + G::BM - 1) / G::BM) * ((g.N + G::BN - 1) / G::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    int M = g.M, N = g.N, K = g.K;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sgemm_flat_kernel<G>),
                           dim3((unsigned)tiles), dim3(G::NT), args, 0, stream);
}

typedef FlatCfg<128, 128, 32, 2, 2, 4, 8, 2> Flat4;
typedef FlatCfg<128, 128, 32, 2, 2, 1, 8, 2> Flat1;

const MfmaVariant kFlatVariants[] = {
    {"m128n128k32_w2x2_vec4_flat", 128, 128, 32, 4, 2, INT64_MAX, INT64_MAX, 0, 0, false, 0.55, 0.75, 7000.0,
     &launch_flat<Flat4>},
    {"m128n128k32_w2x2_vec1_flat", 128, 128, 32, 1, 2, INT64_MAX, INT64_MAX, 0, 0, false, 0.45, 0.60, 7000.0,
     &launch_flat<Flat1>},
};

}  // namespace

int mfma_flat_variant_count() { return (int)(sizeof(kFlatVariants) / sizeof(kFlatVariants[0])); }

const MfmaVariant *mfma_flat_variant(int index)
{
    if (index < 0 || index >= mfma_flat_variant_count()) return nullptr;
    return &kFlatVariants[index];
}

}  // namespace tgemm
