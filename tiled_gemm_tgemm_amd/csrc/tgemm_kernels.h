// Internal interface between the host entry points (api.cpp) and the kernel
// translation units.  Every launcher takes already-validated arguments:
// M, N, K >= 1, all sizes below 2^31, leading dimensions large enough, and
// non-overlapping device buffers.  Each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

// op(A) is M×K and op(B) is K×N.  trans_a: A is stored K×M (op(A) = Aᵀ),
// element (i, k) at A[k*lda + i]; otherwise at A[i*lda + k].  trans_b: B is
// stored N×K, element (k, j) at B[j*ldb + k]; otherwise at B[k*ldb + j].
struct GemmArgs {
    int M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    bool trans_a = false, trans_b = false;
    // K split across work-groups (tiled buffer-load kernels only): `splits`
    // slices of `kchunk` values of k (the last one shorter); slice s reads
    // its k range of A and B and writes its partial product to C + s·c_slice.
    int splits = 1;
    int kchunk = 0;
    int64_t c_slice = 0;
};

// One thread per output, 16×16 blocks.
hipError_t launch_naive(const GemmArgs &g, hipStream_t stream);

// The two-barrier shared-memory tiled kernel; tile in {2, 8, 16, 32}, pad in {0, 1}.
hipError_t launch_lds_tiled(const GemmArgs &g, int tile, int pad, hipStream_t stream);

// 128×128 tiles, 8×8 outputs per thread on the vector ALUs.
hipError_t launch_simt_tiled(const GemmArgs &g, hipStream_t stream);

// C(i,j) = +0 for i < M, j < N (the empty sum, K = 0).
hipError_t launch_fill_zero(int M, int N, float *C, int64_t ldc, hipStream_t stream);

// C = W_0 + W_1 + ... + W_{S-1}, added in slice order (splitk_sum.hip); W_s
// is M×N with leading dimension N at W + s·M·N.
hipError_t launch_splitk_sum(int M, int N, int S, const float *W, float *C, int64_t ldc, hipStream_t stream);

// B (N×M) = Aᵀ for A (M×N): B[j*ldb + i] = A[i*lda + j].  vec4: A and B
// 16-byte aligned and lda, ldb multiples of 4 (16-byte accesses allowed).
struct TransposeArgs {
    int M, N;
    const float *A;
    int64_t lda;
    float *B;
    int64_t ldb;
    bool vec4;
};

enum class TransposeKind { kBlocked, kNaive, kTiled, kTiledPadded };

hipError_t launch_transpose(TransposeKind kind, const TransposeArgs &t, hipStream_t stream);

// Matrix-core tile configurations.
struct MfmaVariant {
    const char *name;
    int bm, bn, bk;      // macro tile; K granularity of a work-group (phase depth × K slices)
    int vec;             // 4: 16-byte loads (alignment required), 1: 4-byte loads
    int wg_per_cu;       // work-groups one compute unit holds at once
    int64_t max_lda;     // largest leading dimensions the configuration takes,
    int64_t max_ldb;     // operands as stored ...
    int64_t max_lda_t;   // ... and transposed
    int64_t max_ldb_t;
    bool trans;          // takes transposed operands
    // Measured fraction of the matrix-core rate a work-group sustains when it
    // is alone on its compute unit, and when wg_per_cu of them share it; plus
    // a fixed cost per round of work-groups (SIMD cycles).  Used only to rank
    // configurations for a shape.
    double eff_alone, eff_full, round_cycles;
    hipError_t (*launch)(const GemmArgs &g, hipStream_t stream);
    bool split_k = false;  // takes GemmArgs::splits > 1
    // measured rate with A stored transposed and B as stored, relative to
    // operands as stored (used only to rank configurations)
    double tn_factor = 1.0;
    // forms its blocks transposed and stores C four columns at a time: chosen
    // by the cost model only when C and its leading dimension are 16-byte
    // aligned (it runs on any C, one store per element otherwise)
    bool c16 = false;
};

// Tiled buffer-load kernels (mfma_sgemm.hip) and the 64-bit-pointer fallback
// (mfma_sgemm_flat.hip).
int mfma_buffer_variant_count();
const MfmaVariant *mfma_buffer_variant(int index);
int mfma_flat_variant_count();
const MfmaVariant *mfma_flat_variant(int index);

// All configurations, in that order.
inline int mfma_variant_count() { return mfma_buffer_variant_count() + mfma_flat_variant_count(); }
inline const MfmaVariant *mfma_variant(int index)
{
    if (index < 0) return nullptr;
    if (index < mfma_buffer_variant_count()) return mfma_buffer_variant(index);
    return mfma_flat_variant(index - mfma_buffer_variant_count());
}

}  // namespace tgemm
