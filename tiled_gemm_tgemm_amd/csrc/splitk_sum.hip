// Second pass of the product with K split across work-groups.
//
// The product is the same (page 1, "[Multi-Core & GPU Programming] CUDA -
// Matrix Multiplication", section [Matrix Multiplication]): every output is a
// sum over k.  When a shape has too few output tiles to fill the chip, the
// tiled kernel runs S slices of the k range side by side, each writing its
// partial product to its own M×N block of a workspace.  This kernel adds the
// blocks into C:
//
//     C(i, j) = W_0(i, j) + W_1(i, j) + ... + W_{S-1}(i, j)
//
// in slice order, one float32 addition at a time, so the result does not
// depend on timing, and integer-valued inputs whose sums stay below 2^24 give
// exact results.  W_s is row-major with leading dimension N at W + s·M·N.
//
// Bound by device memory: (S + 1)·M·N·4 bytes, every byte moved once (with
// one slice's load in flight at a time per thread the pass was bound by
// memory latency instead: 5.0 µs for 16 slices of 256×256).  Each
// thread handles one 16-byte group of a row (4-byte elements where N, ldc or
// C's address rule 16-byte accesses out), consecutive threads along the row,
// so reads of every slice and the writes of C are coalesced.  C is written
// with non-temporal stores: nothing reads it again in this pass.
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct Elem;
template <>
struct Elem<4> {
    typedef f32x4 type;
};
template <>
struct Elem<1> {
    typedef float type;
};

template <int V>
__global__ __launch_bounds__(64) void splitk_sum_kernel(int M, int N, int S, const float *__restrict__ W,
                                                         float *__restrict__ C, int64_t ldc)
{
    typedef typename Elem<V>::type vec_t;
    const int64_t per_row = N / V;
    const int64_t total = (int64_t)M * per_row;
    const int64_t slice = (int64_t)M * N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = t / per_row, j = (t - i * per_row) * V;
        const float *w = W + i * N + j;
        vec_t acc = *reinterpret_cast<const vec_t *>(w);
        // eight slices' loads in flight at once; the additions stay in slice order
        int s = 1;
        for (; s + 8 <= S; s += 8) {
            vec_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const vec_t *>(w + (s + u) * slice);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; s < S; ++s) acc += *reinterpret_cast<const vec_t *>(w + s * slice);
        __builtin_nontemporal_store(acc, reinterpret_cast<vec_t *>(C + i * ldc + j));
    }
}

}  // namespace

hipError_t launch_splitk_sum(int M, int N, int S, const float *W, float *C, int64_t ldc, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    if (S < 1 || ldc < N || W == nullptr || C == nullptr) return hipErrorInvalidValue;
    const bool v4 = N % 4 == 0 && ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(W) % 16 == 0;
    const int64_t total = (int64_t)M * (v4 ? N / 4 : N);
    // one wavefront per work-group, so that even 256×256 spreads over every CU
    const int64_t blocks = (total + 63) / 64;
    const unsigned grid = (unsigned)(blocks < 16384 ? blocks : 16384);
    void *args[] = {&M, &N, &S, &W, &C, &ldc};
    return hipLaunchKernel(v4 ? reinterpret_cast<const void *>(&splitk_sum_kernel<4>)
                              : reinterpret_cast<const void *>(&splitk_sum_kernel<1>),
                           dim3(grid), dim3(64), args, 0, stream);
}

}  // namespace tgemm
