// C = A·B for operands in host memory, with the transfers overlapped with
// the product (page 1, "[Multi-Core & GPU Programming] CUDA - Matrix
// Multiplication", section [CUDA Performance Considerations], "Overlap I/O
// with Computation": run host↔device transfers and computation at the same
// time, on separate streams).
//
// B goes to the device once.  A and C are cut into panels of whole rows;
// panel p's rows of A are copied in on `copy_in` while panel p-1 is
// multiplied on `compute` and panel p-2's rows of C are copied out on
// `copy_out`.  Two device buffers per panel operand (double buffering) and
// events order the three streams:
//
//   copy_in :  B | A0 | A1 | (wait C0 computed) A2 | (wait C1 computed) A3 ...
//   compute :  (wait B, A0) C0 | (wait A1) C1 | (wait A2, C0 copied out) C2 ...
//   copy_out:  (wait C0 computed) C0 | (wait C1 computed) C1 | ...
//
// Each panel is an ordinary tgemm_sgemm call on device buffers, so the
// panel products are computed exactly as the device entry point computes
// them.  The call returns when C is complete in host memory.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "tgemm.h"

namespace {

constexpr int64_t kMaxDim = ((int64_t)1 << 31) - ((int64_t)1 << 16);  // as tgemm_sgemm
constexpr int64_t kAlign = 256;

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t default_panel_rows(int64_t M)
{
    // about four panels, whole 256-row tiles of the product kernel
    const int64_t r = round_up((M + 3) / 4, 256);
    return r < M ? r : M;
}

int64_t panel_rows_for(int64_t M, int64_t panel_rows) { return panel_rows > 0 ? panel_rows : default_panel_rows(M); }

// Layout of the workspace: B (K×N), then A panels 0 and 1 (R×K), then C
// panels 0 and 1 (R×N), each rounded up to 256 bytes.
struct Layout {
    int64_t b, a, c, total;
};

Layout layout(int64_t M, int64_t N, int64_t K, int64_t panel_rows)
{
    const int64_t R = panel_rows_for(M, panel_rows);
    Layout l;
    l.b = round_up(K * N * 4, kAlign);
    l.a = round_up(R * K * 4, kAlign);
    l.c = round_up(R * N * 4, kAlign);
    l.total = l.b + 2 * l.a + 2 * l.c;
    return l;
}

// End (one past the last byte) of a rows×cols host operand with leading
// dimension ld, in 128 bits: rows up to 2^31 times ld up to 2^40 overflows 64.
unsigned __int128 end_of(const void *p, int64_t rows, int64_t cols, int64_t ld)
{
    return (unsigned __int128)reinterpret_cast<uintptr_t>(p) +
           ((unsigned __int128)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * sizeof(float);
}

// Whether the operand runs past the end of the address space (no such operand exists).
bool beyond(const void *p, int64_t rows, int64_t cols, int64_t ld)
{
    return end_of(p, rows, cols, ld) > (unsigned __int128)UINTPTR_MAX;
}

bool overlaps(const void *p, int64_t rows, int64_t cols, int64_t ld, const void *q, int64_t qrows, int64_t qcols,
              int64_t qld)
{
    const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(p), a1 = end_of(p, rows, cols, ld);
    const unsigned __int128 b0 = reinterpret_cast<uintptr_t>(q), b1 = end_of(q, qrows, qcols, qld);
    return a0 < b1 && b0 < a1;
}

bool misaligned(const void *p) { return reinterpret_cast<uintptr_t>(p) % alignof(float) != 0; }

}  // namespace

extern "C" {

int64_t tgemm_sgemm_host_workspace_size(int64_t M, int64_t N, int64_t K, int64_t panel_rows)
{
    if (M < 0 || N < 0 || K < 0 || panel_rows < 0) return -1;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
    if (M == 0 || N == 0 || K == 0) return 0;
    return layout(M, N, K, panel_rows).total;
}

tgemm_status_t tgemm_sgemm_host(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                                int64_t ldb, float *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                                int64_t panel_rows, hipStream_t compute, hipStream_t copy_in, hipStream_t copy_out)
{
    if (M < 0 || N < 0 || K < 0 || panel_rows < 0) return TGEMM_ERROR_INVALID_VALUE;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return TGEMM_ERROR_INVALID_VALUE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return TGEMM_ERROR_NOT_SUPPORTED;
    if (lda > (int64_t)1 << 40 || ldb > (int64_t)1 << 40 || ldc > (int64_t)1 << 40) return TGEMM_ERROR_NOT_SUPPORTED;
    if (M == 0 || N == 0) return TGEMM_SUCCESS;
    if (C == nullptr || misaligned(C) || beyond(C, M, N, ldc)) return TGEMM_ERROR_INVALID_VALUE;
    if (K == 0) {  // the empty sum, written on the host: no device work at all
        for (int64_t i = 0; i < M; ++i) memset(C + i * ldc, 0, (size_t)N * sizeof(float));
        return TGEMM_SUCCESS;
    }
    if (A == nullptr || B == nullptr || misaligned(A) || misaligned(B)) return TGEMM_ERROR_INVALID_VALUE;
    if (beyond(A, M, K, lda) || beyond(B, K, N, ldb)) return TGEMM_ERROR_INVALID_VALUE;
    if (overlaps(C, M, N, ldc, A, M, K, lda) || overlaps(C, M, N, ldc, B, K, N, ldb))
        return TGEMM_ERROR_INVALID_VALUE;
    const Layout l = layout(M, N, K, panel_rows);
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % kAlign || workspace_bytes < l.total)
        return TGEMM_ERROR_INVALID_VALUE;

    const int64_t R = panel_rows_for(M, panel_rows);
    const int64_t panels = (M + R - 1) / R;
    char *ws = static_cast<char *>(workspace);
    float *Bd = reinterpret_cast<float *>(ws);
    float *Ad[2] = {reinterpret_cast<float *>(ws + l.b), reinterpret_cast<float *>(ws + l.b + l.a)};
    float *Cd[2] = {reinterpret_cast<float *>(ws + l.b + 2 * l.a), reinterpret_cast<float *>(ws + l.b + 2 * l.a + l.c)};

    hipEvent_t b_in, a_in[2], c_made[2], c_out[2];
    hipEvent_t *all[] = {&b_in, &a_in[0], &a_in[1], &c_made[0], &c_made[1], &c_out[0], &c_out[1]};
    int created = 0;
    hipError_t err = hipSuccess;
    for (hipEvent_t *e : all) {
        err = hipEventCreateWithFlags(e, hipEventDisableTiming);
        if (err != hipSuccess) break;
        ++created;
    }
    tgemm_status_t st = TGEMM_SUCCESS;
#define TGEMM_STEP(call)                    \
    do {                                    \
        if (err == hipSuccess) err = (call); \
    } while (0)
    if (err == hipSuccess) {
        TGEMM_STEP(hipMemcpy2DAsync(Bd, (size_t)N * 4, B, (size_t)ldb * 4, (size_t)N * 4, (size_t)K,
                                    hipMemcpyHostToDevice, copy_in));
        TGEMM_STEP(hipEventRecord(b_in, copy_in));
        TGEMM_STEP(hipStreamWaitEvent(compute, b_in, 0));
        for (int64_t p = 0; p < panels && err == hipSuccess && st == TGEMM_SUCCESS; ++p) {
            const int b = (int)(p & 1);
            const int64_t r0 = p * R, h = (M - r0 < R) ? M - r0 : R;
            if (p >= 2) TGEMM_STEP(hipStreamWaitEvent(copy_in, c_made[b], 0));  // A buffer b is free
            TGEMM_STEP(hipMemcpy2DAsync(Ad[b], (size_t)K * 4, A + r0 * lda, (size_t)lda * 4, (size_t)K * 4,
                                        (size_t)h, hipMemcpyHostToDevice, copy_in));
            TGEMM_STEP(hipEventRecord(a_in[b], copy_in));
            TGEMM_STEP(hipStreamWaitEvent(compute, a_in[b], 0));
            if (p >= 2) TGEMM_STEP(hipStreamWaitEvent(compute, c_out[b], 0));  // C buffer b is free
            if (err == hipSuccess) st = tgemm_sgemm(h, N, K, Ad[b], K, Bd, N, Cd[b], N, compute);
            TGEMM_STEP(hipEventRecord(c_made[b], compute));
            TGEMM_STEP(hipStreamWaitEvent(copy_out, c_made[b], 0));
            TGEMM_STEP(hipMemcpy2DAsync(C + r0 * ldc, (size_t)ldc * 4, Cd[b], (size_t)N * 4, (size_t)N * 4,
                                        (size_t)h, hipMemcpyDeviceToHost, copy_out));
            TGEMM_STEP(hipEventRecord(c_out[b], copy_out));
        }
    }
#undef TGEMM_STEP
    // Whatever happened, nothing queued here may still run when the call
    // returns: the workspace and the events belong to the caller / this call.
    const hipError_t s1 = hipStreamSynchronize(copy_in);
    const hipError_t s2 = hipStreamSynchronize(compute);
    const hipError_t s3 = hipStreamSynchronize(copy_out);
    for (int i = 0; i < created; ++i) (void)hipEventDestroy(*all[i]);
    if (st != TGEMM_SUCCESS) return st;
    if (err != hipSuccess || s1 != hipSuccess || s2 != hipSuccess || s3 != hipSuccess) return TGEMM_ERROR_HIP;
    return TGEMM_SUCCESS;
}

}  // extern "C"
