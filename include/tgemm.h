/*
 * libtgemm — single-precision C = A·B on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the dense product of page 1 ("[Multi-Core & GPU
 * Programming] CUDA - Matrix Multiplication", section [Matrix
 * Multiplication]): every output is the sum over k of one row of the left
 * matrix times one column of the right one.  The pages call the matrices
 * M, N, P and the size Width; here they are A (M×K), B (K×N) and C (M×N),
 * and M, N, K are sizes.
 *
 * Conventions shared by every compute entry point below
 * ------------------------------------------------------
 * Layout      Row-major float32 with leading dimensions counted in elements:
 *             A(i,k) = A[i*lda + k], B(k,j) = B[k*ldb + j], C(i,j) = C[i*ldc + j]
 *             (page 1, section [Coalescing], indexes M as M[row*width + k]).
 *             Requires lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N).
 * Semantics   C(i,j) = sum_{k<K} A(i,k)·B(k,j).  C is overwritten, never read
 *             (page 1 keeps the sum in a register and writes the output once,
 *             at the end).  K = 0 sets C to +0.0; M = 0 or N = 0 is a no-op.
 * Memory      A, B and C are device pointers (hipMalloc, or a torch CUDA
 *             tensor's storage) owned by the caller.  The library allocates
 *             nothing and keeps no per-call state.  C must not overlap A or B.
 * Streams     Work is queued on `stream` (NULL = the default stream) and the
 *             call returns without waiting; results are ready once the
 *             stream has been synchronised (page 3, "CUDA.3 Writing CUDA SIMT
 *             Kernels", Global Memory: kernels hand results back only through
 *             device memory).
 * Errors      Argument problems are reported before anything is queued, and C
 *             is then left untouched.  TGEMM_ERROR_HIP means the launch itself
 *             failed.  A fault inside a kernel shows up at the caller's next
 *             stream synchronisation, as for any asynchronous HIP work.
 *             Nothing is printed and no C++ exception crosses this interface.
 * Sizes       M, N, K up to 2^31 - 2^16 (TGEMM_ERROR_NOT_SUPPORTED above);
 *             element offsets are 64-bit.
 * Threads     All entry points are re-entrant and may be called concurrently
 *             on different streams.
 * Rounding    The tiled MFMA kernels sum in an order of their own; for real
 *             inputs the result lies within 4·K·2^-24·sum_k|A(i,k)·B(k,j)| of
 *             the exact one, and integer-valued inputs whose partial sums stay
 *             below 2^24 in magnitude give the exact result.  The two
 *             one-product-per-step kernels (naive, LDS-tiled) add the products
 *             one fused multiply-add at a time in ascending k.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as the HIP runtime's, so either header may come first. */
typedef struct ihipStream_t *hipStream_t;

/* How an operand is stored (BLAS's "op"): as is, or transposed. */
typedef enum tgemm_op {
    TGEMM_OP_N = 0, /* op(X) = X */
    TGEMM_OP_T = 1  /* op(X) = Xᵀ */
} tgemm_op_t;

typedef enum tgemm_status {
    TGEMM_SUCCESS = 0,
    TGEMM_ERROR_INVALID_VALUE = 1, /* bad size, leading dimension, pointer or overlap, or an
                                      operand that would run past the end of the address space */
    TGEMM_ERROR_NOT_SUPPORTED = 2, /* a size above 2^31-2^16, or an unknown kernel choice */
    TGEMM_ERROR_HIP = 3            /* the HIP runtime refused the launch */
} tgemm_status_t;

/*
 * C = A·B with the tiled matrix-core kernel: the product of page 1 computed
 * tile by tile as in page 1's section [Shared Memory] and page 2 ("Lec 29 ·
 * GPU Architecture (2)") §1.2 — tiles of A and B staged through on-chip
 * memory in phases, one barrier per phase, sums kept in registers — with
 * the tile shape chosen from M, N, K and the alignment of A, B and C.
 * Arguments and errors: see the conventions above.
 */
tgemm_status_t tgemm_sgemm(int64_t M, int64_t N, int64_t K,
                           const float *A, int64_t lda,
                           const float *B, int64_t ldb,
                           float *C, int64_t ldc, hipStream_t stream);

/*
 * C = op(A)·op(B), op(A) M×K and op(B) K×N, with the tiled matrix-core kernel.
 * op_a = TGEMM_OP_T: A is stored K×M row-major (op(A) = Aᵀ), op(A)(i,k) =
 * A[k*lda + i], lda >= max(1,M); otherwise as tgemm_sgemm.  op_b = TGEMM_OP_T:
 * B is stored N×K, op(B)(k,j) = B[j*ldb + k], ldb >= max(1,K).  Each operand
 * is read along the dimension it is contiguous in and kept that way on chip,
 * the fragments taking whichever order the matrix cores need (page 1,
 * section [Coalescing], "Corner Turning").  Other values of op_a / op_b:
 * TGEMM_ERROR_NOT_SUPPORTED.  Transposed operands need leading dimensions
 * below 2^21 (the 64-bit-pointer configuration takes operands as stored
 * only): otherwise TGEMM_ERROR_NOT_SUPPORTED.  tgemm_sgemm(...) is
 * tgemm_sgemm_ex(TGEMM_OP_N, TGEMM_OP_N, ...).
 */
tgemm_status_t tgemm_sgemm_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda,
                              const float *B, int64_t ldb,
                              float *C, int64_t ldc, hipStream_t stream);

/*
 * C = A·B (row-major operands, as tgemm_sgemm; transposed ones through
 * tgemm_sgemm_splitk_ex below) with the k range split
 * across work-groups: the sum over k of page 1's section [Matrix
 * Multiplication] taken in up to `splits` contiguous slices that run side by
 * side, each slice's partial product written to its own M×N block of
 * `workspace`, and a second pass adding the blocks into C in slice order.
 * For shapes with too few output tiles to fill the GPU and a long K (e.g.
 * 512×512×16384).  Results do not depend on timing; the summation order
 * differs from tgemm_sgemm's, within the same error bound, and integer
 * inputs whose sums stay below 2^24 give the same exact results.
 *   splits: 1 ... 64; 1 runs tgemm_sgemm (workspace unused, may be NULL).
 *     The library may run fewer slices than asked (each slice is a whole
 *     number of its tile configuration's K steps), never more.
 *   workspace: device memory owned by the caller, 16-byte aligned, at least
 *     tgemm_sgemm_splitk_workspace_size(M, N, K, splits) bytes, overlapping
 *     none of A, B, C; its contents on return are unspecified.  The call
 *     allocates nothing.  Two calls in flight at once need two workspaces.
 * Errors as tgemm_sgemm; also TGEMM_ERROR_INVALID_VALUE for splits outside
 * 1 ... 64, a missing, misaligned, overlapping or too small workspace.
 */
tgemm_status_t tgemm_sgemm_splitk(int64_t M, int64_t N, int64_t K,
                                  const float *A, int64_t lda,
                                  const float *B, int64_t ldb,
                                  float *C, int64_t ldc, int splits,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tgemm_sgemm_splitk with operands stored transposed, as tgemm_sgemm_ex
 * (op_a / op_b = TGEMM_OP_T: A stored K×M, B stored N×K); the same
 * workspace.  tgemm_sgemm_splitk(...) is tgemm_sgemm_splitk_ex(TGEMM_OP_N,
 * TGEMM_OP_N, ...).
 */
tgemm_status_t tgemm_sgemm_splitk_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                     const float *A, int64_t lda,
                                     const float *B, int64_t ldb,
                                     float *C, int64_t ldc, int splits,
                                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch behind tgemm_sgemm_splitk_noalloc. */
#define TGEMM_SPLITK_NOALLOC_BYTES ((size_t)32 << 20)

/*
 * tgemm_sgemm_splitk_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same product with the same kernels and slices, so the same
 * results bit for bit, but the slices' partial products live in a fixed
 * scratch array of TGEMM_SPLITK_NOALLOC_BYTES (32 MiB) that the library holds
 * on each GPU it runs on until the process ends, not in a caller's
 * workspace.  The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls whose work overlaps in time on one GPU (two streams, two
 * threads) race and give wrong results, so serialise them.  Argument
 * meaning, layout, ownership and errors as tgemm_sgemm_splitk_ex, with
 * TGEMM_ERROR_NOT_SUPPORTED when tgemm_sgemm_splitk_workspace_size(M, N, K,
 * splits) exceeds TGEMM_SPLITK_NOALLOC_BYTES (e.g. 1024×1024 with more than 8
 * splits), and TGEMM_ERROR_HIP if the array's device address cannot be
 * obtained on the current device.
 */
tgemm_status_t tgemm_sgemm_splitk_noalloc(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                          const float *A, int64_t lda,
                                          const float *B, int64_t ldb,
                                          float *C, int64_t ldc, int splits, hipStream_t stream);

/* Workspace bytes tgemm_sgemm_splitk needs: splits·M·N·4; 0 when splits <= 1,
 * splits > 64, a size is not positive or above 2^31-2^16, or the product does
 * not fit in a size_t. */
size_t tgemm_sgemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits);

/* The split count (1, 2, 4, ..., 64) the library's cost model expects to be
 * fastest for M, N, K with 16-byte-aligned row-major operands; 1 means no
 * split (then tgemm_sgemm is the call to make).  Host-only: no GPU work. */
int tgemm_sgemm_splitk_choose(int64_t M, int64_t N, int64_t K);

/*
 * Same product with an explicitly chosen matrix-core tile configuration,
 * 0 <= variant < tgemm_mfma_variant_count().  Variants with 16-byte loads
 * ("vec4") need A and B 16-byte aligned, lda, ldb and the stored row lengths
 * of A and B (K and N here) multiples of 4; buffer-load variants need their
 * 32-bit offsets to span the leading dimensions; otherwise, and for an
 * unknown variant, TGEMM_ERROR_NOT_SUPPORTED.
 */
tgemm_status_t tgemm_sgemm_mfma(int64_t M, int64_t N, int64_t K,
                                const float *A, int64_t lda,
                                const float *B, int64_t ldb,
                                float *C, int64_t ldc, int variant, hipStream_t stream);

/* tgemm_sgemm_mfma with operand orders, as tgemm_sgemm_ex. */
tgemm_status_t tgemm_sgemm_mfma_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                   const float *A, int64_t lda,
                                   const float *B, int64_t ldb,
                                   float *C, int64_t ldc, int variant, hipStream_t stream);

/* Number of matrix-core tile configurations. */
int tgemm_mfma_variant_count(void);

/*
 * Static description of a variant, e.g. "m256n128k16_w2x2_vec4" (macro tile
 * 256×128, depth 16 per phase, 2×2 wavefronts, 16-byte loads),
 * "m32n32k32_w1x1s8_vec4" (32×32 tile staged through LDS, K split over 8
 * single-wavefront slices), "..._nn" (operands as stored only: TGEMM_OP_T is
 * refused; "m160n128k32_w1x4_vec4_nn" also writes C in 16-byte row pieces,
 * so tgemm_sgemm picks it only when C and ldc are 16-byte aligned, though it
 * runs on any C), "..._flat" (64-bit pointers, any leading dimension,
 * operands as stored only); NULL for an index out of range.
 */
const char *tgemm_mfma_variant_name(int variant);

/* The variant tgemm_sgemm would run for these arguments; -1 if none applies. */
int tgemm_sgemm_variant_for(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            const float *C, int64_t ldc);

/* The variant tgemm_sgemm_ex would run for these arguments; -1 if none applies. */
int tgemm_sgemm_variant_for_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                               const float *A, int64_t lda,
                               const float *B, int64_t ldb,
                               const float *C, int64_t ldc);

/*
 * Ablation 1 — one thread per output (page 1, section [Matrix
 * Multiplication], the simplest kernel and "Work Flow"; page 2 §1.2, naive
 * kernel): a 16×16 thread block per 16×16 output tile; each thread reads its
 * row of A and column of B straight from device memory and adds one fused
 * multiply-add per k in ascending order.  Arguments and errors as above.
 */
tgemm_status_t tgemm_sgemm_naive(int64_t M, int64_t N, int64_t K,
                                 const float *A, int64_t lda,
                                 const float *B, int64_t ldb,
                                 float *C, int64_t ldc, hipStream_t stream);

/*
 * Ablation 2 — the shared-memory tiled kernel (page 1, section [Shared
 * Memory], "Work Flow - Compute Block(0, 0)" and "Tiled Matrix
 * Multiplication Kernel"; page 2 §1.2): tile×tile threads per block, two
 * tile×tile on-chip tiles; per phase every thread copies one element of A
 * and one of B, the block synchronises, every thread adds the tile's
 * products to its register sum (one fused multiply-add per k, ascending),
 * and the block synchronises again.  Out-of-range elements load as zero.
 * tile is 2, 8, 16 or 32.  pad = 1 adds one word to each tile row
 * (page 2 §1.4, tile[32][33]); pad = 0 does not.  Other values:
 * TGEMM_ERROR_NOT_SUPPORTED.  Arguments and errors otherwise as above.
 */
tgemm_status_t tgemm_sgemm_lds(int64_t M, int64_t N, int64_t K,
                               const float *A, int64_t lda,
                               const float *B, int64_t ldb,
                               float *C, int64_t ldc, int tile, int pad, hipStream_t stream);

/*
 * Ablation 3 — the tiled kernel with more work per thread (page 1, end of
 * section [Shared Memory], "Tile Size 결정": let each thread compute several
 * outputs to use more on-chip memory), on the vector ALUs: 256 threads per
 * 128×128 tile, an 8×8 block of outputs per thread in registers, phases of 8
 * values of k staged through LDS (A transposed on the way in, page 1 section
 * [Coalescing], "Corner Turning"), two LDS stages, one barrier per phase.
 * Every output is one fused multiply-add chain in ascending k, so the result
 * equals tgemm_sgemm_naive's bit for bit.  Arguments and errors as above.
 */
tgemm_status_t tgemm_sgemm_simt(int64_t M, int64_t N, int64_t K,
                                const float *A, int64_t lda,
                                const float *B, int64_t ldb,
                                float *C, int64_t ldc, hipStream_t stream);

/* Kernels of tgemm_transpose. */
typedef enum tgemm_transpose_kernel {
    TGEMM_TRANSPOSE_BLOCKED = 0,     /* default: 4×4 blocks per thread, whole cache lines both ways */
    TGEMM_TRANSPOSE_NAIVE = 1,       /* page 2 §1.4: rows in, strided stores out */
    TGEMM_TRANSPOSE_TILED = 2,       /* page 2 §1.4: through a 32×32 LDS tile */
    TGEMM_TRANSPOSE_TILED_PADDED = 3 /* page 2 §1.4: LDS tile with rows of 33 words */
} tgemm_transpose_kernel_t;

/*
 * B = Aᵀ: the matrix transpose of page 2 ("Lec 29 · GPU Architecture (2)"),
 * §1.4.  A is M×N row-major with leading dimension lda >= max(1, N); B is
 * N×M row-major with ldb >= max(1, M); B(j, i) = A(i, j) for i < M, j < N,
 * every element moved as a 32-bit word (bit patterns, NaN payloads and
 * signed zeros arrive unchanged); nothing else of B is written.  Device
 * pointers owned by the caller; B must not overlap A (no in-place
 * transpose).  Asynchronous on `stream`.  M = 0 or N = 0 is a no-op.
 *
 * kernel selects the page's progression on this GPU — NAIVE (32×32 tiles,
 * 32×8 threads, four elements per thread; reads along A's rows, stores down
 * B's columns), TILED (the same tile staged through LDS, barrier, swapped
 * block offsets, stores along B's rows), TILED_PADDED (LDS rows padded to 33
 * words) — or BLOCKED, this library's kernel: no LDS; each thread moves
 * 4×4 blocks, each with four 16-byte reads and four 16-byte writes, so a
 * wavefront's every access is whole 128-byte runs (when A and B are 16-byte
 * aligned and lda, ldb are multiples of 4; otherwise single-word accesses
 * with the same mapping); from 2^24 elements on, four blocks side by side
 * per thread.
 *
 * Errors: TGEMM_ERROR_INVALID_VALUE for negative sizes, short leading
 * dimensions, null or misaligned pointers, or overlap;
 * TGEMM_ERROR_NOT_SUPPORTED for an unknown kernel or a size above
 * 2^31 - 2^16; TGEMM_ERROR_HIP if the launch fails.  Nothing is queued on
 * an error.
 */
tgemm_status_t tgemm_transpose(int64_t M, int64_t N, const float *A, int64_t lda,
                               float *B, int64_t ldb, tgemm_transpose_kernel_t kernel,
                               hipStream_t stream);

/*
 * C = A·B with A, B and C in HOST memory, the transfers overlapped with the
 * product (page 1, section [CUDA Performance Considerations], "Overlap I/O
 * with Computation": host↔device copies and computation at the same time,
 * on streams).  B is copied to the device once; A and C move in panels of
 * panel_rows rows (0: about M/4, rounded up to 256): while panel p is
 * multiplied on `compute` (an ordinary tgemm_sgemm call), panel p+1 of A is
 * copied in on `copy_in` and panel p-1 of C is copied out on `copy_out`.
 * Pass three different streams for the copies to overlap (one stream, or
 * NULL for all three, is correct but serial).  A, B, C should be page-locked
 * (hipHostMalloc, or a pinned torch CPU tensor) for the copies to run
 * asynchronously; pageable memory works but serialises them.
 *
 * Layout and semantics as tgemm_sgemm (row-major, leading dimensions in
 * elements, C overwritten; K = 0 sets C to +0.0 on the host without device
 * work; M = 0 or N = 0 is a no-op).  `workspace` is caller-owned DEVICE
 * memory, 256-byte aligned, of at least tgemm_sgemm_host_workspace_size(M,
 * N, K, panel_rows) bytes (B, two A panels and two C panels); the library
 * allocates nothing.  Unlike the device entry points this call BLOCKS: it
 * returns once C is complete in host memory (or after an error, once
 * everything it queued has finished).
 *
 * Errors: TGEMM_ERROR_INVALID_VALUE for the device entry points' argument
 * errors (host C overlapping host A or B), a negative panel_rows, or a
 * missing, misaligned or too small workspace; TGEMM_ERROR_NOT_SUPPORTED for
 * sizes as above; TGEMM_ERROR_HIP if a copy, event or launch fails (C may
 * then be partly written).
 */
tgemm_status_t tgemm_sgemm_host(int64_t M, int64_t N, int64_t K,
                                const float *A, int64_t lda,
                                const float *B, int64_t ldb,
                                float *C, int64_t ldc,
                                void *workspace, int64_t workspace_bytes, int64_t panel_rows,
                                hipStream_t compute, hipStream_t copy_in, hipStream_t copy_out);

/* Device workspace bytes tgemm_sgemm_host needs; 0 if it needs none (M, N or
 * K zero); -1 for invalid sizes or a negative panel_rows. */
int64_t tgemm_sgemm_host_workspace_size(int64_t M, int64_t N, int64_t K, int64_t panel_rows);

/* Static, human-readable text for a status code. */
const char *tgemm_status_string(tgemm_status_t status);

/* Library version, major*10000 + minor*100 + patch. */
int tgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
