// C entry points of libtgemm: argument checks, quick returns, choice of the
// matrix-core tile configuration, and one launch on the caller's stream.
// The declarations, with the meaning of every argument, are in tgemm.h.
#include "tgemm.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "tgemm_kernels.h"

namespace {

using tgemm::GemmArgs;

// Largest M, N or K: 2^31 - 2^16, so that every kernel's tile and phase
// counts, and the k index of a phase rounded up to its depth, stay within
// 32-bit integers.
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - ((int64_t)1 << 16);

int64_t max1(int64_t v) { return v > 1 ? v : 1; }

// Byte range [lo, hi) spanned by a rows×cols row-major operand with leading
// dimension ld (rows, cols >= 1).  False if the range runs past the end of
// the address space (rows up to 2^31 times ld up to 2^40 can): no such
// operand exists, so the caller reports an invalid argument.
bool span(const void *p, int64_t rows, int64_t cols, int64_t ld, uintptr_t &lo, uintptr_t &hi)
{
    lo = reinterpret_cast<uintptr_t>(p);
    const unsigned __int128 end =
        (unsigned __int128)lo + ((unsigned __int128)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * sizeof(float);
    if (end > (unsigned __int128)UINTPTR_MAX) return false;
    hi = (uintptr_t)end;
    return true;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

enum class Quick { kNone, kDone, kZeroFill };

// Shared checks of every compute entry point.  On success `quick` says
// whether the call is already complete (M or N zero) or only needs C zeroed
// (K zero).  ta / tb: A stored K×M, B stored N×K.
tgemm_status_t validate(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                        const float *B, int64_t ldb, const float *C, int64_t ldc, Quick &quick)
{
    quick = Quick::kNone;
    if (M < 0 || N < 0 || K < 0) return TGEMM_ERROR_INVALID_VALUE;
    if (lda < max1(ta ? M : K) || ldb < max1(tb ? K : N) || ldc < max1(N)) return TGEMM_ERROR_INVALID_VALUE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return TGEMM_ERROR_NOT_SUPPORTED;
    if (lda > (int64_t)1 << 40 || ldb > (int64_t)1 << 40 || ldc > (int64_t)1 << 40)
        return TGEMM_ERROR_NOT_SUPPORTED;
    if (M == 0 || N == 0) {
        quick = Quick::kDone;
        return TGEMM_SUCCESS;
    }
    if (C == nullptr || reinterpret_cast<uintptr_t>(C) % alignof(float)) return TGEMM_ERROR_INVALID_VALUE;
    uintptr_t a0, a1, b0, b1, c0, c1;
    if (!span(C, M, N, ldc, c0, c1)) return TGEMM_ERROR_INVALID_VALUE;
    if (K == 0) {
        quick = Quick::kZeroFill;
        return TGEMM_SUCCESS;
    }
    if (A == nullptr || B == nullptr) return TGEMM_ERROR_INVALID_VALUE;
    if (reinterpret_cast<uintptr_t>(A) % alignof(float) || reinterpret_cast<uintptr_t>(B) % alignof(float))
        return TGEMM_ERROR_INVALID_VALUE;
    if (!span(A, ta ? K : M, ta ? M : K, lda, a0, a1) || !span(B, tb ? N : K, tb ? K : N, ldb, b0, b1))
        return TGEMM_ERROR_INVALID_VALUE;
    if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return TGEMM_ERROR_INVALID_VALUE;
    return TGEMM_SUCCESS;
}

GemmArgs pack(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
              const float *B, int64_t ldb, float *C, int64_t ldc)
{
    return GemmArgs{(int)M, (int)N, (int)K, A, lda, B, ldb, C, ldc, ta, tb};
}

tgemm_status_t from_hip(hipError_t e) { return e == hipSuccess ? TGEMM_SUCCESS : TGEMM_ERROR_HIP; }

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// 16-byte loads need every stored row of A and B to start 16-byte aligned and
// to hold whole float4s: the stored row lengths (K or M for A, N or K for B)
// and the leading dimensions must be multiples of 4.
bool vec4_ok(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
             const float *B, int64_t ldb)
{
    return aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0 && (ta ? M : K) % 4 == 0 &&
           (tb ? K : N) % 4 == 0;
}

// Whether a configuration can run these operands: 16-byte loads need
// vec4_ok, buffer-load configurations bound the leading dimensions, and the
// 64-bit-pointer fallback takes operands as stored only.
bool runs(const tgemm::MfmaVariant &v, bool vec4, bool ta, bool tb, int64_t lda, int64_t ldb)
{
    // a configuration whose work-group does not fit on a compute unit cannot
    // run (and the cost model divides by work-groups per CU)
    if (v.wg_per_cu < 1) return false;
    if ((ta || tb) && !v.trans) return false;
    return (v.vec == 1 || vec4) && lda <= (ta ? v.max_lda_t : v.max_lda) &&
           ldb <= (tb ? v.max_ldb_t : v.max_ldb);
}

// Estimated time of a configuration in SIMD cycles.  Tiles are dealt to the
// 256 compute units in rounds of up to wg_per_cu per CU (the persistent grid
// runs them as each resident work-group's successive tiles); the
// wavefronts of a work-group spread over the CU's 4 SIMDs, each retiring 64
// flops a cycle at the efficiency measured for that many resident
// work-groups (interpolated between alone and full).  The last round may
// leave CUs less full, and is costed at its own residency.  Edge tiles cost
// as much as full ones, which is what makes smaller tiles win on small or
// ragged shapes.
// `order`: the configuration's relative rate for this operand order (its
// tn_factor for Aᵀ·B, else 1).
double cost_tiles(const tgemm::MfmaVariant &v, int64_t tiles, int64_t K, double order = 1.0)
{
    const int64_t cus = 256;
    const int64_t full_rounds = tiles / (cus * v.wg_per_cu);
    const int64_t rest = tiles % (cus * v.wg_per_cu);
    const double kpad = (double)((K + v.bk - 1) / v.bk) * v.bk;
    const double per_wg = 2.0 * v.bm * v.bn * kpad / 4.0 / 64.0;
    auto eff = [&](int64_t r) {
        if (v.wg_per_cu <= 1) return v.eff_full * order;
        return (v.eff_alone + (v.eff_full - v.eff_alone) * (double)(r - 1) / (double)(v.wg_per_cu - 1)) * order;
    };
    double t = (double)full_rounds * ((double)v.wg_per_cu * per_wg / eff(v.wg_per_cu) + v.round_cycles);
    if (rest > 0) {
        const int64_t r = (rest + cus - 1) / cus;
        t += (double)r * per_wg / eff(r) + v.round_cycles;
    }
    return t;
}

// The tiles of the last round finish together and are written out with no
// computation left to cover the stores: the bytes of C they hold, at about
// 5 TB/s (measured on MI355X: 4096×4096×K takes 0.220 µs per unit of K plus
// 14 µs, the 64 MB of C; 16 values of k take 17.9 µs in all).  Earlier
// rounds' stores overlap the next round's work in part, which the fixed cost
// per round stands for.  This is what lets a tile that spreads a ragged shape
// over more, shorter rounds win (3000×1000×5000: 760 tiles of 160×128, the
// second and last round 248 of them, 219-222 µs; 480 tiles of 256×128, all in
// one round, 234 µs).
double final_store_cycles(const tgemm::MfmaVariant &v, int64_t tiles, int64_t M, int64_t N)
{
    const int64_t slots = (int64_t)256 * v.wg_per_cu;
    const int64_t last = tiles % slots != 0 ? tiles % slots : (tiles < slots ? tiles : slots);
    const double tile_bytes = (double)last * v.bm * v.bn * 4.0;
    const double c_bytes = (double)M * N * 4.0;
    return (tile_bytes < c_bytes ? tile_bytes : c_bytes) / 5.0e12 * 2.4e9;
}

double cost(const tgemm::MfmaVariant &v, bool ta, bool tb, int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
    return cost_tiles(v, tiles, K, (ta && !tb) ? v.tn_factor : 1.0) + final_store_cycles(v, tiles, M, N);
}

// K split across work-groups.  Slices are a whole number of a configuration's
// K granularity (phase depth × K slices inside the work-group) long, so only
// the last slice has a partial phase, and a multiple of 4, so 16-byte loads
// stay aligned; `splits` is an upper bound on the slices actually run.
struct Split {
    int variant = -1;
    int slices = 1;
    int kchunk = 0;
    double cycles = 0;
};

int64_t kchunk_for(const tgemm::MfmaVariant &v, int64_t K, int splits)
{
    const int64_t per = (K + splits - 1) / splits;
    return (per + v.bk - 1) / v.bk * v.bk;
}

// The second pass reads S slices of M×N floats and writes C once; costed at
// 5 TB/s (a plain streaming copy on MI355X reaches 5.4-5.6) plus a launch.
double sum_cycles(int64_t M, int64_t N, int slices)
{
    return (double)(slices + 1) * M * N * 4.0 / 5.0e12 * 2.4e9 + 7000.0;
}

// Best configuration for exactly up to `splits` slices (splits >= 2).
Split choose_split(bool ta, bool tb, int64_t M, int64_t N, int64_t K, bool vec4, int64_t lda, int64_t ldb,
                   int splits, bool c16)
{
    Split best;
    for (int i = 0; i < tgemm::mfma_variant_count(); ++i) {
        const tgemm::MfmaVariant *v = tgemm::mfma_variant(i);
        if (!v->split_k || !runs(*v, vec4, ta, tb, lda, ldb) || (v->c16 && !c16)) continue;
        const int64_t kc = kchunk_for(*v, K, splits);
        const int64_t slices = (K + kc - 1) / kc;
        const int64_t tiles = ((M + v->bm - 1) / v->bm) * ((N + v->bn - 1) / v->bn);
        const double c = cost_tiles(*v, tiles * slices, kc, (ta && !tb) ? v->tn_factor : 1.0) +
                         (slices > 1 ? sum_cycles(M, N, (int)slices) : 0.0);
        if (best.variant < 0 || c < best.cycles) {
            best.variant = i;
            best.slices = (int)slices;
            best.kchunk = (int)kc;
            best.cycles = c;
        }
    }
    return best;
}

constexpr int kMaxSplits = 64;
constexpr int64_t kMinSliceK = 1024;

int choose_variant(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                   const float *B, int64_t ldb, const float *C, int64_t ldc)
{
    const bool c16 = aligned16(C) && ldc % 4 == 0;
    const bool vec4 = vec4_ok(ta, tb, M, N, K, A, lda, B, ldb);
    int best = -1;
    double best_cost = 0;
    for (int i = 0; i < tgemm::mfma_variant_count(); ++i) {
        const tgemm::MfmaVariant *v = tgemm::mfma_variant(i);
        if (!runs(*v, vec4, ta, tb, lda, ldb) || (v->c16 && !c16)) continue;
        const double c = cost(*v, ta, tb, M, N, K);
        if (best < 0 || c < best_cost) {
            best = i;
            best_cost = c;
        }
    }
    return best;
}

// The split-K product once arguments are valid and splits > 1: checks the
// workspace (`splits` blocks of M×N floats, 16-byte aligned, apart from A, B
// and C), then the sliced product into it and the in-order sum into C.
tgemm_status_t splitk_launch(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                             const float *B, int64_t ldb, float *C, int64_t ldc, int splits, void *workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    const tgemm_op_t op_a = ta ? TGEMM_OP_T : TGEMM_OP_N, op_b = tb ? TGEMM_OP_T : TGEMM_OP_N;
    const size_t need = tgemm_sgemm_splitk_workspace_size(M, N, K, splits);
    if (need == 0 || workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 || workspace_bytes < need)
        return TGEMM_ERROR_INVALID_VALUE;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace);
    if (workspace_bytes > UINTPTR_MAX - w0) return TGEMM_ERROR_INVALID_VALUE;
    const uintptr_t w1 = w0 + workspace_bytes;
    uintptr_t x0, x1;
    if (span(A, ta ? K : M, ta ? M : K, lda, x0, x1) && overlaps(w0, w1, x0, x1)) return TGEMM_ERROR_INVALID_VALUE;
    if (span(B, tb ? N : K, tb ? K : N, ldb, x0, x1) && overlaps(w0, w1, x0, x1)) return TGEMM_ERROR_INVALID_VALUE;
    if (span(C, M, N, ldc, x0, x1) && overlaps(w0, w1, x0, x1)) return TGEMM_ERROR_INVALID_VALUE;
    const bool vec4 = vec4_ok(ta, tb, M, N, K, A, lda, B, ldb);
    // the slices go to the workspace (16-byte aligned, rows of N floats)
    const Split sp = choose_split(ta, tb, M, N, K, vec4, lda, ldb, splits, N % 4 == 0);
    if (sp.variant < 0) return TGEMM_ERROR_NOT_SUPPORTED;
    if (sp.slices <= 1) return tgemm_sgemm_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream);
    float *W = static_cast<float *>(workspace);
    GemmArgs g = pack(ta, tb, M, N, K, A, lda, B, ldb, W, N);
    g.splits = sp.slices;
    g.kchunk = sp.kchunk;
    g.c_slice = M * N;
    const tgemm::MfmaVariant *v = tgemm::mfma_variant(sp.variant);
    const hipError_t e = v->launch(g, stream);
    if (e != hipSuccess) return TGEMM_ERROR_HIP;
    return from_hip(tgemm::launch_splitk_sum((int)M, (int)N, sp.slices, W, C, ldc, stream));
}

// The fixed device scratch of tgemm_sgemm_splitk_noalloc: room for the
// slices' partial products of callers that cannot allocate.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not a device address: kernels and
// copies are given the address scratch_on_device() looked up instead.
static __device__ __align__(256) float scratch[TGEMM_SPLITK_NOALLOC_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void *scratch_on_device()
{
    static std::atomic<void *> address[kMaxDevices];
    static std::mutex lookup;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = address[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> hold(lookup);
    p = address[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        address[dev].store(p, std::memory_order_release);
    }
    return p;
}

bool op_ok(tgemm_op_t op) { return op == TGEMM_OP_N || op == TGEMM_OP_T; }

}  // namespace

extern "C" {

tgemm_status_t tgemm_sgemm_mfma_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                   const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                                   int64_t ldc, int variant, hipStream_t stream)
{
    const tgemm::MfmaVariant *v = tgemm::mfma_variant(variant);
    if (v == nullptr || !op_ok(op_a) || !op_ok(op_b)) return TGEMM_ERROR_NOT_SUPPORTED;
    const bool ta = op_a == TGEMM_OP_T, tb = op_b == TGEMM_OP_T;
    Quick quick;
    const tgemm_status_t st = validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS || quick == Quick::kDone) return st;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if (!runs(*v, vec4_ok(ta, tb, M, N, K, A, lda, B, ldb), ta, tb, lda, ldb)) return TGEMM_ERROR_NOT_SUPPORTED;
    return from_hip(v->launch(pack(ta, tb, M, N, K, A, lda, B, ldb, C, ldc), stream));
}

tgemm_status_t tgemm_sgemm_mfma(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                                const float *B, int64_t ldb, float *C, int64_t ldc, int variant,
                                hipStream_t stream)
{
    return tgemm_sgemm_mfma_ex(TGEMM_OP_N, TGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, variant, stream);
}

tgemm_status_t tgemm_sgemm_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                              int64_t ldc, hipStream_t stream)
{
    if (!op_ok(op_a) || !op_ok(op_b)) return TGEMM_ERROR_NOT_SUPPORTED;
    const bool ta = op_a == TGEMM_OP_T, tb = op_b == TGEMM_OP_T;
    Quick quick;
    const tgemm_status_t st = validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS || quick == Quick::kDone) return st;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    const int variant = choose_variant(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
    if (variant < 0) return TGEMM_ERROR_NOT_SUPPORTED;
    return from_hip(tgemm::mfma_variant(variant)->launch(pack(ta, tb, M, N, K, A, lda, B, ldb, C, ldc), stream));
}

tgemm_status_t tgemm_sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                           const float *B, int64_t ldb, float *C, int64_t ldc, hipStream_t stream)
{
    return tgemm_sgemm_ex(TGEMM_OP_N, TGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

size_t tgemm_sgemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits)
{
    if (M <= 0 || N <= 0 || K <= 0 || splits <= 1 || splits > kMaxSplits) return 0;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    const unsigned __int128 bytes = (unsigned __int128)splits * (uint64_t)M * (uint64_t)N * sizeof(float);
    return bytes > (unsigned __int128)SIZE_MAX ? 0 : (size_t)bytes;  // 0: no such workspace can exist
}

int tgemm_sgemm_splitk_choose(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 1;
    // row-major operands with 16-byte loads, as tgemm_sgemm would run them
    double best = -1;
    for (int i = 0; i < tgemm::mfma_variant_count(); ++i) {
        const tgemm::MfmaVariant *v = tgemm::mfma_variant(i);
        if (!runs(*v, true, false, false, max1(K), max1(N))) continue;
        const double c = cost(*v, false, false, M, N, K);
        if (best < 0 || c < best) best = c;
    }
    // slices shorter than ~1024 values of k lose more to each work-group's
    // pipeline fill and drain than they gain (measured on MI355X: at
    // 384×640×4096, 23.7 µs with 4 slices against 30.4 with 16)
    int pick = 1;
    for (int splits = 2; splits <= kMaxSplits && (K + splits - 1) / splits >= kMinSliceK; splits *= 2) {
        const Split sp = choose_split(false, false, M, N, K, true, max1(K), max1(N), splits, true);
        if (sp.variant >= 0 && sp.slices > 1 && (best < 0 || sp.cycles < best)) {
            best = sp.cycles;
            pick = splits;
        }
    }
    return pick;
}

tgemm_status_t tgemm_sgemm_splitk_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                     const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                                     int64_t ldc, int splits, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream)
{
    if (!op_ok(op_a) || !op_ok(op_b)) return TGEMM_ERROR_NOT_SUPPORTED;
    const bool ta = op_a == TGEMM_OP_T, tb = op_b == TGEMM_OP_T;
    Quick quick;
    const tgemm_status_t st = validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS) return st;
    if (splits < 1 || splits > kMaxSplits) return TGEMM_ERROR_INVALID_VALUE;
    if (quick == Quick::kDone) return TGEMM_SUCCESS;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if (splits == 1) return tgemm_sgemm_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream);
    return splitk_launch(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_bytes, stream);
}

tgemm_status_t tgemm_sgemm_splitk(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                                  const float *B, int64_t ldb, float *C, int64_t ldc, int splits,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return tgemm_sgemm_splitk_ex(TGEMM_OP_N, TGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, splits, workspace,
                                 workspace_bytes, stream);
}

tgemm_status_t tgemm_sgemm_splitk_noalloc(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                                          const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                                          int64_t ldc, int splits, hipStream_t stream)
{
    if (!op_ok(op_a) || !op_ok(op_b)) return TGEMM_ERROR_NOT_SUPPORTED;
    const bool ta = op_a == TGEMM_OP_T, tb = op_b == TGEMM_OP_T;
    Quick quick;
    const tgemm_status_t st = validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS) return st;
    if (splits < 1 || splits > kMaxSplits) return TGEMM_ERROR_INVALID_VALUE;
    if (quick == Quick::kDone) return TGEMM_SUCCESS;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if (splits == 1) return tgemm_sgemm_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream);
    const size_t need = tgemm_sgemm_splitk_workspace_size(M, N, K, splits);
    if (need == 0 || need > TGEMM_SPLITK_NOALLOC_BYTES) return TGEMM_ERROR_NOT_SUPPORTED;
    void *ws = scratch_on_device();
    if (ws == nullptr) return TGEMM_ERROR_HIP;
    return splitk_launch(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, splits, ws, TGEMM_SPLITK_NOALLOC_BYTES, stream);
}

int tgemm_mfma_variant_count(void) { return tgemm::mfma_variant_count(); }

const char *tgemm_mfma_variant_name(int variant)
{
    const tgemm::MfmaVariant *v = tgemm::mfma_variant(variant);
    return v ? v->name : nullptr;
}

int tgemm_sgemm_variant_for_ex(tgemm_op_t op_a, tgemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                               const float *A, int64_t lda, const float *B, int64_t ldb, const float *C,
                               int64_t ldc)
{
    if (!op_ok(op_a) || !op_ok(op_b)) return -1;
    const bool ta = op_a == TGEMM_OP_T, tb = op_b == TGEMM_OP_T;
    Quick quick;
    if (validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, quick) != TGEMM_SUCCESS || quick != Quick::kNone)
        return -1;
    return choose_variant(ta, tb, M, N, K, A, lda, B, ldb, C, ldc);
}

int tgemm_sgemm_variant_for(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                            const float *B, int64_t ldb, const float *C, int64_t ldc)
{
    return tgemm_sgemm_variant_for_ex(TGEMM_OP_N, TGEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc);
}

tgemm_status_t tgemm_sgemm_naive(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                                 const float *B, int64_t ldb, float *C, int64_t ldc,
                                 hipStream_t stream)
{
    Quick quick;
    const tgemm_status_t st = validate(false, false, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS || quick == Quick::kDone) return st;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if ((M + 15) / 16 > 65535) return TGEMM_ERROR_NOT_SUPPORTED;  // grid rows limit
    return from_hip(tgemm::launch_naive(pack(false, false, M, N, K, A, lda, B, ldb, C, ldc), stream));
}

tgemm_status_t tgemm_sgemm_lds(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                               const float *B, int64_t ldb, float *C, int64_t ldc, int tile,
                               int pad, hipStream_t stream)
{
    if (!(tile == 2 || tile == 8 || tile == 16 || tile == 32) || !(pad == 0 || pad == 1))
        return TGEMM_ERROR_NOT_SUPPORTED;
    Quick quick;
    const tgemm_status_t st = validate(false, false, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS || quick == Quick::kDone) return st;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if ((M + tile - 1) / tile > 65535) return TGEMM_ERROR_NOT_SUPPORTED;  // grid rows limit
    return from_hip(tgemm::launch_lds_tiled(pack(false, false, M, N, K, A, lda, B, ldb, C, ldc), tile, pad, stream));
}

tgemm_status_t tgemm_sgemm_simt(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                                const float *B, int64_t ldb, float *C, int64_t ldc, hipStream_t stream)
{
    Quick quick;
    const tgemm_status_t st = validate(false, false, M, N, K, A, lda, B, ldb, C, ldc, quick);
    if (st != TGEMM_SUCCESS || quick == Quick::kDone) return st;
    if (quick == Quick::kZeroFill) return from_hip(tgemm::launch_fill_zero((int)M, (int)N, C, ldc, stream));
    if ((M + 127) / 128 > 65535) return TGEMM_ERROR_NOT_SUPPORTED;  // grid rows limit
    return from_hip(tgemm::launch_simt_tiled(pack(false, false, M, N, K, A, lda, B, ldb, C, ldc), stream));
}

tgemm_status_t tgemm_transpose(int64_t M, int64_t N, const float *A, int64_t lda, float *B, int64_t ldb,
                               tgemm_transpose_kernel_t kernel, hipStream_t stream)
{
    if (M < 0 || N < 0 || lda < max1(N) || ldb < max1(M)) return TGEMM_ERROR_INVALID_VALUE;
    tgemm::TransposeKind kind;
    switch (kernel) {
        case TGEMM_TRANSPOSE_BLOCKED: kind = tgemm::TransposeKind::kBlocked; break;
        case TGEMM_TRANSPOSE_NAIVE: kind = tgemm::TransposeKind::kNaive; break;
        case TGEMM_TRANSPOSE_TILED: kind = tgemm::TransposeKind::kTiled; break;
        case TGEMM_TRANSPOSE_TILED_PADDED: kind = tgemm::TransposeKind::kTiledPadded; break;
        default: return TGEMM_ERROR_NOT_SUPPORTED;
    }
    if (M > kMaxDim || N > kMaxDim || lda > (int64_t)1 << 40 || ldb > (int64_t)1 << 40)
        return TGEMM_ERROR_NOT_SUPPORTED;
    if (M == 0 || N == 0) return TGEMM_SUCCESS;
    if (A == nullptr || B == nullptr || reinterpret_cast<uintptr_t>(A) % alignof(float) ||
        reinterpret_cast<uintptr_t>(B) % alignof(float))
        return TGEMM_ERROR_INVALID_VALUE;
    uintptr_t a0, a1, b0, b1;
    if (!span(A, M, N, lda, a0, a1) || !span(B, N, M, ldb, b0, b1)) return TGEMM_ERROR_INVALID_VALUE;
    if (overlaps(a0, a1, b0, b1)) return TGEMM_ERROR_INVALID_VALUE;
    const bool vec4 = aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0;
    return from_hip(tgemm::launch_transpose(kind, tgemm::TransposeArgs{(int)M, (int)N, A, lda, B, ldb, vec4},
                                            stream));
}

const char *tgemm_status_string(tgemm_status_t status)
{
    switch (status) {
        case TGEMM_SUCCESS: return "success";
        case TGEMM_ERROR_INVALID_VALUE: return "invalid value (size, leading dimension, pointer or overlap)";
        case TGEMM_ERROR_NOT_SUPPORTED: return "not supported (size above 2^31-2^16, alignment, or unknown kernel choice)";
        case TGEMM_ERROR_HIP: return "HIP runtime refused the launch";
    }
    return "unknown status";
}

int tgemm_version(void) { return 200; }

}  // extern "C"
