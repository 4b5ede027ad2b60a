// The product kernel: tiled fp32 GEMM on the gfx950 matrix cores.
//
// What it computes is page 1's product ("[Multi-Core & GPU Programming] CUDA -
// Matrix Multiplication", section [Matrix Multiplication]); how it is staged
// follows the tiling plan of page 1's section [Shared Memory] and page 2
// ("Lec 29 · GPU Architecture (2)") §1.1-1.2, redone for CDNA4:
//
// * A work-group computes one BM×BN tile of C at a time and walks K in
//   phases of BK (page 1, "Work Flow - Compute Block(0, 0)": tile phases).
// * Per phase the work-group copies a BM×BK slice of A and a BK×BN slice of B
//   from device memory into LDS.  Consecutive lanes read consecutive
//   addresses of one row (page 1, section [Coalescing]; page 2 §1.4, bursts):
//   4 lanes × 16 bytes cover a 64-byte A row segment, 32 lanes a 512-byte B
//   row.
// * The copies are buffer loads: each phase rebases a buffer descriptor on the
//   slice's first element, and every lane keeps a fixed 32-bit offset.  Lanes
//   whose row (A) or column (B) lies outside the matrix carry an offset
//   beyond any extent, which the hardware answers with zero, so edge tiles
//   need no per-element tests and no load leaves the operand.  Whole phases
//   (the main loop) need nothing more: their descriptor takes the largest
//   extent and only its base moves, two scalar additions a phase.  The last
//   phases (the tail loop) carry the exact extent of what remains of the
//   operand; the partial phase of K masks A's columns explicitly, and B's
//   rows past K fall outside its extent on their own.  Recomputing the exact
//   extent every phase, as the tail does, costs 64-bit scalar arithmetic and
//   vector compares among the matrix-core instructions: 1.5-2% at 4096³,
//   and 9% at 1024³.
// * The grid is persistent (configurations without a K split): at most as
//   many work-groups as the chip holds at once, each looping over tiles
//   blockIdx.x, blockIdx.x + gridDim.x, ...  With one work-group per tile
//   dealt in rounds by the hardware, the lean loop above lost 2-4% from the
//   third round on (a work-group starting beside one half-way through its
//   tile, the two sharing the SIMDs unevenly); persistent, it gains at every
//   size measured.
// * LDS holds two stages and registers hold two more phases in flight.
//   Phase p computes from stage p%2; phase p+1, whose loads were issued two
//   phases earlier, is written from registers to the other stage; the loads
//   of phase p+3 are issued into the registers just freed; and there is one
//   barrier per phase.  That barrier covers both of the pages' reasons to
//   synchronise (page 1, "__syncthreads( )"): the stage about to be read is
//   complete, and the stage about to be refilled is read no more.  A load
//   has two phases of matrix-core work (its own wavefront's and, with two
//   work-groups per compute unit, the other wavefront's on the same SIMD)
//   to arrive, so a miss in L2 rarely stalls the LDS write.  The two register
//   sets alternate, so the main loop is unrolled by two and has no branches;
//   the last phases (the partial K phase among them) run in a tail loop.
//   (The 256×128 configuration with 4-byte loads has one register set: its
//   loads run two phases ahead, see below.)
//   Measured on MI355X at 8192³ (4096³), bit-identical results, by how many
//   phases ahead of its computation a phase's loads are issued (before the
//   lean loads and the persistent grid): one (the next phase only, issued
//   after the matrix-core block with its issue priority raised) 92.4%
//   (91.0%) of peak; two (one register set) 93.5% (92.3%); three (this
//   ring) 94.7% (93.4%); four needs a third register set, which spills at
//   this tile and is no better at the smaller ones.  With loads in flight
//   across phases, raising the priority of the matrix-core block costs 4-5
//   points, so it is not raised.  The loads' latency is not what is left:
//   pointing every work-group at one cached tile gains 0.3%.
// * Within a phase the memory work is interleaved with the MFMAs: each
//   k-group's MFMAs cover the reads of the next group's fragments; the
//   first group's also cover the write of phase p+1 (where a group has too
//   few MFMAs for that, the 64×64 tile, A's part of the write goes with the
//   first group and B's with the second); the barrier sits before
//   the last k-group, whose fragments are already in registers, so the last
//   group's MFMAs cover the reads of phase p+1's first fragments and the
//   loads.  Every LDS access then has a k-group of MFMAs to complete in.
//   The compiler is told the interleave (which memory instruction after how
//   many MFMAs): without that it bunches them and the same code is 4-5
//   points slower; with it, 95.6-96.2% of peak at 8192³ against 94.4% for
//   a plain schedule (all k-groups, then the write, the loads and the
//   barrier); 97.4% with the lean loads and persistent grid.  With 4-byte
//   loads (24 a phase at 256×128) two register sets spill at 256×128, so
//   that configuration keeps one (loads two phases ahead); measured at
//   8192³ with 4-byte loads forced: plain schedule 140.3 TFLOP/s,
//   interleaved with one set 148.8, with two sets 134.3 (spilling); at
//   128×128 two sets are ahead (139.3 against 133.3 plain).
// * K split inside a work-group (32×32 tiles with KS = 4 or 8 single
//   wavefronts): on shapes with too few tiles to give every SIMD a
//   wavefront (M·N up to about 640², or skinny shapes with long K), the
//   work-group holds KS groups of wavefronts, each running the pipeline
//   above over its own slice of K (a whole number of phases; the last slice
//   shorter) with its own LDS stages and registers.  Every slice runs the
//   same phases, so the barriers stay uniform; reads past a slice's end
//   return zero.  At the end the slices' sums meet in LDS and slice 0 adds
//   them in slice order and writes C, so the result does not depend on
//   timing.  Measured on MI355X (µs, against the best unsplit tile): 512³
//   7.5 against 11.7; 512×512×16384 94.8 against 156; 2048×256×8192 92.0
//   against 131.  The same split of 64×64 tiles into 2 or 4 groups of four
//   wavefronts lost to the unsplit 64×64 tile once the loads below were
//   whole-phase and the grid persistent (1024×1024×8192: 148 against 133),
//   and is no longer built.
// * K split across work-groups (gridDim.y > 1, from tgemm_sgemm_splitk):
//   work-group (x, s) runs the whole pipeline above over the k range
//   [s·kchunk, min(K, (s+1)·kchunk)) and writes its partial tiles to block s
//   of a workspace; splitk_sum.hip adds the blocks in slice order.  The grid
//   is then one work-group per tile and slice.
// * More work per thread (page 1, end of "Tile Size 결정"): each 64-lane
//   wavefront owns a (BM/WM)×(BN/WN) sub-tile held in accumulator registers
//   for the whole K loop, built from 32×32 blocks of v_mfma_f32_32x32x2_f32.
//   C is written once at the end: by columns (a lane's accumulators are four
//   rows of one column), or, for the 160×128 tile, by rows from blocks
//   formed transposed (mfma_common.h, store_c_t).
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
// * Transposed operands: an operand is read from device memory along the
//   dimension it is contiguous in and kept in LDS the same way — k-contiguous
//   slices as [mn][k] (A as stored, or B transposed), mn-contiguous ones as
//   [k][mn] (B as stored, or A transposed) — and mfma_common.h reads either
//   layout.  No operand is transposed on the way (page 1, section
//   [Coalescing], "Corner Turning": load in the coalesced order, read on chip
//   in the order the arithmetic needs).
#include <atomic>

#include "mfma_common.h"
#include "tgemm_kernels.h"

namespace tgemm {
namespace {

using mfma::f32x16;
using mfma::f32x4;
using mfma::kWave;

constexpr uint32_t kOutside = 0x80000000u;  // an offset beyond every extent (all are < 2^31)

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

// Raw buffer over [base, base + bytes); bytes is clamped to [0, 2^31 - 1],
// which only ever shortens an extent that reaches beyond every offset in use.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const float *base, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n, 0x00020000);
}

// One operand's per-phase copy: a MN×BK slice (MN = BM for A, BN for B) read
// from device memory and written to one LDS stage.
//   KC: the operand is k-contiguous in memory (A as stored, B transposed):
//       element (mn, k) at ptr[mn*ld + k]; LDS keeps [mn][k], row stride BK+4.
//   MC: mn-contiguous (B as stored, A transposed): element (mn, k) at
//       ptr[k*ld + mn]; LDS keeps [k][mn], row stride MN+8.
// Each thread owns L slots of VEC consecutive elements along the contiguous
// dimension; consecutive threads own consecutive slots of a row.
template <bool KC_, int MN, int BK, int VEC, int NT>
struct Loader {
    static constexpr bool KC = KC_;
    static constexpr int ROWS = KC ? MN : BK;           // rows of the slice as stored
    static constexpr int COLS = KC ? BK : MN;           // contiguous extent of a row
    static constexpr int S = KC ? BK + 4 : MN + 8;      // LDS row stride (words)
    static constexpr int WORDS = ROWS * S;              // one LDS stage
    static constexpr int L = ROWS * COLS / (VEC * NT);  // slots per thread
    static constexpr int R = NT * VEC / COLS;           // rows between a thread's slots
    static_assert((NT * VEC) % COLS == 0 && L >= 1 && L * R == ROWS, "slice splits into whole rows");

    typedef typename Vec<VEC>::type vec_t;
    uint32_t off[L];  // byte offset of each slot from the slice's first element
    int c;            // contiguous coordinate of the thread's slots
    int st;           // LDS word offset of slot 0 (slot i adds i*R*S)
    vec_t reg[L];

    // mn_valid: rows (KC) or columns (MC) of this tile inside the matrix.
    __device__ __forceinline__ void init(int t, int64_t ld, int mn_valid)
    {
        const int r0 = t * VEC / COLS;
        c = t * VEC % COLS;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int r = r0 + i * R;
            const bool in = KC ? r < mn_valid : c < mn_valid;
            off[i] = in ? (uint32_t)((r * ld + c) * 4) : kOutside;
        }
        st = r0 * S + c;
    }

    // Issue the loads of the phase starting at k0.  tile = operand pointer at
    // (mn0, 0); K_end: end of the summed range.  Reads past the extent give
    // zero; for KC operands the columns k >= K_end of a partial phase are cut
    // explicitly (for MC they lie past the extent).
    __device__ __forceinline__ void issue(const float *tile, int64_t ld, int k0, int K_end, int mn_valid,
                                          bool partial)
    {
        const __amdgpu_buffer_rsrc_t rs =
            KC ? buffer(tile + k0, ((int64_t)(mn_valid - 1) * ld + (K_end - k0)) * 4)
               : buffer(tile + (int64_t)k0 * ld, ((int64_t)(K_end - k0 - 1) * ld + mn_valid) * 4);
        const bool cut = KC && partial && k0 + c >= K_end;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const uint32_t o = cut ? kOutside : off[i];
            reg[i] = Vec<VEC>::load(rs, o);
        }
    }

    // Issue the loads of a whole phase (every k of it below the end of the
    // summed range).  The extent then only has to exclude the lanes outside
    // the matrix, which carry kOutside, so the descriptor takes the largest
    // extent and only its base moves with k0: two scalar additions a phase
    // instead of the exact extent's 64-bit arithmetic.
    __device__ __forceinline__ void issue_whole(const float *tile, int64_t ld, int k0)
    {
        const float *base = KC ? tile + k0 : tile + (int64_t)k0 * ld;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int i = 0; i < L; ++i) reg[i] = Vec<VEC>::load(rs, off[i]);
    }

    __device__ __forceinline__ void store(float *stage) const
    {
#pragma unroll
        for (int i = 0; i < L; ++i) *reinterpret_cast<vec_t *>(stage + st + i * R * S) = reg[i];
    }
};

template <int BM_, int BN_, int BK_, int WM_, int WN_, int VEC_, int GROUP_M_, int OCC_, bool TA_,
          bool TB_, int KS_ = 1, int NS_ = 2, bool SWAPC_ = false, bool WSPLIT_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, VEC = VEC_;
    static constexpr int KS = KS_;                     // K slices per work-group (see the kernel)
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int OCC = OCC_;                   // wavefronts per SIMD to budget registers for
    static constexpr int NS = NS_;                     // register sets of staged loads (see the kernel)
    static_assert(NS == 1 || NS == 2, "one or two register sets");
    static constexpr bool TA = TA_, TB = TB_;          // operands stored transposed
    static constexpr bool SWAPC = SWAPC_ && KS_ == 1;  // blocks formed transposed, C stored by rows
    static constexpr bool WSPLIT = WSPLIT_ && BK_ >= 24;  // A's LDS writes in k-group 0, B's in k-group 1
    static constexpr int NTS = kWave * WM * WN;        // threads per K slice
    static constexpr int NT = NTS * KS;                // threads per work-group
    static constexpr int TM = BM / WM, TN = BN / WN;   // wavefront sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;   // 32×32 blocks per wavefront
    typedef Loader<!TA, BM, BK, VEC, NTS> LA;          // A as stored is k-contiguous
    typedef Loader<TB, BN, BK, VEC, NTS> LB;           // B as stored is n-contiguous
    static constexpr int A_STAGE = LA::WORDS;
    static constexpr int STAGE = A_STAGE + LB::WORDS;
    static constexpr int LDS_WORDS = 2 * STAGE * KS;   // two stages per K slice
    static_assert(KS == 1 || (KS - 1) * NTS * FM * FN * 16 <= LDS_WORDS, "slice sums fit in LDS");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront sub-tile must be 32-aligned");
    static_assert(BK % 8 == 0, "phase depth must be a multiple of 8");
    static_assert(LDS_WORDS * 4 <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <class G>
__global__ __launch_bounds__(G::NT) __attribute__((amdgpu_waves_per_eu(G::OCC, G::OCC)))
void mfma_sgemm_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
                       const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                       int64_t ldc, int kchunk, int64_t c_slice)
{
    typedef typename G::LA LA;
    typedef typename G::LB LB;

    if (gridDim.y > 1) {
        // K split across work-groups: slice blockIdx.y is the product over
        // its own kchunk values of k, written to its own block of C
        const int kb = (int)blockIdx.y * kchunk;
        A += LA::KC ? (int64_t)kb : (int64_t)kb * lda;
        B += LB::KC ? (int64_t)kb : (int64_t)kb * ldb;
        K = min(kchunk, K - kb);
        C += (int64_t)blockIdx.y * c_slice;
    }

    __shared__ __attribute__((aligned(16))) float lds[G::LDS_WORDS];
    // whether C's rows start 16-byte aligned (only the transposed-block
    // epilogue uses it)
    const bool c_vec = reinterpret_cast<uintptr_t>(C) % 16 == 0 && ldc % 4 == 0;
    (void)c_vec;

    const int tiles_m = (M + G::BM - 1) / G::BM;
    const int tiles_n = (N + G::BN - 1) / G::BN;
    const int ntiles = tiles_m * tiles_n;
    const int wave_id = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    // the grid holds at most as many work-groups as the chip holds at once;
    // each one takes tiles blockIdx.x, blockIdx.x + gridDim.x, ...
    // (a 64-bit tile index, so that tile + gridDim.x cannot wrap for any
    // tile count below 2^31)
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        int tm, tn;
        mfma::tile_of(tiles_m, tiles_n, G::GROUP_M, tm, tn, (int)tile, ntiles);
        const int m0 = tm * G::BM, n0 = tn * G::BN;
        const int rows_valid = min(G::BM, M - m0), cols_valid = min(G::BN, N - n0);

        constexpr bool SPLIT = G::KS > 1;
        // the lane-dependent offsets below are recomputed for every tile (a
        // few integer operations) rather than kept in vector registers across
        // the tile loop: the thread's index is rebuilt from the wavefront's
        // index (a scalar) and the lane's position (v_mbcnt, fed an in-loop
        // zero so that it is not hoisted)
        unsigned zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
        const int tid = wave_id * kWave + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, zero));
        const int ks = SPLIT ? tid / G::NTS : 0;    // K slice of this thread
        const int t = SPLIT ? tid % G::NTS : tid;  // index within the slice
        const int lane = t % kWave, wave = t / kWave;
        const int wm = wave / G::WN, wn = wave % G::WN;
        const int l32 = lane % 32, half = lane / 32;

        // NS register sets of staged loads: phase r travels in set (r - 1) mod NS
        LA la[G::NS];
        LB lb[G::NS];
        la[0].init(t, lda, rows_valid);
        lb[0].init(t, ldb, cols_valid);
#pragma unroll
        for (int s = 1; s < G::NS; ++s) {
            la[s] = la[0];
            lb[s] = lb[0];
        }
        // operand pointers at (m0, 0) and (n0, 0) in their own storage order
        const float *a_tile = A + (LA::KC ? (int64_t)m0 * lda : (int64_t)m0);
        const float *b_tile = B + (LB::KC ? (int64_t)n0 * ldb : (int64_t)n0);

        // the accumulators start from the in-loop zero above, so that no
        // zero vector is kept (or spilled) across the tile loop
        f32x16 acc[G::FM][G::FN];
        const float fzero = __builtin_bit_cast(float, zero);
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
            for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x16(fzero);

        // fragment offsets of k-group 0 (later groups add a constant step)
        int a_frag[G::FM], b_frag[G::FN];
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
            a_frag[i] = mfma::frag_offset<LA::KC, LA::S>(wm * G::TM + i * 32 + l32, 0, half);
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
            b_frag[j] = mfma::frag_offset<LB::KC, LB::S>(wn * G::TN + j * 32 + l32, 0, half);
        // K range [kb, ke) of this thread's slice; `full` phases hold BK values
        // of k, `nphase` phases in all, and phase r is `cut` (its k range reaches
        // past ke: A's columns there are masked) from r = full on.  With K split,
        // slices are kchunk long (a whole number of phases), the last shorter;
        // every slice runs the same phases, so barriers match: `full` counts the
        // phases that are whole in every slice, `nphase` the first slice's, and
        // reads past a slice's end return zero.
        int kb = 0, ke = K, full, nphase;
        if constexpr (SPLIT) {
            const int kchunk = ((K + G::KS - 1) / G::KS + G::BK - 1) / G::BK * G::BK;
            kb = min(K, ks * kchunk);
            ke = min(K, kb + kchunk);
            full = max(0, K - (G::KS - 1) * kchunk) / G::BK;
            nphase = kchunk / G::BK;
        } else {
            full = K / G::BK;
            nphase = full + (K % G::BK != 0);
        }
        float *const slds = SPLIT ? lds + ks * 2 * G::STAGE : lds;  // this slice's two stages
        auto cut = [&] __device__(int r) -> bool {
            if constexpr (SPLIT)
                return kb + (r + 1) * G::BK > ke;
            else
                return r == full;
        };
        // register set s: issue the loads of phase r (`last`: the shorter one) /
        // write phase r to LDS stage r % 2
        auto issue = [&] __device__(int s, int r, bool last) {
            la[s].issue(a_tile, lda, kb + r * G::BK, ke, rows_valid, last);
            lb[s].issue(b_tile, ldb, kb + r * G::BK, ke, cols_valid, last);
        };
        auto issue_whole = [&] __device__(int s, int r) {
            la[s].issue_whole(a_tile, lda, kb + r * G::BK);
            lb[s].issue_whole(b_tile, ldb, kb + r * G::BK);
        };
        auto store = [&] __device__(int s, int r) {
            float *st = slds + (r & 1) * G::STAGE;
            la[s].store(st);
            lb[s].store(st + G::A_STAGE);
        };
        auto store_a = [&] __device__(int s, int r) { la[s].store(slds + (r & 1) * G::STAGE); };
        auto store_b = [&] __device__(int s, int r) { lb[s].store(slds + (r & 1) * G::STAGE + G::A_STAGE); };

        typedef mfma::Fragments<G::FM, G::FN, LA::KC, LA::S, LB::KC, LB::S> Frag;
        constexpr int NG = G::BK / 8;                                             // k-groups per phase
        constexpr int NM = 4 * G::FM * G::FN;                                     // MFMAs per k-group
        constexpr int RD = G::FM * (LA::KC ? 1 : 2) + G::FN * (LB::KC ? 1 : 2);  // LDS reads per k-group
        constexpr int WR = LA::L + LB::L;                                         // LDS writes, loads per phase
        static_assert(NG % 2 == 0, "phase depth must be a multiple of 16");
        Frag f[2];
        auto mgroup = [&] __device__(f32x16(&a)[G::FM][G::FN], const Frag &fr) {
            if constexpr (G::SWAPC)
                mfma::mfma_group_t<G::FM, G::FN>(a, fr);
            else
                mfma::mfma_group<G::FM, G::FN>(a, fr);
        };
        auto rd = [&] __device__(Frag &fr, int stage, int g) {
            const float *st = slds + stage * G::STAGE;
            fr.read(st, st + G::A_STAGE, a_frag, b_frag, g);
        };
        // One phase r, computed from LDS stage r % 2 with register set s holding
        // phase r+1.  next: phase r+1 exists (write it, then the barrier); load:
        // phase r+1+NS exists (issue its loads into set s), load_last: it is the
        // shorter one; whole: it is a whole phase (issue_whole); ng: k-groups
        // whose matrix-core steps run (the partial phase skips the groups that
        // lie wholly past K: they would add products of zero padding to
        // accumulators that start at +0, which changes no bit).
        auto phase = [&] __device__(int s, int r, bool next, bool load, bool load_last, bool whole, int ng) {
            auto issue_next = [&] __device__() {
                if (whole)
                    issue_whole(s, r + 1 + G::NS);
                else if (load)
                    issue(s, r + 1 + G::NS, load_last);
            };
            // k-group g's MFMAs run while group g+1's fragments are read (f[0]
            // holds group 0 on entry); the first group's MFMAs also cover the
            // writes of phase r+1 into the other stage (with WSPLIT, A's part;
            // B's goes with the second group, so that a group of few MFMAs
            // does not issue the whole write in one burst).  The one barrier comes
            // before the last group, whose fragments are already in registers:
            // it certifies that stage r+1 is complete and that stage r is read
            // no more, so the last group's MFMAs cover the reads of phase r+1's
            // first group and the loads of phase r+1+NS.  The compiler is told
            // how to interleave each group (sched_group_barrier); without that
            // it bunches the memory instructions and the kernel runs slower
            // than a plain schedule (all groups, then the write, the loads and
            // the barrier).
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g + 1 < NG) {
                    rd(f[(g + 1) & 1], r & 1, g + 1);
                    if constexpr (G::WSPLIT) {
                        if (g == 0 && next) store_a(s, r + 1);
                        if (g == 1 && next) store_b(s, r + 1);
                    } else {
                        if (g == 0 && next) store(s, r + 1);
                    }
                    if (g < ng) mgroup(acc, f[g & 1]);
                    if (g == 0)
                        mfma::interleave<NM, RD, 0x100, G::WSPLIT ? LA::L : WR, 0x200, 0>();
                    else if (G::WSPLIT && g == 1)
                        mfma::interleave<NM, RD, 0x100, LB::L, 0x200, 1>();
                    else
                        mfma::interleave<NM, RD, 0x100, 0, 0x200, 1>();
                } else {
                    if (next) {
                        __syncthreads();
                        rd(f[0], (r + 1) & 1, 0);
                    }
                    issue_next();
                    if (g < ng) mgroup(acc, f[g & 1]);
                    mfma::interleave<NM, RD, 0x100, WR, 0x020, 2>();
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // phases 0 .. NS-1 are in flight before phase 0 is written, so that
        // the first phases' memory latencies overlap (the set holding phase 0
        // takes phase NS once it is written).  Phases past the last one are
        // loaded too (a buffer extent that ends inside the operand's valid
        // rows or is empty, and never written to LDS): with the loads
        // unconditional the compiler's count of loads in flight at the loop
        // head is exact, and each LDS write waits for its own phase's loads
        // only
        issue(G::NS - 1, 0, cut(0));
#pragma unroll
        for (int s = 0; s + 1 < G::NS; ++s) issue(s, s + 1, cut(s + 1));
        store(G::NS - 1, 0);
        issue(G::NS - 1, G::NS, cut(G::NS));
        __syncthreads();
        rd(f[0], 0, 0);
        int p = 0;
#pragma unroll 1
        for (; p + 2 * G::NS < full; p += G::NS) {  // every phase loaded in here is a full one
#pragma unroll
            for (int s = 0; s < G::NS; ++s) phase(s, p + s, true, true, false, true, NG);
        }
        // k-groups of the partial phase that hold a k below K (without a K
        // split; with one, every slice runs all groups)
        const int ng_last = SPLIT ? NG : (K - full * G::BK + 7) / 8;
#pragma unroll 1
        for (; p < nphase; p += G::NS) {
#pragma unroll
            for (int s = 0; s < G::NS; ++s) {
                const int r = p + s;
                if (r < nphase)
                    phase(s, r, r + 1 < nphase, r + 1 + G::NS < nphase, cut(r + 1 + G::NS), false,
                          r == full ? ng_last : NG);
            }
        }

        if constexpr (G::KS > 1) {
            // the slices' sums meet in LDS (the stages are free once every
            // wavefront has passed the first barrier) and are added in slice order
            constexpr int PER = G::FM * G::FN * 16;  // accumulators per lane
            __syncthreads();
            if (ks > 0) {
                float *red = lds + ((ks - 1) * (G::NTS / kWave) + wave) * PER * kWave + lane;
#pragma unroll
                for (int i = 0; i < G::FM; ++i)
#pragma unroll
                    for (int j = 0; j < G::FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) red[((i * G::FN + j) * 16 + r) * kWave] = acc[i][j][r];
            }
            __syncthreads();
            if (ks > 0) return;  // with K split the grid is one work-group per tile
#pragma unroll
            for (int q = 1; q < G::KS; ++q) {
                const float *red = lds + ((q - 1) * (G::NTS / kWave) + wave) * PER * kWave + lane;
#pragma unroll
                for (int i = 0; i < G::FM; ++i)
#pragma unroll
                    for (int j = 0; j < G::FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * G::FN + j) * 16 + r) * kWave];
            }
        }
        {
            // this thread's place in the tile, rebuilt as at the tile's start
            unsigned zero_c;
            asm volatile("v_mov_b32 %0, 0" : "=v"(zero_c));
            const int lane_c = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, zero_c));
            const int wave_c = (SPLIT ? (wave_id * kWave) % G::NTS : wave_id * kWave) / kWave;
            const int row0 = m0 + (wave_c / G::WN) * G::TM, col0 = n0 + (wave_c % G::WN) * G::TN;
            if constexpr (G::SWAPC)
                mfma::store_c_t<G::FM, G::FN>(acc, C, ldc, M, N, row0, col0, lane_c / 32, lane_c % 32, c_vec);
            else
                mfma::store_c<G::FM, G::FN>(acc, C, ldc, M, N, row0, col0, lane_c / 32, lane_c % 32);
        }
        // the next tile's first write into LDS waits until every wavefront
        // is done reading this tile's last stage
        if (tile + gridDim.x < ntiles) __syncthreads();
    }
}

template <class G>
constexpr int wg_per_cu()
{
    constexpr int by_lds = (160 * 1024) / (G::LDS_WORDS * 4);
    constexpr int by_waves = G::OCC * 4 / (G::WM * G::WN * G::KS);  // OCC wavefronts per SIMD
    return by_lds < by_waves ? by_lds : by_waves;
}

// Compute units of the current device, read once per device (0 if the query
// fails).  Every thread that reads it first stores the same value.
int compute_units()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0)
            return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Without a K split the grid is persistent: at most as many work-groups as
// the chip holds at once (a multiple of the 8 XCDs when the CU count is),
// each looping over tiles.  A grid of one work-group per tile, dealt in
// rounds by the hardware, measured 2-4% slower from the third round on
// (8192³: 150.3 against 151.7 TFLOP/s; 12288×4096×4096: 148.8 against
// 150.7): later rounds start a work-group beside one half-way through its
// tile, and the two then share the SIMDs unevenly.  With K split the grid is
// one work-group per tile (those shapes have few tiles).
template <class G>
hipError_t launch_cfg(const GemmArgs &g, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((g.M + G::BM - 1) / G::BM) * ((g.N + G::BN - 1) / G::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    // every slice holds at least one value of k
    if (g.splits < 1 || g.splits > 65535 || (g.splits > 1 && (g.kchunk < 1 || (int64_t)(g.splits - 1) * g.kchunk >= g.K)))
        return hipErrorInvalidValue;
    // with K split across work-groups the grid is one work-group per tile
    // and slice: a persistent grid per slice would hand the tiles left over
    // after its first round to work-groups with the same blockIdx.x in every
    // slice, which the hardware places on the same few CUs (768×768×8192 in
    // eight slices: 130 µs against ~85 one work-group per tile)
    int64_t grid = tiles;
    if constexpr (G::KS == 1) {
        const int64_t slots = (int64_t)compute_units() * wg_per_cu<G>();
        if (g.splits == 1 && slots > 0 && slots < tiles) grid = slots;
    }
    int M = g.M, N = g.N, K = g.K, kchunk = g.kchunk;
    const float *A = g.A, *B = g.B;
    float *C = g.C;
    int64_t lda = g.lda, ldb = g.ldb, ldc = g.ldc, c_slice = g.c_slice;
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc, &kchunk, &c_slice};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_sgemm_kernel<G>),
                           dim3((unsigned)grid, (unsigned)g.splits), dim3(G::NT), args, 0, stream);
}

// Buffer offsets are 32-bit and kept below 2^31: a slot's offset spans at
// most ROWS rows of its operand as stored, which bounds the leading
// dimensions a configuration takes.
template <class L>
constexpr int64_t max_ld()
{
    return ((((int64_t)1 << 31) - 16) / 4 - L::COLS) / L::ROWS;
}

// One tile shape (with KS slices of K per work-group) in its four operand
// orders (NN, TN, NT, TT).
// W × WN wavefronts per K slice (W along M).  NS_TN: register sets for the
// Aᵀ·B order (A stored transposed, B as stored), whose fragment reads keep
// the most LDS addresses live.  TRANS: the shape also runs transposed
// operands (a transposed slice must split into whole rows per pass too).
template <int BM, int BN, int BK, int VEC, int GM, int OCC, int KS = 1, int NS = 2, int W = 2, int NS_TN = NS,
          int WN = W, bool TRANS = true, bool SWAPC = false, bool WSPLIT = false>
struct Shape {
    template <bool TA, bool TB>
    using C = Cfg<BM, BN, BK, W, WN, VEC, GM, OCC, TA, TB, KS, (TA && !TB) ? NS_TN : NS, SWAPC, WSPLIT>;
    static constexpr bool trans = TRANS;
    static constexpr bool c16 = SWAPC;
    static hipError_t launch(const GemmArgs &g, hipStream_t stream)
    {
        if constexpr (!TRANS) {
            if (g.trans_a || g.trans_b) return hipErrorInvalidValue;
            return launch_cfg<C<false, false>>(g, stream);
        } else {
            switch ((g.trans_a ? 1 : 0) + (g.trans_b ? 2 : 0)) {
                case 0: return launch_cfg<C<false, false>>(g, stream);
                case 1: return launch_cfg<C<true, false>>(g, stream);
                case 2: return launch_cfg<C<false, true>>(g, stream);
                default: return launch_cfg<C<true, true>>(g, stream);
            }
        }
    }
};

// Largest leading dimensions of a shape's transposed operands (0 when it
// takes none).
template <class S>
constexpr int64_t max_lda_t()
{
    if constexpr (S::trans)
        return max_ld<typename S::template C<true, false>::LA>();
    else
        return 0;
}
template <class S>
constexpr int64_t max_ldb_t()
{
    if constexpr (S::trans)
        return max_ld<typename S::template C<false, true>::LB>();
    else
        return 0;
}

//             BM   BN  BK VEC GROUP_M OCC
typedef Shape<256, 128, 16, 4, 4, 2, 1, 2, 2, 1> Large4;  // Aᵀ·B: one register set (two spill)
// one work-group per CU: eight wavefronts, two per SIMD, each holding a
// 128×64 sub-tile (256 registers).  The same tile as four wavefronts of
// 128×128, one per SIMD with 256 accumulators in AGPRs, ran 0.1-1.7% slower
// (mean 0.35%) on 27 shape and operand-order cases, bit-identical
typedef Shape<256, 256, 16, 4, 4, 2, 1, 2, 2, 2, 4> Huge4;
typedef Shape<128, 128, 32, 4, 8, 2> Mid4;
// 160 rows of A as stored (5 passes of 32 at 32 values of k); four wavefronts
// side by side, each 160×32.  Its blocks are formed transposed (operands
// exchanged in the MFMA), so a lane holds four consecutive columns of a row
// of C and the epilogue writes 16-byte pieces of rows: 3000×1000×5000 in
// 219.3 against 223.7 µs with the column-wise epilogue, bit-identical (the
// same exchange costs 0.6-0.9% on 128×128 tiles at 2048³, and 256×256
// tiles spilled with it)
typedef Shape<160, 128, 32, 4, 4, 2, 1, 2, 1, 2, 4, false, true> Wide4;
// 64×64: one 32×32 block per wavefront, so a k-group is only four MFMAs and
// cannot cover the phase's four LDS writes next to its three fragment reads.
// Written in one burst after the first group, the writes filled the LDS data
// queue and the wavefronts then waited to issue their next LDS reads (at
// 1024³, 7.1e5 wave-cycles of SQ_WAIT_INST_LDS and 2.7e5 cycles of
// SQ_LDS_DATA_FIFO_FULL against 1.1e5 and 2.5e4 for the vendor BLAS kernel of
// the same tile); A's writes after group 0 and B's after group 1 took 1024³
// from 20.3 to 19.2 µs and 1024×1024×8192 from 131.4 to 123.2, bit-identical
typedef Shape<64, 64, 32, 4, 8, 4, 1, 2, 2, 2, 2, true, false, true> Small4;
typedef Shape<256, 128, 16, 1, 4, 2, 1, 1> Large1;  // one register set (two spill)
typedef Shape<128, 128, 32, 1, 8, 2> Mid1;
typedef Shape<64, 64, 32, 1, 8, 4, 1, 2, 2, 2, 2, true, false, true> Small1;
typedef Shape<32, 32, 32, 4, 8, 2, 4, 2, 1> Tiny4x4;  // one wavefront per K slice
typedef Shape<32, 32, 32, 4, 8, 2, 8, 2, 1> Tiny4x8;
typedef Shape<32, 32, 32, 1, 8, 2, 4, 2, 1> Tiny1x4;
typedef Shape<32, 32, 32, 1, 8, 2, 8, 2, 1> Tiny1x8;

#define TGEMM_VARIANT_TN(name, S, alone, full, round, tn)                                            \
    {                                                                                                \
        name, S::template C<false, false>::BM, S::template C<false, false>::BN,                     \
            S::template C<false, false>::BK * S::template C<false, false>::KS,                      \
            S::template C<false, false>::VEC,                                                       \
            wg_per_cu<typename S::template C<false, false>>(),                                      \
            max_ld<typename S::template C<false, false>::LA>(),                                     \
            max_ld<typename S::template C<false, false>::LB>(),                                     \
            max_lda_t<S>(), max_ldb_t<S>(), S::trans, alone, full, round, &S::launch, true, tn, S::c16  \
    }
#define TGEMM_VARIANT(name, S, alone, full, round) TGEMM_VARIANT_TN(name, S, alone, full, round, 1.0)

// Efficiencies measured on MI355X, as fractions of the matrix-core peak, with
// one resident work-group per CU (alone) and with the CU full, plus a fixed
// cost per round of work-groups (SIMD cycles); api.cpp adds the exposed store
// of the last round.  Fitted to sweeps of 73 shapes (64³ to 16384×6144×8192:
// square, ragged, skinny, long and short K) timing every configuration, on
// two boxes: the model's pick is the measured fastest or within 1.5% of it on
// every one (mean 0.1%).  The one-work-group-per-CU 256×256 tile runs level
// with 256×128 on some boxes (8192³: 7.16-7.20 ms against 7.18-7.19) and
// ahead on others (7.21 against 7.39 ms, where 256×128 runs at a lower clock)
// while moving 24% fewer bytes (3.49 against 4.57 GB a launch); it pulls
// ahead as K grows (16384×5000×8192: 8.96 against 9.03 ms) and falls behind
// at short K (8192×4096×1024: 477 against 472 µs), which its higher fixed
// cost per round expresses: one work-group per CU leaves its pipeline fill
// uncovered.  256×128 with A transposed keeps one register set of staged
// loads (two spill) and runs 3% slower than as stored (tn 0.969: 148.2
// against 153.0 TFLOP/s at 8192³), so Aᵀ·B goes to the 256×256 tile (153.0).
// The 160×128 tile spreads 3000×1000×5000 over 760 tiles, at most three per
// CU (60 blocks of 32×32 against 64 with 256×128 tiles), and leaves 248
// tiles' stores exposed at the end instead of 480: 219-222 against 234 µs.
// Its phases hold 32 values of k (79 KB of LDS, still two work-groups per
// CU): with 16 a phase is 2560 matrix-core cycles per wavefront and the tile
// ran 228 µs there.  The 64×64 entries were refitted after its LDS writes
// were split over two k-groups, together with the split-K counts, on a sweep
// of 36 shapes with both load widths: 3000³ now runs in 409 µs on 64×64
// tiles against 421 on 160×128, and small products with unaligned operands
// go to the 32×32 K split.  The 4-byte-load
// flavours keep their measured ratio to the 16-byte ones; the 32×32
// K-split configurations were fitted to a sweep of 27 small, ragged, skinny
// and long-K shapes with both load widths (one work-group per CU: 256 tiles
// with K = 16384; CU full: 512 tiles with K = 4096 and 8192; the fixed cost
// from 256³ and 512³).
const MfmaVariant kVariants[] = {
    TGEMM_VARIANT_TN("m256n128k16_w2x2_vec4", Large4, 0.975, 0.977, 7000.0, 0.969),
    TGEMM_VARIANT("m256n256k16_w2x4_vec4", Huge4, 0.979, 0.979, 13000.0),
    TGEMM_VARIANT("m128n128k32_w2x2_vec4", Mid4, 0.965, 0.965, 7000.0),
    TGEMM_VARIANT("m160n128k32_w1x4_vec4_nn", Wide4, 0.93, 0.97, 4000.0),
    TGEMM_VARIANT("m64n64k32_w2x2_vec4", Small4, 0.84, 0.88, 7000.0),
    TGEMM_VARIANT("m256n128k16_w2x2_vec1", Large1, 0.937, 0.957, 7000.0),
    TGEMM_VARIANT("m128n128k32_w2x2_vec1", Mid1, 0.844, 0.895, 7000.0),
    TGEMM_VARIANT("m64n64k32_w2x2_vec1", Small1, 0.64, 0.87, 9000.0),
    TGEMM_VARIANT("m32n32k32_w1x1s4_vec4", Tiny4x4, 0.45, 0.61, 9500.0),
    TGEMM_VARIANT("m32n32k32_w1x1s8_vec4", Tiny4x8, 0.60, 0.60, 11500.0),
    TGEMM_VARIANT("m32n32k32_w1x1s4_vec1", Tiny1x4, 0.24, 0.37, 12000.0),
    TGEMM_VARIANT("m32n32k32_w1x1s8_vec1", Tiny1x8, 0.36, 0.36, 15000.0),
};

}  // namespace

int mfma_buffer_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }

const MfmaVariant *mfma_buffer_variant(int index)
{
    if (index < 0 || index >= mfma_buffer_variant_count()) return nullptr;
    return &kVariants[index];
}

}  // namespace tgemm
