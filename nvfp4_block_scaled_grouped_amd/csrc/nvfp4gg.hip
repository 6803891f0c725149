// nvfp4gg.hip -- NVFP4 block-scaled grouped GEMM for MI355X (gfx950).
//
// C_i = A_i . B_i^T per group, A/B packed FP4 E2M1 with one E4M3 scale per 16
// K of a row, fp32 accumulation, fp16 output (kernelindex page
// kernelbot-nvfp4-group-gemm-444497, kernel-source header comment; page
// kernelbot-nvfp4-group-gemm-505431, custom_kernel_fallback).  Also the same
// GEMM with the scales in the pages' blocked layout, and its MXFP4 form (one
// E8M0 scale per 32 K) on the block-scaled FP4 MFMA (run_segment_mx).  The
// C ABI is declared in include/nvfp4gg.h.
//
// Design (gfx950 first; the pages' Blackwell kernels are prior art only):
//   * Scale resolution: every A and B element is dequantised to fp16 as
//     e2m1(code) * e4m3(scale).  That product has at most 6 significant bits
//     and lies in [2^-10, 2688], so fp16 holds it exactly, and the fp16 x fp16
//     products inside the MFMA are exact in fp32.  The contraction runs on
//     v_mfma_f32_16x16x32_f16 with fp32 accumulation.  (CDNA4's block-scaled
//     f8f6f4 MFMA takes power-of-two E8M0 scales per 32 K; it cannot carry an
//     E4M3 mantissa per 16 K, and no 8-bit operand format holds a 6-bit
//     significand.)
//   * Dequant: v_cvt_scalef32_pk_f16_fp4 turns two FP4 codes into two fp16
//     (its scale operand contributes only a power of two, so it is passed
//     1.0), then v_pk_mul_f16 multiplies by the E4M3 scale converted to fp16
//     (exact: every E4M3 value is an fp16 value).
//   * Tile: up to kMaxFrags fragments of 16 rows of A_i x 256 columns of B_i.  One
//     workgroup of 8 waves per CU, two waves per SIMD.  Wave w owns the 64
//     columns of column group w % 4 for all rows of the tile, and the 128-K
//     stages of parity w / 4 (its K half): the two waves on a SIMD share the
//     columns and split the stages, so each B element is loaded and
//     dequantised once, by the wave that uses it, and the SIMD always has a
//     second wave whose MFMAs cover this one's dequantisation (measured on
//     MI355X: about two VALU operations per 16x16x32 MFMA run for free with
//     two waves per SIMD, none with one).  A dequantised A operand read
//     from LDS feeds 4 MFMAs (one per 16-column B fragment).
//   * A: each K half dequantises its own stages of the tile's rows into a
//     double-buffered LDS image in MFMA operand order (4 buffers of 32 KB).
//     B: each lane loads 16 bytes of its row per stage (the four lanes of a
//     row one 64-byte run) into a register ring two stages deep.
//   * K order: the sum over K is order-free.  A and B use the same order, so
//     every pair (a_k, b_k) meets in the same MFMA slot; it is chosen so that
//     each lane's 16 loaded bytes serve four k-steps.
//   * Accumulation: per wave, one fp32 chain over its K half of a segment
//     (at most 64 stages, 8192 K); the two halves are added through LDS at
//     the end of the segment, segments and chains in fp32 after that.
//   * Schedule: the work is the list of (tile, stage) units (schedule.h) with
//     per-stage costs; a persistent grid of one workgroup per CU takes
//     equal-cost contiguous ranges of it, so ragged groups fill the chip in
//     one launch.  A tile whose stages span several workgroups is finished
//     by the first of them (whose range carries the tile's fix-up cost): the
//     others write their fp32 partial tiles to workspace slots and count
//     themselves in on the tile's counter with a release; the first waits
//     for them with acquires (bounded; on time-out it hands the fix-up over
//     to the last to arrive), adds their partials to its own in workgroup
//     order (deterministic) and writes C.
//   * Loads are raw buffer loads whose range is the exact operand size, so
//     rows past M_i or N_i read as zero without branches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "nvfp4gg.h"
#include "schedule.h"

namespace {

using namespace nvfp4sched;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 8;                    // two waves per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kColGroups = 4;                // waves per K half
constexpr int kColFrags = kTileN / kColGroups / 16;   // 16-column B fragments per wave
constexpr int kKSteps = kStageK / 2 / 32;    // MFMA k-steps of one K half of a stage (32 K each)
constexpr int kStageBytes = kStageK / 2;     // bytes of a row per stage
constexpr int kMaxChainStages = 64;          // stages of one chain (8192 K per K half)
constexpr uint32_t kPieceBytes = kWave * 16; // one wave's 16 x 16 fp32 block
// One fp32 partial tile: every (column group, fragment, column fragment)
// piece at a fixed place, whatever the tile's fragment count.
constexpr uint32_t kSlotBytes = kColGroups * kMaxFrags * kColFrags * kPieceBytes;
constexpr uint32_t kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kWaitVmcnt0 = 0x0F70;            // s_waitcnt vmcnt(0) (expcnt, lgkmcnt not waited)
// Default bound on the first contributor's wait (polls of about a
// microsecond each).
constexpr int kWaitLimit = 1 << 20;

static_assert(kColFrags == 4, "a wave owns 64 columns: four 16-column B fragments");
static_assert(kKSteps == 4, "a K half of a stage is one 16-byte piece of 4 k-steps per lane");
static_assert(kFragRows == 16, "fragments are the MFMA's 16 rows");
static_assert(kMaxFrags == 6, "the kernels instantiate tiles of 1 to 6 fragments");

// LDS of one workgroup (byte offsets).  NVFP4: two buffers of the
// dequantised A of a stage, two blocks of staged scales (two stages of the
// tile's B rows and A rows each), and the raw A codes of the next stage
// (one slot per piece, each used by one wave only).  MXFP4: the same with raw A codes and
// E8M0 scales.  At the end of a segment the first kRedBytes carry the
// exchange of the two K halves' accumulators.
constexpr uint32_t kAFragBytes = 2 * kKSteps * kWave * 16;        // [K half][k-step][lane] x 8 fp16
constexpr uint32_t kABufBytes = kMaxFrags * kAFragBytes;          // 48 KB
constexpr uint32_t kSRow = 2 * kStageK / 16;                      // E4M3 bytes of a row per block
constexpr uint32_t kSBBytes = kTileN * kSRow;                     // also two 128-row bands of 8 atoms
constexpr uint32_t kSABytes = kSBBytes;                           // the A rows' bands likewise
constexpr uint32_t kSBlockBytes = kSBBytes + kSABytes;
constexpr uint32_t kNvScaleOff = 2 * kABufBytes;
constexpr uint32_t kNvRawOff = kNvScaleOff + 2 * kSBlockBytes;    // raw A of the next stage, one slot per piece
constexpr uint32_t kNvLds = kNvRawOff + 2 * kMaxFrags * kPieceBytes;

constexpr uint32_t kMxAFragBytes = 2 * kWave * 16;                // [K half][lane] x 32 codes
constexpr uint32_t kMxABufBytes = kMaxFrags * kMxAFragBytes;
constexpr uint32_t kMxSRow = 2 * kStageK / 32;                    // E8M0 bytes of a row per block
constexpr uint32_t kMxSBBytes = kTileN * kMxSRow;
constexpr uint32_t kMxSABytes = kMaxFrags * kFragRows * kMxSRow;
constexpr uint32_t kMxSBlockBytes = kMxSBBytes + kMxSABytes;
constexpr uint32_t kMxScaleOff = 2 * kMxABufBytes;
constexpr uint32_t kMxLds = kMxScaleOff + 2 * kMxSBlockBytes;

constexpr uint32_t kRedBytes = kColGroups * kMaxFrags * kColFrags * kPieceBytes;
constexpr uint32_t kLdsBytes = kNvLds > kRedBytes ? (kNvLds > kMxLds ? kNvLds : kMxLds)
                                                  : (kRedBytes > kMxLds ? kRedBytes : kMxLds);
static_assert(kLdsBytes <= 160 * 1024, "the LDS of one workgroup fits a CU");

struct GroupArgs {
    const uint8_t* A;
    const uint8_t* B;
    const uint8_t* SFA;
    const uint8_t* SFB;
    uint16_t* C;
    int M, N, K;
    int pad;
};

struct LaunchArgs {
    GroupSched sched[kMaxGroups];
    GroupArgs grp[kMaxGroups];
    uint8_t* partials;    // kSlotsPerWG * G slots of kSlotBytes
    int* counters;        // one per workgroup, zero between calls
    int64_t W;            // total cost
    int G;                // workgroups
    int ngroups;
    int wait_limit;       // polls of a tile's first contributor waiting for the others
    int pad;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufferFlags);
}

// Eight FP4 codes (one dword, nibble order) times a shared fp16 scale.
__device__ __forceinline__ h8_t dequant8(uint32_t packed, _Float16 s)
{
    const h2_t s2 = {s, s};
    const h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * s2;
    const h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * s2;
    const h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * s2;
    const h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * s2;
    return h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// The two E4M3 scale bytes in the low 16 bits of a dword -> fp16.
__device__ __forceinline__ h2_t scales2(uint32_t sc)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
}

// Four E4M3 scale bytes of a dword -> fp16.
__device__ __forceinline__ void scales4(uint32_t sc, _Float16* out)
{
    const h2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
    const h2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);
    out[0] = s01.x;
    out[1] = s01.y;
    out[2] = s23.x;
    out[3] = s23.y;
}

// Buffer loads at voffset (per lane, range-checked) + soffset (wave-uniform,
// in an SGPR, so per-stage offsets cost no vector registers).
__device__ __forceinline__ i4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// A per-lane offset that is out of range of every buffer (operands are
// smaller than 2 GiB): the load reads nothing and returns zeros.
constexpr uint32_t kNoLoad = 0x80000000u;


// fp16 round-to-nearest-even (overflow to inf) of 4 floats, packed.
__device__ __forceinline__ uint2 pack4(f4_t v)
{
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
    return w;
}

// Workgroup barrier that hands LDS over between the waves: this wave's LDS
// accesses complete before it, nobody's global loads are waited for (the
// prefetched stages stay in flight), the asm's memory clobber keeps the
// compiler from moving memory accesses across it, and the scheduling
// barrier keeps it from moving any instruction across it (an instruction of
// the next stage that consumed a just-issued load, moved up, would make the
// wait before it drain the load ring).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int P>
using Parity = std::integral_constant<int, P>;

// threadIdx.x behind an empty asm: values derived from it are computed where
// they are used instead of being hoisted out of the persistent loop, which
// would keep them in registers through the accumulator-heavy epilogue.
__device__ __forceinline__ int opaque_tid()
{
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ f4_t zero_acc() { return f4_t{0.0f, 0.0f, 0.0f, 0.0f}; }

// Compiler fences: the asm takes the value as a register operand (so it is
// computed before it) and clobbers memory (so no load or store moves across
// it).  Placed before a register is re-loaded, it keeps the compiler from
// copying a value whose load is still in flight.
template <typename T>
__device__ __forceinline__ void fence_after(const T& v)
{
    asm volatile("" ::"v"(v) : "memory");
}

// Keeps every accumulator in a register across a stage boundary (an empty
// asm that reads and writes it), so the unrolled stages do not move
// accumulators around between them.
template <int F>
__device__ __forceinline__ void pin_acc(f4_t (*acc)[4])
{
#pragma unroll
    for (int a = 0; a < F; ++a)
#pragma unroll
        for (int f = 0; f < 4; ++f) asm volatile("" : "+v"(acc[a][f]));
}

// The worker index of this workgroup.  Workgroups are dispatched round-robin
// over the XCDs (workgroup b runs on XCD b % kXcds), each with its own L2;
// numbering the workers XCD by XCD gives each XCD a contiguous range of the
// work order, so the tiles that share A rows (same group) or a B strip (same
// n-block) mostly meet in one L2.
__device__ __forceinline__ int worker_id(int G)
{
    const int b = blockIdx.x;
    if (G % kXcds == 0) return (b % kXcds) * (G / kXcds) + b / kXcds;
    return b;
}

// ------------------------------------------------------ end of a segment
//
// Accumulators: acc[a][f] element r of lane (c16, kq) of the wave of column
// group cg is tile row 16 a + c16, tile column 64 cg + 16 f + 4 kq + r.  Both
// K halves hold a partial sum of the same (a, f) blocks.  The exchange
// leaves the complete sum of fragment a in the K half that owns it: half 0
// owns [0, Fh), half 1 [Fh, F) (Fh = ceil(F / 2)).  The K half KH is a
// compile-time parameter of every function here (each wave runs the code
// of its own half), so every loop bound and array index is a constant and
// the accumulators stay in registers.

// Byte offset of piece (cg, a, f) of lane `lane` in a partial-tile slot.
__device__ __forceinline__ uint32_t piece_off(int cg, int a, int f, int lane)
{
    return (((uint32_t)(cg * kMaxFrags + a) * kColFrags + (uint32_t)f) * kWave + (uint32_t)lane) * 16u;
}

// The fragments [lo, hi) that K half KH owns, and those of the other half.
template <int F, int KH>
struct Half {
    static constexpr int Fh = (F + 1) / 2;
    static constexpr int lo = KH == 0 ? 0 : Fh;
    static constexpr int hi = KH == 0 ? Fh : F;
    static constexpr int other_lo = KH == 0 ? Fh : 0;
    static constexpr int other_hi = KH == 0 ? F : Fh;
};

template <int F, int KH>
__device__ __forceinline__ void exchange_halves(uint8_t* lds, f4_t (*acc)[kColFrags], int cg, int lane)
{
    using H = Half<F, KH>;
#pragma unroll
    for (int a = H::other_lo; a < H::other_hi; ++a)
#pragma unroll
        for (int f = 0; f < kColFrags; ++f) *reinterpret_cast<f4_t*>(lds + piece_off(cg, a, f, lane)) = acc[a][f];
    lds_barrier();
#pragma unroll
    for (int a = H::lo; a < H::hi; ++a)
#pragma unroll
        for (int f = 0; f < kColFrags; ++f) acc[a][f] += *reinterpret_cast<const f4_t*>(lds + piece_off(cg, a, f, lane));
    lds_barrier();   // the exchange area is the next segment's A stages
}

// This wave's owned pieces to a slot at base.
template <int F, int KH>
__device__ __forceinline__ void store_own(__amdgpu_buffer_rsrc_t r, uint32_t base, const f4_t (*acc)[kColFrags],
                                          int cg, int lane)
{
    using H = Half<F, KH>;
#pragma unroll
    for (int a = H::lo; a < H::hi; ++a)
#pragma unroll
        for (int f = 0; f < kColFrags; ++f)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i4_t, acc[a][f]), r,
                                                   base + piece_off(cg, a, f, lane), 0, 0);
}

// acc += the pieces stored by store_own at base (owned fragments only).
template <int F, int KH>
__device__ __forceinline__ void add_own(__amdgpu_buffer_rsrc_t r, uint32_t base, f4_t (*acc)[kColFrags], int cg,
                                        int lane)
{
    using H = Half<F, KH>;
#pragma unroll
    for (int a = H::lo; a < H::hi; ++a) {
        f4_t v[kColFrags];
#pragma unroll
        for (int f = 0; f < kColFrags; ++f)
            v[f] = __builtin_bit_cast(
                f4_t, __builtin_amdgcn_raw_buffer_load_b128(r, base + piece_off(cg, a, f, lane), 0, 0));
#pragma unroll
        for (int f = 0; f < kColFrags; ++f) acc[a][f] += v[f];
    }
}

// The owned fragments of the output tile to C: fp32 -> fp16 (round to
// nearest even, overflow to inf), four consecutive columns of one row per
// lane, rows and columns past M, N skipped.
template <int F, int KH>
__device__ __forceinline__ void store_c(const GroupArgs& ga, int m0, int n0, const f4_t (*acc)[kColFrags], int cg,
                                        int lane)
{
    using H = Half<F, KH>;
    const int c16 = lane & 15, kq = lane >> 4;
    const int M = ga.M, N = ga.N;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int a = H::lo; a < H::hi; ++a) {
        const int row = m0 + 16 * a + c16;
        if (row >= M) continue;
        uint16_t* crow = ga.C + (size_t)row * N;
#pragma unroll
        for (int f = 0; f < kColFrags; ++f) {
            const int col = n0 + 64 * cg + 16 * f + 4 * kq;
            const uint2 w = pack4(acc[a][f]);
            if (vec && col + 3 < N) {
                *reinterpret_cast<uint2*>(crow + col) = w;
            } else {
                const uint16_t e0 = (uint16_t)w.x, e1 = (uint16_t)(w.x >> 16);
                const uint16_t e2 = (uint16_t)w.y, e3 = (uint16_t)(w.y >> 16);
                if (col < N) crow[col] = e0;
                if (col + 1 < N) crow[col + 1] = e1;
                if (col + 2 < N) crow[col + 2] = e2;
                if (col + 3 < N) crow[col + 3] = e3;
            }
        }
    }
}

// The end of a segment: the two K halves meet in LDS; chains of one segment
// meet in the scratch slot; the last chain finishes the tile alone, or as
// one of several contributors (partial-tile store, counter, and the fix-up
// by the tile's first contributor).
template <int F, int KH>
__device__ __forceinline__ void finish_segment(const LaunchArgs& args, const Pos& pos, bool first_chain,
                                               bool last_chain, uint8_t* lds, int* s_flag,
                                               f4_t (*acc)[kColFrags], int m0, int n0, int cg, int lane)
{
    exchange_halves<F, KH>(lds, acc, cg, lane);

    const GroupSched& gs = args.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(args.partials, (uint32_t)(kSlotsPerWG * args.G) * kSlotBytes);
    const int me = __builtin_amdgcn_readfirstlane(worker_id(args.G));
    // Chains of one segment meet in the scratch slot (written and read by
    // this workgroup only, in program order).
    const uint32_t scratch = (uint32_t)scratch_slot(me) * kSlotBytes;
    if (!first_chain) add_own<F, KH>(rP, scratch, acc, cg, lane);
    if (!last_chain) {
        store_own<F, KH>(rP, scratch, acc, cg, lane);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        return;
    }

    // Finish the tile: alone, or as one of several contributors.
    const int unit = pos.unit;
    const int64_t c_first = pos.tile_cost0;
    const int64_t c_last = pos.tile_cost0 + (int64_t)(gs.stages - 1) * unit;
    const int w_first = __builtin_amdgcn_readfirstlane(owner(args.W, args.G, c_first));
    const int w_last = __builtin_amdgcn_readfirstlane(owner(args.W, args.G, c_last));
    if (w_first == w_last) {
        store_c<F, KH>(ga, m0, n0, acc, cg, lane);
        return;
    }
    int* counter = args.counters + counter_index(w_first);
    auto slot_base = [&](int w) { return (uint32_t)partial_slot(w, w_last) * kSlotBytes; };
    // Who finishes the tile.  The first contributor's range ends with the
    // tile's first stages and carries the tile's start-up and wind-down cost
    // (kTileCost), so it should: it claims the fix-up and waits for the
    // others, a bounded number of polls (all workgroups of the grid run at
    // once when it fits the chip, so the others are running and never wait
    // themselves).  The others store their partials and count themselves in.
    // If the wait runs out, the first contributor stores its partial too and
    // swaps its claim for a hand-over, and whoever then completes the count
    // finishes the tile: exactly one workgroup does, and nobody waits
    // unboundedly.
    //
    // Memory ordering: every wave waits for its partial stores to complete
    // (reach L2) before the workgroup barrier; thread 0 then publishes them
    // with an agent-scope release add (the compiler writes L2 back first), and
    // the finisher's thread 0 reads the counter with agent-scope acquire loads
    // (the compiler invalidates this CU's caches after them) before the
    // barrier after which its waves read the partials.
    const int others = w_last - w_first;
    bool fix;
    if (me != w_first) {
        store_own<F, KH>(rP, slot_base(me), acc, cg, lane);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            *s_flag = other_finishes(old, others) ? 1 : 0;
        }
        __syncthreads();
        fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
        __syncthreads();   // s_flag is reused below and by the next segment
    } else {
        if (threadIdx.x == 0) {
            const int old = __hip_atomic_fetch_add(counter, kClaim, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            int done = first_finishes(old, others);
            for (int poll = 0; !done && poll < args.wait_limit; ++poll) {
                __builtin_amdgcn_s_sleep(2);
                done = first_finishes(__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT), others);
            }
            *s_flag = done;
        }
        __syncthreads();
        fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
        __syncthreads();
        if (!fix) {
            store_own<F, KH>(rP, slot_base(me), acc, cg, lane);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (threadIdx.x == 0) {
                const int old =
                    __hip_atomic_fetch_add(counter, kHandOver - kClaim, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                *s_flag = first_finishes(old, others);   // the count completed meanwhile: still ours
            }
            __syncthreads();
            fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
            __syncthreads();
        }
    }
    if (!fix) return;
    // Sum the contributors' partials in workgroup order, so the result does
    // not depend on who arrived last.
    if (me == w_first) {
        // This workgroup's partial is still in registers (the first
        // contributor ends its range with the tile's first stages, so it
        // tends to finish last); the others are added to it.
        for (int w = w_first + 1; w <= w_last; ++w) add_own<F, KH>(rP, slot_base(w), acc, cg, lane);
    } else {
        // Every partial, this workgroup's own included, is read back.
        using H = Half<F, KH>;
#pragma unroll
        for (int a = H::lo; a < H::hi; ++a)
#pragma unroll
            for (int f = 0; f < kColFrags; ++f) acc[a][f] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int w = w_first; w <= w_last; ++w) add_own<F, KH>(rP, slot_base(w), acc, cg, lane);
    }
    store_c<F, KH>(ga, m0, n0, acc, cg, lane);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stages J .. L-1 of an unrolled pass: f(Parity<J % 2>, i + J).
template <int J, int L, class Fn>
__device__ __forceinline__ void pair_pass(Fn& f, int i)
{
    if constexpr (J < L) {
        f(Parity<J % 2>{}, i + J);
        pair_pass<J + 1, L>(f, i);
    }
}

// --------------------------------------------------------------- NVFP4
//
// One chain [s_begin, s_end) of the stages of a tile with F fragments: a
// workgroup's segment of a tile runs as chains of at most kMaxChainStages
// stages; first_chain / last_chain place this chain in its segment.  A stage
// is 256 K: 128 bytes of every A and B row and 16 scale bytes.  All 8 waves
// work on the same stage; K half kh of a stage is its row bytes
// [64 kh, 64 kh + 64), run by the 4 waves of half kh as 4 k-steps.
//
// MFMA: v_mfma_f32_16x16x32_f16 with B as the first operand (16 columns of
// B_i) and A as the second (16 rows of A_i).  Lane (c16, kq) = (lane % 16,
// lane / 16) supplies column / row c16 and 8 codes of K; it gets back rows
// 4 kq .. 4 kq + 3 of the first operand's side, i.e. output row c16 and
// output columns 4 kq .. 4 kq + 3 of the 16 x 16 block.
//
// K order within a K half (the sum is order-free; A and B use the same
// order): at k-step v lane (c16, kq) holds dword v of the 16 bytes
// [64 kh + 16 kq, +16) of its row's stage bytes, whose scale is byte
// 8 kh + 2 kq + v / 2 of the row's 16 stage scale bytes.  So every lane
// loads 16 contiguous bytes of B per fragment and stage, the four lanes of
// a row one 64-byte run.
//
// A: the 2 F pieces of a stage (fragment a, K half h: 16 rows x 64 bytes)
// are dequantised by the waves, piece p by wave p % 8; lane (c16, kq) of it
// loads the same 16 bytes that consumer lane (c16, kq) of K half h needs
// and writes dword v, dequantised, as that lane's operand of k-step v.
//
// Scales: the scale bytes of a block of two stages of the tile's B rows and
// A rows are loaded by all threads (16 contiguous bytes per thread), one
// stage later written to one of two LDS blocks, and read from there: B's by
// their consumers, A's by the producers.  A tile that ends with a 128-K
// stage gets zero scales for the missing half of that stage, so its codes
// (the next row's, or zeros past the buffer) contribute exact zeros.
//
// Pipeline, per stage t of the chain (register ring slot p = t % 2):
//   * B of stage t is in bq[p] (loaded two stages earlier).  The B operands
//     of a k-step are dequantised during the MFMAs of the previous one
//     (those of k-step 0 during k-step 3 of the stage before); the slot is
//     re-loaded with stage t + 2 once its last dword is dequantised.
//   * A of stage t is in LDS buffer p.  The raw A of stage t + 1 (in the
//     wave's raw LDS slot) is dequantised into the other buffer, one dword
//     per k-step; the raw A of stage t + 2, loaded at the start of the
//     stage, replaces it in the slot at the end.
//   * Scale block b (stages 2 b, 2 b + 1) is loaded during stage 2 b - 3
//     and written during stage 2 b - 2 into LDS block b % 2; it is read
//     from stage 2 b - 1 on (the B look-ahead and the A production read the
//     next stage's scales), and block b - 2 was last read in stage 2 b - 4.
//   * One LDS-only barrier ends the stage.
template <int F, bool kBlocked, int KH>
__device__ __forceinline__ void run_segment(const LaunchArgs& args, const Pos& pos, int s_begin, int s_end,
                                            bool first_chain, bool last_chain, uint8_t* lds, int* s_flag)
{
    constexpr int kh = KH;
    constexpr int kP = F > 4 ? 2 : 1;   // A pieces per wave: pieces w and w + 8 of 2 F
    const GroupSched& gs = args.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const int tid = opaque_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cg = wave & 3;
    const int lane = tid % kWave;
    const int c16 = lane & 15, kq = lane >> 4;
    const int M = ga.M, N = ga.N, K = ga.K;
    const int m0 = mblock_first_frag(gs.frags, gs.mblocks, pos.mb) * kFragRows;
    const int n0 = pos.nb * kTileN;
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 16;
    const int last_stage = gs.stages - 1;
    const bool half_last = (K % kStageK) != 0;   // the tile's last stage holds 128 K

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(ga.B, (uint32_t)N * row_bytes);
    // Blocked scale arrays hold whole 128-row bands.
    const uint32_t sa_rows = kBlocked ? (uint32_t)(M + 127) / 128u * 128u : (uint32_t)M;
    const uint32_t sb_rows = kBlocked ? (uint32_t)(N + 127) / 128u * 128u : (uint32_t)N;
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(ga.SFA, sa_rows * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(ga.SFB, sb_rows * row_scales);

    // B operand of lane (c16, kq) in fragment f: row n0 + 64 cg + 16 f + c16
    // (rows past N read 0), bytes [64 kh + 16 kq, +16) of each stage.
    uint32_t offB[kColFrags];
#pragma unroll
    for (int f = 0; f < kColFrags; ++f)
        offB[f] = (uint32_t)(n0 + 64 * cg + 16 * f + c16) * row_bytes + 64u * kh + 16u * kq;
    // Staged scales (both layouts: thread t copies 16 bytes to byte 16 t of
    // the block's B part, and of its A part).  Row-major: the B part is
    // [row][32 bytes], the row's 16 scale bytes of each of the two stages;
    // the A part likewise for the tile's rows.  Blocked: the B part is the
    // two 128-row bands of the tile's B rows, 8 atoms of 512 bytes each (4
    // scale columns of 128 rows; the 4 atoms of a stage in column order,
    // stage 0 first); the A part the same for the two bands from the one
    // holding row m0.  Byte offset of (row r, scale column c of stage part
    // q) in a part:
    //   row-major: 32 r + 16 q + c
    //   blocked:   512 (8 (r / 128) + 4 q + c / 4) + 16 (r % 32) + 4 ((r / 32) % 4) + c % 4
    auto sf_lds = [&](uint32_t r, uint32_t c) -> uint32_t {
        return kBlocked ? 512u * (8u * (r >> 7) + (c >> 2)) + 16u * (r & 31u) + 4u * ((r >> 5) & 3u) + (c & 3u)
                        : kSRow * r + c;
    };
    constexpr uint32_t kPartStride = kBlocked ? 2048u : 16u;   // stage part 1 of a block
    // This lane's B scales: tile row 64 cg + 16 f + c16, column 8 kh + 2 kq
    // (two bytes: k-steps 0-1 and 2-3).  Fragment f adds sfb_frag(f).
    const uint32_t sbsrc = kNvScaleOff + sf_lds((uint32_t)(64 * cg + c16), 8u * kh + 2u * kq);
    auto sfb_frag = [&](int f) -> uint32_t {
        return kBlocked ? 256u * (uint32_t)(f & 1) + 4u * (uint32_t)(f >> 1) : 16u * kSRow * (uint32_t)f;
    };

    // This wave's A pieces: piece p = wave + 8 x is fragment p / 2, K half
    // p % 2 (real when p < 2 F).
    bool areal[kP];
    uint32_t offA[kP], adst[kP], asrc[kP], araw[kP];
#pragma unroll
    for (int x = 0; x < kP; ++x) {
        const int p = wave + 8 * x;
        areal[x] = (x == 0 && F >= 4) || p < 2 * F;   // waves are 0..7
        const int a = areal[x] ? p >> 1 : 0, h = p & 1;
        offA[x] = (uint32_t)(m0 + 16 * a + c16) * row_bytes + 64u * h + 16u * kq;
        adst[x] = (uint32_t)((a * 2 + h) * kKSteps) * kPieceBytes + 16u * lane;
        // Its scales: staged row m0 + 16 a + c16 (blocked: relative to the
        // first staged band), column 8 h + 2 kq.
        const uint32_t ra = kBlocked ? (uint32_t)(m0 + 16 * a + c16) - (uint32_t)(m0 >> 7) * 128u
                                     : (uint32_t)(16 * a + c16);
        asrc[x] = kNvScaleOff + kSBBytes + sf_lds(ra, 8u * h + 2u * kq);
        araw[x] = kNvRawOff + (uint32_t)(a * 2 + h) * kPieceBytes + 16u * lane;
    }

    f4_t acc[F][kColFrags];

    {
        const int n = s_end - s_begin;
        // Stage j of the chain, clamped to its last stage (loads past the
        // chain re-read it, so every load is unconditional and in range).
        auto sidx = [&](int j) { return s_begin + (j < n ? j : n - 1); };
        // Stage offset of the code loads of chain stage j for K half h.  In
        // a 128-K last stage K half 1 has no codes: it re-reads bytes of its
        // row (or of the next; none past the buffer), which its zero scales
        // cancel.
        const int half1_max = (int)row_bytes - kStageBytes > 0 ? (int)row_bytes - kStageBytes : 0;
        auto soff = [&](int j, int h) {
            const int o = sidx(j) * kStageBytes;
            return (uint32_t)__builtin_amdgcn_readfirstlane(h == 1 && o > half1_max ? half1_max : o);
        };
        // LDS offset of the staged scales of stage j: its block, its part.
        auto sblk = [&](int j) { return (uint32_t)((j >> 1) & 1) * kSBlockBytes + kPartStride * (uint32_t)(j & 1); };
        auto lds_u16 = [&](uint32_t off) -> uint32_t { return *reinterpret_cast<const uint16_t*>(lds + off); };
        // Whether chain stage j is a 128-K last stage, whose K half 1 gets
        // zero scales (its codes are the next row's, or zeros past the
        // buffer).
        auto half_stage = [&](int j) { return half_last && sidx(j) == last_stage; };

        // ---- scale staging: block beta = stages 2 beta, 2 beta + 1, one
        // 16-byte load per thread for each part (A: row-major waves 0-2).
        const uint32_t band_bytes = (uint32_t)K * 8u;   // 128 rows x K/16 scales
        i4_t stb, sta;
        auto stage_load = [&](int beta) {
            if constexpr (!kBlocked) {
                // Two 8-byte loads, so that the second half of a 128-K last
                // stage (past the row's scales) is read by none.
                const int part = tid & 1, r = tid >> 1;
                const int sg = sidx(2 * beta + part);
                const bool hs = half_last && sg == last_stage;
                auto load_row = [&](__amdgpu_buffer_rsrc_t rs, int row) {
                    const uint32_t o = (uint32_t)row * row_scales + 16u * (uint32_t)sg;
                    const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0));
                    const uint2 hi =
                        __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, hs ? kNoLoad : o + 8u, 0, 0));
                    return i4_t{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
                };
                stb = load_row(rSB, n0 + r);
                if (wave < 3) sta = load_row(rSA, m0 + r);
            } else {
                const int atom = tid >> 5, band = atom >> 3, part = (atom >> 2) & 1, quad = atom & 3;
                const uint32_t sg = (uint32_t)sidx(2 * beta + part);
                const uint32_t in_band = 512u * (4u * sg + (uint32_t)quad) + 16u * (uint32_t)(tid & 31);
                stb = load16(rSB, (uint32_t)((n0 >> 7) + band) * band_bytes + in_band, 0);
                sta = load16(rSA, (uint32_t)((m0 >> 7) + band) * band_bytes + in_band, 0);
            }
        };
        auto stage_store = [&](int beta) {
            uint8_t* blk = lds + kNvScaleOff + (uint32_t)(beta & 1) * kSBlockBytes;
            *reinterpret_cast<i4_t*>(blk + 16u * tid) = stb;
            if (kBlocked || wave < 3) *reinterpret_cast<i4_t*>(blk + kSBBytes + 16u * tid) = sta;
        };
        // A scales of piece x for chain stage j, and B scale bytes of
        // fragment f (zero for K half 1 of a 128-K last stage).
        auto a_scales = [&](int x, int j) {
            const uint32_t raw = lds_u16(asrc[x] + sblk(j));
            return scales2(((wave & 1) != 0 && half_stage(j)) ? 0u : raw);
        };
        auto b_scale_bytes = [&](int f, int j) {
            const uint32_t raw = lds_u16(sbsrc + sblk(j) + sfb_frag(f));
            return (kh == 1 && half_stage(j)) ? 0u : raw;
        };

        i4_t bq[2][kColFrags];   // B codes of stages t, t + 1
        h2_t scl[kColFrags];     // B scales of the current stage
        h8_t bcur;               // the B operand of the next MFMAs
        // Dword v of raw A codes q with scales s2 into A buffer buf.
        auto put_a = [&](int buf, int x, uint32_t q, h2_t s2, int v) {
            *reinterpret_cast<h8_t*>(lds + (uint32_t)buf * kABufBytes + adst[x] + (uint32_t)v * kPieceBytes) =
                dequant8(q, s2[v >> 1]);
        };

        // Prologue: scale block 0 staged, block 1 loaded; B of stages 0, 1;
        // A of stage 0 into buffer 0, raw A of stage 1 into the raw slots.
        {
            // (Block 1's scales are loaded before the other loads, as in the
            // loop, where B and A loads follow a block's.)
            i4_t a0[kP], a1[kP];
            stage_load(0);
            i4_t st0b = stb, st0a = sta;
            stage_load(1);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int f = 0; f < kColFrags; ++f) bq[j][f] = load16(rB, offB[f], soff(j, kh));
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) {
                    a0[x] = load16(rA, offA[x], soff(0, wave & 1));
                    a1[x] = load16(rA, offA[x], soff(1, wave & 1));
                }
            {
                uint8_t* blk = lds + kNvScaleOff;
                *reinterpret_cast<i4_t*>(blk + 16u * tid) = st0b;
                if (kBlocked || wave < 3) *reinterpret_cast<i4_t*>(blk + kSBBytes + 16u * tid) = st0a;
            }
            lds_barrier();
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) {
                    const h2_t s2 = a_scales(x, 0);
#pragma unroll
                    for (int v = 0; v < kKSteps; ++v) put_a(0, x, (uint32_t)a0[x][v], s2, v);
                    *reinterpret_cast<i4_t*>(lds + araw[x]) = a1[x];
                }
#pragma unroll
            for (int f = 0; f < kColFrags; ++f) scl[f] = scales2(b_scale_bytes(f, 0));
            bcur = dequant8((uint32_t)bq[0][0][0], scl[0][0]);
        }
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
            for (int f = 0; f < kColFrags; ++f) acc[i][f] = zero_acc();
        pin_acc<F>(acc);
        lds_barrier();

        // Stage t at ring slot p = t % 2 (the loop below is unrolled by 2,
        // so p is a compile-time constant and the stage has no branch on it).
        // The B operands are dequantised one MFMA group ahead: (fragment f,
        // k-step v) during the MFMAs of the operand before it, (0, 0) of the
        // next stage during those of (3, 3).
        auto stage = [&](auto parity, int t) {
            constexpr int p = decltype(parity)::value;
            const uint8_t* ard = lds + (uint32_t)p * kABufBytes + (uint32_t)(kh * kKSteps) * kPieceBytes + 16u * lane;
            auto read_av = [&](int a, int v) {
                return *reinterpret_cast<const h8_t*>(ard + (uint32_t)a * kAFragBytes + (uint32_t)v * kPieceBytes);
            };
            auto read_raw = [&](int x, int v) { return *reinterpret_cast<const uint32_t*>(lds + araw[x] + 4u * v); };
            uint32_t snext[kColFrags];   // B scale bytes of stage t + 1
            h2_t as2[kP];                // A scales of stage t + 1
            uint32_t ar[kP];             // raw A of stage t + 1, dword of the current k-step
            i4_t anext[kP];              // raw A of stage t + 2
            h8_t av[F];                  // A operands of the current k-step
            // Stage start: the A operands of k-step 0, the production's first
            // raw dword and scales, the raw A of stage t + 2.
#pragma unroll
            for (int a = 0; a < F; ++a) av[a] = read_av(a, 0);
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) {
                    ar[x] = read_raw(x, 0);
                    as2[x] = a_scales(x, t + 1);
                    anext[x] = load16(rA, offA[x], soff(t + 2, wave & 1));
                }
#pragma unroll
            for (int v = 0; v < kKSteps; ++v) {
                if (v == 2) {
#pragma unroll
                    for (int f = 0; f < kColFrags; ++f) snext[f] = b_scale_bytes(f, t + 1);
                }
                // The MFMAs of k-step v, fragment-major; the B operand of the
                // next group is dequantised during each group, and during
                // the last group the A operands of k-step v + 1 are read into
                // the registers each MFMA has just consumed.
                if (v > 0) {
#pragma unroll
                    for (int a = 0; a < F; ++a) av[a] = read_av(a, v);
                }
#pragma unroll
                for (int f = 0; f < kColFrags; ++f) {
#pragma unroll
                    for (int a = 0; a < F; ++a) {
                        acc[a][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bcur, av[a], acc[a][f], 0, 0, 0);
                    }
                    h8_t bnext;
                    if (f + 1 < kColFrags) {
                        bnext = dequant8((uint32_t)bq[p][f + 1][v], scl[f + 1][v >> 1]);
                    } else if (v + 1 < kKSteps) {
                        bnext = dequant8((uint32_t)bq[p][0][v + 1], scl[0][(v + 1) >> 1]);
                    } else {
#pragma unroll
                        for (int g = 0; g < kColFrags; ++g) scl[g] = scales2(snext[g]);
                        bnext = dequant8((uint32_t)bq[p ^ 1][0][0], scl[0][0]);
                    }
                    // A register of the ring whose last dword was just
                    // dequantised is re-loaded with stage t + 2.
                    const int done = f + 1 < kColFrags ? (v == kKSteps - 1 ? f + 1 : -1)
                                                       : (v == kKSteps - 2 ? 0 : -1);
                    if (done >= 0) {
                        fence_after(bnext);
                        bq[p][done] = load16(rB, offB[done], soff(t + 2, kh));
                    }
                    bcur = bnext;
                }
                // Dword v of the A pieces of stage t + 1 into the other
                // buffer (its readers of stage t - 1 passed the last barrier);
                // the next dword is read one k-step ahead.
#pragma unroll
                for (int x = 0; x < kP; ++x)
                    if (areal[x]) {
                        put_a(p ^ 1, x, ar[x], as2[x], v);
                        if (v + 1 < kKSteps)
                            ar[x] = read_raw(x, v + 1);
                        else
                            *reinterpret_cast<i4_t*>(lds + araw[x]) = anext[x];
                    }
                if (v == 1) {
                    if constexpr (p == 0)
                        stage_store((t >> 1) + 1);
                    else
                        stage_load((t >> 1) + 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            pin_acc<F>(acc);
            lds_barrier();
        };

        int t = 0;
        for (; t + 1 < n; t += 2) pair_pass<0, 2>(stage, t);
        if (t < n) stage(Parity<0>{}, t);
    }
    finish_segment<F, KH>(args, pos, first_chain, last_chain, lds, s_flag, acc, m0, n0, cg, lane);
}

// ------------------------------------------------------------------ MXFP4
//
// MXFP4 operands: the same packed E2M1 codes, with one E8M0 scale (the value
// 2^(code - 127)) per 32 consecutive K of a row, row-major M x K/32 and
// N x K/32 bytes.  gfx950's block-scaled MFMA takes this form as it is:
// v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands (format code 4)
// multiplies each lane's 32 codes by that lane's E8M0 scale.  Lane (c16, kq)
// supplies row c16 of an operand fragment and 32 K, here the 16 bytes
// [64 kh + 16 kq, +16) of the row's stage bytes (K half kh of the stage, in
// the natural nibble order), whose scale is byte 4 kh + kq of the row's 8
// stage scale bytes.  No dequantisation: one MFMA per fragment pair per K
// half of a stage.
using v8i_t = int __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4_t mfma_mx(i4_t b, uint32_t sb, i4_t a, uint32_t sa, f4_t c)
{
    const v8i_t bv = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    const v8i_t av = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    // src0 = B fragment (output columns), src1 = A fragment (output rows),
    // both FP4; scale byte 0 of each scale register.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av, c, 4, 4, 0, (int)sb, 0, (int)sa);
}

// One chain of an MXFP4 tile (same tile shape, stages, K halves, schedule
// and end of segment as run_segment):
//   * B: each lane loads its 16 bytes per fragment and stage (the MFMA
//     operand as it is), two stages ahead in a register ring.
//   * A: the waves copy the 2 F pieces of the next stage (fragment, K half)
//     to LDS as they are, piece p by wave p % 8.
//   * Scales: staged through LDS in blocks of two stages (8 bytes per row
//     and stage), as in run_segment; each consumer reads its bytes there.
//     A tile that ends with a 128-K stage gets zero scales and zero A codes
//     for the missing half of that stage.
//   * Per stage each wave runs 4 F MFMAs of 16 x 16 x 128; one LDS-only
//     barrier ends the stage.
template <int F, int KH>
__device__ __forceinline__ void run_segment_mx(const LaunchArgs& args, const Pos& pos, int s_begin, int s_end,
                                               bool first_chain, bool last_chain, uint8_t* lds, int* s_flag)
{
    constexpr int kh = KH;
    constexpr int kP = F > 4 ? 2 : 1;
    const GroupSched& gs = args.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const int tid = opaque_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cg = wave & 3;
    const int lane = tid % kWave;
    const int c16 = lane & 15, kq = lane >> 4;
    const int M = ga.M, N = ga.N, K = ga.K;
    const int m0 = mblock_first_frag(gs.frags, gs.mblocks, pos.mb) * kFragRows;
    const int n0 = pos.nb * kTileN;
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 32;
    const int last_stage = gs.stages - 1;
    const bool half_last = (K % kStageK) != 0;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(ga.B, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(ga.SFA, (uint32_t)M * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(ga.SFB, (uint32_t)N * row_scales);

    uint32_t offB[kColFrags];
#pragma unroll
    for (int f = 0; f < kColFrags; ++f)
        offB[f] = (uint32_t)(n0 + 64 * cg + 16 * f + c16) * row_bytes + 64u * kh + 16u * kq;
    const uint32_t sbsrc = kMxScaleOff + (uint32_t)(64 * cg + c16) * kMxSRow + 4u * kh + (uint32_t)kq;
    const uint32_t sasrc = kMxScaleOff + kMxSBBytes + (uint32_t)c16 * kMxSRow + 4u * kh + (uint32_t)kq;

    bool areal[kP];
    bool ahalf1[kP];
    uint32_t offA[kP], adst[kP];
#pragma unroll
    for (int x = 0; x < kP; ++x) {
        const int p = wave + 8 * x;
        areal[x] = (x == 0 && F >= 4) || p < 2 * F;   // waves are 0..7
        const int a = areal[x] ? p >> 1 : 0, h = p & 1;
        ahalf1[x] = h == 1;
        offA[x] = (uint32_t)(m0 + 16 * a + c16) * row_bytes + 64u * h + 16u * kq;
        adst[x] = (uint32_t)(a * 2 + h) * kPieceBytes + 16u * lane;
    }

    f4_t acc[F][kColFrags];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int f = 0; f < kColFrags; ++f) acc[i][f] = zero_acc();

    {
        const int n = s_end - s_begin;
        auto sidx = [&](int j) { return s_begin + (j < n ? j : n - 1); };
        // As in run_segment: K half 1 of a 128-K last stage re-reads bytes
        // of its row (its A codes are zeroed, its scales are zero).
        const int half1_max = (int)row_bytes - kStageBytes > 0 ? (int)row_bytes - kStageBytes : 0;
        auto soff = [&](int j, int h) {
            const int o = sidx(j) * kStageBytes;
            return (uint32_t)__builtin_amdgcn_readfirstlane(h == 1 && o > half1_max ? half1_max : o);
        };
        auto sblk = [&](int j) { return (uint32_t)((j >> 1) & 1) * kMxSBlockBytes + 8u * (uint32_t)(j & 1); };
        auto lds_u8 = [&](uint32_t off) -> uint32_t { return lds[off]; };

        // Scale staging: thread t loads the 8 scale bytes of stage t % 2 of
        // B row t / 2 (and waves 0-2 of A row t / 2), as two 4-byte loads,
        // so that the second half of a 128-K last stage (past the row's
        // scales) is read by none.
        uint2 stb, sta;
        auto stage_load = [&](int beta) {
            const int part = tid & 1, r = tid >> 1;
            const int sg = sidx(2 * beta + part);
            const bool hs = half_last && sg == last_stage;
            auto load_row = [&](__amdgpu_buffer_rsrc_t rs, int row) {
                const uint32_t o = (uint32_t)row * row_scales + 8u * (uint32_t)sg;
                return uint2{__builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0),
                             __builtin_amdgcn_raw_buffer_load_b32(rs, hs ? kNoLoad : o + 4u, 0, 0)};
            };
            stb = load_row(rSB, n0 + r);
            if (wave < 3) sta = load_row(rSA, m0 + r);
        };
        auto stage_store = [&](int beta, uint2 vb, uint2 va) {
            uint8_t* blk = lds + kMxScaleOff + (uint32_t)(beta & 1) * kMxSBlockBytes;
            *reinterpret_cast<uint2*>(blk + 8u * tid) = vb;
            if (wave < 3) *reinterpret_cast<uint2*>(blk + kMxSBBytes + 8u * tid) = va;
        };

        i4_t bq[2][kColFrags], aq[2][kP];
        auto load_b = [&](int slot, int j) {
#pragma unroll
            for (int f = 0; f < kColFrags; ++f) bq[slot][f] = load16(rB, offB[f], soff(j, kh));
        };
        auto load_a = [&](int slot, int j) {
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) aq[slot][x] = load16(rA, offA[x], soff(j, wave & 1));
        };
        // Raw A of chain stage j into buffer buf (zero codes for the missing
        // half of a 128-K last stage).
        auto put_a = [&](int buf, int x, i4_t q, int j) {
            if (ahalf1[x] && half_last && sidx(j) == last_stage) q = i4_t{0, 0, 0, 0};
            *reinterpret_cast<i4_t*>(lds + kMxABufBytes * (uint32_t)buf + adst[x]) = q;
        };
        {
            // Scale block 0 and the raw A of stage 0 first, then the loads
            // in the order two stages of the loop issue them (so the waits
            // the compiler derives for the loop's first stage are those of
            // every other).
            i4_t a0[kP];
            stage_load(0);
            const uint2 st0b = stb, st0a = sta;
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) a0[x] = load16(rA, offA[x], soff(0, wave & 1));
            load_b(0, 0);
            load_a(1, 1);
            stage_load(1);
            load_b(1, 1);
            load_a(0, 2);
            stage_store(0, st0b, st0a);
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) put_a(0, x, a0[x], 0);
        }
        lds_barrier();

        auto stage = [&](auto parity, int t) {
            constexpr int p = decltype(parity)::value;
            uint32_t sb[kColFrags];
#pragma unroll
            for (int f = 0; f < kColFrags; ++f) sb[f] = lds_u8(sbsrc + sblk(t) + 16u * kMxSRow * f);
#pragma unroll
            for (int a = 0; a < F; ++a) {
                const i4_t av = *reinterpret_cast<const i4_t*>(lds + kMxABufBytes * (uint32_t)p +
                                                               (uint32_t)(a * 2 + kh) * kPieceBytes + 16u * lane);
                const uint32_t sa = lds_u8(sasrc + sblk(t) + 16u * kMxSRow * a);
#pragma unroll
                for (int f = 0; f < kColFrags; ++f) acc[a][f] = mfma_mx(bq[p][f], sb[f], av, sa, acc[a][f]);
            }
            // A of stage t + 1 into the other buffer (its readers of stage
            // t - 1 passed the previous barrier), then the ring slots'
            // re-loads: B of stage t + 2, A of stage t + 3.
#pragma unroll
            for (int x = 0; x < kP; ++x)
                if (areal[x]) put_a(p ^ 1, x, aq[p ^ 1][x], t + 1);
            load_b(p, t + 2);
            load_a(p ^ 1, t + 3);
            if constexpr (p == 0)
                stage_store((t >> 1) + 1, stb, sta);
            else
                stage_load((t >> 1) + 2);
            pin_acc<F>(acc);
            lds_barrier();
        };
        int t = 0;
        for (; t + 1 < n; t += 2) pair_pass<0, 2>(stage, t);
        if (t < n) stage(Parity<0>{}, t);
    }
    finish_segment<F, KH>(args, pos, first_chain, last_chain, lds, s_flag, acc, m0, n0, cg, lane);
}

// Wave-uniform values computed in vector registers (64-bit divisions have
// no scalar form) moved back to scalar registers, so they do not occupy
// vector registers through the whole loop.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v)
{
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ Pos uniform(const Pos& p)
{
    Pos r;
    r.group = uniform(p.group);
    r.nb = uniform(p.nb);
    r.mb = uniform(p.mb);
    r.stage = uniform(p.stage);
    r.frags = uniform(p.frags);
    r.unit = uniform(p.unit);
    r.tile_cost0 = uniform(p.tile_cost0);
    return r;
}

// One chain, each wave running the code of its K half (waves 0-3 half 0,
// waves 4-7 half 1).  Both halves meet the same barriers in the same order.
template <bool kMx, bool kBlocked, int F>
__device__ __forceinline__ void run_chain(const LaunchArgs& args, const Pos& pos, int c0, int c1, bool first,
                                          bool last, uint8_t* lds, int* s_flag)
{
    const bool half1 = __builtin_amdgcn_readfirstlane(opaque_tid() / kWave) >= kColGroups;
    if constexpr (kMx) {
        if (half1)
            run_segment_mx<F, 1>(args, pos, c0, c1, first, last, lds, s_flag);
        else
            run_segment_mx<F, 0>(args, pos, c0, c1, first, last, lds, s_flag);
    } else {
        if (half1)
            run_segment<F, kBlocked, 1>(args, pos, c0, c1, first, last, lds, s_flag);
        else
            run_segment<F, kBlocked, 0>(args, pos, c0, c1, first, last, lds, s_flag);
    }
}

// The persistent walk of one workgroup over its cost range: every segment
// (a tile's stages in the range) as chains of at most kMaxChainStages
// stages, each by the segment kernel of its fragment count.
template <bool kMx, bool kBlocked>
__device__ __forceinline__ void walk_range(const LaunchArgs& args, uint8_t* lds, int* s_flag)
{
    const int w = uniform(worker_id(args.G));
    const int64_t b1 = uniform(boundary(args.W, args.G, w + 1));
    Pos pos = uniform(locate(args.sched, args.ngroups, uniform(boundary(args.W, args.G, w))));
    while (pos.group < args.ngroups && stage_cost(pos, pos.stage) < b1) {
        const GroupSched& gs = args.sched[pos.group];
        const int unit = pos.unit;
        // Stages of this tile that start before b1.
        const int64_t s_end64 = uniform((int64_t)((b1 - pos.tile_cost0 + unit - 1) / unit));
        const int s_end = s_end64 < gs.stages ? (int)s_end64 : gs.stages;
        // The segment runs as chains of at most kMaxChainStages stages.
        for (int c0 = pos.stage; c0 < s_end; c0 += kMaxChainStages) {
            const int c1 = c0 + kMaxChainStages < s_end ? c0 + kMaxChainStages : s_end;
            const bool first = c0 == pos.stage, last = c1 == s_end;
            switch (pos.frags) {
                case 1: run_chain<kMx, kBlocked, 1>(args, pos, c0, c1, first, last, lds, s_flag); break;
                case 2: run_chain<kMx, kBlocked, 2>(args, pos, c0, c1, first, last, lds, s_flag); break;
                case 3: run_chain<kMx, kBlocked, 3>(args, pos, c0, c1, first, last, lds, s_flag); break;
                case 4: run_chain<kMx, kBlocked, 4>(args, pos, c0, c1, first, last, lds, s_flag); break;
                case 5: run_chain<kMx, kBlocked, 5>(args, pos, c0, c1, first, last, lds, s_flag); break;
                default: run_chain<kMx, kBlocked, 6>(args, pos, c0, c1, first, last, lds, s_flag); break;
            }
        }
        if (s_end < gs.stages) break;
        pos = uniform(locate(args.sched, args.ngroups, pos.tile_cost0 + (int64_t)unit * gs.stages));
    }
}

__global__ __launch_bounds__(kThreads) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    __shared__ int s_flag;
    walk_range<false, false>(args, lds, &s_flag);
}

// NVFP4 with the scales in the blocked layout.
__global__ __launch_bounds__(kThreads) void nvfp4_blocked_sf_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    __shared__ int s_flag;
    walk_range<false, true>(args, lds, &s_flag);
}

__global__ __launch_bounds__(kThreads) void mxfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    __shared__ int s_flag;
    walk_range<true, false>(args, lds, &s_flag);
}

// Writes zeros to C of a group with K == 0 (the empty sum).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint16_t* C, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        C[i] = 0;
}

// Dequantisation alone, with the same conversion code as the GEMM: one
// thread per 64 consecutive codes of a row (8 dwords) and the 4 scale bytes
// that cover them.  Blocks past the end of the row are skipped.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(int rows, int K, const uint8_t* X,
                                                            const uint8_t* SFX, h8_t* out)
{
    const int blocks = K / 16;                 // scale blocks per row
    const int quads = (blocks + 3) / 4;        // 4-block pieces per row
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)rows * quads) return;
    const int64_t r = t / quads;
    const int b0 = (int)(t % quads) * 4;
    const int nb = blocks - b0 < 4 ? blocks - b0 : 4;

    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sc = 0;
    const uint32_t* xrow = reinterpret_cast<const uint32_t*>(X + r * (K / 2));
    for (int b = 0; b < nb; ++b) {
        w[2 * b] = xrow[2 * (b0 + b)];
        w[2 * b + 1] = xrow[2 * (b0 + b) + 1];
        sc |= (uint32_t)SFX[r * blocks + b0 + b] << (8 * b);
    }
    _Float16 s[4];
    scales4(sc, s);
    h8_t* orow = out + r * (K / 8);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < 2 * nb) orow[2 * b0 + j] = dequant8(w[j], s[j >> 1]);
}

thread_local std::string g_last_error;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace of the split-tile fix-up, one per (device, stream): kSlotsPerWG
// partial-tile slots per workgroup and one counter per workgroup (zero
// between calls; the workgroup that finishes a tile resets its counter).
// Sized for the device's compute units (a launch never has more workgroups),
// allocated by the first call on the pair and never resized or freed, so a
// later call on it allocates, frees and synchronises nothing.
struct Workspace {
    uint8_t* partials = nullptr;
    int* counters = nullptr;
    int workers = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;
std::map<int, int> g_cus;

int device_cus_locked(int dev)
{
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) return it->second;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_cus[dev] = v;
    return v;
}

int get_workspace(int dev, hipStream_t s, Workspace& out)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto key = std::make_pair(dev, (void*)s);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        out = it->second;
        return NVFP4GG_OK;
    }
    Workspace w;
    w.workers = device_cus_locked(dev);
    const size_t pbytes = (size_t)kSlotsPerWG * w.workers * kSlotBytes;
    if (hipMalloc(&w.partials, pbytes) != hipSuccess) return fail(NVFP4GG_HIP_ERROR, "workspace allocation failed");
    if (hipMalloc(&w.counters, (size_t)w.workers * sizeof(int)) != hipSuccess) {
        (void)hipFree(w.partials);
        return fail(NVFP4GG_HIP_ERROR, "workspace allocation failed");
    }
    if (hipMemsetAsync(w.counters, 0, (size_t)w.workers * sizeof(int), s) != hipSuccess) {
        (void)hipFree(w.partials);
        (void)hipFree(w.counters);
        return fail(NVFP4GG_HIP_ERROR, "workspace initialisation failed");
    }
    g_ws[key] = w;
    out = w;
    return NVFP4GG_OK;
}

// Bound on a first contributor's wait (see finish_segment), process-wide.
std::atomic<int> g_wait_limit{kWaitLimit};
// m-block size forced for every launch (0: chosen per launch), process-wide.
std::atomic<int> g_max_frags{0};

}  // namespace

extern "C" const char* nvfp4_group_gemm_last_error(void) { return g_last_error.c_str(); }

extern "C" int nvfp4_group_gemm_version(void) { return 6; }

extern "C" int nvfp4_group_gemm_set_wait_limit(int polls)
{
    if (polls < 0) return fail(NVFP4GG_INVALID_ARG, "the wait limit must be >= 0");
    g_wait_limit.store(polls);
    return NVFP4GG_OK;
}

extern "C" int nvfp4_group_gemm_set_max_frags(int frags)
{
    if (frags < 0 || frags > kMaxFrags)
        return fail(NVFP4GG_INVALID_ARG, "the m-block size must be 0 (automatic) or 1.." + std::to_string(kMaxFrags));
    g_max_frags.store(frags);
    return NVFP4GG_OK;
}

namespace {

// Every grouped-GEMM entry point: fmt selects NVFP4 (E4M3 per 16 K) or
// MXFP4 (E8M0 per 32 K), blocked_sf the blocked layout of NVFP4 scales.
int group_gemm_impl(int g, const int* M, const int* N, const int* K, const void* const* A_ptrs,
                    const void* const* B_ptrs, const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                    void* const* C_ptrs, void* stream, int blocked_sf, int fmt)
{
    g_last_error.clear();
    if (g <= 0) return fail(NVFP4GG_INVALID_ARG, "g must be >= 1");
    if (!M || !N || !K || !A_ptrs || !B_ptrs || !SFA_ptrs || !SFB_ptrs || !C_ptrs)
        return fail(NVFP4GG_INVALID_ARG, "a size or pointer array is NULL");
    for (int i = 0; i < g; ++i) {
        const std::string gs = "group " + std::to_string(i) + ": ";
        if (M[i] < 0 || N[i] < 0 || K[i] < 0) return fail(NVFP4GG_INVALID_ARG, gs + "negative size");
        if (K[i] % 16 != 0) return fail(NVFP4GG_INVALID_ARG, gs + "K must be a multiple of 16");
        if (M[i] == 0 || N[i] == 0) continue;
        if (!C_ptrs[i] || !aligned16(C_ptrs[i]))
            return fail(NVFP4GG_INVALID_ARG, gs + "C pointer is NULL or not 16-byte aligned");
        if (K[i] == 0) continue;
        const void* ops[4] = {A_ptrs[i], B_ptrs[i], SFA_ptrs[i], SFB_ptrs[i]};
        for (const void* p : ops)
            if (!p || !aligned16(p))
                return fail(NVFP4GG_INVALID_ARG, gs + "an operand pointer is NULL or not 16-byte aligned");
        if (K[i] % (kStageK / 2) != 0)
            return fail(NVFP4GG_UNSUPPORTED, gs + "this kernel needs K % 128 == 0");
        // Byte offsets of the buffer loads are 32-bit and may run one tile
        // past the last row.
        const int64_t rows = (int64_t)(M[i] > N[i] ? M[i] : N[i]) + kTileN;
        if (rows * (K[i] / 2) >= ((int64_t)1 << 31))
            return fail(NVFP4GG_UNSUPPORTED, gs + "operand larger than 2 GiB");
        if ((int64_t)M[i] * N[i] >= ((int64_t)1 << 31))
            return fail(NVFP4GG_UNSUPPORTED, gs + "output larger than 2^31 elements");
    }

    bool any_work = false;
    for (int i = 0; i < g; ++i) any_work |= (M[i] > 0 && N[i] > 0);
    if (!any_work) return NVFP4GG_OK;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(NVFP4GG_HIP_ERROR, "hipGetDevice failed");

    // Groups with K == 0 get C = 0 (the empty sum).
    for (int i = 0; i < g; ++i) {
        if (M[i] == 0 || N[i] == 0 || K[i] != 0) continue;
        const int64_t count = (int64_t)M[i] * N[i];
        const int blocks = (int)((count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096);
        hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint16_t*>(C_ptrs[i]),
                           count);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
    }

    Workspace ws;
    bool have_ws = false;
    LaunchArgs args;
    int gi = 0;
    while (gi < g) {
        std::memset(&args, 0, sizeof(args));
        // The next (up to) kMaxGroups non-empty groups form one launch.
        int idx[kMaxGroups], bM[kMaxGroups], bN[kMaxGroups], bK[kMaxGroups];
        int n = 0;
        for (; gi < g && n < kMaxGroups; ++gi) {
            if (M[gi] == 0 || N[gi] == 0 || K[gi] == 0) continue;
            idx[n] = gi;
            bM[n] = M[gi];
            bN[n] = N[gi];
            bK[n] = K[gi];
            ++n;
        }
        if (n == 0) continue;
        if (!have_ws) {
            const int rc = get_workspace(dev, s, ws);
            if (rc != NVFP4GG_OK) return rc;
            have_ws = true;
        }
        const int forced = g_max_frags.load();
        const int maxf = forced > 0 ? forced : choose_max_frags(n, bM, bN, bK, ws.workers, fmt);
        int tiles = 0;
        int64_t cost = 0;
        for (int j = 0; j < n; ++j) {
            const int q = idx[j];
            GroupSched& sc = args.sched[j];
            GroupArgs& ga = args.grp[j];
            ga.A = static_cast<const uint8_t*>(A_ptrs[q]);
            ga.B = static_cast<const uint8_t*>(B_ptrs[q]);
            ga.SFA = static_cast<const uint8_t*>(SFA_ptrs[q]);
            ga.SFB = static_cast<const uint8_t*>(SFB_ptrs[q]);
            ga.C = static_cast<uint16_t*>(C_ptrs[q]);
            ga.M = M[q];
            ga.N = N[q];
            ga.K = K[q];
            sc = make_group_sched(M[q], N[q], K[q], cost, tiles, maxf, fmt);
            cost += group_cost(sc);
            tiles += sc.mblocks * sc.nblocks;
        }
        args.ngroups = n;
        args.W = cost;
        args.G = grid_size(cost, ws.workers);
        if ((uint64_t)kSlotsPerWG * args.G * kSlotBytes >= ((uint64_t)1 << 32))
            return fail(NVFP4GG_UNSUPPORTED, "too many compute units for the partial-tile workspace");
        args.partials = ws.partials;
        args.counters = ws.counters;
        const void* kernel = fmt == kFmtMxfp4 ? reinterpret_cast<const void*>(&mxfp4_group_gemm_kernel)
                             : blocked_sf     ? reinterpret_cast<const void*>(&nvfp4_blocked_sf_gemm_kernel)
                                              : reinterpret_cast<const void*>(&nvfp4_group_gemm_kernel);
        args.wait_limit = g_wait_limit.load();
        void* kargs[] = {&args};
        const hipError_t le = hipLaunchKernel(kernel, dim3(args.G), dim3(kThreads), kargs, 0, s);
        if (le != hipSuccess)
            return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(le));
    }
    return NVFP4GG_OK;
}

}  // namespace

extern "C" int nvfp4_group_gemm(int g, const int* M, const int* N, const int* K,
                                const void* const* A_ptrs, const void* const* B_ptrs,
                                const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                void* const* C_ptrs, void* stream)
{
    return group_gemm_impl(g, M, N, K, A_ptrs, B_ptrs, SFA_ptrs, SFB_ptrs, C_ptrs, stream, 0, kFmtNvfp4);
}

extern "C" int nvfp4_group_gemm_blocked(int g, const int* M, const int* N, const int* K,
                                        const void* const* A_ptrs, const void* const* B_ptrs,
                                        const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                        void* const* C_ptrs, void* stream)
{
    return group_gemm_impl(g, M, N, K, A_ptrs, B_ptrs, SFA_ptrs, SFB_ptrs, C_ptrs, stream, 1, kFmtNvfp4);
}

extern "C" int nvfp4_group_gemm_batched(int g, const int* M, const int* N, const int* K, const int* L,
                                        const void* const* A_ptrs, const void* const* B_ptrs,
                                        const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                        void* const* C_ptrs, void* stream)
{
    g_last_error.clear();
    if (g <= 0) return fail(NVFP4GG_INVALID_ARG, "g must be >= 1");
    if (!M || !N || !K || !L || !A_ptrs || !B_ptrs || !SFA_ptrs || !SFB_ptrs || !C_ptrs)
        return fail(NVFP4GG_INVALID_ARG, "a size or pointer array is NULL");
    // Every batch slice becomes a group of its own.
    std::vector<int> eM, eN, eK;
    std::vector<const void*> eA, eB, eSA, eSB;
    std::vector<void*> eC;
    for (int i = 0; i < g; ++i) {
        const std::string gs = "group " + std::to_string(i) + ": ";
        if (L[i] < 0 || M[i] < 0 || N[i] < 0 || K[i] < 0) return fail(NVFP4GG_INVALID_ARG, gs + "negative size");
        if (K[i] % 16 != 0) return fail(NVFP4GG_INVALID_ARG, gs + "K must be a multiple of 16");
        const int64_t a_bytes = (int64_t)M[i] * K[i] / 2, b_bytes = (int64_t)N[i] * K[i] / 2;
        const int64_t sa_bytes = (int64_t)M[i] * K[i] / 16, sb_bytes = (int64_t)N[i] * K[i] / 16;
        const int64_t c_bytes = (int64_t)M[i] * N[i] * 2;
        if (L[i] > 1 && ((a_bytes | b_bytes | sa_bytes | sb_bytes | c_bytes) & 15) != 0)
            return fail(NVFP4GG_UNSUPPORTED, gs + "a batch slice of an operand is not a multiple of 16 bytes, so "
                                                  "later slices would not be 16-byte aligned");
        for (int l = 0; l < L[i]; ++l) {
            eM.push_back(M[i]);
            eN.push_back(N[i]);
            eK.push_back(K[i]);
            eA.push_back(static_cast<const uint8_t*>(A_ptrs[i]) + l * a_bytes);
            eB.push_back(static_cast<const uint8_t*>(B_ptrs[i]) + l * b_bytes);
            eSA.push_back(static_cast<const uint8_t*>(SFA_ptrs[i]) + l * sa_bytes);
            eSB.push_back(static_cast<const uint8_t*>(SFB_ptrs[i]) + l * sb_bytes);
            eC.push_back(static_cast<uint8_t*>(C_ptrs[i]) + l * c_bytes);
        }
    }
    if (eM.empty()) return NVFP4GG_OK;
    return group_gemm_impl((int)eM.size(), eM.data(), eN.data(), eK.data(), eA.data(), eB.data(), eSA.data(),
                           eSB.data(), eC.data(), stream, 0, kFmtNvfp4);
}

extern "C" int mxfp4_group_gemm(int g, const int* M, const int* N, const int* K, const void* const* A_ptrs,
                                const void* const* B_ptrs, const void* const* SFA_ptrs,
                                const void* const* SFB_ptrs, void* const* C_ptrs, void* stream)
{
    return group_gemm_impl(g, M, N, K, A_ptrs, B_ptrs, SFA_ptrs, SFB_ptrs, C_ptrs, stream, 0, kFmtMxfp4);
}

extern "C" int nvfp4_dequant_f16(int rows, int K, const void* X, const void* SFX, void* out, void* stream)
{
    g_last_error.clear();
    if (rows < 0 || K < 0) return fail(NVFP4GG_INVALID_ARG, "negative size");
    if (K % 16 != 0) return fail(NVFP4GG_INVALID_ARG, "K must be a multiple of 16");
    if (rows == 0 || K == 0) return NVFP4GG_OK;
    if (!X || !SFX || !out || !aligned16(X) || !aligned16(SFX) || !aligned16(out))
        return fail(NVFP4GG_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
    const int64_t total = (int64_t)rows * ((K / 16 + 3) / 4);
    if (total > ((int64_t)1 << 31) - 256) return fail(NVFP4GG_UNSUPPORTED, "too many elements");
    const int nblk = (int)((total + 255) / 256);
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3(nblk), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       rows, K, static_cast<const uint8_t*>(X), static_cast<const uint8_t*>(SFX),
                       static_cast<h8_t*>(out));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return NVFP4GG_OK;
}
