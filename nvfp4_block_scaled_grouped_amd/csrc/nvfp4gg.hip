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
//   * Tile: one workgroup of 8 waves per CU owns all rows of A_i (up to 192,
//     in m-blocks of at most 6 fragments of 32 rows when M_i is larger) x 256
//     columns of B_i, so every byte of B_i is streamed from memory once per
//     m-block.  Wave w owns columns [32 w, 32 w + 32) for all rows of the
//     tile over the whole K.  A is shared: each stage of the tile's A rows is
//     dequantised once by the workgroup into LDS as fp16, already in MFMA
//     operand order, and the waves read it with 16-byte LDS loads.  B is
//     private to a wave: the four lanes of a B row load its 64 stage bytes as
//     one contiguous run straight into registers (kept two stages ahead)
//     and dequantise them there, so one dequantised B fragment feeds up to 12
//     MFMAs.
//   * K order: the sum over K is order-free.  A and B use the same order, so
//     every pair (a_k, b_k) meets in the same MFMA slot; it is chosen so that
//     each lane's 16 loaded bytes serve four k-steps.
//   * Accumulation: one fp32 chain per output over at most 8192 K of a
//     workgroup's segment; segments and chains are added in fp32 at the end.
//   * Schedule: the work is the list of (tile, stage) units (schedule.h) with
//     measured per-stage costs; a persistent grid of one workgroup per CU
//     takes equal-cost contiguous ranges of it, so ragged groups fill the
//     chip in one launch.  A tile whose stages span several workgroups is
//     finished by the first of them (whose range carries the tile's fix-up
//     cost): the others write their fp32 partial tiles to workspace slots
//     and count themselves in on the tile's counter; the first waits for
//     them (bounded; on time-out it hands the fix-up over to the last to
//     arrive), adds their partials to its own in workgroup order
//     (deterministic) and writes C.
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
constexpr int kKSteps = kStageK / 32;        // MFMA k-steps per stage (32 K each)
constexpr int kMaxAFrags = kMaxFrags;        // 16-row A fragments of a tile
constexpr int kMaxChainStages = 64;          // stages one fp32 chain accumulates (8192 K)
constexpr int kSlotFloats = kWaves * kMaxAFrags * 2 * kWave * 4;   // one partial tile
constexpr uint32_t kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kCoherent = 16;                  // cache-policy bit sc1: device-scope coherent access
constexpr int kWaitVmcnt0 = 0x0F70;            // s_waitcnt vmcnt(0) (expcnt, lgkmcnt not waited)
// A partial-slot offset past the end of every workspace (the host checks
// that the workspace stays below it): buffer loads there return zeros.
constexpr uint32_t kNoSlot = 0xF0000000u;
// Default bound on the first contributor's wait (polls of about a
// microsecond each).
constexpr int kWaitLimit = 1 << 20;

// Issue-order hints that interleave the B dequantisation with the MFMAs of
// each k-step (0 leaves the order to the compiler).
#ifndef NVFP4_INTERLEAVE
#define NVFP4_INTERLEAVE 1
#endif

#ifndef NVFP4_XCD_REMAP
#define NVFP4_XCD_REMAP 1
#endif

static_assert(kTileN == kWaves * 32, "each wave owns two 16-column B fragments");
static_assert(kMaxFrags == 12 && kFragRows == 16, "the kernel instantiates m-blocks of 1 to 12 fragments of 16 rows");
static_assert(kKSteps == 4, "a stage is one 16-byte piece of 4 k-steps per lane");

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
    float* partials;      // G * 2 slots of kSlotFloats
    int* counters;        // one per workgroup, zero between calls
    int64_t W;            // total cost
    int G;                // workgroups
    int ngroups;
    int blocked_sf;       // scales in the blocked (128 x 4 atom) layout, else row-major
    int wait_limit;       // polls of a tile's first contributor waiting for the others
    Bounds bounds;        // the workgroup boundaries of W over G (schedule.h)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             (int)kBufferFlags);
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

// Buffer loads at voffset (per lane) + soffset (wave-uniform, kept in an
// SGPR so per-stage offsets cost no vector registers).
__device__ __forceinline__ i4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}


// LDS image of the dequantised A rows of one stage, in MFMA operand order:
// [16-row fragment][k-step][lane] x 8 fp16 (48 KB).
struct AStage {
    h8_t v[kMaxAFrags][kKSteps][kWave];
};

// The workgroup's LDS: two A stages (dequantised fp16 for NVFP4, raw codes
// for MXFP4).  At the end of a segment the same
// memory carries the fp16 output tile on its way to C (rows padded by 16
// bytes against bank conflicts).
constexpr int kCTileStride = kTileN + 8;   // halves per LDS row of the output tile
// MXFP4 kernel: the raw A codes of a stage in MFMA operand order (16 bytes
// per lane per 16-row fragment) and each lane's E8M0 scale byte.
struct MxStage {
    i4_t v[kMaxAFrags][kWave];
    uint32_t s[kMaxAFrags][kWave];
};

// The segment a workgroup runs next (walk_range): computed by wave 0 and
// read by every wave.
struct WalkRec {
    int next;      // wave 0's walk: the next segment's cost position
    int end;       // wave 0's walk: the range's end
    Pos pos;
    int s_end;     // stages of the tile that start before the range's end
    int w_first;   // the tile's first contributor
    int w_last;    // the tile's last contributor
    int go;        // 0: the range is done
};

struct SharedMem {
    WalkRec walk;
    // The launch's group table, copied from the kernel arguments at entry
    // (walk_range): the walk and the segments read it from here.
    GroupSched sched[kMaxGroups];
    union {
        AStage a[2];
        MxStage mx[2];
        uint16_t ctile[kMaxFrags * kFragRows][kCTileStride];
    };
    // Target of the A pieces of waves with a unit past the tile's fragments
    // (their writes are discarded), so the k-step needs no branch.
    h8_t discard[kKSteps][kWave];
    // Per-wave staging of the scale bytes of 4 stages (two blocks in
    // flight): rows 0..31 are the wave's B rows, rows 32 + 16 x .. are its
    // A unit x's rows; 8 dwords per row (4 stages x 8 scale bytes).  A wave
    // loads a block with one 16-byte load per lane and redistributes it to
    // the lanes that need each dword through its own rows of this array.
    uint32_t sscr[2][kWaves][64][8];
};
static_assert(sizeof(SharedMem) <= 160 * 1024, "the LDS of one workgroup fits a CU");

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
// prefetched stages stay in flight), and the asm's memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// A zero accumulator written by opaque moves, so the compiler does not keep
// a zero constant alive across the persistent loop to copy from.
__device__ __forceinline__ f4_t zero_acc()
{
    f4_t z;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float v;
        asm volatile("v_mov_b32 %0, 0" : "=v"(v));
        z[e] = v;
    }
    return z;
}

// Piece (i, f) of the output tile, fp32 -> fp16 (round to nearest even,
// overflow to inf), into the LDS copy of the tile.  Wave w holds B fragments
// 2w, 2w + 1 (16 columns each): element r of lane (c16, kq) is tile row
// 16 i + c16, tile column 32 w + 16 f + 4 kq + r.
__device__ __forceinline__ void stage_c(SharedMem& sm, int i, int f, const f4_t& v, int wave, int lane)
{
    const int c16 = lane & 15, kq = lane >> 4;
    *reinterpret_cast<uint2*>(&sm.ctile[16 * i + c16][32 * wave + 16 * f + 4 * kq]) = pack4(v);
}

// The LDS copy of the output tile to C, every global store 16 contiguous
// bytes of a row.  Called by every thread of the workgroup once all pieces
// are staged; the LDS is free on return.
template <int NF>
__device__ __forceinline__ void write_c(SharedMem& sm, const GroupArgs& ga, int m0, int n0)
{
    const int tid = opaque_tid();
    lds_barrier();
    const int M = ga.M, N = ga.N;
    const int rows = M - m0 < NF * kFragRows ? M - m0 : NF * kFragRows;
    const int chunk = tid % (kTileN / 8);          // 8 columns = 16 bytes
    const int n = n0 + 8 * chunk;
    const bool vec_ok = (N & 7) == 0;
    for (int r = tid / (kTileN / 8); r < rows; r += kThreads / (kTileN / 8)) {
        if (n >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.ctile[r][8 * chunk]);
        uint16_t* dst = ga.C + (size_t)(m0 + r) * N + n;
        if (vec_ok && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
    lds_barrier();
}

// The output tile of the workgroup from the accumulators of its waves.
template <int NF>
__device__ __forceinline__ void store_c(SharedMem& sm, const GroupArgs& ga, int m0, int n0,
                                        const f4_t (*acc)[2], int wave)
{
    const int lane = opaque_tid() % kWave;
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f) stage_c(sm, i, f, acc[i][f], wave, lane);
    write_c<NF>(sm, ga, m0, n0);
}

// One wave's fp32 block of a partial tile (NF x 2 x 4 floats per lane) at
// base, in 1 KB lane-contiguous pieces.
template <int NF>
__device__ __forceinline__ void store_block(__amdgpu_buffer_rsrc_t r, uint32_t base, const f4_t (*acc)[2])
{
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i4_t, acc[i][f]), r,
                                                   base + (uint32_t)(2 * i + f) * (kWave * 16u), 0, kCoherent);
}

// acc += the block stored by store_block at base, kChunk pieces at a time
// (the scheduling barrier keeps the loads of later chunks from being
// hoisted, which bounds the registers in flight).
template <int NF>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t r, uint32_t base, f4_t (*acc)[2])
{
    constexpr int kPieces = 2 * NF;
    constexpr int kChunk = 12;
#pragma unroll
    for (int q0 = 0; q0 < kPieces; q0 += kChunk) {
        f4_t v[kChunk];
#pragma unroll
        for (int q = q0; q < q0 + kChunk && q < kPieces; ++q)
            v[q - q0] = __builtin_bit_cast(
                f4_t, __builtin_amdgcn_raw_buffer_load_b128(r, base + (uint32_t)q * (kWave * 16u), 0, kCoherent));
#pragma unroll
        for (int q = q0; q < q0 + kChunk && q < kPieces; ++q) acc[q >> 1][q & 1] += v[q - q0];
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The worker index of this workgroup.  Workgroups are dispatched round-robin
// over the XCDs (workgroup b runs on XCD b % kXcds), each with its own L2;
// numbering the workers XCD by XCD gives each XCD a contiguous range of the
// work order, so the tiles that share A rows (same group) or a B strip (same
// n-block) mostly meet in one L2.
__device__ __forceinline__ int worker_id(int G)
{
    const int b = blockIdx.x;
#if NVFP4_XCD_REMAP
    if (G % kXcds == 0) return (b % kXcds) * (G / kXcds) + b / kXcds;
#endif
    return b;
}

// Compiler fences: the asm takes the values as register operands (so they
// are computed before it) and clobbers memory (so no load or store moves
// across it).  Placed before a register is re-loaded, they keep the
// compiler from copying a value whose load is still in flight.
template <typename T>
__device__ __forceinline__ void fence_after(const T& v)
{
    asm volatile("" ::"v"(v) : "memory");
}

// The two E4M3 scale bytes at bits [shift, shift + 16) of a dword -> fp16.
__device__ __forceinline__ h2_t scales2(uint32_t sc, uint32_t shift)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc >> shift, 1.0f, false);
}

// Stages J .. L-1 of an unrolled pass: f(slot J % R, phase J % 4, i + J),
// all of them, or (the tail) those below n.
template <int J, int L, int R, class F>
__device__ __forceinline__ void phase_pass(F& f, int i)
{
    if constexpr (J < L) {
        f(Parity<J % R>{}, Parity<J % 4>{}, i + J);
        phase_pass<J + 1, L, R>(f, i);
    }
}

template <int J, int L, int R, class F>
__device__ __forceinline__ void phase_tail(F& f, int i, int n)
{
    if constexpr (J < L) {
        if (i + J < n) {
            f(Parity<J % R>{}, Parity<J % 4>{}, i + J);
            phase_tail<J + 1, L, R>(f, i, n);
        }
    }
}

// The end of a segment: chains of one segment meet in the scratch slot; the
// last chain finishes the tile alone, or as one of several contributors
// (partial-tile store, counter, and the fix-up by the last to arrive).
// acc holds the wave's part of the segment's sum: acc[i][f] element r of lane
// (c16, kq) is tile row 16 i + c16, column 32 wave + 16 f + 4 kq + r.
template <int NF>
__device__ __forceinline__ void finish_segment(const LaunchArgs& args, const Pos& pos, bool first_chain,
                                               bool last_chain, SharedMem& sm, int* s_flag, f4_t (*acc)[2],
                                               int m0, int n0, int wave)
{
    const GroupArgs& ga = args.grp[pos.group];
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(args.partials, (uint32_t)(kSlotsPerWG * args.G) * kSlotFloats * 4u);
    // Epilogue addresses, recomputed here rather than kept through the loop.
    const uint32_t ewave_in_slot =
        (uint32_t)wave * (kMaxAFrags * 2) * (kWave * 16u) + (uint32_t)(opaque_tid() % kWave) * 16u;
    const uint32_t scratch_base =
        (uint32_t)scratch_slot(worker_id(args.G)) * kSlotFloats * 4u + ewave_in_slot;
    // Chains of one segment meet in the scratch slot.
    if (!first_chain) load_block<NF>(rP, scratch_base, acc);
    if (!last_chain) {
        store_block<NF>(rP, scratch_base, acc);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        return;
    }

    // Finish the tile: alone, or as one of several contributors.  Every
    // wave holds its part of the segment's sum in acc.  The tile's
    // contributors come from walk_range's record of this segment (rewritten
    // only after the barriers below).
    const int w_first = __builtin_amdgcn_readfirstlane(sm.walk.w_first);
    const int w_last = __builtin_amdgcn_readfirstlane(sm.walk.w_last);
    if (w_first == w_last) {
        asm volatile("; whole tile" ::: "memory");   // keeps this store_c apart from the fix-up's
        store_c<NF>(sm, ga, m0, n0, acc, wave);
        return;
    }
    const int me = __builtin_amdgcn_readfirstlane(worker_id(args.G));
    int* counter = args.counters + counter_index(w_first);
    // Partial tile -> this workgroup's slot (partial_slot).
    auto slot_base = [&](int w) {
        return (uint32_t)partial_slot(w, w_last) * kSlotFloats * 4u + ewave_in_slot;
    };
    // Who finishes the tile.  The first contributor's range ends with the
    // tile's first stages and carries the tile's start-up and wind-down cost
    // (tile_cost), so it should: it claims the fix-up and waits for the
    // others, a bounded number of polls (all workgroups of the grid run at
    // once when it fits the chip, so the others are running and never wait
    // themselves).  The others store their partials and count themselves in.
    // If the wait runs out, the first contributor stores its partial too and
    // swaps its claim for a hand-over, and whoever then completes the count
    // finishes the tile: exactly one workgroup does, and nobody waits
    // unboundedly.
    //
    // Memory ordering.  Every value that passes between workgroups here (the
    // partials and the counter) moves by agent-scope coherent accesses: the
    // partial stores and loads carry the sc1 cache-policy bit, which is how
    // gfx950 performs agent-scope relaxed atomic stores and loads (they write
    // through to, and read from, the level that all XCDs share), and the
    // counter operations are agent-scope atomics.  A contributor's waves wait
    // until their partial stores have completed (s_waitcnt vmcnt(0)) before
    // the workgroup barrier after which thread 0 adds to the counter, so the
    // partials are in the shared level before the add is performed.  The
    // finisher's thread 0 has the counter value back (the loop waits for it)
    // before the barrier after which its waves issue their partial loads, so
    // those loads are performed after the last add and read the stored
    // values.  Release and acquire orderings would add what these accesses do
    // not need: a write-back of the XCD's whole L2 before each add and an
    // invalidation of it after each poll, which drops the B strips that the
    // other workgroups of the XCD share (measured: up to 2x slower calls).
    const int others = w_last - w_first;
    bool fix;
    if (me != w_first) {
        store_block<NF>(rP, slot_base(me), acc);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int old =
                __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_flag = other_finishes(old, others) ? 1 : 0;
        }
        __syncthreads();
        fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
        __syncthreads();   // s_flag is reused below and by the next segment
    } else {
        if (threadIdx.x == 0) {
            const int old =
                __hip_atomic_fetch_add(counter, kClaim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int done = first_finishes(old, others);
            for (int poll = 0; !done && poll < args.wait_limit; ++poll) {
                __builtin_amdgcn_s_sleep(2);
                done = first_finishes(
                    __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), others);
            }
            *s_flag = done;
        }
        __syncthreads();
        fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
        __syncthreads();
        if (!fix) {
            store_block<NF>(rP, slot_base(me), acc);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (threadIdx.x == 0) {
                const int old = __hip_atomic_fetch_add(counter, kHandOver - kClaim, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                *s_flag = first_finishes(old, others);   // the count completed meanwhile: still ours
            }
            __syncthreads();
            fix = __builtin_amdgcn_readfirstlane(*s_flag) != 0;
            __syncthreads();
        }
    }
    if (!fix) return;
    // Sum the contributors' partials in workgroup order, so the result does
    // not depend on who arrived last.  Loads carry the device-scope
    // coherence bit; a contributor index past w_last gets an offset beyond
    // the buffer, whose loads return zeros.
    constexpr int kPieces = 2 * NF;
    auto load_piece = [&](int w, int q) {
        const uint32_t base = w <= w_last ? slot_base(w) : kNoSlot;
        return __builtin_bit_cast(
            f4_t, __builtin_amdgcn_raw_buffer_load_b128(rP, base + (uint32_t)q * (kWave * 16u), 0, kCoherent));
    };
    if (me == w_first) {
        // This workgroup's partial is still in the accumulators (often the
        // case: the first contributor ends its range with the tile's first
        // stages, so it tends to finish last); the others are added to it,
        // kChunk pieces of kBatch contributors in flight.  Tiles of 7 or more
        // fragments take one contributor at a time (in two halves for 11 and
        // 12 fragments): their accumulators hold the registers.
        constexpr int kChunk = NF <= 10 ? kPieces : kPieces / 2;
        constexpr int kBatch = NF <= 6 ? 24 / kChunk : 1;
        for (int w0 = w_first + 1; w0 <= w_last; w0 += kBatch) {
#pragma unroll
            for (int q0 = 0; q0 < kPieces; q0 += kChunk) {
                f4_t v[kBatch][kChunk];
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
#pragma unroll
                    for (int q = 0; q < kChunk && q0 + q < kPieces; ++q) v[b][q] = load_piece(w0 + b, q0 + q);
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
#pragma unroll
                    for (int q = 0; q < kChunk && q0 + q < kPieces; ++q)
                        acc[(q0 + q) >> 1][(q0 + q) & 1] += v[b][q];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        asm volatile("; fix-up, first contributor" ::: "memory");
        store_c<NF>(sm, ga, m0, n0, acc, wave);
    } else {
        // Every partial, this workgroup's own included, is read back, so the
        // accumulators are free: kChunk pieces of kBatch contributors in
        // flight, each summed chunk straight to the LDS copy of the tile.
        constexpr int kChunk = NF <= 6 ? kPieces : (kPieces + 1) / 2;
        constexpr int kBatch = (NF <= 4 ? 32 : 24) / kChunk;
        const int flane = opaque_tid() % kWave;
#pragma unroll
        for (int q0 = 0; q0 < kPieces; q0 += kChunk) {
            f4_t sum[kChunk];
#pragma unroll
            for (int q = 0; q < kChunk; ++q) sum[q] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            for (int w0 = w_first; w0 <= w_last; w0 += kBatch) {
                f4_t v[kBatch][kChunk];
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
#pragma unroll
                    for (int q = 0; q < kChunk && q0 + q < kPieces; ++q) v[b][q] = load_piece(w0 + b, q0 + q);
#pragma unroll
                for (int b = 0; b < kBatch; ++b)
#pragma unroll
                    for (int q = 0; q < kChunk && q0 + q < kPieces; ++q) sum[q] += v[b][q];
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < kChunk && q0 + q < kPieces; ++q)
                stage_c(sm, (q0 + q) >> 1, (q0 + q) & 1, sum[q], wave, flane);
        }
        asm volatile("; fix-up" ::: "memory");
        write_c<NF>(sm, ga, m0, n0);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// One chain [s_begin, s_end) of the stages of a tile of NA fragments of 16
// rows: a
// workgroup's segment of a tile runs as chains of at most kMaxChainStages
// stages (one chain for any K <= 8192); first_chain / last_chain place this
// chain in its segment.
//
// MFMA: v_mfma_f32_16x16x32_f16 with B as the first operand (16 columns of
// B_i) and A as the second (16 rows of A_i).  Lane (c16, kq) = (lane % 16,
// lane / 16) supplies column / row c16 and 8 codes of K; it gets back rows
// 4 kq .. 4 kq + 3 of the first operand's side, i.e. output row c16 and
// output columns 4 kq .. 4 kq + 3 of the 16 x 16 block.
//
// Waves: wave w owns columns [32 w, 32 w + 32) of the tile (B fragments
// f = 0, 1 of 16 columns) for all NA 16-row A fragments, over the whole K
// of the chain, so every byte of B is loaded and dequantised once per tile,
// by one wave, and one dequantised B fragment feeds NA MFMAs.
//
// K order within a stage (128 K, 64 bytes of a row; the sum is order-free
// and A and B use the same order): at k-step v lane (c16, kq) holds the 8
// codes at K 32 kq + 8 v, i.e. dword v of the 16 bytes [16 kq, +16) of the
// row's stage bytes, whose scale block is 2 kq + v / 2 (scale bytes
// 2 (kq % 2), + 1 of dword kq / 2 of the row's 8 stage scale bytes).  So the
// four lanes of a row read its 64 stage bytes as one contiguous run, and
// one 16-byte load per B fragment and stage feeds all four k-steps.
//
// A: each stage of the tile's NA fragments of 16 rows is dequantised once
// by the workgroup into LDS, in operand order.  Fragment a belongs to wave
// a % 8 (its unit a / 8), so a wave has at most two units.
//
// Pipeline, per stage i of the chain (register ring slot p = i % kRing):
//   * B of stage i is in bq[p], bs[p] (loaded kRing stages earlier); it is
//     re-loaded with stage i + kRing once its last k-step is dequantised.
//   * A of stage i is in LDS buffer i % 2.  The raw A of stage i + 1 (aq[p],
//     as[p], loaded kRing stages earlier) is dequantised into the other
//     buffer, one piece per k-step of the MFMA loop, then re-loaded with
//     stage i + 1 + kRing.
//   * One LDS-only barrier ends the stage.
template <int NA, bool kBlocked>
__device__ __forceinline__ void run_segment(const LaunchArgs& args, const Pos& pos, int s_begin, int s_end,
                                            bool first_chain, bool last_chain, SharedMem& sm, int* s_flag)
{
    const GroupSched& gs = sm.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const int tid = opaque_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int lane = tid % kWave;
    const int c16 = lane & 15;
    const int kq = lane >> 4;
    const int M = ga.M, N = ga.N, K = ga.K;
    const int m0 = mblock_first_frag(__builtin_amdgcn_readfirstlane(gs.frags), __builtin_amdgcn_readfirstlane(gs.mblocks), pos.mb) * kFragRows;
    const int n0 = pos.nb * kTileN;
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 16;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(ga.B, (uint32_t)N * row_bytes);
    // Blocked scales: rows padded to a multiple of 128 (the layout's atoms
    // are 128 rows x 4 scales; K / 16 is a multiple of 8 here).
    constexpr bool blocked = kBlocked;
    const uint32_t sf_rows_a = blocked ? (uint32_t)(M + 127) & ~127u : (uint32_t)M;
    const uint32_t sf_rows_b = blocked ? (uint32_t)(N + 127) & ~127u : (uint32_t)N;
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(ga.SFA, sf_rows_a * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(ga.SFB, sf_rows_b * row_scales);
    const uint32_t sshift = 16u * (uint32_t)(kq & 1);   // this lane's scale bytes within a dword

    // B operand of lane (c16, kq) in fragment f: row n0 + 32 wave + 16 f + c16
    // (rows past N read 0).
    uint32_t offB[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const uint32_t brow = (uint32_t)(n0 + 32 * wave + 16 * f + c16);
        offB[f] = brow * row_bytes + 16u * kq;
    }

    // This wave's A units: kU = 1 for NA <= 8, else 2 (unit x is fragment
    // a = w + 8 x).  A unit past the tile's fragments (a >= NA) loads the
    // rows of fragment a % NA again (cache hits) and writes the discard
    // area.
    constexpr int kU = NA > kWaves ? 2 : 1;
    // Register ring depth: stage i's loads go out kRing stages ahead.
    // (Measured on MI355X: rings of 1, 2 and 4 stages time the same; the
    // stage is bound by its issue, not by the load latency.)
    constexpr int kRing = 2;
    static_assert(4 % kRing == 0, "the ring depth divides the 4-stage scale block");
    uint32_t offA[2];
    h8_t* adst[2];          // k-step 0 of the unit's fragment in LDS buffer 0
    uint32_t abuf_step[2];  // bytes from buffer 0 to buffer 1 (0 for the discard area)
#pragma unroll
    for (int x = 0; x < kU; ++x) {
        const int a = wave + kWaves * x;
        const bool real = a < NA;
        const uint32_t arow = (uint32_t)(m0 + 16 * (a % NA) + c16);   // rows past M read 0
        offA[x] = arow * row_bytes + 16u * kq;
        adst[x] = real ? &sm.a[0].v[a][0][lane] : &sm.discard[0][lane];
        abuf_step[x] = real ? (uint32_t)sizeof(AStage) : 0u;
    }

    f4_t acc[NA][2];

    {
        const int n = s_end - s_begin;
        // Stage offsets (wave-uniform, in SGPRs); stages past the chain
        // re-read its last stage, so every load is unconditional and in range.
        auto sbyte = [&](int t) {
            return (uint32_t)__builtin_amdgcn_readfirstlane((s_begin + (t < n ? t : n - 1)) * (kStageK / 2));
        };

        i4_t bq[kRing][2];
        i4_t aq[kRing][2];

        // Scale staging: lane L loads 16 bytes (2 stages) of the scale row
        // L / 2 of the wave (B rows, then each A unit's 16 rows) for a block of
        // 4 stages, and writes them to its rows of sm.sscr.  Only the wave
        // itself reads its rows, and a wave's LDS accesses complete in issue
        // order, so no barrier guards them.  A block that runs past the end
        // of K reads the next row's bytes or, past the buffer, zeros; the
        // stages that would use them do not exist.
        //
        // Row-major scales: the 16 bytes are contiguous.  Blocked scales
        // (the 128 x 4 atom layout): scale column c of row r is byte
        // 512 ((r / 128) (K / 64) + c / 4) + 16 (r % 32) + 4 ((r / 32) % 4)
        // + c % 4, so the 16 bytes are four 4-byte runs (scale columns
        // 4q .. 4q + 3 of consecutive atoms), 512 bytes apart.
        const int slane = lane;
        auto sf_off = [&](int r) {
            return blocked ? (uint32_t)(r >> 7) * (uint32_t)K * 8u + (uint32_t)(r & 31) * 16u +
                                 (uint32_t)((r >> 5) & 3) * 4u + 2048u * (slane & 1)
                           : (uint32_t)r * row_scales + 16u * (slane & 1);
        };
        const uint32_t offSBs = sf_off(n0 + 32 * wave + (slane >> 1));
        uint32_t offSAs[2];
#pragma unroll
        for (int x = 0; x < kU; ++x) {
            const int a = wave + kWaves * x;
            offSAs[x] = sf_off(m0 + 16 * (a % NA) + ((slane >> 1) & 15));
        }
        // Offset of the block starting at stage b of the chain: 8 scale
        // bytes per stage, in row-major scales one atom (512 bytes) per 4
        // scale columns in blocked ones.
        auto sblock = [&](int b) {
            return (uint32_t)__builtin_amdgcn_readfirstlane((s_begin + b) * (blocked ? 1024 : kStageK / 16));
        };
        auto sload = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
            if (!blocked) return load16(r, voff, soff);
            i4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 512u * j, soff, 0);
            return v;
        };
        // The block offset goes into the per-lane offset, which the buffer's
        // range check covers (the scalar offset is not checked): a block
        // that runs past the end of the last row reads zeros there.
        i4_t sregB, sregA[2];
        auto scale_load = [&](int b) {
            sregB = sload(rSB, offSBs + sblock(b), 0);
#pragma unroll
            for (int x = 0; x < kU; ++x) sregA[x] = sload(rSA, offSAs[x] + sblock(b), 0);
        };
        auto scale_store = [&](int buf) {
            *reinterpret_cast<i4_t*>(&sm.sscr[buf][wave][slane >> 1][4 * (slane & 1)]) = sregB;
#pragma unroll
            for (int x = 0; x < kU; ++x)
                *reinterpret_cast<i4_t*>(&sm.sscr[buf][wave][32 + 16 * x + ((slane >> 1) & 15)][4 * (slane & 1)]) =
                    sregA[x];
        };
        // The scale dword of this lane for stage t of the chain: B fragment f,
        // or A unit x.
        auto scale_b = [&](int t, int f) {
            return sm.sscr[(t >> 2) & 1][wave][16 * f + c16][2 * (t & 3) + (kq >> 1)];
        };
        auto scale_a = [&](int t, int x) {
            return sm.sscr[(t >> 2) & 1][wave][32 + 16 * x + c16][2 * (t & 3) + (kq >> 1)];
        };

        // Prologue: raw A of stage 0, then ring slot j < kRing (B of stage j,
        // raw A of stage j + 1), in the order the stages issue their loads;
        // stage 0 of A into LDS buffer 0.
        {
            i4_t a0[2];
            scale_load(0);
#pragma unroll
            for (int x = 0; x < kU; ++x) a0[x] = load16(rA, offA[x], sbyte(0));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kRing; ++j) {
#pragma unroll
                for (int f = 0; f < 2; ++f) bq[j][f] = load16(rB, offB[f], sbyte(j));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int x = 0; x < kU; ++x) aq[j][x] = load16(rA, offA[x], sbyte(j + 1));
                __builtin_amdgcn_sched_barrier(0);
            }
            scale_store(0);
#pragma unroll
            for (int x = 0; x < kU; ++x) {
                const h2_t sa = scales2(scale_a(0, x), sshift);
#pragma unroll
                for (int v = 0; v < kKSteps; ++v) adst[x][v * kWave] = dequant8((uint32_t)a0[x][v], sa[v >> 1]);
            }
        }
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[i][f] = zero_acc();
        lds_barrier();

        // Stage i of the chain, at ring slot p = i % kRing and scale-block
        // phase q = i % 4, both known at compile time (the loop below is
        // unrolled by 4), so the stage has no branch: a branch here would
        // make the compiler's wait counts at its join conservative, which
        // drains the load ring.
        auto stage = [&](auto parity, auto phase, int i) {
            constexpr int p = decltype(parity)::value;
            constexpr int q = decltype(phase)::value;
            const uint32_t sb2 = sbyte(i + kRing);
            const uint32_t sb3 = sbyte(i + 1 + kRing);
            // LDS A buffers: this stage reads buffer i % 2 and writes the other.
            const int lb = i & 1;
            const AStage& ard = sm.a[lb];
            h8_t* awr[2];
#pragma unroll
            for (int x = 0; x < kU; ++x)
                awr[x] = reinterpret_cast<h8_t*>(reinterpret_cast<char*>(adst[x]) + (lb ^ 1) * abuf_step[x]);
            // Scales of this stage (B) and of the A being dequantised
            // (stage i + 1, or this one past the chain's end), from the
            // staging array.  Block b + 1's scales go out at the first stage
            // of block b and are staged at its third stage, before the A of
            // its first stage needs them.
            const int ia = i + 1 < n ? i + 1 : i;
            const h2_t sbf[2] = {scales2(scale_b(i, 0), sshift), scales2(scale_b(i, 1), sshift)};
            h2_t saf[2];
#pragma unroll
            for (int x = 0; x < kU; ++x) saf[x] = scales2(scale_a(ia, x), sshift);
            // Past the chain's end these read bytes never used (zeros past
            // the buffer) and fill a staging buffer nobody reads.
            if constexpr (q == 0) scale_load(i + 4);
            if constexpr (q == 2) scale_store(((i >> 2) + 1) & 1);

            // k-step pipeline: the B dequant of k-step v + 1 is issued before
            // the MFMAs of k-step v; the scheduling barrier at the end of each
            // k-step keeps the compiler from hoisting work across k-steps.
            h8_t bv[2] = {dequant8((uint32_t)bq[p][0][0], sbf[0][0]), dequant8((uint32_t)bq[p][1][0], sbf[1][0])};
            // Raised priority from the first dequantised B piece to the
            // barrier: a wave inside its k-steps issues ahead of one that is
            // still waiting at the stage's start (measured: 12-fragment tiles
            // about 5% faster, g8 K2048 N7168 about 2%).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int v = 0; v < kKSteps; ++v) {
                h8_t av[NA];
#pragma unroll
                for (int a = 0; a < NA; ++a) av[a] = ard.v[a][v][lane];
                h8_t nbv[2] = {bv[0], bv[1]};
                if (v + 1 < kKSteps) {
#pragma unroll
                    for (int f = 0; f < 2; ++f)
                        nbv[f] = dequant8((uint32_t)bq[p][f][v + 1], sbf[f][(v + 1) >> 1]);
                }
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int f = 0; f < 2; ++f)
                        acc[a][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[f], av[a], acc[a][f], 0, 0, 0);
                // Piece v of each A unit of stage i + 1 -> the other LDS buffer.
#pragma unroll
                for (int x = 0; x < kU; ++x)
                    awr[x][v * kWave] = dequant8((uint32_t)aq[p][x][v], saf[x][v >> 1]);
                if (v == kKSteps - 2) {
                    // B is fully dequantised (the last k-step is in nbv).
                    fence_after(nbv[0]);
                    fence_after(nbv[1]);
#pragma unroll
                    for (int f = 0; f < 2; ++f) bq[p][f] = load16(rB, offB[f], sb2);
                }
                if (v == kKSteps - 1) {
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int x = 0; x < kU; ++x) aq[p][x] = load16(rA, offA[x], sb3);
                }
                bv[0] = nbv[0];
                bv[1] = nbv[1];
#if NVFP4_INTERLEAVE
                // Issue order: the A operands are read from LDS a few MFMAs
                // ahead of their use (so few are live at once), and the MFMAs
                // alternate with the VALU work, so the dequantisation runs
                // while the matrix core is busy.
                constexpr int kLead = NA <= 8 ? NA : 8;   // A operands read ahead of their MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);   // LDS reads
#pragma unroll
                for (int g = 0; g < 2 * NA; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // up to two VALU
                    if ((g & 1) && (g >> 1) + kLead < NA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#endif
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
        };

        int i = 0;
        for (; i + 3 < n; i += 4) phase_pass<0, 4, kRing>(stage, i);
        phase_tail<0, 4, kRing>(stage, i, n);
    }
    finish_segment<NA>(args, pos, first_chain, last_chain, sm, s_flag, acc, m0, n0, wave);
}

// ------------------------------------------------------------------ MXFP4
//
// MXFP4 operands: the same packed E2M1 codes, with one E8M0 scale (the value
// 2^(code - 127)) per 32 consecutive K of a row, row-major M x K/32 and
// N x K/32 bytes.  gfx950's block-scaled MFMA takes this form as it is:
// v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands (format code 4)
// multiplies each lane's 32 codes by that lane's E8M0 scale.  Lane (c16, kq)
// supplies row c16 of an operand fragment and K = 32 kq .. 32 kq + 31 of the
// 128-K step, which are bytes 16 kq .. 16 kq + 15 of the row's 64 bytes of
// the stage, in the natural nibble order; its scale is byte 4 s + kq of the
// row's scales at stage s.  No dequantisation, one MFMA per fragment pair
// per stage.
using v8i_t = int __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4_t mfma_mx(i4_t b, uint32_t sb, i4_t a, uint32_t sa, f4_t c)
{
    const v8i_t bv = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    const v8i_t av = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    // src0 = B fragment (output columns), src1 = A fragment (output rows),
    // both FP4; scale byte 0 of each scale register.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av, c, 4, 4, 0, (int)sb, 0, (int)sa);
}

// One segment of an MXFP4 tile (same tile shape, schedule, wave layout and
// end of segment as run_segment):
//   * B: each lane loads 16 bytes of its row per stage (the MFMA operand as
//     it is), kRing stages ahead in a register ring.
//   * A: wave w loads fragment w (and w + 8 for more than 8 fragments) the
//     same way, one stage ahead of its use, and stores it with its scale
//     bytes into a double-buffered LDS stage that every wave reads.
//   * Scales: one 16-byte load per lane per block of 4 stages, staged
//     through the wave's rows of LDS (a byte load per fragment and stage
//     kept the texture address unit's queue full: measured 6x the full
//     cycles of the NVFP4 kernel).
//   * Per stage each wave runs 2 x NA MFMAs of 16 x 16 x 128; one LDS-only
//     barrier ends the stage.
template <int NA>
__device__ __forceinline__ void run_segment_mx(const LaunchArgs& args, const Pos& pos, int s_begin, int s_end,
                                               bool first_chain, bool last_chain, SharedMem& sm, int* s_flag)
{
    constexpr int kU = NA > kWaves ? 2 : 1;
    // Stages of B in flight.  Measured on MI355X: 2 beats 4 and 4 beats 8
    // on every workload (a deeper ring's first burst of loads delays every
    // workgroup's first stage by several us, and one stage ahead already
    // covers the load latency: a ring of 1 times the same as 2); depths of 6
    // and 3 compiled to loops whose wait counts drained the ring every pass.
    constexpr int kRing = 2;
    // A fragments read from LDS per group (the scheduling barrier between
    // groups keeps the compiler from loading every fragment of the stage up
    // front, which large tiles have no registers for).
    constexpr int kAGroup = NA <= 8 ? NA : 4;
    const GroupSched& gs = sm.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const int tid = opaque_tid();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int c16 = lane & 15;
    const int kq = lane >> 4;
    const int M = ga.M, N = ga.N, K = ga.K;
    const int m0 = mblock_first_frag(__builtin_amdgcn_readfirstlane(gs.frags), __builtin_amdgcn_readfirstlane(gs.mblocks), pos.mb) * kFragRows;
    const int n0 = pos.nb * kTileN;
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 32;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(ga.B, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(ga.SFA, (uint32_t)M * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(ga.SFB, (uint32_t)N * row_scales);

    // Rows past M or N are beyond the buffers and read zeros.
    uint32_t offB[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) offB[f] = (uint32_t)(n0 + 32 * wave + 16 * f + c16) * row_bytes + 16u * kq;
    uint32_t offA[2];
#pragma unroll
    for (int x = 0; x < kU; ++x)
        offA[x] = (uint32_t)(m0 + 16 * ((wave + kWaves * x) % NA) + c16) * row_bytes + 16u * kq;
    // Scale staging, as in the NVFP4 kernel: lane L loads the 16 scale bytes
    // (4 stages x 4) of one row for a block of 4 stages and writes them to
    // row L of the wave's part of sm.sscr: rows 0..31 are the wave's B rows,
    // rows 32 + 16 x .. its A unit x's rows (with one unit, lanes 48..63 load
    // unit 0's rows again, into the same place).  Only the wave itself reads
    // its rows, and a wave's LDS accesses complete in order, so no barrier
    // guards them.  A block that runs past the end of K reads the next row's
    // bytes or, past the buffer, zeros; the stages that would use them do not
    // exist.  Lane (c16, kq) takes scale byte kq of its row's stage dword.
    // Every lane issues the block's load from both scale arrays, the one it
    // does not use at an offset past the array (which reads zeros), so each
    // load's buffer descriptor is the same for the whole wave.
    const bool sa_lane = lane >= 32;
    const int sx = kU == 2 ? (lane >> 4) & 1 : 0;
    const int srow = sa_lane ? 32 + 16 * sx + (lane & 15) : lane;
    const uint32_t offSBl = sa_lane ? kNoSlot : (uint32_t)(n0 + 32 * wave + lane) * row_scales;
    const uint32_t offSAl =
        sa_lane ? (uint32_t)(m0 + 16 * ((wave + kWaves * sx) % NA) + (lane & 15)) * row_scales : kNoSlot;
    const uint32_t kshift = 8u * (uint32_t)kq;

    f4_t acc[NA][2];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = zero_acc();

    {
        const int n = s_end - s_begin;
        // Stage offsets in a row of codes; stages past the chain repeat its
        // last stage (loaded, never used).
        auto sbyte = [&](int t) {
            return (uint32_t)__builtin_amdgcn_readfirstlane((s_begin + (t < n ? t : n - 1)) * (kStageK / 2));
        };
        // A stores of waves whose unit is past the tile's fragments go to a
        // discard area, so the stage has no branch (a branch would let the
        // compiler sink each stage's MFMAs into later blocks).
        i4_t* vdst[2];
        uint32_t* sdst[2];
        uint32_t mstep[2];
#pragma unroll
        for (int x = 0; x < kU; ++x) {
            const int a = wave + kWaves * x;
            const bool real = a < NA;
            vdst[x] = real ? &sm.mx[0].v[a][lane] : reinterpret_cast<i4_t*>(&sm.discard[0][0]) + lane;
            sdst[x] = real ? &sm.mx[0].s[a][lane]
                           : reinterpret_cast<uint32_t*>(reinterpret_cast<i4_t*>(&sm.discard[0][0]) + kWave) + lane;
            mstep[x] = real ? (uint32_t)sizeof(MxStage) : 0u;
        }
        auto put_a = [&](int buf, int x, i4_t v, uint32_t sc) {
            *reinterpret_cast<i4_t*>(reinterpret_cast<char*>(vdst[x]) + buf * mstep[x]) = v;
            *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(sdst[x]) + buf * mstep[x]) = sc;
        };

        // The scale block starting at stage b of the chain (4 bytes per stage),
        // in the per-lane offset, which the buffer's range check covers.
        auto sblock = [&](int b) { return (uint32_t)__builtin_amdgcn_readfirstlane((s_begin + b) * (kStageK / 32)); };
        // The two halves are combined only where the block is staged, so the
        // loads are waited for there (combined at the load, the wait would
        // drain every load in flight).
        i4_t sregB, sregA;
        auto scale_load = [&](int b) {
            const uint32_t sb = sblock(b);
            sregB = __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(rSB, offSBl + sb, 0, 0));
            sregA = __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(rSA, offSAl + sb, 0, 0));
        };
        auto scale_store = [&](int buf) {
            *reinterpret_cast<i4_t*>(&sm.sscr[buf][wave][srow][0]) = sregB | sregA;
        };
        // The E8M0 byte of this lane for stage t of the chain: B fragment f,
        // or A unit x (the MFMA reads byte 0 of the scale operand).
        auto scale_b = [&](int t, int f) { return sm.sscr[(t >> 2) & 1][wave][16 * f + c16][t & 3] >> kshift; };
        auto scale_a = [&](int t, int x) { return sm.sscr[(t >> 2) & 1][wave][32 + 16 * x + c16][t & 3] >> kshift; };

        i4_t bq[kRing][2], aq[kRing][2];
        {
            i4_t a0[2];
            scale_load(0);
#pragma unroll
            for (int x = 0; x < kU; ++x) a0[x] = load16(rA, offA[x], sbyte(0));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kRing; ++j) {
#pragma unroll
                for (int f = 0; f < 2; ++f) bq[j][f] = load16(rB, offB[f], sbyte(j));
#pragma unroll
                for (int x = 0; x < kU; ++x) aq[j][x] = load16(rA, offA[x], sbyte(j + 1));
                __builtin_amdgcn_sched_barrier(0);
            }
            scale_store(0);
#pragma unroll
            for (int x = 0; x < kU; ++x) put_a(0, x, a0[x], scale_a(0, x));
        }
        lds_barrier();

        // Stage i of the chain at ring slot p = i % kRing and scale-block phase
        // q = i % 4, both known at compile time (the loop is unrolled by 4).
        auto stage = [&](auto parity, auto phase, int i) {
            constexpr int p = decltype(parity)::value;
            constexpr int q = decltype(phase)::value;
            const int lb = i & 1;
            const uint32_t sbv[2] = {scale_b(i, 0), scale_b(i, 1)};
            // The A scale of stage i + 1 (or this one past the chain's end).
            const int ia = i + 1 < n ? i + 1 : i;
            uint32_t sav[2];
#pragma unroll
            for (int x = 0; x < kU; ++x) sav[x] = scale_a(ia, x);
            // Block b + 1's scales go out at the first stage of block b and
            // are staged at its third stage, before the A of its last stage
            // needs them.
            if constexpr (q == 0) scale_load(i + 4);
            if constexpr (q == 2) scale_store(((i >> 2) + 1) & 1);
#pragma unroll
            for (int a0 = 0; a0 < NA; a0 += kAGroup) {
#pragma unroll
                for (int a = a0; a < a0 + kAGroup && a < NA; ++a) {
                    const i4_t av = sm.mx[lb].v[a][lane];
                    const uint32_t sa = sm.mx[lb].s[a][lane];
#pragma unroll
                    for (int f = 0; f < 2; ++f) acc[a][f] = mfma_mx(bq[p][f], sbv[f], av, sa, acc[a][f]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // A of stage i + 1 into the other buffer (its readers of stage
            // i - 1 passed the previous barrier), then the ring slot's
            // reloads: B of stage i + kRing, A of stage i + 1 + kRing.
#pragma unroll
            for (int x = 0; x < kU; ++x) put_a(lb ^ 1, x, aq[p][x], sav[x]);
            // The slot's old values are consumed before its reloads are
            // issued, so the reloads can take the same registers (otherwise
            // the compiler copies ring values whose loads are in flight and
            // waits for them).
#pragma unroll
            for (int f = 0; f < 2; ++f) fence_after(bq[p][f]);
#pragma unroll
            for (int x = 0; x < kU; ++x) fence_after(aq[p][x]);
#pragma unroll
            for (int f = 0; f < 2; ++f) bq[p][f] = load16(rB, offB[f], sbyte(i + kRing));
#pragma unroll
            for (int x = 0; x < kU; ++x) aq[p][x] = load16(rA, offA[x], sbyte(i + 1 + kRing));
            lds_barrier();
        };
        int i = 0;
        for (; i + 3 < n; i += 4) phase_pass<0, 4, kRing>(stage, i);
        phase_tail<0, 4, kRing>(stage, i, n);
    }
    finish_segment<NA>(args, pos, first_chain, last_chain, sm, s_flag, acc, m0, n0, wave);
}

// Wave-uniform values computed in vector registers (divisions and LDS reads
// have no scalar form) moved back to scalar registers, so they do not occupy
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

// The segment kernel of a tile of `frags` fragments (F .. kMaxFrags).
template <bool kMx, bool kBlocked, int F>
__device__ __forceinline__ void run_segment_of(int frags, const LaunchArgs& args, const Pos& pos, int c0, int c1,
                                               bool first, bool last, SharedMem& sm, int* s_flag)
{
    if constexpr (F < kMaxFrags) {
        if (frags != F) {
            run_segment_of<kMx, kBlocked, F + 1>(frags, args, pos, c0, c1, first, last, sm, s_flag);
            return;
        }
    }
    if constexpr (kMx)
        run_segment_mx<F>(args, pos, c0, c1, first, last, sm, s_flag);
    else
        run_segment<F, kBlocked>(args, pos, c0, c1, first, last, sm, s_flag);
}

// Wave 0's step of the walk: the segment that starts at cost position c in
// a range ending at b1, and c moved to the tile after it.  gs is the LDS
// copy of the group table.  The group of c comes from one LDS read per lane
// and a ballot (so locate scans no further), and the tile's contributors
// from owner_b, whose boundaries take no division.
__device__ __forceinline__ void walk_step(const LaunchArgs& args, const GroupSched* gs, int32_t& c, int32_t b1,
                                          WalkRec& r)
{
    const int ng = args.ngroups;
    const int lane = opaque_tid() % kWave;
    const int32_t cb = lane < kMaxGroups ? (int32_t)gs[lane].cost_begin : 0;
    const int gi = __builtin_popcountll(__ballot(lane >= 1 && lane < ng && cb <= c));
    r.pos = locate<int32_t>(gs, ng, c, gi);
    const int32_t t0 = (int32_t)r.pos.tile_cost0;
    const int unit = r.pos.unit;
    r.go = r.pos.group < ng && t0 + r.pos.stage * unit < b1;
    r.s_end = r.w_first = r.w_last = 0;
    if (r.go) {
        const int stages = uniform(gs[r.pos.group].stages);
        // Stages of this tile that start before b1.
        const int32_t s_end = (b1 - t0 + unit - 1) / unit;
        r.s_end = s_end < stages ? s_end : stages;
        const int32_t W = (int32_t)args.W;
        r.w_first = owner_b(args.bounds, W, t0);
        r.w_last = owner_b(args.bounds, W, t0 + (stages - 1) * unit);
        c = t0 + unit * stages;   // the next tile's start
    }
}

// The persistent walk of one workgroup over its cost range: every segment
// (a tile's stages in the range) as chains of at most kMaxChainStages
// stages, each by the segment kernel of its fragment count.
//
// The walk's arithmetic runs largely on the scalar unit, which all waves of
// a CU share: done by every wave it took about 3 us per segment (measured,
// with 64-bit costs), so wave 0 alone computes each segment (its position,
// its end, the tile's first and last contributors) and publishes it in
// sm.walk.
template <bool kMx, bool kBlocked>
__device__ __forceinline__ void walk_range(const LaunchArgs& args, SharedMem& sm, int* s_flag)
{
    // The cost arithmetic is 32-bit (the host keeps the total cost below
    // kMaxLaunchCost).  Wave 0's walk state (the next position and the
    // range's end) lives in LDS between segments, so no register holds it
    // through a segment.
    //
    // The group table goes to LDS with one 16-byte load per lane, issued
    // before anything waits for the scalar loads of W and G: its lines then
    // arrive in the same memory round trip as those, where the walk's scan of
    // the table in kernel-argument memory would wait for one cold line after
    // another.
    static_assert(sizeof(GroupSched) * kMaxGroups == kWave * 16, "the group table is one 16-byte piece per lane");
    const int tlane = opaque_tid() % kWave;
    const i4_t table = reinterpret_cast<const i4_t*>(args.sched)[tlane];
    __builtin_amdgcn_sched_barrier(0);
    const bool leader = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave) == 0;
    if (leader) {
        // The boundaries of W (below 2^31, checked by the host) over G,
        // loaded together (the empty asm takes every field, so no load sinks
        // below another's use).
        Bounds bd = args.bounds;
        asm volatile("" : "+s"(bd.q), "+s"(bd.r), "+s"(bd.R), "+s"(bd.G));
        const int w = uniform(worker_id(bd.G));
        const int32_t b1 = bound_at(bd, w + 1);
        const int32_t c = bound_at(bd, w);
        if (threadIdx.x == 0) {
            sm.walk.next = c;
            sm.walk.end = b1;
        }
        reinterpret_cast<i4_t*>(sm.sched)[tlane] = table;
    }
    for (;;) {
        if (leader) {
            WalkRec r;
            int32_t c = uniform(sm.walk.next);
            const int32_t b1 = uniform(sm.walk.end);
            walk_step(args, sm.sched, c, b1, r);
            r.next = c;
            r.end = b1;
            if (threadIdx.x == 0) sm.walk = r;
        }
        __syncthreads();
        const Pos pos = uniform(sm.walk.pos);
        const int s_end = uniform(sm.walk.s_end);
        if (!uniform(sm.walk.go)) break;
        // The segment runs as chains of at most kMaxChainStages stages.
        for (int c0 = pos.stage; c0 < s_end; c0 += kMaxChainStages) {
            const int c1 = c0 + kMaxChainStages < s_end ? c0 + kMaxChainStages : s_end;
            const bool first = c0 == pos.stage, last = c1 == s_end;
            run_segment_of<kMx, kBlocked, 1>(pos.frags, args, pos, c0, c1, first, last, sm, s_flag);
        }
        if (s_end < uniform(sm.sched[pos.group].stages)) break;
        __syncthreads();   // every wave has read sm.walk before wave 0 rewrites it
    }
}

__global__ __launch_bounds__(kThreads) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ SharedMem sm;
    __shared__ int s_flag;
    walk_range<false, false>(args, sm, &s_flag);
}

// NVFP4 with the scales in the blocked layout.
__global__ __launch_bounds__(kThreads) void nvfp4_blocked_sf_gemm_kernel(const LaunchArgs args)
{
    __shared__ SharedMem sm;
    __shared__ int s_flag;
    walk_range<false, true>(args, sm, &s_flag);
}

__global__ __launch_bounds__(kThreads) void mxfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ SharedMem sm;
    __shared__ int s_flag;
    walk_range<true, false>(args, sm, &s_flag);
}

// Writes zeros to C of a group with K == 0 (the empty sum).
// Scratch of nvfp4_group_gemm_noalloc (the workspace of the split-tile
// fix-up for callers that cannot allocate): the partial-tile slots of
// kScratchWorkers workgroups, then one counter per workgroup.  Each device
// the library runs on holds its own copy, from the load of the library's
// code on it until the process ends.  Host code never uses this name as an
// address: it takes the device's copy from hipGetSymbolAddress.
constexpr int kScratchWorkers = 256;
constexpr size_t kScratchPartialBytes = (size_t)kSlotsPerWG * kScratchWorkers * kSlotFloats * sizeof(float);
constexpr size_t kScratchBytes = kScratchPartialBytes + (size_t)kScratchWorkers * sizeof(int);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchPartialBytes % 256 == 0, "the counters start 256-byte aligned");
static_assert(kScratchPartialBytes < kNoSlot, "the partial slots stay below the zero-read offset");

// counters[0 .. n) = 0 (before a call that uses the static scratch: that
// memory keeps whatever the previous call left).
__global__ __launch_bounds__(256) void clear_counters_kernel(int* counters, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) counters[i] = 0;
}

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
    float* partials = nullptr;
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
    if ((uint64_t)kSlotsPerWG * w.workers * kSlotFloats * 4u >= kNoSlot)
        return fail(NVFP4GG_UNSUPPORTED, "too many compute units for the partial-tile workspace");
    const size_t pbytes = (size_t)kSlotsPerWG * w.workers * kSlotFloats * sizeof(float);
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

extern "C" int nvfp4_group_gemm_version(void) { return 7; }

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

// Device addresses of each device's copy of `scratch`, looked up once per
// device (fixed-size table: the lookup path allocates nothing either).
constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_cus[kMaxDevices];

// The static-scratch workspace of the current device dev.
int scratch_workspace(int dev, Workspace& out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return fail(NVFP4GG_UNSUPPORTED, "device index beyond the static scratch table");
    uint8_t* ptr = g_scratch_ptr[dev].load();
    int cus = g_scratch_cus[dev].load();
    if (!ptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return fail(NVFP4GG_HIP_ERROR, "hipGetSymbolAddress of the static scratch failed");
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = kScratchWorkers;
        g_scratch_cus[dev].store(cus);
        ptr = static_cast<uint8_t*>(p);
        g_scratch_ptr[dev].store(ptr);
    }
    // A launch has at most one workgroup per compute unit; the scratch holds
    // the workspace of kScratchWorkers of them.
    if (cus > kScratchWorkers)
        return fail(NVFP4GG_UNSUPPORTED, "the device has " + std::to_string(cus) +
                                             " compute units; the static scratch holds the fix-up workspace of " +
                                             std::to_string(kScratchWorkers) + " workgroups");
    out.partials = reinterpret_cast<float*>(ptr);
    out.counters = reinterpret_cast<int*>(ptr + kScratchPartialBytes);
    out.workers = cus;
    return NVFP4GG_OK;
}

// Every grouped-GEMM entry point: fmt selects NVFP4 (E4M3 per 16 K) or
// MXFP4 (E8M0 per 32 K), blocked_sf the blocked layout of NVFP4 scales,
// static_scratch the fix-up workspace in the static scratch (no allocation)
// instead of the per-stream one.
int group_gemm_impl(int g, const int* M, const int* N, const int* K, const void* const* A_ptrs,
                    const void* const* B_ptrs, const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                    void* const* C_ptrs, void* stream, int blocked_sf, int fmt, bool static_scratch = false)
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
        if (K[i] % kStageK != 0)
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
            if (static_scratch) {
                const int rc = scratch_workspace(dev, ws);
                if (rc != NVFP4GG_OK) return rc;
                // That memory keeps the last call's contents: the counters
                // start from zero (a fill kernel, not a memset, so that the
                // call can be captured into a graph).
                hipLaunchKernelGGL(clear_counters_kernel, dim3((ws.workers + 255) / 256), dim3(256), 0, s,
                                   ws.counters, ws.workers);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
            } else {
                const int rc = get_workspace(dev, s, ws);
                if (rc != NVFP4GG_OK) return rc;
            }
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
        args.blocked_sf = blocked_sf;
        args.W = cost;
        args.G = grid_size(cost, ws.workers);
        if (cost > kMaxLaunchCost)
            return fail(NVFP4GG_UNSUPPORTED, "launch too large: its schedule cost exceeds 2^31 units");
        if (args.G > kMaxBoundsG)
            return fail(NVFP4GG_UNSUPPORTED, "more workgroups than the schedule's boundary arithmetic supports");
        args.bounds = make_bounds(cost, args.G);
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

extern "C" int nvfp4_group_gemm_noalloc(int g, const int* M, const int* N, const int* K,
                                        const void* const* A_ptrs, const void* const* B_ptrs,
                                        const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                        void* const* C_ptrs, void* stream)
{
    return group_gemm_impl(g, M, N, K, A_ptrs, B_ptrs, SFA_ptrs, SFB_ptrs, C_ptrs, stream, 0, kFmtNvfp4, true);
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
