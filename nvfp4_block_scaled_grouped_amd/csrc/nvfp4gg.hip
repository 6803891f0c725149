// nvfp4gg.hip -- NVFP4 block-scaled grouped GEMM for MI355X (gfx950).
//
// C_i = A_i . B_i^T per group, A/B packed FP4 E2M1 with one E4M3 scale per 16
// K of a row, fp32 accumulation, fp16 output (kernelindex page
// kernelbot-nvfp4-group-gemm-444497, kernel-source header comment; page
// kernelbot-nvfp4-group-gemm-505431, custom_kernel_fallback).  The C ABI is
// declared in include/nvfp4gg.h.
//
// Design (gfx950 first; the pages' Blackwell kernels are prior art only):
//   * Scale resolution: every A and B element is dequantised to fp16 as
//     e2m1(code) * e4m3(scale).  That product has at most 6 significant bits
//     and lies in [2^-10, 2688], so fp16 holds it exactly, and the fp16 x fp16
//     products inside the MFMA are exact in fp32.  The contraction runs on
//     v_mfma_f32_32x32x16_f16 with fp32 accumulation.  (CDNA4's block-scaled
//     f8f6f4 MFMA takes power-of-two E8M0 scales per 32 K; it cannot carry an
//     E4M3 mantissa per 16 K, and no 8-bit operand format holds a 6-bit
//     significand.)
//   * Dequant: v_cvt_scalef32_pk_f16_fp4 turns two FP4 codes into two fp16
//     (its scale operand contributes only a power of two, so it is passed
//     1.0), then v_pk_mul_f16 multiplies by the E4M3 scale converted to fp16
//     (exact: every E4M3 value is an fp16 value).
//   * Tile: one workgroup of 8 waves per CU owns up to 96 rows of A_i
//     (1..3 fragments of 32 rows) x 256 columns of B_i.  Wave w = 4 kh + cg
//     owns columns [64 cg, 64 cg + 64) for all rows, over K half kh of every
//     256-K stage.  A is shared: each stage of the tile's A rows is
//     dequantised once by the workgroup into LDS as fp16, already in MFMA
//     operand order, and the waves read it with 16-byte LDS loads.  B is
//     private to a wave: each lane loads its own MFMA operand bytes straight
//     into registers and dequantises them there, so one dequantised B
//     fragment feeds up to 3 MFMAs.
//   * K order: the sum over K is order-free.  A and B use the same order, so
//     every pair (a_k, b_k) meets in the same MFMA slot; it is chosen so that
//     the two lanes holding a row read one contiguous 64-byte run.
//   * Accumulation: the two K halves of a stage are summed by different
//     waves into separate fp32 accumulators (two interleaved chains, each at
//     most 4096 K long), added at the end; this keeps the rounding error of
//     long K sums small next to outputs near zero.
//   * Schedule: the work is the list of (tile, stage) units (schedule.h); a
//     persistent grid of one workgroup per CU takes equal-cost contiguous
//     ranges of it, so ragged groups fill the chip in one launch.  A tile
//     whose stages span several workgroups is finished by the last of them
//     to arrive: each writes its fp32 partial tile to a workspace slot and
//     bumps the tile's counter; the one that sees all others done sums the
//     partials in workgroup order (deterministic) and writes C.  No
//     workgroup ever waits for another.
//   * Loads are raw buffer loads whose range is the exact operand size, so
//     rows past M_i or N_i read as zero without branches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>

#include "nvfp4gg.h"
#include "schedule.h"

namespace {

using namespace nvfp4sched;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef int i4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 8;                    // two waves per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kNF = 2;                       // 32-column B fragments per wave
constexpr int kColGroups = 4;                // 64-column groups of the tile
constexpr int kKSteps = kStageK / 16;        // MFMA k-steps per stage (16 K each: 8 per lane half)
constexpr int kHalfSteps = kKSteps / 2;      // k-steps of one wave per stage (its K half)
constexpr int kMaxChainStages = 32;          // stages one fp32 chain accumulates (4096 K per wave)
constexpr int kSlotFloats = kColGroups * kNF * kMaxFrags * kWave * 16;   // one partial tile
constexpr uint32_t kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kCoherent = 16;                  // cache-policy bit sc1: device-scope coherent access
constexpr int kWaitVmcnt0 = 0x0F70;            // s_waitcnt vmcnt(0) (expcnt, lgkmcnt not waited)

// Issue-order hints that interleave the B dequantisation with the MFMAs of
// each k-step (0 leaves the order to the compiler).
#ifndef NVFP4_INTERLEAVE
#define NVFP4_INTERLEAVE 1
#endif
#ifndef NVFP4_XCD_REMAP
#define NVFP4_XCD_REMAP 1
#endif
constexpr int kXcds = 8;   // XCDs of the chip; workgroups are dealt to them round-robin

static_assert(kTileN == kColGroups * kNF * 32, "each column group owns kNF 32-column fragments");
static_assert(kMaxFrags == 3, "the kernel instantiates m-blocks of 1, 2 and 3 fragments");
static_assert(kWaves == 2 * kColGroups, "two K halves per column group");

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
    int* counters;        // one per tile, zero between calls
    int64_t W;            // total cost
    int G;                // workgroups
    int ngroups;
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
// [fragment][k-step][lane] x 8 fp16 (64 KB).
struct AStage {
    h8_t v[kMaxFrags][kKSteps][kWave];
};

// The workgroup's LDS: two A stages.  At the end of a segment the same
// memory first carries the exchange of the two K halves' fp32 fragments
// ([column group][B fragment][A fragment][quad][lane]) and then the fp16
// output tile on its way to C (rows padded by 16 bytes against bank
// conflicts).
constexpr int kCTileStride = kTileN + 8;   // halves per LDS row of the output tile
struct SharedMem {
    union {
        AStage a[2];
        f4_t xch[kColGroups][kNF][kMaxFrags][4][kWave];
        uint16_t ctile[kMaxFrags * kFragRows][kCTileStride];
    };
    // Target of the A-store of waves that have no A fragment in the tile
    // (their writes are discarded), so the k-step needs no branch.
    h8_t discard[kKSteps / 2][kWave];
};
static_assert(sizeof(f4_t) * kColGroups * kNF * kMaxFrags * 4 * kWave <= 2 * sizeof(AStage),
              "the exchange fits in the A buffers");
static_assert(sizeof(uint16_t) * kMaxFrags * kFragRows * kCTileStride <= 2 * sizeof(AStage),
              "the output tile fits in the A buffers");

// fp16 round-to-nearest-even (overflow to inf) of 4 floats, packed.
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d)
{
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)c) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)d) << 16);
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

// The output tile of the workgroup, fp32 -> fp16 (round to nearest even,
// overflow to inf), written to C through LDS so that every global store is
// 16 contiguous bytes of a row.  Wave (cg, kh) holds fragment f = kh of
// column group cg: own[fm] element r of lane (l32, h) is tile row
// 32 fm + l32, tile column 64 cg + 32 kh + 8 (r / 4) + 4 h + r % 4.
// Called by every thread of the workgroup; the LDS is free on return.
template <int MF>
__device__ __forceinline__ void store_c(SharedMem& sm, const GroupArgs& ga, int m0, int n0, const f16x_t* own,
                                        int cg, int kh)
{
    const int lane = threadIdx.x % kWave;
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int col = 64 * cg + 32 * kh + 8 * q4 + 4 * h;
            *reinterpret_cast<uint2*>(&sm.ctile[32 * fm + l32][col]) =
                pack4(own[fm][4 * q4], own[fm][4 * q4 + 1], own[fm][4 * q4 + 2], own[fm][4 * q4 + 3]);
        }
    lds_barrier();
    const int M = ga.M, N = ga.N;
    const int rows = M - m0 < MF * kFragRows ? M - m0 : MF * kFragRows;
    const int chunk = threadIdx.x % (kTileN / 8);          // 8 columns = 16 bytes
    const int n = n0 + 8 * chunk;
    const bool vec_ok = (N & 7) == 0;
    for (int r = threadIdx.x / (kTileN / 8); r < rows; r += kThreads / (kTileN / 8)) {
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

// One wave's fp32 fragment block of a partial tile (MF x 16 floats per
// lane) at base, laid out in 1 KB lane-contiguous pieces.
template <int MF>
__device__ __forceinline__ void store_block(__amdgpu_buffer_rsrc_t r, uint32_t base, const f16x_t* own)
{
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(i4_t, f4_t{own[fm][4 * q], own[fm][4 * q + 1], own[fm][4 * q + 2],
                                              own[fm][4 * q + 3]}),
                r, base + (uint32_t)(fm * 4 + q) * (kWave * 16u), 0, kCoherent);
}

// acc (+)= the block stored by store_block at base (assign when first).
template <int MF>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t r, uint32_t base, f16x_t* acc, bool first)
{
#pragma unroll
    for (int fm = 0; fm < MF; ++fm)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4_t v = __builtin_bit_cast(
                f4_t, __builtin_amdgcn_raw_buffer_load_b128(r, base + (uint32_t)(fm * 4 + q) * (kWave * 16u), 0,
                                                             kCoherent));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[fm][4 * q + e] = first ? v[e] : acc[fm][4 * q + e] + v[e];
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

// One chain [s_begin, s_end) of the stages of a tile with MF fragments: a
// workgroup's segment of a tile runs as chains of at most kMaxChainStages
// stages (one chain for any K <= 8192); first_chain / last_chain place this
// chain in its segment.
//
// Waves: wave w = 4 kh + cg owns columns [64 cg, 64 cg + 64) of the tile
// (kNF = 2 fragments of 32) for all MF x 32 rows, over K half kh of every
// stage (k-steps 8 kh .. 8 kh + 7).  The two K halves are independent fp32
// chains, added through LDS at the end of the chain: splitting the sum into
// two interleaved chains halves the magnitude each fp32 accumulator reaches
// and the number of additions it makes, and capping a chain at 4096 K per
// wave bounds both.  The chains of one segment meet in the workgroup's
// scratch slot; the last one finishes the tile.
//
// Pipeline, per stage i of a chain:
//   * B of stage i is in registers, loaded during stage i - 1: each 16-byte
//     piece is re-loaded with stage i + 1 as soon as its four k-steps are
//     dequantised.
//   * A of stage i is in LDS buffer i % 2, dequantised during stage i - 1:
//     wave w writes fragment w / 2, k-steps 8 (w % 2) .. 8 (w % 2) + 7, one
//     k-step per k-step of its own MFMA loop, from raw bytes loaded during
//     stage i - 2.
//   * One LDS-only barrier ends the stage.
template <int MF>
__device__ __forceinline__ void run_segment(const LaunchArgs& args, const Pos& pos, int s_begin, int s_end,
                                            bool first_chain, bool last_chain, SharedMem& sm, int* s_flag)
{
    const GroupSched& gs = args.sched[pos.group];
    const GroupArgs& ga = args.grp[pos.group];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int cg = wave % kColGroups;
    const int kh = wave / kColGroups;
    const int af = wave >> 1;            // A fragment this wave dequantises
    const int ah = wave & 1;             // and which half of its k-steps
    const int lane = threadIdx.x % kWave;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int M = ga.M, N = ga.N, K = ga.K;
    const int m0 = mblock_first_frag(gs.frags, gs.mblocks, pos.mb) * kFragRows;
    const int ncol = pos.nb * kTileN + cg * (kNF * 32);
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 16;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ga.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(ga.B, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(ga.SFA, (uint32_t)M * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(ga.SFB, (uint32_t)N * row_scales);

    // K order within a stage (the sum is order-free; A and B use the same
    // order): k-step j = 8 q + u (K half q, u < 8) feeds lane half h the 8
    // codes at K 128 q + 64 h + 8 u, i.e. dword u of the 32 bytes
    // [64 q + 32 h, +32) of the row's stage bytes, whose scale block is
    // 8 q + 4 h + u / 2.  So the two lanes of a row read one contiguous,
    // 64-byte aligned run per K half.
    // B operand of lane (l32, h) in fragment f: row ncol + 32 f + l32, the 32
    // bytes of its half of K half kh and their 4 scale bytes.
    uint32_t offB[kNF], offSB[kNF];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
        const uint32_t brow = (uint32_t)(ncol + 32 * f + l32);
        offB[f] = brow * row_bytes + 64u * kh + 32u * h;
        offSB[f] = brow * row_scales + 8u * kh + 4u * h;
    }
    // A bytes this lane dequantises: row m0 + 32 af + l32, its half of K half
    // ah (k-steps 8 ah .. 8 ah + 7).
    const bool a_active = af < MF;
    // Waves without a fragment of this tile load (and discard) the rows of
    // fragment af % MF, which the L1 already fetches for its owner.
    const uint32_t arow = (uint32_t)(m0 + 32 * (af % MF) + l32);
    const uint32_t offA = arow * row_bytes + 64u * ah + 32u * h;
    const uint32_t offSA = arow * row_scales + 8u * ah + 4u * h;

    f16x_t part[kNF][kMaxFrags];
    f16x_t own[kMaxFrags];   // after a chain: fragment f = kh of this wave's column group, both K halves
    const __amdgpu_buffer_rsrc_t rP =
        make_rsrc(args.partials, (uint32_t)(kSlotsPerWG * args.G) * kSlotFloats * 4u);
    // This wave's block of a slot: [column group][B fragment] blocks of
    // kMaxFrags x 4 x 1 KB; wave (cg, kh) owns block (cg, kh).
    const uint32_t wave_in_slot =
        (uint32_t)(cg * kNF + kh) * (kMaxFrags * 4) * (kWave * 16u) + (uint32_t)lane * 16u;
    const uint32_t scratch_base =
        (uint32_t)scratch_slot(worker_id(args.G)) * kSlotFloats * 4u + wave_in_slot;

    {
        const int c_begin = s_begin;
        const int n = s_end - s_begin;

        // Register stage buffers, each one stage ahead of its use: B of the
        // stage being multiplied (each 16-byte piece re-loaded with the next
        // stage's as soon as its four k-steps are dequantised), and the raw A
        // of the stage being dequantised into LDS (likewise re-loaded with
        // the stage after).
        i4_t bq[kNF][2];
        uint32_t bs[kNF];
        i4_t aq[2] = {i4_t{}, i4_t{}};
        uint32_t as = 0u;

        // Prologue: B of stage 0 and A of stages 0 and 1 in flight; stage 0
        // of A into LDS buffer 0.
        {
            const uint32_t sbyte = __builtin_amdgcn_readfirstlane(c_begin * (kStageK / 2));
            const uint32_t sscale = __builtin_amdgcn_readfirstlane(c_begin * (kStageK / 16));
            i4_t a0[2] = {i4_t{}, i4_t{}};
            uint32_t as0 = 0u;
            if (a_active) {
                a0[0] = load16(rA, offA, sbyte);
                a0[1] = load16(rA, offA + 16, sbyte);
                as0 = __builtin_amdgcn_raw_buffer_load_b32(rSA, offSA, sscale, 0);
            }
#pragma unroll
            for (int f = 0; f < kNF; ++f) {
                bq[f][0] = load16(rB, offB[f], sbyte);
                bq[f][1] = load16(rB, offB[f] + 16, sbyte);
                bs[f] = __builtin_amdgcn_raw_buffer_load_b32(rSB, offSB[f], sscale, 0);
            }
            if (a_active && n > 1) {
                aq[0] = load16(rA, offA, sbyte + kStageK / 2);
                aq[1] = load16(rA, offA + 16, sbyte + kStageK / 2);
                as = __builtin_amdgcn_raw_buffer_load_b32(rSA, offSA, sscale + kStageK / 16, 0);
            }
            if (a_active) {
                _Float16 sa[4];
                scales4(as0, sa);
#pragma unroll
                for (int u = 0; u < kHalfSteps; ++u)
                    sm.a[0].v[af][kHalfSteps * ah + u][lane] = dequant8((uint32_t)a0[u >> 2][u & 3], sa[u >> 1]);
            }
        }
#pragma unroll
        for (int f = 0; f < kNF; ++f)
#pragma unroll
            for (int fm = 0; fm < MF; ++fm) part[f][fm] = f16x_t{};
        lds_barrier();

        auto stage = [&](auto parity, int i) {
            constexpr int p = decltype(parity)::value;
            const bool has1 = i + 1 < n;
            const bool has2 = i + 2 < n;
            // Stage offsets are wave-uniform; readfirstlane keeps them in
            // SGPRs (the buffer loads' soffset) where the compiler would
            // otherwise not prove it.
            const uint32_t sbyte1 = __builtin_amdgcn_readfirstlane((c_begin + i + 1) * (kStageK / 2));
            const uint32_t sscale1 = __builtin_amdgcn_readfirstlane((c_begin + i + 1) * (kStageK / 16));
            const uint32_t sbyte2 = sbyte1 + kStageK / 2;
            const uint32_t sscale2 = sscale1 + kStageK / 16;
            const uint32_t sbyte_n = has1 ? sbyte1 : sbyte1 - kStageK / 2;    // B loads: next stage, or this one
            const uint32_t sbyte_nn = has2 ? sbyte2 : sbyte1 - kStageK / 2;   // A loads: stage i + 2, or this one

            _Float16 sbf[kNF][4];
#pragma unroll
            for (int f = 0; f < kNF; ++f) scales4(bs[f], sbf[f]);
            _Float16 sa[4];
            scales4(as, sa);
            if (has1) {
#pragma unroll
                for (int f = 0; f < kNF; ++f) bs[f] = __builtin_amdgcn_raw_buffer_load_b32(rSB, offSB[f], sscale1, 0);
            }
            if (a_active && has2) as = __builtin_amdgcn_raw_buffer_load_b32(rSA, offSA, sscale2, 0);
            // Where this wave's A dequantisation goes: its fragment of the
            // next stage's buffer, or the discard area.  (In a chain's last
            // stage the next buffer is written but never read.)
            h8_t* const a_dst = a_active ? &sm.a[p ^ 1].v[af][kHalfSteps * ah][lane] : &sm.discard[0][lane];

            // k-step pipeline: the A-operand LDS reads and the B dequant of
            // k-step u + 1 are issued before the MFMAs of k-step u, so their
            // latency hides behind those MFMAs.  The scheduling barrier at the
            // end of each k-step keeps the compiler from hoisting work across
            // k-steps (register pressure).
            h8_t bv[kNF], av[MF];
#pragma unroll
            for (int f = 0; f < kNF; ++f) bv[f] = dequant8((uint32_t)bq[f][0][0], sbf[f][0]);
#pragma unroll
            for (int fm = 0; fm < MF; ++fm) av[fm] = sm.a[p].v[fm][kHalfSteps * kh][lane];
#pragma unroll
            for (int u = 0; u < kHalfSteps; ++u) {
                h8_t nbv[kNF], nav[MF];
                if (u + 1 < kHalfSteps) {
#pragma unroll
                    for (int fm = 0; fm < MF; ++fm) nav[fm] = sm.a[p].v[fm][kHalfSteps * kh + u + 1][lane];
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
                        nbv[f] = dequant8((uint32_t)bq[f][(u + 1) >> 2][(u + 1) & 3], sbf[f][(u + 1) >> 1]);
                }
#pragma unroll
                for (int fm = 0; fm < MF; ++fm)
#pragma unroll
                    for (int f = 0; f < kNF; ++f)
                        part[f][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[f], av[fm], part[f][fm], 0, 0, 0);
                // Dequantise k-step u of the raw A into LDS (before piece
                // u / 4 of the raw A is re-loaded below).
                a_dst[u * kWave] = dequant8((uint32_t)aq[u >> 2][u & 3], sa[u >> 1]);
                // Piece c (k-steps 4c .. 4c+3) of B is dequantised in full at
                // u = 4c + 2 (one k-step ahead), that of the raw A at u = 4c + 3:
                // fetch the next stage's B and stage i + 2's raw A.  The loads
                // are unconditional (a stage past the chain re-reads the last
                // one; rows past the tile read other rows or zeros), which
                // keeps the k-step one scheduling region.
                if (u == kHalfSteps - 2) {
#pragma unroll
                    for (int f = 0; f < kNF; ++f) {
                        bq[f][0] = load16(rB, offB[f], sbyte_n);
                        bq[f][1] = load16(rB, offB[f] + 16, sbyte_n);
                    }
                }
                if (u == kHalfSteps - 1) {
                    aq[0] = load16(rA, offA, sbyte_nn);
                    aq[1] = load16(rA, offA + 16, sbyte_nn);
                }
                if (u + 1 < kHalfSteps) {
#pragma unroll
                    for (int f = 0; f < kNF; ++f) bv[f] = nbv[f];
#pragma unroll
                    for (int fm = 0; fm < MF; ++fm) av[fm] = nav[fm];
                }
#if NVFP4_INTERLEAVE
                // Issue order: each MFMA followed by a share of the VALU work,
                // so the dequantisation runs while the matrix core is busy.
#pragma unroll
                for (int g = 0; g < MF * kNF; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // up to five VALU
                }
#endif
                __builtin_amdgcn_sched_barrier(0);
            }
            lds_barrier();
        };

        for (int i = 0; i < n; i += 2) {
            stage(Parity<0>{}, i);
            if (i + 1 >= n) break;
            stage(Parity<1>{}, i + 1);
        }

        // Add the two K halves through LDS (the A buffers are free: every
        // wave is past the last stage's barrier).  Wave (cg, kh) hands
        // fragment 1 - kh to its partner (cg, 1 - kh) and keeps fragment kh,
        // so both halves of the workgroup carry the epilogue.  The indices
        // are spelled out per kh to keep the register arrays statically
        // indexed.
        if (kh == 0) {
#pragma unroll
            for (int fm = 0; fm < MF; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sm.xch[cg][1][fm][q][lane] = f4_t{part[1][fm][4 * q], part[1][fm][4 * q + 1],
                                                      part[1][fm][4 * q + 2], part[1][fm][4 * q + 3]};
        } else {
#pragma unroll
            for (int fm = 0; fm < MF; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sm.xch[cg][0][fm][q][lane] = f4_t{part[0][fm][4 * q], part[0][fm][4 * q + 1],
                                                      part[0][fm][4 * q + 2], part[0][fm][4 * q + 3]};
        }
        lds_barrier();
        if (kh == 0) {
#pragma unroll
            for (int fm = 0; fm < MF; ++fm) own[fm] = part[0][fm];
        } else {
#pragma unroll
            for (int fm = 0; fm < MF; ++fm) own[fm] = part[1][fm];
        }
#pragma unroll
        for (int fm = 0; fm < MF; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4_t v = sm.xch[cg][kh][fm][q][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) own[fm][4 * q + e] += v[e];
            }
        lds_barrier();   // the exchange is read before anything else is written to the LDS
    }
    // Chains of one segment meet in the scratch slot.
    if (!first_chain) load_block<MF>(rP, scratch_base, own, false);
    if (!last_chain) {
        store_block<MF>(rP, scratch_base, own);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        return;
    }

    // Finish the tile: alone, or as one of several contributors.  Every
    // wave holds its fragment of the segment's sum in own.
    const int unit = unit_cost(pos.frags);
    const int64_t c_first = pos.tile_cost0;
    const int64_t c_last = pos.tile_cost0 + (int64_t)(gs.stages - 1) * unit;
    const int w_first = owner(args.W, args.G, c_first);
    const int w_last = owner(args.W, args.G, c_last);
    const int n0 = pos.nb * kTileN;
    if (w_first == w_last) {
        store_c<MF>(sm, ga, m0, n0, own, cg, kh);
        return;
    }
    const int me = worker_id(args.G);
    const int tile = tile_index(args.sched, pos);
    // Partial tile -> this workgroup's slot (partial_slot).  The stores carry
    // the device-scope coherence bit (sc1), so they are written through past
    // this XCD's L2; waiting for them before the counter update publishes
    // them to whichever workgroup finishes the tile, with no cache flush.
    auto slot_base = [&](int w) {
        return (uint32_t)partial_slot(w, w_last) * kSlotFloats * 4u + wave_in_slot;
    };
    store_block<MF>(rP, slot_base(me), own);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old =
            __hip_atomic_fetch_add(args.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = (old == w_last - w_first) ? 1 : 0;
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    __syncthreads();   // s_flag is reused by the next segment
    if (!last) return;
    // Sum the contributors' partials in workgroup order, so the result does
    // not depend on who arrived last.  When this workgroup is the first
    // contributor its partial is still in registers; otherwise it is read
    // back like the others.  The loads carry the device-scope coherence bit
    // as well.
    for (int w = me == w_first ? w_first + 1 : w_first; w <= w_last; ++w)
        load_block<MF>(rP, slot_base(w), own, w == w_first);
    store_c<MF>(sm, ga, m0, n0, own, cg, kh);
    if (threadIdx.x == 0)
        __hip_atomic_store(args.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kThreads) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    __shared__ SharedMem sm;
    __shared__ int s_flag;

    const int w = worker_id(args.G);
    const int64_t b1 = boundary(args.W, args.G, w + 1);
    Pos pos = locate(args.sched, args.ngroups, boundary(args.W, args.G, w));
    while (pos.group < args.ngroups && stage_cost(pos, pos.stage) < b1) {
        const GroupSched& gs = args.sched[pos.group];
        const int unit = unit_cost(pos.frags);
        // Stages of this tile that start before b1.
        const int64_t s_end64 = (b1 - pos.tile_cost0 + unit - 1) / unit;
        const int s_end = s_end64 < gs.stages ? (int)s_end64 : gs.stages;
        // The segment runs as chains of at most kMaxChainStages stages.
        for (int c0 = pos.stage; c0 < s_end; c0 += kMaxChainStages) {
            const int c1 = c0 + kMaxChainStages < s_end ? c0 + kMaxChainStages : s_end;
            const bool first = c0 == pos.stage, last = c1 == s_end;
            switch (pos.frags) {
                case 1: run_segment<1>(args, pos, c0, c1, first, last, sm, &s_flag); break;
                case 2: run_segment<2>(args, pos, c0, c1, first, last, sm, &s_flag); break;
                default: run_segment<3>(args, pos, c0, c1, first, last, sm, &s_flag); break;
            }
        }
        if (s_end < gs.stages) break;
        pos = locate(args.sched, args.ngroups, pos.tile_cost0 + (int64_t)unit * gs.stages);
    }
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

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Minimum cost handed to one workgroup: keeps every workgroup range longer
// than the costliest stage, which the fixup relies on.
constexpr int64_t kMinUnitsPerWG = 8;
static_assert(kMinUnitsPerWG >= kMaxFrags + kStageFixedCost, "a workgroup range must hold a stage");

// Workspace of the split-tile fixup, one per (device, stream): three
// partial-tile slots per workgroup and the per-tile counters (zero between calls; the last contributor
// of a tile resets its counter).  Allocated on first use and kept.
struct Workspace {
    float* partials = nullptr;
    size_t slots = 0;
    int* counters = nullptr;
    size_t ncounters = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;
std::map<int, int> g_cus;

int get_workspace(int dev, hipStream_t s, int G, int tiles, Workspace& out)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[std::make_pair(dev, (void*)s)];
    const size_t need_slots = kSlotsPerWG * (size_t)G;
    if (w.slots < need_slots) {
        if (w.partials) {
            if (hipStreamSynchronize(s) != hipSuccess || hipFree(w.partials) != hipSuccess)
                return fail(NVFP4GG_HIP_ERROR, "workspace release failed");
            w.partials = nullptr;
            w.slots = 0;
        }
        if (hipMalloc(&w.partials, need_slots * kSlotFloats * sizeof(float)) != hipSuccess) {
            w.partials = nullptr;
            return fail(NVFP4GG_HIP_ERROR, "workspace allocation failed");
        }
        w.slots = need_slots;
    }
    if (w.ncounters < (size_t)tiles) {
        if (w.counters) {
            if (hipStreamSynchronize(s) != hipSuccess || hipFree(w.counters) != hipSuccess)
                return fail(NVFP4GG_HIP_ERROR, "workspace release failed");
            w.counters = nullptr;
            w.ncounters = 0;
        }
        const size_t n = tiles > 4096 ? (size_t)tiles : 4096;
        if (hipMalloc(&w.counters, n * sizeof(int)) != hipSuccess ||
            hipMemset(w.counters, 0, n * sizeof(int)) != hipSuccess) {
            w.counters = nullptr;
            return fail(NVFP4GG_HIP_ERROR, "workspace allocation failed");
        }
        w.ncounters = n;
    }
    out = w;
    return NVFP4GG_OK;
}

int device_cus(int dev)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) return it->second;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_cus[dev] = v;
    return v;
}

}  // namespace

extern "C" const char* nvfp4_group_gemm_last_error(void) { return g_last_error.c_str(); }

extern "C" int nvfp4_group_gemm_version(void) { return 1; }

extern "C" int nvfp4_group_gemm(int g, const int* M, const int* N, const int* K,
                                const void* const* A_ptrs, const void* const* B_ptrs,
                                const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                void* const* C_ptrs, void* stream)
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
            return fail(NVFP4GG_UNSUPPORTED, gs + "this kernel needs K % 256 == 0");
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
    const int cus = device_cus(dev);

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

    LaunchArgs args;
    int gi = 0;
    while (gi < g) {
        std::memset(&args, 0, sizeof(args));
        int n = 0;
        int tiles = 0;
        int64_t cost = 0;
        for (; gi < g && n < kMaxGroups; ++gi) {
            if (M[gi] == 0 || N[gi] == 0 || K[gi] == 0) continue;
            GroupSched& sc = args.sched[n];
            GroupArgs& ga = args.grp[n];
            ++n;
            ga.A = static_cast<const uint8_t*>(A_ptrs[gi]);
            ga.B = static_cast<const uint8_t*>(B_ptrs[gi]);
            ga.SFA = static_cast<const uint8_t*>(SFA_ptrs[gi]);
            ga.SFB = static_cast<const uint8_t*>(SFB_ptrs[gi]);
            ga.C = static_cast<uint16_t*>(C_ptrs[gi]);
            ga.M = M[gi];
            ga.N = N[gi];
            ga.K = K[gi];
            sc.frags = ceil_div(M[gi], kFragRows);
            sc.mblocks = ceil_div(sc.frags, kMaxFrags);
            sc.nblocks = ceil_div(N[gi], kTileN);
            sc.stages = K[gi] / kStageK;
            sc.cost_begin = cost;
            sc.tile_begin = tiles;
            cost += group_cost(sc);
            tiles += sc.mblocks * sc.nblocks;
        }
        if (n == 0) continue;
        args.ngroups = n;
        args.W = cost;
        int64_t G = cost / kMinUnitsPerWG;
        if (G > cus) G = cus;
        if (G < 1) G = 1;
        args.G = (int)G;
        Workspace ws;
        const int rc = get_workspace(dev, s, args.G, tiles, ws);
        if (rc != NVFP4GG_OK) return rc;
        args.partials = ws.partials;
        args.counters = ws.counters;
        hipLaunchKernelGGL(nvfp4_group_gemm_kernel, dim3(args.G), dim3(kThreads), 0, s, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
    }
    return NVFP4GG_OK;
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
