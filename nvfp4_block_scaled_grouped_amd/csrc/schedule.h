// schedule.h -- work decomposition of the grouped GEMM into (tile, K-stage)
// units and their even split over a persistent grid (stream-K style).
//
// Plain C++ usable from host and device code; the kernel and the host
// launcher include it, and a CPU test compiles it on its own.
//
// Terms:
//   * fragment: 16 rows of A_i (the MFMA tile height), so a group's last
//     fragment carries at most 15 padding rows.
//   * m-block: up to maxf <= kMaxFrags fragments of one group, processed
//     together (maxf is chosen per launch).  A group with F = ceil(M/16)
//     fragments has nmb = ceil(F / maxf) m-blocks; fragments are spread
//     evenly, so the first F % nmb m-blocks get F / nmb + 1 fragments and
//     the rest F / nmb.
//   * n-block: kTileN columns of B_i.
//   * tile: (group, n-block, m-block); tiles are ordered by group, then
//     n-block, then m-block, so the m-blocks that share a B strip are
//     adjacent in the order.
//   * stage: kStageK consecutive K of a tile.  A stage of a tile with f
//     fragments costs unit_cost(f, fmt) units (about 50 ns of MI355X time
//     each, fitted to measured stage times).  NVFP4 (fp16 MFMA after
//     dequantisation): the B stream and its dequantisation do not grow with
//     f, the MFMAs do, and tiles of more than 8 fragments give some waves a
//     second piece of A to dequantise.  MXFP4 (native FP4 MFMA, no
//     dequantisation): a stage is mostly its B stream.
//   * A tile's cost range is tile_cost(f) (the start-up and wind-down of
//     the segment that starts it: first loads, the fix-up, the output
//     store) followed by its stages.
//   * Workgroup w of G takes the cost range [w*W/G, (w+1)*W/G), rounded up
//     to stage starts, so every stage belongs to exactly one workgroup.
#ifndef NVFP4GG_SCHEDULE_H
#define NVFP4GG_SCHEDULE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define NVFP4_HD __host__ __device__ __forceinline__
#else
#define NVFP4_HD inline
#endif

namespace nvfp4sched {

constexpr int kMaxFrags = 12;      // fragments per m-block
constexpr int kFragRows = 16;      // rows per fragment
constexpr int kTileN = 256;        // columns per n-block
constexpr int kStageK = 128;       // K per stage
constexpr int kMaxGroups = 32;     // groups per launch
#ifndef NVFP4_TILE_COST_BASE
#define NVFP4_TILE_COST_BASE 40
#endif
#ifndef NVFP4_TILE_COST_PER_FRAG
#define NVFP4_TILE_COST_PER_FRAG 25
#endif
// Cost units of a tile of f fragments beyond its stages: tile_cost(f).  It
// is carried by the tile's first contributor, which starts the tile and
// finishes it (waits for the others, reads their partial tiles of 16 f
// rows each and stores C): that part grows with the tile's rows.  Swept on
// MI355X over the five workloads (flat 100 to 300, and 0 to 60 plus 15 to
// 45 per fragment); 40 + 25 f beat the flat 200 on every workload (c4 by
// 1.6 us, c2 by 1.3 us, c5 by about 2 us).
constexpr int kTileCostBase = NVFP4_TILE_COST_BASE;
constexpr int kTileCostPerFrag = NVFP4_TILE_COST_PER_FRAG;
constexpr int kMaxUnitCost = 56;   // the costliest stage (NVFP4, 12 fragments)
constexpr int kFmtNvfp4 = 0;       // E4M3 scale per 16 K, fp16 MFMA
constexpr int kFmtMxfp4 = 1;       // E8M0 scale per 32 K, FP4 MFMA
// Least cost handed to one workgroup: keeps every workgroup range longer
// than the costliest stage, so the workgroups sharing a tile are
// consecutive.
constexpr int64_t kMinUnitsPerWG = 64;
static_assert(kMinUnitsPerWG >= kMaxUnitCost, "a workgroup range must hold a stage");

struct GroupSched {
    int64_t cost_begin;   // cost units before this group
    int frags;            // ceil(M / 16)
    int mblocks;          // ceil(frags / kMaxFrags)
    int nblocks;          // ceil(N / kTileN)
    int stages;           // K / kStageK
    int tile_begin;       // tiles before this group
    int fmt;              // kFmtNvfp4 or kFmtMxfp4 (selects the stage costs)
};

NVFP4_HD int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// The schedule entry of a group with M, N >= 1 and K a positive multiple of
// kStageK, in m-blocks of at most maxf (1..kMaxFrags) fragments.
NVFP4_HD GroupSched make_group_sched(int M, int N, int K, int64_t cost_begin, int tile_begin, int maxf = kMaxFrags,
                                     int fmt = kFmtNvfp4)
{
    GroupSched g;
    g.cost_begin = cost_begin;
    g.tile_begin = tile_begin;
    g.fmt = fmt;
    g.frags = ceil_div_i(M, kFragRows);
    g.mblocks = ceil_div_i(g.frags, maxf);
    g.nblocks = ceil_div_i(N, kTileN);
    g.stages = K / kStageK;
    return g;
}

// Cost of one stage of a tile with f = 1..kMaxFrags fragments, in units of
// about 50 ns.  NVFP4: measured MI355X stage times 1.2, 1.45, 1.75, 2.3 and
// 2.8 us for 4, 6, 8, 10 and 12 fragments; odd counts interpolated (the
// MFMAs grow linearly with f), 1 and 2 extrapolated.  MXFP4 (scales staged
// in 4-stage blocks): one tile per workgroup at K 7168 and K 3584 gives
// 1.01, 1.07, 1.16, 1.12, 1.17, 1.22, 1.23, 1.18, 1.47, 1.54, 1.52 and
// 1.66 us per stage for 1..12 fragments, taken monotone in units of the
// NVFP4 table's 1-fragment stage (the step at 9: every wave then stages a
// second A fragment).
NVFP4_HD int tile_cost(int f) { return kTileCostBase + kTileCostPerFrag * f; }

NVFP4_HD int unit_cost(int f, int fmt = kFmtNvfp4)
{
    // One byte per fragment count (1..8 in the first word, 9..12 in the
    // second), read with a select, a shift and a mask: the kernel evaluates
    // this many times per walk, where a chain of comparisons compiles to a
    // chain of branches (measured: about 2 us per walk).
    //            f =   8  7  6  5  4  3  2  1                 12 11 10  9
    // NVFP4:          35 32 29 27 24 23 21 20                 56 51 46 41
    // MXFP4:          23 23 22 22 21 21 20 19                 31 29 28 27
    const bool mx = fmt == kFmtMxfp4;
    const uint64_t word = f <= 8 ? (mx ? 0x1717161615151413ull : 0x23201d1b18171514ull) : (mx ? 0x000000001f1d1c1bull : 0x0000000038332e29ull);
    const int i = (f <= 1 ? 0 : f > kMaxFrags ? kMaxFrags - 1 : f - 1) & 7;
    return (int)((word >> (8 * i)) & 0xFF);
}

// Fragments of m-block i of a group with F fragments in nmb m-blocks.
NVFP4_HD int mblock_frags(int F, int nmb, int i)
{
    const int base = F / nmb, extra = F % nmb;
    return base + (i < extra ? 1 : 0);
}

// First fragment of m-block i.
NVFP4_HD int mblock_first_frag(int F, int nmb, int i)
{
    const int base = F / nmb, extra = F % nmb;
    return i * base + (i < extra ? i : extra);
}

// Cost positions are int64_t on the host.  The functions below take the
// cost type C as a parameter: the kernel walks the schedule in int32_t (the
// host keeps a launch's total cost below kMaxLaunchCost, and no product of
// a cost and a workgroup count is formed), because the GPU's scalar unit
// has no 64-bit less-than: 64-bit cost comparisons become vector compares
// and branches on their result (measured: about 2 us per walk).
constexpr int64_t kMaxLaunchCost = ((int64_t)1 << 31) - 1;

// Cost before m-block i of a column (i <= mblocks): i tiles, each its
// tile_cost plus its stages.
template <typename C = int64_t>
NVFP4_HD C mblock_cost0(const GroupSched& g, int i)
{
    const int base = g.frags / g.mblocks, extra = g.frags % g.mblocks;
    const int big = i < extra ? i : extra;             // m-blocks of base + 1 fragments before i
    const C stage_sum = (C)(i - big) * unit_cost(base, g.fmt) + (C)big * unit_cost(base + 1, g.fmt);
    const C tile_sum = (C)(i - big) * tile_cost(base) + (C)big * tile_cost(base + 1);
    return tile_sum + stage_sum * g.stages;
}

// Cost of one n-block column of a group (all m-blocks, all stages).
template <typename C = int64_t>
NVFP4_HD C column_cost(const GroupSched& g) { return mblock_cost0<C>(g, g.mblocks); }

template <typename C = int64_t>
NVFP4_HD C group_cost(const GroupSched& g) { return column_cost<C>(g) * g.nblocks; }

// A unit position: tile (group, n-block, m-block) and stage.
struct Pos {
    int group, nb, mb, stage;
    int frags;            // fragments of the m-block
    int unit;             // cost of one of its stages
    int64_t tile_cost0;   // cost position of the tile's stage 0
};

// The stage-aligned position of cost point p: the first stage that starts at
// or after p.  Every group must have cost > 0 (the host launches no empty
// group).  For p >= the total cost the result has group == ngroups.
// gi0 may name any group at or before p's group (the scan starts there).
template <typename C = int64_t>
NVFP4_HD Pos locate(const GroupSched* gs, int ngroups, C p, int gi0 = 0)
{
    Pos r;
    int gi = gi0;   // p only grows below, so the scan resumes where it stopped
    for (;;) {
        while (gi + 1 < ngroups && (C)gs[gi + 1].cost_begin <= p) ++gi;
        const GroupSched& g = gs[gi];
        const C cb = (C)g.cost_begin;
        C q = p - cb;
        if (q >= group_cost<C>(g)) {
            r.group = ngroups;
            r.nb = r.mb = r.stage = r.frags = 0;
            r.unit = 1;
            r.tile_cost0 = p;
            return r;
        }
        const C cc = column_cost<C>(g);
        r.group = gi;
        r.nb = (int)(q / cc);
        q -= (C)r.nb * cc;
        int mb = 0;
        while (mb + 1 < g.mblocks && mblock_cost0<C>(g, mb + 1) <= q) ++mb;
        r.mb = mb;
        r.frags = mblock_frags(g.frags, g.mblocks, mb);
        r.unit = unit_cost(r.frags, g.fmt);
        const C mcost0 = mblock_cost0<C>(g, mb);
        q -= mcost0 + tile_cost(r.frags);   // relative to the start of stage 0
        r.stage = q <= 0 ? 0 : (int)((q + r.unit - 1) / r.unit);
        const C t0 = cb + (C)r.nb * cc + mcost0 + tile_cost(r.frags);
        r.tile_cost0 = t0;
        if (r.stage < g.stages) return r;
        p = t0 + (C)r.unit * g.stages;   // rounded past the tile: next tile
    }
}

// Cost position of stage s of the tile at position p.
NVFP4_HD int64_t stage_cost(const Pos& p, int s) { return p.tile_cost0 + (int64_t)s * p.unit; }

// XCDs of the chip: workgroups are dealt to them round-robin, and each has
// its own L2.
constexpr int kXcds = 8;

// Grid size for total cost W on cus CUs: one workgroup per CU at most, each
// range at least kMinUnitsPerWG long, rounded down to a multiple of kXcds
// above it.
NVFP4_HD int grid_size(int64_t W, int cus)
{
    int64_t G = W / kMinUnitsPerWG;
    if (G > cus) G = cus;
    if (G > kXcds) G -= G % kXcds;
    if (G < 1) G = 1;
    return (int)G;
}

// Cost of splitting a tile once more (about 3.9 us, measured): one more
// partial tile stored by a contributor and read back by the fix-up.
constexpr int kSplitCost = 78;

// Estimated time of a launch of total cost W over G workgroups holding
// `tiles` tiles, in cost units: one workgroup's range, plus kSplitCost for
// each contributor beyond the first of an average tile.
inline double launch_estimate(int64_t W, int G, int tiles)
{
    const double extra = (double)G / tiles - 1.0;
    return (double)W / G + (extra > 0.0 ? kSplitCost * extra : 0.0);
}

// The m-block size (1..kMaxFrags fragments) of a launch of n non-empty
// groups on cus CUs with the least launch_estimate, the largest on ties.
// Large m-blocks stream each B strip once and run the MFMAs densest; smaller
// ones give problems with few tiles more of them, so fewer workgroups share
// a tile.
inline int choose_max_frags(int n, const int* M, const int* N, const int* K, int cus, int fmt = kFmtNvfp4)
{
    int best = kMaxFrags;
    double best_t = 0.0;
    for (int maxf = kMaxFrags; maxf >= 1; --maxf) {
        int64_t W = 0;
        int tiles = 0;
        for (int i = 0; i < n; ++i) {
            const GroupSched g = make_group_sched(M[i], N[i], K[i], W, tiles, maxf, fmt);
            W += group_cost(g);
            tiles += g.mblocks * g.nblocks;
        }
        const double t = launch_estimate(W, grid_size(W, cus), tiles);
        if (maxf == kMaxFrags || t < best_t) {
            best = maxf;
            best_t = t;
        }
    }
    return best;
}

// Workgroup boundary b_w = floor(w * W / G) (w = 0..G), as
// (W / G) w + ((W % G) w) / G, which never forms W w.
template <typename C = int64_t>
NVFP4_HD C boundary(C W, int G, int w)
{
    return (W / G) * (C)w + ((W % G) * (C)w) / G;
}

// The workgroup that owns the stage starting at cost position c
// (the largest w with b_w <= c): a float estimate of c G / W (off by at
// most one for G <= 512), corrected exactly against boundary().
template <typename C = int64_t>
NVFP4_HD int owner(C W, int G, C c)
{
    int w = (int)((float)c * (float)G / (float)W);
    if (w > G - 1) w = G - 1;
    if (w < 0) w = 0;
    while (w > 0 && boundary<C>(W, G, w) > c) --w;
    while (w + 1 < G && boundary<C>(W, G, w + 1) <= c) ++w;
    return w;
}

// The boundaries of one launch without a division (the kernel's walk):
// b_w = q w + floor(r w / G) with q = W / G, r = W % G, and the last
// quotient as the high word of (r w) R, R = ceil(2^32 / G).  That is exact:
// R G = 2^32 + e with 0 <= e < G, so (r w) R / 2^32 exceeds (r w) / G by
// (r w) e / (G 2^32) < G^2 / 2^32, below 1 / G (the least distance from
// (r w) / G up to the next integer) while G^3 < 2^32.  Valid for
// W <= kMaxLaunchCost and 1 <= G <= kMaxBoundsG.
constexpr int kMaxBoundsG = 1024;
struct Bounds {
    int32_t q;    // W / G
    int32_t r;    // W % G
    uint32_t R;   // ceil(2^32 / G); unused (0) for G = 1, where r = 0
    int32_t G;
};

inline Bounds make_bounds(int64_t W, int G)
{
    Bounds b;
    b.q = (int32_t)(W / G);
    b.r = (int32_t)(W % G);
    b.R = G > 1 ? (uint32_t)((((uint64_t)1 << 32) + (uint64_t)G - 1) / (uint64_t)G) : 0u;
    b.G = G;
    return b;
}

NVFP4_HD int32_t bound_at(const Bounds& b, int w)
{
    const uint32_t t = (uint32_t)b.r * (uint32_t)w;   // < G^2
    return b.q * w + (int32_t)(((uint64_t)t * b.R) >> 32);
}

// owner() on Bounds: the same float estimate, corrected against bound_at().
NVFP4_HD int owner_b(const Bounds& b, int32_t W, int32_t c)
{
    const int G = b.G;
    int w = (int)((float)c * (float)G / (float)W);
    if (w > G - 1) w = G - 1;
    if (w < 0) w = 0;
    while (w > 0 && bound_at(b, w) > c) --w;
    while (w + 1 < G && bound_at(b, w + 1) <= c) ++w;
    return w;
}

// Workspace slots of workgroup w (one fp32 partial tile each): a tile split
// over workgroups w_first..w_last gets one partial from each contributor; w
// writes it to slot 0 when it is the tile's last contributor (the tile is the
// first of w's range) and to slot 1 otherwise (the tile is the last of w's
// range; a range inside one tile also uses slot 1).  Slot 2 is w's scratch.
constexpr int kSlotsPerWG = 3;
NVFP4_HD int partial_slot(int w, int w_last) { return w * kSlotsPerWG + (w < w_last ? 1 : 0); }
NVFP4_HD int scratch_slot(int w) { return w * kSlotsPerWG + 2; }

// A workgroup is the first contributor of at most one split tile (the last
// tile of its range), so the counter of a split tile is indexed by its first
// contributor: one counter per workgroup.
NVFP4_HD int counter_index(int w_first) { return w_first; }

// Counter of a tile split over workgroups w_first..w_last (finish_segment):
// arrivals of the contributors after the first in the low bits, plus the
// first contributor's claim of the fix-up or its hand-over.  The first adds
// kClaim, waits (bounded) until the count is complete, and on time-out swaps
// the claim for kHandOver by adding kHandOver - kClaim; every other adds 1.
constexpr int kCountMask = 0xFFFF;
constexpr int kClaim = 1 << 16;
constexpr int kHandOver = 1 << 17;

// Whether the first contributor finishes the tile, given the counter value
// it read (on claiming, while waiting, or returned by its hand-over add).
NVFP4_HD bool first_finishes(int counter, int others) { return (counter & kCountMask) == others; }

// Whether a later contributor finishes the tile, given the value its add
// returned: its arrival completes the count after the first handed over.
NVFP4_HD bool other_finishes(int old, int others)
{
    return (old & kCountMask) + 1 == others && (old & kHandOver) != 0;
}

// Global tile index of a position.
NVFP4_HD int tile_index(const GroupSched* gs, const Pos& p)
{
    const GroupSched& g = gs[p.group];
    return g.tile_begin + p.nb * g.mblocks + p.mb;
}

}  // namespace nvfp4sched

#endif  // NVFP4GG_SCHEDULE_H
