// schedule.h -- work decomposition of the grouped GEMM into (tile, K-stage)
// units and their even split over a persistent grid (stream-K style).
//
// Plain C++ usable from host and device code; the kernel and the host
// launcher include it, and a CPU test compiles it on its own.
//
// Terms:
//   * fragment: 32 rows of A_i (the MFMA tile height).
//   * m-block: up to kMaxFrags fragments of one group, processed together.
//     A group with F = ceil(M/32) fragments has nmb = ceil(F / kMaxFrags)
//     m-blocks; fragments are spread evenly, so the first F % nmb m-blocks
//     get F / nmb + 1 fragments and the rest F / nmb.
//   * n-block: kTileN columns of B_i.
//   * tile: (group, n-block, m-block); tiles are ordered by group, then
//     n-block, then m-block, so the m-blocks that share a B strip are
//     adjacent in the order.
//   * stage: kStageK consecutive K of a tile.  A stage of a tile with f
//     fragments costs unit_cost(f) units (about 50 ns of MI355X time each,
//     fitted to measured stage times): the B stream and its dequantisation
//     do not grow with f, the MFMAs do, and tiles of more than 4 fragments
//     give every wave a second piece of A to dequantise.
//   * A tile's cost range is kTileCost (the start-up and wind-down of the
//     segment that starts it: first loads, partial-tile stores, the fix-up)
//     followed by its stages.
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

constexpr int kMaxFrags = 6;       // fragments per m-block
constexpr int kFragRows = 32;      // rows per fragment
constexpr int kTileN = 256;        // columns per n-block
constexpr int kStageK = 128;       // K per stage
constexpr int kMaxGroups = 32;     // groups per launch
constexpr int kTileCost = 200;     // cost units of a tile beyond its stages
constexpr int kMaxUnitCost = 53;   // the costliest stage (6 fragments)
// Least cost handed to one workgroup: keeps every workgroup range longer
// than the costliest stage, so the workgroups sharing a tile are
// consecutive.
constexpr int64_t kMinUnitsPerWG = 64;
static_assert(kMinUnitsPerWG >= kMaxUnitCost, "a workgroup range must hold a stage");

struct GroupSched {
    int64_t cost_begin;   // cost units before this group
    int frags;            // ceil(M / 32)
    int mblocks;          // ceil(frags / kMaxFrags)
    int nblocks;          // ceil(N / kTileN)
    int stages;           // K / kStageK
    int tile_begin;       // tiles before this group
};

NVFP4_HD int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// The schedule entry of a group with M, N >= 1 and K a positive multiple of
// kStageK.
NVFP4_HD GroupSched make_group_sched(int M, int N, int K, int64_t cost_begin, int tile_begin)
{
    GroupSched g;
    g.cost_begin = cost_begin;
    g.tile_begin = tile_begin;
    g.frags = ceil_div_i(M, kFragRows);
    g.mblocks = ceil_div_i(g.frags, kMaxFrags);
    g.nblocks = ceil_div_i(N, kTileN);
    g.stages = K / kStageK;
    return g;
}

// Cost of one stage of a tile with f = 1..kMaxFrags fragments, in units of
// about 50 ns (measured MI355X stage times: 1.5, 1.6, 1.8, 2.3 and 2.7 us for
// 2 to 6 fragments; one fragment extrapolated).
NVFP4_HD int unit_cost(int f)
{
    return f <= 1 ? 28 : f == 2 ? 30 : f == 3 ? 32 : f == 4 ? 35 : f == 5 ? 47 : kMaxUnitCost;
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

// Cost before m-block i of a column (i <= mblocks): i tiles of kTileCost
// plus their stages.
NVFP4_HD int64_t mblock_cost0(const GroupSched& g, int i)
{
    const int base = g.frags / g.mblocks, extra = g.frags % g.mblocks;
    const int big = i < extra ? i : extra;             // m-blocks of base + 1 fragments before i
    const int64_t stage_sum = (int64_t)(i - big) * unit_cost(base) + (int64_t)big * unit_cost(base + 1);
    return (int64_t)kTileCost * i + stage_sum * g.stages;
}

// Cost of one n-block column of a group (all m-blocks, all stages).
NVFP4_HD int64_t column_cost(const GroupSched& g) { return mblock_cost0(g, g.mblocks); }

NVFP4_HD int64_t group_cost(const GroupSched& g) { return column_cost(g) * g.nblocks; }

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
NVFP4_HD Pos locate(const GroupSched* gs, int ngroups, int64_t p)
{
    Pos r;
    for (;;) {
        int gi = 0;
        while (gi + 1 < ngroups && gs[gi + 1].cost_begin <= p) ++gi;
        const GroupSched& g = gs[gi];
        int64_t q = p - g.cost_begin;
        if (q >= group_cost(g)) {
            r.group = ngroups;
            r.nb = r.mb = r.stage = r.frags = 0;
            r.unit = 1;
            r.tile_cost0 = p;
            return r;
        }
        const int64_t cc = column_cost(g);
        r.group = gi;
        r.nb = (int)(q / cc);
        q -= (int64_t)r.nb * cc;
        int mb = 0;
        while (mb + 1 < g.mblocks && mblock_cost0(g, mb + 1) <= q) ++mb;
        r.mb = mb;
        r.frags = mblock_frags(g.frags, g.mblocks, mb);
        r.unit = unit_cost(r.frags);
        const int64_t mcost0 = mblock_cost0(g, mb);
        q -= mcost0 + kTileCost;   // relative to the start of stage 0
        r.stage = q <= 0 ? 0 : (int)((q + r.unit - 1) / r.unit);
        r.tile_cost0 = g.cost_begin + (int64_t)r.nb * cc + mcost0 + kTileCost;
        if (r.stage < g.stages) return r;
        p = r.tile_cost0 + (int64_t)r.unit * g.stages;   // rounded past the tile: next tile
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

// Workgroup boundary b_w = floor(w * W / G) (w = 0..G).
NVFP4_HD int64_t boundary(int64_t W, int G, int w) { return (W * (int64_t)w) / G; }

// The workgroup that owns the stage starting at cost position c
// (the largest w with b_w <= c).
NVFP4_HD int owner(int64_t W, int G, int64_t c)
{
    int64_t w = (c * G + G - 1) / W;
    if (w > G - 1) w = G - 1;
    while (w > 0 && boundary(W, G, (int)w) > c) --w;
    while (w + 1 < G && boundary(W, G, (int)w + 1) <= c) ++w;
    return (int)w;
}

// Workspace slots of workgroup w (one fp32 partial tile each): a tile split
// over workgroups w_first..w_last gets one partial from each contributor; w
// writes it to slot 0 when it is the tile's last contributor (the tile is the
// first of w's range) and to slot 1 otherwise (the tile is the last of w's
// range; a range inside one tile also uses slot 1).  Slot 2 is w's scratch.
constexpr int kSlotsPerWG = 3;
NVFP4_HD int partial_slot(int w, int w_last) { return w * kSlotsPerWG + (w < w_last ? 1 : 0); }
NVFP4_HD int scratch_slot(int w) { return w * kSlotsPerWG + 2; }

// Global tile index of a position.
NVFP4_HD int tile_index(const GroupSched* gs, const Pos& p)
{
    const GroupSched& g = gs[p.group];
    return g.tile_begin + p.nb * g.mblocks + p.mb;
}

}  // namespace nvfp4sched

#endif  // NVFP4GG_SCHEDULE_H
