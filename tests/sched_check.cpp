// CPU check of the work decomposition in schedule.h: replays every
// workgroup's walk over (tile, stage) units exactly as the kernel does and
// verifies the partition and the split-tile bookkeeping.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "../nvfp4_block_scaled_grouped_amd/csrc/schedule.h"

using namespace nvfp4sched;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { ++fails; std::printf("FAIL %s:%d: ", __FILE__, __LINE__); std::printf(__VA_ARGS__); std::printf("\n"); return; } } while (0)

static void run_case(const std::vector<int>& M, const std::vector<int>& N, const std::vector<int>& K, int cus, int maxf,
                     int fmt)
{
    int ng = (int)M.size();
    CHECK(maxf >= 1 && maxf <= kMaxFrags, "m-block size %d", maxf);
    GroupSched gs[kMaxGroups];
    int64_t cost = 0;
    int tiles = 0;
    for (int i = 0; i < ng; ++i) {
        gs[i] = make_group_sched(M[i], N[i], K[i], cost, tiles, maxf, fmt);
        cost += group_cost(gs[i]);
        tiles += gs[i].mblocks * gs[i].nblocks;
        // m-block partition covers all fragments, each block 1..maxf, sizes
        // differing by at most one
        int sum = 0;
        for (int b = 0; b < gs[i].mblocks; ++b) {
            int f = mblock_frags(gs[i].frags, gs[i].mblocks, b);
            CHECK(f >= 1 && f <= maxf, "mblock frags %d", f);
            CHECK(f >= mblock_frags(gs[i].frags, gs[i].mblocks, gs[i].mblocks - 1), "uneven m-blocks");
            CHECK(f <= mblock_frags(gs[i].frags, gs[i].mblocks, gs[i].mblocks - 1) + 1, "uneven m-blocks");
            CHECK(mblock_first_frag(gs[i].frags, gs[i].mblocks, b) == sum, "first frag");
            sum += f;
        }
        CHECK(sum == gs[i].frags, "frag sum");
        CHECK(gs[i].mblocks == (gs[i].frags + maxf - 1) / maxf, "m-block count");
        // the closed-form m-block cost prefix matches the sum of its tiles
        int64_t c = 0;
        for (int b = 0; b <= gs[i].mblocks; ++b) {
            CHECK(mblock_cost0(gs[i], b) == c, "mblock_cost0 group %d block %d", i, b);
            if (b < gs[i].mblocks)
                c += tile_cost(mblock_frags(gs[i].frags, gs[i].mblocks, b)) +
                     (int64_t)gs[i].stages * unit_cost(mblock_frags(gs[i].frags, gs[i].mblocks, b), fmt);
        }
    }
    const int64_t W = cost;
    const int G = grid_size(W, cus);
    CHECK(G >= 1 && G <= cus, "grid size %d", G);
    CHECK(G == 1 || W / G >= kMinUnitsPerWG, "workgroup range shorter than kMinUnitsPerWG");
    // covered[(tile, stage)] = workgroup
    std::map<std::pair<int, int>, int> covered;
    std::map<int, std::set<int>> contrib;         // tile -> workgroups
    std::map<std::pair<int, int>, int> slot_use;  // (wg, slot) -> tile
    std::map<int, int> counter_use;               // counter index -> split tile
    for (int w = 0; w < G; ++w) {
        const int64_t b1 = boundary(W, G, w + 1);
        Pos pos = locate(gs, ng, boundary(W, G, w));
        int guard = 0;
        while (pos.group < ng && stage_cost(pos, pos.stage) < b1) {
            CHECK(++guard < 1000000, "runaway walk");
            const GroupSched& g = gs[pos.group];
            const int unit = pos.unit;
            CHECK(unit == unit_cost(pos.frags, fmt), "unit cost");
            const int64_t s_end64 = (b1 - pos.tile_cost0 + unit - 1) / unit;
            const int s_end = s_end64 < g.stages ? (int)s_end64 : g.stages;
            CHECK(s_end > pos.stage, "empty segment w=%d", w);
            const int t = tile_index(gs, pos);
            CHECK(t >= 0 && t < tiles, "tile index %d", t);
            for (int s = pos.stage; s < s_end; ++s) {
                auto key = std::make_pair(t, s);
                CHECK(!covered.count(key), "stage covered twice t=%d s=%d", t, s);
                covered[key] = w;
                CHECK(owner(W, G, stage_cost(pos, s)) == w, "owner mismatch t=%d s=%d w=%d", t, s, w);
            }
            contrib[t].insert(w);
            const int64_t c_first = pos.tile_cost0;
            const int64_t c_last = pos.tile_cost0 + (int64_t)(g.stages - 1) * unit;
            const int wf = owner(W, G, c_first), wl = owner(W, G, c_last);
            CHECK(wf <= w && w <= wl, "contributor range");
            if (wf != wl) {
                // one counter per split tile, indexed by its first contributor
                const int ci = counter_index(wf);
                CHECK(ci >= 0 && ci < G, "counter index %d outside [0, %d)", ci, G);
                auto cu = counter_use.find(ci);
                CHECK(cu == counter_use.end() || cu->second == t, "counter %d shared by tiles %d and %d", ci,
                      cu == counter_use.end() ? -1 : cu->second, t);
                counter_use[ci] = t;
                const int slot = partial_slot(w, wl);
                auto sk = std::make_pair(w, slot);
                CHECK(!slot_use.count(sk), "slot reused w=%d slot=%d", w, slot);
                slot_use[sk] = t;
                CHECK(slot >= w * kSlotsPerWG && slot < (w + 1) * kSlotsPerWG, "slot outside w's slots");
                CHECK(slot != scratch_slot(w), "partial in the scratch slot");
                CHECK(slot < kSlotsPerWG * G, "slot bound");
            }
            if (W <= kMaxLaunchCost) {
                // the kernel's 32-bit walk finds the same segment and contributors
                const Pos p32 = locate<int32_t>(gs, ng, (int32_t)pos.tile_cost0 + (int32_t)pos.stage * unit);
                CHECK(p32.group == pos.group && p32.nb == pos.nb && p32.mb == pos.mb && p32.stage == pos.stage &&
                          p32.tile_cost0 == pos.tile_cost0 && p32.unit == pos.unit, "32-bit locate w=%d", w);
                CHECK(owner<int32_t>((int32_t)W, G, (int32_t)c_first) == wf &&
                          owner<int32_t>((int32_t)W, G, (int32_t)c_last) == wl, "32-bit owner w=%d", w);
                CHECK(boundary<int32_t>((int32_t)W, G, w + 1) == b1, "32-bit boundary w=%d", w);
                // the kernel's walk: division-free boundaries and owners, and
                // locate started at the group a ballot over the table counts
                const Bounds bd = make_bounds(W, G);
                CHECK(bound_at(bd, w + 1) == b1 && bound_at(bd, w) == boundary(W, G, w), "bound_at w=%d", w);
                CHECK(owner_b(bd, (int32_t)W, (int32_t)c_first) == wf && owner_b(bd, (int32_t)W, (int32_t)c_last) == wl,
                      "owner_b w=%d", w);
                const int32_t cp = (int32_t)pos.tile_cost0 + (int32_t)pos.stage * unit;
                int gi = 0;
                for (int j = 1; j < ng; ++j) gi += (int32_t)gs[j].cost_begin <= cp ? 1 : 0;
                const Pos ph = locate<int32_t>(gs, ng, cp, gi);
                CHECK(ph.group == p32.group && ph.nb == p32.nb && ph.mb == p32.mb && ph.stage == p32.stage &&
                          ph.tile_cost0 == p32.tile_cost0, "locate from the counted group w=%d", w);
            }
            if (s_end < g.stages) break;
            pos = locate(gs, ng, pos.tile_cost0 + (int64_t)unit * g.stages);
        }
    }
    // every stage of every tile covered exactly once
    int64_t expect = 0;
    for (int i = 0; i < ng; ++i) expect += (int64_t)gs[i].mblocks * gs[i].nblocks * gs[i].stages;
    CHECK((int64_t)covered.size() == expect, "covered %zu of %lld stages", covered.size(), (long long)expect);
    // contributors of each tile form the contiguous range [owner(first), owner(last)]
    for (auto& kv : contrib) {
        const std::set<int>& ws = kv.second;
        const int lo = *ws.begin(), hi = *ws.rbegin();
        CHECK((int)ws.size() == hi - lo + 1, "tile %d contributors not contiguous", kv.first);
    }
}

// The launch's m-block size as the host picks it, then the schedule check.
static void run_launch(const std::vector<int>& M, const std::vector<int>& N, const std::vector<int>& K, int cus,
                       int fmt)
{
    const int maxf = choose_max_frags((int)M.size(), M.data(), N.data(), K.data(), cus, fmt);
    run_case(M, N, K, cus, maxf, fmt);
}

// Division-free boundaries and owners against boundary() and owner() over
// every workgroup count up to kMaxBoundsG, at random totals up to
// kMaxLaunchCost and at the extremes.
static void check_bounds()
{
    std::mt19937 brng(777);
    for (int G = 1; G <= kMaxBoundsG; ++G) {
        for (int rep = 0; rep < 4; ++rep) {
            const int64_t W = rep == 0   ? kMaxLaunchCost
                              : rep == 1 ? (int64_t)G * kMinUnitsPerWG
                                         : 1 + (int64_t)(brng() % (uint32_t)kMaxLaunchCost);
            const Bounds bd = make_bounds(W, G);
            for (int w = 0; w <= G; ++w)
                CHECK(bound_at(bd, w) == boundary(W, G, w), "bound_at G=%d W=%lld w=%d", G, (long long)W, w);
            for (int k = 0; k < 16; ++k) {
                const int32_t c = (int32_t)(brng() % (uint64_t)W);
                CHECK(owner_b(bd, (int32_t)W, c) == owner(W, G, (int64_t)c), "owner_b G=%d W=%lld c=%d", G,
                      (long long)W, c);
            }
        }
    }
}

int main()
{
    // The five workloads, at the size the host picks and at every size.
    const std::vector<std::vector<std::vector<int>>> five = {
        {{64, 96}, {256, 256}, {512, 512}},
        {{128, 384}, {4096, 4096}, {1536, 1536}},
        {{192, 320}, {3072, 3072}, {4096, 4096}},
        {{40, 76, 168, 72, 164, 148, 196, 160}, std::vector<int>(8, 7168), std::vector<int>(8, 2048)},
        {{80, 176, 128, 72, 64, 248, 96, 160}, std::vector<int>(8, 4096), std::vector<int>(8, 7168)},
    };
    for (int fmt : {kFmtNvfp4, kFmtMxfp4})
        for (const auto& w : five) {
            run_launch(w[0], w[1], w[2], 256, fmt);
            for (int maxf = 1; maxf <= kMaxFrags; ++maxf) run_case(w[0], w[1], w[2], 256, maxf, fmt);
        }
    check_bounds();
    // Random shapes, grid sizes and m-block sizes.
    std::mt19937 rng(12345);
    for (int it = 0; it < 3000; ++it) {
        const int ng = 1 + rng() % 12;
        std::vector<int> M, N, K;
        for (int i = 0; i < ng; ++i) {
            M.push_back(1 + rng() % 700);
            N.push_back(1 + rng() % 3000);
            K.push_back(kStageK * (1 + rng() % 48));
        }
        const int cus = 1 + rng() % 300;
        const int fmt = (it / 2) % 2 ? kFmtMxfp4 : kFmtNvfp4;
        if (it % 2 == 0)
            run_launch(M, N, K, cus, fmt);
        else
            run_case(M, N, K, cus, 1 + rng() % kMaxFrags, fmt);
        if (fails) break;
    }
    if (fails) { std::printf("FAILED %d\n", fails); return 1; }
    std::printf("OK\n");
    return 0;
}
