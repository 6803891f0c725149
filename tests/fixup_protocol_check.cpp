// CPU model check of the split-tile counter protocol (schedule.h's
// first_finishes / other_finishes, as finish_segment uses them): threads
// play the contributors of a tile, with random delays and wait limits
// (including 0, the hand-over path), on a std::atomic counter.  Checks that
// exactly one finishes the tile and that every partial was published before
// the finisher looked.
//
// Orderings follow the kernel: every counter operation is relaxed, and the
// partials are relaxed atomic stores and loads (the kernel's sc1 accesses).
// The kernel orders a contributor's partial stores before its counter add by
// waiting for their completion (s_waitcnt vmcnt(0)) ahead of the add, and the
// finisher's partial loads after its counter read by waiting for the read's
// value before issuing them; in the C++ memory model those waits are a
// release fence before the add and an acquire fence after the read, which is
// what the model uses.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "../nvfp4_block_scaled_grouped_amd/csrc/schedule.h"

using namespace nvfp4sched;

static int trial(int P, int wait_limit, unsigned seed)
{
    std::atomic<int> counter{0};
    std::vector<std::atomic<int>> published(P);
    for (auto& p : published) p.store(0);
    std::atomic<int> finishers{0}, bad{0};
    const int others = P - 1;
    auto check_all = [&] {
        for (int w = 0; w < P; ++w)
            if (published[w].load(std::memory_order_relaxed) == 0) bad.fetch_add(1);
    };
    std::vector<std::thread> ts;
    for (int w = 0; w < P; ++w) {
        ts.emplace_back([&, w] {
            std::mt19937 rng(seed * 131 + w);
            std::this_thread::sleep_for(std::chrono::microseconds(rng() % 300));
            if (w != 0) {
                published[w].store(1, std::memory_order_relaxed);   // the partial store
                std::atomic_thread_fence(std::memory_order_release);  // its completion wait
                const int old = counter.fetch_add(1, std::memory_order_relaxed);
                if (other_finishes(old, others)) {
                    std::atomic_thread_fence(std::memory_order_acquire);
                    finishers.fetch_add(1);
                    check_all();
                }
                return;
            }
            // First contributor: its partial stays private unless it hands over.
            const int old = counter.fetch_add(kClaim, std::memory_order_relaxed);
            bool done = first_finishes(old, others);
            for (int poll = 0; !done && poll < wait_limit; ++poll) {
                std::this_thread::sleep_for(std::chrono::microseconds(1));
                done = first_finishes(counter.load(std::memory_order_relaxed), others);
            }
            if (!done) {
                published[0].store(1, std::memory_order_relaxed);
                std::atomic_thread_fence(std::memory_order_release);
                done = first_finishes(counter.fetch_add(kHandOver - kClaim, std::memory_order_relaxed), others);
            } else {
                published[0].store(1, std::memory_order_relaxed);   // in registers: present by definition
            }
            if (done) {
                std::atomic_thread_fence(std::memory_order_acquire);
                finishers.fetch_add(1);
                check_all();
            }
        });
    }
    for (auto& t : ts) t.join();
    if (finishers.load() != 1 || bad.load() != 0) {
        std::printf("FAIL P=%d wait_limit=%d seed=%u: %d finishers, %d missing partials\n", P, wait_limit, seed,
                    finishers.load(), bad.load());
        return 1;
    }
    return 0;
}

int main()
{
    int fails = 0;
    unsigned seed = 1;
    for (int P : {2, 3, 5, 8})
        for (int limit : {0, 1, 20, 100000})
            for (int r = 0; r < 60; ++r) fails += trial(P, limit, seed++);
    if (fails) {
        std::printf("FAILED %d\n", fails);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
