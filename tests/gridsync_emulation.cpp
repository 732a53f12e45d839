// CPU emulation of the device-wide barrier protocol of
// draft_verify_sampling_prev_amd/csrc/dspark_gridsync.hpp: each std::thread
// plays one workgroup of the persistent draft kernel.  Built and run by
// tests/test_gridsync_cpu.py.
//
//   gridsync_emulation order  <groups> <barriers>   every group passes every barrier; no group passes
//                                                    barrier j before all groups arrived at it
//   gridsync_emulation phantom <groups> <limit>      one more arrival than groups is required: every
//                                                    group gives up, the error word is set
//   gridsync_emulation dead    <groups> <limit>      group 0 never arrives at barrier 1: every other
//                                                    group gives up there, the error word is set
#define __host__
#define __device__
#include "dspark_gridsync.hpp"

#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <thread>
#include <vector>

struct HostOps {
    std::atomic<unsigned>* ctr;
    std::atomic<unsigned>* err;
    void arrive() { ctr->fetch_add(1u, std::memory_order_release); }
    unsigned count() { return ctr->load(std::memory_order_relaxed); }
    void acquire() { std::atomic_thread_fence(std::memory_order_acquire); }
    bool failed() { return err->load(std::memory_order_relaxed) != 0u; }
    void fail() { err->store(1u, std::memory_order_relaxed); }
    void pause() { std::this_thread::yield(); }
};

int main(int argc, char** argv)
{
    if (argc < 4) return 2;
    const std::string mode = argv[1];
    const unsigned groups = (unsigned)atoi(argv[2]);
    const unsigned arg = (unsigned)atoi(argv[3]);
    std::atomic<unsigned> ctr{0}, err{0};
    std::vector<std::atomic<unsigned>> phase(groups);  // barriers each group has arrived at
    for (auto& p : phase) p = 0;
    std::atomic<int> violations{0}, passed{0}, gave_up{0};
    const unsigned barriers = mode == "order" ? arg : 3u;
    const unsigned limit = mode == "order" ? 4000000000u : arg;
    const unsigned arrivals = groups + (mode == "phantom" ? 1u : 0u);
    auto t0 = std::chrono::steady_clock::now();
    std::vector<std::thread> th;
    for (unsigned g = 0; g < groups; ++g)
        th.emplace_back([&, g]() {
            std::mt19937 rng(1234u + g);
            HostOps ops{&ctr, &err};
            for (unsigned j = 0; j < barriers; ++j) {
                for (int spin = rng() % 2000; spin > 0; --spin) std::this_thread::yield();  // uneven work
                if (mode == "dead" && g == 0 && j == 1) return;  // this group stops arriving
                phase[g].store(j + 1, std::memory_order_relaxed);
                const bool ok = dspark::gridsync_arrive_and_wait(ops, (j + 1) * arrivals, limit);
                if (!ok) {
                    gave_up++;
                    return;  // a workgroup that gives up exits
                }
                for (unsigned h = 0; h < groups; ++h)
                    if (phase[h].load(std::memory_order_relaxed) < j + 1) violations++;
                passed++;
            }
        });
    for (auto& t : th) t.join();
    const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    printf("mode=%s groups=%u passed=%d gave_up=%d violations=%d error=%u counter=%u seconds=%.3f\n", mode.c_str(),
           groups, passed.load(), gave_up.load(), violations.load(), err.load(), ctr.load(), secs);
    return 0;
}
