// dspark_gridsync.hpp -- device-wide barrier with a bounded wait, for a
// persistent kernel whose workgroups are all resident at once (cooperative
// launch).
//
// Protocol.  One counter and one error word, both zero before the launch.
// Every workgroup arrives once at each barrier by adding one to the counter
// (a release: the workgroup's writes before the barrier become visible to
// whoever observes the new count), so barrier j is passed once the counter
// reaches (j + 1) * arrivals, arrivals = the number of workgroups.  A waiter
// polls the counter and, once it has seen the target, performs an acquire
// (so that what the other workgroups wrote before arriving is visible to
// it); it gives up after `limit` polls, or at once when the error word is
// set, and a waiter that gives up sets the error word.  (On the device the
// release and acquire are the waits of the kernel's own barrier wrapper:
// its cross-workgroup data goes through device-coherent accesses.)
// So every waiter returns: true when the barrier completed, false when it
// gave up (and then every other waiter gives up within one poll, and the
// kernel's workgroups exit).  The host reads the error word after the
// kernel to learn that the outputs are invalid.
//
// The protocol is a template over its atomic operations: the kernel passes
// AgentSyncOps (agent-scope HIP atomics, vector memory instructions only),
// and the CPU test of the protocol passes std::atomic-based operations.
#pragma once

namespace dspark {

template <class Ops>
__host__ __device__ inline bool gridsync_arrive_and_wait(Ops& ops, unsigned target, unsigned limit)
{
    ops.arrive();
    for (unsigned n = 0;; ++n) {
        if (ops.count() >= target) {
            ops.acquire();
            return true;
        }
        if (ops.failed() || n >= limit) {
            ops.fail();
            return false;
        }
        ops.pause();
    }
}

}  // namespace dspark
