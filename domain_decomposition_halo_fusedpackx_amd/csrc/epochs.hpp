// epochs.hpp -- the host's count of fused launches per kernel family (host
// code only, no HIP types).
//
// "Redesigning GROMACS Halo Exchange" (paper review), Algorithm 5: every
// exchange signals with a new value (sigVal), and a waiter compares the
// counters with the value of its own exchange. Here the value is an epoch:
// the number of this family's launches so far, plus one. Eager launches are
// handed the epoch the host counted. A launch recorded into a HIP graph is
// replayed with its arguments unchanged, so once any launch of a plan has
// been captured, the host no longer sees every launch: it passes 0 from then
// on and the kernels infer the epoch from launch counts on the device.
//
// The count moves only for launches that were enqueued: a launch that fails
// leaves the device counters where they were, and counting it anyway would
// make every later eager exchange of the family wait for an epoch that never
// completes.
#pragma once

#include <cstdint>

namespace halo {

template <int kFam>
struct EpochBook {
    uint32_t count[kFam] = {};
    bool on_device = false;  // a launch was captured: the kernels infer their epoch

    // The epoch argument of the next launch of `family` (0: inferred on the
    // device). `capturing`: the launch stream is being captured. A count that
    // wraps to 0 asks the kernels to infer that one epoch.
    uint32_t next(int family, bool capturing)
    {
        if (capturing) on_device = true;
        return on_device ? 0u : count[family] + 1u;
    }

    // Record whether the launch that next() was asked for was enqueued.
    void launched(int family, bool ok)
    {
        if (ok && !on_device) ++count[family];
    }

    void reset()
    {
        for (uint32_t &c : count) c = 0;
    }
};

}  // namespace halo
